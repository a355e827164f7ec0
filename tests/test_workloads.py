"""The synthetic workloads have the shapes and structure the pages describe."""
import numpy as np
import torch

import oracle
import workloads as wl
from test_oracle_pins import u16


def test_32b_class_footprint_closed_form():
    """The pages' KV footprint of a 32B-class GQA model (paperlayer summary,
    section 2; fixture tests/golden/kv_footprint_32b_class.txt): the
    workload's KV heads and head dim over 64 layers give the printed 256 KiB
    per token in bf16, 8.6 GB per request at 32.7K context and nine requests
    in 80 GB."""
    from test_oracle_pins import _golden
    g = _golden("kv_footprint_32b_class.txt")
    w = wl.WORKLOADS["gqa32b_ragged_b16_staged"]
    per_token = int(g["layers"]) * w.H_kv * w.D * 2 * 2
    assert per_token == g["kib_per_token"] * 1024
    assert round(g["avg_context_tokens"] * per_token / 1e9, 1) == g["gb_per_request"]
    assert int(g["hbm_gb"] * 1e9 // (g["avg_context_tokens"] * per_token)) == g["requests_fit"]


def test_qwen3_8b_shapes():
    w = wl.WORKLOADS["qwen3_8b_16k_b128_staged"]
    assert (w.H_q, w.H_kv, w.D, w.bs, w.K_b, w.NB_max) == (32, 8, 128, 16, 128, 1024)
    assert oracle.fetch_cap_blocks(w.cap, w.K_b) == 6
    # one block of one KV head, K then V, is 8 KiB
    assert 2 * w.bs * w.D * 2 == 8192


def test_ragged_contexts_in_range_and_padding():
    w = wl.WORKLOADS["gqa32b_ragged_b16_staged"].shrink(B=6, ctx=(50, 400))
    ctx = wl.context_lengths(w)
    assert ctx.min() >= 50 and ctx.max() <= 400
    kv = wl.kv_pool(w).float()
    for r in range(w.B):
        flat = kv[r, :, :, 0].reshape(w.H_kv, -1, w.D)
        assert (flat[:, int(ctx[r]):] == wl.PAD_VALUE).all()
        assert (flat[:, : int(ctx[r])].abs() < wl.PAD_VALUE).all()


def test_drift_turns_over_about_five_percent_per_step():
    """The staged workloads' predicted set drifts by about 5% of the budget
    per step, so a 0.05 fetch cap keeps up (section 5, eviction strategy)."""
    w = wl.WORKLOADS["qwen3_8b_16k_b128_staged"].shrink(B=2)
    ctx = wl.context_lengths(w).numpy()
    kv = u16(wl.kv_pool(w))
    summ = oracle.build_summaries(kv, ctx, w.bs)
    prev = None
    changes = []
    for s in range(6):
        sc = oracle.score(u16(wl.lookahead(w, s)), summ, ctx, w.bs, w.H_kv)
        sel, _ = oracle.select(sc, ctx, w.bs, w.K_b)
        if prev is not None:
            for r in range(w.B):
                for h in range(w.H_kv):
                    changes.append(len(set(sel[r, h]) - set(prev[r, h])))
        prev = sel
    frac = np.mean(changes) / w.K_b
    assert 0.02 < frac < 0.10, frac


def test_true_next_query_is_the_first_draft_plus_noise():
    w = wl.WORKLOADS["qwen3_8b_16k_b128_staged"].shrink(B=4)
    base = wl.lookahead(w, 3)[:, 0]
    assert torch.equal(wl.true_next_query(w, 3, 0.0), base)
    noisy = wl.true_next_query(w, 3, 0.5).float()
    diff = noisy - wl.lookahead_f32(w, 3)[:, 0]
    assert abs(float(diff.std()) - 0.5) < 0.02
    assert torch.equal(wl.true_next_query(w, 3, 0.5), wl.true_next_query(w, 3, 0.5))   # seeded
