"""The synthetic workloads have the shapes and structure the pages describe."""
import numpy as np
import torch

import oracle
import workloads as wl
from test_oracle_pins import u16


def test_32b_class_footprint_closed_form():
    """A 32B-class GQA model keeps 256 KiB of KV per token in bf16 over its 64
    layers, 8.6 GB per request at 32.7K context, 9 requests in 80 GB
    (paperlayer summary, section 2; agihunt summary)."""
    w = wl.WORKLOADS["gqa32b_ragged_b16_staged"]
    per_token = 64 * w.H_kv * w.D * 2 * 2
    assert per_token == 256 * 1024
    assert round(32.7e3 * per_token / 1e9, 1) == 8.6
    assert int(80e9 // (32.7e3 * per_token)) == 9


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
