"""The Python binding refuses mismatched shapes before anything reaches the
library.  The C entry points see only pointers, so a tensor of the wrong
size would otherwise become an out-of-bounds device access.

No GPU: the library handle is replaced by a recorder, the device test by one
that accepts CPU tensors, and every case checks that a mismatch raises
ValueError with no library call made (a matching call is recorded)."""
import pytest
import torch

from prefetch_block_scoring_amd import binding

bf16, f32, i32, i64 = torch.bfloat16, torch.float32, torch.int32, torch.int64
B, H_q, H_kv, NB, D, bs, K_b, T, S = 2, 8, 2, 40, 128, 16, 8, 8, 11


class Recorder:
    """Stands in for the library: records each entry point called."""

    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        def call(*args):
            self.calls.append(name)
            return 0
        return call


@pytest.fixture
def lib(monkeypatch):
    rec = Recorder()
    monkeypatch.setattr(binding, "_lib", rec)
    monkeypatch.setattr(binding, "_on_device", lambda t: True)
    return rec


def z(shape, dtype):
    return torch.zeros(shape, dtype=dtype)


def score_args():
    return dict(q_look=z((B, 1, H_q, D), bf16), kminmax=z((B, H_kv, NB, 2, D), bf16), ctx_len=z((B,), i32),
                scores=z((B, H_kv, NB), f32))


def topk_args():
    return dict(scores=z((B, H_kv, NB), f32), ctx_len=z((B,), i32), K_b=K_b, sel=z((B, H_kv, K_b), i32),
                n_sel=z((B, H_kv), i32))


def attn_args():
    return dict(q=z((B, H_q, D), bf16), kv_pool=z((B, H_kv, S, 2, bs, D), bf16), tbl_slot=z((B, H_kv, T), i32),
                tbl_block=z((B, H_kv, T), i32), tbl_n=z((B, H_kv), i32), ctx_len=z((B,), i32),
                out=z((B, H_q, D), bf16), lse=z((B, H_q), f32))


def lookahead_args():
    a = attn_args()
    a["q"] = z((B, 2, H_q, D), bf16)
    a["out"] = z((B, 2, H_q, D), bf16)
    a["lse"] = z((B, 2, H_q), f32)
    return a


def stage_args():
    return dict(sel=z((B, H_kv, K_b), i32), n_sel=z((B, H_kv), i32), scores=z((B, H_kv, NB), f32),
                ctx_len=z((B,), i32), K_b=K_b, C=3, step=0, slot_block=z((B, H_kv, S), i32),
                slot_stamp=z((B, H_kv, S), i32), host_pool=z((B, H_kv, NB, 2, bs, D), bf16),
                ws_pool=z((B, H_kv, S, 2, bs, D), bf16), tbl_slot=z((B, H_kv, K_b), i32),
                tbl_block=z((B, H_kv, K_b), i32), tbl_n=z((B, H_kv), i32), plan=z((1000,), i32), stream=0,
                stats_accum=z((4,), i64))


def mass_args():
    return dict(q=z((B, H_q, D), bf16), kv_pool=z((B, H_kv, NB, 2, bs, D), bf16), ctx_len=z((B,), i32),
                mass=z((B, H_kv, NB), f32), ws=z((64,), torch.uint8))


def overlap_args():
    return dict(sel_a=z((B, H_kv, K_b), i32), n_a=z((B, H_kv), i32), sel_b=z((B, H_kv, K_b), i32),
                n_b=z((B, H_kv), i32), out=z((B, H_kv), i32))


def append_args():
    return dict(k_new=z((B, H_kv, D), bf16), v_new=z((B, H_kv, D), bf16), ctx_len=z((B,), i32),
                kminmax=z((B, H_kv, NB, 2, D), bf16), pool=z((B, H_kv, NB, 2, bs, D), bf16),
                ws_pool=z((B, H_kv, S, 2, bs, D), bf16), slot_block=z((B, H_kv, S), i32))


CALLS = {
    "score": (binding.oasis_score_blocks, score_args, "oasis_score_blocks"),
    "topk": (binding.oasis_select_topk, topk_args, "oasis_select_topk"),
    "attn": (binding.oasis_sparse_decode_attn, attn_args, "oasis_sparse_decode_attn"),
    "lookahead": (binding.oasis_lookahead_attn, lookahead_args, "oasis_lookahead_attn"),
    "stage": (binding.oasis_stage_blocks, stage_args, "oasis_stage_blocks"),
    "mass": (binding.oasis_block_attention_mass, mass_args, "oasis_block_attention_mass"),
    "overlap": (binding.oasis_topk_overlap, overlap_args, "oasis_topk_overlap"),
    "append": (binding.oasis_append_kv, append_args, "oasis_append_kv"),
}

MISMATCHES = [
    ("score", "kminmax", ((B + 1, H_kv, NB, 2, D), bf16)),
    ("score", "kminmax", ((B, H_kv, NB, 2, 64), bf16)),
    ("score", "ctx_len", ((B + 1,), i32)),
    ("score", "scores", ((B, H_kv, NB - 1), f32)),
    ("score", "q_look", ((B, 1, 7, D), bf16)),          # H_q not a multiple of H_kv
    ("topk", "sel", ((B, H_kv, K_b + 1), i32)),
    ("topk", "n_sel", ((B, H_kv + 1), i32)),
    ("topk", "ctx_len", ((B + 1,), i32)),
    ("attn", "kv_pool", ((B + 1, H_kv, S, 2, bs, D), bf16)),
    ("attn", "tbl_block", ((B, H_kv, T - 1), i32)),
    ("attn", "tbl_n", ((B, H_kv + 1), i32)),
    ("attn", "ctx_len", ((B - 1,), i32)),
    ("attn", "out", ((B, H_q, D - 1), bf16)),
    ("attn", "lse", ((B, H_q + 1), f32)),
    ("attn", "q", ((B, 7, D), bf16)),                   # H_q not a multiple of H_kv
    ("lookahead", "out", ((B, 1, H_q, D), bf16)),
    ("lookahead", "lse", ((B, 2, H_q - 1), f32)),
    ("lookahead", "kv_pool", ((B, H_kv, S, 2, bs, D - 8), bf16)),
    ("stage", "ws_pool", ((B, H_kv, S, 2, bs, D - 8), bf16)),
    ("stage", "ws_pool", ((B + 1, H_kv, S, 2, bs, D), bf16)),
    ("stage", "ctx_len", ((B + 1,), i32)),
    ("stage", "n_sel", ((B, H_kv + 1), i32)),
    ("stage", "tbl_n", ((B + 1, H_kv), i32)),
    ("stage", "slot_stamp", ((B, H_kv, S + 1), i32)),
    ("stage", "sel", ((B + 1, H_kv, K_b), i32)),
    ("stage", "scores", ((B, H_kv, NB + 1), f32)),
    ("stage", "tbl_slot", ((B, H_kv, K_b + 1), i32)),
    ("stage", "stats_accum", ((3,), i64)),
    ("mass", "kv_pool", ((B + 1, H_kv, NB, 2, bs, D), bf16)),
    ("mass", "mass", ((B, H_kv, NB - 1), f32)),
    ("mass", "ctx_len", ((B + 1,), i32)),
    ("overlap", "n_b", ((B, H_kv + 1), i32)),
    ("overlap", "out", ((B + 1, H_kv), i32)),
    ("overlap", "sel_b", ((B, H_kv, K_b - 1), i32)),
    ("append", "slot_block", ((B, H_kv, S - 1), i32)),
    ("append", "ws_pool", ((B, H_kv, S, 2, bs, D - 8), bf16)),
    ("append", "slot_block", None),                      # a working set without its slot table
]


@pytest.mark.parametrize("call", sorted(CALLS))
def test_matching_shapes_reach_the_library(lib, call):
    fn, args, entry = CALLS[call]
    kw = args()
    if call not in ("stage",):
        kw["stream"] = 0
    fn(**kw)
    assert entry in lib.calls


@pytest.mark.parametrize("call,arg,bad", MISMATCHES)
def test_mismatch_raises_before_any_launch(lib, call, arg, bad):
    fn, args, entry = CALLS[call]
    kw = args()
    if call not in ("stage",):
        kw["stream"] = 0
    kw[arg] = None if bad is None else z(*bad)
    with pytest.raises(ValueError):
        fn(**kw)
    assert entry not in lib.calls


def test_stage_stats_struct_round_trip():
    st = binding.oasis_stage_stats(admits=3, evictions=2, deferred=5, capped_pairs=1, bytes=3 * 8192)
    assert st.as_dict() == {"admits": 3, "evictions": 2, "deferred": 5, "capped_pairs": 1, "bytes": 24576}
