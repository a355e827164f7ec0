"""The C ABI library loads, exports every declared entry point, and rejects bad
arguments on the host (no device work is enqueued, so no GPU is needed)."""
import ctypes
import os
import re

import pytest

import prefetch_block_scoring_amd as oa
from prefetch_block_scoring_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "oasis.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(oasis_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported_and_bound():
    names = declared_functions()
    assert len(names) >= 12
    lib = ctypes.CDLL(binding.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
        assert n in binding._SIGNATURES, n


def test_version_and_cap_mapping():
    assert oa.oasis_version().startswith("oasis")
    assert oa.oasis_fetch_cap_blocks(0.05, 128) == 6
    assert oa.oasis_fetch_cap_blocks(0.01, 128) == 1
    assert oa.oasis_fetch_cap_blocks(1.0, 128) == 128
    assert oa.oasis_fetch_cap_blocks(0.0, 128) == 0
    assert oa.oasis_fetch_cap_blocks(float("nan"), 128) == 0
    assert oa.oasis_fetch_cap_blocks(0.5, 0) == -1


def test_fetch_cap_matches_oracle_over_a_sweep():
    import oracle
    for K_b in (1, 7, 32, 128, 1000):
        for cap in (0.0, 1e-6, 0.01, 0.05, 0.1, 0.333, 0.5, 0.99, 1.0, 2.0):
            assert oa.oasis_fetch_cap_blocks(cap, K_b) == oracle.fetch_cap_blocks(cap, K_b)


L = binding.library()
NULL = None


def d(**kw):
    base = dict(B=2, H_q=8, H_kv=2, D=128, bs=16, NB_max=64)
    base.update(kw)
    return binding.oasis_dims(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(D=64), oa.OASIS_EUNSUPPORTED),
    (dict(bs=32), oa.OASIS_EUNSUPPORTED),
    (dict(H_q=6, H_kv=4), oa.OASIS_EINVAL),
    (dict(H_q=64, H_kv=2), oa.OASIS_EUNSUPPORTED),
    (dict(NB_max=0), oa.OASIS_EINVAL),
    (dict(NB_max=1 << 20), oa.OASIS_EUNSUPPORTED),
    (dict(B=-1), oa.OASIS_EINVAL),
])
def test_bad_dims_rejected_by_every_call(kw, code):
    dd = d(**kw)
    p = ctypes.c_void_p(16)
    assert L.oasis_build_summaries(ctypes.byref(dd), p, p, p, NULL) == code
    assert L.oasis_score_blocks(ctypes.byref(dd), p, 1, p, p, p, NULL) == code
    assert L.oasis_select_topk(ctypes.byref(dd), p, p, 8, p, p, NULL) == code
    assert L.oasis_sparse_decode_attn(ctypes.byref(dd), p, p, 4, p, p, p, 4, p, 0.1, p, p, p, 1 << 30, 1,
                                      NULL) == code
    assert oa.oasis_last_error() != ""


def test_null_pointers_and_bad_values():
    dd = d()
    p = ctypes.c_void_p(16)
    assert L.oasis_score_blocks(None, p, 1, p, p, p, NULL) == oa.OASIS_EINVAL
    assert L.oasis_score_blocks(ctypes.byref(dd), NULL, 1, p, p, p, NULL) == oa.OASIS_EINVAL
    assert "q_look" in oa.oasis_last_error()
    assert L.oasis_score_blocks(ctypes.byref(dd), p, 0, p, p, p, NULL) == oa.OASIS_EINVAL
    assert L.oasis_select_topk(ctypes.byref(dd), p, p, 0, p, p, NULL) == oa.OASIS_EINVAL
    assert L.oasis_select_topk(ctypes.byref(dd), p, NULL, 4, p, p, NULL) == oa.OASIS_EINVAL
    assert L.oasis_build_summaries(ctypes.byref(dd), p, p, NULL, NULL) == oa.OASIS_EINVAL
    # attention: P < 1, T < 0, n_split out of range, NaN scale, missing table
    att = L.oasis_sparse_decode_attn
    assert att(ctypes.byref(dd), p, p, 0, p, p, p, 4, p, 0.1, p, p, p, 0, 1, NULL) == oa.OASIS_EINVAL
    assert att(ctypes.byref(dd), p, p, 4, p, p, p, -1, p, 0.1, p, p, p, 0, 1, NULL) == oa.OASIS_EINVAL
    assert att(ctypes.byref(dd), p, p, 4, p, p, p, 4, p, 0.1, p, p, p, 0, 65, NULL) == oa.OASIS_EINVAL
    assert att(ctypes.byref(dd), p, p, 4, p, p, p, 4, p, float("nan"), p, p, p, 0, 1, NULL) == oa.OASIS_EINVAL
    assert att(ctypes.byref(dd), p, p, 4, NULL, p, p, 4, p, 0.1, p, p, p, 0, 1, NULL) == oa.OASIS_EINVAL
    # workspace too small for an explicit split
    need = L.oasis_attn_workspace_bytes(ctypes.byref(dd), 64, 4)
    assert need == 2 * 8 * 4 * 130 * 4
    assert att(ctypes.byref(dd), p, p, 64, p, p, p, 64, p, 0.1, p, p, p, need - 4, 4, NULL) == oa.OASIS_ENOSPACE
    assert att(ctypes.byref(dd), p, p, 64, p, p, p, 64, p, 0.1, p, p, NULL, need, 4, NULL) == oa.OASIS_EINVAL


def test_empty_batch_is_a_no_op():
    dd = d(B=0)
    assert L.oasis_score_blocks(ctypes.byref(dd), NULL, 1, NULL, NULL, NULL, NULL) == oa.OASIS_OK
    assert L.oasis_select_topk(ctypes.byref(dd), NULL, NULL, 4, NULL, NULL, NULL) == oa.OASIS_OK
    assert L.oasis_sparse_decode_attn(ctypes.byref(dd), NULL, NULL, 4, NULL, NULL, NULL, 4, NULL, 0.1,
                                      NULL, NULL, NULL, 0, 1, NULL) == oa.OASIS_OK


def stage_args(**kw):
    a = binding.oasis_stage_args()
    p = 16
    for f in ("sel", "n_sel", "scores", "slot_block", "slot_stamp", "ctx_len", "host_pool", "ws_pool",
              "tbl_slot", "tbl_block", "tbl_n", "plan"):
        setattr(a, f, p)
    a.K_sel, a.K_b, a.C, a.S, a.step = 8, 8, 2, 10, 0
    a.plan_bytes = 1 << 20
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,code", [
    (dict(C=-1), oa.OASIS_EINVAL),
    (dict(C=9), oa.OASIS_EINVAL),
    (dict(S=7), oa.OASIS_EINVAL),
    (dict(K_b=0), oa.OASIS_EINVAL),
    (dict(step=-1), oa.OASIS_EINVAL),
    (dict(copy_mode=7), oa.OASIS_EINVAL),
    (dict(S=5000), oa.OASIS_EUNSUPPORTED),
    (dict(K_sel=2000), oa.OASIS_EUNSUPPORTED),
    (dict(plan=None), oa.OASIS_EINVAL),
    (dict(host_pool=None), oa.OASIS_EINVAL),
    (dict(plan_bytes=4), oa.OASIS_ENOSPACE),
    (dict(copy_mode=1, host_plan=None, stage_host=16, stage_dev=16), oa.OASIS_EINVAL),
    (dict(copy_mode=1, host_plan=16, stage_host=None, stage_dev=16), oa.OASIS_EINVAL),
    (dict(copy_mode=1, host_plan=16, stage_host=16, stage_dev=16, host_plan_bytes=8,
          stage_host_bytes=1 << 20, stage_dev_bytes=1 << 20), oa.OASIS_ENOSPACE),
    (dict(copy_mode=1, host_plan=16, stage_host=16, stage_dev=16, host_plan_bytes=1 << 20,
          stage_host_bytes=8191, stage_dev_bytes=1 << 20), oa.OASIS_ENOSPACE),
    (dict(copy_mode=1, host_plan=16, stage_host=16, stage_dev=16, host_plan_bytes=1 << 20,
          stage_host_bytes=1 << 20, stage_dev_bytes=1 << 20, host_threads=-1), oa.OASIS_EINVAL),
])
def test_stage_argument_errors(kw, code):
    dd = d()
    a = stage_args(**kw)
    st = binding.oasis_stage_stats(admits=7)
    assert L.oasis_stage_blocks(ctypes.byref(dd), ctypes.byref(a), ctypes.byref(st)) == code
    assert oa.oasis_last_error() != ""
    assert L.oasis_stage_blocks(ctypes.byref(dd), ctypes.byref(a), None) == code


def test_plan_and_staging_sizes():
    dd = d(B=3, H_kv=2)
    assert L.oasis_stage_plan_bytes(ctypes.byref(dd), 6) == 4 * (3 * 2 * (4 + 12) + 4)
    assert L.oasis_stage_plan_bytes(ctypes.byref(dd), 0) == 4 * (3 * 2 * 6 + 4)
    assert L.oasis_stage_buffer_bytes(ctypes.byref(dd), 7) == 7 * 8192
    assert oa.oasis_stage_buffer_bytes(3) == 3 * 8192


def _pipeline_desc(L=2, staged=1, copy_mode=0, **kw):
    """A pipeline description whose buffers are fake non-NULL addresses:
    every case below is rejected by the host checks before any pointer is
    used or any device call is made."""
    bufs = (binding.oasis_layer_buffers * L)()
    fake = 0x1000
    for b in bufs:
        b.scores = fake
        for k in range(2):
            b.sel[k] = b.n_sel[k] = b.plan[k] = b.stage_host[k] = fake
        for k in range(3):
            b.tbl_slot[k] = b.tbl_block[k] = b.tbl_n[k] = fake
        b.attn_ws, b.attn_ws_bytes = fake, 1 << 30
        b.ws_pool = b.slot_block = b.slot_stamp = b.host_plan = b.stage_dev = fake
        b.plan_bytes = 1 << 30
        b.stage_bytes = 1 << 20
    d = binding.oasis_pipeline_desc(n_layers=L, K_b=128, C=6, J=1, n_q=1, staged=staged, copy_mode=copy_mode,
                                    host_threads=0, n_split=0, sm_scale=0.088, pool=fake, kminmax=fake,
                                    ctx_len=fake, main_stream=None,
                                    layers=ctypes.cast(bufs, ctypes.POINTER(binding.oasis_layer_buffers)))
    for k, v in kw.items():
        setattr(d, k, v)
    return d, bufs


@pytest.mark.parametrize("change,code", [
    ({"n_layers": 0}, oa.OASIS_EINVAL),
    ({"K_b": 0}, oa.OASIS_EINVAL),
    ({"J": 0}, oa.OASIS_EINVAL),
    ({"C": 129}, oa.OASIS_EINVAL),
    ({"copy_mode": 7}, oa.OASIS_EINVAL),
    ({"staged": 2}, oa.OASIS_EINVAL),
    ({"pool": None}, oa.OASIS_EINVAL),
    ({"n_split": 65}, oa.OASIS_EINVAL),
    ({"compute_streams": 3}, oa.OASIS_EINVAL),
    ({"compute_streams": -2}, oa.OASIS_EINVAL),
    ({"issue_threads": 2}, oa.OASIS_EINVAL),
    ({"issue_threads": -2}, oa.OASIS_EINVAL),
    ({"n_q": 0}, oa.OASIS_EINVAL),
    ({"n_q": 5}, oa.OASIS_EUNSUPPORTED),     # 5 queries x 4 heads > 16 columns
])
def test_pipeline_create_rejects_bad_descriptions(change, code):
    d, bufs = _pipeline_desc(**change)
    with pytest.raises(oa.OasisError) as e:
        oa.oasis_pipeline_create(oa.dims(4, 32, 8, 1024), d)
    assert e.value.code == code


@pytest.mark.parametrize("field,code", [("ws_pool", oa.OASIS_EINVAL), ("plan_bytes", oa.OASIS_ENOSPACE),
                                        ("attn_ws_bytes", oa.OASIS_ENOSPACE), ("stage_dev", oa.OASIS_EINVAL)])
def test_pipeline_create_rejects_bad_layer_buffers(field, code):
    d, bufs = _pipeline_desc(copy_mode=oa.OASIS_COPY_DMA)
    setattr(bufs[1], field, 0 if "bytes" in field else None)
    with pytest.raises(oa.OasisError) as e:
        # n_split = 4 needs an attention workspace, so its size is checked
        d.n_split = 4
        oa.oasis_pipeline_create(oa.dims(4, 32, 8, 1024), d)
    assert e.value.code == code
    assert "layer 1" in oa.oasis_last_error()


def test_pipeline_calls_reject_null_handles():
    lib = binding.library()
    assert lib.oasis_pipeline_layer_step(None, 0, 0, None, None, None, None) == oa.OASIS_EINVAL
    assert lib.oasis_pipeline_drain(None) == oa.OASIS_EINVAL
    assert lib.oasis_pipeline_timing(None, 4, 1, 1) == oa.OASIS_EINVAL
    assert lib.oasis_pipeline_issue_threads(None, None) == oa.OASIS_EINVAL
    assert lib.oasis_pipeline_destroy(None) == oa.OASIS_OK


def test_lookahead_attention_argument_errors():
    lib = binding.library()
    d = oa.dims(2, 32, 8, 64)     # G = 4
    call = lambda n_q, n_split=0: lib.oasis_lookahead_attn(ctypes.byref(d), n_q, None, None, 8, None, None, None, 4,
                                                           None, 0.1, None, None, None, 0, n_split, None)
    assert call(0) == oa.OASIS_EINVAL
    assert call(5) == oa.OASIS_EUNSUPPORTED      # 5 * 4 = 20 columns > 16
    assert call(4, n_split=65) == oa.OASIS_EINVAL
    assert call(4) == oa.OASIS_EINVAL            # then the NULL pointers
    assert oa.oasis_lookahead_attn_workspace_bytes(2, 32, 8, 3, 128, 3) == 2 * 3 * 32 * 3 * 130 * 4
    assert oa.oasis_lookahead_attn_workspace_bytes(2, 32, 8, 1, 128, 3) == oa.oasis_attn_workspace_bytes(
        2, 32, 8, 128, 3)


def test_mixed_copy_mode_needs_dma_buffers_on_even_layers_only():
    """OASIS_COPY_MIXED stages even layers through the DMA engine: their
    host staging buffers are required, the odd layers' are not."""
    d, bufs = _pipeline_desc(L=3, copy_mode=oa.OASIS_COPY_MIXED)
    bufs[0].stage_dev = None
    with pytest.raises(oa.OasisError) as e:
        oa.oasis_pipeline_create(oa.dims(4, 32, 8, 1024), d)
    assert e.value.code == oa.OASIS_EINVAL
    assert "layer 0" in oa.oasis_last_error()
    # an odd layer without them passes the buffer checks: the description
    # is then refused for the next layer that needs them (layer 2)
    d, bufs = _pipeline_desc(L=3, copy_mode=oa.OASIS_COPY_MIXED)
    bufs[1].stage_dev = None
    bufs[1].host_plan = None
    bufs[2].stage_dev = None
    with pytest.raises(oa.OasisError) as e:
        oa.oasis_pipeline_create(oa.dims(4, 32, 8, 1024), d)
    assert e.value.code == oa.OASIS_EINVAL
    assert "layer 2" in oa.oasis_last_error()


def test_timing_values_rejects_bad_arguments():
    lib = binding.library()
    n = ctypes.c_int32()
    assert lib.oasis_pipeline_timing_values(None, 0, None, 0, ctypes.byref(n)) == oa.OASIS_EINVAL


def test_static_attention_scratch_limit_is_checked_on_the_host():
    """The allocation-free attention entry point refuses split-K partials
    larger than its fixed scratch before any device call (fake pointers are
    never dereferenced)."""
    assert L.oasis_sparse_decode_attn_static_bytes() == 8 << 20
    dd = d(B=512, H_q=64, H_kv=4, NB_max=64)
    p = ctypes.c_void_p(16)
    assert L.oasis_sparse_decode_attn_static(ctypes.byref(dd), p, p, 64, p, p, p, 128, p, 0.1, p, None, 16,
                                             None) == oa.OASIS_ENOSPACE
    assert "fixed scratch" in oa.oasis_last_error()
    assert L.oasis_sparse_decode_attn_static(ctypes.byref(dd), p, p, 0, p, p, p, 128, p, 0.1, p, None, 16,
                                             None) == oa.OASIS_EINVAL


def test_attention_launch_shape_rule():
    """The attention launch shape (host logic; 256 compute units, as MI355X
    has and as the library assumes where no GPU answers): one split of
    four-wave workgroups with enough (request, KV head) pairs, else splits
    of eight-wave workgroups (four past eight query columns) with at least
    four table entries per wave (two with four waves); an explicit split
    count keeps its splits and the waves follow."""
    shape = oa.oasis_attn_launch_shape
    assert shape(128, 32, 8, 1, 128) == (1, 4)    # 1024 pairs
    assert shape(64, 32, 8, 1, 128) == (1, 4)     # 512 pairs
    assert shape(32, 32, 8, 1, 128) == (1, 8)     # 256 pairs
    assert shape(16, 64, 8, 1, 128) == (2, 8)     # 128 pairs: 2 splits of eight waves fill the machine
    assert shape(32, 32, 8, 3, 128) == (2, 4)     # 12 columns: attn_pv_kernel, four waves
    assert shape(1, 8, 2, 1, 32) == (1, 8)        # 2 pairs, 32 entries: one split, four per wave
    assert shape(1, 8, 2, 1, 64) == (2, 8)        # 64 entries: two splits of four per wave
    assert shape(1, 8, 2, 2, 32) == (1, 8)        # 8 columns: still the VALU kernel
    assert shape(1, 8, 2, 3, 32) == (4, 4)        # 12 columns: attn_pv_kernel, two entries per wave
    assert shape(1, 8, 2, 1, 8) == (1, 4)         # 8 entries: one split, four waves
    assert shape(32, 32, 8, 1, 128, 1) == (1, 8)
    assert shape(32, 32, 8, 1, 128, 2) == (2, 4)
    assert shape(16, 64, 8, 1, 128, 2) == (2, 8)
    assert shape(128, 32, 8, 1, 128, 1) == (1, 4)
    for B in (1, 7, 32, 128):
        sp, _ = shape(B, 32, 8, 1, 128)
        assert sp == oa.oasis_attn_num_splits(B, 32, 8, 128)
    with pytest.raises(oa.OasisError):
        shape(32, 32, 8, 0, 128)
    with pytest.raises(oa.OasisError):
        shape(32, 64, 8, 3, 128)  # 24 query columns
    assert binding.library().oasis_attn_launch_shape(None, 1, 128, 0, None, None) == oa.OASIS_EINVAL
