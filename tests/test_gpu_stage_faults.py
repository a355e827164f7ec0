"""Staging when a step does not go as planned (OasisKV, paperlayer summary,
section 3: a block that misses its transfer either costs attention context or
a fetch on the critical path).  Every condition is forced from the host; no
kernel is made to fault.

  - a pageable (not pinned) host pool is refused with OASIS_EINVAL before
    anything is enqueued: the slot table and the attention table stay as
    they were;
  - a step whose plan ran but whose copy was held back: the previous
    attention table still holds exactly the previous resident set (admits
    only go to slots that were free before the step, evicted slots are not
    refilled until the next step), so attention over it equals the oracle's
    attention over that set; the slot stamps already equal the oracle's
    after the step; issuing the copy late completes the step;
  - a step dropped entirely (no plan, no copy) on both sides: the states
    stay equal and the next step proceeds from them.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from helpers import assert_attn_close, bf16_to_f64, gpu_stage_state, u16

pytestmark = pytest.mark.gpu

DEV = "cuda"


def oa():
    import prefetch_block_scoring_amd as m
    return m


class Staged:
    """GPU buffers of one small staged layer, three rotating tables."""

    def __init__(self, C=3, copy_mode=0, turnover=8, steps=8, seed=41):
        m = oa()
        self.w = w = wl.Workload("faults", B=2, H_q=8, H_kv=2, ctx=(1500, 3000), budget=512, J=1,
                                 structure="none", seed=seed)
        self.C, self.K_b, self.S, self.copy_mode = C, w.K_b, w.K_b + C, copy_mode
        self.ctx_cpu = wl.context_lengths(w)
        self.ctx = self.ctx_cpu.to(DEV)
        self.kv_cpu = wl.kv_pool(w)
        self.host = m.oasis_host_empty((w.B, w.H_kv, w.NB_max, 2, w.bs, w.D))
        self.host.copy_(self.kv_cpu)
        self.host_np = u16(self.host)
        self.sels, self.nsels, self.scores = wl.predicted_set_sequence(w, steps, turnover)
        i32 = torch.int32
        self.slot_block = torch.full((w.B, w.H_kv, self.S), -1, dtype=i32, device=DEV)
        self.slot_stamp = torch.full_like(self.slot_block, -1)
        self.ws = torch.zeros((w.B, w.H_kv, self.S, 2, w.bs, w.D), dtype=torch.bfloat16, device=DEV)
        self.tabs = [(torch.full((w.B, w.H_kv, self.K_b), -1, dtype=i32, device=DEV),
                      torch.full((w.B, w.H_kv, self.K_b), -1, dtype=i32, device=DEV),
                      torch.zeros((w.B, w.H_kv), dtype=i32, device=DEV)) for _ in range(3)]
        nbytes = m.oasis_stage_plan_bytes(w.B, w.H_kv, self.K_b)
        self.plans = [torch.empty(nbytes // 4, dtype=i32, device=DEV) for _ in range(2)]
        self.host_plan = m.oasis_host_empty((nbytes // 4,), i32)
        sbytes = m.oasis_stage_buffer_bytes(w.B * w.H_kv * self.K_b)
        self.stage_host = m.oasis_host_empty((sbytes,), torch.uint8)
        self.stage_dev = torch.empty(sbytes, dtype=torch.uint8, device=DEV)
        self.state = oracle.StageState(w.B, w.H_kv, w.NB_max)

    def kw(self, s, pool=None):
        t = self.tabs[s % 3]
        return dict(sel=self.sels[s].to(DEV), n_sel=self.nsels[s].to(DEV), scores=self.scores[s].to(DEV),
                    ctx_len=self.ctx, K_b=self.K_b, C=self.K_b if s == 0 else self.C, step=s,
                    slot_block=self.slot_block, slot_stamp=self.slot_stamp,
                    host_pool=self.host if pool is None else pool, ws_pool=self.ws, tbl_slot=t[0],
                    tbl_block=t[1], tbl_n=t[2], plan=self.plans[s % 2], host_plan=self.host_plan,
                    stage_host=self.stage_host, stage_dev=self.stage_dev, copy_mode=self.copy_mode)

    def oracle_step(self, s):
        w = self.w
        oracle.stage(self.state, self.sels[s].numpy(), self.nsels[s].numpy(), self.scores[s].numpy(),
                     self.ctx_cpu.numpy(), w.bs, self.K_b, self.K_b if s == 0 else self.C, s)

    def step(self, s):
        oa().oasis_stage_blocks(**self.kw(s))
        torch.cuda.synchronize()
        self.oracle_step(s)

    def check_state(self, msg):
        got = gpu_stage_state(self.slot_block, self.slot_stamp, self.w.NB_max)
        np.testing.assert_array_equal(got, self.state.stamp, err_msg=msg)

    def attend_table(self, k, seed):
        """Attention over table k with a fresh query; returns (GPU output,
        the table's blocks and counts)."""
        w = self.w
        g = torch.Generator().manual_seed(seed)
        q = torch.randn((w.B, w.H_q, w.D), generator=g).to(torch.bfloat16)
        t = self.tabs[k]
        out = oa().oasis_sparse_decode_attn(q.to(DEV), self.ws, t[0], t[1], t[2], self.ctx)
        torch.cuda.synchronize()
        return q, u16(out), t[1].cpu().numpy(), t[2].cpu().numpy()

    def check_attention_over_resident(self, k, seed, resident):
        """Table k lists exactly `resident` (per (r, h) sorted block lists)
        and attention over it equals the oracle's over those blocks."""
        w = self.w
        q, out, blk, nblk = self.attend_table(k, seed)
        for r in range(w.B):
            for h in range(w.H_kv):
                assert sorted(blk[r, h, :nblk[r, h]].tolist()) == resident[r][h], (k, r, h)
        ref, _ = oracle.attend(u16(q), u16(self.kv_cpu), self.ctx_cpu.numpy(), blk, nblk, 1 / math.sqrt(w.D))
        assert_attn_close(bf16_to_f64(out), ref)

    def resident(self):
        return [[self.state.resident(r, h).tolist() for h in range(self.w.H_kv)] for r in range(self.w.B)]

    def check_slot_bytes(self):
        wsn = u16(self.ws)
        sb = self.slot_block.cpu().numpy()
        for r, h, i in zip(*np.nonzero(sb >= 0)):
            assert np.array_equal(wsn[r, h, i], self.host_np[r, h, sb[r, h, i]]), (r, h, i)


@pytest.mark.parametrize("split", [False, True])
def test_pageable_host_pool_is_refused_before_any_work(split):
    m = oa()
    st = Staged()
    st.step(0)
    before = (st.slot_block.cpu().clone(), st.slot_stamp.cpu().clone(), st.tabs[1][2].cpu().clone())
    pageable = torch.zeros_like(st.kv_cpu)  # ordinary CPU memory, not pinned
    assert not pageable.is_pinned()
    with pytest.raises(m.OasisError) as e:
        if split:
            m.oasis_stage_copy(**st.kw(1, pool=pageable))
        else:
            m.oasis_stage_blocks(**st.kw(1, pool=pageable))
    assert e.value.code == m.OASIS_EINVAL
    assert "host_pool" in m.oasis_last_error() or "host_pool" in str(e.value)
    torch.cuda.synchronize()
    assert torch.equal(st.slot_block.cpu(), before[0])
    assert torch.equal(st.slot_stamp.cpu(), before[1])
    assert torch.equal(st.tabs[1][2].cpu(), before[2])
    # the state is intact: the same step through the pinned pool matches the oracle
    st.step(1)
    st.check_state("after the refused call")
    st.check_slot_bytes()


@pytest.mark.parametrize("copy_mode", [0, 1])
def test_copy_held_back_keeps_previous_table_attendable(copy_mode):
    m = oa()
    st = Staged(copy_mode=copy_mode)
    for s in range(3):
        st.step(s)
    st.check_state("step 2")
    r_prev = st.resident()
    # step 3: the plan runs, the copy is held back
    planned = torch.cuda.Event()
    m.oasis_stage_plan(plan_event=planned, **st.kw(3))
    torch.cuda.synchronize()
    st.oracle_step(3)
    st.check_state("step 3, plan only")
    # the previous table (step 2's) still holds exactly R_2, whatever step 3 admitted or evicted
    st.check_attention_over_resident(2 % 3, seed=7, resident=r_prev)
    # the copy, issued late, completes the step
    m.oasis_stage_copy(plan_event=planned, **st.kw(3))
    torch.cuda.synchronize()
    st.check_slot_bytes()
    st.check_attention_over_resident(3 % 3, seed=8, resident=st.resident())
    # and the next step proceeds normally
    st.step(4)
    st.check_state("step 4")
    st.check_slot_bytes()
    st.check_attention_over_resident(4 % 3, seed=9, resident=st.resident())


@pytest.mark.parametrize("copy_mode", [0, 1])
def test_dropped_step_leaves_equal_states(copy_mode):
    st = Staged(copy_mode=copy_mode)
    st.step(0)
    st.step(1)
    r1 = st.resident()
    # step 2 is dropped on both sides: neither plan nor copy
    st.check_attention_over_resident(1 % 3, seed=11, resident=r1)
    for s in (3, 4, 5):
        st.step(s)
        st.check_state(f"step {s} after a dropped step 2")
        st.check_slot_bytes()
        st.check_attention_over_resident(s % 3, seed=12 + s, resident=st.resident())
