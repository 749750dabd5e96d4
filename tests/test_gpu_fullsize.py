"""Full-size parity: every output and every final state of the decode and
prefill workloads against the float64 oracle, in the launch configuration
the benchmark times (plans: metadata validated and uploaded once).

* decode: a 1024-slot pool, 256 random ids in random order, H=32, bf16
  inputs, 100 consecutive steps; the oracle carries its own state from the
  initial states through all 100 steps (never re-seeded from the device);
  every step's outputs are compared, and the states after steps 1, 50 and 100;
* prefill: 8 sequences of 4096 tokens, H=32, zero start, bf16 inputs and
  fp32 inputs (the precise plan): every (sequence, head) pair's outputs and
  final state;
* large pool: 4096 slots, H=64: a decode step over 1024 slots and 32 fresh
  prefills with lengths uniform in [128, 8192], every slot and every head.

The oracle here is the plain-C float64 one (oracle/wkv7_ref.c, pinned by the
same pins as the numpy oracle), run on worker threads. The metric is max
|err| / rms over every compared element of a workload (tests/parity.py); the
worst single (sequence, head) part is printed too. Bars: 2e-2 for bf16
inputs, 1e-3 for fp32 inputs; tighter guards record what each kernel
reaches.
"""
import numpy as np
import pytest
import torch

import wkv7_inputs as G
from linear_attention_rnn_amd import wkv7 as W
from oracle import wkv7_cref as C
from tests.gpu_util import DEV, say, set_states, get_states
from tests.parity import ParityMeter, report

pytestmark = pytest.mark.gpu

BAR = 2e-2           # bf16-input workloads
BAR_F32 = 1e-3       # fp32-input workloads
SEQ_GUARD = 1e-5     # the sequential kernel: fp32 FMAs, rounding only
CHUNK_GUARD = 1e-2   # the chunked kernel's fast plan (bf16 inputs)
PRECISE_GUARD = 5e-4  # its precise plan (fp32 inputs)
N = 64


def _bits_equal(a, b):
    return torch.equal(a.contiguous().view(torch.int32),
                       b.contiguous().view(torch.int32))


def _report(*meters):
    for m in meters:
        say("  " + m.summary())
        report(m.summary())


def test_decode_100_chained_steps():
    wl = G.cfg_decode(seed=1)
    ids, H = wl.batch.slot_ids, wl.H
    B = len(ids)
    steps = 100
    say(f"decode {wl.name}: {B} ids x H={H}, {steps} chained steps")
    xs = [G.decode_step_inputs(1, s, ids, H, N) for s in range(steps)]
    xdev = [{n: x.inputs[n].to(DEV) for n in G.NAMES} for x in xs]
    o_dev = torch.empty((steps, B, H, N), dtype=torch.float32, device=DEV)
    check_at = (1, 50, 100)
    snaps = {s: torch.empty((B, H, N, N), dtype=torch.float32,
                            pin_memory=True) for s in check_at}
    pool = W.wkv7_pool_create(wl.n_slots, H, N)
    try:
        rng = np.random.default_rng(99)
        others = np.setdiff1d(np.arange(wl.n_slots), ids).astype(np.int32)
        other_states = G.draw_states(rng, len(others), H, N, std=1.0)
        set_states(pool, others, other_states)
        set_states(pool, ids, wl.init_states)
        cu = np.arange(B + 1, dtype=np.int32)
        plan = W.wkv7_plan_create(pool, ids, cu)
        try:
            for s in range(steps):
                x = xdev[s]
                W.wkv7_forward_plan(pool, plan, x["r"], x["w"], x["k"],
                                    x["v"], x["a"], x["b"], o_dev[s])
                if s + 1 in snaps:          # stream-ordered copy of the slots
                    W.wkv7_hibernate(pool, ids, snaps[s + 1])
            torch.cuda.synchronize()
        finally:
            W.wkv7_plan_destroy(plan)
        after = get_states(pool, others)
    finally:
        W.wkv7_pool_destroy(pool)
    assert _bits_equal(after, other_states), "inactive slots changed"

    m_o, m_s = ParityMeter("decode o, 100 steps"), ParityMeter("decode S")
    S = np.ascontiguousarray(G.as_f64(wl.init_states).reshape(B * H, N, N))
    o_host = o_dev.cpu()
    for s in range(steps):
        o_ref = C.run_heads(S, xs[s].inputs, 1, B * H, N)
        e = m_o.add(o_host[s], o_ref.reshape(B, H, N), where=f"step {s + 1}")
        if s + 1 in snaps:
            es = m_s.add(snaps[s + 1], S.reshape(B, H, N, N),
                         where=f"step {s + 1}")
            say(f"  step {s + 1}: o err {e:.3e}  S err {es:.3e}")
    _report(m_o, m_s)
    assert m_o.value() < BAR and m_s.value() < BAR
    assert m_o.value() < SEQ_GUARD and m_s.value() < SEQ_GUARD


@pytest.mark.parametrize("dtype", [G.BF16, G.F32])
def test_prefill_all_pairs(dtype):
    wl = G.cfg_prefill(seed=2, dtype=dtype)
    b, H = wl.batch, wl.H
    say(f"prefill {wl.name}: T_tot={b.T_tot}, every (sequence, head) pair")
    x = {n: b.inputs[n].to(DEV) for n in G.NAMES}
    o = torch.full((b.T_tot, H, N), float("nan"), dtype=torch.float32,
                   device=DEV)
    pool = W.wkv7_pool_create(wl.n_slots, H, N)
    try:
        plan = W.wkv7_plan_create(pool, b.slot_ids, b.cu_seqlens)
        try:
            W.wkv7_forward_plan(pool, plan, x["r"], x["w"], x["k"], x["v"],
                                x["a"], x["b"], o)
            torch.cuda.synchronize()
        finally:
            W.wkv7_plan_destroy(plan)
        S = get_states(pool, b.slot_ids)
    finally:
        W.wkv7_pool_destroy(pool)
    o = o.cpu()
    m_o = ParityMeter(f"prefill 8 x 4096 ({dtype} inputs) o")
    m_s = ParityMeter(f"prefill 8 x 4096 ({dtype} inputs) S")
    for s in range(len(b.slot_ids)):
        lo, hi = int(b.cu_seqlens[s]), int(b.cu_seqlens[s + 1])
        S_ref = np.zeros((H, N, N))
        o_ref = C.run_heads(S_ref, {n: b.inputs[n][lo:hi] for n in G.NAMES},
                            hi - lo, H, N)
        for h in range(H):
            m_o.add(o[lo:hi, h], o_ref[:, h], where=(s, h))
            m_s.add(S[s, h], S_ref[h], where=(s, h))
    _report(m_o, m_s)
    assert m_o.count == b.T_tot * H * N and m_s.count == 8 * H * N * N
    bar, guard = (BAR, CHUNK_GUARD) if dtype == G.BF16 else (BAR_F32, PRECISE_GUARD)
    assert m_o.value() < bar and m_s.value() < bar
    assert m_o.worst_part < guard and m_s.worst_part < guard


def test_large_pool_every_slot_and_head():
    n_slots, H, seed = 4096, 64, 4
    rng = np.random.default_rng(seed)
    perm = rng.permutation(n_slots).astype(np.int32)
    dec_ids, pre_ids = perm[:1024], perm[1024:1056]
    lens = np.random.default_rng(seed).integers(128, 8193, size=32)
    T = int(lens.sum())
    say(f"large pool: 4096 x H=64; decode 1024 slots; 32 prefills, "
        f"{T} tokens")
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    pool = W.wkv7_pool_create(n_slots, H, N)
    try:
        init = torch.randn((1024, H, N, N), device=DEV, generator=gen) * 0.1
        W.wkv7_resume(pool, dec_ids, init)
        xd = G.draw_tokens_device(gen, 1024, H, N, G.BF16, DEV)
        od = torch.empty((1024, H, N), dtype=torch.float32, device=DEV)
        xp = G.draw_tokens_device(gen, T, H, N, G.BF16, DEV)
        op = torch.full((T, H, N), float("nan"), dtype=torch.float32,
                        device=DEV)
        cu_d = np.arange(1025, dtype=np.int32)
        cu_p = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        W.wkv7_reset(pool, pre_ids)
        plan_d = W.wkv7_plan_create(pool, dec_ids, cu_d)
        plan_p = W.wkv7_plan_create(pool, pre_ids, cu_p)
        try:
            W.wkv7_forward_plan(pool, plan_d, xd["r"], xd["w"], xd["k"],
                                xd["v"], xd["a"], xd["b"], od)
            W.wkv7_forward_plan(pool, plan_p, xp["r"], xp["w"], xp["k"],
                                xp["v"], xp["a"], xp["b"], op)
            torch.cuda.synchronize()
        finally:
            W.wkv7_plan_destroy(plan_d)
            W.wkv7_plan_destroy(plan_p)
        S_dec = get_states(pool, dec_ids)
        S_pre = get_states(pool, pre_ids)
        init_h = init.cpu()
        del init
    finally:
        W.wkv7_pool_destroy(pool)

    # decode: all 1024 slots x 64 heads
    m_do, m_ds = ParityMeter("4096-slot pool, decode o"), ParityMeter("4096-slot pool, decode S")
    S = np.ascontiguousarray(init_h.double().numpy().reshape(1024 * H, N, N))
    o_ref = C.run_heads(S, {n: xd[n].cpu() for n in G.NAMES}, 1, 1024 * H, N)
    m_do.add(od.cpu(), o_ref.reshape(1024, H, N), where="decode")
    m_ds.add(S_dec, S.reshape(1024, H, N, N), where="decode")
    _report(m_do, m_ds)
    assert m_do.value() < BAR and m_ds.value() < BAR
    assert m_do.value() < SEQ_GUARD and m_ds.value() < SEQ_GUARD

    # prefill: every sequence and head, one sequence at a time
    m_po, m_ps = ParityMeter("4096-slot pool, ragged prefill o"), ParityMeter("4096-slot pool, ragged prefill S")
    for s in range(32):
        lo, hi = int(cu_p[s]), int(cu_p[s + 1])
        S_ref = np.zeros((H, N, N))
        x = {n: xp[n][lo:hi].cpu() for n in G.NAMES}
        o_ref = C.run_heads(S_ref, x, hi - lo, H, N)
        o_got = op[lo:hi].cpu()
        for h in range(H):
            m_po.add(o_got[:, h], o_ref[:, h], where=(s, hi - lo, h))
            m_ps.add(S_pre[s, h], S_ref[h], where=(s, hi - lo, h))
    _report(m_po, m_ps)
    assert m_po.count == T * H * N
    assert m_po.value() < BAR and m_ps.value() < BAR
    assert m_po.worst_part < CHUNK_GUARD and m_ps.worst_part < CHUNK_GUARD
