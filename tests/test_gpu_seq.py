"""Parity of the sequential kernel (decode and short sequences) with the
float64 oracle, on the GPU through the C ABI."""
import numpy as np
import pytest
import torch

import wkv7_inputs as G
from linear_attention_rnn_amd import wkv7 as W
from oracle import wkv7_forward as oracle_forward, wkv7_decode_batch
from tests.gpu_util import (DEV, say, set_states, get_states, run_forward,
                            rel_err, tol_for)
from tests.parity import report

pytestmark = pytest.mark.gpu

ALL_SEQUENTIAL = 1 << 30


def _pool(n, H, seq_only=False):
    p = W.wkv7_pool_create(n, H, 64)
    if seq_only:
        W.wkv7_pool_set_option(p, W.WKV7_OPT_PREFILL_MIN_LEN, ALL_SEQUENTIAL)
    return p


def _oracle(batch, states):
    return oracle_forward(states, batch.slot_ids, batch.cu_seqlens,
                          batch.inputs64(), batch.H, batch.N)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_small_config_sequential(dtype):
    """H=2, one sequence of T=64, zero state, every token sequentially."""
    say(f"small config, sequential kernel, dtype={dtype}")
    rng = np.random.default_rng(0)
    b = G.make_batch(rng, [0], [64], 2, 64, dtype)
    pool = _pool(1, 2, seq_only=True)
    try:
        o = run_forward(pool, b)
        S = get_states(pool, [0])
    finally:
        W.wkv7_pool_destroy(pool)
    o_ref, S_ref = _oracle(b, {})
    e_o, e_s = rel_err(o, o_ref), rel_err(S[0], S_ref[0])
    say(f"  o err {e_o:.3e}  S err {e_s:.3e}")
    report(f"small case (H=2, T=64, {dtype}), sequential kernel: o "
           f"{e_o:.3e}, S {e_s:.3e}")
    assert e_o < 1e-5 and e_s < 1e-5   # fp32 sequential: rounding only
    assert e_o < tol_for(dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ragged_sequential(dtype):
    """Ragged lengths incl. 0, 1, a tile edge and a ragged tail; mixed
    initial states; every sequence on the sequential kernel."""
    lens = [1, 0, 5, 63, 64, 65, 130, 2]
    H = 3
    rng = np.random.default_rng(7)
    ids = rng.permutation(20)[:len(lens)].astype(np.int32)
    say(f"ragged sequential dtype={dtype} lens={lens} ids={ids.tolist()}")
    b = G.make_batch(rng, ids, lens, H, 64, dtype)
    init = G.draw_states(rng, len(ids), H, 64)
    pool = _pool(20, H, seq_only=True)
    try:
        set_states(pool, ids, init)
        o = run_forward(pool, b)
        S = get_states(pool, ids)
    finally:
        W.wkv7_pool_destroy(pool)
    states = {int(i): G.as_f64(init[n]) for n, i in enumerate(ids)}
    o_ref, S_ref = _oracle(b, states)
    e_o = rel_err(o, o_ref)
    e_s = max(rel_err(S[n], S_ref[int(i)]) for n, i in enumerate(ids))
    say(f"  o err {e_o:.3e}  S err {e_s:.3e}")
    assert e_o < 1e-5 and e_s < 1e-5


def test_same_call_twice_and_permuted_order_bitwise():
    """A slot's result depends only on its own state and inputs."""
    H = 4
    rng = np.random.default_rng(8)
    lens = [1, 3, 1, 7, 1]
    ids = np.array([5, 2, 9, 0, 7], np.int32)
    b = G.make_batch(rng, ids, lens, H, 64, "bf16")
    init = G.draw_states(rng, len(ids), H, 64)
    outs = []
    for order in (None, None, [3, 0, 4, 1, 2]):
        pool = _pool(10, H)
        try:
            set_states(pool, ids, init)
            if order is None:
                o = run_forward(pool, b)
                S = get_states(pool, ids)
            else:
                lens_p = [lens[i] for i in order]
                cu = np.concatenate([[0], np.cumsum(lens_p)]).astype(np.int32)
                rows = np.concatenate([np.arange(b.cu_seqlens[i],
                                                 b.cu_seqlens[i + 1])
                                       for i in order]).astype(np.int64)
                bp = G.Batch(b.dtype, H, 64, ids[order], cu,
                             {n: b.inputs[n][rows] for n in G.NAMES})
                op = run_forward(pool, bp)
                o = torch.empty_like(op)
                o[torch.from_numpy(rows)] = op
                S = get_states(pool, ids)
        finally:
            W.wkv7_pool_destroy(pool)
        outs.append((o, S))
    for o, S in outs[1:]:
        assert torch.equal(o.view(torch.int32), outs[0][0].view(torch.int32))
        assert torch.equal(S.view(torch.int32), outs[0][1].view(torch.int32))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_multi_token_sequential_equals_token_steps_bitwise(dtype):
    """Short multi-token sequences (four wavefronts per (sequence, head),
    inputs through a ring loaded ahead, the ring's tail run as no-ops) give
    the same bits as feeding the same tokens one call at a time (single-
    token calls run the one-wavefront decode kernel): lengths around the
    ring depths (8 tokens for bf16 inputs, 4 for fp32)."""
    H = 3
    lens = [2, 3, 4, 5, 7, 8, 9, 16, 17, 63]
    rng = np.random.default_rng(31)
    n = len(lens)
    ids = rng.permutation(24)[:n].astype(np.int32)
    say(f"multi-token sequential vs token steps dtype={dtype} lens={lens}")
    b = G.make_batch(rng, ids, lens, H, 64, dtype)
    init = G.draw_states(rng, n, H, 64)
    init[0, 0, 0, :4] = torch.tensor([-0.0, 0.0, -0.0, 1e-40])  # signed zeros, a denormal
    x = {k: b.inputs[k].to(DEV).contiguous() for k in G.NAMES}
    pool = _pool(24, H, seq_only=True)
    try:
        set_states(pool, ids, init)
        o_all = torch.full((b.T_tot, H, 64), float("nan"), device=DEV)
        W.wkv7_forward(pool, ids, b.cu_seqlens, x["r"], x["w"], x["k"],
                       x["v"], x["a"], x["b"], o_all)
        torch.cuda.synchronize()
        S_all = get_states(pool, ids)
        set_states(pool, ids, init)
        o_step = torch.full_like(o_all, float("nan"))
        for t in range(max(lens)):
            live = [s for s in range(n) if lens[s] > t]
            rows = torch.tensor([int(b.cu_seqlens[s]) + t for s in live],
                                device=DEV)
            cu = np.arange(len(live) + 1, dtype=np.int32)
            xt = {k: x[k][rows].contiguous() for k in G.NAMES}
            ot = torch.empty((len(live), H, 64), device=DEV)
            W.wkv7_forward(pool, ids[live], cu, xt["r"], xt["w"], xt["k"],
                           xt["v"], xt["a"], xt["b"], ot)
            o_step[rows] = ot
        torch.cuda.synchronize()
        S_step = get_states(pool, ids)
    finally:
        W.wkv7_pool_destroy(pool)
    assert torch.equal(o_all.cpu().view(torch.int32), o_step.cpu().view(torch.int32))
    assert torch.equal(S_all.view(torch.int32), S_step.view(torch.int32))


def test_many_short_sequences_same_bits_either_kernel():
    """Short multi-token sequences take the four-wavefront kernel while a
    call has at most 8 (sequence, head) chains per CU and the one-wavefront
    kernel beyond that: 36 sequences x H=64 (2304 chains, more than the 2048
    of a 256-CU part) in one call, then the same sequences four at a time.
    Same bits both ways, and both against the oracle."""
    H = 64
    rng = np.random.default_rng(41)
    n = 36
    lens = rng.integers(2, 21, n).tolist()
    ids = np.arange(n, dtype=np.int32)
    say(f"many short sequences H={H} n={n} lens={lens}")
    b = G.make_batch(rng, ids, lens, H, 64, "bf16")
    init = G.draw_states(rng, n, H, 64)
    x = {k: b.inputs[k].to(DEV).contiguous() for k in G.NAMES}
    pool = _pool(n, H)
    try:
        set_states(pool, ids, init)
        o_big = torch.full((b.T_tot, H, 64), float("nan"), device=DEV)
        W.wkv7_forward(pool, ids, b.cu_seqlens, x["r"], x["w"], x["k"],
                       x["v"], x["a"], x["b"], o_big)
        torch.cuda.synchronize()
        S_big = get_states(pool, ids)
        set_states(pool, ids, init)
        o_small = torch.full_like(o_big, float("nan"))
        for g0 in range(0, n, 4):
            grp = list(range(g0, min(n, g0 + 4)))
            lo, hi = int(b.cu_seqlens[grp[0]]), int(b.cu_seqlens[grp[-1] + 1])
            cu = (b.cu_seqlens[grp[0]:grp[-1] + 2] - lo).astype(np.int32)
            xg = {k: x[k][lo:hi].contiguous() for k in G.NAMES}
            og = torch.empty((hi - lo, H, 64), device=DEV)
            W.wkv7_forward(pool, ids[grp], cu, xg["r"], xg["w"], xg["k"],
                           xg["v"], xg["a"], xg["b"], og)
            o_small[lo:hi] = og
        torch.cuda.synchronize()
        S_small = get_states(pool, ids)
    finally:
        W.wkv7_pool_destroy(pool)
    assert torch.equal(o_big.cpu().view(torch.int32), o_small.cpu().view(torch.int32))
    assert torch.equal(S_big.view(torch.int32), S_small.view(torch.int32))
    states = {int(i): G.as_f64(init[m]) for m, i in enumerate(ids)}
    o_ref, S_ref = _oracle(b, states)
    e_o = rel_err(o_big.cpu(), o_ref)
    e_s = max(rel_err(S_big[m], S_ref[int(i)]) for m, i in enumerate(ids))
    say(f"  o err {e_o:.3e}  S err {e_s:.3e}")
    assert e_o < 1e-5 and e_s < 1e-5


def test_forward_errors_leave_pool_untouched():
    H = 2
    rng = np.random.default_rng(9)
    pool = _pool(4, H)
    try:
        init = G.draw_states(rng, 4, H, 64)
        ids = np.arange(4, dtype=np.int32)
        set_states(pool, ids, init)
        b = G.make_batch(rng, [0, 1], [1, 1], H, 64, "bf16")
        x = {n: b.inputs[n].to(DEV) for n in G.NAMES}
        o = torch.zeros((2, H, 64), dtype=torch.float32, device=DEV)
        cases = [
            ([0, 4], [0, 1, 2], W.WKV7_ERR_OUT_OF_RANGE),
            ([1, 1], [0, 1, 2], W.WKV7_ERR_DUPLICATE_SLOT),
            ([0, 1], [0, 2, 1], W.WKV7_ERR_INVALID_ARG),
            ([0, 1], [1, 1, 2], W.WKV7_ERR_INVALID_ARG),
        ]
        for sids, cu, code in cases:
            with pytest.raises(W.Wkv7Error) as e:
                W.wkv7_forward(pool, sids, cu, x["r"], x["w"], x["k"], x["v"],
                               x["a"], x["b"], o)
            assert e.value.status == code, e.value.message
        with pytest.raises(W.Wkv7Error) as e:
            W.wkv7_forward(pool, [0, 1], [0, 1, 2], x["r"].half(), x["w"],
                           x["k"], x["v"], x["a"], x["b"], o)
        assert e.value.status == W.WKV7_ERR_UNSUPPORTED
        # misaligned device pointer
        rr = torch.zeros(2 * H * 64 + 1, dtype=torch.bfloat16, device=DEV)[1:]
        with pytest.raises(W.Wkv7Error) as e:
            W.wkv7_forward(pool, [0, 1], [0, 1, 2], rr, x["w"], x["k"],
                           x["v"], x["a"], x["b"], o, dtype=W.WKV7_BF16)
        assert e.value.status == W.WKV7_ERR_INVALID_ARG
        # the pool's device, and tensors claimed for another one refused by
        # the binding (a one-GPU machine has no second device to put them on)
        assert W.wkv7_pool_device(pool) == torch.cuda.current_device()
        with pytest.raises(ValueError, match="pool's memory is on device"):
            W._check_io(2, H, None, [x[n] for n in G.NAMES], o,
                        W.wkv7_pool_device(pool) + 1)
        torch.cuda.synchronize()
        assert torch.equal(o, torch.zeros_like(o))
        after = get_states(pool, ids)
        assert torch.equal(after.view(torch.int32), init.view(torch.int32))
        # zero tokens / zero sequences are no-ops
        W.wkv7_forward(pool, [], [0], x["r"], x["w"], x["k"], x["v"], x["a"],
                       x["b"], o)
        W.wkv7_forward(pool, [2, 3], [0, 0, 0], x["r"], x["w"], x["k"],
                       x["v"], x["a"], x["b"], o)
        torch.cuda.synchronize()
        assert torch.equal(get_states(pool, ids).view(torch.int32),
                           init.view(torch.int32))
    finally:
        W.wkv7_pool_destroy(pool)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_streams_large_state_nontemporally(dtype):
    """300 slots x H=64 is 300 MiB of active state, above the 256 MB
    Infinity Cache: the decode kernel takes its non-temporal variant. Two
    steps (the second also short sequences of 3 tokens) against the oracle
    on 24 sampled slots, every head."""
    n, H = 300, 64
    rng = np.random.default_rng(71)
    ids = rng.permutation(320)[:n].astype(np.int32)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(71)
    init = torch.randn((n, H, 64, 64), device=DEV, generator=gen) * 0.1
    pool = _pool(320, H)
    try:
        W.wkv7_resume(pool, ids, init)
        torch.cuda.synchronize()
        samp = rng.choice(n, 24, replace=False)
        S = init[samp].double().cpu().numpy()
        for lens in ([1] * n, [3] * n):
            b = G.make_batch(np.random.default_rng(len(lens) + lens[0]), ids,
                             lens, H, 64, dtype)
            o = run_forward(pool, b)
            x = b.inputs64()
            cu = b.cu_seqlens
            err = 0.0
            for s_i, n_i in enumerate(samp):
                sl = slice(cu[n_i], cu[n_i + 1])
                st = {0: S[s_i]}
                o_ref, st = oracle_forward(st, np.array([0], np.int32),
                                           np.array([0, lens[n_i]], np.int32),
                                           {k: x[k][sl] for k in G.NAMES}, H, 64)
                S[s_i] = st[0]
                err = max(err, rel_err(o[sl], o_ref))
            Sg = get_states(pool, ids[samp])
            err = max(err, rel_err(Sg, S))
            say(f"large-state decode {dtype} lens {lens[0]}: err {err:.3e}")
            assert err < tol_for(dtype)
    finally:
        W.wkv7_pool_destroy(pool)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_streaming_form(dtype):
    """A decode step whose active state exceeds the 256 MB Infinity Cache
    (520 slots x H=32 = 272 MB) takes the streaming form of the row steps
    (contiguous rows, each stored as it is updated): every slot and head
    against the float64 oracle, and untouched slots bit-identical."""
    from oracle import wkv7_cref as C
    n_active, H = 520, 32
    rng = np.random.default_rng(31)
    ids = rng.permutation(600)[:n_active].astype(np.int32)
    say(f"streaming decode, {n_active} slots x H={H}, dtype={dtype}")
    b = G.make_batch(rng, ids, [1] * n_active, H, 64, dtype)
    init = G.draw_states(rng, n_active, H, 64)
    others = np.setdiff1d(np.arange(600), ids).astype(np.int32)
    other_states = G.draw_states(rng, len(others), H, 64, std=1.0)
    pool = _pool(600, H)
    try:
        set_states(pool, others, other_states)
        set_states(pool, ids, init)
        o = run_forward(pool, b)
        S = get_states(pool, ids)
        after = get_states(pool, others)
    finally:
        W.wkv7_pool_destroy(pool)
    S_ref = np.ascontiguousarray(G.as_f64(init).reshape(n_active * H, 64, 64))
    o_ref = C.run_heads(S_ref, b.inputs, 1, n_active * H, 64)
    e_o = rel_err(o, o_ref.reshape(n_active, H, 64))
    e_s = rel_err(S, S_ref.reshape(n_active, H, 64, 64))
    say(f"  o err {e_o:.3e}  S err {e_s:.3e}")
    assert e_o < 1e-5 and e_s < 1e-5
    assert torch.equal(after.view(torch.int32), other_states.view(torch.int32))
