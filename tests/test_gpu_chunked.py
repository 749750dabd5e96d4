"""Parity of the chunked-prefill kernel with the float64 oracle (GPU)."""
import numpy as np
import pytest
import torch

import wkv7_inputs as G
from linear_attention_rnn_amd import wkv7 as W
from oracle import wkv7_forward as oracle_forward, wkv7_sequence
from tests.gpu_util import (DEV, say, set_states, get_states, run_forward,
                            rel_err, tol_for)
from tests.parity import report

pytestmark = pytest.mark.gpu


# what each chunked path reaches (regression guards, inside the bars of
# 1e-3 for fp32 inputs and 2e-2 for bf16 inputs)
GUARD = {("f32", 0): 5e-4, ("f32", 1): 5e-4, ("bf16", 1): 5e-4,
         ("bf16", 0): 1e-2}


def _run(ids, lens, H, dtype, n_slots, init=None, min_len=None, seed=0,
         precise=0, scale=None, edit=None, **draw):
    rng = np.random.default_rng(seed)
    b = G.make_batch(rng, ids, lens, H, 64, dtype, **draw)
    if scale is not None:
        for name, f in scale.items():
            b.inputs[name] = (b.inputs[name].double() * f).to(b.inputs[name].dtype)
    if edit is not None:
        edit(b.inputs)      # in place, on the rounded inputs both sides use
    pool = W.wkv7_pool_create(n_slots, H, 64)
    try:
        W.wkv7_pool_set_option(pool, W.WKV7_OPT_CHUNK_PRECISE, precise)
        if min_len is not None:
            W.wkv7_pool_set_option(pool, W.WKV7_OPT_PREFILL_MIN_LEN, min_len)
        if init is not None:
            set_states(pool, ids, init)
        o = run_forward(pool, b)
        S = get_states(pool, ids)
    finally:
        W.wkv7_pool_destroy(pool)
    states = {} if init is None else \
        {int(i): G.as_f64(init[n]) for n, i in enumerate(ids)}
    o_ref, S_ref = oracle_forward(states, b.slot_ids, b.cu_seqlens,
                                  b.inputs64(), H, 64)
    e_o = rel_err(o, o_ref)
    e_s = max(rel_err(S[n], S_ref[int(i)]) for n, i in enumerate(ids))
    return e_o, e_s, o, S


PATHS = [("f32", 0), ("bf16", 0), ("bf16", 1)]


@pytest.mark.parametrize("dtype,precise", PATHS)
def test_small_config_chunked(dtype, precise):
    """H=2, one sequence of T=64 (exactly one chunk), zero state."""
    say(f"small config chunked dtype={dtype} precise={precise}")
    e_o, e_s, _, _ = _run([0], [64], 2, dtype, 1, precise=precise)
    say(f"  o err {e_o:.3e}  S err {e_s:.3e}")
    report(f"small case (H=2, T=64, {dtype}), chunked kernel, "
           f"{'precise' if precise or dtype == 'f32' else 'fast'} plan: o "
           f"{e_o:.3e}, S {e_s:.3e}")
    assert e_o < tol_for(dtype) and e_s < tol_for(dtype)
    assert e_o < GUARD[dtype, precise] and e_s < GUARD[dtype, precise]


@pytest.mark.parametrize("dtype,precise", PATHS)
def test_ragged_chunked_with_state(dtype, precise):
    """Several tiles and ragged tails, non-zero initial states, chunked and
    sequential sequences in one call."""
    lens = [64, 65, 1, 127, 200, 3, 130, 128]
    H = 3
    ids = np.arange(len(lens), dtype=np.int32)[::-1].copy()
    init = G.draw_states(np.random.default_rng(11), len(ids), H, 64)
    say(f"ragged chunked dtype={dtype} precise={precise} lens={lens}")
    e_o, e_s, _, _ = _run(ids, lens, H, dtype, len(ids), init=init, seed=1,
                          precise=precise)
    say(f"  o err {e_o:.3e}  S err {e_s:.3e}")
    assert e_o < GUARD[dtype, precise] and e_s < GUARD[dtype, precise]


@pytest.mark.parametrize("precise", [0, 1])
def test_every_length_chunked(precise):
    """PREFILL_MIN_LEN=1: every sequence (lengths 1..70) on the chunked
    kernel, so single partial chunks of every size are covered."""
    lens = list(range(1, 71))
    H = 1
    ids = np.arange(len(lens), dtype=np.int32)
    init = G.draw_states(np.random.default_rng(12), len(ids), H, 64)
    e_o, e_s, _, _ = _run(ids, lens, H, "bf16", len(ids), init=init,
                          min_len=1, seed=2, precise=precise)
    say(f"every length precise={precise}: o err {e_o:.3e}  S err {e_s:.3e}")
    assert e_o < GUARD["bf16", precise] and e_s < GUARD["bf16", precise]


@pytest.mark.parametrize("dtype,precise", PATHS)
@pytest.mark.parametrize("w", [0.02, 1e-4])
def test_extreme_decay_chunks(w, dtype, precise):
    """Decay so strong that the scaled operands would leave fp32 range:
    those chunks run token by token inside the chunked kernel (exact)."""
    lens = [64, 150]
    H = 2
    ids = np.array([0, 1], np.int32)
    init = G.draw_states(np.random.default_rng(13), 2, H, 64)
    e_o, e_s, o, S = _run(ids, lens, H, dtype, 2, init=init, seed=3,
                          w_override=w, precise=precise)
    say(f"extreme w={w} {dtype} precise={precise}: o err {e_o:.3e}  "
        f"S err {e_s:.3e}")
    assert np.all(np.isfinite(o.numpy())) and np.all(np.isfinite(S.numpy()))
    assert e_o < 1e-4 and e_s < 1e-4


@pytest.mark.parametrize("dtype,precise", PATHS)
@pytest.mark.parametrize("name,factor", [("v", 1e5), ("k", 3e4)])
def test_out_of_fp16_range_runs_exactly(name, factor, dtype, precise):
    """Inputs at 2^15 or beyond make the chunked kernel run their chunks
    token by token, in either plan (the fast plan's fp16 operands would
    overflow; the precise plan keeps the same rule): exact, to fp32
    rounding (about 1e-6 here, against 3e-5 and more for either plan's
    products, so a chunk left on the MFMA path would fail the bound)."""
    lens = [130]
    H = 2
    ids = np.array([0], np.int32)
    e_o, e_s, o, S = _run(ids, lens, H, dtype, 1, seed=6,
                          scale={name: factor}, precise=precise)
    say(f"large {name} x{factor:g} {dtype} precise={precise}: o err {e_o:.3e}  "
        f"S err {e_s:.3e}")
    assert np.all(np.isfinite(o.numpy())) and np.all(np.isfinite(S.numpy()))
    assert e_o < 1e-5 and e_s < 1e-5


@pytest.mark.parametrize("dtype,precise", PATHS)
@pytest.mark.parametrize("name", ["a", "b", "r"])
def test_single_large_input_runs_exactly(name, dtype, precise):
    """One element of a, b or r at 4e4 (beyond the fp16 operand range, one
    token): its chunk runs token by token (the raw-input range flags of
    both key roles), the others on the chunked products."""
    def edit(x):
        x[name][5, 1, 3] = 4.0e4
    e_o, e_s, o, S = _run(np.array([0], np.int32), [100], 2, dtype, 1,
                          seed=7, edit=edit, precise=precise)
    say(f"large single {name} {dtype} precise={precise}: o err {e_o:.3e}  "
        f"S err {e_s:.3e}")
    assert np.all(np.isfinite(o.numpy())) and np.all(np.isfinite(S.numpy()))
    assert e_o < GUARD[dtype, precise] and e_s < GUARD[dtype, precise]


@pytest.mark.parametrize("dtype,precise", PATHS)
def test_growing_decay_runs_exactly(dtype, precise):
    """w above 1 (1.0625 on every channel): outside the chunked form's
    range (its check runs when a chunk's inputs are prepared), so every
    chunk runs token by token."""
    e_o, e_s, o, S = _run(np.array([0], np.int32), [130], 2, dtype, 1,
                          seed=8, w_override=1.0625, precise=precise)
    say(f"w = 1.0625 {dtype} precise={precise}: o err {e_o:.3e}  S err {e_s:.3e}")
    assert np.all(np.isfinite(o.numpy())) and np.all(np.isfinite(S.numpy()))
    # fp32 rounding of the token-by-token path (about 4e-6 here, against
    # 3e-5 and more for either plan's products)
    assert e_o < 1e-5 and e_s < 1e-5


@pytest.mark.parametrize("dtype,precise", PATHS)
@pytest.mark.parametrize("c", [1.0, 2.0])
def test_t_out_of_fp16_range_runs_exactly(c, dtype, precise):
    """a = b = u with |u|^2 = c and w = 1 make A_ab = c below the
    diagonal, so T = (I - A_ab)^-1 grows like (1 + c)^(t - s) within the
    first 32-token chunk: with c = 1 only the off-diagonal block T_10
    leaves the fp16 range (checked on every value wavefront), with c = 2
    the diagonal blocks D_0 and D_1 too (checked where they are built).
    The chunk runs token by token; the 8-token tail chunk on the fast path."""
    u = torch.zeros(64, dtype=torch.float64)
    u[0] = 1.0
    u[1] = (c - 1.0) ** 0.5

    def edit(x):
        for name in ("a", "b"):
            x[name][:] = u.to(x[name].dtype)
        x["w"][:] = 1.0
    e_o, e_s, o, S = _run(np.array([0], np.int32), [40], 2, dtype, 1,
                          seed=9, edit=edit, precise=precise)
    say(f"T out of range, c = {c} {dtype} precise={precise}: o err {e_o:.3e}  "
        f"S err {e_s:.3e}")
    assert np.all(np.isfinite(o.numpy())) and np.all(np.isfinite(S.numpy()))
    assert e_o < GUARD[dtype, precise] and e_s < GUARD[dtype, precise]


def test_chunked_matches_sequential_within_rounding():
    """Both kernels on the same inputs agree to fp32 rounding, not bitwise."""
    lens = [300, 64]
    H = 4
    ids = np.array([0, 1], np.int32)
    init = G.draw_states(np.random.default_rng(14), 2, H, 64)
    _, _, o1, S1 = _run(ids, lens, H, "bf16", 2, init=init, seed=4)
    _, _, o2, S2 = _run(ids, lens, H, "bf16", 2, init=init, seed=4,
                        min_len=1 << 30)
    assert rel_err(o1, o2.double().numpy()) < GUARD["bf16", 0]
    assert rel_err(S1, S2.double().numpy()) < GUARD["bf16", 0]
