"""The two composite workloads on the GPU through the C ABI:

* a 12-layer RWKV-X-0.2B-shaped stack (H=12) with a mixed batch of 64 decode
  slots and 4 ragged prefills per layer, then 16 forks whose continuation
  must equal the parent's bit for bit;
* a large pool (4096 slots, H=64, 4 GiB) with a 1024-slot decode step, 32
  ragged prefills of 128..8192 tokens, and hibernate/resume of 256 slots.
"""
import numpy as np
import pytest
import torch

import wkv7_inputs as G
from linear_attention_rnn_amd import wkv7 as W
from oracle import wkv7_forward as oracle_forward, wkv7_decode_batch
from oracle import wkv7_cref as C
from tests.gpu_util import (DEV, say, set_states, get_states, run_forward,
                            rel_err)
from tests.parity import report

pytestmark = pytest.mark.gpu
TOL = 2e-2          # bf16 inputs
TIGHT = 1e-2        # what the default kernels reach, with margin


def _bits_equal(a, b):
    return torch.equal(a.contiguous().view(torch.int32),
                       b.contiguous().view(torch.int32))


@pytest.mark.parametrize("shuffle", [False, True])
def test_mixed_stack_and_fork_continuation(shuffle):
    layers = G.cfg_mixed_layers(seed=3, shuffle=shuffle)
    H, n_slots = 12, 128
    say(f"mixed stack: {len(layers)} layers, shuffle={shuffle}")
    rng = np.random.default_rng(33)
    pools = [W.wkv7_pool_create(n_slots, H, 64) for _ in layers]
    try:
        worst = 0.0
        for li, (lay, pool) in enumerate(zip(layers, pools)):
            set_states(pool, lay.decode_ids, lay.init_states)
            b = lay.batch
            o = run_forward(pool, b)
            S = get_states(pool, b.slot_ids)
            states = {int(i): G.as_f64(lay.init_states[n])
                      for n, i in enumerate(lay.decode_ids)}
            # decode rows against the oracle in one batch
            dec_rows = [n for n in range(len(b.slot_ids))
                        if b.cu_seqlens[n + 1] - b.cu_seqlens[n] == 1]
            x = b.inputs64()
            S0 = np.stack([states[int(b.slot_ids[n])] for n in dec_rows])
            xd = {k: x[k][b.cu_seqlens[dec_rows]] for k in G.NAMES}
            o_ref, S_ref = wkv7_decode_batch(S0, xd)
            e = max(rel_err(o[b.cu_seqlens[dec_rows]], o_ref),
                    rel_err(S[dec_rows], S_ref))
            # prefills: outputs and final states of every head
            for n in range(len(b.slot_ids)):
                lo, hi = b.cu_seqlens[n], b.cu_seqlens[n + 1]
                if hi - lo == 1:
                    continue
                o_p, S_p = C.sequence(np.zeros((H, 64, 64)),
                                      **{k: b.inputs[k][lo:hi]
                                         for k in G.NAMES}, threads=None)
                e = max(e, rel_err(o[lo:hi], o_p), rel_err(S[n], S_p))
            worst = max(worst, e)
            say(f"  layer {li}: max err {e:.3e}")
        report(f"12-layer mixed stack (shuffle={shuffle}): worst max|err|/rms "
               f"{worst:.3e} over the layers' outputs and final states")
        assert worst < TIGHT

        # fork 16 of the 68 live slots into 16 free ones, in every layer
        live = np.concatenate([layers[0].decode_ids, layers[0].prefill_ids])
        parents = rng.choice(live, 16, replace=False).astype(np.int32)
        free = np.setdiff1d(np.arange(n_slots), live)
        children = rng.choice(free, 16, replace=False).astype(np.int32)
        for pool in pools:
            W.wkv7_fork(pool, parents, children)
        torch.cuda.synchronize()
        for li, pool in enumerate(pools):
            assert _bits_equal(get_states(pool, parents),
                               get_states(pool, children)), f"fork layer {li}"
        # continue parent and child with identical inputs: one decode token,
        # then a 130-token prefill (crosses a chunk boundary, ragged tail)
        for steps in ([1] * 16, [130] * 16):
            for li, pool in enumerate(pools):
                ids = np.concatenate([parents, children])
                lens = list(steps) * 2
                half = G.make_batch(np.random.default_rng([li, steps[0]]),
                                    parents, steps, H, 64, G.BF16)
                inputs = {k: torch.cat([half.inputs[k], half.inputs[k]])
                          for k in G.NAMES}
                cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
                b = G.Batch(G.BF16, H, 64, ids, cu, inputs)
                before = get_states(pool, parents)
                o = run_forward(pool, b)
                T1 = int(half.cu_seqlens[-1])
                assert _bits_equal(o[:T1], o[T1:]), f"fork o, layer {li}"
                Sp, Sc = get_states(pool, parents), get_states(pool, children)
                assert _bits_equal(Sp, Sc), f"fork state, layer {li}"
                # and the parent's continuation matches the oracle
                st = {int(i): G.as_f64(before[n]) for n, i in enumerate(parents)}
                o_ref, S_ref = oracle_forward(st, parents, half.cu_seqlens,
                                              half.inputs64(), H, 64)
                e = max(rel_err(o[:T1], o_ref),
                        max(rel_err(Sp[n], S_ref[int(i)])
                            for n, i in enumerate(parents)))
                assert e < TIGHT, (li, steps[0], e)
            say(f"  fork continuation of {steps[0]} token(s): bitwise equal")
    finally:
        for pool in pools:
            W.wkv7_pool_destroy(pool)


def test_large_pool_decode_prefill_hibernate():
    """Decode and prefill in one 4 GiB pool, then hibernate 256 touched slots
    to pinned host memory, scribble, resume (bit-exact), and decode the
    resumed slots once more against the oracle."""
    n_slots, H = 4096, 64
    seed = 4
    rng = np.random.default_rng(seed)
    perm = rng.permutation(n_slots).astype(np.int32)
    dec_ids, pre_ids = perm[:1024], perm[1024:1056]
    lens = rng.integers(128, 8193, size=32)
    say(f"large pool: 4096 x H=64; prefill lengths sum {int(lens.sum())}")
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    pool = W.wkv7_pool_create(n_slots, H, 64)
    try:
        # resident decode states N(0, 0.1)
        init = (torch.randn((1024, H, 64, 64), device=DEV, generator=gen)
                * 0.1)
        W.wkv7_resume(pool, dec_ids, init)
        torch.cuda.synchronize()
        # one decode step over 1024 slots
        xd = G.draw_tokens_device(gen, 1024, H, 64, G.BF16, DEV)
        od = torch.empty((1024, H, 64), dtype=torch.float32, device=DEV)
        cu_d = np.arange(1025, dtype=np.int32)
        W.wkv7_forward(pool, dec_ids, cu_d, xd["r"], xd["w"], xd["k"],
                       xd["v"], xd["a"], xd["b"], od)
        # 32 ragged prefills from zero
        T = int(lens.sum())
        xp = G.draw_tokens_device(gen, T, H, 64, G.BF16, DEV)
        op = torch.empty((T, H, 64), dtype=torch.float32, device=DEV)
        cu_p = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        W.wkv7_forward(pool, pre_ids, cu_p, xp["r"], xp["w"], xp["k"],
                       xp["v"], xp["a"], xp["b"], op)
        torch.cuda.synchronize()

        # every decode slot and prefill head is compared against the oracle
        # in test_gpu_fullsize.py; here the results only need to be finite
        assert torch.isfinite(od).all() and torch.isfinite(op).all()

        # hibernate 256 touched slots, scribble, resume: bit-exact
        touched = np.concatenate([dec_ids, pre_ids])
        hib = rng.choice(touched, 256, replace=False).astype(np.int32)
        img = torch.empty((256, H, 64, 64), dtype=torch.float32,
                          pin_memory=True)
        ref_img = get_states(pool, hib)
        W.wkv7_hibernate(pool, hib, img)
        W.wkv7_reset(pool, hib)
        torch.cuda.synchronize()
        assert _bits_equal(img, ref_img)
        W.wkv7_resume(pool, hib, img)
        torch.cuda.synchronize()
        assert _bits_equal(get_states(pool, hib), ref_img)
        say("  hibernate/resume of 256 slots: bit-exact")

        # one more decode step on the resumed slots against the oracle
        dec_hib = np.intersect1d(hib, dec_ids)
        x2 = G.draw_tokens_device(gen, len(dec_hib), H, 64, G.BF16, DEV)
        o2 = torch.empty((len(dec_hib), H, 64), dtype=torch.float32,
                         device=DEV)
        before = get_states(pool, dec_hib)
        W.wkv7_forward(pool, dec_hib, np.arange(len(dec_hib) + 1, dtype=np.int32),
                       x2["r"], x2["w"], x2["k"], x2["v"], x2["a"], x2["b"], o2)
        torch.cuda.synchronize()
        o_ref2, S_ref2 = wkv7_decode_batch(
            before.double().numpy(),
            {k: x2[k].double().cpu().numpy() for k in G.NAMES})
        e2 = max(rel_err(o2.cpu(), o_ref2),
                 rel_err(get_states(pool, dec_hib), S_ref2))
        say(f"  decode after resume ({len(dec_hib)} slots): err {e2:.3e}")
        assert e2 < TIGHT
    finally:
        W.wkv7_pool_destroy(pool)
