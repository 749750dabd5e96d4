"""Decode items riding in a chunked launch (GPU): when a batch mixes decode
tokens with chunked prefills and both fit the CUs in one round, the decode
items run in trailing workgroups of the chunked kernel. They must give the
same bits as the sequential kernel alone, unsplit and with segment-parallel
prefill, and the prefills must match the oracle."""
import numpy as np
import pytest
import torch

import wkv7_inputs as G
from linear_attention_rnn_amd import wkv7 as W
from oracle import wkv7_forward as oracle_forward
from tests.gpu_util import DEV, say, set_states, get_states, run_forward, rel_err

pytestmark = pytest.mark.gpu
H = 12
# bars of the mixed batch against the oracle per (input type, precise mode):
# the fast plan for bf16 inputs, the precise plan otherwise
GUARD = {(G.BF16, 0): 1e-2, (G.BF16, 1): 5e-4, (G.F32, 0): 5e-4}


def _bits(t):
    return t.contiguous().view(torch.int32)


def _concat(a, b):
    """Batch a's sequences followed by batch b's."""
    inputs = {n: torch.cat([a.inputs[n], b.inputs[n]]) for n in G.NAMES}
    cu = np.concatenate([a.cu_seqlens, a.cu_seqlens[-1] + b.cu_seqlens[1:]])
    ids = np.concatenate([a.slot_ids, b.slot_ids]).astype(np.int32)
    return G.Batch(a.dtype, a.H, a.N, ids, cu.astype(np.int32), inputs)


CASES = [(0, [2048], G.BF16, 0), (0, [300, 64, 1100], G.BF16, 0),
         (512, [2048], G.BF16, 0), (512, [1100, 2048], G.BF16, 0),
         (0, [300, 64, 1100], G.F32, 0), (512, [1100, 2048], G.F32, 0),
         (512, [1100, 2048], G.BF16, 1)]


@pytest.mark.parametrize("seg,pre_lens,dtype,precise", CASES)
def test_fused_decode_equals_own_launch(seg, pre_lens, dtype, precise):
    rng = np.random.default_rng(len(pre_lens) * 10 + seg)
    n_dec = 64
    dec_ids = rng.permutation(128)[:n_dec].astype(np.int32)
    free = np.setdiff1d(np.arange(128), dec_ids)
    pre_ids = rng.choice(free, len(pre_lens), replace=False).astype(np.int32)
    init = G.draw_states(np.random.default_rng(5), n_dec, H, 64)
    dec = G.make_batch(np.random.default_rng(6), dec_ids, [1] * n_dec, H, 64,
                       dtype)
    pre = G.make_batch(np.random.default_rng(7), pre_ids, pre_lens, H, 64,
                       dtype)
    mixed = _concat(dec, pre)
    say(f"fused decode, segments {seg}, prefills {pre_lens}, {dtype}, "
        f"precise {precise}")
    outs = []
    for batch in (dec, mixed):
        pool = W.wkv7_pool_create(128, H, 64)
        try:
            W.wkv7_pool_set_option(pool, W.WKV7_OPT_SEGMENT_LEN, seg)
            W.wkv7_pool_set_option(pool, W.WKV7_OPT_CHUNK_PRECISE, precise)
            set_states(pool, dec_ids, init)
            o = run_forward(pool, batch)
            S = get_states(pool, batch.slot_ids)
        finally:
            W.wkv7_pool_destroy(pool)
        outs.append((o, S))
    (o_a, S_a), (o_b, S_b) = outs
    assert torch.equal(_bits(o_a), _bits(o_b[:n_dec]))
    assert torch.equal(_bits(S_a), _bits(S_b[:n_dec]))
    # the whole mixed batch against the oracle
    st = {int(i): G.as_f64(init[n]) for n, i in enumerate(dec_ids)}
    o_ref, S_ref = oracle_forward(st, mixed.slot_ids, mixed.cu_seqlens,
                                  mixed.inputs64(), H, 64)
    e = max(rel_err(o_b, o_ref),
            max(rel_err(S_b[n], S_ref[int(i)])
                for n, i in enumerate(mixed.slot_ids)))
    say(f"  decode bits equal; mixed batch err {e:.3e}")
    assert e < GUARD[dtype, precise]
