"""The allocation-free forward (wkv7_forward_noalloc) against wkv7_forward,
through the C ABI: the same bits for outputs and slot states on two calls in
a row, the second with a smaller batch, with segment-parallel prefill off
and on (segment buffers in the static scratch; bf16 inputs, and fp32 inputs,
whose chunked sequences take the kernel's precise plan), and the size
limits rejected before any device work."""
import numpy as np
import pytest
import torch

import wkv7_inputs as G
from linear_attention_rnn_amd import wkv7 as W
from tests.gpu_util import DEV, say, set_states, get_states

pytestmark = pytest.mark.gpu
N = 64


def _bits_equal(a, b):
    return torch.equal(a.contiguous().view(torch.int32),
                       b.contiguous().view(torch.int32))


def _call(fn, pool, ids, cu, x, T, H):
    o = torch.full((T, H, N), float("nan"), dtype=torch.float32, device=DEV)
    fn(pool, ids, cu, x["r"], x["w"], x["k"], x["v"], x["a"], x["b"], o)
    return o


def _as_f32(b):
    """The same batch with fp32 inputs (the bf16 values, exactly)."""
    return G.Batch(G.F32, b.H, b.N, b.slot_ids, b.cu_seqlens,
                   {n: b.inputs[n].to(torch.float32) for n in G.NAMES})


@pytest.mark.parametrize("seg_len,dtype", [(0, G.BF16), (512, G.BF16),
                                           (512, G.F32)])
def test_noalloc_equals_forward_on_two_calls(seg_len, dtype):
    H, n_slots = 12, 128
    lay = G.cfg_mixed_layers(seed=3, n_layers=1)[0]
    rng = np.random.default_rng(40)
    # second call, smaller: 16 of the decode slots and two prefills into
    # other slots (one long enough to be split when segments are on)
    dec2 = lay.decode_ids[:16]
    free = np.setdiff1d(np.arange(n_slots),
                        np.concatenate([lay.decode_ids, lay.prefill_ids]))
    pre2 = rng.choice(free, 2, replace=False).astype(np.int32)
    ids2 = np.concatenate([dec2, pre2]).astype(np.int32)
    b2 = G.make_batch(rng, ids2, [1] * 16 + [130, 1100], H, N, G.BF16)
    b1 = lay.batch
    if dtype == G.F32:
        b1, b2 = _as_f32(b1), _as_f32(b2)
    calls = [(b1.slot_ids, b1.cu_seqlens, b1), (b2.slot_ids, b2.cu_seqlens, b2)]
    say(f"noalloc vs forward, segment length {seg_len}, {dtype}: calls of "
        f"{lay.batch.T_tot} and {b2.T_tot} tokens")
    pools = [W.wkv7_pool_create(n_slots, H, N) for _ in range(2)]
    try:
        for p in pools:
            W.wkv7_pool_set_option(p, W.WKV7_OPT_SEGMENT_LEN, seg_len)
            set_states(p, lay.decode_ids, lay.init_states)
        for ci, (ids, cu, b) in enumerate(calls):
            x = {n: b.inputs[n].to(DEV) for n in G.NAMES}
            o_ref = _call(W.wkv7_forward, pools[0], ids, cu, x, b.T_tot, H)
            o_got = _call(W.wkv7_forward_noalloc, pools[1], ids, cu, x,
                          b.T_tot, H)
            torch.cuda.synchronize()
            assert torch.isfinite(o_ref).all()
            assert _bits_equal(o_got, o_ref), f"call {ci}: outputs differ"
            S_ref, S_got = get_states(pools[0], ids), get_states(pools[1], ids)
            assert _bits_equal(S_got, S_ref), f"call {ci}: states differ"
            say(f"  call {ci}: outputs and states bit-identical")
    finally:
        for p in pools:
            W.wkv7_pool_destroy(p)


def test_noalloc_rejects_oversized_batches_without_device_work():
    # work description beyond 64 KiB: 4097 one-token sequences (16 B each)
    n, H = 4097, 1
    pool = W.wkv7_pool_create(n, H, N)
    try:
        rng = np.random.default_rng(41)
        b = G.make_batch(rng, np.arange(n, dtype=np.int32), [1] * n, H, N,
                         G.BF16)
        x = {k: b.inputs[k].to(DEV) for k in G.NAMES}
        with pytest.raises(W.Wkv7Error) as ei:
            _call(W.wkv7_forward_noalloc, pool, b.slot_ids, b.cu_seqlens, x,
                  b.T_tot, H)
        assert ei.value.status == W.WKV7_ERR_INVALID_ARG
        assert "static scratch" in str(ei.value)
        torch.cuda.synchronize()
        S = get_states(pool, np.arange(8, dtype=np.int32))
        assert not S.any(), "a rejected call changed a slot"
        # 4096 sequences fit (exactly 64 KiB of work description)
        o = _call(W.wkv7_forward_noalloc, pool, b.slot_ids[:4096],
                  b.cu_seqlens[:4097], x, 4096, H)
        torch.cuda.synchronize()
        assert torch.isfinite(o[:4096]).all()
    finally:
        W.wkv7_pool_destroy(pool)
    # segment buffers beyond the array: one 4096-token prompt at H=32 in
    # segments of 64 needs 64 x 3 x 32 x 16 KiB = 96 MiB
    H = 32
    pool = W.wkv7_pool_create(1, H, N)
    try:
        W.wkv7_pool_set_option(pool, W.WKV7_OPT_SEGMENT_LEN, 64)
        rng = np.random.default_rng(42)
        b = G.make_batch(rng, [0], [4096], H, N, G.BF16)
        x = {k: b.inputs[k].to(DEV) for k in G.NAMES}
        with pytest.raises(W.Wkv7Error) as ei:
            o = torch.full((4096, H, N), float("nan"), dtype=torch.float32,
                           device=DEV)
            W.wkv7_forward_noalloc(pool, b.slot_ids, b.cu_seqlens, x["r"],
                                   x["w"], x["k"], x["v"], x["a"], x["b"], o)
        assert ei.value.status == W.WKV7_ERR_INVALID_ARG
        torch.cuda.synchronize()
        assert torch.isnan(o).all(), "a rejected call wrote outputs"
        assert not get_states(pool, [0]).any()
    finally:
        W.wkv7_pool_destroy(pool)
