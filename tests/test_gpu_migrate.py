"""live-migrate between pools and self-describing slot images (GPU)."""
import ctypes

import numpy as np
import pytest
import torch

import wkv7_inputs as G
from linear_attention_rnn_amd import wkv7 as W
from tests.gpu_util import DEV, say, set_states, get_states, run_forward

pytestmark = pytest.mark.gpu
H = 3


def _bits_equal(a, b):
    return torch.equal(a.contiguous().view(torch.int32),
                       b.contiguous().view(torch.int32))


def test_migrate_is_bitexact_and_continues_identically():
    src_ids = np.array([5, 0, 9, 5], np.int32)          # a source may repeat
    dst_ids = np.array([1, 7, 3, 6], np.int32)
    init = G.draw_states(np.random.default_rng(41), 3, H, 64)
    a = W.wkv7_pool_create(12, H, 64)
    b = W.wkv7_pool_create(8, H, 64)
    try:
        set_states(a, np.array([5, 0, 9], np.int32), init)
        before_b = get_states(b, [0, 2, 4, 5])
        W.wkv7_migrate(a, src_ids, b, dst_ids)
        torch.cuda.synchronize()
        assert _bits_equal(get_states(a, src_ids), get_states(b, dst_ids))
        assert _bits_equal(get_states(b, [0, 2, 4, 5]), before_b)
        # the same decode token and a 70-token prefill on both sides
        for lens in ([1, 1, 1], [70, 3, 70]):
            ba = G.make_batch(np.random.default_rng(len(lens) + lens[0]),
                              src_ids[:3], lens, H, 64, G.BF16)
            bb = G.Batch(ba.dtype, H, 64, dst_ids[:3], ba.cu_seqlens, ba.inputs)
            oa, ob = run_forward(a, ba), run_forward(b, bb)
            assert _bits_equal(oa, ob)
            assert _bits_equal(get_states(a, src_ids[:3]),
                               get_states(b, dst_ids[:3]))
        say("migrated slots continue bit for bit like their sources")
    finally:
        W.wkv7_pool_destroy(a)
        W.wkv7_pool_destroy(b)


def test_migrate_rejections():
    a = W.wkv7_pool_create(4, H, 64)
    b = W.wkv7_pool_create(4, H, 64)
    c = W.wkv7_pool_create(4, H + 1, 64)
    try:
        cases = [
            ((a, [0], c, [0]), W.WKV7_ERR_UNSUPPORTED),      # other shape
            ((a, [0, 1], b, [2, 2]), W.WKV7_ERR_DUPLICATE_SLOT),
            ((a, [4], b, [0]), W.WKV7_ERR_OUT_OF_RANGE),
            ((a, [0], b, [4]), W.WKV7_ERR_OUT_OF_RANGE),
            ((a, [0], a, [0]), W.WKV7_ERR_DUPLICATE_SLOT),   # same pool: fork
        ]
        for args, code in cases:
            with pytest.raises(W.Wkv7Error) as e:
                W.wkv7_migrate(*args)
            assert e.value.status == code, args
        W.wkv7_migrate(a, [], b, [])
    finally:
        for p in (a, b, c):
            W.wkv7_pool_destroy(p)


def test_serialized_images_with_header_roundtrip():
    """header + hibernated images in one pinned buffer; a reader checks the
    header against its pool and resumes the images bit-exactly."""
    ids = np.array([2, 3, 4, 8], np.int32)
    init = G.draw_states(np.random.default_rng(42), len(ids), H, 64)
    a = W.wkv7_pool_create(10, H, 64)
    b = W.wkv7_pool_create(6, H, 64)
    try:
        set_states(a, ids, init)
        sb = W.wkv7_slot_bytes(a)
        buf = torch.empty(64 + len(ids) * sb, dtype=torch.uint8,
                          pin_memory=True)
        hdr = W.wkv7_image_header_init(H, 64, len(ids))
        buf[:64].numpy()[:] = np.frombuffer(bytes(hdr), np.uint8)
        W.wkv7_hibernate(a, ids, buf[64:])
        torch.cuda.synchronize()
        # reader side
        got = W.wkv7_image_header.from_buffer_copy(buf[:64].numpy().tobytes())
        W.wkv7_image_header_check(got, H, 64)
        dst = np.array([5, 0, 1, 3], np.int32)
        W.wkv7_resume(b, dst[:got.n_slots], buf[64:])
        torch.cuda.synchronize()
        assert _bits_equal(get_states(b, dst), get_states(a, ids))
        with pytest.raises(W.Wkv7Error) as e:
            W.wkv7_image_header_check(got, H + 1, 64)
        assert e.value.status == W.WKV7_ERR_UNSUPPORTED
    finally:
        W.wkv7_pool_destroy(a)
        W.wkv7_pool_destroy(b)
