"""Slot verbs on the GPU: bit-exact copies (fork, snapshot, reset,
hibernate, resume), admission, and their error paths."""
import numpy as np
import pytest
import torch

from linear_attention_rnn_amd import wkv7 as W
from tests.gpu_util import DEV, say, set_states, get_states

pytestmark = pytest.mark.gpu


def _bits(rng, n, H, N=64):
    """Arbitrary 32-bit patterns incl. NaN payloads, -0.0 and denormals."""
    u = rng.integers(0, 2**32, size=(n, H, N, N), dtype=np.uint64)
    u = u.astype(np.uint32)
    flat = u.reshape(-1)
    flat[0::97] = 0x80000000          # -0.0
    flat[1::89] = 0x7FC01234          # quiet NaN with payload
    flat[2::83] = 0x7F800001          # signalling NaN
    flat[3::79] = 0x00000001          # smallest denormal
    return torch.from_numpy(u.view(np.int32).copy()).view(torch.float32)


def _eq_bits(a, b):
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_fork_snapshot_reset_bitexact():
    H, n_slots = 5, 24
    rng = np.random.default_rng(30)
    say(f"verbs: H={H} n_slots={n_slots}")
    pool = W.wkv7_pool_create(n_slots, H, 64)
    try:
        assert W.wkv7_slot_bytes(pool) == H * 64 * 64 * 4
        ids = np.arange(n_slots, dtype=np.int32)
        img = _bits(rng, n_slots, H)
        set_states(pool, ids, img)
        assert _eq_bits(get_states(pool, ids), img)
        # fork: 6 pairs, one source used twice
        src = np.array([0, 3, 3, 7, 11, 2], np.int32)
        dst = np.array([12, 13, 20, 14, 15, 23], np.int32)
        W.wkv7_fork(pool, src, dst)
        expect = img.clone()
        expect[torch.from_numpy(dst).long()] = img[torch.from_numpy(src).long()]
        assert _eq_bits(get_states(pool, ids), expect)
        # snapshot of one slot into a device buffer
        buf = torch.empty((H, 64, 64), dtype=torch.float32, device=DEV)
        W.wkv7_snapshot(pool, 13, buf)
        torch.cuda.synchronize()
        assert _eq_bits(buf.cpu(), expect[13])
        # reset
        W.wkv7_reset(pool, [1, 13, 22])
        expect[[1, 13, 22]] = 0.0
        assert _eq_bits(get_states(pool, ids), expect)
        # resume from the device snapshot restores it
        W.wkv7_resume(pool, [13], buf)
        torch.cuda.synchronize()
        expect[13] = img[3]
        assert _eq_bits(get_states(pool, ids), expect)
    finally:
        W.wkv7_pool_destroy(pool)


def test_hibernate_resume_roundtrip_bitexact():
    H, n_slots = 8, 64
    rng = np.random.default_rng(31)
    pool = W.wkv7_pool_create(n_slots, H, 64)
    try:
        ids_all = np.arange(n_slots, dtype=np.int32)
        img = _bits(rng, n_slots, H)
        set_states(pool, ids_all, img)
        # runs of consecutive ids and scattered ids, in a shuffled order
        hib = np.array([5, 6, 7, 8, 40, 2, 3, 63, 30, 31], np.int32)
        host = torch.empty((len(hib), H, 64, 64), dtype=torch.float32,
                           pin_memory=True)
        W.wkv7_hibernate(pool, hib, host)
        torch.cuda.synchronize()
        assert _eq_bits(host, img[torch.from_numpy(hib).long()])
        # scribble over the device copies, then resume
        W.wkv7_reset(pool, hib)
        torch.cuda.synchronize()
        W.wkv7_resume(pool, hib, host)
        torch.cuda.synchronize()
        assert _eq_bits(get_states(pool, ids_all), img)
        # resume into other slots (a different order)
        tgt = np.array([50, 51, 52, 53, 54, 55, 56, 57, 58, 59], np.int32)
        W.wkv7_resume(pool, tgt, host)
        torch.cuda.synchronize()
        exp = img.clone()
        exp[torch.from_numpy(tgt).long()] = img[torch.from_numpy(hib).long()]
        assert _eq_bits(get_states(pool, ids_all), exp)
    finally:
        W.wkv7_pool_destroy(pool)


def test_admission_and_verb_errors():
    H, n_slots = 2, 6
    pool = W.wkv7_pool_create(n_slots, H, 64)
    try:
        got = W.wkv7_slot_alloc(pool, 4)
        assert len(set(got.tolist())) == 4
        with pytest.raises(W.Wkv7Error) as e:
            W.wkv7_slot_alloc(pool, 3)
        assert e.value.status == W.WKV7_ERR_POOL_FULL
        more = W.wkv7_slot_alloc(pool, 2)       # the rest fit
        assert set(got.tolist()) | set(more.tolist()) == set(range(n_slots))
        with pytest.raises(W.Wkv7Error) as e:
            W.wkv7_slot_alloc(pool, 1)
        assert e.value.status == W.WKV7_ERR_POOL_FULL
        W.wkv7_slot_free(pool, got[:2])
        with pytest.raises(W.Wkv7Error) as e:
            W.wkv7_slot_free(pool, got[:1])     # already free
        assert e.value.status == W.WKV7_ERR_INVALID_ARG
        with pytest.raises(W.Wkv7Error) as e:
            W.wkv7_slot_free(pool, [got[2], got[2]])
        assert e.value.status == W.WKV7_ERR_DUPLICATE_SLOT
        assert len(W.wkv7_slot_alloc(pool, 2)) == 2

        ids = np.arange(n_slots, dtype=np.int32)
        img = _bits(np.random.default_rng(32), n_slots, H)
        set_states(pool, ids, img)
        bad = [
            (lambda: W.wkv7_fork(pool, [0], [6]), W.WKV7_ERR_OUT_OF_RANGE),
            (lambda: W.wkv7_fork(pool, [0, 1], [2, 2]),
             W.WKV7_ERR_DUPLICATE_SLOT),
            (lambda: W.wkv7_fork(pool, [0, 1], [1, 3]),
             W.WKV7_ERR_DUPLICATE_SLOT),
            (lambda: W.wkv7_reset(pool, [0, 0]), W.WKV7_ERR_DUPLICATE_SLOT),
            (lambda: W.wkv7_reset(pool, [-1]), W.WKV7_ERR_OUT_OF_RANGE),
            (lambda: W.wkv7_snapshot(pool, 6, torch.empty(1, device=DEV)),
             W.WKV7_ERR_OUT_OF_RANGE),
            (lambda: W.wkv7_hibernate(
                pool, [0, 1], torch.empty((1, H, 64, 64), pin_memory=True)),
             W.WKV7_ERR_INVALID_ARG),
            (lambda: W.wkv7_resume(
                pool, [0, 0], torch.empty((2, H, 64, 64), device=DEV)),
             W.WKV7_ERR_DUPLICATE_SLOT),
            (lambda: W.wkv7_pool_set_option(pool, W.WKV7_OPT_PREFILL_MIN_LEN, 0),
             W.WKV7_ERR_INVALID_ARG),
            (lambda: W.wkv7_pool_set_option(pool, 99, 1),
             W.WKV7_ERR_UNSUPPORTED),
        ]
        for fn, code in bad:
            with pytest.raises(W.Wkv7Error) as e:
                fn()
            assert e.value.status == code, e.value.message
        torch.cuda.synchronize()
        assert _eq_bits(get_states(pool, ids), img), "a failed verb wrote"
    finally:
        W.wkv7_pool_destroy(pool)


def test_new_pool_is_zero():
    pool = W.wkv7_pool_create(3, 4, 64)
    try:
        s = get_states(pool, [0, 1, 2])
        assert torch.equal(s.view(torch.int32), torch.zeros_like(s).view(torch.int32))
    finally:
        W.wkv7_pool_destroy(pool)
