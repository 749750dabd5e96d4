"""hibernate/resume of scattered slots (GPU): the staged path (a gather or
scatter kernel plus one DMA per group of slots), its several-group case,
resume straight from a device buffer, and the per-run DMA path for ids with
few runs. Every image is compared bit for bit with the pool's own memory,
read through the pool's buffer rather than through hibernate."""
import numpy as np
import pytest
import torch

from linear_attention_rnn_amd import wkv7 as W
from tests.gpu_util import DEV, say

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.contiguous().view(torch.int32)


def _fill(pool, seed):
    view = W.pool_state(pool)
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    view.copy_(torch.randn(view.shape, generator=g, device=DEV))
    torch.cuda.synchronize()
    return view


@pytest.mark.parametrize("H,n_slots,n_ids", [(64, 200, 150), (3, 600, 500)])
def test_scattered_hibernate_resume_bitexact(H, n_slots, n_ids):
    # H=64: 1 MiB slots, 64 per staging group, so 150 ids take three groups
    say(f"xfer H={H} slots={n_slots} ids={n_ids}")
    rng = np.random.default_rng(H)
    pool = W.wkv7_pool_create(n_slots, H, 64)
    try:
        view = _fill(pool, 7)
        ids = rng.permutation(n_slots)[:n_ids].astype(np.int32)
        ids[-1] = ids[0]                       # hibernate allows repeats
        host = torch.empty((n_ids, H, 64, 64), dtype=torch.float32,
                           pin_memory=True)
        W.wkv7_hibernate(pool, ids, host)
        torch.cuda.synchronize()
        want = view[torch.from_numpy(ids).long().to(DEV)].cpu()
        assert torch.equal(_bits(host), _bits(want))

        # resume the images into other scattered, distinct slots
        dst = rng.permutation(n_slots)[:n_ids - 1].astype(np.int32)
        before = view.clone()
        W.wkv7_resume(pool, dst, host[:n_ids - 1])
        torch.cuda.synchronize()
        expect = before.clone()
        expect[torch.from_numpy(dst).long().to(DEV)] = host[:n_ids - 1].to(DEV)
        assert torch.equal(_bits(view), _bits(expect))
    finally:
        W.wkv7_pool_destroy(pool)


@pytest.mark.parametrize("offset_floats", [0, 1])
def test_resume_from_device_buffer(offset_floats):
    # aligned: one scatter kernel from the buffer; misaligned by 4 bytes:
    # the staged path with a device-to-device DMA
    say(f"xfer resume from device, offset {offset_floats}")
    H, n_slots, n = 4, 64, 40
    rng = np.random.default_rng(3)
    pool = W.wkv7_pool_create(n_slots, H, 64)
    try:
        view = _fill(pool, 8)
        flat = torch.randn(n * H * 64 * 64 + offset_floats, device=DEV)
        src = flat[offset_floats:]
        dst = rng.permutation(n_slots)[:n].astype(np.int32)
        before = view.clone()
        W.wkv7_resume(pool, dst, src)
        torch.cuda.synchronize()
        expect = before.clone()
        expect[torch.from_numpy(dst).long().to(DEV)] = src.view(n, H, 64, 64)
        assert torch.equal(_bits(view), _bits(expect))
    finally:
        W.wkv7_pool_destroy(pool)


def test_few_runs_take_direct_copies():
    say("xfer few runs")
    H = 2
    pool = W.wkv7_pool_create(32, H, 64)
    try:
        view = _fill(pool, 9)
        ids = np.array([5, 6, 7, 20, 21], np.int32)      # two runs
        host = torch.empty((5, H, 64, 64), dtype=torch.float32,
                           pin_memory=True)
        W.wkv7_hibernate(pool, ids, host)
        torch.cuda.synchronize()
        assert torch.equal(_bits(host),
                           _bits(view[torch.from_numpy(ids).long().to(DEV)].cpu()))
        host2 = torch.randn((5, H, 64, 64)).pin_memory()
        W.wkv7_resume(pool, ids, host2)
        torch.cuda.synchronize()
        assert torch.equal(_bits(view[torch.from_numpy(ids).long().to(DEV)].cpu()),
                           _bits(host2))
    finally:
        W.wkv7_pool_destroy(pool)


def test_staging_is_reused_across_calls_and_pools_stay_separate():
    say("xfer repeated calls")
    H = 64
    a = W.wkv7_pool_create(100, H, 64)
    b = W.wkv7_pool_create(100, H, 64)
    try:
        va, vb = _fill(a, 10), _fill(b, 11)
        rng = np.random.default_rng(5)
        host = torch.empty((70, H, 64, 64), dtype=torch.float32,
                           pin_memory=True)
        for rep in range(3):
            ids = rng.permutation(100)[:70 - 20 * rep].astype(np.int32)
            m = len(ids)
            W.wkv7_hibernate(a, ids, host[:m])
            W.wkv7_resume(b, ids[::-1].copy(), host[:m])
            torch.cuda.synchronize()
            got = vb[torch.from_numpy(ids[::-1].copy()).long().to(DEV)]
            want = va[torch.from_numpy(ids).long().to(DEV)]
            assert torch.equal(_bits(got), _bits(want))
    finally:
        W.wkv7_pool_destroy(a)
        W.wkv7_pool_destroy(b)
