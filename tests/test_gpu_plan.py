"""Plans: metadata validated once and kept on the device, launched without
any host work, and captured into a HIP graph (GPU)."""
import numpy as np
import pytest
import torch

import wkv7_inputs as G
from linear_attention_rnn_amd import wkv7 as W
from oracle import wkv7_forward as oracle_forward
from tests.gpu_util import (DEV, say, set_states, get_states, to_dev,
                            rel_err, tol_for)

pytestmark = pytest.mark.gpu

H = 4
LENS = [1, 1, 70, 1, 3, 130, 1, 64]        # decode tokens and ragged prefills


def _bits_equal(a, b):
    return torch.equal(a.contiguous().view(torch.int32),
                       b.contiguous().view(torch.int32))


def _pool_with_states(ids, init):
    pool = W.wkv7_pool_create(16, H, 64)
    set_states(pool, ids, init)
    return pool


def _batch(seed, ids):
    return G.make_batch(np.random.default_rng(seed), ids, LENS, H, 64, G.BF16)


def test_plan_matches_forward_bitwise():
    ids = np.array([9, 2, 14, 0, 5, 7, 11, 3], np.int32)
    init = G.draw_states(np.random.default_rng(21), len(ids), H, 64)
    b = _batch(22, ids)
    x = to_dev(b)
    pa, pb = _pool_with_states(ids, init), _pool_with_states(ids, init)
    plan = W.wkv7_plan_create(pb, ids, b.cu_seqlens)
    try:
        assert W.wkv7_plan_tokens(plan) == b.T_tot
        oa = torch.empty((b.T_tot, H, 64), dtype=torch.float32, device=DEV)
        ob = torch.empty_like(oa)
        for _ in range(2):          # two steps: the state carries over
            W.wkv7_forward(pa, ids, b.cu_seqlens, x["r"], x["w"], x["k"],
                           x["v"], x["a"], x["b"], oa)
            W.wkv7_forward_plan(pb, plan, x["r"], x["w"], x["k"], x["v"],
                                x["a"], x["b"], ob)
            torch.cuda.synchronize()
            assert _bits_equal(oa, ob)
        assert _bits_equal(get_states(pa, ids), get_states(pb, ids))
        say("plan forward == forward, bit for bit, over two steps")
    finally:
        W.wkv7_plan_destroy(plan)
        W.wkv7_pool_destroy(pa)
        W.wkv7_pool_destroy(pb)


def test_plan_rejects_what_forward_rejects():
    pool = W.wkv7_pool_create(8, H, 64)
    other = W.wkv7_pool_create(8, H, 64)
    try:
        cases = [
            (([1, 1], [0, 1, 2]), W.WKV7_ERR_DUPLICATE_SLOT),
            (([1, 8], [0, 1, 2]), W.WKV7_ERR_OUT_OF_RANGE),
            (([1, -1], [0, 1, 2]), W.WKV7_ERR_OUT_OF_RANGE),
            (([1, 2], [0, 2, 1]), W.WKV7_ERR_INVALID_ARG),
            (([1, 2], [1, 2, 3]), W.WKV7_ERR_INVALID_ARG),
        ]
        for (ids, cu), code in cases:
            with pytest.raises(W.Wkv7Error) as e:
                W.wkv7_plan_create(pool, ids, cu)
            assert e.value.status == code, (ids, cu)
        plan = W.wkv7_plan_create(pool, [3], [0, 1])
        try:
            x = {n: torch.zeros((1, H, 64), dtype=torch.bfloat16, device=DEV)
                 for n in G.NAMES}
            o = torch.empty((1, H, 64), dtype=torch.float32, device=DEV)
            with pytest.raises(W.Wkv7Error) as e:
                W.wkv7_forward_plan(other, plan, x["r"], x["w"], x["k"],
                                    x["v"], x["a"], x["b"], o)
            assert e.value.status == W.WKV7_ERR_INVALID_ARG
            with pytest.raises(W.Wkv7Error) as e:
                W.wkv7_forward_plan(pool, plan, x["r"], x["w"], x["k"],
                                    x["v"], x["a"], x["b"], o, dtype=7)
            assert e.value.status == W.WKV7_ERR_UNSUPPORTED
        finally:
            W.wkv7_plan_destroy(plan)
        # an empty plan is valid and launches nothing
        empty = W.wkv7_plan_create(pool, [], [0])
        W.wkv7_forward_plan(pool, empty, *([None] * 7), dtype=W.WKV7_BF16)
        W.wkv7_plan_destroy(empty)
    finally:
        W.wkv7_pool_destroy(pool)
        W.wkv7_pool_destroy(other)


def test_graph_of_plan_steps_replays_like_eager():
    """Capture 3 steps (decode and prefill kernels) into one HIP graph;
    replay it 4 times with new inputs copied into its buffers and eager work
    in between; every replay equals the same steps run eagerly on a twin
    pool, bit for bit, and the first matches the oracle."""
    ids = np.array([4, 12, 1, 6, 15, 8, 10, 13], np.int32)
    init = G.draw_states(np.random.default_rng(31), len(ids), H, 64)
    ga, eb = _pool_with_states(ids, init), _pool_with_states(ids, init)
    n_steps, n_replays = 3, 4
    batches = [[_batch(1000 * r + s, ids) for s in range(n_steps)]
               for r in range(n_replays)]
    T = batches[0][0].T_tot
    bufs = [{n: torch.empty((T, H, 64), dtype=torch.bfloat16, device=DEV)
             for n in G.NAMES} for _ in range(n_steps)]
    outs = [torch.empty((T, H, 64), dtype=torch.float32, device=DEV)
            for _ in range(n_steps)]
    plan_a = W.wkv7_plan_create(ga, ids, batches[0][0].cu_seqlens)
    plan_b = W.wkv7_plan_create(eb, ids, batches[0][0].cu_seqlens)
    try:
        graph = torch.cuda.CUDAGraph()
        # capture only (on torch's capture stream, which is current inside
        # the block): the kernels run when the graph is replayed
        with torch.cuda.graph(graph):
            for s in range(n_steps):
                x = bufs[s]
                W.wkv7_forward_plan(ga, plan_a, x["r"], x["w"], x["k"],
                                    x["v"], x["a"], x["b"], outs[s])
        torch.cuda.synchronize()
        for r in range(n_replays):
            S_before = get_states(eb, ids)
            for s in range(n_steps):
                for n in G.NAMES:
                    bufs[s][n].copy_(batches[r][s].inputs[n].to(DEV))
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            got = [o.cpu() for o in outs]
            # the same steps eagerly on the twin pool
            for s in range(n_steps):
                x = to_dev(batches[r][s])
                o = torch.empty((T, H, 64), dtype=torch.float32, device=DEV)
                W.wkv7_forward_plan(eb, plan_b, x["r"], x["w"], x["k"],
                                    x["v"], x["a"], x["b"], o)
                torch.cuda.synchronize()
                assert _bits_equal(got[s], o.cpu()), (r, s)
            Sa, Sb = get_states(ga, ids), get_states(eb, ids)
            assert _bits_equal(Sa, Sb), r
            if r == 0:
                st = {int(i): G.as_f64(S_before[n]) for n, i in enumerate(ids)}
                err = 0.0
                for s in range(n_steps):
                    b = batches[r][s]
                    o_ref, st = oracle_forward(st, ids, b.cu_seqlens,
                                               b.inputs64(), H, 64)
                    err = max(err, rel_err(got[s], o_ref))
                err = max(err, max(rel_err(Sa[n], st[int(i)])
                                   for n, i in enumerate(ids)))
                say(f"graph replay 0 vs oracle: {err:.3e}")
                assert err < 1e-2 and err < tol_for("bf16")
            say(f"graph replay {r}: equal to eager, bit for bit")
        del graph
    finally:
        W.wkv7_plan_destroy(plan_a)
        W.wkv7_plan_destroy(plan_b)
        W.wkv7_pool_destroy(ga)
        W.wkv7_pool_destroy(eb)
