"""A pool larger than 4 GiB: slot offsets beyond 2^32 bytes (GPU).

16,384 slots of H=64 heads (1 MiB each, 16 GiB). Decode, a short
multi-token sequence and a chunked prefill on slots at the start, middle and
end of the pool, through wkv7_forward and a plan, against the oracle; fork,
hibernate, resume and reset on the last slots, bit for bit.
"""
import numpy as np
import pytest
import torch

import wkv7_inputs as G
from linear_attention_rnn_amd import wkv7 as W
from oracle import wkv7_forward as oracle_forward
from tests.gpu_util import DEV, say, set_states, get_states, rel_err, tol_for

pytestmark = pytest.mark.gpu

N_SLOTS, H = 16384, 64


def test_pool_beyond_4gib():
    say(f"pool of {N_SLOTS} slots x H={H}: "
        f"{N_SLOTS * H * 64 * 64 * 4 / 2**30:.0f} GiB")
    rng = np.random.default_rng(21)
    ids = np.array([16383, 8191, 12345, 0], dtype=np.int32)
    lens = [1, 300, 5, 1]
    b = G.make_batch(rng, ids, lens, H, 64, "bf16")
    init = G.draw_states(rng, len(ids), H, 64)
    pool = W.wkv7_pool_create(N_SLOTS, H, 64)
    plan = None
    try:
        assert W.wkv7_slot_bytes(pool) * N_SLOTS > 2**32
        set_states(pool, ids, init)
        x = {n: b.inputs[n].to(DEV).contiguous() for n in G.NAMES}
        args = [x[n] for n in ("r", "w", "k", "v", "a", "b")]
        o = torch.full((b.T_tot, H, 64), float("nan"), dtype=torch.float32,
                       device=DEV)
        W.wkv7_forward(pool, b.slot_ids, b.cu_seqlens, *args, o)
        torch.cuda.synchronize()
        got_o, got_S = o.cpu(), get_states(pool, ids)
        states = {int(s): G.as_f64(init[n]) for n, s in enumerate(ids)}
        o_ref, S_ref = oracle_forward(states, b.slot_ids, b.cu_seqlens,
                                      b.inputs64(), H, 64)
        e_o = rel_err(got_o, o_ref)
        e_s = max(rel_err(got_S[n], S_ref[int(s)]) for n, s in enumerate(ids))
        say(f"  forward: o err {e_o:.3e}  S err {e_s:.3e}")
        assert e_o < tol_for("bf16") and e_s < tol_for("bf16")

        # the same batch again through a plan, from the same start states:
        # the same bits as the first call
        set_states(pool, ids, init)
        plan = W.wkv7_plan_create(pool, b.slot_ids, b.cu_seqlens)
        o2 = torch.full_like(o, float("nan"))
        W.wkv7_forward_plan(pool, plan, *args, o2)
        torch.cuda.synchronize()
        assert torch.equal(o2.cpu().view(torch.int32), got_o.view(torch.int32))
        assert torch.equal(get_states(pool, ids).view(torch.int32),
                           got_S.view(torch.int32))

        # verbs on the last slots
        W.wkv7_fork(pool, [16383], [16382])
        pair = get_states(pool, [16383, 16382])
        assert torch.equal(pair[0].view(torch.int32), pair[1].view(torch.int32))
        host = torch.empty((2, H, 64, 64), dtype=torch.float32, pin_memory=True)
        W.wkv7_hibernate(pool, [16382, 8191], host)
        torch.cuda.synchronize()
        W.wkv7_reset(pool, [16382, 8191])
        assert not get_states(pool, [16382, 8191]).any()
        W.wkv7_resume(pool, [16382, 8191], host)
        back = get_states(pool, [16382, 8191])
        assert torch.equal(back.view(torch.int32), host.view(torch.int32))
        assert torch.equal(back[1].view(torch.int32), got_S[1].view(torch.int32))
        say("  verbs: fork, hibernate, reset, resume bit-exact")
    finally:
        if plan is not None:
            W.wkv7_plan_destroy(plan)
        W.wkv7_pool_destroy(pool)
