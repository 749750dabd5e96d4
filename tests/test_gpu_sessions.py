"""Sessions over a real pool (GPU): a multi-turn conversation reuses the
parked state, matches the oracle run on the whole history, survives
eviction to host memory bit for bit, and restarts from zero on an edit."""
import numpy as np
import pytest
import torch

import wkv7_inputs as G
from linear_attention_rnn_amd import wkv7 as W
from oracle import wkv7_sequence
from tests.gpu_util import DEV, say, get_states, rel_err

pytestmark = pytest.mark.gpu
H, V = 2, 64


def _bits_equal(a, b):
    return torch.equal(a.contiguous().view(torch.int32),
                       b.contiguous().view(torch.int32))


class Vocab:
    """Per-token WKV inputs looked up by token id (a stand-in for the
    projections of a token's embedding), bf16 on the device and the same
    values in float64 for the oracle."""

    def __init__(self, seed):
        b = G.make_batch(np.random.default_rng(seed), np.array([0], np.int32),
                         [V], H, 64, G.BF16)
        self.dev = {n: b.inputs[n].to(DEV) for n in G.NAMES}
        self.f64 = b.inputs64()

    def run(self, pool, slot, toks):
        idx = torch.tensor(np.asarray(toks), dtype=torch.long, device=DEV)
        x = {n: self.dev[n].index_select(0, idx).contiguous() for n in G.NAMES}
        o = torch.empty((len(toks), H, 64), dtype=torch.float32, device=DEV)
        W.wkv7_forward(pool, [slot], [0, len(toks)], x["r"], x["w"], x["k"],
                       x["v"], x["a"], x["b"], o)
        torch.cuda.synchronize()

    def oracle_state(self, toks):
        t = np.asarray(toks)
        _, S = wkv7_sequence(np.zeros((H, 64, 64)),
                             **{n: self.f64[n][t] for n in G.NAMES})
        return S


def test_conversation_reuse_eviction_and_edit():
    voc = Vocab(51)
    rng = np.random.default_rng(52)
    pool = W.wkv7_pool_create(2, H, 64)
    s = W.wkv7_sessions_create(pool, 0, 1, 0)
    try:
        # turn 1: a 70-token prompt (chunked kernel), 5 decoded answer tokens
        p1 = list(rng.integers(0, V, 70))
        slot, reuse, oc = W.wkv7_session_begin(s, 1, 1, 1, 0, p1)
        assert (reuse, oc) == (0, W.WKV7_SESSION_NEW)
        voc.run(pool, slot, p1)
        a1 = list(rng.integers(0, V, 5))
        for t in a1:
            voc.run(pool, slot, [t])
        h1 = p1 + a1
        W.wkv7_session_end(s, slot, 100, h1)
        # turn 2 continues: only the new prompt runs
        h2 = h1 + list(rng.integers(0, V, 3))
        slot, reuse, oc = W.wkv7_session_begin(s, 1, 1, 1, 100, h2)
        assert (reuse, oc) == (len(h1), W.WKV7_SESSION_HIT)
        voc.run(pool, slot, h2[reuse:])
        for t in rng.integers(0, V, 4):
            h2.append(int(t))
            voc.run(pool, slot, [int(t)])
        err = rel_err(get_states(pool, [slot])[0], voc.oracle_state(h2))
        say(f"turn 2 state vs oracle on the whole history: {err:.3e}")
        assert err < 1e-2
        W.wkv7_session_end(s, slot, 101, h2)
        parked = get_states(pool, [slot])
        # two other chats take both slots: chat 1 moves to host memory
        for chat in (2, 3):
            sl, _, oc = W.wkv7_session_begin(s, 1, 1, chat, 0, [1, 2, 3])
            assert oc == W.WKV7_SESSION_NEW
            voc.run(pool, sl, [1, 2, 3])
            W.wkv7_session_end(s, sl, 200 + chat, [1, 2, 3])
        st = W.wkv7_sessions_stats(s)
        assert (st["hibernates"], st["parked_host"]) == (1, 1)
        # chat 1 continues: its state comes back bit for bit
        h3 = h2 + [5, 6]
        slot, reuse, oc = W.wkv7_session_begin(s, 1, 1, 1, 101, h3)
        assert (reuse, oc) == (len(h2), W.WKV7_SESSION_HIT)
        assert _bits_equal(get_states(pool, [slot]), parked)
        voc.run(pool, slot, h3[reuse:])
        err = rel_err(get_states(pool, [slot])[0], voc.oracle_state(h3))
        say(f"turn 3 (after host parking) vs oracle: {err:.3e}")
        assert err < 1e-2
        W.wkv7_session_end(s, slot, 102, h3)
        # an edited first message restarts from a zero state
        sl, reuse, oc = W.wkv7_session_begin(s, 1, 1, 1, 102, [9] + h3[1:])
        assert (reuse, oc) == (0, W.WKV7_SESSION_RESTART_EDIT)
        assert not get_states(pool, [sl]).any()
        W.wkv7_session_abort(s, sl)
        say(f"stats: {W.wkv7_sessions_stats(s)}")
    finally:
        W.wkv7_sessions_destroy(s)
        W.wkv7_pool_destroy(pool)


def test_keep_parent_fork_is_exact():
    voc = Vocab(53)
    pool = W.wkv7_pool_create(3, H, 64)
    s = W.wkv7_sessions_create(pool, 0, 0, W.WKV7_SESSIONS_KEEP_PARENT)
    try:
        toks = list(np.random.default_rng(54).integers(0, V, 40))
        slot, _, _ = W.wkv7_session_begin(s, 1, 1, 1, 0, toks)
        voc.run(pool, slot, toks)
        W.wkv7_session_end(s, slot, 100, toks)
        parent = get_states(pool, [slot])
        for _ in range(2):              # answer, then regenerate
            sl, reuse, oc = W.wkv7_session_begin(s, 1, 1, 1, 100, toks + [3])
            assert (reuse, oc) == (len(toks), W.WKV7_SESSION_HIT)
            assert sl != slot
            assert _bits_equal(get_states(pool, [sl]), parent)
            voc.run(pool, sl, [3])
            W.wkv7_session_abort(s, sl)
        assert _bits_equal(get_states(pool, [slot]), parent)
    finally:
        W.wkv7_sessions_destroy(s)
        W.wkv7_pool_destroy(pool)
