"""The session manager against a model of its documented policy, on random
turn sequences (CPU; host-only managers, which count the device work they
would do).

The model follows the contract the session header states: a parked state is
reused only by a turn of the same model, user and chat whose parent is the
parked message and whose history extends the parked one (hit); otherwise
the turn restarts (edit, unknown parent, or a parent whose state admission
dropped); a turn needs a device slot, and when none is free the least
recently used parked state on the device (used = parked, or hit) moves to
a host image, the least recently used host image being dropped first when
all are taken (no host images: the device state is dropped); turns in flight
are never moved; with KEEP_PARENT a hit forks (or resumes) into a new slot
and leaves the parent parked. Which free slot a turn gets is not part of the
contract: the model checks that it is free and then follows it.

After every call the outcome, the reused length, the slot and the
manager's counters and occupancy must agree with the model.
"""
import numpy as np
import pytest

from linear_attention_rnn_amd import wkv7 as W

HIT = W.WKV7_SESSION_HIT
NEW = W.WKV7_SESSION_NEW
EDIT = W.WKV7_SESSION_RESTART_EDIT
PARENT = W.WKV7_SESSION_RESTART_PARENT
EVICTED = W.WKV7_SESSION_RESTART_EVICTED
COUNTERS = ("hits", "news", "restarts_edit", "restarts_parent",
            "restarts_evicted", "resets", "forks", "hibernates", "resumes",
            "drops")


class PoolFull(Exception):
    pass


class Model:
    def __init__(self, n_slots, n_images, keep):
        self.n_slots, self.n_images, self.keep = n_slots, n_images, keep
        self.active = {}        # slot -> chat (model, user, chat)
        self.parked = {}        # (model, user, chat, message) -> [tokens, slot or None, last use]
        self.evicted = set()
        self.clock = 0
        self.c = dict.fromkeys(COUNTERS, 0)

    def free_slots(self):
        used = set(self.active) | {p[1] for p in self.parked.values()
                                   if p[1] is not None}
        return set(range(self.n_slots)) - used

    def n_host(self):
        return sum(1 for p in self.parked.values() if p[1] is None)

    def drop(self, k, evicted):
        del self.parked[k]
        if evicted:
            self.evicted.add(k)
        self.c["drops"] += 1

    def lru(self, on_device, pinned):
        cand = [(p[2], k) for k, p in self.parked.items()
                if k != pinned and (p[1] is not None) == on_device]
        return min(cand)[1] if cand else None

    def make_room(self, pinned):
        """Evict until a device slot is free (admission)."""
        while not self.free_slots():
            d = self.lru(True, pinned)
            if d is None:
                raise PoolFull
            if self.n_host() == self.n_images:
                h = self.lru(False, pinned)
                if h is not None:
                    self.drop(h, True)
            if self.n_host() < self.n_images:
                self.parked[d][1] = None          # moved to a host image
                self.c["hibernates"] += 1
            else:
                self.drop(d, True)

    def begin(self, chat, parent, tokens):
        """Expected (outcome, n_reuse, slot or None = any free slot); state
        is updated after the caller confirms the slot (take)."""
        want = chat + (parent,)
        r = self.parked.get(want) if parent else None
        if r is not None and list(tokens[:len(r[0])]) == r[0] and \
                len(r[0]) <= len(tokens):
            oc = HIT
        elif r is not None:
            oc = EDIT
        elif parent == 0:
            oc = NEW
        elif want in self.evicted:
            oc = EVICTED
        else:
            oc = PARENT
        if oc == HIT:
            self.clock += 1
            r[2] = self.clock
            if not self.keep and r[1] is not None:
                return oc, len(r[0]), r[1], want
            self.make_room(want)
            return oc, len(r[0]), None, want
        self.make_room(None)
        return oc, 0, None, want

    def take(self, oc, want, slot):
        chat = want[:3]
        if oc == HIT:
            r = self.parked[want]
            if self.keep:
                self.c["forks" if r[1] is not None else "resumes"] += 1
            else:
                if r[1] is None:
                    self.c["resumes"] += 1
                del self.parked[want]
            self.c["hits"] += 1
        else:
            self.c["resets"] += 1
            self.c[{NEW: "news", EDIT: "restarts_edit",
                    EVICTED: "restarts_evicted",
                    PARENT: "restarts_parent"}[oc]] += 1
        self.active[slot] = chat

    def end(self, slot, message, tokens):
        chat = self.active.pop(slot)
        k = chat + (message,)
        if k in self.parked:
            self.drop(k, False)
        self.clock += 1
        self.parked[k] = [list(tokens), slot, self.clock]
        self.evicted.discard(k)

    def abort(self, slot):
        del self.active[slot]

    def drop_chat(self, chat):
        for k in [k for k in self.parked if k[:3] == chat]:
            self.drop(k, False)


def check(s, m):
    st = W.wkv7_sessions_stats(s)
    for n in COUNTERS:
        assert st[n] == m.c[n], (n, st[n], m.c[n])
    assert st["active"] == len(m.active)
    assert st["parked_device"] == len(m.parked) - m.n_host()
    assert st["parked_host"] == m.n_host()
    assert st["free_host_images"] == m.n_images - m.n_host()


@pytest.mark.parametrize("seed", range(24))
def test_random_turns_follow_the_policy(seed):
    rng = np.random.default_rng(700 + seed)
    n_slots = int(rng.integers(1, 6))
    n_images = int(rng.integers(0, 4))
    keep = bool(rng.integers(0, 2))
    s = W.wkv7_sessions_create(None, n_slots, n_images,
                               W.WKV7_SESSIONS_KEEP_PARENT if keep else 0)
    m = Model(n_slots, n_images, keep)
    chats = [(1, 10, c) for c in range(1, 5)] + [(1, 11, 1), (2, 10, 1)]
    history = {c: [] for c in chats}      # (message, tokens) the chat ended with
    flight = {}                            # slot -> (chat, tokens)
    next_msg = 100
    try:
        for _ in range(300):
            op = rng.random()
            if op < 0.5 or not flight:
                chat = chats[int(rng.integers(len(chats)))]
                h = history[chat]
                kind = rng.random()
                if not h or kind < 0.15:
                    parent, tokens = 0, list(rng.integers(1, 50, size=rng.integers(1, 6)))
                elif kind < 0.65:                      # continue the last message
                    parent, prev = h[-1]
                    tokens = prev + list(rng.integers(1, 50, size=rng.integers(0, 4)))
                elif kind < 0.8:                       # branch from an older one
                    parent, prev = h[int(rng.integers(len(h)))]
                    tokens = prev + [int(rng.integers(1, 50))]
                elif kind < 0.9:                       # edit an earlier token
                    parent, prev = h[-1]
                    tokens = list(prev) + [7]
                    tokens[int(rng.integers(len(tokens)))] += 1000
                else:                                  # a parent never seen
                    parent, tokens = 99999, [1, 2, 3]
                try:
                    oc, reuse, slot, want = m.begin(chat, parent, tokens)
                except PoolFull:
                    with pytest.raises(W.Wkv7Error) as e:
                        W.wkv7_session_begin(s, *chat, parent, tokens)
                    assert e.value.status == W.WKV7_ERR_POOL_FULL
                    check(s, m)
                    continue
                free = m.free_slots()
                got = W.wkv7_session_begin(s, *chat, parent, tokens)
                assert got[2] == oc and got[1] == reuse, (got, oc, reuse)
                if slot is not None:
                    assert got[0] == slot
                else:
                    assert got[0] in free, (got[0], free)
                m.take(oc, want, got[0])
                flight[got[0]] = (chat, tokens)
            elif op < 0.85:
                slot = list(flight)[int(rng.integers(len(flight)))]
                chat, tokens = flight.pop(slot)
                full = tokens + list(rng.integers(1, 50, size=rng.integers(1, 4)))
                msg = next_msg
                if history[chat] and rng.random() < 0.1:
                    msg = history[chat][int(rng.integers(len(history[chat])))][0]
                else:
                    next_msg += 1
                W.wkv7_session_end(s, slot, msg, full)
                m.end(slot, msg, full)
                history[chat] = [(a, b) for a, b in history[chat] if a != msg]
                history[chat].append((msg, full))
            elif op < 0.97:
                slot = list(flight)[int(rng.integers(len(flight)))]
                flight.pop(slot)
                W.wkv7_session_abort(s, slot)
                m.abort(slot)
            else:
                chat = chats[int(rng.integers(len(chats)))]
                W.wkv7_session_drop_chat(s, *chat)
                m.drop_chat(chat)
            check(s, m)
    finally:
        W.wkv7_sessions_destroy(s)
