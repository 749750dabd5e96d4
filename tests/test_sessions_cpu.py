"""The session layer's policy on the CPU: a host-only manager (no pool)
that counts the device work it would do. Covers the parent-token binding
(hit, edit, branch or stale parent, eviction), LRU admission with host
parking, keep-parent forks, abort, drop and the error paths."""
import pytest

from linear_attention_rnn_amd import wkv7 as W

HIT = W.WKV7_SESSION_HIT
NEW = W.WKV7_SESSION_NEW
EDIT = W.WKV7_SESSION_RESTART_EDIT
PARENT = W.WKV7_SESSION_RESTART_PARENT
EVICTED = W.WKV7_SESSION_RESTART_EVICTED
MODEL, USER = 7, 11


@pytest.fixture
def mk():
    made = []

    def make(dry_slots=4, host_images=0, flags=0):
        s = W.wkv7_sessions_create(None, dry_slots, host_images, flags)
        made.append(s)
        return s
    yield make
    for s in made:
        W.wkv7_sessions_destroy(s)


def turn(s, chat, parent, tokens):
    return W.wkv7_session_begin(s, MODEL, USER, chat, parent, tokens)


def test_first_turn_then_hit_reuses_the_slot(mk):
    s = mk()
    slot, reuse, oc = turn(s, 1, 0, [5, 6, 7])
    assert (reuse, oc) == (0, NEW)
    W.wkv7_session_end(s, slot, 100, [5, 6, 7, 8, 9])      # prompt + answer
    slot2, reuse2, oc2 = turn(s, 1, 100, [5, 6, 7, 8, 9, 10, 11])
    assert (slot2, reuse2, oc2) == (slot, 5, HIT)
    st = W.wkv7_sessions_stats(s)
    assert (st["hits"], st["news"], st["resets"]) == (1, 1, 1)
    assert (st["active"], st["parked_device"]) == (1, 0)


def test_restart_reasons(mk):
    s = mk()
    slot, _, _ = turn(s, 1, 0, [1, 2])
    W.wkv7_session_end(s, slot, 100, [1, 2, 3])
    # an edited earlier message: same parent, different history
    slot, reuse, oc = turn(s, 1, 100, [1, 9, 3, 4])
    assert (reuse, oc) == (0, EDIT)
    W.wkv7_session_abort(s, slot)
    # a history that is shorter than what the state consumed cannot reuse it
    slot, reuse, oc = turn(s, 1, 100, [1, 2])
    assert (reuse, oc) == (0, EDIT)
    W.wkv7_session_abort(s, slot)
    # a parent this chat has no state for (branch from elsewhere, stale id)
    slot, reuse, oc = turn(s, 1, 555, [1, 2, 3, 4])
    assert (reuse, oc) == (0, PARENT)
    W.wkv7_session_abort(s, slot)
    # another user or model never matches
    slot, reuse, oc = W.wkv7_session_begin(s, MODEL, USER + 1, 1, 100, [1, 2, 3])
    assert oc == PARENT
    W.wkv7_session_abort(s, slot)
    slot, reuse, oc = W.wkv7_session_begin(s, MODEL + 1, USER, 1, 100, [1, 2, 3])
    assert oc == PARENT
    W.wkv7_session_abort(s, slot)
    # the parked state is still there for a real continuation
    slot, reuse, oc = turn(s, 1, 100, [1, 2, 3, 4])
    assert (reuse, oc) == (3, HIT)
    st = W.wkv7_sessions_stats(s)
    assert (st["restarts_edit"], st["restarts_parent"]) == (2, 3)


def test_lru_eviction_to_host_and_back(mk):
    """Two slots, one host image. Each step's expected state is spelled out;
    LRU order follows the last begin or end of each chat."""
    s = mk(dry_slots=2, host_images=1)
    slots = {}
    for chat in (1, 2):
        slot, _, oc = turn(s, chat, 0, [chat])
        assert oc == NEW
        W.wkv7_session_end(s, slot, 10 * chat, [chat, chat])
        slots[chat] = slot
    # chat 3 needs a slot: chat 1 (least recently used) moves to host
    slot3, _, oc = turn(s, 3, 0, [3])
    assert oc == NEW and slot3 == slots[1]
    st = W.wkv7_sessions_stats(s)
    assert (st["hibernates"], st["parked_host"], st["parked_device"]) == (1, 1, 1)
    W.wkv7_session_end(s, slot3, 30, [3, 3])
    # chat 1 continues from host: it needs a slot, chat 2 is the LRU device
    # state, and the only host image still holds chat 1, so chat 2 is dropped
    slot1, reuse, oc = turn(s, 1, 10, [1, 1, 4])
    assert (reuse, oc) == (2, HIT) and slot1 == slots[2]
    st = W.wkv7_sessions_stats(s)
    assert (st["resumes"], st["drops"], st["parked_host"]) == (1, 1, 0)
    assert st["free_host_images"] == 1
    W.wkv7_session_end(s, slot1, 11, [1, 1, 4, 4])
    # chat 4: chat 3 (LRU) moves to the free host image
    slot, _, oc = turn(s, 4, 0, [4])
    assert oc == NEW
    W.wkv7_session_end(s, slot, 40, [4, 4])
    # chat 5: chat 1 is LRU on the device; the host image holds chat 3, which
    # is dropped so that chat 1 can move there
    slot, _, oc = turn(s, 5, 0, [5])
    assert oc == NEW
    W.wkv7_session_end(s, slot, 50, [5, 5])
    st = W.wkv7_sessions_stats(s)
    assert (st["hibernates"], st["drops"]) == (3, 2)
    assert (st["parked_device"], st["parked_host"]) == (2, 1)
    # chat 1 is on the host: a hit (chat 4, now LRU, moves out for it)
    slot, reuse, oc = turn(s, 1, 11, [1, 1, 4, 4, 7])
    assert (reuse, oc) == (4, HIT)
    W.wkv7_session_abort(s, slot)
    assert turn_abort(s, 2, 20, [2, 2, 9]) == EVICTED
    assert turn_abort(s, 3, 30, [3, 3, 9]) == EVICTED


def turn_abort(s, chat, parent, tokens):
    slot, _, oc = turn(s, chat, parent, tokens)
    W.wkv7_session_abort(s, slot)
    return oc


def test_no_host_parking_drops_and_pool_full(mk):
    s = mk(dry_slots=2, host_images=0)
    a, _, _ = turn(s, 1, 0, [1])
    turn(s, 2, 0, [2])
    with pytest.raises(W.Wkv7Error) as e:          # both slots in flight
        turn(s, 3, 0, [3])
    assert e.value.status == W.WKV7_ERR_POOL_FULL
    W.wkv7_session_end(s, a, 10, [1, 1])
    c, _, oc = turn(s, 3, 0, [3])                  # chat 1's state is dropped
    assert oc == NEW and c == a
    W.wkv7_session_abort(s, c)
    st = W.wkv7_sessions_stats(s)
    assert st["drops"] == 1 and st["hibernates"] == 0
    slot, _, oc = turn(s, 1, 10, [1, 1, 2])
    assert oc == EVICTED


def test_keep_parent_forks_for_regenerate(mk):
    s = mk(dry_slots=3, flags=W.WKV7_SESSIONS_KEEP_PARENT)
    slot, _, _ = turn(s, 1, 0, [1, 2])
    W.wkv7_session_end(s, slot, 100, [1, 2, 3])
    first, reuse, oc = turn(s, 1, 100, [1, 2, 3, 4])
    assert (reuse, oc) == (3, HIT) and first != slot
    W.wkv7_session_abort(s, first)                 # "regenerate"
    again, reuse, oc = turn(s, 1, 100, [1, 2, 3, 5])
    assert (reuse, oc) == (3, HIT)
    st = W.wkv7_sessions_stats(s)
    assert st["forks"] == 2 and st["parked_device"] == 1


def test_end_replaces_and_drop_chat(mk):
    s = mk(dry_slots=3)
    slot, _, _ = turn(s, 1, 0, [1])
    W.wkv7_session_end(s, slot, 100, [1, 2])
    other, _, oc = turn(s, 1, 0, [1])              # a second first turn
    assert oc == NEW
    W.wkv7_session_end(s, other, 100, [1, 3])      # same message id: replaces
    st = W.wkv7_sessions_stats(s)
    assert st["parked_device"] == 1 and st["drops"] == 1
    assert turn_abort(s, 1, 100, [1, 2, 4]) == EDIT
    W.wkv7_session_drop_chat(s, MODEL, USER, 1)
    assert W.wkv7_sessions_stats(s)["parked_device"] == 0
    assert turn_abort(s, 1, 100, [1, 3, 4]) == PARENT


def test_session_errors(mk):
    s = mk(dry_slots=1)
    with pytest.raises(W.Wkv7Error) as e:
        W.wkv7_session_end(s, 0, 1, [1])           # slot 0 holds no turn
    assert e.value.status == W.WKV7_ERR_INVALID_ARG
    slot, _, _ = turn(s, 1, 0, [1])
    with pytest.raises(W.Wkv7Error) as e:
        W.wkv7_session_end(s, slot, 0, [1])        # message id 0
    assert e.value.status == W.WKV7_ERR_INVALID_ARG
    with pytest.raises(W.Wkv7Error) as e:
        W.wkv7_session_abort(s, slot + 1)
    assert e.value.status == W.WKV7_ERR_INVALID_ARG
    for args in [(0, 0, 0),        # a host-only manager needs slots
                 (1, -1, 0),       # negative host images
                 (1, 0, 8)]:       # unknown flag
        with pytest.raises(W.Wkv7Error) as e:
            W.wkv7_sessions_create(None, *args)
        assert e.value.status == W.WKV7_ERR_INVALID_ARG, args
    assert W.lib.wkv7_sessions_destroy(None) == W.WKV7_OK


def test_every_turn_uses_the_first_turns_stream(mk):
    """The manager's own device work is ordered after a slot's last forward
    only through one stream, so a turn on another stream is refused (a
    host-only manager never touches the handles)."""
    s = mk()
    slot, _, _ = W.wkv7_session_begin(s, MODEL, USER, 1, 0, [1, 2],
                                      stream=0x1000)
    W.wkv7_session_end(s, slot, 100, [1, 2, 3])
    before = W.wkv7_sessions_stats(s)
    with pytest.raises(W.Wkv7Error) as ei:
        W.wkv7_session_begin(s, MODEL, USER, 1, 100, [1, 2, 3, 4],
                             stream=0x2000)
    assert ei.value.status == W.WKV7_ERR_INVALID_ARG
    assert "stream" in ei.value.message
    assert W.wkv7_sessions_stats(s) == before     # nothing moved or counted
    slot2, reuse, oc = W.wkv7_session_begin(s, MODEL, USER, 1, 100,
                                            [1, 2, 3, 4], stream=0x1000)
    assert (slot2, reuse, oc) == (slot, 3, HIT)
