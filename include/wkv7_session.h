/*
 * libwkv7 sessions — multi-turn state reuse over a slot pool.
 *
 * C ABI, host side. A session manager parks the state a chat turn leaves in
 * its slot and hands it to the follow-up turn when, and only when, the
 * follow-up provably continues it; otherwise the turn restarts from a zero
 * state. This is the stateful contract the page "wkvm: state-slot inference
 * for RWKV, GDN and Mamba hybrids" describes (section "Two engines under one
 * name, and the contract between them", parent-token-v1): a parked state is
 * bound to the model, the user, the chat and the assistant message it ends
 * with, and to the exact raw-token history it has consumed; an edit, a
 * branch, a stale parent or missing metadata restarts instead of reusing a
 * wrong state. Here the history is kept and compared token for token (a
 * digest alone could collide).
 *
 * Admission (page "Virtual Memory for KV Cache and Model Weights"): a turn
 * needs a device slot. When the pool has none free, the least recently used
 * parked state is moved to host memory preallocated at creation (a fixed
 * number of host images), and when that is full too, the least recently
 * used host image is dropped (its chat restarts next time). States of turns
 * in flight are never moved.
 *
 * Device work (reset, fork, hibernate, resume) is enqueued on the stream
 * given to wkv7_session_begin; the caller runs wkv7_forward on the returned
 * slot on the same stream. Every turn of a manager must use one stream, the
 * stream of its first turn (wkv7_session_begin fails with
 * WKV7_ERR_INVALID_ARG on any other): the manager moves, forks and resets
 * slots whose last forward it knows to be finished only through that
 * stream's order. A manager and its pool belong to one host thread.
 */
#ifndef WKV7_SESSION_H
#define WKV7_SESSION_H

#include "wkv7.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct wkv7_sessions wkv7_sessions;

/* What a turn continues: caller-chosen ids (for example hashes of names).
 * parent is the id of the assistant message the turn follows, 0 for a
 * chat's first turn. */
typedef struct {
  uint64_t model, user, chat;
  uint64_t parent;
} wkv7_turn_key;

/* Outcome of wkv7_session_begin. */
enum {
  WKV7_SESSION_HIT = 0,             /* the parked state continues the turn */
  WKV7_SESSION_NEW = 1,             /* nothing parked for this chat */
  WKV7_SESSION_RESTART_EDIT = 2,    /* parent parked, history differs */
  WKV7_SESSION_RESTART_PARENT = 3,  /* chat parked, but not at this parent */
  WKV7_SESSION_RESTART_EVICTED = 4  /* the parent's state was dropped */
};

/* Flags for wkv7_sessions_create. */
enum {
  /* On a hit, fork the parked state into a new slot and leave the parent
   * parked, so a regenerated answer or a second branch from the same
   * parent hits too. Without it the parked state becomes the turn's. */
  WKV7_SESSIONS_KEEP_PARENT = 1
};

/* Create a manager over `pool`, with host_images host slot images
 * (pinned, preallocated here; 0 = parked states are dropped instead of
 * moved to host memory). pool == NULL makes a host-only manager over
 * dry_slots imaginary slots that counts the device work it would do
 * instead of doing it (for tests of the policy); with a pool, dry_slots
 * must be 0. */
wkv7_status wkv7_sessions_create(wkv7_pool* pool, int32_t dry_slots,
                                 int32_t host_images, int32_t flags,
                                 wkv7_sessions** out);

/* Wait for the device, free the host images and return every slot the
 * manager holds to the pool's free list. NULL is a no-op. */
wkv7_status wkv7_sessions_destroy(wkv7_sessions* s);

/* Begin a turn whose full raw-token history (prompt included, as the
 * model saw it) is tokens[n_tokens] (host array). On success *slot holds
 * the turn's slot, its state the effect of tokens[0, *n_reuse); the caller
 * runs tokens[*n_reuse, n_tokens) through wkv7_forward on that slot, then
 * calls wkv7_session_end or wkv7_session_abort. *outcome is one of
 * WKV7_SESSION_*. A parked state is reused only if its key matches (same
 * model, user, chat, and its message == key->parent) and its history is a
 * prefix of tokens. WKV7_ERR_POOL_FULL if every slot belongs to a turn in
 * flight. */
wkv7_status wkv7_session_begin(wkv7_sessions* s, const wkv7_turn_key* key,
                               const int32_t* tokens, int64_t n_tokens,
                               void* stream, int32_t* slot, int64_t* n_reuse,
                               int32_t* outcome);

/* End the turn running in `slot`: its state now holds the effect of
 * tokens[n_tokens] (host array: the turn's whole history including the
 * generated answer), and it is parked as the state after assistant message
 * `message` (non-zero). A parked state with the same chat and message is
 * replaced. */
wkv7_status wkv7_session_end(wkv7_sessions* s, int32_t slot, uint64_t message,
                             const int32_t* tokens, int64_t n_tokens);

/* Abandon the turn running in `slot` (its state is discarded). */
wkv7_status wkv7_session_abort(wkv7_sessions* s, int32_t slot);

/* Drop every parked state of a chat (for example when it is deleted). */
wkv7_status wkv7_session_drop_chat(wkv7_sessions* s, uint64_t model,
                                   uint64_t user, uint64_t chat);

typedef struct {
  int64_t hits, news, restarts_edit, restarts_parent, restarts_evicted;
  int64_t resets, forks, hibernates, resumes, drops;
  int32_t active, parked_device, parked_host, free_host_images;
} wkv7_session_stats;

/* Counters since creation and the current occupancy. */
wkv7_status wkv7_sessions_stats(const wkv7_sessions* s,
                                wkv7_session_stats* out);

#ifdef __cplusplus
}
#endif

#endif /* WKV7_SESSION_H */
