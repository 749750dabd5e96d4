// Session manager: parks the state a chat turn leaves in its slot and hands
// it to the follow-up turn only when the follow-up provably continues it
// (same model, user and chat, the parked assistant message as its parent,
// and the parked raw-token history as a prefix of its own); everything else
// restarts from a zero state. Page "wkvm: state-slot inference for RWKV, GDN
// and Mamba hybrids", section "Two engines under one name, and the contract
// between them" (the parent-token-v1 binding); admission and host parking
// follow the page "Virtual Memory for KV Cache and Model Weights" (a
// request needs a free recurrent-state slot; host capacity is preallocated;
// buffers stay retained until their transfers finish).

#include "../../include/wkv7_session.h"
#include "host.h"

#include <hip/hip_runtime.h>

#include <cstring>
#include <deque>
#include <initializer_list>
#include <memory>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

using wkv7::host_fail;

namespace {

struct Key {
  uint64_t model, user, chat, message;
  bool operator==(const Key& o) const {
    return model == o.model && user == o.user && chat == o.chat &&
           message == o.message;
  }
};

struct KeyHash {
  size_t operator()(const Key& k) const {
    uint64_t h = 0xcbf29ce484222325ull;   // FNV-1a offset basis
    for (uint64_t v : {k.model, k.user, k.chat, k.message}) {
      for (int b = 0; b < 8; ++b) {
        h ^= (v >> (8 * b)) & 0xffu;
        h *= 0x100000001b3ull;             // FNV-1a 64-bit prime
      }
    }
    return static_cast<size_t>(h);
  }
};

Key chat_of(const Key& k) { return Key{k.model, k.user, k.chat, 0}; }

// One state: a turn in flight (active) or a parked state after `message`.
struct Record {
  Key key{};                     // key.message == 0 while active
  std::vector<int32_t> tokens;   // history the state has consumed (parked)
  int32_t slot = -1;             // device slot, or -1 while on the host
  int32_t image = -1;            // host image while on the host
  bool active = false;
  bool pinned = false;           // excluded from eviction for a moment
  uint64_t last_use = 0;
};

constexpr size_t kEvictedMemory = 1 << 16;   // remembered dropped keys

}  // namespace

struct wkv7_sessions {
  wkv7_pool* pool = nullptr;
  bool dry = false;
  // The stream of the first turn: every turn must use it, because the
  // manager's own device work (hibernate, fork, reset of a recycled slot)
  // touches slots whose last forward it can only know to be done in that
  // stream's order.
  bool stream_set = false;
  void* stream = nullptr;
  int flags = 0;
  std::vector<int32_t> dry_free;
  // host parking
  char* host = nullptr;
  size_t slot_bytes = 0;
  int32_t n_images = 0;
  std::vector<int32_t> free_images;
  std::vector<hipEvent_t> image_ev;
  std::vector<uint8_t> image_ev_set;
  // records
  std::vector<std::unique_ptr<Record>> records;
  std::unordered_map<Key, Record*, KeyHash> parked;
  std::unordered_map<Key, int32_t, KeyHash> parked_per_chat;
  std::unordered_map<int32_t, Record*> active_by_slot;
  std::unordered_set<Key, KeyHash> evicted;
  std::deque<Key> evicted_order;
  uint64_t clock = 0;
  wkv7_session_stats st{};
};

namespace {

using S = wkv7_sessions;

void remember_evicted(S* s, const Key& k) {
  if (s->evicted.insert(k).second) {
    s->evicted_order.push_back(k);
    if (s->evicted_order.size() > kEvictedMemory) {
      s->evicted.erase(s->evicted_order.front());
      s->evicted_order.pop_front();
    }
  }
}

wkv7_status release_slot(S* s, int32_t slot) {
  if (s->dry) {
    s->dry_free.push_back(slot);
    return WKV7_OK;
  }
  return wkv7_slot_free(s->pool, &slot, 1);
}

// Order `stream` after the last copy that used host image i.
wkv7_status wait_image(S* s, int32_t i, hipStream_t stream) {
  if (s->dry || !s->image_ev_set[i]) return WKV7_OK;
  hipError_t e = hipStreamWaitEvent(stream, s->image_ev[i], 0);
  if (e != hipSuccess)
    return host_fail(WKV7_ERR_HIP, "hipStreamWaitEvent(host image): %s",
                     hipGetErrorString(e));
  return WKV7_OK;
}

wkv7_status mark_image(S* s, int32_t i, hipStream_t stream) {
  if (s->dry) return WKV7_OK;
  hipError_t e = hipEventRecord(s->image_ev[i], stream);
  if (e != hipSuccess)
    return host_fail(WKV7_ERR_HIP, "hipEventRecord(host image): %s",
                     hipGetErrorString(e));
  s->image_ev_set[i] = 1;
  return WKV7_OK;
}

void erase_record(S* s, Record* r) {
  for (size_t i = 0; i < s->records.size(); ++i) {
    if (s->records[i].get() == r) {
      s->records[i] = std::move(s->records.back());
      s->records.pop_back();
      return;
    }
  }
}

void unpark(S* s, Record* r) {
  s->parked.erase(r->key);
  auto it = s->parked_per_chat.find(chat_of(r->key));
  if (it != s->parked_per_chat.end() && --it->second == 0)
    s->parked_per_chat.erase(it);
}

// Drop a parked record: its slot and host image are released.
wkv7_status drop_parked(S* s, Record* r, bool evicted) {
  unpark(s, r);
  wkv7_status st = WKV7_OK;
  if (r->slot >= 0) st = release_slot(s, r->slot);
  if (r->image >= 0) s->free_images.push_back(r->image);
  if (evicted) remember_evicted(s, r->key);
  s->st.drops += 1;
  erase_record(s, r);
  return st;
}

Record* lru(S* s, bool on_device) {
  Record* best = nullptr;
  for (auto& up : s->records) {
    Record* r = up.get();
    if (r->active || r->pinned) continue;
    if (on_device ? r->slot < 0 : r->image < 0) continue;
    if (!best || r->last_use < best->last_use) best = r;
  }
  return best;
}

// Free one device slot by moving (or dropping) the least recently used
// parked state that holds one.
wkv7_status evict_one(S* s, hipStream_t stream) {
  Record* d = lru(s, true);
  if (!d)
    return host_fail(WKV7_ERR_POOL_FULL,
                     "session_begin: every slot holds a turn in flight");
  if (s->free_images.empty()) {
    if (Record* h = lru(s, false)) {
      if (wkv7_status st = drop_parked(s, h, true)) return st;
    }
  }
  if (s->free_images.empty())   // no host parking at all: drop the state
    return drop_parked(s, d, true);
  const int32_t img = s->free_images.back();
  s->free_images.pop_back();
  if (!s->dry) {
    if (wkv7_status st = wait_image(s, img, stream)) return st;
    if (wkv7_status st = wkv7_hibernate(s->pool, &d->slot, 1,
                                        s->host + img * s->slot_bytes,
                                        s->slot_bytes, stream))
      return st;
    if (wkv7_status st = mark_image(s, img, stream)) return st;
  }
  s->st.hibernates += 1;
  wkv7_status st = release_slot(s, d->slot);
  d->slot = -1;
  d->image = img;
  return st;
}

wkv7_status alloc_slot(S* s, hipStream_t stream, int32_t* out) {
  for (;;) {
    if (s->dry) {
      if (!s->dry_free.empty()) {
        *out = s->dry_free.back();
        s->dry_free.pop_back();
        return WKV7_OK;
      }
    } else {
      int32_t id = -1;
      wkv7_status st = wkv7_slot_alloc(s->pool, 1, &id);
      if (st == WKV7_OK) {
        *out = id;
        return WKV7_OK;
      }
      if (st != WKV7_ERR_POOL_FULL) return st;
    }
    if (wkv7_status st = evict_one(s, stream)) return st;
  }
}

// Bring a parked host image into device slot `slot`.
wkv7_status resume_into(S* s, Record* r, int32_t slot, hipStream_t stream) {
  if (!s->dry) {
    if (wkv7_status st = wait_image(s, r->image, stream)) return st;
    if (wkv7_status st = wkv7_resume(s->pool, &slot, 1,
                                     s->host + r->image * s->slot_bytes,
                                     s->slot_bytes, stream))
      return st;
    if (wkv7_status st = mark_image(s, r->image, stream)) return st;
  }
  s->st.resumes += 1;
  return WKV7_OK;
}

bool is_prefix(const std::vector<int32_t>& a, const int32_t* b, int64_t n) {
  return static_cast<int64_t>(a.size()) <= n &&
         (a.empty() || std::memcmp(a.data(), b, a.size() * 4) == 0);
}

Record* new_active(S* s, const Key& chat, int32_t slot) {
  auto up = std::make_unique<Record>();
  Record* r = up.get();
  r->key = chat;
  r->slot = slot;
  r->active = true;
  s->records.push_back(std::move(up));
  s->active_by_slot[slot] = r;
  return r;
}

}  // namespace

extern "C" {

wkv7_status wkv7_sessions_create(wkv7_pool* pool, int32_t dry_slots,
                                 int32_t host_images, int32_t flags,
                                 wkv7_sessions** out) {
  wkv7::host_clear_error();
  if (!out) return host_fail(WKV7_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (host_images < 0)
    return host_fail(WKV7_ERR_INVALID_ARG, "host_images=%d < 0", host_images);
  if (flags & ~WKV7_SESSIONS_KEEP_PARENT)
    return host_fail(WKV7_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  if (pool ? dry_slots != 0 : dry_slots < 1)
    return host_fail(WKV7_ERR_INVALID_ARG,
                     pool ? "dry_slots must be 0 with a pool"
                          : "a host-only manager needs dry_slots >= 1");
  std::unique_ptr<wkv7_sessions> s(new (std::nothrow) wkv7_sessions());
  if (!s) return host_fail(WKV7_ERR_OOM, "host allocation failed");
  s->pool = pool;
  s->dry = pool == nullptr;
  s->flags = flags;
  s->n_images = host_images;
  if (s->dry) {
    for (int32_t i = dry_slots - 1; i >= 0; --i) s->dry_free.push_back(i);
  } else if (host_images > 0) {
    s->slot_bytes = wkv7_slot_bytes(pool);
    const int dev = wkv7::pool_device(pool);
    int prev = -1;
    (void)hipGetDevice(&prev);
    (void)hipSetDevice(dev);
    hipError_t e = hipHostMalloc(reinterpret_cast<void**>(&s->host),
                                 s->slot_bytes * host_images);
    s->image_ev.assign(static_cast<size_t>(host_images), nullptr);
    for (int32_t i = 0; e == hipSuccess && i < host_images; ++i)
      e = hipEventCreateWithFlags(&s->image_ev[i], hipEventDisableTiming);
    if (prev >= 0) (void)hipSetDevice(prev);
    if (e != hipSuccess) {
      for (hipEvent_t ev : s->image_ev)
        if (ev) (void)hipEventDestroy(ev);
      if (s->host) (void)hipHostFree(s->host);
      return host_fail(WKV7_ERR_OOM, "host parking of %d images: %s",
                       host_images, hipGetErrorString(e));
    }
  }
  s->image_ev_set.assign(static_cast<size_t>(host_images), 0);
  for (int32_t i = host_images - 1; i >= 0; --i) s->free_images.push_back(i);
  *out = s.release();
  return WKV7_OK;
}

wkv7_status wkv7_sessions_destroy(wkv7_sessions* s) {
  wkv7::host_clear_error();
  if (!s) return WKV7_OK;
  wkv7_status st = WKV7_OK;
  if (!s->dry) {
    int prev = -1;
    (void)hipGetDevice(&prev);
    (void)hipSetDevice(wkv7::pool_device(s->pool));
    if (hipDeviceSynchronize() != hipSuccess)
      st = host_fail(WKV7_ERR_HIP, "hipDeviceSynchronize(sessions destroy)");
    for (auto& up : s->records)
      if (up->slot >= 0) (void)wkv7_slot_free(s->pool, &up->slot, 1);
    for (hipEvent_t ev : s->image_ev)
      if (ev) (void)hipEventDestroy(ev);
    if (s->host) (void)hipHostFree(s->host);
    if (prev >= 0) (void)hipSetDevice(prev);
  }
  delete s;
  return st;
}

wkv7_status wkv7_session_begin(wkv7_sessions* s, const wkv7_turn_key* key,
                               const int32_t* tokens, int64_t n_tokens,
                               void* stream, int32_t* slot, int64_t* n_reuse,
                               int32_t* outcome) {
  wkv7::host_clear_error();
  if (!s || !key || !slot || !n_reuse || !outcome)
    return host_fail(WKV7_ERR_INVALID_ARG, "session_begin: NULL argument");
  if (n_tokens < 0 || (n_tokens > 0 && !tokens))
    return host_fail(WKV7_ERR_INVALID_ARG, "session_begin: bad tokens");
  if (s->stream_set && stream != s->stream)
    return host_fail(WKV7_ERR_INVALID_ARG,
                     "session_begin: every turn of a manager must use the "
                     "stream of its first turn");
  s->stream_set = true;
  s->stream = stream;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const Key chat{key->model, key->user, key->chat, 0};
  const Key want{key->model, key->user, key->chat, key->parent};
  Record* r = nullptr;
  if (key->parent != 0) {
    auto it = s->parked.find(want);
    if (it != s->parked.end()) r = it->second;
  }
  int32_t oc;
  if (r && is_prefix(r->tokens, tokens, n_tokens)) oc = WKV7_SESSION_HIT;
  else if (r) oc = WKV7_SESSION_RESTART_EDIT;
  else if (key->parent == 0) oc = WKV7_SESSION_NEW;
  else if (s->evicted.count(want)) oc = WKV7_SESSION_RESTART_EVICTED;
  else oc = WKV7_SESSION_RESTART_PARENT;

  int32_t sl = -1;
  int64_t reuse = 0;
  if (oc == WKV7_SESSION_HIT) {
    reuse = static_cast<int64_t>(r->tokens.size());
    r->last_use = ++s->clock;
    if (s->flags & WKV7_SESSIONS_KEEP_PARENT) {
      r->pinned = true;
      wkv7_status st = alloc_slot(s, hs, &sl);
      if (st == WKV7_OK) {
        if (r->slot >= 0) {
          if (!s->dry) st = wkv7_fork(s->pool, &r->slot, &sl, 1, stream);
          if (st == WKV7_OK) s->st.forks += 1;
        } else {
          st = resume_into(s, r, sl, hs);
        }
        if (st != WKV7_OK) (void)release_slot(s, sl);
      }
      r->pinned = false;
      if (st) return st;
      new_active(s, chat, sl);
    } else {
      r->pinned = true;
      wkv7_status st = WKV7_OK;
      if (r->slot >= 0) {
        sl = r->slot;
      } else {
        st = alloc_slot(s, hs, &sl);
        if (st == WKV7_OK) st = resume_into(s, r, sl, hs);
        if (st != WKV7_OK && sl >= 0) (void)release_slot(s, sl);
      }
      r->pinned = false;
      if (st) return st;
      unpark(s, r);
      if (r->image >= 0) s->free_images.push_back(r->image);
      r->image = -1;
      r->slot = sl;
      r->key = chat;
      r->tokens.clear();
      r->active = true;
      s->active_by_slot[sl] = r;
    }
    s->st.hits += 1;
  } else {
    if (wkv7_status st = alloc_slot(s, hs, &sl)) return st;
    if (!s->dry) {
      if (wkv7_status st = wkv7_reset(s->pool, &sl, 1, stream)) {
        (void)release_slot(s, sl);
        return st;
      }
    }
    s->st.resets += 1;
    new_active(s, chat, sl);
    if (oc == WKV7_SESSION_NEW) s->st.news += 1;
    else if (oc == WKV7_SESSION_RESTART_EDIT) s->st.restarts_edit += 1;
    else if (oc == WKV7_SESSION_RESTART_EVICTED) s->st.restarts_evicted += 1;
    else s->st.restarts_parent += 1;
  }
  *slot = sl;
  *n_reuse = reuse;
  *outcome = oc;
  return WKV7_OK;
}

wkv7_status wkv7_session_end(wkv7_sessions* s, int32_t slot, uint64_t message,
                             const int32_t* tokens, int64_t n_tokens) {
  wkv7::host_clear_error();
  if (!s) return host_fail(WKV7_ERR_INVALID_ARG, "sessions is NULL");
  auto it = s->active_by_slot.find(slot);
  if (it == s->active_by_slot.end())
    return host_fail(WKV7_ERR_INVALID_ARG,
                     "session_end: slot %d holds no turn in flight", slot);
  if (message == 0)
    return host_fail(WKV7_ERR_INVALID_ARG, "session_end: message id 0");
  if (n_tokens < 0 || (n_tokens > 0 && !tokens))
    return host_fail(WKV7_ERR_INVALID_ARG, "session_end: bad tokens");
  Record* r = it->second;
  const Key k{r->key.model, r->key.user, r->key.chat, message};
  auto old = s->parked.find(k);
  if (old != s->parked.end())
    if (wkv7_status st = drop_parked(s, old->second, false)) return st;
  s->active_by_slot.erase(it);
  r->key = k;
  r->tokens.assign(tokens, tokens + n_tokens);
  r->active = false;
  r->last_use = ++s->clock;
  s->parked[k] = r;
  s->parked_per_chat[chat_of(k)] += 1;
  if (s->evicted.erase(k)) {
    for (auto e = s->evicted_order.begin(); e != s->evicted_order.end(); ++e)
      if (*e == k) { s->evicted_order.erase(e); break; }
  }
  return WKV7_OK;
}

wkv7_status wkv7_session_abort(wkv7_sessions* s, int32_t slot) {
  wkv7::host_clear_error();
  if (!s) return host_fail(WKV7_ERR_INVALID_ARG, "sessions is NULL");
  auto it = s->active_by_slot.find(slot);
  if (it == s->active_by_slot.end())
    return host_fail(WKV7_ERR_INVALID_ARG,
                     "session_abort: slot %d holds no turn in flight", slot);
  Record* r = it->second;
  s->active_by_slot.erase(it);
  wkv7_status st = release_slot(s, r->slot);
  erase_record(s, r);
  return st;
}

wkv7_status wkv7_session_drop_chat(wkv7_sessions* s, uint64_t model,
                                   uint64_t user, uint64_t chat) {
  wkv7::host_clear_error();
  if (!s) return host_fail(WKV7_ERR_INVALID_ARG, "sessions is NULL");
  std::vector<Record*> victims;
  for (auto& up : s->records) {
    Record* r = up.get();
    if (!r->active && r->key.model == model && r->key.user == user &&
        r->key.chat == chat)
      victims.push_back(r);
  }
  for (Record* r : victims)
    if (wkv7_status st = drop_parked(s, r, false)) return st;
  return WKV7_OK;
}

wkv7_status wkv7_sessions_stats(const wkv7_sessions* s,
                                wkv7_session_stats* out) {
  wkv7::host_clear_error();
  if (!s || !out) return host_fail(WKV7_ERR_INVALID_ARG, "NULL argument");
  *out = s->st;
  out->active = static_cast<int32_t>(s->active_by_slot.size());
  int32_t dev = 0, host = 0;
  for (auto& up : s->records) {
    if (up->active) continue;
    if (up->slot >= 0) ++dev;
    else if (up->image >= 0) ++host;
  }
  out->parked_device = dev;
  out->parked_host = host;
  out->free_host_images = static_cast<int32_t>(s->free_images.size());
  return WKV7_OK;
}

}  // extern "C"
