// libwkv7 host library: the C ABI, argument validation, the slot pool and
// its free list, per-call metadata staging, kernel dispatch and slot verbs.
//
// Every entry point validates all of its arguments before it enqueues any
// device work, so a failed call leaves the pool and the stream untouched.

#include "../../include/wkv7.h"
#include "host.h"
#include "internal.h"

#include <algorithm>
#include <climits>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <type_traits>
#include <utility>
#include <vector>

using wkv7::WorkItem;

namespace {

thread_local std::string g_last_error;

wkv7_status fail(wkv7_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

wkv7_status fail_hip(hipError_t e, const char* what) {
  return fail(WKV7_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e),
              static_cast<int>(e));
}

// Metadata staging: a ring of pinned host buffers and device buffers. An
// entry is reused only after the event recorded behind its last use has
// completed, so the host never overwrites data a queued copy still reads,
// whatever stream the calls used.
constexpr int kRing = 8;
// Every entry holds at least this many int32 (allocated at pool creation, so
// the allocation-free forward can stage through any entry).
constexpr size_t kStageMinInts = wkv7::kStaticMetaBytes / 4;

struct Stage {
  int32_t* host = nullptr;
  int32_t* dev = nullptr;
  size_t cap_ints = 0;
  size_t n_ints = 0;          // what `dev` holds (a copy of host[0, n_ints))
  hipStream_t stream = nullptr;
  hipEvent_t ev = nullptr;
  bool pending = false;
};

// Runs a call on the pool's device and restores the caller's device.
struct DeviceGuard {
  int prev = -1;
  bool ok = true;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) { ok = false; return; }
    if (prev != dev && hipSetDevice(dev) != hipSuccess) ok = false;
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev)
      (void)hipSetDevice(prev);
  }
};

}  // namespace

struct wkv7_pool {
  int device = 0;
  int32_t n_slots = 0, H = 0, N = 0;
  float* state = nullptr;
  size_t slot_floats = 0;
  int64_t prefill_min_len = 32;
  bool chunk_precise = false;
  int64_t segment_len = 0;           // 0: segment-parallel prefill off
  float* seg_scratch = nullptr;      // wkv7_forward's segment buffers
  size_t seg_scratch_floats = 0;
  float* xfer_stage = nullptr;       // staging of scattered hibernate/resume
  size_t xfer_stage_bytes = 0;
  void* static_scratch = nullptr;    // the device's static scratch array
  // Buffers a call has outgrown, freed at destroy: releasing memory waits
  // for the whole device on this runtime, so no other call frees anything.
  // (pointer, true for pinned host memory)
  std::vector<std::pair<void*, bool>> retired;
  int n_cus = 0;                     // compute units of the pool's device
  std::vector<int32_t> free_ids;     // stack; top = back
  std::vector<uint8_t> allocated;
  Stage ring[kRing];
  int ring_pos = 0;
};

// Work items of one batch, validated once and kept on the pool's device.
struct wkv7_plan {
  const wkv7_pool* pool = nullptr;
  int device = 0;
  void* dev = nullptr;               // serialized work description
  float* scratch = nullptr;          // segment buffers (segment prefill)
  wkv7::Launch launch;               // pointers into dev
  int64_t T_tot = 0;
};

namespace {

size_t slot_bytes_of(const wkv7_pool* p) { return p->slot_floats * sizeof(float); }

// Copy `n` int32 values to the device through the staging ring. On success
// *dev_out points at them and *stage_out must be committed after the
// launches that read them.
//
// Steady-state decode passes the same metadata every step. If an entry last
// used on the same stream already holds identical data on the device, that
// copy is reused and nothing is uploaded: stream order puts the new launches
// after the old upload, and the entry cannot be overwritten before its event
// (re-recorded at commit) has passed.
wkv7_status stage_upload(wkv7_pool* p, const int32_t* data, size_t n,
                         hipStream_t stream, const int32_t** dev_out,
                         Stage** stage_out) {
  for (int i = 0; i < kRing; ++i) {
    Stage& c = p->ring[i];
    if (c.dev && c.n_ints == n && c.stream == stream &&
        std::memcmp(c.host, data, n * 4) == 0) {
      *dev_out = c.dev;
      *stage_out = &c;
      return WKV7_OK;
    }
  }
  Stage& s = p->ring[p->ring_pos];
  p->ring_pos = (p->ring_pos + 1) % kRing;
  hipError_t e;
  if (s.pending) {
    e = hipEventSynchronize(s.ev);
    if (e != hipSuccess) return fail_hip(e, "hipEventSynchronize(staging)");
    s.pending = false;
  }
  if (s.cap_ints < n) {
    size_t cap = std::max<size_t>(n, kStageMinInts);
    if (s.host) p->retired.emplace_back(s.host, true);
    if (s.dev) p->retired.emplace_back(s.dev, false);
    s.host = nullptr;
    s.dev = nullptr;
    s.cap_ints = 0;
    if (hipHostMalloc(reinterpret_cast<void**>(&s.host), cap * 4) != hipSuccess)
      return fail(WKV7_ERR_OOM, "pinned staging allocation of %zu bytes failed",
                  cap * 4);
    if (hipMalloc(reinterpret_cast<void**>(&s.dev), cap * 4) != hipSuccess) {
      p->retired.emplace_back(s.host, true);
      s.host = nullptr;
      return fail(WKV7_ERR_OOM, "device staging allocation of %zu bytes failed",
                  cap * 4);
    }
    s.cap_ints = cap;
  }
  s.n_ints = 0;
  std::memcpy(s.host, data, n * 4);
  e = hipMemcpyAsync(s.dev, s.host, n * 4, hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return fail_hip(e, "hipMemcpyAsync(metadata)");
  s.n_ints = n;
  s.stream = stream;
  // Guard the copy at once, so that a failed launch after it cannot let the
  // next call overwrite a host buffer still being read.
  e = hipEventRecord(s.ev, stream);
  if (e != hipSuccess) return fail_hip(e, "hipEventRecord(staging)");
  s.pending = true;
  *dev_out = s.dev;
  *stage_out = &s;
  return WKV7_OK;
}

wkv7_status stage_commit(Stage* s, hipStream_t stream) {
  hipError_t e = hipEventRecord(s->ev, stream);
  if (e != hipSuccess) return fail_hip(e, "hipEventRecord(staging)");
  s->pending = true;
  return WKV7_OK;
}

wkv7_status check_pool(const wkv7_pool* p) {
  if (!p) return fail(WKV7_ERR_INVALID_ARG, "pool is NULL");
  return WKV7_OK;
}

// ids[0..n) in range; if `distinct`, no id twice.
wkv7_status check_ids(const wkv7_pool* p, const int32_t* ids, int32_t n,
                      bool distinct, const char* what) {
  if (n < 0) return fail(WKV7_ERR_INVALID_ARG, "%s: n=%d < 0", what, n);
  if (n > 0 && !ids) return fail(WKV7_ERR_INVALID_ARG, "%s: ids is NULL", what);
  std::vector<uint8_t> seen;
  if (distinct) seen.assign(static_cast<size_t>(p->n_slots), 0);
  for (int32_t i = 0; i < n; ++i) {
    int32_t id = ids[i];
    if (id < 0 || id >= p->n_slots)
      return fail(WKV7_ERR_OUT_OF_RANGE, "%s: slot id %d at %d outside [0, %d)",
                  what, id, i, p->n_slots);
    if (distinct) {
      if (seen[id]) return fail(WKV7_ERR_DUPLICATE_SLOT,
                                "%s: slot id %d appears twice", what, id);
      seen[id] = 1;
    }
  }
  return WKV7_OK;
}

bool aligned16(const void* q) {
  return (reinterpret_cast<uintptr_t>(q) & 15u) == 0;
}

// A validated batch: work items with the sequential-kernel items first
// (single-token ones, then longer ones), then the chunked ones, longest
// first.
struct Batch {
  std::vector<WorkItem> items;       // sequential items, then all chunked
  int32_t n_seq_items = 0;
  int32_t n_seq_single = 0;          // leading single-token items
  int64_t T_tot = 0;
  // with segment-parallel prefill on: chunked items run whole (unsplit) and
  // those split into segments of `seg_len` tokens
  std::vector<WorkItem> unsplit, split;
  int64_t seg_len = 0, n_segments = 0;
  int32_t n_chunk_items() const {
    return static_cast<int32_t>(items.size()) - n_seq_items;
  }
};

// Checks slot_ids / cu_seqlens exactly as wkv7_forward documents and splits
// the sequences by length (PREFILL_MIN_LEN).
wkv7_status build_batch(const wkv7_pool* p, const int32_t* slot_ids,
                        const int32_t* cu_seqlens, int32_t n_seqs,
                        const char* what, Batch* out) {
  if (n_seqs < 0) return fail(WKV7_ERR_INVALID_ARG, "n_seqs=%d < 0", n_seqs);
  if (n_seqs == 0) return WKV7_OK;
  if (!cu_seqlens) return fail(WKV7_ERR_INVALID_ARG, "cu_seqlens is NULL");
  if (cu_seqlens[0] != 0)
    return fail(WKV7_ERR_INVALID_ARG, "cu_seqlens[0]=%d, must be 0",
                cu_seqlens[0]);
  for (int32_t s = 0; s < n_seqs; ++s)
    if (cu_seqlens[s + 1] < cu_seqlens[s])
      return fail(WKV7_ERR_INVALID_ARG,
                  "cu_seqlens decreases at %d (%d -> %d)", s, cu_seqlens[s],
                  cu_seqlens[s + 1]);
  if (wkv7_status st = check_ids(p, slot_ids, n_seqs, true, what)) return st;
  out->T_tot = cu_seqlens[n_seqs];
  std::vector<WorkItem> chunk_items, multi_items;
  out->items.reserve(static_cast<size_t>(n_seqs));
  for (int32_t s = 0; s < n_seqs; ++s) {
    const int32_t len = cu_seqlens[s + 1] - cu_seqlens[s];
    if (len == 0) continue;
    WorkItem it{slot_ids[s], cu_seqlens[s], len, 0};
    if (len >= p->prefill_min_len) chunk_items.push_back(it);
    else if (len > 1) multi_items.push_back(it);
    else out->items.push_back(it);
  }
  out->n_seq_single = static_cast<int32_t>(out->items.size());
  out->items.insert(out->items.end(), multi_items.begin(), multi_items.end());
  std::stable_sort(chunk_items.begin(), chunk_items.end(),
                   [](const WorkItem& x, const WorkItem& y) {
                     return x.len > y.len;
                   });
  out->n_seq_items = static_cast<int32_t>(out->items.size());
  out->items.insert(out->items.end(), chunk_items.begin(), chunk_items.end());
  // segment-parallel prefill: a sequence of at least two segments is split
  // (the rule looks at the sequence's own length only)
  out->seg_len = p->segment_len;
  if (p->segment_len > 0) {
    for (const WorkItem& it : chunk_items) {
      if (it.len >= 2 * p->segment_len) {
        out->split.push_back(it);
        out->n_segments += (it.len + p->segment_len - 1) / p->segment_len;
      } else {
        out->unsplit.push_back(it);
      }
    }
    if (out->split.empty()) out->unsplit.clear();
  }
  return WKV7_OK;
}

// Floats of segment buffers a batch needs: P, Hs and Sin per segment-head.
size_t seg_scratch_floats(const wkv7_pool* p, const Batch& bt) {
  return static_cast<size_t>(bt.n_segments) * 3 * p->H * wkv7::kN * wkv7::kN;
}

// Serializes a batch's work for the device: work items, segment items and
// scan items with their device addresses (pool slots and `scratch`), each
// section 16-byte aligned. `lay` receives section offsets (bytes, in
// Launch's pointer fields) and counts.
std::vector<int32_t> serialize(const wkv7_pool* p, const Batch& bt,
                               float* scratch, wkv7::Launch* lay) {
  using wkv7::SegItem;
  using wkv7::ScanItem;
  std::vector<int32_t> out;
  auto put = [&](const void* src, size_t bytes) -> size_t {
    const size_t off = out.size() * 4;
    const size_t words = bytes / 4;
    out.resize(out.size() + words);
    std::memcpy(out.data() + off / 4, src, bytes);
    return off;
  };
  auto at = [](size_t off) { return reinterpret_cast<const void*>(off); };
  *lay = wkv7::Launch{};
  lay->n_seq = bt.n_seq_items;
  lay->n_seq_single = bt.n_seq_single;
  lay->n_chunk_all = bt.n_chunk_items();
  lay->seq = static_cast<const WorkItem*>(at(put(bt.items.data(),
                                                 bt.items.size() * sizeof(WorkItem))));
  lay->chunk_all = lay->seq + bt.n_seq_items;
  if (bt.split.empty()) return out;
  const size_t nn = static_cast<size_t>(wkv7::kN) * wkv7::kN;
  const size_t blk = static_cast<size_t>(p->H) * nn;      // one of P/Hs/Sin
  std::vector<SegItem> ph1, ph3;
  std::vector<ScanItem> scan;
  // chunked sequences that are not split run whole in the first phase's
  // launch, from and back into their slots (longest first, ahead of the
  // segments, which are at most seg_len tokens)
  for (const WorkItem& it : bt.unsplit) {
    float* slot_state = p->state + static_cast<size_t>(it.slot) * p->slot_floats;
    ph1.push_back(SegItem{slot_state, slot_state, it.tok0, it.len, 0, 0});
  }
  int64_t seg0 = 0;
  for (const WorkItem& it : bt.split) {
    const int64_t n_seg = (it.len + bt.seg_len - 1) / bt.seg_len;
    float* slot_state = p->state + static_cast<size_t>(it.slot) * p->slot_floats;
    float* base = scratch + static_cast<size_t>(seg0) * 3 * blk;
    for (int64_t j = 0; j < n_seg; ++j) {
      float* b = base + static_cast<size_t>(j) * 3 * blk;
      const int32_t tok0 = it.tok0 + static_cast<int32_t>(j * bt.seg_len);
      const int32_t len = static_cast<int32_t>(
          std::min<int64_t>(bt.seg_len, it.len - j * bt.seg_len));
      if (j + 1 < n_seg) {
        ph1.push_back(SegItem{nullptr, b + blk, tok0, len, wkv7::kSegNoOut, 0});
        ph1.push_back(SegItem{nullptr, b, tok0, len,
                              wkv7::kSegIdentity | wkv7::kSegZeroV |
                                  wkv7::kSegNoOut, 0});
      }
      ph3.push_back(SegItem{b + 2 * blk, j + 1 == n_seg ? slot_state : nullptr,
                            tok0, len, 0, 0});
    }
    scan.push_back(ScanItem{slot_state, base, static_cast<int32_t>(n_seg), {0, 0, 0}});
    seg0 += n_seg;
  }
  lay->n_phase1 = static_cast<int32_t>(ph1.size());
  lay->n_phase3 = static_cast<int32_t>(ph3.size());
  lay->n_scan = static_cast<int32_t>(scan.size());
  lay->phase1 = static_cast<const SegItem*>(at(put(ph1.data(), ph1.size() * sizeof(SegItem))));
  lay->phase3 = static_cast<const SegItem*>(at(put(ph3.data(), ph3.size() * sizeof(SegItem))));
  lay->scan = static_cast<const ScanItem*>(at(put(scan.data(), scan.size() * sizeof(ScanItem))));
  return out;
}

// Turns the section offsets of `lay` into addresses within `dev`.
void relocate(wkv7::Launch* lay, const void* dev) {
  auto fix = [&](auto*& ptr) {
    using T = std::remove_reference_t<decltype(ptr)>;
    ptr = reinterpret_cast<T>(static_cast<const char*>(dev) +
                              reinterpret_cast<uintptr_t>(ptr));
  };
  fix(lay->seq);
  lay->chunk_all = lay->seq + lay->n_seq;
  if (lay->n_phase3 > 0) {
    fix(lay->phase1);
    fix(lay->phase3);
    fix(lay->scan);
  }
}

wkv7_status check_forward_args(int32_t dtype, int64_t T_tot, const void* r,
                               const void* w, const void* k, const void* v,
                               const void* a, const void* b, const float* o) {
  if (dtype != WKV7_F32 && dtype != WKV7_BF16)
    return fail(WKV7_ERR_UNSUPPORTED, "dtype %d unsupported", dtype);
  if (T_tot == 0) return WKV7_OK;
  const void* ptrs[7] = {r, w, k, v, a, b, o};
  const char* names[7] = {"r", "w", "k", "v", "a", "b", "o"};
  for (int i = 0; i < 7; ++i) {
    if (!ptrs[i]) return fail(WKV7_ERR_INVALID_ARG, "%s is NULL", names[i]);
    if (!aligned16(ptrs[i]))
      return fail(WKV7_ERR_INVALID_ARG, "%s is not 16-byte aligned", names[i]);
  }
  return WKV7_OK;
}

// Launches the kernels of a batch whose work description is on the device.
// Split sequences run segment-parallel (three launches: segment transitions
// and zero-start states together with the unsplit chunked sequences, the
// carry scan, the segments' outputs); otherwise every chunked sequence runs
// whole. The chunked launches take the precise plan for fp32 inputs and
// with CHUNK_PRECISE.
// Decode items (single-token sequences) ride in trailing workgroups of the
// batch's chunked launch when the two together fit the CUs in one round
// (the chunked kernel holds one workgroup per CU); with segment-parallel
// prefill that is the output launch (phase 3: one item per segment, never
// more than the transition launch, which has two per non-last segment plus
// the unsplit sequences). Otherwise they get a launch of their own. Short multi-token sequences take
// the four-wavefront sequential kernel while the batch has few of them.
// Every route computes the same bits for a sequential item.
wkv7_status launch_batch(const wkv7_pool* p, const wkv7::Launch& L,
                         int32_t dtype, const void* r, const void* w,
                         const void* k, const void* v, const void* a,
                         const void* b, float* o, hipStream_t hs) {
  wkv7::SeqArgs args{p->state, nullptr, 0, p->H, dtype, r, w, k, v, a, b, o};
  const bool precise = p->chunk_precise;
  const bool segmented = L.n_phase3 > 0;
  const int32_t n_single = L.n_seq_single;
  const int32_t n_multi = L.n_seq - L.n_seq_single;
  bool fuse = false;
  if (n_single > 0) {
    const int64_t chunk_items = segmented ? L.n_phase3 : L.n_chunk_all;
    fuse = chunk_items > 0 &&
           chunk_items * p->H + wkv7::chunk_decode_blocks(n_single, p->H) <= p->n_cus;
  }
  if (n_single > 0 && !fuse) {
    args.items = L.seq;
    args.n_items = n_single;
    hipError_t e = wkv7::launch_seq1(args, hs);
    if (e != hipSuccess) return fail_hip(e, "sequential kernel launch");
  }
  if (n_multi > 0) {
    // Four wavefronts per (sequence, head) cut a short sequence's latency
    // about fourfold while the batch leaves the GPU room (up to 8 chains per
    // CU, four wavefronts each); beyond that the one-wavefront kernel's
    // throughput is better (it reads each token's inputs once, not four
    // times). Both compute the same bits, so the choice cannot change a
    // result.
    args.items = L.seq + n_single;
    args.n_items = n_multi;
    const bool wide = static_cast<int64_t>(n_multi) * p->H <= 8 * p->n_cus;
    hipError_t e = wide ? wkv7::launch_seq4(args, hs) : wkv7::launch_seq(args, hs);
    if (e != hipSuccess) return fail_hip(e, "sequential kernel launch");
  }
  if (!segmented) {
    if (L.n_chunk_all > 0) {
      args.items = L.chunk_all;
      args.n_items = L.n_chunk_all;
      hipError_t e = fuse ? wkv7::launch_chunked_p(args, precise, hs, L.seq, n_single)
                          : wkv7::launch_chunked_p(args, precise, hs);
      if (e != hipSuccess) return fail_hip(e, "chunked kernel launch");
    }
    return WKV7_OK;
  }
  args.items = nullptr;
  args.n_items = L.n_phase1;
  hipError_t e = wkv7::launch_chunked_p_seg(args, precise, L.phase1, hs);
  if (e != hipSuccess) return fail_hip(e, "segment transition launch");
  e = wkv7::launch_seg_scan(L.scan, L.n_scan, p->H, hs);
  if (e != hipSuccess) return fail_hip(e, "segment scan launch");
  args.n_items = L.n_phase3;
  e = fuse ? wkv7::launch_chunked_p_seg(args, precise, L.phase3, hs, L.seq, n_single)
           : wkv7::launch_chunked_p_seg(args, precise, L.phase3, hs);
  if (e != hipSuccess) return fail_hip(e, "segment prefill launch");
  return WKV7_OK;
}

// Makes the pool's segment buffers hold at least `floats` (grow only; an
// outgrown buffer is kept until destroy, since queued work may still use it
// and freeing would wait for the device).
wkv7_status ensure_seg_scratch(wkv7_pool* p, size_t floats) {
  if (floats <= p->seg_scratch_floats) return WKV7_OK;
  if (p->seg_scratch) p->retired.emplace_back(p->seg_scratch, false);
  p->seg_scratch = nullptr;
  p->seg_scratch_floats = 0;
  if (hipMalloc(reinterpret_cast<void**>(&p->seg_scratch), floats * 4) != hipSuccess)
    return fail(WKV7_ERR_OOM, "segment buffers of %zu bytes", floats * 4);
  p->seg_scratch_floats = floats;
  return WKV7_OK;
}

}  // namespace

namespace wkv7 {

wkv7_status host_fail(wkv7_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

void host_clear_error() { g_last_error.clear(); }

int pool_device(const wkv7_pool* p) { return p->device; }

}  // namespace wkv7

extern "C" {

const char* wkv7_last_error(void) { return g_last_error.c_str(); }

int32_t wkv7_version(void) { return 100; }  // 0.1.0

wkv7_status wkv7_pool_create(int32_t n_slots, int32_t H, int32_t N,
                             wkv7_pool** out) {
  g_last_error.clear();
  if (!out) return fail(WKV7_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (n_slots < 1 || H < 1)
    return fail(WKV7_ERR_INVALID_ARG, "n_slots=%d and H=%d must be >= 1",
                n_slots, H);
  if (N != wkv7::kN)
    return fail(WKV7_ERR_UNSUPPORTED, "head size N=%d unsupported (only %d)",
                N, wkv7::kN);
  const size_t slot_floats = static_cast<size_t>(H) * N * N;
  if (slot_floats > (size_t(1) << 40) / static_cast<size_t>(n_slots))
    return fail(WKV7_ERR_INVALID_ARG, "pool of %d x %zu floats is too large",
                n_slots, slot_floats);
  wkv7_pool* p = new (std::nothrow) wkv7_pool();
  if (!p) return fail(WKV7_ERR_OOM, "host allocation failed");
  hipError_t e = hipGetDevice(&p->device);
  if (e != hipSuccess) { delete p; return fail_hip(e, "hipGetDevice"); }
  e = hipDeviceGetAttribute(&p->n_cus, hipDeviceAttributeMultiprocessorCount,
                            p->device);
  if (e != hipSuccess) { delete p; return fail_hip(e, "hipDeviceGetAttribute"); }
  p->n_slots = n_slots;
  p->H = H;
  p->N = N;
  p->slot_floats = slot_floats;
  const size_t bytes = slot_floats * sizeof(float) * static_cast<size_t>(n_slots);
  e = hipMalloc(reinterpret_cast<void**>(&p->state), bytes);
  if (e != hipSuccess) {
    delete p;
    return fail(WKV7_ERR_OOM, "hipMalloc of %zu bytes for the pool failed: %s",
                bytes, hipGetErrorString(e));
  }
  e = hipMemset(p->state, 0, bytes);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  // The staging events order work only: a copy has finished reading its
  // pinned host buffer, the kernels reading a device copy have finished
  // before the next copy overwrites it. Nothing the device writes is read by
  // the host through them, so they skip the system-scope cache writeback and
  // invalidation of a default event (measured: ~1 us of GPU time per call
  // instead of ~3).
  for (int i = 0; e == hipSuccess && i < kRing; ++i) {
    Stage& st = p->ring[i];
    e = hipEventCreateWithFlags(&st.ev,
                                hipEventDisableTiming | hipEventDisableSystemFence);
    if (e == hipSuccess)
      e = hipHostMalloc(reinterpret_cast<void**>(&st.host), kStageMinInts * 4);
    if (e == hipSuccess)
      e = hipMalloc(reinterpret_cast<void**>(&st.dev), kStageMinInts * 4);
    if (e == hipSuccess) st.cap_ints = kStageMinInts;
  }
  if (e != hipSuccess) {
    std::string msg = std::string("pool initialisation: ") + hipGetErrorString(e);
    wkv7_pool_destroy(p);
    return fail(WKV7_ERR_HIP, "%s", msg.c_str());
  }
  if (wkv7_status st = wkv7::static_scratch_setup(&p->static_scratch)) {
    std::string msg = g_last_error;
    wkv7_pool_destroy(p);
    return fail(st, "%s", msg.c_str());
  }
  p->allocated.assign(static_cast<size_t>(n_slots), 0);
  p->free_ids.resize(static_cast<size_t>(n_slots));
  for (int32_t i = 0; i < n_slots; ++i) p->free_ids[i] = n_slots - 1 - i;
  *out = p;
  return WKV7_OK;
}

wkv7_status wkv7_pool_destroy(wkv7_pool* p) {
  g_last_error.clear();
  if (!p) return WKV7_OK;
  DeviceGuard guard(p->device);
  hipError_t e = hipDeviceSynchronize();
  for (int i = 0; i < kRing; ++i) {
    Stage& s = p->ring[i];
    if (s.host) (void)hipHostFree(s.host);
    if (s.dev) (void)hipFree(s.dev);
    if (s.ev) (void)hipEventDestroy(s.ev);
  }
  if (p->state) (void)hipFree(p->state);
  if (p->seg_scratch) (void)hipFree(p->seg_scratch);
  if (p->xfer_stage) (void)hipFree(p->xfer_stage);
  for (const auto& r : p->retired)
    (void)(r.second ? hipHostFree(r.first) : hipFree(r.first));
  delete p;
  if (e != hipSuccess) return fail_hip(e, "hipDeviceSynchronize(destroy)");
  return WKV7_OK;
}

size_t wkv7_slot_bytes(const wkv7_pool* p) { return p ? slot_bytes_of(p) : 0; }

void* wkv7_pool_state_ptr(wkv7_pool* p) { return p ? p->state : nullptr; }

wkv7_status wkv7_pool_shape(const wkv7_pool* p, int32_t* n_slots, int32_t* H,
                            int32_t* N) {
  g_last_error.clear();
  if (wkv7_status st = check_pool(p)) return st;
  if (n_slots) *n_slots = p->n_slots;
  if (H) *H = p->H;
  if (N) *N = p->N;
  return WKV7_OK;
}

wkv7_status wkv7_pool_device(const wkv7_pool* p, int32_t* device) {
  g_last_error.clear();
  if (wkv7_status st = check_pool(p)) return st;
  if (!device) return fail(WKV7_ERR_INVALID_ARG, "device is NULL");
  *device = p->device;
  return WKV7_OK;
}

wkv7_status wkv7_pool_set_option(wkv7_pool* p, int32_t opt, int64_t val) {
  g_last_error.clear();
  if (wkv7_status st = check_pool(p)) return st;
  if (opt == WKV7_OPT_PREFILL_MIN_LEN) {
    if (val < 1) return fail(WKV7_ERR_INVALID_ARG,
                             "PREFILL_MIN_LEN=%lld must be >= 1",
                             static_cast<long long>(val));
    p->prefill_min_len = val;
    return WKV7_OK;
  }
  if (opt == WKV7_OPT_CHUNK_PRECISE) {
    if (val != 0 && val != 1)
      return fail(WKV7_ERR_INVALID_ARG, "CHUNK_PRECISE=%lld must be 0 or 1",
                  static_cast<long long>(val));
    p->chunk_precise = val != 0;
    return WKV7_OK;
  }
  if (opt == WKV7_OPT_SEGMENT_LEN) {
    if (val != 0 && (val < 64 || val % 32 != 0 || val > (int64_t(1) << 30)))
      return fail(WKV7_ERR_INVALID_ARG,
                  "SEGMENT_LEN=%lld must be 0 or a multiple of 32, >= 64",
                  static_cast<long long>(val));
    p->segment_len = val;
    return WKV7_OK;
  }
  return fail(WKV7_ERR_UNSUPPORTED, "unknown option %d", opt);
}

wkv7_status wkv7_slot_alloc(wkv7_pool* p, int32_t n, int32_t* ids_out) {
  g_last_error.clear();
  if (wkv7_status st = check_pool(p)) return st;
  if (n < 0) return fail(WKV7_ERR_INVALID_ARG, "n=%d < 0", n);
  if (n > 0 && !ids_out) return fail(WKV7_ERR_INVALID_ARG, "ids_out is NULL");
  if (static_cast<size_t>(n) > p->free_ids.size())
    return fail(WKV7_ERR_POOL_FULL, "%d slots requested, %zu free", n,
                p->free_ids.size());
  for (int32_t i = 0; i < n; ++i) {
    int32_t id = p->free_ids.back();
    p->free_ids.pop_back();
    p->allocated[id] = 1;
    ids_out[i] = id;
  }
  return WKV7_OK;
}

wkv7_status wkv7_slot_free(wkv7_pool* p, const int32_t* ids, int32_t n) {
  g_last_error.clear();
  if (wkv7_status st = check_pool(p)) return st;
  if (wkv7_status st = check_ids(p, ids, n, true, "slot_free")) return st;
  for (int32_t i = 0; i < n; ++i)
    if (!p->allocated[ids[i]])
      return fail(WKV7_ERR_INVALID_ARG, "slot_free: slot %d is not allocated",
                  ids[i]);
  for (int32_t i = 0; i < n; ++i) {
    p->allocated[ids[i]] = 0;
    p->free_ids.push_back(ids[i]);
  }
  return WKV7_OK;
}

wkv7_status wkv7_forward(wkv7_pool* p, const int32_t* slot_ids,
                         const int32_t* cu_seqlens, int32_t n_seqs,
                         int32_t dtype, const void* r, const void* w,
                         const void* k, const void* v, const void* a,
                         const void* b, float* o, void* stream) {
  g_last_error.clear();
  if (wkv7_status st = check_pool(p)) return st;
  Batch bt;
  if (wkv7_status st = build_batch(p, slot_ids, cu_seqlens, n_seqs, "forward", &bt))
    return st;
  if (wkv7_status st = check_forward_args(dtype, bt.T_tot, r, w, k, v, a, b, o))
    return st;
  if (bt.items.empty()) return WKV7_OK;

  DeviceGuard guard(p->device);
  if (!guard.ok) return fail(WKV7_ERR_HIP, "cannot select the pool's device");
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (wkv7_status st = ensure_seg_scratch(p, seg_scratch_floats(p, bt))) return st;
  wkv7::Launch L;
  const std::vector<int32_t> words = serialize(p, bt, p->seg_scratch, &L);
  const int32_t* dev = nullptr;
  Stage* stage = nullptr;
  if (wkv7_status st = stage_upload(p, words.data(), words.size(), hs, &dev, &stage))
    return st;
  relocate(&L, dev);
  if (wkv7_status st = launch_batch(p, L, dtype, r, w, k, v, a, b, o, hs))
    return st;
  return stage_commit(stage, hs);
}

wkv7_status wkv7_forward_noalloc(wkv7_pool* p, const int32_t* slot_ids,
                                 const int32_t* cu_seqlens, int32_t n_seqs,
                                 int32_t dtype, const void* r, const void* w,
                                 const void* k, const void* v, const void* a,
                                 const void* b, float* o, void* stream) {
  g_last_error.clear();
  if (wkv7_status st = check_pool(p)) return st;
  Batch bt;
  if (wkv7_status st = build_batch(p, slot_ids, cu_seqlens, n_seqs,
                                   "forward_noalloc", &bt))
    return st;
  if (wkv7_status st = check_forward_args(dtype, bt.T_tot, r, w, k, v, a, b, o))
    return st;
  if (bt.items.empty()) return WKV7_OK;
  if (!p->static_scratch)
    return fail(WKV7_ERR_HIP, "the device's static scratch is not set up");
  // segment buffers at the start of the scratch, the work description after
  // them (256-byte aligned)
  char* base = static_cast<char*>(p->static_scratch);
  const size_t seg_bytes = seg_scratch_floats(p, bt) * 4;
  const size_t meta_off = (seg_bytes + 255) & ~size_t(255);
  wkv7::Launch L;
  const std::vector<int32_t> words =
      serialize(p, bt, reinterpret_cast<float*>(base), &L);
  const size_t meta_bytes = words.size() * 4;
  if (meta_bytes > wkv7::kStaticMetaBytes ||
      meta_off + meta_bytes > wkv7::kStaticScratchBytes)
    return fail(WKV7_ERR_INVALID_ARG,
                "forward_noalloc: the batch needs %zu bytes of work description "
                "and %zu of segment buffers; the static scratch holds %zu "
                "bytes, at most %zu of them work description",
                meta_bytes, seg_bytes, wkv7::kStaticScratchBytes,
                wkv7::kStaticMetaBytes);

  DeviceGuard guard(p->device);
  if (!guard.ok) return fail(WKV7_ERR_HIP, "cannot select the pool's device");
  hipStream_t hs = static_cast<hipStream_t>(stream);
  // Stage through the next ring entry (preallocated, never grown here): wait
  // until the copy that last read its host buffer has finished.
  Stage& sg = p->ring[p->ring_pos];
  p->ring_pos = (p->ring_pos + 1) % kRing;
  hipError_t e;
  if (sg.pending) {
    e = hipEventSynchronize(sg.ev);
    if (e != hipSuccess) return fail_hip(e, "hipEventSynchronize(staging)");
    sg.pending = false;
  }
  sg.n_ints = 0;          // its device buffer no longer mirrors the host one
  std::memcpy(sg.host, words.data(), meta_bytes);
  e = hipMemcpyAsync(base + meta_off, sg.host, meta_bytes,
                     hipMemcpyHostToDevice, hs);
  if (e != hipSuccess) return fail_hip(e, "hipMemcpyAsync(metadata)");
  sg.stream = hs;
  e = hipEventRecord(sg.ev, hs);
  if (e != hipSuccess) return fail_hip(e, "hipEventRecord(staging)");
  sg.pending = true;
  relocate(&L, base + meta_off);
  return launch_batch(p, L, dtype, r, w, k, v, a, b, o, hs);
}

wkv7_status wkv7_plan_create(wkv7_pool* p, const int32_t* slot_ids,
                             const int32_t* cu_seqlens, int32_t n_seqs,
                             wkv7_plan** out) {
  g_last_error.clear();
  if (!out) return fail(WKV7_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (wkv7_status st = check_pool(p)) return st;
  Batch bt;
  if (wkv7_status st = build_batch(p, slot_ids, cu_seqlens, n_seqs, "plan", &bt))
    return st;
  wkv7_plan* pl = new (std::nothrow) wkv7_plan();
  if (!pl) return fail(WKV7_ERR_OOM, "host allocation failed");
  pl->pool = p;
  pl->device = p->device;
  pl->T_tot = bt.T_tot;
  if (!bt.items.empty()) {
    DeviceGuard guard(p->device);
    if (!guard.ok) { delete pl; return fail(WKV7_ERR_HIP, "cannot select the pool's device"); }
    const size_t sf = seg_scratch_floats(p, bt);
    if (sf > 0 &&
        hipMalloc(reinterpret_cast<void**>(&pl->scratch), sf * 4) != hipSuccess) {
      delete pl;
      return fail(WKV7_ERR_OOM, "segment buffers of %zu bytes for the plan", sf * 4);
    }
    const std::vector<int32_t> words = serialize(p, bt, pl->scratch, &pl->launch);
    const size_t bytes = words.size() * 4;
    hipError_t e = hipMalloc(&pl->dev, bytes);
    if (e != hipSuccess) {
      if (pl->scratch) (void)hipFree(pl->scratch);
      delete pl;
      return fail(WKV7_ERR_OOM, "hipMalloc of %zu bytes for the plan failed: %s",
                  bytes, hipGetErrorString(e));
    }
    e = hipMemcpy(pl->dev, words.data(), bytes, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      (void)hipFree(pl->dev);
      if (pl->scratch) (void)hipFree(pl->scratch);
      delete pl;
      return fail_hip(e, "hipMemcpy(plan)");
    }
    relocate(&pl->launch, pl->dev);
  }
  *out = pl;
  return WKV7_OK;
}

int64_t wkv7_plan_tokens(const wkv7_plan* pl) { return pl ? pl->T_tot : 0; }

wkv7_status wkv7_forward_plan(wkv7_pool* p, const wkv7_plan* pl, int32_t dtype,
                              const void* r, const void* w, const void* k,
                              const void* v, const void* a, const void* b,
                              float* o, void* stream) {
  g_last_error.clear();
  if (wkv7_status st = check_pool(p)) return st;
  if (!pl) return fail(WKV7_ERR_INVALID_ARG, "plan is NULL");
  if (pl->pool != p)
    return fail(WKV7_ERR_INVALID_ARG, "the plan was made for another pool");
  if (wkv7_status st = check_forward_args(dtype, pl->T_tot, r, w, k, v, a, b, o))
    return st;
  if (!pl->dev) return WKV7_OK;
  DeviceGuard guard(p->device);
  if (!guard.ok) return fail(WKV7_ERR_HIP, "cannot select the pool's device");
  return launch_batch(p, pl->launch, dtype, r, w, k, v, a, b, o,
                      static_cast<hipStream_t>(stream));
}

wkv7_status wkv7_plan_destroy(wkv7_plan* pl) {
  g_last_error.clear();
  if (!pl) return WKV7_OK;
  hipError_t e = hipSuccess;
  if (pl->dev) {
    DeviceGuard guard(pl->device);
    e = hipDeviceSynchronize();
    (void)hipFree(pl->dev);
    if (pl->scratch) (void)hipFree(pl->scratch);
  }
  delete pl;
  if (e != hipSuccess) return fail_hip(e, "hipDeviceSynchronize(plan destroy)");
  return WKV7_OK;
}

wkv7_status wkv7_snapshot(wkv7_pool* p, int32_t slot, void* dst_device,
                          void* stream) {
  g_last_error.clear();
  if (wkv7_status st = check_pool(p)) return st;
  if (wkv7_status st = check_ids(p, &slot, 1, false, "snapshot")) return st;
  if (!dst_device) return fail(WKV7_ERR_INVALID_ARG, "dst_device is NULL");
  DeviceGuard guard(p->device);
  if (!guard.ok) return fail(WKV7_ERR_HIP, "cannot select the pool's device");
  hipError_t e = hipMemcpyAsync(dst_device, p->state + slot * p->slot_floats,
                                slot_bytes_of(p), hipMemcpyDeviceToDevice,
                                static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail_hip(e, "hipMemcpyAsync(snapshot)");
  return WKV7_OK;
}

wkv7_status wkv7_fork(wkv7_pool* p, const int32_t* src, const int32_t* dst,
                      int32_t n, void* stream) {
  g_last_error.clear();
  if (wkv7_status st = check_pool(p)) return st;
  if (wkv7_status st = check_ids(p, src, n, false, "fork src")) return st;
  if (wkv7_status st = check_ids(p, dst, n, true, "fork dst")) return st;
  if (n == 0) return WKV7_OK;
  std::vector<uint8_t> is_src(static_cast<size_t>(p->n_slots), 0);
  for (int32_t i = 0; i < n; ++i) is_src[src[i]] = 1;
  for (int32_t i = 0; i < n; ++i)
    if (is_src[dst[i]])
      return fail(WKV7_ERR_DUPLICATE_SLOT,
                  "fork: slot %d is both a source and a destination", dst[i]);
  std::vector<int32_t> pairs(2 * static_cast<size_t>(n));
  for (int32_t i = 0; i < n; ++i) {
    pairs[2 * i] = src[i];
    pairs[2 * i + 1] = dst[i];
  }
  DeviceGuard guard(p->device);
  if (!guard.ok) return fail(WKV7_ERR_HIP, "cannot select the pool's device");
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const int32_t* dev = nullptr;
  Stage* stage = nullptr;
  if (wkv7_status st = stage_upload(p, pairs.data(), pairs.size(), hs, &dev,
                                    &stage))
    return st;
  hipError_t e = wkv7::launch_copy_slots(p->state, p->state, p->slot_floats,
                                         dev, n, hs);
  if (e != hipSuccess) return fail_hip(e, "slot copy launch");
  return stage_commit(stage, hs);
}

wkv7_status wkv7_migrate(wkv7_pool* src, const int32_t* src_ids,
                         wkv7_pool* dst, const int32_t* dst_ids, int32_t n,
                         void* stream) {
  g_last_error.clear();
  if (wkv7_status st = check_pool(src)) return st;
  if (wkv7_status st = check_pool(dst)) return st;
  if (src == dst) return wkv7_fork(src, src_ids, dst_ids, n, stream);
  if (src->H != dst->H || src->N != dst->N)
    return fail(WKV7_ERR_UNSUPPORTED,
                "migrate: slot shapes differ (H=%d N=%d vs H=%d N=%d)", src->H,
                src->N, dst->H, dst->N);
  if (src->device != dst->device)
    return fail(WKV7_ERR_UNSUPPORTED,
                "migrate: pools on devices %d and %d (only same-device "
                "migration is built)", src->device, dst->device);
  if (wkv7_status st = check_ids(src, src_ids, n, false, "migrate src")) return st;
  if (wkv7_status st = check_ids(dst, dst_ids, n, true, "migrate dst")) return st;
  if (n == 0) return WKV7_OK;
  std::vector<int32_t> pairs(2 * static_cast<size_t>(n));
  for (int32_t i = 0; i < n; ++i) {
    pairs[2 * i] = src_ids[i];
    pairs[2 * i + 1] = dst_ids[i];
  }
  DeviceGuard guard(dst->device);
  if (!guard.ok) return fail(WKV7_ERR_HIP, "cannot select the pools' device");
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const int32_t* dev = nullptr;
  Stage* stage = nullptr;
  if (wkv7_status st = stage_upload(dst, pairs.data(), pairs.size(), hs, &dev,
                                    &stage))
    return st;
  hipError_t e = wkv7::launch_copy_slots(src->state, dst->state,
                                         dst->slot_floats, dev, n, hs);
  if (e != hipSuccess) return fail_hip(e, "slot migrate launch");
  return stage_commit(stage, hs);
}

wkv7_status wkv7_q8_quantize(const void* x, int32_t dtype, int64_t rows,
                             int64_t cols, int8_t* q, float* scale,
                             void* stream) {
  g_last_error.clear();
  if (dtype != WKV7_F32 && dtype != WKV7_BF16)
    return fail(WKV7_ERR_UNSUPPORTED, "dtype %d unsupported", dtype);
  if (rows < 0 || cols < 1)
    return fail(WKV7_ERR_INVALID_ARG, "rows=%lld must be >= 0 and cols=%lld >= 1",
                static_cast<long long>(rows), static_cast<long long>(cols));
  if (rows == 0) return WKV7_OK;
  if (!x || !q || !scale)
    return fail(WKV7_ERR_INVALID_ARG, "x, q and scale must not be NULL");
  hipError_t e = wkv7::launch_q8_quantize(x, dtype, rows, cols, q, scale,
                                          static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail_hip(e, "quantize launch");
  return WKV7_OK;
}

wkv7_status wkv7_q8_matmul(const int8_t* wq, const float* w_scale,
                           int64_t out, int64_t in, const int8_t* xq,
                           const float* x_scale, int64_t B, float* y,
                           void* stream) {
  g_last_error.clear();
  if (out < 0 || in < 1 || B < 0)
    return fail(WKV7_ERR_INVALID_ARG, "out=%lld, in=%lld, B=%lld",
                static_cast<long long>(out), static_cast<long long>(in),
                static_cast<long long>(B));
  if (in % 64 != 0 || out % 16 != 0)
    return fail(WKV7_ERR_UNSUPPORTED,
                "q8 product needs in %% 64 == 0 and out %% 16 == 0 "
                "(in=%lld, out=%lld)", static_cast<long long>(in),
                static_cast<long long>(out));
  if (out == 0 || B == 0) return WKV7_OK;
  if (out * in >= (int64_t(1) << 31) || B * in >= (int64_t(1) << 31))
    return fail(WKV7_ERR_UNSUPPORTED,
                "q8 product operands must each be under 2 GiB of codes");
  const void* ptrs[5] = {wq, w_scale, xq, x_scale, y};
  const char* names[5] = {"wq", "w_scale", "xq", "x_scale", "y"};
  for (int i = 0; i < 5; ++i) {
    if (!ptrs[i]) return fail(WKV7_ERR_INVALID_ARG, "%s is NULL", names[i]);
    if (i != 3 && !aligned16(ptrs[i]))
      return fail(WKV7_ERR_INVALID_ARG, "%s is not 16-byte aligned", names[i]);
  }
  hipError_t e = wkv7::launch_q8_matmul(wq, w_scale, out, in, xq, x_scale, B,
                                        y, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail_hip(e, "q8 product launch");
  return WKV7_OK;
}

wkv7_status wkv7_q8_linear(const int8_t* wq, const float* w_scale,
                           int64_t out, int64_t in, const void* x,
                           int32_t dtype, int64_t B, int8_t* xq,
                           float* x_scale, float* y, void* stream) {
  g_last_error.clear();
  if (dtype != WKV7_F32 && dtype != WKV7_BF16)
    return fail(WKV7_ERR_UNSUPPORTED, "dtype %d unsupported", dtype);
  if (out < 0 || in < 1 || B < 0)
    return fail(WKV7_ERR_INVALID_ARG, "out=%lld, in=%lld, B=%lld",
                static_cast<long long>(out), static_cast<long long>(in),
                static_cast<long long>(B));
  if (in % 64 != 0 || out % 16 != 0)
    return fail(WKV7_ERR_UNSUPPORTED,
                "q8 product needs in %% 64 == 0 and out %% 16 == 0 "
                "(in=%lld, out=%lld)", static_cast<long long>(in),
                static_cast<long long>(out));
  if (out == 0 || B == 0) return WKV7_OK;
  if (out * in >= (int64_t(1) << 31) || B * in >= (int64_t(1) << 31))
    return fail(WKV7_ERR_UNSUPPORTED,
                "q8 product operands must each be under 2 GiB of codes");
  const void* ptrs[6] = {wq, w_scale, x, xq, x_scale, y};
  const char* names[6] = {"wq", "w_scale", "x", "xq", "x_scale", "y"};
  for (int i = 0; i < 6; ++i) {
    if (!ptrs[i]) return fail(WKV7_ERR_INVALID_ARG, "%s is NULL", names[i]);
    if (i != 4 && !aligned16(ptrs[i]))
      return fail(WKV7_ERR_INVALID_ARG, "%s is not 16-byte aligned", names[i]);
  }
  hipError_t e = wkv7::launch_q8_linear(wq, w_scale, out, in, x, dtype, B, xq,
                                        x_scale, y, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail_hip(e, "q8 linear launch");
  return WKV7_OK;
}

wkv7_status wkv7_image_header_init(wkv7_image_header* hdr, int32_t H,
                                   int32_t N, int32_t n_slots) {
  g_last_error.clear();
  if (!hdr) return fail(WKV7_ERR_INVALID_ARG, "hdr is NULL");
  if (H < 1 || n_slots < 0)
    return fail(WKV7_ERR_INVALID_ARG, "H=%d must be >= 1 and n_slots=%d >= 0",
                H, n_slots);
  if (N != wkv7::kN)
    return fail(WKV7_ERR_UNSUPPORTED, "head size N=%d unsupported (only %d)",
                N, wkv7::kN);
  std::memset(hdr, 0, sizeof(*hdr));
  std::memcpy(hdr->magic, WKV7_IMAGE_MAGIC, 8);
  hdr->version = WKV7_IMAGE_VERSION;
  hdr->header_bytes = sizeof(wkv7_image_header);
  hdr->H = static_cast<uint32_t>(H);
  hdr->N = static_cast<uint32_t>(N);
  hdr->state_dtype = WKV7_F32;
  hdr->n_slots = static_cast<uint32_t>(n_slots);
  hdr->slot_bytes = static_cast<uint64_t>(H) * N * N * sizeof(float);
  return WKV7_OK;
}

wkv7_status wkv7_image_header_check(const wkv7_image_header* hdr, int32_t H,
                                    int32_t N) {
  g_last_error.clear();
  if (!hdr) return fail(WKV7_ERR_INVALID_ARG, "hdr is NULL");
  if (std::memcmp(hdr->magic, WKV7_IMAGE_MAGIC, 8) != 0)
    return fail(WKV7_ERR_INVALID_ARG, "not a slot image (bad magic)");
  if (hdr->version != WKV7_IMAGE_VERSION ||
      hdr->header_bytes != sizeof(wkv7_image_header))
    return fail(WKV7_ERR_UNSUPPORTED,
                "slot image version %u (header %u bytes); this library reads "
                "version %d (%zu bytes)", hdr->version, hdr->header_bytes,
                WKV7_IMAGE_VERSION, sizeof(wkv7_image_header));
  for (int i = 0; i < 3; ++i)
    if (hdr->reserved[i] != 0)
      return fail(WKV7_ERR_INVALID_ARG, "reserved header field %d is not 0", i);
  if (hdr->state_dtype != WKV7_F32 ||
      hdr->slot_bytes != static_cast<uint64_t>(hdr->H) * hdr->N * hdr->N * 4)
    return fail(WKV7_ERR_INVALID_ARG, "inconsistent slot image header");
  if (static_cast<int64_t>(hdr->H) != H || static_cast<int64_t>(hdr->N) != N)
    return fail(WKV7_ERR_UNSUPPORTED,
                "slot images of H=%u N=%u do not fit slots of H=%d N=%d",
                hdr->H, hdr->N, H, N);
  return WKV7_OK;
}

wkv7_status wkv7_reset(wkv7_pool* p, const int32_t* ids, int32_t n,
                       void* stream) {
  g_last_error.clear();
  if (wkv7_status st = check_pool(p)) return st;
  if (wkv7_status st = check_ids(p, ids, n, true, "reset")) return st;
  if (n == 0) return WKV7_OK;
  DeviceGuard guard(p->device);
  if (!guard.ok) return fail(WKV7_ERR_HIP, "cannot select the pool's device");
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const int32_t* dev = nullptr;
  Stage* stage = nullptr;
  if (wkv7_status st = stage_upload(p, ids, static_cast<size_t>(n), hs, &dev,
                                    &stage))
    return st;
  hipError_t e = wkv7::launch_zero_slots(p->state, p->slot_floats, dev, n, hs);
  if (e != hipSuccess) return fail_hip(e, "slot zero-fill launch");
  return stage_commit(stage, hs);
}

namespace {

// Copies between n slots and n consecutive images in `buf`, one copy per
// run of consecutive slot ids.
wkv7_status copy_runs(wkv7_pool* p, const int32_t* ids, int32_t n, char* buf,
                      bool to_pool, hipStream_t hs) {
  const size_t sb = slot_bytes_of(p);
  int32_t i = 0;
  while (i < n) {
    int32_t j = i + 1;
    while (j < n && ids[j] == ids[j - 1] + 1) ++j;
    char* slot_ptr = reinterpret_cast<char*>(p->state) + ids[i] * sb;
    char* img = buf + static_cast<size_t>(i) * sb;
    const size_t bytes = static_cast<size_t>(j - i) * sb;
    hipError_t e = to_pool
        ? hipMemcpyAsync(slot_ptr, img, bytes, hipMemcpyDefault, hs)
        : hipMemcpyAsync(img, slot_ptr, bytes, hipMemcpyDefault, hs);
    if (e != hipSuccess)
      return fail_hip(e, to_pool ? "hipMemcpyAsync(resume)"
                                 : "hipMemcpyAsync(hibernate)");
    i = j;
  }
  return WKV7_OK;
}

// Scattered slots cross PCIe through a device staging buffer: a kernel
// gathers (or scatters) up to kXferStageBytes of slot images and one DMA
// moves the contiguous block, instead of one DMA per run of consecutive
// ids (each DMA has a set-up cost, so many 1 MiB copies reach about two
// thirds of the rate of one large copy). With few runs the per-run DMA is
// kept: it needs no staging and no kernel.
constexpr size_t kXferStageBytes = static_cast<size_t>(64) << 20;
constexpr int32_t kXferMinRuns = 4;

int32_t count_runs(const int32_t* ids, int32_t n) {
  int32_t runs = n > 0 ? 1 : 0;
  for (int32_t i = 1; i < n; ++i) runs += ids[i] != ids[i - 1] + 1;
  return runs;
}

// Grow-only, like the segment buffers (an outgrown buffer is kept until
// destroy).
wkv7_status ensure_xfer_stage(wkv7_pool* p, size_t bytes) {
  if (bytes <= p->xfer_stage_bytes) return WKV7_OK;
  if (p->xfer_stage) p->retired.emplace_back(p->xfer_stage, false);
  p->xfer_stage = nullptr;
  p->xfer_stage_bytes = 0;
  if (hipMalloc(reinterpret_cast<void**>(&p->xfer_stage), bytes) != hipSuccess)
    return fail(WKV7_ERR_OOM, "transfer staging of %zu bytes", bytes);
  p->xfer_stage_bytes = bytes;
  return WKV7_OK;
}

// True if ptr is device memory of the pool's device, 16-byte aligned (a
// snapshot buffer): resume then scatters straight from it with one kernel.
bool is_pool_device_buffer(const wkv7_pool* p, const void* ptr) {
  if (reinterpret_cast<uintptr_t>(ptr) % 16 != 0) return false;
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, ptr) != hipSuccess) {
    (void)hipGetLastError();          // unregistered host memory: not ours
    return false;
  }
  return attr.type == hipMemoryTypeDevice && attr.device == p->device;
}

wkv7_status copy_slots_staged(wkv7_pool* p, const int32_t* ids, int32_t n,
                              char* buf, bool to_pool, bool device_src,
                              hipStream_t hs) {
  const size_t sb = slot_bytes_of(p);
  // slots per group; a device source is one group read in place
  const int32_t g = device_src
      ? n : static_cast<int32_t>(std::max<size_t>(1, kXferStageBytes / sb));
  if (!device_src)
    if (wkv7_status st = ensure_xfer_stage(p, static_cast<size_t>(std::min(g, n)) * sb))
      return st;
  // (source slot, destination slot) per image; the stage and a device
  // source are indexed like pools, from the start of the group
  std::vector<int32_t> pairs(2 * static_cast<size_t>(n));
  for (int32_t i = 0; i < n; ++i) {
    const int32_t local = i % g;
    pairs[2 * i] = to_pool ? local : ids[i];
    pairs[2 * i + 1] = to_pool ? ids[i] : local;
  }
  const int32_t* dev = nullptr;
  Stage* stage = nullptr;
  if (wkv7_status st = stage_upload(p, pairs.data(), pairs.size(), hs, &dev, &stage))
    return st;
  for (int32_t g0 = 0; g0 < n; g0 += g) {
    const int32_t m = std::min(g, n - g0);
    const size_t bytes = static_cast<size_t>(m) * sb;
    char* img = buf + static_cast<size_t>(g0) * sb;
    hipError_t e = hipSuccess;
    if (device_src) {
      e = wkv7::launch_copy_slots(reinterpret_cast<const float*>(img), p->state,
                                  p->slot_floats, dev + 2 * g0, m, hs);
      if (e != hipSuccess) return fail_hip(e, "slot scatter launch");
    } else if (to_pool) {
      e = hipMemcpyAsync(p->xfer_stage, img, bytes, hipMemcpyDefault, hs);
      if (e != hipSuccess) return fail_hip(e, "hipMemcpyAsync(resume)");
      e = wkv7::launch_copy_slots(p->xfer_stage, p->state, p->slot_floats,
                                  dev + 2 * g0, m, hs);
      if (e != hipSuccess) return fail_hip(e, "slot scatter launch");
    } else {
      e = wkv7::launch_copy_slots(p->state, p->xfer_stage, p->slot_floats,
                                  dev + 2 * g0, m, hs);
      if (e != hipSuccess) return fail_hip(e, "slot gather launch");
      e = hipMemcpyAsync(img, p->xfer_stage, bytes, hipMemcpyDefault, hs);
      if (e != hipSuccess) return fail_hip(e, "hipMemcpyAsync(hibernate)");
    }
  }
  return stage_commit(stage, hs);
}

wkv7_status copy_slot_images(wkv7_pool* p, const int32_t* ids, int32_t n,
                             char* buf, bool to_pool, hipStream_t hs) {
  if (count_runs(ids, n) < kXferMinRuns) return copy_runs(p, ids, n, buf, to_pool, hs);
  const bool device_src = to_pool && is_pool_device_buffer(p, buf);
  return copy_slots_staged(p, ids, n, buf, to_pool, device_src, hs);
}

}  // namespace

wkv7_status wkv7_hibernate(wkv7_pool* p, const int32_t* ids, int32_t n,
                           void* host_dst, size_t bytes, void* stream) {
  g_last_error.clear();
  if (wkv7_status st = check_pool(p)) return st;
  if (wkv7_status st = check_ids(p, ids, n, false, "hibernate")) return st;
  if (n == 0) return WKV7_OK;
  if (!host_dst) return fail(WKV7_ERR_INVALID_ARG, "host_dst is NULL");
  if (bytes < static_cast<size_t>(n) * slot_bytes_of(p))
    return fail(WKV7_ERR_INVALID_ARG,
                "hibernate: %zu bytes given, %zu needed for %d slots", bytes,
                static_cast<size_t>(n) * slot_bytes_of(p), n);
  DeviceGuard guard(p->device);
  if (!guard.ok) return fail(WKV7_ERR_HIP, "cannot select the pool's device");
  return copy_slot_images(p, ids, n, static_cast<char*>(host_dst), false,
                          static_cast<hipStream_t>(stream));
}

wkv7_status wkv7_resume(wkv7_pool* p, const int32_t* ids, int32_t n,
                        const void* src, size_t bytes, void* stream) {
  g_last_error.clear();
  if (wkv7_status st = check_pool(p)) return st;
  if (wkv7_status st = check_ids(p, ids, n, true, "resume")) return st;
  if (n == 0) return WKV7_OK;
  if (!src) return fail(WKV7_ERR_INVALID_ARG, "src is NULL");
  if (bytes < static_cast<size_t>(n) * slot_bytes_of(p))
    return fail(WKV7_ERR_INVALID_ARG,
                "resume: %zu bytes given, %zu needed for %d slots", bytes,
                static_cast<size_t>(n) * slot_bytes_of(p), n);
  DeviceGuard guard(p->device);
  if (!guard.ok) return fail(WKV7_ERR_HIP, "cannot select the pool's device");
  return copy_slot_images(p, ids, n,
                          const_cast<char*>(static_cast<const char*>(src)), true,
                          static_cast<hipStream_t>(stream));
}

}  // extern "C"
