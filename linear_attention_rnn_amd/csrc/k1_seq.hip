// Sequential WKV-7 kernel for gfx950: decode steps and short sequences.
//
// Operation (page "RWKV-X Architecture", section "WKV-7 Kernel (Generalized
// Delta Rule)"), per head and timestep, in product form:
//   sa_i   = sum_j S_ij a_j                       (state before the decay)
//   S_ij  <- S_ij w_j + sa_i b_j + v_i k_j
//   o_i    = sum_j S_ij r_j                       (updated state)
//
// Mapping: one 64-lane wavefront owns one (sequence, head). Lane l = 16 g + c
// holds rows i = 16 g + m (m = 0..15) and columns j = 4 c .. 4 c + 3 of the
// 64 x 64 fp32 state: 64 floats in registers. For each m the wavefront
// loads or stores four whole 256-byte rows with one 16-byte access per lane,
// so every HBM line is used in full. Row sums over j are a per-lane partial
// over 4 columns followed by a 16-lane butterfly of DPP adds (no LDS, no
// barrier). The state is read once and written once per call however many
// tokens the sequence has; the token loop prefetches the next token's inputs
// while the current one is computed.
//
// When a call's active state is larger than the 256 MB Infinity Cache
// (MALL), the state is streamed with non-temporal loads and stores: on
// MI355X that moves a 1 GiB decode step 8% faster, while for a state that
// fits, the ordinary accesses let the next step's reads hit the cache, and
// the inputs (read once) are loaded with the non-temporal hint instead, so
// that they do not push the state out of that cache.

#include "internal.h"
#include "../../include/wkv7.h"

namespace wkv7 {
namespace {

constexpr int kWavesPerBlock = 4;

#include "seq_wave.h"
using seqw::In;
using seqw::load_state;
using seqw::row_sum16;
using seqw::store_state;

// One wavefront per (sequence, head), kWavesPerBlock per workgroup; ONE:
// every item has one token (decode).
template <int DT, bool NT, bool ONE>
__global__ __launch_bounds__(64 * kWavesPerBlock)
void seq_kernel(SeqArgs p) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Workgroup b runs on XCD b mod 8. For a state streamed from HBM each XCD
  // takes one contiguous eighth of the blocks (XCD x: `per` blocks, one
  // more while x < rem, from x per + min(x, rem)): measured 392.6 -> 389.0
  // us on the 1 GiB step; a state that stays in the MALL keeps the plain
  // order (45.8 against 46.2 us on the 128 MiB step).
  int64_t blk = blockIdx.x;
  if (NT) {
    const int64_t per = gridDim.x / 8, rem = gridDim.x % 8;
    const int64_t x = blk % 8;
    blk = x * per + min(x, rem) + blk / 8;
  }
  const int64_t gw = blk * kWavesPerBlock + wave;
  const int item = static_cast<int>(gw / p.H);
  const int h = static_cast<int>(gw - static_cast<int64_t>(item) * p.H);
  if (item >= p.n_items) return;
  // one-token items whose state streams from HBM take the streaming form;
  // a state that stays in the MALL is faster in the loop form (measured:
  // 45.7 against 48.0 us on the 128 MiB step)
  if (ONE && NT)
    seqw::seq1_wave<DT, NT>(p, p.items[item], h, lane);
  else
    seqw::seq_wave<DT, NT>(p, p.items[item], h, lane);
}

// Multi-token sequences: four wavefronts per (sequence, head), wavefront w
// owning state rows [16 w, 16 w + 16): lane 16 g + c holds rows
// 16 w + 4 g + m (m < 4), columns 4 c .. 4 c + 3. Each row sum is the
// sequential kernel's (a per-lane partial over the same four columns, then
// the same 16-lane butterfly), so the results are the same bits; each
// wavefront does a quarter of the per-token work, and that chain is what
// bounds a short sequence's latency. Inputs come through a ring of kDepth
// tokens loaded ahead; a load past the sequence's end re-reads its last
// token, and such a token leaves the state as it is and rewrites the last
// output row with the same value. So every load and store is issued
// whatever the length, and the compiler's count of memory operations in
// flight is exact: each wait covers only the token it needs.
template <int DT> struct Ring { static constexpr int depth = DT == WKV7_BF16 ? 8 : 4; };

template <int DT, bool NT>
__global__ __launch_bounds__(256)
void seq4_kernel(SeqArgs p) {
  using I = In<DT>;
  using T = typename I::T;
  constexpr int D = Ring<DT>::depth;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int item = static_cast<int>(blockIdx.x / p.H);
  const int h = static_cast<int>(blockIdx.x - static_cast<unsigned>(item) * p.H);
  if (item >= p.n_items) return;
  const WorkItem it = p.items[item];
  const int g = lane >> 4;
  const int c = lane & 15;
  const int row0 = 16 * wv + 4 * g;        // the lane's rows row0 .. row0 + 3

  float* sbase = p.pool + (static_cast<size_t>(it.slot) * p.H + h) * (kN * kN)
                 + static_cast<size_t>(row0) * kN + 4 * c;
  float4 s[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) s[m] = load_state<NT>(sbase + m * kN);

  const T* src[6] = {static_cast<const T*>(p.r), static_cast<const T*>(p.w),
                     static_cast<const T*>(p.k), static_cast<const T*>(p.v),
                     static_cast<const T*>(p.a), static_cast<const T*>(p.b)};
  const size_t tstride = static_cast<size_t>(p.H) * kN;
  const size_t off0 = (static_cast<size_t>(it.tok0) * p.H + h) * kN;
  const int last = it.len - 1;
  struct Raw { typename I::R4 w, a, b, k, r, v; };
  auto load = [&](Raw& x, int t) {          // token min(t, last)
    const size_t off = off0 + static_cast<size_t>(min(t, last)) * tstride;
    x.r = I::template ld4<!NT>(src[0] + off + 4 * c);
    x.w = I::template ld4<!NT>(src[1] + off + 4 * c);
    x.k = I::template ld4<!NT>(src[2] + off + 4 * c);
    x.a = I::template ld4<!NT>(src[4] + off + 4 * c);
    x.b = I::template ld4<!NT>(src[5] + off + 4 * c);
    x.v = I::template ld4<!NT>(src[3] + off + row0);
  };
  Raw ring[D];
  // slot order as in the loop (the wait counts at the loop's entry are the
  // smaller of the first entry's and the back edge's)
#pragma unroll
  for (int u = 0; u < D; ++u) {
    load(ring[u], u);
    __builtin_amdgcn_sched_barrier(0);
  }
  const int sel = c & 3;                    // the output row this lane writes
  for (int t0 = 0; t0 < it.len; t0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int t = t0 + u;
      float w[4], a[4], b[4], k[4], r[4], v[4];
      I::cvt4(ring[u].w, w); I::cvt4(ring[u].a, a); I::cvt4(ring[u].b, b);
      I::cvt4(ring[u].k, k); I::cvt4(ring[u].r, r); I::cvt4(ring[u].v, v);
      if (t < it.len) {                     // uniform; no memory operations
        float sa[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          float q = s[m].x * a[0];
          q = fmaf(s[m].y, a[1], q);
          q = fmaf(s[m].z, a[2], q);
          q = fmaf(s[m].w, a[3], q);
          sa[m] = row_sum16(q);
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          s[m].x = fmaf(s[m].x, w[0], fmaf(sa[m], b[0], v[m] * k[0]));
          s[m].y = fmaf(s[m].y, w[1], fmaf(sa[m], b[1], v[m] * k[1]));
          s[m].z = fmaf(s[m].z, w[2], fmaf(sa[m], b[2], v[m] * k[2]));
          s[m].w = fmaf(s[m].w, w[3], fmaf(sa[m], b[3], v[m] * k[3]));
        }
      }
      float ov[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        float q = s[m].x * r[0];
        q = fmaf(s[m].y, r[1], q);
        q = fmaf(s[m].z, r[2], q);
        q = fmaf(s[m].w, r[3], q);
        ov[m] = row_sum16(q);
      }
      // lanes c, c + 4, c + 8, c + 12 write row row0 + c % 4 (same value)
      float mine = ov[0];
      mine = sel == 1 ? ov[1] : mine;
      mine = sel == 2 ? ov[2] : mine;
      mine = sel == 3 ? ov[3] : mine;
      p.o[off0 + static_cast<size_t>(min(t, last)) * tstride + row0 + sel] = mine;
      // refill the slot after its last use, so that the load can land in the
      // same registers (a value still live across it would need a copy, and
      // the copy would wait for the load)
      load(ring[u], t + D);
    }
  }

#pragma unroll
  for (int m = 0; m < 4; ++m) store_state<NT>(sbase + m * kN, s[m]);
}

}  // namespace

hipError_t launch_seq4(const SeqArgs& args, hipStream_t stream) {
  if (args.n_items <= 0) return hipSuccess;
  const int64_t blocks = static_cast<int64_t>(args.n_items) * args.H;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  dim3 grid(static_cast<unsigned>(blocks)), block(256);
  const bool nt = blocks * (kN * kN * sizeof(float)) > (int64_t(256) << 20);
  if (args.dtype == WKV7_BF16) {
    if (nt) hipLaunchKernelGGL((seq4_kernel<WKV7_BF16, true>), grid, block, 0, stream, args);
    else hipLaunchKernelGGL((seq4_kernel<WKV7_BF16, false>), grid, block, 0, stream, args);
  } else {
    if (nt) hipLaunchKernelGGL((seq4_kernel<WKV7_F32, true>), grid, block, 0, stream, args);
    else hipLaunchKernelGGL((seq4_kernel<WKV7_F32, false>), grid, block, 0, stream, args);
  }
  return hipGetLastError();
}

template <bool ONE>
hipError_t launch_seq_impl(const SeqArgs& args, hipStream_t stream) {
  if (args.n_items <= 0) return hipSuccess;
  const int64_t waves = static_cast<int64_t>(args.n_items) * args.H;
  const int64_t blocks = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  dim3 grid(static_cast<unsigned>(blocks)), block(64 * kWavesPerBlock);
  // active state of the call against the MALL's 256 MB
  const bool nt = waves * (kN * kN * sizeof(float)) > (int64_t(256) << 20);
  if (args.dtype == WKV7_BF16) {
    if (nt) hipLaunchKernelGGL((seq_kernel<WKV7_BF16, true, ONE>), grid, block, 0, stream, args);
    else hipLaunchKernelGGL((seq_kernel<WKV7_BF16, false, ONE>), grid, block, 0, stream, args);
  } else {
    if (nt) hipLaunchKernelGGL((seq_kernel<WKV7_F32, true, ONE>), grid, block, 0, stream, args);
    else hipLaunchKernelGGL((seq_kernel<WKV7_F32, false, ONE>), grid, block, 0, stream, args);
  }
  return hipGetLastError();
}

hipError_t launch_seq(const SeqArgs& args, hipStream_t stream) {
  return launch_seq_impl<false>(args, stream);
}

hipError_t launch_seq1(const SeqArgs& args, hipStream_t stream) {
  return launch_seq_impl<true>(args, stream);
}

}  // namespace wkv7
