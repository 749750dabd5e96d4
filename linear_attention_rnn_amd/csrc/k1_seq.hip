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
// fits, the ordinary accesses let the next step's reads hit the cache.

#include "internal.h"
#include "../../include/wkv7.h"

namespace wkv7 {
namespace {

constexpr int kWavesPerBlock = 4;

// 16-lane butterfly sum; every lane of a row of 16 gets the same value.
__device__ __forceinline__ float row_sum16(float x) {
  int xi = __builtin_bit_cast(int, x);
  // quad_perm [1,0,3,2]: partner = lane ^ 1
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, xi, 0xB1, 0xF, 0xF, false));
  xi = __builtin_bit_cast(int, x);
  // quad_perm [2,3,0,1]: partner = lane ^ 2
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, xi, 0x4E, 0xF, 0xF, false));
  xi = __builtin_bit_cast(int, x);
  // row_half_mirror: lane 7 - l within each 8 (joins the two quads)
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, xi, 0x141, 0xF, 0xF, false));
  xi = __builtin_bit_cast(int, x);
  // row_mirror: lane 15 - l within each 16 (joins the two halves)
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, xi, 0x140, 0xF, 0xF, false));
  return x;
}

// Raw input fragments: 4 consecutive channels and 16 consecutive channels.
template <int DT> struct In;

template <> struct In<WKV7_BF16> {
  typedef uint16_t T;
  struct R4 { uint2 u; };
  struct R16 { uint4 u[2]; };
  __device__ static R4 ld4(const T* p) {
    R4 r; r.u = *reinterpret_cast<const uint2*>(p); return r;
  }
  __device__ static R16 ld16(const T* p) {
    R16 r;
    r.u[0] = reinterpret_cast<const uint4*>(p)[0];
    r.u[1] = reinterpret_cast<const uint4*>(p)[1];
    return r;
  }
  __device__ static void lo_hi(uint32_t x, float& lo, float& hi) {
    lo = __uint_as_float(x << 16);
    hi = __uint_as_float(x & 0xffff0000u);
  }
  __device__ static void cvt4(const R4& r, float f[4]) {
    lo_hi(r.u.x, f[0], f[1]);
    lo_hi(r.u.y, f[2], f[3]);
  }
  __device__ static void cvt16(const R16& r, float f[16]) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      lo_hi(r.u[q].x, f[8 * q + 0], f[8 * q + 1]);
      lo_hi(r.u[q].y, f[8 * q + 2], f[8 * q + 3]);
      lo_hi(r.u[q].z, f[8 * q + 4], f[8 * q + 5]);
      lo_hi(r.u[q].w, f[8 * q + 6], f[8 * q + 7]);
    }
  }
};

template <> struct In<WKV7_F32> {
  typedef float T;
  struct R4 { float4 u; };
  struct R16 { float4 u[4]; };
  __device__ static R4 ld4(const T* p) {
    R4 r; r.u = *reinterpret_cast<const float4*>(p); return r;
  }
  __device__ static R16 ld16(const T* p) {
    R16 r;
#pragma unroll
    for (int q = 0; q < 4; ++q) r.u[q] = reinterpret_cast<const float4*>(p)[q];
    return r;
  }
  __device__ static void cvt4(const R4& r, float f[4]) {
    f[0] = r.u.x; f[1] = r.u.y; f[2] = r.u.z; f[3] = r.u.w;
  }
  __device__ static void cvt16(const R16& r, float f[16]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f[4 * q + 0] = r.u[q].x; f[4 * q + 1] = r.u[q].y;
      f[4 * q + 2] = r.u[q].z; f[4 * q + 3] = r.u[q].w;
    }
  }
};

template <int DT>
struct TokenRaw {
  typename In<DT>::R4 w, a, b, k, r;
  typename In<DT>::R16 v;
};

template <int DT>
__device__ __forceinline__ void load_token(TokenRaw<DT>& x,
                                           const typename In<DT>::T* const* src,
                                           size_t off, int c, int g) {
  using I = In<DT>;
  x.r = I::ld4(src[0] + off + 4 * c);
  x.w = I::ld4(src[1] + off + 4 * c);
  x.k = I::ld4(src[2] + off + 4 * c);
  x.a = I::ld4(src[4] + off + 4 * c);
  x.b = I::ld4(src[5] + off + 4 * c);
  x.v = I::ld16(src[3] + off + 16 * g);
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ float4 load_state(const float* p) {
  if (NT) {
    const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    return make_float4(x[0], x[1], x[2], x[3]);
  }
  return *reinterpret_cast<const float4*>(p);
}
template <bool NT>
__device__ __forceinline__ void store_state(float* p, float4 s) {
  if (NT) {
    const f32x4 x = {s.x, s.y, s.z, s.w};
    __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(p));
  } else {
    *reinterpret_cast<float4*>(p) = s;
  }
}

template <int DT, bool NT>
__global__ __launch_bounds__(64 * kWavesPerBlock)
void seq_kernel(SeqArgs p) {
  using I = In<DT>;
  using T = typename I::T;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t gw = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave;
  const int item = static_cast<int>(gw / p.H);
  const int h = static_cast<int>(gw - static_cast<int64_t>(item) * p.H);
  if (item >= p.n_items) return;
  const WorkItem it = p.items[item];
  const int g = lane >> 4;
  const int c = lane & 15;

  float* sbase = p.pool + (static_cast<size_t>(it.slot) * p.H + h) * (kN * kN)
                 + (16 * g) * kN + 4 * c;
  float4 s[16];
#pragma unroll
  for (int m = 0; m < 16; ++m) s[m] = load_state<NT>(sbase + m * kN);

  const T* src[6] = {static_cast<const T*>(p.r), static_cast<const T*>(p.w),
                     static_cast<const T*>(p.k), static_cast<const T*>(p.v),
                     static_cast<const T*>(p.a), static_cast<const T*>(p.b)};
  const size_t tstride = static_cast<size_t>(p.H) * kN;
  size_t off = (static_cast<size_t>(it.tok0) * p.H + h) * kN;

  TokenRaw<DT> nxt;
  load_token<DT>(nxt, src, off, c, g);
  for (int t = 0; t < it.len; ++t) {
    TokenRaw<DT> cur = nxt;
    if (t + 1 < it.len) load_token<DT>(nxt, src, off + tstride, c, g);
    float w[4], a[4], b[4], k[4], r[4], v[16];
    I::cvt4(cur.w, w); I::cvt4(cur.a, a); I::cvt4(cur.b, b);
    I::cvt4(cur.k, k); I::cvt4(cur.r, r); I::cvt16(cur.v, v);

    float sa[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      float q = s[m].x * a[0];
      q = fmaf(s[m].y, a[1], q);
      q = fmaf(s[m].z, a[2], q);
      q = fmaf(s[m].w, a[3], q);
      sa[m] = row_sum16(q);
    }
    float ov[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      s[m].x = fmaf(s[m].x, w[0], fmaf(sa[m], b[0], v[m] * k[0]));
      s[m].y = fmaf(s[m].y, w[1], fmaf(sa[m], b[1], v[m] * k[1]));
      s[m].z = fmaf(s[m].z, w[2], fmaf(sa[m], b[2], v[m] * k[2]));
      s[m].w = fmaf(s[m].w, w[3], fmaf(sa[m], b[3], v[m] * k[3]));
      float q = s[m].x * r[0];
      q = fmaf(s[m].y, r[1], q);
      q = fmaf(s[m].z, r[2], q);
      q = fmaf(s[m].w, r[3], q);
      ov[m] = row_sum16(q);
    }
    // lane c of group g writes o row 16 g + c: one coalesced 256-byte store
    float mine = ov[0];
#pragma unroll
    for (int m = 1; m < 16; ++m) mine = (c == m) ? ov[m] : mine;
    p.o[off + 16 * g + c] = mine;
    off += tstride;
  }

#pragma unroll
  for (int m = 0; m < 16; ++m) store_state<NT>(sbase + m * kN, s[m]);
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
    x.r = I::ld4(src[0] + off + 4 * c);
    x.w = I::ld4(src[1] + off + 4 * c);
    x.k = I::ld4(src[2] + off + 4 * c);
    x.a = I::ld4(src[4] + off + 4 * c);
    x.b = I::ld4(src[5] + off + 4 * c);
    x.v = I::ld4(src[3] + off + row0);
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

hipError_t launch_seq(const SeqArgs& args, hipStream_t stream) {
  if (args.n_items <= 0) return hipSuccess;
  const int64_t waves = static_cast<int64_t>(args.n_items) * args.H;
  const int64_t blocks = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  dim3 grid(static_cast<unsigned>(blocks)), block(64 * kWavesPerBlock);
  // active state of the call against the MALL's 256 MB
  const bool nt = waves * (kN * kN * sizeof(float)) > (int64_t(256) << 20);
  if (args.dtype == WKV7_BF16) {
    if (nt) hipLaunchKernelGGL((seq_kernel<WKV7_BF16, true>), grid, block, 0, stream, args);
    else hipLaunchKernelGGL((seq_kernel<WKV7_BF16, false>), grid, block, 0, stream, args);
  } else {
    if (nt) hipLaunchKernelGGL((seq_kernel<WKV7_F32, true>), grid, block, 0, stream, args);
    else hipLaunchKernelGGL((seq_kernel<WKV7_F32, false>), grid, block, 0, stream, args);
  }
  return hipGetLastError();
}

}  // namespace wkv7
