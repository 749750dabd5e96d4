// Per-wavefront body of the sequential WKV-7 recurrence: the one source of
// the sequential kernel (k1_seq.hip) and of the decode work items that the
// chunked kernel runs in trailing workgroups of its own launch, so both give
// the same bits. One 64-lane wavefront owns one (sequence, head). Included
// inside an anonymous namespace within namespace wkv7.

#ifndef WKV7_SEQ_WAVE_H
#define WKV7_SEQ_WAVE_H

namespace seqw {

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
// With STREAM the loads carry the non-temporal hint: a call reads each
// input once, and a state that stays in the Infinity Cache (MALL) from one
// step to the next keeps more of it there when the inputs do not claim
// cache lines (measured: the 256-slot decode step 45.8 -> 44.8 us with
// fresh inputs every step; no gain where the state itself streams).
template <int DT> struct In;

typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
template <bool STREAM, typename V>
__device__ __forceinline__ V ld_in(const V* p) {
  if (STREAM) return __builtin_nontemporal_load(p);
  return *p;
}

template <> struct In<WKV7_BF16> {
  typedef uint16_t T;
  struct R4 { uint2 u; };
  struct R16 { uint4 u[2]; };
  template <bool STREAM = false>
  __device__ static R4 ld4(const T* p) {
    const u32x2_t x = ld_in<STREAM>(reinterpret_cast<const u32x2_t*>(p));
    R4 r; r.u = make_uint2(x[0], x[1]); return r;
  }
  template <bool STREAM = false>
  __device__ static R16 ld16(const T* p) {
    R16 r;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const u32x4_t x = ld_in<STREAM>(reinterpret_cast<const u32x4_t*>(p) + q);
      r.u[q] = make_uint4(x[0], x[1], x[2], x[3]);
    }
    return r;
  }
  __device__ static float ld1(const T* p) {
    return __uint_as_float(static_cast<uint32_t>(*p) << 16);
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
  template <bool STREAM = false>
  __device__ static R4 ld4(const T* p) {
    const f32x4_t x = ld_in<STREAM>(reinterpret_cast<const f32x4_t*>(p));
    R4 r; r.u = make_float4(x[0], x[1], x[2], x[3]); return r;
  }
  template <bool STREAM = false>
  __device__ static R16 ld16(const T* p) {
    R16 r;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4_t x = ld_in<STREAM>(reinterpret_cast<const f32x4_t*>(p) + q);
      r.u[q] = make_float4(x[0], x[1], x[2], x[3]);
    }
    return r;
  }
  __device__ static float ld1(const T* p) { return *p; }
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

template <int DT, bool STREAM>
__device__ __forceinline__ void load_token(TokenRaw<DT>& x,
                                           const typename In<DT>::T* const* src,
                                           size_t off, int c, int g) {
  using I = In<DT>;
  x.r = I::template ld4<STREAM>(src[0] + off + 4 * c);
  x.w = I::template ld4<STREAM>(src[1] + off + 4 * c);
  x.k = I::template ld4<STREAM>(src[2] + off + 4 * c);
  x.a = I::template ld4<STREAM>(src[4] + off + 4 * c);
  x.b = I::template ld4<STREAM>(src[5] + off + 4 * c);
  x.v = I::template ld16<STREAM>(src[3] + off + 16 * g);
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

// One state row (row 16 g + m of the lane's group, columns 4 c .. 4 c + 3)
// through one token: the delta-rule sum over the row before this step's
// decay, the update, and the readout of the updated row. Returns `mine`,
// replaced by the row's output in the lane (c == m) that stores row 16 g + c.
__device__ __forceinline__ float row_step(float4& s, const float (&w)[4],
                                          const float (&a)[4],
                                          const float (&b)[4],
                                          const float (&k)[4],
                                          const float (&r)[4], float vm,
                                          int c, int m, float mine) {
  float q = s.x * a[0];
  q = fmaf(s.y, a[1], q);
  q = fmaf(s.z, a[2], q);
  q = fmaf(s.w, a[3], q);
  const float sa = row_sum16(q);
  s.x = fmaf(s.x, w[0], fmaf(sa, b[0], vm * k[0]));
  s.y = fmaf(s.y, w[1], fmaf(sa, b[1], vm * k[1]));
  s.z = fmaf(s.z, w[2], fmaf(sa, b[2], vm * k[2]));
  s.w = fmaf(s.w, w[3], fmaf(sa, b[3], vm * k[3]));
  q = s.x * r[0];
  q = fmaf(s.y, r[1], q);
  q = fmaf(s.z, r[2], q);
  q = fmaf(s.w, r[3], q);
  const float om = row_sum16(q);
  return (c == m) ? om : mine;
}

// The recurrence of work item `it`, head h, on this wavefront (lane = its
// lane id): the state is read from the pool once, every token of the item
// is applied in order with its output written, and the state is written
// back once.
template <int DT, bool NT>
__device__ __forceinline__ void seq_wave(const SeqArgs& p, const WorkItem it,
                                         int h, int lane) {
  using I = In<DT>;
  using T = typename I::T;
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
  load_token<DT, !NT>(nxt, src, off, c, g);   // state cached: inputs streamed
  for (int t = 0; t < it.len; ++t) {
    TokenRaw<DT> cur = nxt;
    if (t + 1 < it.len) load_token<DT, !NT>(nxt, src, off + tstride, c, g);
    float w[4], a[4], b[4], k[4], r[4], v[16];
    I::cvt4(cur.w, w); I::cvt4(cur.a, a); I::cvt4(cur.b, b);
    I::cvt4(cur.k, k); I::cvt4(cur.r, r); I::cvt16(cur.v, v);

    // Row by row: the delta-rule sum over the row before this step's
    // decay, the update, the readout of the updated row. Rows are
    // independent, so this order gives the same bits as summing every row
    // first; it keeps fewer values live (139 VGPRs for bf16 inputs against
    // 169 with all 16 sums and outputs held, three wavefronts per SIMD).
    float mine = 0.f;
#pragma unroll
    for (int m = 0; m < 16; ++m)
      mine = row_step(s[m], w, a, b, k, r, v[m], c, m, mine);
    p.o[off + 16 * g + c] = mine;
    off += tstride;
  }

#pragma unroll
  for (int m = 0; m < 16; ++m) store_state<NT>(sbase + m * kN, s[m]);
}

// Lane m's value to every lane of its row of 16 (DPP row_newbcast).
template <int M>
__device__ __forceinline__ float row_bcast_t(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      0, __builtin_bit_cast(int, x), 0x150 + M, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_bcast(float x, int m) {
  switch (m) {   // m is a constant once the caller's loop is unrolled
    case 0: return row_bcast_t<0>(x);   case 1: return row_bcast_t<1>(x);
    case 2: return row_bcast_t<2>(x);   case 3: return row_bcast_t<3>(x);
    case 4: return row_bcast_t<4>(x);   case 5: return row_bcast_t<5>(x);
    case 6: return row_bcast_t<6>(x);   case 7: return row_bcast_t<7>(x);
    case 8: return row_bcast_t<8>(x);   case 9: return row_bcast_t<9>(x);
    case 10: return row_bcast_t<10>(x); case 11: return row_bcast_t<11>(x);
    case 12: return row_bcast_t<12>(x); case 13: return row_bcast_t<13>(x);
    case 14: return row_bcast_t<14>(x); default: return row_bcast_t<15>(x);
  }
}

// A one-token work item (decode) whose state streams from HBM: the same
// row steps as seq_wave, with lane 16 g + c owning rows 4 m + g (m < 16),
// so each state access of the wavefront covers four consecutive rows (1 KB
// contiguous); the inputs are requested first and the state rows after
// them, and row m is computed as soon as it has arrived and stored at once
// while later rows are still in flight. Lane 16 g + c loads v[4 c + g]; row
// 4 m + g takes v from lane m of its row of 16. Each row's arithmetic is
// seq_wave's, so the results are the same bits.
template <int DT, bool NT>
__device__ __forceinline__ void seq1_wave(const SeqArgs& p, const WorkItem it,
                                          int h, int lane) {
  using I = In<DT>;
  using T = typename I::T;
  const int g = lane >> 4;
  const int c = lane & 15;
  const T* src[6] = {static_cast<const T*>(p.r), static_cast<const T*>(p.w),
                     static_cast<const T*>(p.k), static_cast<const T*>(p.v),
                     static_cast<const T*>(p.a), static_cast<const T*>(p.b)};
  const size_t off = (static_cast<size_t>(it.tok0) * p.H + h) * kN;
  const typename I::R4 rr = I::ld4(src[0] + off + 4 * c);
  const typename I::R4 ww = I::ld4(src[1] + off + 4 * c);
  const typename I::R4 kk = I::ld4(src[2] + off + 4 * c);
  const typename I::R4 aa = I::ld4(src[4] + off + 4 * c);
  const typename I::R4 bb = I::ld4(src[5] + off + 4 * c);
  const float vmine = I::ld1(src[3] + off + 4 * c + g);
  float* sbase = p.pool + (static_cast<size_t>(it.slot) * p.H + h) * (kN * kN)
                 + g * kN + 4 * c;
  // every load is issued before the first use and in row order (the
  // scheduler would otherwise hold later rows back behind the stores, or
  // reorder them so that the first rows' waits cover later loads too)
  float4 s[16];
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    s[m] = load_state<NT>(sbase + 4 * m * kN);
    __builtin_amdgcn_sched_barrier(0);
  }
  float w[4], a[4], b[4], k[4], r[4];
  I::cvt4(ww, w); I::cvt4(aa, a); I::cvt4(bb, b);
  I::cvt4(kk, k); I::cvt4(rr, r);
  float mine = 0.f;
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    mine = row_step(s[m], w, a, b, k, r, row_bcast(vmine, m), c, m, mine);
    store_state<NT>(sbase + 4 * m * kN, s[m]);
  }
  // lane c of group g holds the output of row 4 c + g
  p.o[off + 4 * c + g] = mine;
}

}  // namespace seqw

#endif  // WKV7_SEQ_WAVE_H
