// Pipelined chunked-prefill WKV-7 kernel on gfx950.
//
// Same operation as the other kernels (page "RWKV-X Architecture", section
// "WKV-7 Kernel (Generalized Delta Rule)", product-form reading
// S_t = S_{t-1}(diag(w_t) + a_t b_t^T) + v_t k_t^T, o_t = S_t r_t), in the
// chunked (WY/UT) form with chunks of L = 32 tokens. Per chunk, with
// Lambda_t = prod_{u<=t} w_u and suf_t = prod_{u>t} w_u per key channel,
//   Abar_t = a_t Lambda_{t-1}, Rbar_t = r_t Lambda_t,
//   Bbar_s = b_s suf_s,        Kbar_s = k_s suf_s,
//   A_ab = strict_lower(<Abar_t / Lambda_L, Bbar_s>), A_ak likewise with Kbar,
//   M_rb = lower(<Rbar_t / Lambda_L, Bbar_s>),        M_rk likewise with Kbar,
//   T = (I - A_ab)^-1,
//   X = Abar S0^T + A_ak V,  U = T X,
//   O = Rbar S0^T + M_rb U + M_rk V,
//   S_L = Lambda_L S0 + U^T Bbar + V^T Kbar.
// Every Gram term <., .> is the exact decay between s and t (<= 1) times
// the inputs; only the operands Abar / Lambda_L, Rbar / Lambda_L are large.
//
// Organisation: one 768-thread workgroup (12 wavefronts, three per SIMD:
// wavefront w runs on SIMD w mod 4) per (sequence, head), as a two-stage
// pipeline over chunks. In step c the key side builds chunk c while the
// value side runs chunk c - 1:
//   * t wavefronts 0-3 build the operands made from r and a, then (after
//     the mid-step barrier) t wavefront W computes Gram matrix W;
//   * s wavefronts 4-7 build the operands made from k, b and v and prepare
//     the next chunk's decay products;
//   * value wavefronts 8-11: wavefront 8 + w owns state rows
//     i in [16 w, 16 w + 16), kept in registers as MFMA accumulator tiles of
//     S^T; value wavefronts 0 and 1 also form T from A_ab.
// Two workgroup barriers per step (mid-step and end); the fallback flags of
// a chunk travel with the end-of-step barrier (a ballot per wavefront,
// posted to LDS).
//
// Precision, two plans (template parameter PRE):
//   * fast (bf16 inputs): Gram products from split bf16 (hi + lo) operands,
//     three MFMAs with fp32 accumulation; T from fp16 A_ab by products on
//     the matrix cores; every value-side product with single fp16 operands,
//     the state, X and U scaled by powers of two (exact) before conversion.
//     About 3e-3 of max|err|/rms against the float64 oracle on the
//     workloads' inputs (bf16 bar: 2e-2).
//   * precise (fp32 inputs, or bf16 inputs on request): the same Gram
//     products and T; every value-side product from split bf16 operands as
//     well (three MFMAs), no scaling. About 1e-4 (fp32 bar: 1e-3).
// A chunk whose Lambda_L falls below 2^-100 in some channel, whose inputs
// reach 2^15, or whose Gram matrices or T leave the fp16 range runs token by
// token on the value wavefronts instead (exact for any w in (0, 1]).
//
// MFMA fragments (verified lane layout of v_mfma_f32_16x16x32_{bf16,f16}
// and 16x16x16): lane l = 16 g + n holds operand row n and, for a 32-wide k
// range at kb, k = kb + {4g..4g+3, 16+4g..16+4g+3}; the result lane holds
// C[4g + r][n]. With this k order two 16-row result tiles form the operand
// fragment of the next product in registers.

#include "internal.h"
#include "../../include/wkv7.h"

namespace wkv7 {
namespace {

#include "seq_wave.h"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
// The state pointers of segment items come from memory; accessed as plain
// pointers they would compile to flat instructions, which also count
// against the LDS wait counter.
typedef __attribute__((address_space(1))) f32x4 gf32x4;

constexpr int kL = 32;                   // chunk length
constexpr int kP64 = 68;                 // pitch of 64-wide rows (elements)
constexpr int kP32 = 36;                 // pitch of 32-wide rows (elements)
constexpr int kM64 = kL * kP64;          // [32][64] matrix, elements
constexpr int kM32 = kL * kP32;          // [32][32] matrix
constexpr int kMT = 64 * kP32;           // [64][32] matrix

// LDS map (bytes). The value side's operands (VO: Abar, Rbar [32][64],
// Bbar^T, Kbar^T, V^T [64][32]; LL: A_ak, M_rb, M_rk [32][32]) are single
// fp16 matrices in the fast plan and split bf16 pairs (hi matrix, lo matrix
// after it) in the precise plan; everything else is common.
template <bool PRE> struct Map {
  static constexpr int kVO = PRE ? 2 : 1;                  // matrices per operand
  static constexpr int GR = 0;                             // 4 pairs [32][64]
  static constexpr int AB = GR + 4 * 2 * kM64 * 2;         // fp16 A_ab, A_ab^T
  static constexpr int TOT = AB + 2 * kM32 * 2;            // fp32 [8][64]
  static constexpr int VOBytes = kVO * (2 * kM64 + 3 * kMT) * 2;  // per buffer
  static constexpr int VO = TOT + 8 * 64 * 4;              // 2 buffers
  static constexpr int LLBytes = kVO * 3 * kM32 * 2;
  static constexpr int LL = VO + 2 * VOBytes;              // 2 buffers
  static constexpr int LAM = LL + 2 * LLBytes;             // fp32 [2][64]
  static constexpr int TT = LAM + 2 * 64 * 4;              // fp16 T [32][32]
  static constexpr int YC = TT + kM32 * 2;                 // fp16x4 [64]: col(Y)
  static constexpr int D1R = YC + 64 * 8;                  // fp16x4 [64]: row(D_1)
  static constexpr int TFL = D1R + 64 * 8;                 // u32 [2]: D_0, D_1 range
  static constexpr int FLG = TFL + 2 * 4;                  // u32 [16]
  static constexpr int Bytes = FLG + 16 * 4;
  static_assert(Bytes <= 160 * 1024, "LDS budget");
  // element offsets of the operands within a VO / LL buffer
  static constexpr int Abar = 0, Rbar = kVO * kM64, BbT = 2 * kVO * kM64,
                       KbT = BbT + kVO * kMT, Vt = KbT + kVO * kMT;
  static constexpr int Aak = 0, Mrb = kVO * kM32, Mrk = 2 * kVO * kM32;
};
// element type of the value side's LDS operands
template <bool PRE> struct VOElem { typedef _Float16 T; };
template <> struct VOElem<true> { typedef __bf16 T; };

constexpr float kHalfSafe = 32768.f;            // fp16 operand bound
constexpr float kMinLamL = 7.88860905e-31f;     // 2^-100

template <int V> struct IntC { static constexpr int value = V; };

struct F8 { bf16x8 h, l; };
struct F4 { bf16x4 h, l; };

__device__ __forceinline__ void split(float x, __bf16& h, __bf16& l) {
  h = static_cast<__bf16>(x);
  l = static_cast<__bf16>(x - static_cast<float>(h));
}
__device__ __forceinline__ f32x4 mmab(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mmab16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mmah(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mm3(const F8& p, const F8& q, f32x4 c) {
  c = mmab(p.l, q.h, c);
  c = mmab(p.h, q.l, c);
  return mmab(p.h, q.h, c);
}
__device__ __forceinline__ f32x4 mm3(const F4& p, const F4& q, f32x4 c) {
  c = mmab16(p.l, q.h, c);
  c = mmab16(p.h, q.l, c);
  return mmab16(p.h, q.h, c);
}

template <typename V8, typename V4, typename E>
__device__ __forceinline__ V8 ld8(const E* m, int pitch, int row, int kb,
                                  int g) {
  const E* p = m + row * pitch + kb + 4 * g;
  V4 a = *reinterpret_cast<const V4*>(p);
  V4 b = *reinterpret_cast<const V4*>(p + 16);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
// split-bf16 pair fragment; the lo matrix follows the hi matrix at +mat
__device__ __forceinline__ F8 ldp8(const __bf16* pair, int mat, int pitch,
                                   int row, int kb, int g) {
  return F8{ld8<bf16x8, bf16x4>(pair, pitch, row, kb, g),
            ld8<bf16x8, bf16x4>(pair + mat, pitch, row, kb, g)};
}
__device__ __forceinline__ F4 ldp4(const __bf16* pair, int mat, int pitch,
                                   int row, int kb, int g) {
  const int o = row * pitch + kb + 4 * g;
  return F4{*reinterpret_cast<const bf16x4*>(pair + o),
            *reinterpret_cast<const bf16x4*>(pair + mat + o)};
}
__device__ __forceinline__ f16x8 ldh8(const _Float16* m, int pitch, int row,
                                      int kb, int g) {
  return ld8<f16x8, f16x4>(m, pitch, row, kb, g);
}
__device__ __forceinline__ F4 frag4(f32x4 t) {
  F4 f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    __bf16 h, l;
    split(t[r], h, l); f.h[r] = h; f.l[r] = l;
  }
  return f;
}
__device__ __forceinline__ f16x8 frag8h(f32x4 t0, f32x4 t1, float s) {
  f16x8 f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    f[r] = static_cast<_Float16>(t0[r] * s);
    f[4 + r] = static_cast<_Float16>(t1[r] * s);
  }
  return f;
}
__device__ __forceinline__ float bf_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// Products of the per-group decay totals g[q] of row groups q < 2 W and
// q > 2 W + 1 (two channels), for the key wavefront W.
template <int W>
__device__ __forceinline__ void outer_products(const float (&g0)[8], const float (&g1)[8],
                                               float& lo0, float& lo1, float& hi0,
                                               float& hi1) {
  lo0 = lo1 = hi0 = hi1 = 1.f;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    if (q < 2 * W) { lo0 *= g0[q]; lo1 *= g1[q]; }
    if (q > 2 * W + 1) { hi0 *= g0[q]; hi1 *= g1[q]; }
  }
}

// Two channels at once: one packed conversion for the high parts, the
// residuals from the packed bits (exact), one packed conversion for them.
// The same values as split() per channel.
__device__ __forceinline__ void split2(float x0, float x1, bf16x2& h, bf16x2& l) {
  h = __builtin_convertvector(f32x2{x0, x1}, bf16x2);
  const uint32_t hb = __builtin_bit_cast(uint32_t, h);
  const float h0 = __uint_as_float(hb << 16);
  const float h1 = __uint_as_float(hb & 0xffff0000u);
  l = __builtin_convertvector(f32x2{x0 - h0, x1 - h1}, bf16x2);
}
__device__ __forceinline__ void put2p(__bf16* pair, int mat, int pitch,
                                      int row, int col, float x0, float x1) {
  bf16x2 h, l;
  split2(x0, x1, h, l);
  *reinterpret_cast<bf16x2*>(pair + row * pitch + col) = h;
  *reinterpret_cast<bf16x2*>(pair + mat + row * pitch + col) = l;
}
// four consecutive elements of a pair-matrix row, split
__device__ __forceinline__ void put4p(__bf16* pair, int mat, int pitch,
                                      int row, int col, f32x4 x) {
  bf16x2 h0, l0, h1, l1;
  split2(x[0], x[1], h0, l0);
  split2(x[2], x[3], h1, l1);
  *reinterpret_cast<bf16x4*>(pair + row * pitch + col) =
      __builtin_shufflevector(h0, h1, 0, 1, 2, 3);
  *reinterpret_cast<bf16x4*>(pair + mat + row * pitch + col) =
      __builtin_shufflevector(l0, l1, 0, 1, 2, 3);
}
// operand fragment of two result tiles (k = 4g + r, then 16 + 4g + r), split
__device__ __forceinline__ F8 frag8p(f32x4 t0, f32x4 t1) {
  bf16x2 h[4], l[4];
  split2(t0[0], t0[1], h[0], l[0]);
  split2(t0[2], t0[3], h[1], l[1]);
  split2(t1[0], t1[1], h[2], l[2]);
  split2(t1[2], t1[3], h[3], l[3]);
  F8 f;
  f.h = __builtin_shufflevector(__builtin_shufflevector(h[0], h[1], 0, 1, 2, 3),
                                __builtin_shufflevector(h[2], h[3], 0, 1, 2, 3),
                                0, 1, 2, 3, 4, 5, 6, 7);
  f.l = __builtin_shufflevector(__builtin_shufflevector(l[0], l[1], 0, 1, 2, 3),
                                __builtin_shufflevector(l[2], l[3], 0, 1, 2, 3),
                                0, 1, 2, 3, 4, 5, 6, 7);
  return f;
}
// fp16 values as split bf16 pairs: exact (11 significant bits = 8 + 3)
__device__ __forceinline__ F8 split_f16(f16x8 x) {
  f32x4 a, b;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    a[r] = static_cast<float>(x[r]);
    b[r] = static_cast<float>(x[4 + r]);
  }
  return frag8p(a, b);
}
__device__ __forceinline__ void put2h(_Float16* m, int pitch, int row, int col,
                                      float x0, float x1) {
  f16x2 v = {static_cast<_Float16>(x0), static_cast<_Float16>(x1)};
  *reinterpret_cast<f16x2*>(m + row * pitch + col) = v;
}
__device__ __forceinline__ void put4h(_Float16* m, int pitch, int row, int col,
                                      f32x4 x) {
  f16x4 v;
#pragma unroll
  for (int r = 0; r < 4; ++r) v[r] = static_cast<_Float16>(x[r]);
  *reinterpret_cast<f16x4*>(m + row * pitch + col) = v;
}

// Maxima of non-negative floats as unsigned bit patterns: the same order,
// and a NaN (any sign cleared) sorts above +Inf, so it is never dropped.
__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint32_t dpp_umax16(uint32_t x) {
  x = umax(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0xB1, 0xF, 0xF, false)));
  x = umax(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x4E, 0xF, 0xF, false)));
  x = umax(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x141, 0xF, 0xF, false)));
  x = umax(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x140, 0xF, 0xF, false)));
  return x;
}
// max over the wavefront of x >= 0 (or NaN): rows of 16 by DPP (every lane
// of a row then holds the row's maximum), then the four rows through scalar
// registers (no LDS round trip). The result is wavefront-uniform.
// max(m, |x_r|) as floats, for the power-of-two scale of an operand: one
// max3 with |x| source modifiers per two values, no sign masking. A NaN
// among the x_r is skipped (its row stays NaN after scaling); an infinity
// makes the scale 1, as in pow2_scale.
__device__ __forceinline__ float scale_max4(f32x4 x, float m) {
#pragma unroll
  for (int r = 0; r < 4; ++r) m = fmaxf(m, fabsf(x[r]));
  return m;
}
__device__ __forceinline__ float wave_max(float x) {
  const uint32_t u = dpp_umax16(__float_as_uint(x));
  const uint32_t r0 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(u), 0));
  const uint32_t r1 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(u), 16));
  const uint32_t r2 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(u), 32));
  const uint32_t r3 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(u), 48));
  return __uint_as_float(umax(umax(r0, r1), umax(r2, r3)));
}
// power of two s with max|x s| < 2^14 for max|x| = m (1 if m is 0 or not
// finite); 1/s in *inv
__device__ __forceinline__ float pow2_scale(float m, float* inv) {
  const uint32_t bits = __float_as_uint(m);
  const int e = static_cast<int>((bits >> 23) & 0xffu) - 127;
  if (!(m > 0.f) || e > 126 || e < -100) { *inv = 1.f; return 1.f; }
  const int k = 13 - e;
  *inv = __uint_as_float(static_cast<uint32_t>(127 - k) << 23);
  return __uint_as_float(static_cast<uint32_t>(127 + k) << 23);
}
// max(m, |x_r|) on bit patterns (NaN propagates, see umax)
__device__ __forceinline__ float abs_max4(f32x4 x, float m) {
  uint32_t u = __float_as_uint(m);
#pragma unroll
  for (int r = 0; r < 4; ++r) u = umax(u, __float_as_uint(x[r]) & 0x7fffffffu);
  return __uint_as_float(u);
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
// per-half max of |bf16| bit patterns (sign cleared; NaN/Inf sort highest)
// over n words, as a tree of depth log2(n): the masked words are
// independent
template <int n>
__device__ __forceinline__ uint32_t absmax_tree(const uint32_t* x) {
  uint32_t m[n];
#pragma unroll
  for (int u = 0; u < n; ++u) m[u] = x[u] & 0x7fff7fffu;
#pragma unroll
  for (int w = 1; w < n; w *= 2)
#pragma unroll
    for (int u = 0; u + w < n; u += 2 * w)
      m[u] = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(
          __builtin_bit_cast(u16x2, m[u]), __builtin_bit_cast(u16x2, m[u + w])));
  return m[0];
}
// true if either half of a per-half max of bf16 bit patterns is >= limit
__device__ __forceinline__ bool any_half_ge(uint32_t m, uint32_t limit) {
  return ((m & 0xffffu) >= limit) | ((m >> 16) >= limit);
}

// max of |x| over n pairs of floats, as bit patterns (sign cleared; NaN and
// Inf sort highest), a tree of depth log2(2 n)
template <int n>
__device__ __forceinline__ uint32_t absmax_tree(const u32x2* x) {
  uint32_t m[n];
#pragma unroll
  for (int u = 0; u < n; ++u) m[u] = umax(x[u][0] & 0x7fffffffu, x[u][1] & 0x7fffffffu);
#pragma unroll
  for (int w = 1; w < n; w *= 2)
#pragma unroll
    for (int u = 0; u + w < n; u += 2 * w) m[u] = umax(m[u], m[u + w]);
  return m[0];
}

// Raw inputs of a key thread: for each of its rows, the bits of channels
// 2 jp and 2 jp + 1, a bf16 pair (bf16 inputs) or two floats (fp32 inputs).
template <int DT> struct Raw;
template <> struct Raw<WKV7_BF16> {
  typedef uint32_t W;
  static constexpr int kElem = 2;                       // bytes per element
  __device__ static float c0(W x) { return bf_lo(x); }
  __device__ static float c1(W x) { return bf_hi(x); }
  __device__ static W zero() { return 0u; }
  __device__ static W one() { return 0x3f803f80u; }
  __device__ static W load(__amdgpu_buffer_rsrc_t rs, int voff) {
    return __builtin_amdgcn_raw_buffer_load_b32(rs, voff, 0, 0);
  }
  // some |x| >= 2^15 (or NaN/Inf)
  template <int n> __device__ static bool big(const W (&x)[n]) {
    return any_half_ge(absmax_tree<n>(x), 0x4700u);
  }
  // some |x| > 1 (or NaN)
  template <int n> __device__ static bool above_one(const W (&x)[n]) {
    return any_half_ge(absmax_tree<n>(x), 0x3f81u);
  }
};
template <> struct Raw<WKV7_F32> {
  typedef u32x2 W;
  static constexpr int kElem = 4;
  __device__ static float c0(W x) { return __uint_as_float(x[0]); }
  __device__ static float c1(W x) { return __uint_as_float(x[1]); }
  __device__ static W zero() { return W{0u, 0u}; }
  __device__ static W one() { return W{0x3f800000u, 0x3f800000u}; }
  __device__ static W load(__amdgpu_buffer_rsrc_t rs, int voff) {
    return __builtin_amdgcn_raw_buffer_load_b64(rs, voff, 0, 0);
  }
  template <int n> __device__ static bool big(const W (&x)[n]) {
    return absmax_tree<n>(x) >= 0x47000000u;
  }
  template <int n> __device__ static bool above_one(const W (&x)[n]) {
    return absmax_tree<n>(x) > 0x3f800000u;
  }
};

// rows 4 rg + e (e < 4): a t wavefront holds r, a and w, an s wavefront k,
// b, v and w
template <int DT> struct RawT { static constexpr int kDT = DT; typename Raw<DT>::W r[4], a[4], w[4]; };
template <int DT> struct RawS { static constexpr int kDT = DT; typename Raw<DT>::W k[4], b[4], v[4], w[4]; };

// Loads through buffer resources based at the chunk's first row and sized
// to its n rows, with a 32-bit lane offset and no branch: a row past the
// chunk's end lies outside the resource, and the buffer load returns zero
// for it without touching memory. Zero is the padding of every input but
// w, whose padding (1) the caller sets (pad_raw) when it consumes the
// rows, so nothing waits on the loads here.
template <int DT, int NA>
__device__ __forceinline__ void load_rows(typename Raw<DT>::W (*const dst[NA])[4],
                                          const void* const src[NA],
                                          const SeqArgs& p, int t0, int n,
                                          int h, int rg, int jp) {
  constexpr int es = Raw<DT>::kElem;
  const size_t row0 = (static_cast<size_t>(t0) * p.H + h) * (kN * es);  // bytes
  const uint32_t rowb = static_cast<uint32_t>(p.H) * (kN * es);
  const int bytes = static_cast<int>(static_cast<uint32_t>(n) * rowb);
  __amdgpu_buffer_rsrc_t rs[NA];
#pragma unroll
  for (int u = 0; u < NA; ++u)
    rs[u] = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(static_cast<const char*>(src[u]) + row0), 0, bytes,
        0x00020000);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int voff = static_cast<int>(
        static_cast<uint32_t>(4 * rg + e) * rowb + 2 * es * jp);
#pragma unroll
    for (int u = 0; u < NA; ++u) (*dst[u])[e] = Raw<DT>::load(rs[u], voff);
  }
}
template <int DT>
__device__ __forceinline__ void load_raw(RawT<DT>& x, const SeqArgs& p, int t0,
                                         int n, int h, int rg, int jp) {
  typename Raw<DT>::W (*const dst[3])[4] = {&x.r, &x.a, &x.w};
  const void* const src[3] = {p.r, p.a, p.w};
  load_rows<DT, 3>(dst, src, p, t0, n, h, rg, jp);
}
// rows 4 rg + e >= n become padding: w = 1, everything else 0 (the loads
// returned zero for them), which leaves the state unchanged
template <typename X>
__device__ __forceinline__ void pad_raw(X& x, int n, int rg) {
  typedef Raw<X::kDT> R;
#pragma unroll
  for (int e = 0; e < 4; ++e) x.w[e] = 4 * rg + e >= n ? R::one() : x.w[e];
}

// ---- T = (I - A_ab)^-1 from fp16 fragments (value wavefronts 0 and 1) ----
// A 16x16 matrix M is held as two fp16 operand fragments and their fp32
// values:
//   row(M): lane (g, n) holds M[n][4g + e]   (left operand of a product)
//   col(M): lane (g, n) holds M[4g + e][n]   (right operand; also the
//                                             result layout of a product)
// so L*R gives col(LR) = mfma(row(L), col(R)) and row(LR) = col((LR)^T) =
// mfma(col(R), row(L)): every product yields both fragments of its result.
// T is kept in fp16 (the precise plan splits its fp16 values exactly into
// bf16 pairs), so fp16 operands with fp32 accumulation suffice.
struct Frag { f16x4 row, col; f32x4 frow, fcol; };

__device__ __forceinline__ f32x4 mmh16(f16x4 a, f16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f16x4 h4(f32x4 x) {
  f16x4 h;
#pragma unroll
  for (int r = 0; r < 4; ++r) h[r] = static_cast<_Float16>(x[r]);
  return h;
}
__device__ __forceinline__ Frag frag_of(f32x4 frow, f32x4 fcol) {
  return Frag{h4(frow), h4(fcol), frow, fcol};
}
__device__ __forceinline__ Frag product(const Frag& L, const Frag& R) {
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  return frag_of(mmh16(R.col, L.row, z), mmh16(L.row, R.col, z));
}
// P + P*N
__device__ __forceinline__ Frag product_add(const Frag& P, const Frag& N) {
  return frag_of(mmh16(N.col, P.row, P.frow), mmh16(P.row, N.col, P.fcol));
}
__device__ __forceinline__ f32x4 f32_of(f16x4 h) {
  f32x4 x;
#pragma unroll
  for (int r = 0; r < 4; ++r) x[r] = static_cast<float>(h[r]);
  return x;
}
// D = (I - A)^-1 = (I + A)(I + A^2)(I + A^4)(I + A^8) for strictly lower
// 16x16 A (A^16 = 0)
__device__ __forceinline__ Frag inverse_unit_lower(f16x4 arow, f16x4 acol,
                                                   int g, int n16) {
  Frag N{arow, acol, f32_of(arow), f32_of(acol)};
  f32x4 prow = N.frow, pcol = N.fcol;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (4 * g + r == n16) { prow[r] += 1.f; pcol[r] += 1.f; }
  }
  Frag P = frag_of(prow, pcol);
#pragma unroll
  for (int it = 0; it < 3; ++it) {
    N = product(N, N);
    P = product_add(P, N);
  }
  return P;
}
__device__ __forceinline__ f16x4 ldh4(const _Float16* m, int pitch, int row,
                                      int col) {
  return *reinterpret_cast<const f16x4*>(m + row * pitch + col);
}

// Workgroup OR of two flag bits with one barrier: lane 0 of every wave
// posts its wave's bits; all threads read the twelve posts after the
// barrier.
__device__ __forceinline__ uint32_t barrier_or2(uint32_t* slot, int wv,
                                                int lane, bool b0, bool b1) {
  const uint32_t m0 = __builtin_amdgcn_ballot_w64(b0) != 0 ? 1u : 0u;
  const uint32_t m1 = __builtin_amdgcn_ballot_w64(b1) != 0 ? 2u : 0u;
  if (lane == 0) slot[wv] = m0 | m1;
  __syncthreads();
  uint32_t r = 0;
#pragma unroll
  for (int w = 0; w < kChunkPWaves; ++w) r |= slot[w];
  return r;
}

// one input element as float
__device__ __forceinline__ float in_elem(const void* p, size_t i, IntC<WKV7_BF16>) {
  return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(p)[i]) << 16);
}
__device__ __forceinline__ float in_elem(const void* p, size_t i, IntC<WKV7_F32>) {
  return static_cast<const float*>(p)[i];
}

// Exact token-by-token recurrence for one chunk on a value wavefront (rows
// i = 16 vb + n16 of the state, held as S[jt][r] = S[i][16 jt + 4 g + r]).
template <int DT>
__device__ __forceinline__ void exact_chunk(const SeqArgs& p, f32x4* S, int t0,
                                         int n, int h, int vb, int g,
                                         int n16, bool zero_v, bool no_out) {
  const IntC<DT> dt;
  const int i = 16 * vb + n16;
  for (int t = 0; t < n; ++t) {
    const size_t base = (static_cast<size_t>(t0 + t) * p.H + h) * kN;
    float rr[16], ww[16], kk[16], aa[16], bb[16];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const size_t o = base + 16 * jt + 4 * g + r;
        rr[4 * jt + r] = in_elem(p.r, o, dt);
        ww[4 * jt + r] = in_elem(p.w, o, dt);
        kk[4 * jt + r] = in_elem(p.k, o, dt);
        aa[4 * jt + r] = in_elem(p.a, o, dt);
        bb[4 * jt + r] = in_elem(p.b, o, dt);
      }
    }
    const float vi = zero_v ? 0.f : in_elem(p.v, base + i, dt);
    float sa = 0.f;
#pragma unroll
    for (int jt = 0; jt < 4; ++jt)
#pragma unroll
      for (int r = 0; r < 4; ++r) sa = fmaf(S[jt][r], aa[4 * jt + r], sa);
    sa += __shfl_xor(sa, 16);
    sa += __shfl_xor(sa, 32);
    float o = 0.f;
#pragma unroll
    for (int jt = 0; jt < 4; ++jt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        S[jt][r] = fmaf(S[jt][r], ww[4 * jt + r],
                        fmaf(sa, bb[4 * jt + r], vi * kk[4 * jt + r]));
        o = fmaf(S[jt][r], rr[4 * jt + r], o);
      }
    o += __shfl_xor(o, 16);
    o += __shfl_xor(o, 32);
    if (g == 0 && !no_out) p.o[base + i] = o;
  }
}

// SEG = false: items are pool slots (p.items); true: segments (segs) with
// their own state buffers and flags.
// Workgroups past the (item, head) grid run the decode work items `dec` of
// the same call, twelve (item, head) pairs per workgroup, one per
// wavefront, with the sequential recurrence (the same bits as the
// sequential kernel): a batch's decode tokens then fill CUs that its
// prefills leave idle, in the same launch.
// DT: input type (WKV7_BF16 or WKV7_F32); PRE: the precise plan.
template <bool SEG, int DT, bool PRE>
__global__ __launch_bounds__(64 * kChunkPWaves, 1)
void chunk_p_kernel(SeqArgs p, const SegItem* segs, const WorkItem* dec,
                    int32_t n_dec) {
  typedef Raw<DT> R;
  typedef Map<PRE> M;
  typedef typename VOElem<PRE>::T VE;
  __shared__ __attribute__((aligned(16))) unsigned char lds[M::Bytes];
  __bf16* GR = reinterpret_cast<__bf16*>(lds + M::GR);
  __bf16* Ahat = GR;                       // pair [t][j]
  __bf16* Rhat = GR + 2 * kM64;            // pair [t][j]
  __bf16* Bbar = GR + 4 * kM64;            // pair [s][j]
  __bf16* Kbar = GR + 6 * kM64;            // pair [s][j]
  // fast plan: A_ab [t][s], then [s][t]; precise plan: T [t][s] of chunks
  // of even and odd index
  _Float16* AB = reinterpret_cast<_Float16*>(lds + M::AB);
  float* TOT = reinterpret_cast<float*>(lds + M::TOT);
  float* LAMb = reinterpret_cast<float*>(lds + M::LAM);
  uint32_t* FLG = reinterpret_cast<uint32_t*>(lds + M::FLG);
  _Float16* TT = reinterpret_cast<_Float16*>(lds + M::TT);       // T [t][s]
  _Float16* YC = reinterpret_cast<_Float16*>(lds + M::YC);
  _Float16* D1R = reinterpret_cast<_Float16*>(lds + M::D1R);
  uint32_t* TFL = reinterpret_cast<uint32_t*>(lds + M::TFL);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t n_main = static_cast<int64_t>(p.n_items) * p.H;
  if (static_cast<int64_t>(blockIdx.x) >= n_main) {
    const int64_t q = (static_cast<int64_t>(blockIdx.x) - n_main) * kChunkPWaves + wv;
    const int di = static_cast<int>(q / p.H);
    const int dh = static_cast<int>(q - static_cast<int64_t>(di) * p.H);
    if (di < n_dec) seqw::seq_wave<DT, false>(p, dec[di], dh, lane);
    return;
  }
  // roles: t wavefronts 0-3, s wavefronts 4-7, value wavefronts 8-11
  const int role = wv >> 2;
  const int g = lane >> 4;
  const int n16 = lane & 15;
  const int item = blockIdx.x / p.H;
  const int h = blockIdx.x - item * p.H;
  if (item >= p.n_items) return;
  int32_t tok0, len, flags = 0;
  const float* s_in;
  float* s_out;
  if (SEG) {
    const SegItem it = segs[item];
    tok0 = it.tok0;
    len = it.len;
    flags = it.flags;
    s_in = it.s_in ? it.s_in + static_cast<size_t>(h) * (kN * kN) : nullptr;
    s_out = it.s_out ? it.s_out + static_cast<size_t>(h) * (kN * kN) : nullptr;
  } else {
    const WorkItem it = p.items[item];
    tok0 = it.tok0;
    len = it.len;
    s_out = p.pool + (static_cast<size_t>(it.slot) * p.H + h) * (kN * kN);
    s_in = s_out;
  }
  // Every item holds at least one token (the host drops empty sequences,
  // and segments are never empty).
  if (len <= 0) return;
  const bool zero_v = (flags & kSegZeroV) != 0;
  const bool no_out = (flags & kSegNoOut) != 0;
  const int nch = (len + kL - 1) / kL;
  const size_t rowstride = static_cast<size_t>(p.H) * kN;

  // key-thread ownership (t and s wavefronts alike): channel pair jp, rows
  // 4 rg .. 4 rg + 3
  const int jp = lane & 31;
  const int j0 = 2 * jp;
  const int rg = 2 * (wv & 3) + (lane >> 5);
  // value-wavefront ownership: state rows i in [16 vb, 16 vb + 16)
  const int vb = wv & 3;
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};

  // Key side, split over two roles that own the same rows and channels:
  // the t wavefronts build the operands made from r and a (and then the
  // Gram matrices and T), the s wavefronts those made from k, b and v and
  // the chunk's decay totals. A chunk's raw inputs are loaded right after
  // the operands of the chunk before have been built from the same
  // registers, and prepared one step before their operands are built
  // (padded; running products of w over the thread's 4 rows in P0/P1; the
  // s wavefronts post the rows' totals in TOT), in the previous step's
  // second interval. The end-of-step barrier orders the TOT writes before
  // their reads. Each loop is instantiated once per wavefront W (= wv & 3): its
  // row groups, Gram matrix and LDS destinations are then constants.
  // The next chunk's loads and preparation happen on every path, with the
  // chunk index clamped to the last one (whose totals no step then reads):
  // a load under a branch leaves the raw registers to be merged at its
  // end, and the copies that merge them wait for the loads.
  auto load_next = [&](auto& x, int c) {
    const int cl = min(c + 1, nch - 1);
    load_raw(x, p, tok0 + cl * kL, min(kL, len - cl * kL), h, rg, jp);
  };
  float w0[4], w1[4], P0[4], P1[4];
  auto decays = [&](const typename R::W (&wr)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) { w0[e] = R::c0(wr[e]); w1[e] = R::c1(wr[e]); }
    P0[0] = w0[0]; P1[0] = w1[0];
#pragma unroll
    for (int e = 1; e < 4; ++e) { P0[e] = P0[e - 1] * w0[e]; P1[e] = P1[e - 1] * w1[e]; }
  };
  // Decay over the row groups before the thread's group (pre), after it
  // (suf) and over the whole chunk (lam), from the group totals in TOT. A
  // wavefront's two groups are 2 W and 2 W + 1, so the products outside
  // them have wavefront-uniform bounds.
  struct Dec { float pre0, pre1, suf0, suf1, lam0, lam1; };
  auto chunk_decays = [&](auto Wc) {
    constexpr int W = decltype(Wc)::value;
    float g0[8], g1[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) { g0[q] = TOT[q * 64 + j0]; g1[q] = TOT[q * 64 + j0 + 1]; }
    float lo0, lo1, hi0, hi1;      // products below and above the pair
    outer_products<W>(g0, g1, lo0, lo1, hi0, hi1);
    constexpr int wq = 2 * W;
    const bool second = (lane >> 5) != 0;   // group wq + 1
    const float ga0 = g0[wq], ga1 = g1[wq], gb0 = g0[wq + 1], gb1 = g1[wq + 1];
    Dec d;
    d.pre0 = second ? lo0 * ga0 : lo0;
    d.pre1 = second ? lo1 * ga1 : lo1;
    d.suf0 = second ? hi0 : gb0 * hi0;
    d.suf1 = second ? hi1 : gb1 * hi1;
    d.lam0 = (lo0 * ga0) * (gb0 * hi0);
    d.lam1 = (lo1 * ga1) * (gb1 * hi1);
    return d;
  };

  auto t_loop = [&](auto Wc) {
    constexpr int W = decltype(Wc)::value;
    RawT<DT> x;
    auto prep = [&](int c) {
      if (len - c * kL < kL) pad_raw(x, len - c * kL, rg);   // the last chunk
      decays(x.w);
    };
    load_raw(x, p, tok0, min(kL, len), h, rg, jp);
    prep(0);
    __syncthreads();                                              // TOT of chunk 0
    for (int step = 0; step <= nch; ++step) {
      const int cK = step;          // chunk whose operands and Grams are built
      const bool k_on = cK < nch;
      const int bK = cK & 1;
      VE* VOk = reinterpret_cast<VE*>(lds + M::VO + bK * M::VOBytes);
      VE* LLk = reinterpret_cast<VE*>(lds + M::LL + bK * M::LLBytes);
      // ===== interval 1 =====
      bool bad_k = false;
      if (k_on) {
        const Dec d = chunk_decays(Wc);
        // hardware reciprocal (1 ulp): the scaled Gram operands are split into
        // bf16 pairs, far coarser; a lam below the chunked form's range takes the
        // token-by-token path, which does not use these operands
        const float inv0 = __builtin_amdgcn_rcpf(d.lam0), inv1 = __builtin_amdgcn_rcpf(d.lam1);
        VE* Abar = VOk + M::Abar;
        VE* Rbar = VOk + M::Rbar;
        // range of the raw inputs (|Abar| <= |a| etc. when every |w| <= 1;
        // w and lam are checked on the s side)
        const typename R::W xs[8] = {x.a[0], x.a[1], x.a[2], x.a[3],
                                     x.r[0], x.r[1], x.r[2], x.r[3]};
        bad_k = R::big(xs);                                  // |x| >= 2^15 (or NaN/Inf)
  #pragma unroll
        for (int e = 3; e >= 0; --e) {
          const int t = 4 * rg + e;
          const float lp0 = e == 0 ? d.pre0 : d.pre0 * P0[e - 1];
          const float lp1 = e == 0 ? d.pre1 : d.pre1 * P1[e - 1];
          const float lt0 = d.pre0 * P0[e], lt1 = d.pre1 * P1[e];
          const float ab0 = R::c0(x.a[e]) * lp0, ab1 = R::c1(x.a[e]) * lp1;
          const float rb0 = R::c0(x.r[e]) * lt0, rb1 = R::c1(x.r[e]) * lt1;
          put2p(Ahat, kM64, kP64, t, j0, ab0 * inv0, ab1 * inv1);
          put2p(Rhat, kM64, kP64, t, j0, rb0 * inv0, rb1 * inv1);
          if constexpr (PRE) {
            put2p(Abar, kM64, kP64, t, j0, ab0, ab1);
            put2p(Rbar, kM64, kP64, t, j0, rb0, rb1);
          } else {
            put2h(Abar, kP64, t, j0, ab0, ab1);
            put2h(Rbar, kP64, t, j0, rb0, rb1);
          }
        }
      }
      // next chunk's inputs, in flight from here on
      load_next(x, cK);
      // no code moves across: work of the second interval hoisted above
      // the barrier would wait there for the loads just issued
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();                                            // mid-step barrier
      __builtin_amdgcn_sched_barrier(0);
      // ===== interval 2 =====
      float gmax = 0.f;
      if (k_on) {
        // Gram matrix W, tiles (tt, st) = (0,0), (1,0), (1,1) as C[s][t]
        const __bf16* Pm = (W & 1) ? Kbar : Bbar;
        const __bf16* Qm = (W >= 2) ? Rhat : Ahat;
        constexpr bool strict = W < 2;
        f32x4 gt[3];
        int ti = 0;
  #pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
  #pragma unroll
          for (int st = 0; st <= tt; ++st) {
            f32x4 c = z;
  #pragma unroll
            for (int kc = 0; kc < 2; ++kc)
              c = mm3(ldp8(Pm, kM64, kP64, 16 * st + n16, 32 * kc, g),
                      ldp8(Qm, kM64, kP64, 16 * tt + n16, 32 * kc, g), c);
            const int t = 16 * tt + n16;
            if (st == tt) {            // tile (1, 0) lies wholly below the diagonal
  #pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int s = 16 * st + 4 * g + r;
                const bool keep = strict ? (s < t) : (s <= t);
                c[r] = keep ? c[r] : 0.f;
              }
            }
            gt[ti++] = c;
          }
        }
        if (W == 0 && PRE) {
          // T = (I - A_ab)^-1 of this chunk, from the Gram tiles in
          // registers: tile ti holds C[s][t] = A_ab[t][s], so lane (g, n)
          // holds A_ab[16 tt + n][16 st + 4 g + r], the row fragment of
          // block (tt, st); a block's column fragment is its product with
          // the identity. The value side reads T's rows a step later; T's
          // range joins the Gram flag.
          f32x4 icol;
  #pragma unroll
          for (int r = 0; r < 4; ++r) icol[r] = (4 * g + r == n16) ? 1.f : 0.f;
          const f16x4 ic = h4(icol);
          const f16x4 r00 = h4(gt[0]), r10 = h4(gt[1]), r11 = h4(gt[2]);
          const Frag D0 = inverse_unit_lower(r00, h4(mmh16(r00, ic, z)), g, n16);
          const Frag D1 = inverse_unit_lower(r11, h4(mmh16(r11, ic, z)), g, n16);
          // col(Y) = A_10 D_0; row(T_10) = row(D_1 Y) from col(Y) and row(D_1)
          const f16x4 ycol = h4(mmh16(r10, D0.col, z));
          const f32x4 t10 = mmh16(ycol, D1.row, z);
  #pragma unroll
          for (int ti2 = 0; ti2 < 3; ++ti2) gmax = abs_max4(gt[ti2], gmax);
          gmax = abs_max4(D0.frow, abs_max4(D1.frow, abs_max4(t10, gmax)));
          _Float16* Tb = AB + bK * kM32;
          put4h(Tb, kP32, n16, 4 * g, D0.frow);
          put4h(Tb, kP32, n16, 16 + 4 * g, z);
          put4h(Tb, kP32, 16 + n16, 4 * g, t10);
          put4h(Tb, kP32, 16 + n16, 16 + 4 * g, D1.frow);
        } else if (W == 0) {
          // A_ab in fp16 as [t][s] rows and as [s][t] rows (tile ti holds
          // C[s][t] = A_ab[t][s]): T's operand fragments, read by the value
          // side in the next step
          _Float16* ABr = AB;
          _Float16* ABt = ABr + kM32;
          ti = 0;
  #pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
  #pragma unroll
            for (int st = 0; st <= tt; ++st, ++ti) {
              gmax = abs_max4(gt[ti], gmax);
              put4h(ABr, kP32, 16 * tt + n16, 16 * st + 4 * g, gt[ti]);
  #pragma unroll
              for (int r = 0; r < 4; ++r)
                ABt[(16 * st + 4 * g + r) * kP32 + 16 * tt + n16] =
                    static_cast<_Float16>(gt[ti][r]);
            }
          }
        } else {
          VE* dst = LLk + (W - 1) * M::kVO * kM32;
          ti = 0;
  #pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
  #pragma unroll
            for (int st = 0; st <= tt; ++st, ++ti) {
              gmax = abs_max4(gt[ti], gmax);
              if constexpr (PRE)
                put4p(dst, kM32, kP32, 16 * tt + n16, 16 * st + 4 * g, gt[ti]);
              else
                put4h(dst, kP32, 16 * tt + n16, 16 * st + 4 * g, gt[ti]);
            }
          }
          if constexpr (PRE)
            put4p(dst, kM32, kP32, n16, 16 + 4 * g, z);
          else
            put4h(dst, kP32, n16, 16 + 4 * g, z);
        }
      }
      prep(min(cK + 1, nch - 1));   // the next chunk
      (void)barrier_or2(FLG, wv, lane, k_on && bad_k,
                        k_on && !(gmax < kHalfSafe));  // end-of-step barrier
    }
  };

  auto s_loop = [&](auto Wc) {
    RawS<DT> x;
    // The s wavefronts load a chunk's w at the start of the first interval
    // of the step before its preparation (the build uses the decays
    // prepared from it, not x.w), and its k, b and v at the start of the
    // second interval: the preparation, which waits for w only, then needs
    // no load issued in the same interval.
    auto load_w = [&](int c) {
      const int cl = min(c, nch - 1);
      typename R::W (*const dst[1])[4] = {&x.w};
      const void* const src[1] = {p.w};
      load_rows<DT, 1>(dst, src, p, tok0 + cl * kL, min(kL, len - cl * kL), h, rg, jp);
    };
    auto load_kbv = [&](int c) {
      const int cl = min(c, nch - 1);
      typename R::W (*const dst[3])[4] = {&x.k, &x.b, &x.v};
      const void* const src[3] = {p.k, p.b, p.v};
      load_rows<DT, 3>(dst, src, p, tok0 + cl * kL, min(kL, len - cl * kL), h, rg, jp);
    };
    bool bad_w = false;   // |w| > 1 (or NaN) in the prepared chunk
    auto prep = [&](int c) {
      if (len - c * kL < kL) pad_raw(x, len - c * kL, rg);   // the last chunk
      bad_w = R::above_one(x.w);
      decays(x.w);
      TOT[rg * 64 + j0] = P0[3];
      TOT[rg * 64 + j0 + 1] = P1[3];
    };
    load_w(0);
    load_kbv(0);
    prep(0);
    __syncthreads();                                              // TOT of chunk 0
    for (int step = 0; step <= nch; ++step) {
      const int cK = step;          // chunk whose operands are built
      const bool k_on = cK < nch;
      const int bK = cK & 1;
      VE* VOk = reinterpret_cast<VE*>(lds + M::VO + bK * M::VOBytes);
      // ===== interval 1 =====
      load_w(cK + 1);
      bool bad_k = false;
      // decay-scaled b and k of the thread's rows and channels: the Gram
      // operands now, the value side's operands in the second interval
      float bt0[4], bt1[4], kt0[4], kt1[4];
      if (k_on) {
        const Dec d = chunk_decays(Wc);
        if (rg == 0) { LAMb[bK * 64 + j0] = d.lam0; LAMb[bK * 64 + j0 + 1] = d.lam1; }
        // range of the raw inputs (|Bbar| <= |b| etc. when every |w| <= 1);
        // v is zero on a run with kSegZeroV
        const typename R::W v0m = zero_v ? R::zero() : x.v[0], v1m = zero_v ? R::zero() : x.v[1];
        const typename R::W v2m = zero_v ? R::zero() : x.v[2], v3m = zero_v ? R::zero() : x.v[3];
        const typename R::W xs[12] = {x.b[0], x.b[1], x.b[2], x.b[3], x.k[0], x.k[1],
                                      x.k[2], x.k[3], v0m, v1m, v2m, v3m};
        // bitwise, not short-circuit: no branches
        bad_k = !(d.lam0 >= kMinLamL) | !(d.lam1 >= kMinLamL) |
                R::big(xs) |                                   // |x| >= 2^15 (or NaN/Inf)
                bad_w;
        // the Gram operands, read after the mid-step barrier
        float sfx0 = d.suf0, sfx1 = d.suf1;
  #pragma unroll
        for (int e = 3; e >= 0; --e) {
          const int t = 4 * rg + e;
          bt0[e] = R::c0(x.b[e]) * sfx0; bt1[e] = R::c1(x.b[e]) * sfx1;
          kt0[e] = R::c0(x.k[e]) * sfx0; kt1[e] = R::c1(x.k[e]) * sfx1;
          put2p(Bbar, kM64, kP64, t, j0, bt0[e], bt1[e]);
          put2p(Kbar, kM64, kP64, t, j0, kt0[e], kt1[e]);
          sfx0 *= w0[e]; sfx1 *= w1[e];
        }
      }
      // no code moves across: work of the second interval hoisted above
      // the barrier would wait there for loads
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();                                            // mid-step barrier
      __builtin_amdgcn_sched_barrier(0);
      // ===== interval 2 =====
      if (k_on) {
        // the value side's operands, read in the next step: built here,
        // where this role waits on the value side anyway, from the Gram
        // operands' products
        VE* BbT = VOk + M::BbT;
        VE* KbT = VOk + M::KbT;
        VE* Vt = VOk + M::Vt;
        float vt0[4], vt1[4];
  #pragma unroll
        for (int e = 0; e < 4; ++e) {
          vt0[e] = zero_v ? 0.f : R::c0(x.v[e]);
          vt1[e] = zero_v ? 0.f : R::c1(x.v[e]);
        }
        auto put4 = [&](VE* m, int row, const float (&v)[4]) {
          if constexpr (PRE)
            put4p(m, kMT, kP32, row, 4 * rg, f32x4{v[0], v[1], v[2], v[3]});
          else
            put4h(m, kP32, row, 4 * rg, f32x4{v[0], v[1], v[2], v[3]});
        };
        put4(BbT, j0, bt0);
        put4(BbT, j0 + 1, bt1);
        put4(KbT, j0, kt0);
        put4(KbT, j0 + 1, kt1);
        put4(Vt, j0, vt0);
        put4(Vt, j0 + 1, vt1);
      }
      load_kbv(cK + 1);
      prep(min(cK + 1, nch - 1));   // the next chunk
      (void)barrier_or2(FLG, wv, lane, k_on && bad_k, false);  // end of step
    }
  };

  if (role == 0) {
    switch (wv) {
      case 0: t_loop(IntC<0>{}); break;
      case 1: t_loop(IntC<1>{}); break;
      case 2: t_loop(IntC<2>{}); break;
      default: t_loop(IntC<3>{}); break;
    }
  } else if (role == 1) {
    switch (wv) {
      case 4: s_loop(IntC<0>{}); break;
      case 5: s_loop(IntC<1>{}); break;
      case 6: s_loop(IntC<2>{}); break;
      default: s_loop(IntC<3>{}); break;
    }
  } else {
    // The value wavefronts carry the chunk-to-chunk chain; the key
    // wavefronts on the same SIMDs have slack at the barriers. Issue
    // priority goes to the value wavefronts.
    __builtin_amdgcn_s_setprio(3);
    const size_t soff = static_cast<size_t>(16 * vb + n16) * kN + 4 * g;
    f32x4 S[4] = {};   // S[jt][r] = S[i = 16 vb + n16][j = 16 jt + 4 g + r]
    if (flags & kSegIdentity) {
#pragma unroll
      for (int jt = 0; jt < 4; ++jt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          S[jt][r] = (16 * vb + n16 == 16 * jt + 4 * g + r) ? 1.f : 0.f;
    } else if (s_in) {
#pragma unroll
      for (int jt = 0; jt < 4; ++jt)   // global accesses (see gf32x4)
        S[jt] = *(const gf32x4*)(s_in + soff + 16 * jt);
    }
    __syncthreads();                                              // TOT of chunk 0
    // fallback flags of chunk step - 1, known from the end of the step
    // before: early (its inputs or decays out of the chunked form's range)
    // and gram (its Gram matrices, in the precise plan also T, out of the
    // fp16 range; the fast plan checks T in the second interval)
    bool early_prev = false, gram_prev = false;
    // The start state has arrived before the loop: without this wait the
    // compiler keeps S's registers pending from these loads and, at every
    // state update, waits for the step's output stores as well.
    __builtin_amdgcn_s_waitcnt(0x0F70);                // vmcnt(0)
    for (int step = 0; step <= nch; ++step) {
      const int cV = step - 1;      // chunk whose value side is run
      const bool v_on = cV >= 0;
      const int bV = cV & 1;
      const VE* VOv = reinterpret_cast<const VE*>(lds + M::VO + bV * M::VOBytes);
      const VE* LLv = reinterpret_cast<const VE*>(lds + M::LL + bV * M::LLBytes);
      const int nV = min(kL, len - cV * kL);
      const int t0V = tok0 + cV * kL;
      // ===== interval 1 =====
      // value side, first half: X of chunk cV (or the whole chunk exactly)
      bool v_exact_done = false;
      float inv_s = 1.f;
      f16x8 Sf0 = {}, Sf1 = {}, Vf = {}, Xf = {};
      // precise plan: V and X as split pairs, and the part of O that
      // involves neither U nor the new state
      F8 Vp = {}, Xp = {};
      f32x4 Op[2] = {};
      float inv_x = 1.f;
      if (v_on) {
        const bool exact = early_prev || gram_prev;
        if (!exact) {
          if constexpr (PRE) {
            // X, and O's products with the old state and with V (T was
            // formed on the key side): the split state is not needed after
            // this interval
            const __bf16* Abar = VOv + M::Abar;
            const __bf16* Rbar = VOv + M::Rbar;
            const __bf16* Vt = VOv + M::Vt;
            const __bf16* Aak = LLv + M::Aak;
            const __bf16* Mrk = LLv + M::Mrk;
            const F8 Sp0 = frag8p(S[0], S[1]);
            const F8 Sp1 = frag8p(S[2], S[3]);
            Vp = ldp8(Vt, kMT, kP32, 16 * vb + n16, 0, g);
            f32x4 X[2];
  #pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
              f32x4 c = mm3(ldp8(Abar, kM64, kP64, 16 * tt + n16, 0, g), Sp0, z);
              c = mm3(ldp8(Abar, kM64, kP64, 16 * tt + n16, 32, g), Sp1, c);
              X[tt] = mm3(ldp8(Aak, kM32, kP32, 16 * tt + n16, 0, g), Vp, c);
            }
            Xp = frag8p(X[0], X[1]);
  #pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
              Op[tt] = mm3(Sp0, ldp8(Rbar, kM64, kP64, 16 * tt + n16, 0, g), z);
              Op[tt] = mm3(Sp1, ldp8(Rbar, kM64, kP64, 16 * tt + n16, 32, g), Op[tt]);
              Op[tt] = mm3(Vp, ldp8(Mrk, kM32, kP32, 16 * tt + n16, 0, g), Op[tt]);
            }
          } else {
            f32x4 X[2];
            const _Float16* Abar = VOv + M::Abar;
            const _Float16* Vt = VOv + M::Vt;
            const _Float16* Aak = LLv + M::Aak;
            float m = 0.f;
  #pragma unroll
            for (int jt = 0; jt < 4; ++jt) m = scale_max4(S[jt], m);
            const float sS = pow2_scale(wave_max(m), &inv_s);
            Sf0 = frag8h(S[0], S[1], sS);
            Sf1 = frag8h(S[2], S[3], sS);
            Vf = ldh8(Vt, kP32, 16 * vb + n16, 0, g);
  #pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
              f32x4 cs = mmah(ldh8(Abar, kP64, 16 * tt + n16, 0, g), Sf0, z);
              cs = mmah(ldh8(Abar, kP64, 16 * tt + n16, 32, g), Sf1, cs);
              const f32x4 cv = mmah(ldh8(Aak, kP32, 16 * tt + n16, 0, g), Vf, z);
  #pragma unroll
              for (int r = 0; r < 4; ++r) X[tt][r] = fmaf(cs[r], inv_s, cv[r]);
            }
            // X scaled into the fp16 range here, where the value side has
            // slack, so that the second interval starts with U
            const float sX = pow2_scale(wave_max(scale_max4(X[1], scale_max4(X[0], 0.f))), &inv_x);
            Xf = frag8h(X[0], X[1], sX);
            // T = [[D_0, 0], [T_10, D_1]], D_p = (I - A_pp)^-1, T_10 = D_1 A_10 D_0,
            // from A_ab of chunk cV: value wavefront 0 computes D_0 and
            // Y = A_10 D_0, wavefront 1 computes D_1, each value wavefront then
            // T_10 = D_1 Y in the second interval. Each posts whether its
            // part left the fp16 range.
            const _Float16* ABr = AB;
            const _Float16* ABt = ABr + kM32;
            if (vb == 0) {
              const Frag D0 = inverse_unit_lower(ldh4(ABr, kP32, n16, 4 * g),
                                                 ldh4(ABt, kP32, n16, 4 * g), g, n16);
              // col(Y) = A_10 D_0 from row(A_10) and col(D_0)
              const f16x4 ycol = h4(mmh16(ldh4(ABr, kP32, 16 + n16, 4 * g), D0.col, z));
              put4h(TT, kP32, n16, 4 * g, D0.frow);
              put4h(TT, kP32, n16, 16 + 4 * g, z);
              *reinterpret_cast<f16x4*>(YC + 4 * lane) = ycol;
              const bool out = __builtin_amdgcn_ballot_w64(!(abs_max4(D0.frow, 0.f) < kHalfSafe)) != 0;
              if (lane == 0) TFL[0] = out ? 1u : 0u;
            } else if (vb == 1) {
              const Frag D1 = inverse_unit_lower(ldh4(ABr, kP32, 16 + n16, 16 + 4 * g),
                                                 ldh4(ABt, kP32, 16 + n16, 16 + 4 * g), g, n16);
              put4h(TT, kP32, 16 + n16, 16 + 4 * g, D1.frow);
              *reinterpret_cast<f16x4*>(D1R + 4 * lane) = D1.row;
              const bool out = __builtin_amdgcn_ballot_w64(!(abs_max4(D1.frow, 0.f) < kHalfSafe)) != 0;
              if (lane == 0) TFL[1] = out ? 1u : 0u;
            }
          }
        }
        if (exact) {
          // the whole chunk token by token
          exact_chunk<DT>(p, S, t0V, nV, h, vb, g, n16, zero_v, no_out);
          v_exact_done = true;
        }
      }
      __syncthreads();                                            // mid-step barrier
      // ===== interval 2 =====
      bool t_exact = false;
      f32x4 t10 = z;
      // (the precise plan formed T and checked its range on the key side)
      if (!PRE && v_on && !v_exact_done) {
        t10 = mmh16(*reinterpret_cast<const f16x4*>(YC + 4 * lane),
                    *reinterpret_cast<const f16x4*>(D1R + 4 * lane), z);
        t_exact = (TFL[0] | TFL[1]) != 0 ||
                  __builtin_amdgcn_ballot_w64(!(abs_max4(t10, 0.f) < kHalfSafe)) != 0;
        if (t_exact) {
          // T out of the fp16 range: the whole chunk token by token
          exact_chunk<DT>(p, S, t0V, nV, h, vb, g, n16, zero_v, no_out);
        }
      }
      if (v_on && !v_exact_done && !t_exact) {
        if constexpr (PRE) {
          // value side, second half: U, the rest of O, the state update of
          // chunk cV, every product from split bf16 operands. The state's
          // products with V are issued first; T's fp16 values split exactly.
          const __bf16* BbT = VOv + M::BbT;
          const __bf16* KbT = VOv + M::KbT;
          const __bf16* Mrb = LLv + M::Mrb;
          const float* lam = LAMb + bV * 64;
  #pragma unroll
          for (int jt = 0; jt < 4; ++jt) {
            const f32x4 lm = *reinterpret_cast<const f32x4*>(lam + 16 * jt + 4 * g);
            f32x4 c;
  #pragma unroll
            for (int r = 0; r < 4; ++r) c[r] = lm[r] * S[jt][r];
            S[jt] = mm3(ldp8(KbT, kMT, kP32, 16 * jt + n16, 0, g), Vp, c);
          }
          const _Float16* Tb = AB + bV * kM32;
          const f32x4 U0 = mm3(split_f16(ldh8(Tb, kP32, n16, 0, g)), Xp, z);
          const f32x4 U1 = mm3(split_f16(ldh8(Tb, kP32, 16 + n16, 0, g)), Xp, z);
          const F8 Up = frag8p(U0, U1);
  #pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            const f32x4 c = mm3(Up, ldp8(Mrb, kM32, kP32, 16 * tt + n16, 0, g), Op[tt]);
            const int t = 16 * tt + n16;
            if (t < nV && !no_out)
              *reinterpret_cast<float4*>(p.o + static_cast<size_t>(t0V + t) * rowstride
                                         + static_cast<size_t>(h) * kN + 16 * vb + 4 * g) =
                  make_float4(c[0], c[1], c[2], c[3]);
          }
  #pragma unroll
          for (int jt = 0; jt < 4; ++jt)
            S[jt] = mm3(ldp8(BbT, kMT, kP32, 16 * jt + n16, 0, g), Up, S[jt]);
        } else {
          // value side, second half: U, O, state update of chunk cV
          const _Float16* Rbar = VOv + M::Rbar;
          const _Float16* BbT = VOv + M::BbT;
          const _Float16* KbT = VOv + M::KbT;
          const _Float16* Mrb = LLv + M::Mrb;
          const _Float16* Mrk = LLv + M::Mrk;
          const float* lam = LAMb + bV * 64;
          // Every LDS operand of the step's products is read first, and the
          // products that do not involve U are issued before X and U are
          // scaled, so that the LDS reads and those products overlap the two
          // wavefront reductions instead of waiting one by one. Each sum is
          // formed in the same order as when computed term by term.
          f16x8 rb[2][2], mb[2], mk[2], bt[4], kt[4];
          f32x4 lm[4];
          // operand fragments of T's row tiles: k in [0,16) then [16,32)
          const f16x8 Tf0 = ldh8(TT, kP32, n16, 0, g);
          f16x8 Tf1;
          {
            const f16x4 t10h = h4(t10);
            const f16x4 d1 = ldh4(TT, kP32, 16 + n16, 16 + 4 * g);
  #pragma unroll
            for (int r = 0; r < 4; ++r) { Tf1[r] = t10h[r]; Tf1[4 + r] = d1[r]; }
          }
  #pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            rb[tt][0] = ldh8(Rbar, kP64, 16 * tt + n16, 0, g);
            rb[tt][1] = ldh8(Rbar, kP64, 16 * tt + n16, 32, g);
            mk[tt] = ldh8(Mrk, kP32, 16 * tt + n16, 0, g);
            mb[tt] = ldh8(Mrb, kP32, 16 * tt + n16, 0, g);
          }
  #pragma unroll
          for (int jt = 0; jt < 4; ++jt) {
            kt[jt] = ldh8(KbT, kP32, 16 * jt + n16, 0, g);
            bt[jt] = ldh8(BbT, kP32, 16 * jt + n16, 0, g);
            lm[jt] = *reinterpret_cast<const f32x4*>(lam + 16 * jt + 4 * g);
          }
          f32x4 cs[2], cvo[2], cvs[4];
  #pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            cs[tt] = mmah(Sf0, rb[tt][0], z);
            cs[tt] = mmah(Sf1, rb[tt][1], cs[tt]);
            cvo[tt] = mmah(Vf, mk[tt], z);
          }
  #pragma unroll
          for (int jt = 0; jt < 4; ++jt) cvs[jt] = mmah(kt[jt], Vf, z);
          f32x4 U[2];
          U[0] = mmah(Tf0, Xf, z);
          U[1] = mmah(Tf1, Xf, z);
          float inv_u;
          const float sU = pow2_scale(wave_max(scale_max4(U[1], scale_max4(U[0], 0.f))), &inv_u);
          const float inv_ux = inv_u * inv_x;
          const f16x8 Uf = frag8h(U[0], U[1], sU);
  #pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            const f32x4 cu = mmah(Uf, mb[tt], z);
            const int t = 16 * tt + n16;
            if (t < nV && !no_out) {
              float4 ov;
              ov.x = fmaf(cs[tt][0], inv_s, fmaf(cu[0], inv_ux, cvo[tt][0]));
              ov.y = fmaf(cs[tt][1], inv_s, fmaf(cu[1], inv_ux, cvo[tt][1]));
              ov.z = fmaf(cs[tt][2], inv_s, fmaf(cu[2], inv_ux, cvo[tt][2]));
              ov.w = fmaf(cs[tt][3], inv_s, fmaf(cu[3], inv_ux, cvo[tt][3]));
              *reinterpret_cast<float4*>(p.o + static_cast<size_t>(t0V + t) * rowstride
                                         + static_cast<size_t>(h) * kN + 16 * vb + 4 * g) = ov;
            }
          }
  #pragma unroll
          for (int jt = 0; jt < 4; ++jt) {
            const f32x4 cu = mmah(bt[jt], Uf, z);
  #pragma unroll
            for (int r = 0; r < 4; ++r)
              S[jt][r] = fmaf(lm[jt][r], S[jt][r], fmaf(cu[r], inv_ux, cvs[jt][r]));
          }
        }
      }
      const uint32_t f3 = barrier_or2(FLG, wv, lane, false, false);  // end of step
      early_prev = (f3 & 1u) != 0;
      gram_prev = (f3 & 2u) != 0;
    }
    if (s_out) {
#pragma unroll
      for (int jt = 0; jt < 4; ++jt)
        *(gf32x4*)(s_out + soff + 16 * jt) = S[jt];
    }
  }
}

// The kernel instance for an input type and plan: fp32 inputs always take
// the precise plan.
template <bool SEG>
hipError_t launch_p(const SeqArgs& args, bool precise, const SegItem* segs,
                    hipStream_t stream, const WorkItem* dec, int32_t n_dec) {
  if (args.n_items <= 0) return hipSuccess;
  const int64_t blocks = static_cast<int64_t>(args.n_items) * args.H +
                         chunk_decode_blocks(n_dec, args.H);
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(blocks)), block(64 * kChunkPWaves);
  if (args.dtype == WKV7_F32)
    hipLaunchKernelGGL((chunk_p_kernel<SEG, WKV7_F32, true>), grid, block, 0,
                       stream, args, segs, dec, n_dec);
  else if (precise)
    hipLaunchKernelGGL((chunk_p_kernel<SEG, WKV7_BF16, true>), grid, block, 0,
                       stream, args, segs, dec, n_dec);
  else
    hipLaunchKernelGGL((chunk_p_kernel<SEG, WKV7_BF16, false>), grid, block, 0,
                       stream, args, segs, dec, n_dec);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_chunked_p(const SeqArgs& args, bool precise,
                            hipStream_t stream, const WorkItem* dec,
                            int32_t n_dec) {
  return launch_p<false>(args, precise, nullptr, stream, dec, n_dec);
}

hipError_t launch_chunked_p_seg(const SeqArgs& args, bool precise,
                                const SegItem* segs, hipStream_t stream,
                                const WorkItem* dec, int32_t n_dec) {
  return launch_p<true>(args, precise, segs, stream, dec, n_dec);
}

}  // namespace wkv7
