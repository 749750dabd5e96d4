// Chunked-prefill WKV-7 kernel for bf16 inputs on gfx950: split-bf16 Gram
// matrices, fp16 value side.
//
// Same operation and chunked (WY/UT) algebra as the split-precision chunked
// kernel (page "RWKV-X Architecture", section "WKV-7 Kernel (Generalized
// Delta Rule)", product-form reading). Differences, all for speed:
//
// * Decays are running products: Lambda_t = prod_{u<=t} w_u and
//   suf_t = prod_{u>t} w_u per key channel, with no per-element
//   transcendental. The Gram operands are scaled about the chunk END:
//     A_ab[t][s] = <Abar_t / Lambda_L, Bbar_s>,  A_ak[t][s] = <Abar_t / Lambda_L, Kbar_s>
//     M_rb[t][s] = <Rbar_t / Lambda_L, Bbar_s>,  M_rk[t][s] = <Rbar_t / Lambda_L, Kbar_s>
//   with Abar_t = a_t Lambda_{t-1}, Rbar_t = r_t Lambda_t, Bbar_s = b_s suf_s,
//   Kbar_s = k_s suf_s; each product term is the exact decay between s and t
//   (<= 1). A chunk with Lambda_L < 2^-100 in some channel (the scaled
//   operands Abar / Lambda_L could leave fp32 range) runs token by token.
// * Gram products use bf16 hi + lo operands (three MFMAs, fp32 accumulate);
//   everything on the value side (X = Abar S0^T + A_ak V, U = T X,
//   O = Rbar S0^T + M_rb U + M_rk V, S_L = Lambda_L S0 + U^T Bbar + V^T Kbar) uses
//   single fp16 operands (v_mfma_f32_16x16x32_f16). The state, X and U are
//   scaled by powers of two before each fp16 conversion (exact), so their
//   magnitude never limits the range; every other fp16 operand is checked
//   against the fp16 range and a chunk that fails runs token by token.
//   Measured against the float64 oracle on the workloads' inputs this gives
//   ~3e-3 of max|err|/rms (the bf16-input bar is 2e-2).
// * T = (I - A_ab)^-1 by column blocks: diagonal blocks by forward
//   substitution, then each wavefront walks its column block down with the
//   previous result tiles chained in registers (no LDS round trip, no
//   barrier between levels).
// * The next chunk's inputs are loaded while the current chunk's value side
//   runs.
//
// Work split: one 256-thread workgroup per (sequence, head); wavefront w owns
// state rows i in [16 w, 16 w + 16) (S^T accumulator tiles) for the value
// side, computes Gram matrix w, and column block w of T. For element-wise
// work a thread owns two key channels and eight token rows.

#include "internal.h"
#include "../../include/wkv7.h"

namespace wkv7 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kChunk = 64;
constexpr int kPitch = 68;                  // elements per LDS matrix row
constexpr int kMat = 64 * kPitch;           // elements per matrix
constexpr int kMatB = kMat * 2;             // bytes per 16-bit matrix
constexpr int kPairB = 2 * kMatB;           // bytes per hi/lo pair
// LDS map (bytes)
constexpr int kOffGR = 0;                        // 4 bf16 pairs
constexpr int kOffVO = kOffGR + 4 * kPairB;      // 5 fp16 matrices
constexpr int kOffLL = kOffVO + 5 * kMatB;       // 4 fp16 matrices
constexpr int kOffDG = kOffLL + 4 * kMatB;       // fp32 [4][16][16]
constexpr int kOffTOT = kOffDG + 4 * 256 * 4;    // fp32 [8][64]
constexpr int kOffLAM = kOffTOT + 8 * 64 * 4;    // fp32 [64]
constexpr int kLdsBytes = kOffLAM + 64 * 4;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
static_assert(6 * 64 * 64 * 4 <= kOffLL, "raw staging fits in GR + VO");

constexpr float kHalfSafe = 32768.f;             // fp16 operand bound
constexpr float kMinLamL = 7.88860905e-31f;      // 2^-100

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

// Fragment of row `row`, k = kb + {4g..4g+3, 16+4g..16+4g+3} (16-bit types).
template <typename V8, typename V4, typename E>
__device__ __forceinline__ V8 ld8(const E* m, int row, int kb, int g) {
  const E* p = m + row * kPitch + kb + 4 * g;
  V4 a = *reinterpret_cast<const V4*>(p);
  V4 b = *reinterpret_cast<const V4*>(p + 16);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ F8 ldp8(const __bf16* pair, int row, int kb, int g) {
  return F8{ld8<bf16x8, bf16x4>(pair, row, kb, g),
            ld8<bf16x8, bf16x4>(pair + kMat, row, kb, g)};
}
__device__ __forceinline__ F4 ldp4(const __bf16* pair, int row, int kb, int g) {
  const int o = row * kPitch + kb + 4 * g;
  return F4{*reinterpret_cast<const bf16x4*>(pair + o),
            *reinterpret_cast<const bf16x4*>(pair + kMat + o)};
}
__device__ __forceinline__ f16x8 ldh8(const _Float16* m, int row, int kb,
                                      int g) {
  return ld8<f16x8, f16x4>(m, row, kb, g);
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
__device__ __forceinline__ F8 frag8(f32x4 t0, f32x4 t1) {
  F8 f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    __bf16 h, l;
    split(t0[r], h, l); f.h[r] = h; f.l[r] = l;
    split(t1[r], h, l); f.h[4 + r] = h; f.l[4 + r] = l;
  }
  return f;
}
// fp16 operand fragment from two result tiles, scaled
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

// two adjacent bf16 pair-matrix elements (4-byte aligned)
__device__ __forceinline__ void put2p(__bf16* pair, int row, int col, float x0,
                                      float x1) {
  __bf16 h0, l0, h1, l1;
  split(x0, h0, l0);
  split(x1, h1, l1);
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 h = {h0, h1}, l = {l0, l1};
  *reinterpret_cast<bf16x2*>(pair + row * kPitch + col) = h;
  *reinterpret_cast<bf16x2*>(pair + kMat + row * kPitch + col) = l;
}
__device__ __forceinline__ void put2h(_Float16* m, int row, int col, float x0,
                                      float x1) {
  f16x2 v = {static_cast<_Float16>(x0), static_cast<_Float16>(x1)};
  *reinterpret_cast<f16x2*>(m + row * kPitch + col) = v;
}
// eight consecutive fp16 (16-byte aligned when col % 8 == 0 and row pitch ok)
__device__ __forceinline__ void put8h(_Float16* m, int row, int col,
                                      const float* x) {
  f16x4 a, b;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    a[e] = static_cast<_Float16>(x[e]);
    b[e] = static_cast<_Float16>(x[4 + e]);
  }
  f16x4* p = reinterpret_cast<f16x4*>(m + row * kPitch + col);
  p[0] = a;
  p[1] = b;
}
__device__ __forceinline__ void put4p(__bf16* pair, int row, int col,
                                      f32x4 x) {
  F4 f = frag4(x);
  *reinterpret_cast<bf16x4*>(pair + row * kPitch + col) = f.h;
  *reinterpret_cast<bf16x4*>(pair + kMat + row * kPitch + col) = f.l;
}
__device__ __forceinline__ void put4h(_Float16* m, int row, int col, f32x4 x) {
  f16x4 v;
#pragma unroll
  for (int r = 0; r < 4; ++r) v[r] = static_cast<_Float16>(x[r]);
  *reinterpret_cast<f16x4*>(m + row * kPitch + col) = v;
}

__device__ __forceinline__ float dpp_max16(float x) {
  int xi = __builtin_bit_cast(int, x);
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, xi, 0xB1, 0xF, 0xF, false)));
  xi = __builtin_bit_cast(int, x);
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, xi, 0x4E, 0xF, 0xF, false)));
  xi = __builtin_bit_cast(int, x);
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, xi, 0x141, 0xF, 0xF, false)));
  xi = __builtin_bit_cast(int, x);
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, xi, 0x140, 0xF, 0xF, false)));
  return x;
}
// max over the wavefront
__device__ __forceinline__ float wave_max(float x) {
  x = dpp_max16(x);
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}
// Power of two s with max|x * s| < 2^14 for max|x| = m (s = 1 if m is 0 or
// not finite); returns s, and 1/s in *inv.
__device__ __forceinline__ float pow2_scale(float m, float* inv) {
  const uint32_t bits = __float_as_uint(m);
  const int e = static_cast<int>((bits >> 23) & 0xffu) - 127;  // floor(log2 m)
  if (!(m > 0.f) || e > 126 || e < -100) { *inv = 1.f; return 1.f; }
  const int k = 13 - e;            // m * 2^k in [2^13, 2^14)
  *inv = __uint_as_float(static_cast<uint32_t>(127 - k) << 23);
  return __uint_as_float(static_cast<uint32_t>(127 + k) << 23);
}

__device__ __forceinline__ float abs_max4(f32x4 x, float m) {
  return fmaxf(fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])),
                     fmaxf(fabsf(x[2]), fabsf(x[3]))), m);
}

// raw inputs of one thread: rows 8 rg + e, channels 2 jp, 2 jp + 1 (bf16 x2)
struct Raw { uint32_t r[8], w[8], k[8], a[8], b[8], v[8]; };

__device__ __forceinline__ void load_raw(Raw& x, const SeqArgs& p, int t0,
                                         int n, int h, int rg, int jp) {
  const uint32_t* R = static_cast<const uint32_t*>(p.r);
  const uint32_t* Wp = static_cast<const uint32_t*>(p.w);
  const uint32_t* K = static_cast<const uint32_t*>(p.k);
  const uint32_t* A = static_cast<const uint32_t*>(p.a);
  const uint32_t* B = static_cast<const uint32_t*>(p.b);
  const uint32_t* V = static_cast<const uint32_t*>(p.v);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int t = 8 * rg + e;
    if (t < n) {
      // 32 uint32 words per (token, head) row of 64 bf16
      const size_t off = (static_cast<size_t>(t0 + t) * p.H + h) * (kN / 2) + jp;
      x.r[e] = R[off]; x.w[e] = Wp[off]; x.k[e] = K[off];
      x.a[e] = A[off]; x.b[e] = B[off]; x.v[e] = V[off];
    } else {
      // padding rows: w = 1, everything else 0 (leaves the state unchanged)
      x.r[e] = 0u; x.w[e] = 0x3f803f80u; x.k[e] = 0u;
      x.a[e] = 0u; x.b[e] = 0u; x.v[e] = 0u;
    }
  }
}

// Column block Q of T = (I - A_ab)^-1, walked down from its diagonal block:
// T[p][Q] = D_p sum_{m=Q}^{p-1} A_pm T[m][Q]. Result tiles stay in registers
// (lane holds T[16 p + 4 g + r][16 Q + n16]) and feed the next level as
// operand fragments; the finished column block is written to Tm as fp16.
template <int Q>
__device__ __forceinline__ void col_block(const __bf16* Aab, const __bf16* Dp,
                                          _Float16* Tm, f32x4 dq, int g,
                                          int n16, float& tmax) {
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  f32x4 T[4];
  T[Q] = dq;
#pragma unroll
  for (int pb = Q + 1; pb < 4; ++pb) {
    f32x4 y = z;
#pragma unroll
    for (int m = Q; m < pb; m += 2) {
      if (m + 1 < pb)
        y = mm3(ldp8(Aab, 16 * pb + n16, 16 * m, g), frag8(T[m], T[m + 1]), y);
      else
        y = mm3(ldp4(Aab, 16 * pb + n16, 16 * m, g), frag4(T[m]), y);
    }
    T[pb] = mm3(ldp4(Dp, 16 * pb + n16, 16 * pb, g), frag4(y), z);
  }
#pragma unroll
  for (int pb = Q; pb < 4; ++pb) {
    tmax = abs_max4(T[pb], tmax);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      Tm[(16 * pb + 4 * g + r) * kPitch + 16 * Q + n16] =
          static_cast<_Float16>(T[pb][r]);
  }
  // upper tiles read by 32-wide fragments: (0,1) and (2,3)
  if (Q == 1 || Q == 3) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      Tm[(16 * (Q - 1) + 4 * g + r) * kPitch + 16 * Q + n16] =
          static_cast<_Float16>(0.f);
  }
}

__global__ __launch_bounds__(256, 1)
void chunk_h_kernel(SeqArgs p) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[kLdsBytes];
  __bf16* GR = reinterpret_cast<__bf16*>(lds + kOffGR);
  _Float16* VO = reinterpret_cast<_Float16*>(lds + kOffVO);
  _Float16* LL = reinterpret_cast<_Float16*>(lds + kOffLL);
  float* DG = reinterpret_cast<float*>(lds + kOffDG);
  float* TOT = reinterpret_cast<float*>(lds + kOffTOT);
  float* LAM = reinterpret_cast<float*>(lds + kOffLAM);
  __bf16* Ahat = GR;                              // [t][j]
  __bf16* Rhat = GR + kMat * 2;                   // [t][j]
  __bf16* Bbar = GR + kMat * 4;                   // [s][j]
  __bf16* Kbar = GR + kMat * 6;                   // [s][j]
  _Float16* Abar = VO;                            // [t][j]
  _Float16* Rbar = VO + kMat;                     // [t][j]
  _Float16* BbT = VO + 2 * kMat;                  // [j][s]
  _Float16* KbT = VO + 3 * kMat;                  // [j][s]
  _Float16* Vt = VO + 4 * kMat;                   // [i][s]
  _Float16* Aak = LL;
  _Float16* Mrb = LL + kMat;
  _Float16* Mrk = LL + 2 * kMat;
  _Float16* Tm = LL + 3 * kMat;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4;
  const int n16 = lane & 15;
  const int item = blockIdx.x / p.H;
  const int h = blockIdx.x - item * p.H;
  if (item >= p.n_items) return;
  const WorkItem it = p.items[item];
  const int jp = lane & 31;             // channel pair: j0 = 2 jp
  const int j0 = 2 * jp;
  const int rg = 2 * wv + (lane >> 5);  // row group: rows 8 rg .. 8 rg + 7

  float* sbase = p.pool + (static_cast<size_t>(it.slot) * p.H + h) * (kN * kN)
                 + (16 * wv + n16) * kN + 4 * g;
  f32x4 S[4];      // S[jt][r] = S[i = 16 wv + n16][j = 16 jt + 4 g + r]
#pragma unroll
  for (int jt = 0; jt < 4; ++jt) {
    float4 x = *reinterpret_cast<const float4*>(sbase + 16 * jt);
    S[jt] = f32x4{x.x, x.y, x.z, x.w};
  }

  const int nchunks = (it.len + kChunk - 1) / kChunk;
  Raw nxt;
  load_raw(nxt, p, it.tok0, min(kChunk, it.len), h, rg, jp);

  for (int ch = 0; ch < nchunks; ++ch) {
    const int t0 = it.tok0 + ch * kChunk;
    const int n = min(kChunk, it.len - ch * kChunk);
    const Raw x = nxt;

    // ---- decays: running products over this thread's 8 rows ----
    float w0[8], w1[8], P0[8], P1[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) { w0[e] = bf_lo(x.w[e]); w1[e] = bf_hi(x.w[e]); }
    P0[0] = w0[0]; P1[0] = w1[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) { P0[e] = P0[e - 1] * w0[e]; P1[e] = P1[e - 1] * w1[e]; }
    TOT[rg * 64 + j0] = P0[7];
    TOT[rg * 64 + j0 + 1] = P1[7];
    __syncthreads();
    float pre0 = 1.f, pre1 = 1.f, lam0 = 1.f, lam1 = 1.f, suf0 = 1.f, suf1 = 1.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float g0 = TOT[q * 64 + j0], g1 = TOT[q * 64 + j0 + 1];
      lam0 *= g0; lam1 *= g1;
      if (q < rg) { pre0 *= g0; pre1 *= g1; }
    }
#pragma unroll
    for (int q = 7; q > 0; --q) {
      if (q > rg) {
        suf0 *= TOT[q * 64 + j0];
        suf1 *= TOT[q * 64 + j0 + 1];
      }
    }
    if (rg == 0) { LAM[j0] = lam0; LAM[j0 + 1] = lam1; }
    const float inv0 = 1.f / lam0, inv1 = 1.f / lam1;
    bool bad = !(lam0 >= kMinLamL) || !(lam1 >= kMinLamL);

    // ---- operands ----
    float sfx0 = suf0, sfx1 = suf1;         // prod_{u > t} w_u, built backwards
    float bt0[8], bt1[8], kt0[8], kt1[8], vt0[8], vt1[8];
    float amax = 0.f;
#pragma unroll
    for (int e = 7; e >= 0; --e) {
      const int t = 8 * rg + e;
      const float lp0 = e == 0 ? pre0 : pre0 * P0[e - 1];   // Lambda_{t-1}
      const float lp1 = e == 0 ? pre1 : pre1 * P1[e - 1];
      const float lt0 = pre0 * P0[e], lt1 = pre1 * P1[e];    // Lambda_t
      const float a0 = bf_lo(x.a[e]), a1 = bf_hi(x.a[e]);
      const float r0 = bf_lo(x.r[e]), r1 = bf_hi(x.r[e]);
      const float b0 = bf_lo(x.b[e]), b1 = bf_hi(x.b[e]);
      const float k0 = bf_lo(x.k[e]), k1 = bf_hi(x.k[e]);
      const float v0 = bf_lo(x.v[e]), v1 = bf_hi(x.v[e]);
      const float ab0 = a0 * lp0, ab1 = a1 * lp1;          // Abar
      const float rb0 = r0 * lt0, rb1 = r1 * lt1;          // Rbar
      const float bb0 = b0 * sfx0, bb1 = b1 * sfx1;        // Bbar
      const float kb0 = k0 * sfx0, kb1 = k1 * sfx1;        // Kbar
      // every value that becomes an fp16 operand, and the raw a, r that
      // scale into the Gram operands
      amax = fmaxf(amax, fmaxf(fmaxf(fabsf(a0), fabsf(a1)), fmaxf(fabsf(r0), fabsf(r1))));
      amax = fmaxf(amax, fmaxf(fmaxf(fabsf(ab0), fabsf(ab1)), fmaxf(fabsf(rb0), fabsf(rb1))));
      amax = fmaxf(amax, fmaxf(fmaxf(fabsf(bb0), fabsf(bb1)), fmaxf(fabsf(kb0), fabsf(kb1))));
      amax = fmaxf(amax, fmaxf(fabsf(v0), fabsf(v1)));
      put2p(Ahat, t, j0, ab0 * inv0, ab1 * inv1);
      put2p(Rhat, t, j0, rb0 * inv0, rb1 * inv1);
      put2p(Bbar, t, j0, bb0, bb1);
      put2p(Kbar, t, j0, kb0, kb1);
      put2h(Abar, t, j0, ab0, ab1);
      put2h(Rbar, t, j0, rb0, rb1);
      bt0[e] = bb0; bt1[e] = bb1; kt0[e] = kb0; kt1[e] = kb1;
      vt0[e] = v0; vt1[e] = v1;
      sfx0 *= w0[e]; sfx1 *= w1[e];
    }
    put8h(BbT, j0, 8 * rg, bt0);
    put8h(BbT, j0 + 1, 8 * rg, bt1);
    put8h(KbT, j0, 8 * rg, kt0);
    put8h(KbT, j0 + 1, 8 * rg, kt1);
    put8h(Vt, j0, 8 * rg, vt0);
    put8h(Vt, j0 + 1, 8 * rg, vt1);
    bad = bad || !(amax < kHalfSafe);
    int extreme = __syncthreads_or(bad);

    if (!extreme) {
      // ---- Gram matrices: wavefront wv computes one; C[s][t] tiles ----
      const __bf16* Pm = (wv & 1) ? Kbar : Bbar;
      const __bf16* Qm = (wv >= 2) ? Rhat : Ahat;
      const bool strict = wv < 2;
      f32x4 gt[10];
      int ti = 0;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
        for (int st = 0; st <= tt; ++st) {
          f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kc = 0; kc < 2; ++kc)
            c = mm3(ldp8(Pm, 16 * st + n16, 32 * kc, g),
                    ldp8(Qm, 16 * tt + n16, 32 * kc, g), c);
          const int t = 16 * tt + n16;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int s = 16 * st + 4 * g + r;
            const bool keep = strict ? (s < t) : (s <= t);
            c[r] = keep ? c[r] : 0.f;
          }
          gt[ti++] = c;
        }
      }
      float gmax = 0.f;
      if (wv == 0) {
        // A_ab: diagonal blocks in fp32 for the forward substitution
        ti = 0;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
          for (int st = 0; st <= tt; ++st, ++ti) {
            if (tt == st) {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                DG[(tt * 16 + n16) * 16 + 4 * g + r] = gt[ti][r];
            }
          }
        }
      } else {
        _Float16* dst = LL + (wv - 1) * kMat;
        ti = 0;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
          for (int st = 0; st <= tt; ++st, ++ti) {
            gmax = abs_max4(gt[ti], gmax);
            put4h(dst, 16 * tt + n16, 16 * st + 4 * g, gt[ti]);
          }
        }
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        put4h(dst, n16, 16 + 4 * g, z);
        put4h(dst, 32 + n16, 48 + 4 * g, z);
      }
      bad = !(gmax < kHalfSafe);
      __syncthreads();   // Gram operands are dead from here on

      // ---- T = (I - A_ab)^-1 ----
      __bf16* Aab = GR;                    // pair [t][s]
      __bf16* Dp = GR + kMat * 2;          // pair, diagonal blocks [t][s]
      if (wv == 0) {
        ti = 0;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
          for (int st = 0; st <= tt; ++st, ++ti)
            put4p(Aab, 16 * tt + n16, 16 * st + 4 * g, gt[ti]);
        }
      }
      // diagonal block D_wv, column n16, by forward substitution; every
      // lane group computes the same column and keeps rows 4 g .. 4 g + 3,
      // i.e. the result tile T[16 wv + 4 g + r][16 wv + n16]
      f32x4 dq;
      {
        const float* Dg = DG + wv * 256;
        float d[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float s = (i == n16) ? 1.f : 0.f;
#pragma unroll
          for (int k = 0; k < i; ++k) s = fmaf(Dg[i * 16 + k], d[k], s);
          d[i] = s;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v = d[r];
#pragma unroll
          for (int gg = 1; gg < 4; ++gg) v = (g == gg) ? d[4 * gg + r] : v;
          dq[r] = v;
        }
        // D_wv as a P operand [t][s]
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          __bf16 hh, ll;
          split(dq[r], hh, ll);
          Dp[(16 * wv + 4 * g + r) * kPitch + 16 * wv + n16] = hh;
          Dp[kMat + (16 * wv + 4 * g + r) * kPitch + 16 * wv + n16] = ll;
        }
      }
      __syncthreads();
      {
        float tmax = 0.f;
        switch (wv) {
          case 0: col_block<0>(Aab, Dp, Tm, dq, g, n16, tmax); break;
          case 1: col_block<1>(Aab, Dp, Tm, dq, g, n16, tmax); break;
          case 2: col_block<2>(Aab, Dp, Tm, dq, g, n16, tmax); break;
          default: col_block<3>(Aab, Dp, Tm, dq, g, n16, tmax); break;
        }
        bad = bad || !(tmax < kHalfSafe);
      }
      extreme = __syncthreads_or(bad);
    }

    if (extreme) {
      // ---- exact token-by-token path for this chunk ----
      float* raw = reinterpret_cast<float*>(lds);   // [6][64][64] fp32
      __syncthreads();
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int t = 8 * rg + e;
        const uint32_t* src[6] = {x.r, x.w, x.k, x.a, x.b, x.v};
#pragma unroll
        for (int u = 0; u < 6; ++u) {
          raw[(u * 64 + t) * 64 + j0] = bf_lo(src[u][e]);
          raw[(u * 64 + t) * 64 + j0 + 1] = bf_hi(src[u][e]);
        }
      }
      __syncthreads();
      const int i = 16 * wv + n16;
      for (int t = 0; t < n; ++t) {
        float4 rr[4], ww[4], kk[4], aa[4], bb[4];
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
          const int c0 = t * 64 + 16 * jt + 4 * g;
          rr[jt] = *reinterpret_cast<const float4*>(raw + 0 * 4096 + c0);
          ww[jt] = *reinterpret_cast<const float4*>(raw + 1 * 4096 + c0);
          kk[jt] = *reinterpret_cast<const float4*>(raw + 2 * 4096 + c0);
          aa[jt] = *reinterpret_cast<const float4*>(raw + 3 * 4096 + c0);
          bb[jt] = *reinterpret_cast<const float4*>(raw + 4 * 4096 + c0);
        }
        const float vi = raw[5 * 4096 + t * 64 + i];
        float sa = 0.f;
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
          sa = fmaf(S[jt][0], aa[jt].x, sa);
          sa = fmaf(S[jt][1], aa[jt].y, sa);
          sa = fmaf(S[jt][2], aa[jt].z, sa);
          sa = fmaf(S[jt][3], aa[jt].w, sa);
        }
        sa += __shfl_xor(sa, 16);
        sa += __shfl_xor(sa, 32);
        float o = 0.f;
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
          S[jt][0] = fmaf(S[jt][0], ww[jt].x, fmaf(sa, bb[jt].x, vi * kk[jt].x));
          S[jt][1] = fmaf(S[jt][1], ww[jt].y, fmaf(sa, bb[jt].y, vi * kk[jt].y));
          S[jt][2] = fmaf(S[jt][2], ww[jt].z, fmaf(sa, bb[jt].z, vi * kk[jt].z));
          S[jt][3] = fmaf(S[jt][3], ww[jt].w, fmaf(sa, bb[jt].w, vi * kk[jt].w));
          o = fmaf(S[jt][0], rr[jt].x, o);
          o = fmaf(S[jt][1], rr[jt].y, o);
          o = fmaf(S[jt][2], rr[jt].z, o);
          o = fmaf(S[jt][3], rr[jt].w, o);
        }
        o += __shfl_xor(o, 16);
        o += __shfl_xor(o, 32);
        if (g == 0)
          p.o[(static_cast<size_t>(t0 + t) * p.H + h) * kN + i] = o;
      }
      if (ch + 1 < nchunks)
        load_raw(nxt, p, t0 + kChunk, min(kChunk, it.len - (ch + 1) * kChunk),
                 h, rg, jp);
      __syncthreads();
      continue;
    }

    // next chunk's inputs, in flight during the value side
    if (ch + 1 < nchunks)
      load_raw(nxt, p, t0 + kChunk, min(kChunk, it.len - (ch + 1) * kChunk),
               h, rg, jp);

    // ---- value side: wavefront wv, value rows i in [16 wv, 16 wv + 16) ----
    {
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      // state as fp16 operand, scaled
      float m = 0.f;
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) m = abs_max4(S[jt], m);
      float inv_s;
      const float sS = pow2_scale(wave_max(m), &inv_s);
      const f16x8 Sf[2] = {frag8h(S[0], S[1], sS), frag8h(S[2], S[3], sS)};
      const f16x8 Vf[2] = {ldh8(Vt, 16 * wv + n16, 0, g),
                           ldh8(Vt, 16 * wv + n16, 32, g)};
      // X[t][i] = Abar S0^T + A_ak V
      f32x4 X[4];
      float mx = 0.f;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        f32x4 cs = z, cv = z;
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
          cs = mmah(ldh8(Abar, 16 * tt + n16, 32 * kc, g), Sf[kc], cs);
#pragma unroll
        for (int kc = 0; kc <= (tt >> 1); ++kc)
          cv = mmah(ldh8(Aak, 16 * tt + n16, 32 * kc, g), Vf[kc], cv);
#pragma unroll
        for (int r = 0; r < 4; ++r) X[tt][r] = fmaf(cs[r], inv_s, cv[r]);
        mx = abs_max4(X[tt], mx);
      }
      float inv_x;
      const float sX = pow2_scale(wave_max(mx), &inv_x);
      const f16x8 Xf[2] = {frag8h(X[0], X[1], sX), frag8h(X[2], X[3], sX)};
      // U (scaled by sX) = T (X sX)
      f32x4 U[4];
      float mu = 0.f;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        f32x4 c = z;
#pragma unroll
        for (int kc = 0; kc <= (tt >> 1); ++kc)
          c = mmah(ldh8(Tm, 16 * tt + n16, 32 * kc, g), Xf[kc], c);
        U[tt] = c;
        mu = abs_max4(c, mu);
      }
      float inv_u;
      const float sU = pow2_scale(wave_max(mu), &inv_u);
      const float inv_ux = inv_u * inv_x;     // U_true = U_frag * inv_ux
      const f16x8 Uf[2] = {frag8h(U[0], U[1], sU), frag8h(U[2], U[3], sU)};
      // O^T[i][t] = S0 Rbar^T + U^T M_rb^T + V^T M_rk^T
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        f32x4 cs = z, cu = z, cv = z;
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
          cs = mmah(Sf[kc], ldh8(Rbar, 16 * tt + n16, 32 * kc, g), cs);
#pragma unroll
        for (int kc = 0; kc <= (tt >> 1); ++kc) {
          cu = mmah(Uf[kc], ldh8(Mrb, 16 * tt + n16, 32 * kc, g), cu);
          cv = mmah(Vf[kc], ldh8(Mrk, 16 * tt + n16, 32 * kc, g), cv);
        }
        const int t = 16 * tt + n16;
        if (t < n) {
          float4 ov;
          ov.x = fmaf(cs[0], inv_s, fmaf(cu[0], inv_ux, cv[0]));
          ov.y = fmaf(cs[1], inv_s, fmaf(cu[1], inv_ux, cv[1]));
          ov.z = fmaf(cs[2], inv_s, fmaf(cu[2], inv_ux, cv[2]));
          ov.w = fmaf(cs[3], inv_s, fmaf(cu[3], inv_ux, cv[3]));
          *reinterpret_cast<float4*>(p.o + (static_cast<size_t>(t0 + t) * p.H + h) * kN
                                     + 16 * wv + 4 * g) = ov;
        }
      }
      // S^T[j][i] <- Lambda_L[j] S0^T + Bbar^T U + Kbar^T V
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        f32x4 cu = z, cv = z;
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
          cu = mmah(ldh8(BbT, 16 * jt + n16, 32 * kc, g), Uf[kc], cu);
          cv = mmah(ldh8(KbT, 16 * jt + n16, 32 * kc, g), Vf[kc], cv);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
          S[jt][r] = fmaf(LAM[16 * jt + 4 * g + r], S[jt][r],
                          fmaf(cu[r], inv_ux, cv[r]));
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int jt = 0; jt < 4; ++jt)
    *reinterpret_cast<float4*>(sbase + 16 * jt) =
        make_float4(S[jt][0], S[jt][1], S[jt][2], S[jt][3]);
}

}  // namespace

hipError_t launch_chunked_h(const SeqArgs& args, hipStream_t stream) {
  if (args.n_items <= 0) return hipSuccess;
  const int64_t blocks = static_cast<int64_t>(args.n_items) * args.H;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(chunk_h_kernel, dim3(static_cast<unsigned>(blocks)),
                     dim3(256), 0, stream, args);
  return hipGetLastError();
}

}  // namespace wkv7
