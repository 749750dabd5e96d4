// Chunked-prefill WKV-7 kernel for gfx950 (MFMA).
//
// Same operation as the sequential kernel (page "RWKV-X Architecture",
// section "WKV-7 Kernel (Generalized Delta Rule)"; product-form reading
// S_t = S_{t-1}(diag(w_t) + a_t b_t^T) + v_t k_t^T, o_t = S_t r_t), computed
// 64 tokens at a time in the chunked (WY/UT) form. That page names a batched
// forward only as a prefill optimisation; the chunked algebra is derived
// here. Within a chunk starting from S0, with c_t = sum_{u<=t} log2 w_u per
// key channel j and u_t = S_{t-1} a_t:
//
//   U   = T (Abar S0^T + A_ak V),       T = (I - A_ab)^-1 (unit lower)
//   O   = Rbar S0^T + M_rb U + M_rk V
//   S_L = S0 diag(2^c_L) + U^T Bbar + V^T Kbar
//
// Abar_t = a_t 2^c_{t-1}, Rbar_t = r_t 2^c_t, Bbar_s = b_s 2^(c_L - c_s),
// Kbar_s = k_s 2^(c_L - c_s). The four L x L matrices are Gram products of
// operands scaled about the chunk's middle, rho = c_31:
//   A_ab[t][s] = <a_t 2^(c_{t-1}-rho), b_s 2^(rho-c_s)>  for s < t (else 0)
//   A_ak[t][s] = <a_t 2^(c_{t-1}-rho), k_s 2^(rho-c_s)>  for s < t
//   M_rb[t][s] = <r_t 2^(c_t-rho),     b_s 2^(rho-c_s)>  for s <= t
//   M_rk[t][s] = <r_t 2^(c_t-rho),     k_s 2^(rho-c_s)>  for s <= t
// A chunk whose decay from its middle to either end exceeds 2^120 in some
// channel would overflow these scaled operands; such a chunk is run token
// by token instead (exact for any w in (0, 1]).
//
// Work split: one 256-thread workgroup (4 wavefronts) per (sequence, head),
// chunks in order. Key-side quantities (decays, scaled operands, the Gram
// matrices, T) are shared through LDS; the value side is separable by value
// row, so wavefront w owns state rows i in [16w, 16w + 16) and keeps them in
// registers across chunks, in the MFMA accumulator layout of S^T.
//
// Precision: every MFMA operand is split into bf16 hi + lo and a product is
// hi*hi + hi*lo + lo*hi, accumulated in fp32 (v_mfma_f32_16x16x32_bf16);
// a bf16 input operand (V) is exact and needs only hi. All element-wise
// work is fp32.
//
// MFMA fragments (verified lane layout of the 16x16x32 / 16x16x16 bf16
// instructions): lane l = 16 g + n holds operand row n and, for a 32-wide
// k range starting at kb, k = kb + {4g..4g+3, 16+4g..16+4g+3}; the result
// lane holds C[4g + r][n], r = 0..3. With this k order a result pair of
// 16-row tiles is directly the operand fragment of the next product, so
// X -> U -> (O, S) chain in registers.

#include "internal.h"
#include "../../include/wkv7.h"

namespace wkv7 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kChunk = 64;
constexpr int kPitch = 68;                 // bf16 per LDS matrix row (64 + pad)
constexpr int kMat = 64 * kPitch;          // bf16 per matrix
constexpr int kPair = 2 * kMat;            // hi matrix, then lo matrix
constexpr int kRegionBytes = 4 * kPair * 2;  // four pairs
constexpr int kOffG = 0;
constexpr int kOffL = kRegionBytes;
constexpr int kOffV = 2 * kRegionBytes;
constexpr int kOffX = kOffV + kPair * 2;
constexpr int kLdsBytes = kOffX + 256 + 16;
constexpr float kMaxExp2 = 120.f;          // scaled-operand exponent bound

static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
// the sequential path keeps six raw fp32 64x64 inputs in regions G and L
static_assert(6 * 64 * 64 * 4 <= 2 * kRegionBytes, "raw staging");

struct F8 { bf16x8 h, l; };
struct F4 { bf16x4 h, l; };

__device__ __forceinline__ void split(float x, __bf16& h, __bf16& l) {
  h = static_cast<__bf16>(x);
  l = static_cast<__bf16>(x - static_cast<float>(h));
}

__device__ __forceinline__ f32x4 mma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
// split-operand products (small terms first)
__device__ __forceinline__ f32x4 mm3(const F8& p, const F8& q, f32x4 c) {
  c = mma32(p.l, q.h, c);
  c = mma32(p.h, q.l, c);
  return mma32(p.h, q.h, c);
}
__device__ __forceinline__ f32x4 mm3(const F4& p, const F4& q, f32x4 c) {
  c = mma16(p.l, q.h, c);
  c = mma16(p.h, q.l, c);
  return mma16(p.h, q.h, c);
}
// q exact in bf16 (a bf16 input)
__device__ __forceinline__ f32x4 mm2q(const F8& p, bf16x8 q, f32x4 c) {
  c = mma32(p.l, q, c);
  return mma32(p.h, q, c);
}
__device__ __forceinline__ f32x4 mm2p(bf16x8 p, const F8& q, f32x4 c) {
  c = mma32(p, q.l, c);
  return mma32(p, q.h, c);
}

// fragment of rows `row` (= base + n) and k range starting at kb
__device__ __forceinline__ bf16x8 ld8(const __bf16* m, int row, int kb, int g) {
  const __bf16* p = m + row * kPitch + kb + 4 * g;
  bf16x4 a = *reinterpret_cast<const bf16x4*>(p);
  bf16x4 b = *reinterpret_cast<const bf16x4*>(p + 16);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ F8 ldp8(const __bf16* pair, int row, int kb, int g) {
  return F8{ld8(pair, row, kb, g), ld8(pair + kMat, row, kb, g)};
}
__device__ __forceinline__ F4 ldp4(const __bf16* pair, int row, int kb, int g) {
  const int o = row * kPitch + kb + 4 * g;
  return F4{*reinterpret_cast<const bf16x4*>(pair + o),
            *reinterpret_cast<const bf16x4*>(pair + kMat + o)};
}
// operand fragment from two result tiles (k = 4g + r, then 16 + 4g + r)
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
__device__ __forceinline__ F4 frag4(f32x4 t0) {
  F4 f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    __bf16 h, l;
    split(t0[r], h, l); f.h[r] = h; f.l[r] = l;
  }
  return f;
}
// one element of a pair matrix
__device__ __forceinline__ void put(__bf16* pair, int row, int col, float x) {
  __bf16 h, l;
  split(x, h, l);
  pair[row * kPitch + col] = h;
  pair[kMat + row * kPitch + col] = l;
}
// 16 consecutive elements of a pair-matrix row (32-byte aligned)
__device__ __forceinline__ void put16(__bf16* pair, int row, int col,
                                      const float* x) {
  bf16x8 h0, l0, h1, l1;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    __bf16 h, l;
    split(x[e], h, l); h0[e] = h; l0[e] = l;
    split(x[8 + e], h, l); h1[e] = h; l1[e] = l;
  }
  bf16x4* ph = reinterpret_cast<bf16x4*>(pair + row * kPitch + col);
  bf16x4* pl = reinterpret_cast<bf16x4*>(pair + kMat + row * kPitch + col);
  ph[0] = __builtin_shufflevector(h0, h0, 0, 1, 2, 3);
  ph[1] = __builtin_shufflevector(h0, h0, 4, 5, 6, 7);
  ph[2] = __builtin_shufflevector(h1, h1, 0, 1, 2, 3);
  ph[3] = __builtin_shufflevector(h1, h1, 4, 5, 6, 7);
  pl[0] = __builtin_shufflevector(l0, l0, 0, 1, 2, 3);
  pl[1] = __builtin_shufflevector(l0, l0, 4, 5, 6, 7);
  pl[2] = __builtin_shufflevector(l1, l1, 0, 1, 2, 3);
  pl[3] = __builtin_shufflevector(l1, l1, 4, 5, 6, 7);
}
// four consecutive elements (8-byte aligned) of a pair-matrix row
__device__ __forceinline__ void put4(__bf16* pair, int row, int col,
                                     f32x4 x) {
  F4 f = frag4(x);
  *reinterpret_cast<bf16x4*>(pair + row * kPitch + col) = f.h;
  *reinterpret_cast<bf16x4*>(pair + kMat + row * kPitch + col) = f.l;
}

template <int DT> __device__ __forceinline__ float ldx(const void* p, size_t i);
template <> __device__ __forceinline__ float ldx<WKV7_BF16>(const void* p,
                                                           size_t i) {
  return __uint_as_float(
      static_cast<uint32_t>(static_cast<const uint16_t*>(p)[i]) << 16);
}
template <> __device__ __forceinline__ float ldx<WKV7_F32>(const void* p,
                                                          size_t i) {
  return static_cast<const float*>(p)[i];
}

// V^T fragment: exact bf16 for bf16 inputs, split for fp32 inputs.
template <int DT> struct VFrag;
template <> struct VFrag<WKV7_BF16> {
  bf16x8 v;
  __device__ void load(const __bf16* pair, int row, int kb, int g) {
    v = ld8(pair, row, kb, g);
  }
  __device__ f32x4 as_q(const F8& p, f32x4 c) const { return mm2q(p, v, c); }
  __device__ f32x4 as_p(const F8& q, f32x4 c) const { return mm2p(v, q, c); }
};
template <> struct VFrag<WKV7_F32> {
  F8 v;
  __device__ void load(const __bf16* pair, int row, int kb, int g) {
    v = ldp8(pair, row, kb, g);
  }
  __device__ f32x4 as_q(const F8& p, f32x4 c) const { return mm3(p, v, c); }
  __device__ f32x4 as_p(const F8& q, f32x4 c) const { return mm3(v, q, c); }
};

template <int DT>
__global__ __launch_bounds__(256, 1)
void chunk_kernel(SeqArgs p) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[kLdsBytes];
  __bf16* G = reinterpret_cast<__bf16*>(lds + kOffG);
  __bf16* Lr = reinterpret_cast<__bf16*>(lds + kOffL);
  __bf16* Vt = reinterpret_cast<__bf16*>(lds + kOffV);
  float* lamL = reinterpret_cast<float*>(lds + kOffX);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4;
  const int n16 = lane & 15;
  const int item = blockIdx.x / p.H;
  const int h = blockIdx.x - item * p.H;
  if (item >= p.n_items) return;
  const WorkItem it = p.items[item];
  const size_t hstride = static_cast<size_t>(p.H) * kN;

  // this wavefront's state rows, as S^T result tiles:
  // S[jt][r] = S[i = 16 wv + n16][j = 16 jt + 4 g + r]
  float* sbase = p.pool + (static_cast<size_t>(it.slot) * p.H + h) * (kN * kN)
                 + (16 * wv + n16) * kN + 4 * g;
  f32x4 S[4];
#pragma unroll
  for (int jt = 0; jt < 4; ++jt) {
    float4 x = *reinterpret_cast<const float4*>(sbase + 16 * jt);
    S[jt] = f32x4{x.x, x.y, x.z, x.w};
  }

  // element-wise ownership: channel j = lane, rows 16 q .. 16 q + 15
  const int j = lane;
  const int q = wv;

  const int nchunks = (it.len + kChunk - 1) / kChunk;
  for (int ch = 0; ch < nchunks; ++ch) {
    const int t0 = it.tok0 + ch * kChunk;
    const int n = min(kChunk, it.len - ch * kChunk);

    // ---- inputs of this chunk; rows past the end are w = 1, rest 0 ----
    // Every load is issued, rows past the end re-reading the last row, and
    // the padding is selected afterwards: a conditional load becomes a
    // branch, and the compiler then waits for each token's loads before
    // issuing the next token's.
    float xr[16], xw[16], xk[16], xa[16], xb[16], xv[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int t = 16 * q + e;
      const int tc = t < n ? t : n - 1;                 // n >= 1
      const size_t off = (static_cast<size_t>(t0 + tc) * p.H + h) * kN + j;
      xr[e] = ldx<DT>(p.r, off);
      xw[e] = ldx<DT>(p.w, off);
      xk[e] = ldx<DT>(p.k, off);
      xa[e] = ldx<DT>(p.a, off);
      xb[e] = ldx<DT>(p.b, off);
      xv[e] = ldx<DT>(p.v, off);
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const bool pad = 16 * q + e >= n;
      xr[e] = pad ? 0.f : xr[e];
      xw[e] = pad ? 1.f : xw[e];
      xk[e] = pad ? 0.f : xk[e];
      xa[e] = pad ? 0.f : xa[e];
      xb[e] = pad ? 0.f : xb[e];
      xv[e] = pad ? 0.f : xv[e];
    }
    // V^T[i = j][s = 16 q + e]
    put16(Vt, j, 16 * q, xv);

    // ---- c_t = cumulative log2 w, per channel ----
    float c2[16];
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      acc += __log2f(xw[e]);
      c2[e] = acc;
    }
    float* tot = reinterpret_cast<float*>(Lr);   // 4 x 64 floats
    tot[q * 64 + j] = acc;
    __syncthreads();
    const float t0s = tot[j], t1s = tot[64 + j], t2s = tot[128 + j],
                t3s = tot[192 + j];
    const float p01 = t0s + t1s;
    const float p012 = p01 + t2s;
    const float rho = p01;             // c at row 31
    const float cL = p012 + t3s;       // c at row 63
    const float pre = q == 0 ? 0.f : q == 1 ? t0s : q == 2 ? p01 : p012;
    float cp[16];                      // c_{t-1}
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      c2[e] += pre;
      cp[e] = e == 0 ? pre : c2[e - 1];
    }
    if (q == 0) lamL[j] = exp2f(cL);
    const bool far = (-rho > kMaxExp2) || (rho - cL > kMaxExp2);
    const int extreme = __syncthreads_or(q == 0 && far);

    if (extreme) {
      // ---- exact token-by-token path for this chunk ----
      float* raw = reinterpret_cast<float*>(lds);   // [6][64][64] fp32
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int t = 16 * q + e;
        raw[(0 * 64 + t) * 64 + j] = xr[e];
        raw[(1 * 64 + t) * 64 + j] = xw[e];
        raw[(2 * 64 + t) * 64 + j] = xk[e];
        raw[(3 * 64 + t) * 64 + j] = xa[e];
        raw[(4 * 64 + t) * 64 + j] = xb[e];
        raw[(5 * 64 + t) * 64 + j] = xv[e];
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
      __syncthreads();
      continue;
    }

    // ---- Gram operands (scaled about the chunk middle) -> region G ----
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int t = 16 * q + e;
      const float eA = exp2f(cp[e] - rho);
      const float eR = exp2f(c2[e] - rho);
      const float eB = exp2f(rho - c2[e]);
      put(G + 0 * kPair, t, j, xa[e] * eA);   // A-hat[t][j]
      put(G + 1 * kPair, t, j, xr[e] * eR);   // R-hat[t][j]
      put(G + 2 * kPair, t, j, xb[e] * eB);   // B-hat[s][j]
      put(G + 3 * kPair, t, j, xk[e] * eB);   // K-hat[s][j]
    }
    __syncthreads();

    // ---- Gram matrices: wavefront wv computes one of the four ----
    // tile (tt, st), st <= tt, as C[s][t] = <P_s, Q_t>: P = B-hat / K-hat,
    // Q = A-hat / R-hat. wv: 0 A_ab, 1 A_ak, 2 M_rb, 3 M_rk.
    {
      const __bf16* Pm = G + ((wv & 1) ? 3 : 2) * kPair;
      const __bf16* Qm = G + ((wv >= 2) ? 1 : 0) * kPair;
      const bool strict = wv < 2;
      f32x4 gt[10];
      int ti = 0;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
        for (int st = 0; st <= tt; ++st) {
          f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kc = 0; kc < 2; ++kc) {
            F8 P = ldp8(Pm, 16 * st + n16, 32 * kc, g);
            F8 Q = ldp8(Qm, 16 * tt + n16, 32 * kc, g);
            c = mm3(P, Q, c);
          }
          gt[ti++] = c;
        }
      }
      __syncthreads();   // region G free: A_ab goes there
      __bf16* dst = wv == 0 ? G : Lr + (wv - 1) * kPair;
      float* diag = reinterpret_cast<float*>(G + 2 * kPair);  // [4][16][16]
      ti = 0;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
        for (int st = 0; st <= tt; ++st) {
          f32x4 c = gt[ti++];
          const int t = 16 * tt + n16;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int s = 16 * st + 4 * g + r;
            const bool keep = strict ? (s < t) : (s <= t);
            c[r] = keep ? c[r] : 0.f;
          }
          put4(dst, t, 16 * st + 4 * g, c);
          if (wv == 0 && tt == st) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              diag[(tt * 16 + n16) * 16 + 4 * g + r] = c[r];
          }
        }
      }
      // upper tiles read by 32-wide k fragments must be zero: (0,1), (2,3)
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      put4(dst, n16, 16 + 4 * g, z);
      put4(dst, 32 + n16, 48 + 4 * g, z);
    }
    __syncthreads();

    // ---- T = (I - A_ab)^-1 ----
    __bf16* Tm = Lr + 3 * kPair;        // T[t][s]
    __bf16* TmT = G + 1 * kPair;        // T^T[s][t]
    const __bf16* Aab = G;
    {
      const float* diag = reinterpret_cast<const float*>(G + 2 * kPair);
      if (wv == 0) {
        // diagonal blocks D_p = (I - A_pp)^-1 by forward substitution;
        // lane: block p = g, column n16
        const float* Dg = diag + g * 256;
        float d[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float s = (i == n16) ? 1.f : 0.f;
#pragma unroll
          for (int k = 0; k < i; ++k) s = fmaf(Dg[i * 16 + k], d[k], s);
          d[i] = s;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) put(Tm, 16 * g + i, 16 * g + n16, d[i]);
        put16(TmT, 16 * g + n16, 16 * g, d);
      } else {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        if (wv == 1) put4(Tm, n16, 16 + 4 * g, z);
        if (wv == 2) put4(Tm, 32 + n16, 48 + 4 * g, z);
      }
    }
    __syncthreads();
    // T_{p+1,p} = D_{p+1} (A_{p+1,p} D_p)
    if (wv < 3) {
      const int pb = wv;
      F4 Pa = ldp4(Aab, 16 * (pb + 1) + n16, 16 * pb, g);
      F4 Qd = ldp4(TmT, 16 * pb + n16, 16 * pb, g);
      f32x4 y = mm3(Pa, Qd, f32x4{0.f, 0.f, 0.f, 0.f});
      F4 Pd = ldp4(Tm, 16 * (pb + 1) + n16, 16 * (pb + 1), g);
      f32x4 tv = mm3(Pd, frag4(y), f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int r = 0; r < 4; ++r)
        put(Tm, 16 * (pb + 1) + 4 * g + r, 16 * pb + n16, tv[r]);
      put4(TmT, 16 * pb + n16, 16 * (pb + 1) + 4 * g, tv);
    }
    __syncthreads();
    // T_{p+2,p} = D_{p+2} (A_{p+2,p..p+1} T_{p..p+1,p})
    if (wv < 2) {
      const int pb = wv;
      F8 Pa = ldp8(Aab, 16 * (pb + 2) + n16, 16 * pb, g);
      F8 Qt = ldp8(TmT, 16 * pb + n16, 16 * pb, g);
      f32x4 y = mm3(Pa, Qt, f32x4{0.f, 0.f, 0.f, 0.f});
      F4 Pd = ldp4(Tm, 16 * (pb + 2) + n16, 16 * (pb + 2), g);
      f32x4 tv = mm3(Pd, frag4(y), f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int r = 0; r < 4; ++r)
        put(Tm, 16 * (pb + 2) + 4 * g + r, 16 * pb + n16, tv[r]);
      put4(TmT, 16 * pb + n16, 16 * (pb + 2) + 4 * g, tv);
    }
    __syncthreads();
    // T_{3,0} = D_3 (A_{3,0..2} T_{0..2,0})
    if (wv == 0) {
      F8 Pa = ldp8(Aab, 48 + n16, 0, g);
      F8 Qt = ldp8(TmT, n16, 0, g);
      f32x4 y = mm3(Pa, Qt, f32x4{0.f, 0.f, 0.f, 0.f});
      F4 Pa2 = ldp4(Aab, 48 + n16, 32, g);
      F4 Qt2 = ldp4(TmT, n16, 32, g);
      y = mm3(Pa2, Qt2, y);
      F4 Pd = ldp4(Tm, 48 + n16, 48, g);
      f32x4 tv = mm3(Pd, frag4(y), f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int r = 0; r < 4; ++r) put(Tm, 48 + 4 * g + r, n16, tv[r]);
    }
    __syncthreads();

    // ---- value-side operands -> region G ----
    {
      float bt[16], kt[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int t = 16 * q + e;
        put(G + 0 * kPair, t, j, xa[e] * exp2f(cp[e]));   // A-bar[t][j]
        put(G + 1 * kPair, t, j, xr[e] * exp2f(c2[e]));   // R-bar[t][j]
        const float eL = exp2f(cL - c2[e]);
        bt[e] = xb[e] * eL;
        kt[e] = xk[e] * eL;
      }
      put16(G + 2 * kPair, j, 16 * q, bt);                // B-bar^T[j][s]
      put16(G + 3 * kPair, j, 16 * q, kt);                // K-bar^T[j][s]
    }
    __syncthreads();

    // ---- value side: wavefront wv, value rows i in [16 wv, 16 wv + 16) ----
    {
      const __bf16* Abar = G;
      const __bf16* Rbar = G + kPair;
      const __bf16* BbT = G + 2 * kPair;
      const __bf16* KbT = G + 3 * kPair;
      const __bf16* Aak = Lr;
      const __bf16* Mrb = Lr + kPair;
      const __bf16* Mrk = Lr + 2 * kPair;
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      F8 Sf[2] = {frag8(S[0], S[1]), frag8(S[2], S[3])};
      VFrag<DT> Vf[2];
      Vf[0].load(Vt, 16 * wv + n16, 0, g);
      Vf[1].load(Vt, 16 * wv + n16, 32, g);

      // X[t][i] = Abar S0^T + A_ak V
      f32x4 X[4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        f32x4 c = z;
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
          c = mm3(ldp8(Abar, 16 * tt + n16, 32 * kc, g), Sf[kc], c);
#pragma unroll
        for (int kc = 0; kc <= (tt >> 1); ++kc)
          c = Vf[kc].as_q(ldp8(Aak, 16 * tt + n16, 32 * kc, g), c);
        X[tt] = c;
      }
      // U[t][i] = T X
      const F8 Xf[2] = {frag8(X[0], X[1]), frag8(X[2], X[3])};
      f32x4 U[4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        f32x4 c = z;
#pragma unroll
        for (int kc = 0; kc <= (tt >> 1); ++kc)
          c = mm3(ldp8(Tm, 16 * tt + n16, 32 * kc, g), Xf[kc], c);
        U[tt] = c;
      }
      const F8 Uf[2] = {frag8(U[0], U[1]), frag8(U[2], U[3])};
      // O^T[i][t] = S0 Rbar^T + U^T M_rb^T + V^T M_rk^T
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        f32x4 c = z;
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
          c = mm3(Sf[kc], ldp8(Rbar, 16 * tt + n16, 32 * kc, g), c);
#pragma unroll
        for (int kc = 0; kc <= (tt >> 1); ++kc) {
          c = mm3(Uf[kc], ldp8(Mrb, 16 * tt + n16, 32 * kc, g), c);
          c = Vf[kc].as_p(ldp8(Mrk, 16 * tt + n16, 32 * kc, g), c);
        }
        const int t = 16 * tt + n16;
        if (t < n) {
          float* dst = p.o + (static_cast<size_t>(t0 + t) * p.H + h) * kN
                       + 16 * wv + 4 * g;
          *reinterpret_cast<float4*>(dst) = make_float4(c[0], c[1], c[2], c[3]);
        }
      }
      // S^T[j][i] <- 2^cL[j] S0^T + Bbar^T U + Kbar^T V
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        f32x4 c;
#pragma unroll
        for (int r = 0; r < 4; ++r) c[r] = lamL[16 * jt + 4 * g + r] * S[jt][r];
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
          c = mm3(ldp8(BbT, 16 * jt + n16, 32 * kc, g), Uf[kc], c);
          c = Vf[kc].as_q(ldp8(KbT, 16 * jt + n16, 32 * kc, g), c);
        }
        S[jt] = c;
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

hipError_t launch_chunked(const SeqArgs& args, bool precise,
                          hipStream_t stream) {
  if (args.n_items <= 0) return hipSuccess;
  const int64_t blocks = static_cast<int64_t>(args.n_items) * args.H;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (args.dtype == WKV7_BF16 && !precise) return launch_chunked_p(args, stream);
  dim3 grid(static_cast<unsigned>(blocks)), block(256);
  if (args.dtype == WKV7_BF16)
    hipLaunchKernelGGL(chunk_kernel<WKV7_BF16>, grid, block, 0, stream, args);
  else
    hipLaunchKernelGGL(chunk_kernel<WKV7_F32>, grid, block, 0, stream, args);
  return hipGetLastError();
}

}  // namespace wkv7
