// INT8 per-row symmetric quantization and the INT8 matrix product of the
// projections that feed the recurrence (page "RWKV-X Architecture",
// section "INT8 Quantization": each weight row gets the scale max|row|/127
// and codes round(w / scale); the input is quantized once and every output
// row is an integer dot product, rescaled).
//
// Quantization decides integers in float32 exactly as single-precision C
// would (IEEE division, roundf: halves away from zero; an all-zero row has
// scale 0 and codes 0), so codes and scales are reproducible bit for bit.
//
// The product y[b][o] = (sum_i wq[o][i] xq[b][i]) * ws[o] * xs[b] is exact
// int32 accumulation followed by one float32 rescale, in two kernels that
// give the same bits: for more than four tokens a tiled kernel on
// v_mfma_i32_32x32x32_i8 (96 output rows x 128 tokens per workgroup, a
// staging wavefront feeding the tokens' codes into LDS by direct-to-LDS
// loads, the weights streamed into registers; described at the kernel),
// for up to four tokens a stream over the weight codes with packed int8
// dot products.

#include "internal.h"
#include "../../include/wkv7.h"

namespace wkv7 {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));

// ---------------- quantization: one wavefront per row ----------------

template <int DT> struct Elem;
template <> struct Elem<WKV7_F32> {
  typedef float T;
  __device__ static float get(const T* p, int64_t i) { return p[i]; }
  // 8 consecutive values (32 bytes)
  __device__ static void get8(const T* p, float v[8]) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};
template <> struct Elem<WKV7_BF16> {
  typedef uint16_t T;
  __device__ static float get(const T* p, int64_t i) {
    return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
  }
  // 8 consecutive values (16 bytes)
  __device__ static void get8(const T* p, float v[8]) {
    const uint4 a = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};

__device__ __forceinline__ float wave_max_abs(float m) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  return m;
}

__device__ __forceinline__ uint32_t code(float x, float s) {
  const float v = s > 0.f ? roundf(x / s) : 0.f;   // IEEE divide, roundf
  return static_cast<uint32_t>(static_cast<int>(v)) & 0xffu;
}

// One wavefront per row. Rows whose length is a multiple of 8 with 16-byte
// aligned starts (VEC) move 8 values per lane and load; rows of at most
// 4096 such values are read once, all loads issued together, and quantized
// from registers. Other rows take two passes, one value at a time.
constexpr int kMaxCh = 8;        // 8 x 512 = 4096 values per row in registers

template <int DT>
__device__ __forceinline__ void quantize_row_regs(
    const typename Elem<DT>::T* xr, int64_t cols, int8_t* qr, float* srow,
    int lane) {
  using E = Elem<DT>;
  const int nch = static_cast<int>((cols + 511) / 512);
  float v[kMaxCh][8];
  float m = 0.f;
  // every load unconditional, from the row's start where a lane has no
  // values (zeroed afterwards): a conditional load becomes a branch, and the
  // compiler then waits for each load before issuing the next
#pragma unroll
  for (int c = 0; c < kMaxCh; ++c) {
    const int64_t i = 512 * c + 8 * lane;
    const bool ok = c < nch && i < cols;
    E::get8(xr + (ok ? i : 0), v[c]);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[c][e] = ok ? v[c][e] : 0.f;
  }
#pragma unroll
  for (int c = 0; c < kMaxCh; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[c][e]));
  m = wave_max_abs(m);
  const float s = m / 127.0f;                 // IEEE float32 division
  if (lane == 0) *srow = s;
#pragma unroll
  for (int c = 0; c < kMaxCh; ++c) {
    const int64_t i = 512 * c + 8 * lane;
    if (c < nch && i < cols) {
      uint2 packed;
      packed.x = code(v[c][0], s) | code(v[c][1], s) << 8 |
                 code(v[c][2], s) << 16 | code(v[c][3], s) << 24;
      packed.y = code(v[c][4], s) | code(v[c][5], s) << 8 |
                 code(v[c][6], s) << 16 | code(v[c][7], s) << 24;
      *reinterpret_cast<uint2*>(qr + i) = packed;
    }
  }
}

template <int DT, bool VEC>
__global__ __launch_bounds__(256)
void quantize_rows_kernel(const typename Elem<DT>::T* __restrict__ x,
                          int64_t rows, int64_t cols, int8_t* __restrict__ q,
                          float* __restrict__ scale) {
  using E = Elem<DT>;
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const typename E::T* xr = x + row * cols;
  int8_t* qr = q + row * cols;
  if (VEC) {
    quantize_row_regs<DT>(xr, cols, qr, scale + row, lane);
    return;
  }
  float m = 0.f;
  for (int64_t i = lane; i < cols; i += 64) m = fmaxf(m, fabsf(E::get(xr, i)));
  m = wave_max_abs(m);
  const float s = m / 127.0f;                 // IEEE float32 division
  if (lane == 0) scale[row] = s;
  for (int64_t i = lane; i < cols; i += 64)
    qr[i] = static_cast<int8_t>(code(E::get(xr, i), s));
}

// Few rows (the tokens of one step): one 256-thread workgroup per row, the
// four wavefronts taking the row's 512-value chunks in turn (at most two
// each), so that every SIMD works; the wavefront maxima meet in LDS. The
// same maximum (max is exact in any order), division and rounding as the
// one-wavefront kernel, so the same codes and scales.
constexpr int kSplitMaxRows = 1024;    // fewer rows take this kernel

template <int DT>
__global__ __launch_bounds__(256)
void quantize_split_kernel(const typename Elem<DT>::T* __restrict__ x,
                           int64_t rows, int64_t cols, int8_t* __restrict__ q,
                           float* __restrict__ scale) {
  using E = Elem<DT>;
  __shared__ float red[4];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int64_t row = blockIdx.x;
  if (row >= rows) return;
  const typename E::T* xr = x + row * cols;
  int8_t* qr = q + row * cols;
  const int nch = static_cast<int>((cols + 511) / 512);
  float v[2][8];
  float m = 0.f;
  // unconditional loads (see quantize_row_regs)
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int c = wv + 4 * u;
    const int64_t i = 512 * c + 8 * lane;
    const bool ok = c < nch && i < cols;
    E::get8(xr + (ok ? i : 0), v[u]);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[u][e] = ok ? v[u][e] : 0.f;
  }
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[u][e]));
  m = wave_max_abs(m);
  if (lane == 0) red[wv] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = m / 127.0f;                 // IEEE float32 division
  if (threadIdx.x == 0) scale[row] = s;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int c = wv + 4 * u;
    const int64_t i = 512 * c + 8 * lane;
    if (c < nch && i < cols) {
      uint2 packed;
      packed.x = code(v[u][0], s) | code(v[u][1], s) << 8 |
                 code(v[u][2], s) << 16 | code(v[u][3], s) << 24;
      packed.y = code(v[u][4], s) | code(v[u][5], s) << 8 |
                 code(v[u][6], s) << 16 | code(v[u][7], s) << 24;
      *reinterpret_cast<uint2*>(qr + i) = packed;
    }
  }
}

// ---------------- INT8 product on MFMA ----------------

constexpr int kRowsW = 32;       // output rows per compute wavefront
constexpr int kCompW = 3;        // compute wavefronts per workgroup
constexpr int kRowsWG = kRowsW * kCompW;
constexpr int kTokWG = 128;      // tokens per workgroup (4 tiles of 32)
constexpr int kKS = 128;         // k per super-chunk (4 MFMA k-steps of 32)
constexpr int kNBuf = 6;         // LDS token buffers (super-chunks)
constexpr int kWRing = 8;        // weight register ring (super-chunks)
constexpr int kBufBytes = kTokWG * kKS;
typedef int i32x16 __attribute__((ext_vector_type(16)));

// Barrier without a wait on the wavefront's own LDS reads (those in flight
// target a buffer nobody writes before the next barrier); the asm
// statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void plain_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Workgroup: 96 output rows x 128 tokens, 256 threads. Wavefronts 0-2
// compute, 32 rows each, on v_mfma_i32_32x32x32_i8 (four 32 x 32 tiles of
// int32 accumulators); wavefront 3 stages the tokens' codes.
//
// k advances in super-chunks of 128. The staging wavefront copies each
// super-chunk's codes (128 tokens x 128 bytes) from HBM straight into one
// of six LDS buffers (16-byte direct-to-LDS loads, no registers), five
// super-chunks ahead, and before each step's barrier waits for the
// super-chunk two ahead; the compute wavefronts may therefore read the
// next super-chunk's first fragments before that barrier, and their LDS
// reads run one k-step ahead of the MFMAs throughout. Each compute
// wavefront streams its 32 weight rows through a ring of eight
// super-chunk register buffers (loads seven super-chunks ahead). Every
// load is issued whether or not its super-chunk exists (past the end:
// zeros or unused), so within each role the compiler's count of loads in
// flight is exact and each wait covers only the load it needs.
//
// LDS layout of a buffer: token r's 16-byte chunk c (k = 16 c .. 16 c + 15
// of the super-chunk) sits at r * 128 + 16 (c ^ (r & 7)): the eight tokens
// read together by a quarter wavefront then hit eight different bank
// groups, and each direct-to-LDS load (lane i to byte 16 i) still covers
// eight whole token rows.
//
// MFMA operands: lane 32 h + n supplies row n of its operand with 16 bytes
// for k = kb + 16 h .. kb + 16 h + 15 (the same k assignment for both
// operands); accumulator register a of lane 32 h + n holds
// C[8 (a / 4) + 4 h + a % 4][n].
__global__ __launch_bounds__(256, 1)
void q8_matmul_kernel(const int8_t* __restrict__ wq,
                      const float* __restrict__ ws, int64_t O, int64_t I,
                      const int8_t* __restrict__ xq,
                      const float* __restrict__ xs, int64_t B,
                      float* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) int8_t xl[kNBuf * kBufBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t b0 = static_cast<int64_t>(blockIdx.y) * kTokWG;
  const int64_t n_sc = (I + kKS - 1) / kKS;   // I % 64 == 0
  // Loads go through buffer resources sized to the arrays: a token past B
  // or a row past O reads as zeros (or, past 2^32 bytes of offset, codes
  // of other rows and tokens, whose results are never stored); k past I
  // is zero on the weight side, so whatever the token side reads there
  // adds 0.
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(xq), 0, static_cast<int>(B * I), 0x00020000);
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(wq), 0, static_cast<int>(O * I), 0x00020000);

  if (wv == kCompW) {
    // ---- staging wavefront ----
    // load q (0..15) of a super-chunk fills buffer rows 8 q .. 8 q + 7;
    // lane i: row 8 q + i / 8, position i % 8, so chunk (i % 8) ^ (i / 8)
    // (offsets are 32-bit unsigned: past 2^32 they wrap, see above)
    const int pr = lane >> 3;
    const int ch = (lane & 7) ^ pr;
    const uint32_t xo = static_cast<uint32_t>((b0 + pr) * I) + 16u * ch;
    const uint32_t qstride = static_cast<uint32_t>(8 * I);
    auto fill = [&](int64_t sc) {
      int8_t* buf = xl + static_cast<int>(sc % kNBuf) * kBufBytes;
      const uint32_t ko = xo + static_cast<uint32_t>(sc * kKS);
#pragma unroll
      for (int q = 0; q < 16; ++q)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            xres, (__attribute__((address_space(3))) void*)(buf + 1024 * q), 16,
            static_cast<int>(ko + q * qstride), 0, 0, 0);
    };
    // super-chunks 0 .. kNBuf - 2 in flight; 0 and 1 complete before the
    // first barrier (16 loads per super-chunk, counted in order)
#pragma unroll
    for (int c = 0; c < kNBuf - 1; ++c) fill(c);
    __builtin_amdgcn_s_waitcnt(0x0F70 | (((kNBuf - 3) * 16) & 15) |
                               ((((kNBuf - 3) * 16) >> 4) << 14));
    plain_barrier();
    for (int64_t sc = 0; sc < n_sc; ++sc) {
      // buffer (sc - 1) % kNBuf was read in the step before, which every
      // compute wavefront has left
      fill(sc + kNBuf - 1);
      // super-chunk sc + 2 complete (sc + 3 .. sc + kNBuf - 1 in flight)
      __builtin_amdgcn_s_waitcnt(0x0F70 | (((kNBuf - 3) * 16) & 15) |
                                 ((((kNBuf - 3) * 16) >> 4) << 14));
      plain_barrier();
    }
    // the last loads (past the end, never read) have landed before the
    // compute wavefronts reuse the buffers for their outputs
    __builtin_amdgcn_s_waitcnt(0x0F70);
    plain_barrier();
    return;
  }

  // ---- compute wavefronts ----
  const int h = lane >> 5;
  const int n = lane & 31;
  const int64_t o0 = static_cast<int64_t>(blockIdx.x) * kRowsWG + kRowsW * wv;
  // weight fragment of k-step j: bytes kb + 32 j + 16 h of row o0 + n
  const uint32_t woff = static_cast<uint32_t>((o0 + n) * I) + 16u * h;
  const uint32_t wend = static_cast<uint32_t>(O * I);
  auto load_w = [&](i32x4 (&w)[4], int64_t sc) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t k = sc * kKS + 32 * j;
      const uint32_t off = k < I ? woff + static_cast<uint32_t>(k) : wend;
      w[j] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(
          wres, static_cast<int>(off), 0, 0));
    }
  };
  // token fragment of tile t, k-step j: token 32 t + n, chunk 2 j + h
  auto read_x = [&](i32x4 (&x)[4], int64_t sc, int j) {
    const int8_t* buf = xl + static_cast<int>(sc % kNBuf) * kBufBytes;
#pragma unroll
    for (int t = 0; t < 4; ++t)
      x[t] = *reinterpret_cast<const i32x4*>(
          buf + (32 * t + n) * kKS + 16 * ((2 * j + h) ^ (n & 7)));
  };

  i32x16 acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = i32x16{};
  i32x4 xa[4], xb[4];
  // one super-chunk: load the weights kWRing - 1 super-chunks ahead into
  // wn (the slot freed by the super-chunk before), then four k-steps, each
  // reading the next k-step's token fragments before its MFMAs
  auto step = [&](int64_t sc, i32x4 (&wc)[4], i32x4 (&wn)[4]) {
    load_w(wn, sc + kWRing - 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      i32x4 (&cur)[4] = (j & 1) ? xb : xa;
      i32x4 (&nxt)[4] = (j & 1) ? xa : xb;
      if (j < 3) read_x(nxt, sc, j + 1);
      else read_x(nxt, sc + 1, 0);        // complete since the last barrier
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < 4; ++t)
        acc[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wc[j], cur[t], acc[t], 0, 0, 0);
      // keeps each accumulator in its own AGPRs; one pin per k-step, since
      // an asm statement also bounds instruction scheduling
      asm volatile("" : "+a"(acc[0]), "+a"(acc[1]), "+a"(acc[2]), "+a"(acc[3]));
    }
    plain_barrier();
  };

  i32x4 w0[4], w1[4], w2[4], w3[4], w4[4], w5[4], w6[4], w7[4];
  load_w(w0, 0);
  load_w(w1, 1);
  load_w(w2, 2);
  load_w(w3, 3);
  load_w(w4, 4);
  load_w(w5, 5);
  load_w(w6, 6);
  plain_barrier();                          // super-chunks 0 and 1 staged
  read_x(xa, 0, 0);
  int64_t sc = 0;
  for (; sc + kWRing <= n_sc; sc += kWRing) {
    step(sc, w0, w7);
    step(sc + 1, w1, w0);
    step(sc + 2, w2, w1);
    step(sc + 3, w3, w2);
    step(sc + 4, w4, w3);
    step(sc + 5, w5, w4);
    step(sc + 6, w6, w5);
    step(sc + 7, w7, w6);
  }
  if (sc < n_sc) step(sc, w0, w7);
  if (sc + 1 < n_sc) step(sc + 1, w1, w0);
  if (sc + 2 < n_sc) step(sc + 2, w2, w1);
  if (sc + 3 < n_sc) step(sc + 3, w3, w2);
  if (sc + 4 < n_sc) step(sc + 4, w4, w3);
  if (sc + 5 < n_sc) step(sc + 5, w5, w4);
  if (sc + 6 < n_sc) step(sc + 6, w6, w5);

  plain_barrier();                          // staging loads all landed

  // Outputs, one 32 x 32 tile at a time through this wavefront's own LDS
  // region (rows of 36 floats, so the quarter-wavefront writes hit eight
  // bank groups): lane (h, n), register 4 q + r of tile t holds row
  // o0 + 8 q + 4 h + r, token b0 + 32 t + n. Written to LDS as [token][row],
  // read back as 16-byte row chunks, so that each store instruction writes
  // eight whole 128-byte output rows. Rescaled on the way in, with the same
  // expression as the matrix-vector kernel (equal bits).
  constexpr int kTP = 36;
  float* tl = reinterpret_cast<float*>(xl) + wv * (32 * kTP);
  float4 wsc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t o = o0 + 8 * q + 4 * h;    // rows in fours, all below O or none
    wsc[q] = o < O ? *reinterpret_cast<const float4*>(ws + o)
                   : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const int rn = lane >> 3;                  // read-back: token rn + 8 e
  const int rc = lane & 7;                   // 16-byte chunk: rows 4 rc .. + 3
  const bool row_ok = o0 + 4 * rc < O;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int64_t bw = b0 + 32 * t + n;
    const float sx = bw < B ? xs[bw] : 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float4 v;
      v.x = static_cast<float>(acc[t][4 * q + 0]) * (wsc[q].x * sx);
      v.y = static_cast<float>(acc[t][4 * q + 1]) * (wsc[q].y * sx);
      v.z = static_cast<float>(acc[t][4 * q + 2]) * (wsc[q].z * sx);
      v.w = static_cast<float>(acc[t][4 * q + 3]) * (wsc[q].w * sx);
      *reinterpret_cast<float4*>(tl + n * kTP + 8 * q + 4 * h) = v;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float4 v = *reinterpret_cast<const float4*>(tl + (rn + 8 * e) * kTP + 4 * rc);
      const int64_t b = b0 + 32 * t + rn + 8 * e;
      if (row_ok && b < B)
        *reinterpret_cast<float4*>(y + b * O + o0 + 4 * rc) = v;
    }
  }
}

// ---------------- few tokens: matrix-vector form ----------------
//
// With at most kGemvMaxB tokens the product is a stream over the weight
// codes: one wavefront per kGemvRows output rows, each lane taking 16 bytes
// of every row per 1024-byte chunk of k (two chunks of all rows per pass,
// their loads issued together),
// packed int8 dot products into int32, then a wavefront sum per (token,
// row). The sums are exact, so the result equals the tiled kernel's bit for
// bit.

constexpr int kGemvRows = 8;     // output rows per wavefront (O % 16 == 0)
constexpr int kGemvMaxB = 4;     // tokens handled this way

// sum over the wavefront; the result is wavefront-uniform
__device__ __forceinline__ int wave_sum_i32(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false);   // lane ^ 1
  x += __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);   // lane ^ 2
  x += __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false);  // 7 - l in 8
  x += __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, false);  // 15 - l in 16
  return __builtin_amdgcn_readlane(x, 0) + __builtin_amdgcn_readlane(x, 16) +
         __builtin_amdgcn_readlane(x, 32) + __builtin_amdgcn_readlane(x, 48);
}

template <int NB>
__global__ __launch_bounds__(256)
void q8_gemv_kernel(const int8_t* __restrict__ wq,
                    const float* __restrict__ ws, int64_t O, int64_t I,
                    const int8_t* __restrict__ xq,
                    const float* __restrict__ xs, float* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int64_t o0 = wave * kGemvRows;
  if (o0 >= O) return;                     // O % 16 == 0: all rows or none
  // the scales go out first, so the end does not wait on a fresh load
  const float wsl = ws[o0 + (lane & (kGemvRows - 1))];   // lane r: row r's scale
  float sxb[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) sxb[b] = xs[b];
  int acc[NB][kGemvRows];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int r = 0; r < kGemvRows; ++r) acc[b][r] = 0;
  // two 1024-byte chunks of every row per pass, all loads issued before the
  // first dot product (the scheduling barrier keeps them together)
  for (int64_t c0 = 0; c0 < I; c0 += 2048) {
    // unconditional loads (a lane past the row reads from the row's start
    // and its token codes are then zeroed): a conditional load becomes a
    // branch, and the compiler then waits for every load in flight
    i32x4 w[2][kGemvRows], x[2][NB];
    bool ok[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t k = c0 + 1024 * h + 16 * lane;
      ok[h] = k < I;                         // I % 64 == 0: whole 16-byte groups
      const int64_t kl = ok[h] ? k : 0;
#pragma unroll
      for (int r = 0; r < kGemvRows; ++r)
        w[h][r] = *reinterpret_cast<const i32x4*>(wq + (o0 + r) * I + kl);
#pragma unroll
      for (int b = 0; b < NB; ++b)
        x[h][b] = *reinterpret_cast<const i32x4*>(xq + b * I + kl);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int b = 0; b < NB; ++b)
        if (!ok[h]) x[h][b] = i32x4{0, 0, 0, 0};
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < kGemvRows; ++r)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            acc[b][r] = __builtin_amdgcn_sdot4(w[h][r][q], x[h][b][q], acc[b][r], false);
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    float mine = 0.f;                      // lane r: row r's sum
#pragma unroll
    for (int r = 0; r < kGemvRows; ++r) {
      const float sum = static_cast<float>(wave_sum_i32(acc[b][r]));
      mine = lane == r ? sum : mine;
    }
    if (lane < kGemvRows) y[b * O + o0 + lane] = mine * (wsl * sxb[b]);
  }
}

// Quantize and multiply in one launch, for few tokens with in <= 2048.
// A workgroup's four wavefronts (32 output rows) each load a quarter of
// every input row (8 values per lane), then start their weight loads; the
// wait counter drains in issue order, so waiting for the inputs leaves the
// weight stream in flight, and the quantization runs under it. The
// quarters' maxima meet in LDS (the maximum of a set does not depend on the
// order: it is the row's, as in quantize_rows_kernel), each lane codes its
// 8 values with the row's scale exactly as quantize_rows_kernel does, and
// the codes meet in LDS for the matrix-vector product. The first workgroup
// also stores the codes and scales. Same codes, same integer sums, same
// rescale: the same bits as the two separate launches.
constexpr int64_t kFusedMaxI = 2048;

template <int DT, int NB>
__global__ __launch_bounds__(256)
void q8_linear_kernel(const int8_t* __restrict__ wq,
                      const float* __restrict__ ws, int64_t O, int64_t I,
                      const typename Elem<DT>::T* __restrict__ x,
                      int8_t* __restrict__ xq, float* __restrict__ xs,
                      float* __restrict__ y) {
  using E = Elem<DT>;
  using T = typename E::T;
  constexpr int kLd = static_cast<int>(8 * sizeof(T) / 16);  // 16-byte loads
  __shared__ float part[4][NB];
  __shared__ __align__(16) uint8_t codes[NB][kFusedMaxI];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int64_t o0 = (static_cast<int64_t>(blockIdx.x) * 4 + wv) * kGemvRows;
  // O % 16 == 0: a wavefront has all its rows or none; one with none still
  // takes part in the quantization and reads a valid block of rows
  const bool rows_ok = o0 < O;
  const int64_t oc = rows_ok ? o0 : O - kGemvRows;
  // the wavefront's quarter of each input row (I % 64 == 0: a lane's 8
  // values lie wholly inside or wholly outside the row)
  const int kq = 512 * wv + 8 * lane;
  const bool in_ok = kq < I;
  const int64_t kql = in_ok ? kq : 0;
  i32x4 raw[NB][kLd];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int u = 0; u < kLd; ++u)
      raw[b][u] = reinterpret_cast<const i32x4*>(x + b * I + kql)[u];
  // weights, unconditionally (a lane past the row reads its start: its
  // codes are zero, so those products vanish); a conditional load would
  // become a branch, and the compiler then waits for every load
  i32x4 w[2][kGemvRows];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int64_t k = 1024 * h + 16 * lane;
    const int64_t kl = k < I ? k : 0;
#pragma unroll
    for (int r = 0; r < kGemvRows; ++r)
      w[h][r] = *reinterpret_cast<const i32x4*>(wq + (oc + r) * I + kl);
  }
  const float wsl = ws[oc + (lane & (kGemvRows - 1))];   // lane r: row r's scale
  __builtin_amdgcn_sched_barrier(0);       // every load goes out first
  float v[NB][8];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    E::get8(reinterpret_cast<const T*>(raw[b]), v[b]);
    float m = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[b][e] = in_ok ? v[b][e] : 0.f;
      m = fmaxf(m, fabsf(v[b][e]));
    }
    m = wave_max_abs(m);
    if (lane == 0) part[wv][b] = m;
  }
  lds_barrier();
  float sx[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const float m = fmaxf(fmaxf(part[0][b], part[1][b]), fmaxf(part[2][b], part[3][b]));
    const float sc = m / 127.0f;           // IEEE float32 division
    sx[b] = sc;
    uint2 c;
    c.x = code(v[b][0], sc) | code(v[b][1], sc) << 8 | code(v[b][2], sc) << 16 |
          code(v[b][3], sc) << 24;
    c.y = code(v[b][4], sc) | code(v[b][5], sc) << 8 | code(v[b][6], sc) << 16 |
          code(v[b][7], sc) << 24;
    *reinterpret_cast<uint2*>(&codes[b][kq]) = c;
    if (blockIdx.x == 0) {
      if (in_ok) *reinterpret_cast<uint2*>(xq + b * I + kq) = c;
      if (threadIdx.x == 0) xs[b] = sc;
    }
  }
  lds_barrier();
  int acc[NB][kGemvRows];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    i32x4 xc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
      xc[h] = *reinterpret_cast<const i32x4*>(&codes[b][1024 * h + 16 * lane]);
#pragma unroll
    for (int r = 0; r < kGemvRows; ++r) {
      int a = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          a = __builtin_amdgcn_sdot4(w[h][r][q], xc[h][q], a, false);
      acc[b][r] = a;
    }
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    float mine = 0.f;                      // lane r: row r's sum
#pragma unroll
    for (int r = 0; r < kGemvRows; ++r) {
      const float sum = static_cast<float>(wave_sum_i32(acc[b][r]));
      mine = lane == r ? sum : mine;
    }
    if (rows_ok && lane < kGemvRows) y[b * O + o0 + lane] = mine * (wsl * sx[b]);
  }
}

}  // namespace

hipError_t launch_q8_quantize(const void* x, int dtype, int64_t rows,
                              int64_t cols, int8_t* q, float* scale,
                              hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  const int64_t blocks = (rows + 3) / 4;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  dim3 grid(static_cast<unsigned>(blocks)), block(256);
  // 8 values per lane, the whole row in registers: whole 16-byte groups on
  // every row and at most 4096 values
  const size_t esz = dtype == WKV7_BF16 ? 2 : 4;
  const bool vec = cols % 8 == 0 && cols <= 512 * kMaxCh &&
                   reinterpret_cast<uintptr_t>(x) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(q) % 8 == 0 &&
                   (cols * esz) % 16 == 0;
  if (vec && rows < kSplitMaxRows) {
    const dim3 g1(static_cast<unsigned>(rows));
    if (dtype == WKV7_BF16)
      hipLaunchKernelGGL((quantize_split_kernel<WKV7_BF16>), g1, block, 0, stream,
                         static_cast<const uint16_t*>(x), rows, cols, q, scale);
    else
      hipLaunchKernelGGL((quantize_split_kernel<WKV7_F32>), g1, block, 0, stream,
                         static_cast<const float*>(x), rows, cols, q, scale);
    return hipGetLastError();
  }
  if (dtype == WKV7_BF16) {
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    if (vec) hipLaunchKernelGGL((quantize_rows_kernel<WKV7_BF16, true>), grid, block, 0, stream, xb, rows, cols, q, scale);
    else hipLaunchKernelGGL((quantize_rows_kernel<WKV7_BF16, false>), grid, block, 0, stream, xb, rows, cols, q, scale);
  } else {
    const float* xf = static_cast<const float*>(x);
    if (vec) hipLaunchKernelGGL((quantize_rows_kernel<WKV7_F32, true>), grid, block, 0, stream, xf, rows, cols, q, scale);
    else hipLaunchKernelGGL((quantize_rows_kernel<WKV7_F32, false>), grid, block, 0, stream, xf, rows, cols, q, scale);
  }
  return hipGetLastError();
}

hipError_t launch_q8_matmul(const int8_t* wq, const float* ws, int64_t O,
                            int64_t I, const int8_t* xq, const float* xs,
                            int64_t B, float* y, hipStream_t stream) {
  if (O <= 0 || B <= 0) return hipSuccess;
  if (B <= kGemvMaxB) {
    const int64_t blocks = (O / kGemvRows + 3) / 4;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    const dim3 grid(static_cast<unsigned>(blocks)), block(256);
    switch (B) {
      case 1: hipLaunchKernelGGL(q8_gemv_kernel<1>, grid, block, 0, stream, wq, ws, O, I, xq, xs, y); break;
      case 2: hipLaunchKernelGGL(q8_gemv_kernel<2>, grid, block, 0, stream, wq, ws, O, I, xq, xs, y); break;
      case 3: hipLaunchKernelGGL(q8_gemv_kernel<3>, grid, block, 0, stream, wq, ws, O, I, xq, xs, y); break;
      default: hipLaunchKernelGGL(q8_gemv_kernel<4>, grid, block, 0, stream, wq, ws, O, I, xq, xs, y); break;
    }
    return hipGetLastError();
  }
  const int64_t gx = (O + kRowsWG - 1) / kRowsWG;
  const int64_t gy = (B + kTokWG - 1) / kTokWG;
  if (gx > 0x7fffffff || gy > 65535) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(q8_matmul_kernel,
                     dim3(static_cast<unsigned>(gx), static_cast<unsigned>(gy)),
                     dim3(64 * (kCompW + 1)), 0, stream, wq, ws, O, I, xq, xs, B, y);
  return hipGetLastError();
}

hipError_t launch_q8_linear(const int8_t* wq, const float* ws, int64_t O,
                            int64_t I, const void* x, int dtype, int64_t B,
                            int8_t* xq, float* xs, float* y,
                            hipStream_t stream) {
  if (O <= 0 || B <= 0) return hipSuccess;
  const bool fused = B <= kGemvMaxB && I <= kFusedMaxI &&
                     reinterpret_cast<uintptr_t>(x) % 16 == 0;
  if (!fused) {
    hipError_t e = launch_q8_quantize(x, dtype, B, I, xq, xs, stream);
    if (e != hipSuccess) return e;
    return launch_q8_matmul(wq, ws, O, I, xq, xs, B, y, stream);
  }
  const int64_t blocks = (O / kGemvRows + 3) / 4;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(blocks)), block(256);
#define WKV7_Q8_LINEAR(DT, NB)                                                  \
  hipLaunchKernelGGL((q8_linear_kernel<DT, NB>), grid, block, 0, stream, wq,     \
                     ws, O, I, static_cast<const typename Elem<DT>::T*>(x), xq,  \
                     xs, y)
  if (dtype == WKV7_BF16) {
    switch (B) {
      case 1: WKV7_Q8_LINEAR(WKV7_BF16, 1); break;
      case 2: WKV7_Q8_LINEAR(WKV7_BF16, 2); break;
      case 3: WKV7_Q8_LINEAR(WKV7_BF16, 3); break;
      default: WKV7_Q8_LINEAR(WKV7_BF16, 4); break;
    }
  } else {
    switch (B) {
      case 1: WKV7_Q8_LINEAR(WKV7_F32, 1); break;
      case 2: WKV7_Q8_LINEAR(WKV7_F32, 2); break;
      case 3: WKV7_Q8_LINEAR(WKV7_F32, 3); break;
      default: WKV7_Q8_LINEAR(WKV7_F32, 4); break;
    }
  }
#undef WKV7_Q8_LINEAR
  return hipGetLastError();
}

}  // namespace wkv7
