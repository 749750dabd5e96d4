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
// The product y[b][o] = (sum_i wq[o][i] xq[b][i]) * ws[o] * xs[b] runs on
// v_mfma_i32_16x16x64_i8 with exact int32 accumulation. A workgroup of 4 to
// 8 wavefronts owns 16 output rows per wavefront and up to 128 tokens; the
// launch takes the fewest wavefronts that put the grid on the CUs in one
// round (otherwise four, two workgroups per CU). k advances in super-chunks
// of 256: the tokens' codes go through two LDS buffers (staged by the first
// four wavefronts; the next super-chunk's codes are loaded while the
// current one is multiplied, one barrier per super-chunk), and each
// wavefront streams its 16 weight rows through a ring of four super-chunk
// register buffers, loaded three super-chunks ahead, reusing each fragment
// for 8 token tiles. The weight codes are read from HBM once per token
// block. A k-step's eight token fragments are read from LDS together before
// its MFMAs, so their latencies overlap.
//
// MFMA operands: lane 16 g + n supplies row n of its operand with 16 bytes
// for k = kb + 16 g .. kb + 16 g + 15 (the same k assignment for both
// operands, so the sum is over every k once); the result lane holds
// C[4 g + r][n].

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
#pragma unroll
  for (int c = 0; c < kMaxCh; ++c) {
    const int64_t i = 512 * c + 8 * lane;
    if (c < nch && i < cols) {
      E::get8(xr + i, v[c]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[c][e] = 0.f;
    }
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

// ---------------- INT8 product on MFMA ----------------

constexpr int kTokWG = 128;      // tokens per workgroup (8 tiles of 16)
constexpr int kKS = 256;         // k per super-chunk (4 MFMA k-steps)
constexpr int kWD = 3;           // weight prefetch distance (super-chunks)
constexpr int kPitch = kKS + 16; // LDS bytes per token row (padded)

// blockDim.x = 64 W for W = 4..8 wavefronts (16 output rows each): the
// launch picks W so that the grid fits the CUs in one round when it can.
__global__ __launch_bounds__(512, 1)
void q8_matmul_kernel(const int8_t* __restrict__ wq,
                      const float* __restrict__ ws, int64_t O, int64_t I,
                      const int8_t* __restrict__ xq,
                      const float* __restrict__ xs, int64_t B,
                      float* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) int8_t xl[2][kTokWG * kPitch];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int g = lane >> 4;
  const int n = lane & 15;
  const int64_t o0 = static_cast<int64_t>(blockIdx.x) * (blockDim.x >> 2) + 16 * wv;
  const bool stager = tid < 256;           // the first four wavefronts stage
  const int64_t b0 = static_cast<int64_t>(blockIdx.y) * kTokWG;
  const bool rows_ok = o0 < O;             // O % 16 == 0: all 16 rows or none
  // Loads go through buffer resources sized to the arrays: a token past B or
  // a row past O reads as zeros, with no branch. k-steps past I are zeroed
  // on the weight side, so whatever the token side reads there adds 0.
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(xq), 0, static_cast<int>(B * I), 0x00020000);
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(wq), 0, static_cast<int>(O * I), 0x00020000);
  // staging: thread t copies 16 bytes of tokens 16 e + t / 16 (e = 0..7) at
  // k offset 16 (t % 16): each load instruction covers four whole 256-byte
  // token rows of the super-chunk
  const int st_tok = tid >> 4;
  const int st_off = 16 * (tid & 15);
  const int xoff = static_cast<int>((b0 + st_tok) * I) + st_off;
  const int xstride = static_cast<int>(16 * I);         // 16 tokens
  // weight fragment of k-step j: bytes kb + 64 j + 16 g of row o0 + n
  const int woff = static_cast<int>((o0 + n) * I) + 16 * g;
  const int64_t n_sc = (I + kKS - 1) / kKS;    // I % 64 == 0

  i32x4 acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = i32x4{0, 0, 0, 0};

  i32x4 xr[8];
  auto load_x = [&](int64_t kb) {
    if (!stager) return;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      xr[e] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(
          xres, xoff + static_cast<int>(kb) + xstride * e, 0, 0));
  };
  auto store_x = [&](int buf) {
    if (!stager) return;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      *reinterpret_cast<i32x4*>(&xl[buf][(16 * e + st_tok) * kPitch + st_off]) =
          xr[e];
  };

  // the wavefront's weight fragments of one super-chunk (its 16 rows, 256
  // k): k-steps past I are zero
  auto load_w = [&](i32x4 (&w)[4], int64_t sc) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t k = sc * kKS + 64 * j;
      const i32x4 v = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(
          wres, woff + static_cast<int>(k), 0, 0));
      w[j] = k < I ? v : i32x4{0, 0, 0, 0};
    }
  };
  // one super-chunk: multiply with weights wc, load the weights of the
  // super-chunk kWD ahead into wn (the ring slot freed by the one before),
  // stage the next tokens' codes and load the ones after
  auto step = [&](int64_t sc, i32x4 (&wc)[4], i32x4 (&wn)[4]) {
    if (sc >= n_sc) return;
    if (sc + kWD < n_sc) load_w(wn, sc + kWD);
    const int buf = static_cast<int>(sc & 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // the k-step's eight token fragments are read together, so their LDS
      // latencies overlap, then multiplied
      i32x4 xf[8];
#pragma unroll
      for (int t = 0; t < 8; ++t)
        xf[t] = *reinterpret_cast<const i32x4*>(
            &xl[buf][(16 * t + n) * kPitch + 64 * j + 16 * g]);
#pragma unroll
      for (int t = 0; t < 8; ++t)
        acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wc[j], xf[t], acc[t], 0, 0, 0);
      // keeps each accumulator in its own AGPRs (without it the compiler
      // rotates all 32 accumulator registers every pass); one pin per
      // k-step, since an asm statement also bounds instruction scheduling
      asm volatile("" : "+a"(acc[0]), "+a"(acc[1]), "+a"(acc[2]), "+a"(acc[3]),
                        "+a"(acc[4]), "+a"(acc[5]), "+a"(acc[6]), "+a"(acc[7]));
    }
    if (sc + 1 < n_sc) {
      store_x(buf ^ 1);                     // buffer read two steps ago
      if (sc + 2 < n_sc) load_x((sc + 2) * kKS);
      lds_barrier();                        // loads stay in flight
    }
  };

  i32x4 w0[4], w1[4], w2[4], w3[4];
  load_x(0);
  load_w(w0, 0);
  if (n_sc > 1) load_w(w1, 1);
  if (n_sc > 2) load_w(w2, 2);
  store_x(0);
  if (n_sc > 1) load_x(kKS);
  lds_barrier();                            // super-chunk 0 staged
  for (int64_t sc = 0; sc < n_sc; sc += kWD + 1) {
    step(sc, w0, w3);
    step(sc + 1, w1, w0);
    step(sc + 2, w2, w1);
    step(sc + 3, w3, w2);
  }
  if (!rows_ok) return;
  // lane (g, n) of tile t: rows o0 + 4 g + r, token b0 + 16 t + n
  const float4 wsc = *reinterpret_cast<const float4*>(ws + o0 + 4 * g);
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int64_t b = b0 + 16 * t + n;
    if (b >= B) continue;
    const float sx = xs[b];
    float4 out;
    out.x = static_cast<float>(acc[t][0]) * (wsc.x * sx);
    out.y = static_cast<float>(acc[t][1]) * (wsc.y * sx);
    out.z = static_cast<float>(acc[t][2]) * (wsc.z * sx);
    out.w = static_cast<float>(acc[t][3]) * (wsc.w * sx);
    *reinterpret_cast<float4*>(y + b * O + o0 + 4 * g) = out;
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
  int acc[NB][kGemvRows];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int r = 0; r < kGemvRows; ++r) acc[b][r] = 0;
  // two 1024-byte chunks of every row per pass, all loads issued before the
  // first dot product (the scheduling barrier keeps them together)
  for (int64_t c0 = 0; c0 < I; c0 += 2048) {
    i32x4 w[2][kGemvRows], x[2][NB];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t k = c0 + 1024 * h + 16 * lane;
      const bool ok = k < I;                 // I % 64 == 0: whole 16-byte groups
#pragma unroll
      for (int r = 0; r < kGemvRows; ++r)
        w[h][r] = ok ? *reinterpret_cast<const i32x4*>(wq + (o0 + r) * I + k)
                     : i32x4{0, 0, 0, 0};
#pragma unroll
      for (int b = 0; b < NB; ++b)
        x[h][b] = ok ? *reinterpret_cast<const i32x4*>(xq + b * I + k)
                     : i32x4{0, 0, 0, 0};
    }
    __builtin_amdgcn_sched_barrier(0);
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
    const float sx = xs[b];
#pragma unroll
    for (int r = 0; r < kGemvRows; ++r) {
      const int sum = wave_sum_i32(acc[b][r]);
      if (lane == r)
        y[b * O + o0 + r] = static_cast<float>(sum) * (ws[o0 + r] * sx);
    }
  }
}

// Quantize and multiply in one launch, for few tokens with in <= 2048:
// every wavefront starts its weight loads, then quantizes the inputs'
// values at its lanes' k positions exactly as quantize_rows_kernel does
// (the wavefront covers the whole row, so its maximum is the row's), and
// runs the matrix-vector product on those codes. The first wavefront also
// stores the codes and scales. Same codes, same integer sums, same rescale:
// the same bits as the two separate launches.
constexpr int64_t kFusedMaxI = 2048;

template <int DT, int NB>
__global__ __launch_bounds__(256)
void q8_linear_kernel(const int8_t* __restrict__ wq,
                      const float* __restrict__ ws, int64_t O, int64_t I,
                      const typename Elem<DT>::T* __restrict__ x,
                      int8_t* __restrict__ xq, float* __restrict__ xs,
                      float* __restrict__ y) {
  using E = Elem<DT>;
  const int lane = threadIdx.x & 63;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int64_t o0 = wave * kGemvRows;
  if (o0 >= O) return;                     // O % 16 == 0: all rows or none
  i32x4 w[2][kGemvRows];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int64_t k = 1024 * h + 16 * lane;
    const bool ok = k < I;                 // I % 64 == 0: whole 16-byte groups
#pragma unroll
    for (int r = 0; r < kGemvRows; ++r)
      w[h][r] = ok ? *reinterpret_cast<const i32x4*>(wq + (o0 + r) * I + k)
                   : i32x4{0, 0, 0, 0};
  }
  __builtin_amdgcn_sched_barrier(0);       // weight loads go out first
  i32x4 xc[2][NB];
  float sx[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    float v[2][16];
    float m = 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t k = 1024 * h + 16 * lane;
      if (k < I) {
        E::get8(x + b * I + k, v[h]);
        E::get8(x + b * I + k + 8, v[h] + 8);
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) v[h][e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(v[h][e]));
    }
    m = wave_max_abs(m);
    const float sc = m / 127.0f;           // IEEE float32 division
    sx[b] = sc;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        xc[h][b][q] = static_cast<int>(code(v[h][4 * q], sc) | code(v[h][4 * q + 1], sc) << 8 |
                                       code(v[h][4 * q + 2], sc) << 16 |
                                       code(v[h][4 * q + 3], sc) << 24);
      const int64_t k = 1024 * h + 16 * lane;
      if (wave == 0 && k < I) *reinterpret_cast<i32x4*>(xq + b * I + k) = xc[h][b];
    }
    if (wave == 0 && lane == 0) xs[b] = sc;
  }
  int acc[NB][kGemvRows];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int r = 0; r < kGemvRows; ++r) {
      int a = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          a = __builtin_amdgcn_sdot4(w[h][r][q], xc[h][b][q], a, false);
      acc[b][r] = a;
    }
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int r = 0; r < kGemvRows; ++r) {
      const int sum = wave_sum_i32(acc[b][r]);
      if (lane == r)
        y[b * O + o0 + r] = static_cast<float>(sum) * (ws[o0 + r] * sx[b]);
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
  // Wavefronts per workgroup: the fewest (4..8) that put the grid on the
  // 256 CUs in one round, one workgroup per CU; else 4 (two workgroups per
  // CU, several rounds). With 4 and more workgroups than CUs, part of the
  // CUs would hold two while the rest hold one and finish early.
  const int64_t gy = (B + kTokWG - 1) / kTokWG;
  int waves = 4;
  for (int wc = 4; wc <= 8; ++wc) {
    if (((O + 16 * wc - 1) / (16 * wc)) * gy <= 256) { waves = wc; break; }
  }
  const int64_t gx = (O + 16 * waves - 1) / (16 * waves);
  if (gx > 0x7fffffff || gy > 65535) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(q8_matmul_kernel,
                     dim3(static_cast<unsigned>(gx), static_cast<unsigned>(gy)),
                     dim3(64 * waves), 0, stream, wq, ws, O, I, xq, xs, B, y);
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
