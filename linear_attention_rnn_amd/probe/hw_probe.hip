// Hardware ceilings for reading the roofline fractions against what the
// chip sustains rather than only its published peaks: a streaming copy
// (in place or source to destination, optionally with non-temporal loads
// and stores) and a matrix-core loop. Built as its own library, separate
// from the WKV-7 library; only measurement code loads it.

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;

// dst may equal src (an in-place read and write of every word), so neither
// pointer is restrict. Every index is checked against n16.
template <bool NT>
__global__ __launch_bounds__(kCopyThreads)
void probe_copy_kernel(const u32x4* src, u32x4* dst, size_t n16) {
  const size_t stride = static_cast<size_t>(gridDim.x) * kCopyThreads * kCopyUnroll;
  for (size_t base = static_cast<size_t>(blockIdx.x) * kCopyThreads * kCopyUnroll + threadIdx.x;
       base < n16; base += stride) {
    u32x4 x[kCopyUnroll];
    if (base + static_cast<size_t>(kCopyUnroll - 1) * kCopyThreads < n16) {
#pragma unroll
      for (int u = 0; u < kCopyUnroll; ++u)
        x[u] = NT ? __builtin_nontemporal_load(src + base + u * kCopyThreads)
                  : src[base + u * kCopyThreads];
#pragma unroll
      for (int u = 0; u < kCopyUnroll; ++u) {
        if (NT) __builtin_nontemporal_store(x[u], dst + base + u * kCopyThreads);
        else dst[base + u * kCopyThreads] = x[u];
      }
      continue;
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const size_t i = base + static_cast<size_t>(u) * kCopyThreads;
      if (i < n16) x[u] = NT ? __builtin_nontemporal_load(src + i) : src[i];
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const size_t i = base + static_cast<size_t>(u) * kCopyThreads;
      if (i < n16) {
        if (NT) __builtin_nontemporal_store(x[u], dst + i);
        else dst[i] = x[u];
      }
    }
  }
}

constexpr int kMfmaThreads = 256;   // four wavefronts
constexpr int kAcc = 8;             // independent accumulator chains per wavefront

// kAcc independent chains of v_mfma_f32_16x16x32_bf16 per wavefront; one
// float per wavefront is written so that nothing is dead.
__global__ __launch_bounds__(kMfmaThreads)
void probe_mfma_bf16_kernel(float* out, int iters, float seed) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<__bf16>(seed * static_cast<float>((lane + e) & 7));
    b[e] = static_cast<__bf16>(seed * static_cast<float>((lane * 3 + e) & 7));
  }
  f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0, c4 = c0, c5 = c0,
        c6 = c0, c7 = c0;
  // Each chain accumulates in place (tied operand), so the loop carries no
  // register moves; dependent instructions are eight apart.
#define PROBE_MFMA_BF16(c) \
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b))
  for (int it = 0; it < iters; ++it) {
    PROBE_MFMA_BF16(c0); PROBE_MFMA_BF16(c1); PROBE_MFMA_BF16(c2); PROBE_MFMA_BF16(c3);
    PROBE_MFMA_BF16(c4); PROBE_MFMA_BF16(c5); PROBE_MFMA_BF16(c6); PROBE_MFMA_BF16(c7);
  }
#undef PROBE_MFMA_BF16
  const f32x4 t = c0 + c1 + c2 + c3 + c4 + c5 + c6 + c7;
  const float s = t[0] + t[1] + t[2] + t[3];
  if (lane == 0) out[blockIdx.x * (kMfmaThreads / 64) + (threadIdx.x >> 6)] = s;
}

// The same with v_mfma_i32_16x16x64_i8 (int8 operands, int32 accumulators).
__global__ __launch_bounds__(kMfmaThreads)
void probe_mfma_i8_kernel(float* out, int iters, float seed) {
  const int lane = threadIdx.x & 63;
  const int sv = static_cast<int>(seed);
  i32x4 av, bv;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    av[e] = (lane + e + sv) & 0x03030303;
    bv[e] = (lane * 3 + e + sv) & 0x03030303;
  }
  i32x4 c0 = {0, 0, 0, 0}, c1 = c0, c2 = c0, c3 = c0, c4 = c0, c5 = c0, c6 = c0,
        c7 = c0;
#define PROBE_MFMA_I8(c) \
  asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(c) : "v"(av), "v"(bv))
  for (int it = 0; it < iters; ++it) {
    PROBE_MFMA_I8(c0); PROBE_MFMA_I8(c1); PROBE_MFMA_I8(c2); PROBE_MFMA_I8(c3);
    PROBE_MFMA_I8(c4); PROBE_MFMA_I8(c5); PROBE_MFMA_I8(c6); PROBE_MFMA_I8(c7);
  }
#undef PROBE_MFMA_I8
  const i32x4 t = c0 + c1 + c2 + c3 + c4 + c5 + c6 + c7;
  const int s = t[0] + t[1] + t[2] + t[3];
  if (lane == 0)
    out[blockIdx.x * (kMfmaThreads / 64) + (threadIdx.x >> 6)] = static_cast<float>(s);
}

// The same with v_mfma_i32_32x32x32_i8 (int8 operands, 32 x 32 tile of
// int32 accumulators, 16 registers per lane).
__global__ __launch_bounds__(kMfmaThreads)
void probe_mfma_i8_32_kernel(float* out, int iters, float seed) {
  const int lane = threadIdx.x & 63;
  const int sv = static_cast<int>(seed);
  i32x4 av, bv;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    av[e] = (lane + e + sv) & 0x03030303;
    bv[e] = (lane * 3 + e + sv) & 0x03030303;
  }
  i32x16 c0 = {}, c1 = c0, c2 = c0, c3 = c0, c4 = c0, c5 = c0, c6 = c0, c7 = c0;
#define PROBE_MFMA_I8_32(c) \
  asm volatile("v_mfma_i32_32x32x32_i8 %0, %1, %2, %0" : "+a"(c) : "v"(av), "v"(bv))
  for (int it = 0; it < iters; ++it) {
    PROBE_MFMA_I8_32(c0); PROBE_MFMA_I8_32(c1); PROBE_MFMA_I8_32(c2); PROBE_MFMA_I8_32(c3);
    PROBE_MFMA_I8_32(c4); PROBE_MFMA_I8_32(c5); PROBE_MFMA_I8_32(c6); PROBE_MFMA_I8_32(c7);
  }
#undef PROBE_MFMA_I8_32
  const i32x16 t = c0 + c1 + c2 + c3 + c4 + c5 + c6 + c7;
  int s = 0;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += t[r];
  if (lane == 0)
    out[blockIdx.x * (kMfmaThreads / 64) + (threadIdx.x >> 6)] = static_cast<float>(s);
}

}  // namespace

extern "C" {

// Copies `bytes` (a multiple of 16, both pointers 16-byte aligned) from src
// to dst on `stream` with `blocks` workgroups of 256 threads (0: enough for
// one pass, at most 8192). src == dst is allowed (in place); other overlap
// is not. Returns a hipError_t value.
int hwprobe_copy(const void* src, void* dst, size_t bytes, int nontemporal,
                 int blocks, void* stream) {
  if (!src || !dst || bytes % 16 != 0 ||
      reinterpret_cast<uintptr_t>(src) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(dst) % 16 != 0 || blocks < 0)
    return hipErrorInvalidValue;
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const size_t per_block = static_cast<size_t>(kCopyThreads) * kCopyUnroll;
  size_t g = blocks > 0 ? static_cast<size_t>(blocks) : (n16 + per_block - 1) / per_block;
  if (g > 8192) g = 8192;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const u32x4* in = static_cast<const u32x4*>(src);
  u32x4* o = static_cast<u32x4*>(dst);
  if (nontemporal)
    hipLaunchKernelGGL(probe_copy_kernel<true>, dim3(static_cast<unsigned>(g)),
                       dim3(kCopyThreads), 0, s, in, o, n16);
  else
    hipLaunchKernelGGL(probe_copy_kernel<false>, dim3(static_cast<unsigned>(g)),
                       dim3(kCopyThreads), 0, s, in, o, n16);
  return hipGetLastError();
}

// Runs `blocks` workgroups of four wavefronts, each wavefront issuing
// iters x 8 matrix instructions (kind 0: v_mfma_f32_16x16x32_bf16, 16,384
// flops each; kind 1: v_mfma_i32_16x16x64_i8, 32,768 ops each; kind 2:
// v_mfma_i32_32x32x32_i8, 65,536 ops each). `out` must hold blocks x 4
// floats. Returns a hipError_t value.
int hwprobe_mfma(int kind, int blocks, int iters, float* out, size_t out_floats,
                 void* stream) {
  if (!out || blocks <= 0 || blocks > 65536 || iters < 0 || (kind < 0 || kind > 2) ||
      out_floats < static_cast<size_t>(blocks) * (kMfmaThreads / 64))
    return hipErrorInvalidValue;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (kind == 0)
    hipLaunchKernelGGL(probe_mfma_bf16_kernel, dim3(blocks), dim3(kMfmaThreads), 0, s,
                       out, iters, 0.125f);
  else if (kind == 1)
    hipLaunchKernelGGL(probe_mfma_i8_kernel, dim3(blocks), dim3(kMfmaThreads), 0, s,
                       out, iters, 1.0f);
  else
    hipLaunchKernelGGL(probe_mfma_i8_32_kernel, dim3(blocks), dim3(kMfmaThreads), 0, s,
                       out, iters, 1.0f);
  return hipGetLastError();
}

// Matrix instructions each wavefront issues per loop iteration.
int hwprobe_mfma_per_iter(void) { return kAcc; }

}  // extern "C"
