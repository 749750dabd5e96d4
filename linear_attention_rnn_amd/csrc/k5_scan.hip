// Carry scan of the segment-parallel prefill. A sequence split into
// segments is run in three launches: every segment's transition P (the
// recurrence from the identity with v = 0, so that S_out = S_in P for the
// homogeneous part) and zero-start final state Hs, all segments at once;
// then this scan, which chains the segments' carries,
//   Sin_0 = S0,   Sin_{j+1} = Sin_j P_j + Hs_j,
// (the recurrence of page "RWKV-X Architecture", section "WKV-7 Kernel
// (Generalized Delta Rule)", is affine in the state, so a segment maps its
// initial state S to S P + Hs); then every segment again from its true
// initial state, producing the outputs.
//
// One 256-thread workgroup per (sequence, head). Thread t owns the 4 x 4
// block rows 4 (t / 16) .. + 3, columns 4 (t % 16) .. + 3 of the state. The
// state is kept transposed in LDS (St[k][i] = S[i][k]) and P row-major, so a
// k step is two 16-byte LDS reads and 16 FMAs; the sum over k runs in order
// in fp32. The next segment's P and Hs are loaded into registers while the
// current product is computed.

#include "internal.h"

namespace wkv7 {
namespace {

constexpr int kPitch = kN + 4;   // LDS row pitch (floats, 16-byte rows)

__device__ __forceinline__ float4 ld4(const float* p) {
  return *reinterpret_cast<const float4*>(p);
}
// HBM accesses through global-address-space pointers: the work item's
// pointers come from memory, so plain accesses would compile to flat
// instructions, which also count against the LDS wait counter, and every
// LDS wait in the product would then wait for the prefetch as well.
typedef float gvec4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) gvec4 gfloat4;
__device__ __forceinline__ float4 ldg4(const float* p) {
  const gvec4 v = *(const gfloat4*)(p);
  return make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void stg4(float* p, float4 v) {
  *(gfloat4*)(p) = gvec4{v.x, v.y, v.z, v.w};
}

__global__ __launch_bounds__(256)
void seg_scan_kernel(const ScanItem* items, int32_t n_items, int32_t H) {
  __shared__ __attribute__((aligned(16))) float St[kN * kPitch];
  __shared__ __attribute__((aligned(16))) float Psh[kN * kPitch];
  const int item = blockIdx.x / H;
  const int h = blockIdx.x - item * H;
  if (item >= n_items) return;
  const ScanItem it = items[item];
  const int tid = threadIdx.x;
  const size_t hoff = static_cast<size_t>(h) * (kN * kN);
  const size_t blk = static_cast<size_t>(H) * (kN * kN);   // one of P/Hs/Sin
  const int r0 = 4 * (tid >> 4);     // block rows
  const int c0 = 4 * (tid & 15);     // block columns
  // P staging: thread t moves elements 16 t .. 16 t + 15 (row 16 t / 64)
  const int pr = (16 * tid) / kN;
  const int pc = (16 * tid) % kN;

  float4 s[4];                       // S block rows r0 + i, columns c0 .. + 3
#pragma unroll
  for (int i = 0; i < 4; ++i) s[i] = ldg4(it.s0 + hoff + (r0 + i) * kN + c0);
  float4 pn[4], hn[4];               // next segment's P slice and Hs block
  auto fetch = [&](int j) {
    const float* seg = it.base + static_cast<size_t>(j) * 3 * blk;
#pragma unroll
    for (int q = 0; q < 4; ++q) pn[q] = ldg4(seg + hoff + pr * kN + pc + 4 * q);
#pragma unroll
    for (int i = 0; i < 4; ++i) hn[i] = ldg4(seg + blk + hoff + (r0 + i) * kN + c0);
  };
  if (it.n_seg > 1) fetch(0);
  for (int j = 0; j < it.n_seg; ++j) {
    float* seg = it.base + static_cast<size_t>(j) * 3 * blk;
#pragma unroll
    for (int i = 0; i < 4; ++i)          // Sin_j
      stg4(seg + 2 * blk + hoff + (r0 + i) * kN + c0, s[i]);
    if (j + 1 == it.n_seg) break;
    __syncthreads();                     // previous step's LDS reads done
#pragma unroll
    for (int i = 0; i < 4; ++i) {        // St[c][r] = S[r][c]
      St[(c0 + 0) * kPitch + r0 + i] = s[i].x;
      St[(c0 + 1) * kPitch + r0 + i] = s[i].y;
      St[(c0 + 2) * kPitch + r0 + i] = s[i].z;
      St[(c0 + 3) * kPitch + r0 + i] = s[i].w;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<float4*>(&Psh[pr * kPitch + pc + 4 * q]) = pn[q];
    float4 acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = hn[i];
    __syncthreads();                     // St and Psh complete
    if (j + 2 < it.n_seg) fetch(j + 1);  // in flight during the product
    for (int k = 0; k < kN; ++k) {
      const float4 sv = ld4(&St[k * kPitch + r0]);
      const float4 pv = ld4(&Psh[k * kPitch + c0]);
      const float si[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i].x = fmaf(si[i], pv.x, acc[i].x);
        acc[i].y = fmaf(si[i], pv.y, acc[i].y);
        acc[i].z = fmaf(si[i], pv.z, acc[i].z);
        acc[i].w = fmaf(si[i], pv.w, acc[i].w);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = acc[i];
  }
}

}  // namespace

hipError_t launch_seg_scan(const ScanItem* items, int32_t n_items, int32_t H,
                           hipStream_t stream) {
  if (n_items <= 0) return hipSuccess;
  const int64_t blocks = static_cast<int64_t>(n_items) * H;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(seg_scan_kernel, dim3(static_cast<unsigned>(blocks)),
                     dim3(256), 0, stream, items, n_items, H);
  return hipGetLastError();
}

}  // namespace wkv7
