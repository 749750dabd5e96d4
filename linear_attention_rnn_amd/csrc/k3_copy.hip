// Slot-copy kernels for the fork, migrate and reset verbs (page "wkvm: state-slot
// inference for RWKV, GDN and Mamba hybrids", section "The allocation unit
// wkvm changes": a fixed-size slot can be copied and restored cheaply).
//
// A slot image moves as raw 16-byte words (uint4), never as floats, so
// copies are bit-exact for every pattern (NaN payloads, -0.0, denormals).
// The grid is flat: block b works on slot b / blocks_per_slot, segment
// b % blocks_per_slot, striding over that slot's words.

#include "internal.h"

namespace wkv7 {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads)
void copy_slots_kernel(const uint4* src_pool, uint4* dst_pool,
                       size_t slot_words, const int32_t* pairs, int32_t n,
                       int32_t blocks_per_slot) {
  const int32_t pi = blockIdx.x / blocks_per_slot;
  const int32_t part = blockIdx.x - pi * blocks_per_slot;
  if (pi >= n) return;
  const uint4* src = src_pool + static_cast<size_t>(pairs[2 * pi]) * slot_words;
  uint4* dst = dst_pool + static_cast<size_t>(pairs[2 * pi + 1]) * slot_words;
  const size_t stride = static_cast<size_t>(blocks_per_slot) * kThreads;
  for (size_t i = static_cast<size_t>(part) * kThreads + threadIdx.x;
       i < slot_words; i += stride)
    dst[i] = src[i];
}

__global__ __launch_bounds__(kThreads)
void zero_slots_kernel(uint4* pool, size_t slot_words, const int32_t* ids,
                       int32_t n, int32_t blocks_per_slot) {
  const int32_t si = blockIdx.x / blocks_per_slot;
  const int32_t part = blockIdx.x - si * blocks_per_slot;
  if (si >= n) return;
  uint4* dst = pool + static_cast<size_t>(ids[si]) * slot_words;
  const size_t stride = static_cast<size_t>(blocks_per_slot) * kThreads;
  const uint4 z = make_uint4(0u, 0u, 0u, 0u);
  for (size_t i = static_cast<size_t>(part) * kThreads + threadIdx.x;
       i < slot_words; i += stride)
    dst[i] = z;
}

int32_t blocks_per_slot(size_t slot_words) {
  // about 4 words per thread, at most 64 blocks per slot
  size_t b = (slot_words + 4 * kThreads - 1) / (4 * kThreads);
  if (b < 1) b = 1;
  if (b > 64) b = 64;
  return static_cast<int32_t>(b);
}

}  // namespace

hipError_t launch_copy_slots(const float* src_pool, float* dst_pool,
                             size_t slot_floats, const int32_t* pairs,
                             int32_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const size_t words = slot_floats / 4;
  const int32_t bps = blocks_per_slot(words);
  const int64_t blocks = static_cast<int64_t>(n) * bps;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(copy_slots_kernel, dim3(static_cast<unsigned>(blocks)),
                     dim3(kThreads), 0, stream,
                     reinterpret_cast<const uint4*>(src_pool),
                     reinterpret_cast<uint4*>(dst_pool), words, pairs, n, bps);
  return hipGetLastError();
}

hipError_t launch_zero_slots(float* pool, size_t slot_floats,
                             const int32_t* ids, int32_t n,
                             hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const size_t words = slot_floats / 4;
  const int32_t bps = blocks_per_slot(words);
  const int64_t blocks = static_cast<int64_t>(n) * bps;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(zero_slots_kernel, dim3(static_cast<unsigned>(blocks)),
                     dim3(kThreads), 0, stream, reinterpret_cast<uint4*>(pool),
                     words, ids, n, bps);
  return hipGetLastError();
}

}  // namespace wkv7
