// Internal interface between the C-ABI host code and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace wkv7 {

constexpr int kN = 64;            // head size the kernels are written for

// One sequence of a forward call, as the kernels read it (16 bytes).
struct WorkItem {
  int32_t slot;   // slot id in the pool
  int32_t tok0;   // first token row in r..b / o
  int32_t len;    // number of tokens (>= 1)
  int32_t pad;
};

struct SeqArgs {
  float* pool;                 // [n_slots][H][N][N]
  const WorkItem* items;       // device array
  int32_t n_items;
  int32_t H;
  int32_t dtype;               // WKV7_F32 / WKV7_BF16
  const void* r; const void* w; const void* k;
  const void* v; const void* a; const void* b;
  float* o;                    // [T_tot][H][N]
};

// Sequential kernel: one wavefront per (sequence, head), state in registers.
hipError_t launch_seq(const SeqArgs& args, hipStream_t stream);

// Chunked-prefill kernel for sequences of at least one chunk. bf16 inputs
// take the fp16-value-side kernel unless `precise`; fp32 inputs always take
// the split-bf16 kernel.
hipError_t launch_chunked(const SeqArgs& args, bool precise,
                          hipStream_t stream);

// Pipelined chunked-prefill kernel for bf16 inputs with an fp16 value side
// (32-token chunks).
hipError_t launch_chunked_p(const SeqArgs& args, hipStream_t stream);

// Slot copies from src_pool to dst_pool (the same pool for a fork). `pairs`
// holds n (src slot, dst slot) int32 pairs on the device.
hipError_t launch_copy_slots(const float* src_pool, float* dst_pool,
                             size_t slot_floats, const int32_t* pairs,
                             int32_t n, hipStream_t stream);
// Zero-fill n slots listed (device int32) in `ids`.
hipError_t launch_zero_slots(float* pool, size_t slot_floats,
                             const int32_t* ids, int32_t n,
                             hipStream_t stream);

}  // namespace wkv7
