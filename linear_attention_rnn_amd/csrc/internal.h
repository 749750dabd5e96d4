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

// One segment of a sequence split by the segment-parallel prefill (32
// bytes): its own initial and final state buffers instead of a pool slot.
struct SegItem {
  const float* s_in;   // initial state of head 0 (head h at + h*N*N); NULL: 0
  float* s_out;        // final state of head 0; NULL: not stored
  int32_t tok0;        // first token row in r..b / o
  int32_t len;         // number of tokens (>= 1)
  int32_t flags;       // kSeg* below
  int32_t pad;
};
constexpr int32_t kSegIdentity = 1;   // initial state I (s_in ignored)
constexpr int32_t kSegZeroV = 2;      // v taken as 0
constexpr int32_t kSegNoOut = 4;      // o not written

// The carry scan of one split sequence: its segments' blocks follow each
// other, segment j at base + j * 3 * H*N*N floats, each block holding the
// segment's transition P, zero-start final state Hs and initial state Sin
// ([3][H][N][N]). Sin_0 = S0 and Sin_{j+1} = Sin_j P_j + Hs_j (32 bytes).
struct ScanItem {
  const float* s0;     // the sequence's initial state, head 0 (a pool slot)
  float* base;         // block of segment 0
  int32_t n_seg;
  int32_t pad[3];
};

// Where one launch's work description lives on the device: sequential
// items, all chunked items, and for segment-parallel prefill the segment
// items of its two kernel phases (the first also runs the chunked sequences
// that are not split) and the scan items.
struct Launch {
  // sequential items: the single-token ones first (n_seq_single of them)
  const WorkItem* seq = nullptr;           int32_t n_seq = 0;
  int32_t n_seq_single = 0;
  const WorkItem* chunk_all = nullptr;     int32_t n_chunk_all = 0;
  const SegItem* phase1 = nullptr;         int32_t n_phase1 = 0;
  const SegItem* phase3 = nullptr;         int32_t n_phase3 = 0;
  const ScanItem* scan = nullptr;          int32_t n_scan = 0;
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

// Workgroup barrier that orders LDS only. __syncthreads() also waits for the
// wavefront's outstanding global loads and stores (s_waitcnt vmcnt(0)),
// which would stall loads prefetched just before the barrier; here only this
// wavefront's LDS operations must be complete (lgkmcnt(0); the vmcnt and
// expcnt fields of the s_waitcnt immediate are left at their maxima). The
// empty asm statements keep the compiler from moving memory accesses across
// the barrier. Only for kernels whose waves share data through LDS alone.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Sequential kernel: one wavefront per (sequence, head), state in registers.
hipError_t launch_seq(const SeqArgs& args, hipStream_t stream);
// The same for items of exactly one token (decode), each state row stored
// as soon as it is updated; the same bits as launch_seq.
hipError_t launch_seq1(const SeqArgs& args, hipStream_t stream);
// The same recurrence with four wavefronts per (sequence, head) (the same
// bits), for items of more than one token.
hipError_t launch_seq4(const SeqArgs& args, hipStream_t stream);

// Pipelined chunked-prefill kernel (32-token chunks) for sequences of at
// least one chunk, over pool slots (args.items). bf16 inputs take the plan
// with an fp16 value side unless `precise`; fp32 inputs, and bf16 inputs
// with `precise`, the plan with split bf16 operands throughout. n_dec
// decode items `dec` run in trailing workgroups of the same launch.
hipError_t launch_chunked_p(const SeqArgs& args, bool precise,
                            hipStream_t stream, const WorkItem* dec = nullptr,
                            int32_t n_dec = 0);
// Segment items (SegItem, n_items of them; args.items unused) instead of
// pool slots; same kernel code.
hipError_t launch_chunked_p_seg(const SeqArgs& args, bool precise,
                                const SegItem* segs, hipStream_t stream,
                                const WorkItem* dec = nullptr, int32_t n_dec = 0);
// Wavefronts per workgroup of the chunked kernel.
constexpr int kChunkPWaves = 12;
// Trailing workgroups of a chunked-kernel launch that run n_dec decode
// items (one (item, head) pair per wavefront).
inline int64_t chunk_decode_blocks(int32_t n_dec, int32_t H) {
  return n_dec > 0
             ? (static_cast<int64_t>(n_dec) * H + kChunkPWaves - 1) / kChunkPWaves
             : 0;
}
// Carry scan of split sequences: one workgroup per (sequence, head).
hipError_t launch_seg_scan(const ScanItem* items, int32_t n_items, int32_t H,
                           hipStream_t stream);

// Slot copies from src_pool to dst_pool (the same pool for a fork). `pairs`
// holds n (src slot, dst slot) int32 pairs on the device.
hipError_t launch_copy_slots(const float* src_pool, float* dst_pool,
                             size_t slot_floats, const int32_t* pairs,
                             int32_t n, hipStream_t stream);
// INT8 per-row quantization of x [rows][cols] (fp32 or bf16) into codes q
// and float32 scales, and the INT8 product y[B][O] of codes wq [O][I] with
// codes xq [B][I] (I % 64 == 0, O % 16 == 0).
hipError_t launch_q8_quantize(const void* x, int dtype, int64_t rows,
                              int64_t cols, int8_t* q, float* scale,
                              hipStream_t stream);
hipError_t launch_q8_matmul(const int8_t* wq, const float* ws, int64_t O,
                            int64_t I, const int8_t* xq, const float* xs,
                            int64_t B, float* y, hipStream_t stream);
// Quantize x [B][I] (fp32 or bf16) into xq, xs and multiply: one launch for
// at most four tokens with I <= 2048, otherwise the two launches above.
hipError_t launch_q8_linear(const int8_t* wq, const float* ws, int64_t O,
                            int64_t I, const void* x, int dtype, int64_t B,
                            int8_t* xq, float* xs, float* y,
                            hipStream_t stream);

// Zero-fill n slots listed (device int32) in `ids`.
hipError_t launch_zero_slots(float* pool, size_t slot_floats,
                             const int32_t* ids, int32_t n,
                             hipStream_t stream);

}  // namespace wkv7
