/*
 * libwkv7 — the RWKV-7 WKV state-slot hot path on MI355X (gfx950).
 *
 * C ABI. Every argument is a plain pointer or size; no framework types.
 *
 * The operation (page "RWKV-X Architecture", section "WKV-7 Kernel
 * (Generalized Delta Rule)"): per head, a fixed-size [N, N] recurrent state
 * is updated each timestep. Reading of that section taken here:
 *
 *     S_t = S_{t-1} (diag(w_t) + a_t b_t^T) + v_t k_t^T,      o_t = S_t r_t
 *
 * with S[i][j], i = value index (row), j = key index (column): the delta-rule
 * term reads the state before this step's decay, the readout uses the
 * updated state. w is used as given (expected in (0, 1]).
 *
 * State slots (page "wkvm: state-slot inference for RWKV, GDN and Mamba
 * hybrids", section "The allocation unit wkvm changes"): each request owns a
 * fixed-size slot instead of a growing KV chain, and slots support the verbs
 * create, snapshot, fork, hibernate and resume. A pool is one device
 * allocation of n_slots slots made up front (page "Virtual Memory for KV
 * Cache and Model Weights": recurrent states stay resident and are reserved
 * separately; admission needs a free recurrent-state slot).
 *
 * Layouts (all row-major, little-endian):
 *   slot image      float32 [H][N][N], S[h][i][j] at ((h*N)+i)*N+j.
 *                   wkv7_slot_bytes() = H*N*N*4. The pool is
 *                   float32 [n_slots][H][N][N].
 *   r,w,k,v,a,b     [T_tot][H][N] in the call's dtype (fp32 or bf16);
 *                   the tokens of sequence s are rows
 *                   cu_seqlens[s] .. cu_seqlens[s+1]-1.
 *   o               float32 [T_tot][H][N].
 *   N must be 64. Device pointers must be 16-byte aligned.
 *
 * Errors: every call returns a wkv7_status. On any non-zero status no device
 * work has been enqueued and the pool is unchanged, except WKV7_ERR_HIP,
 * which reports a failed HIP runtime call (message from the runtime).
 * wkv7_last_error() returns the calling thread's last message. There is no
 * fallback path: an unsupported shape or dtype is an error.
 *
 * Threading and ordering: a pool belongs to one host thread; calls on one
 * pool are not thread-safe. Device work is enqueued on the caller's stream
 * (a hipStream_t passed as void*, NULL = the null stream). Calls on one pool
 * that use different streams must be ordered by the caller.
 *
 * Host waits. The library waits for device work only here:
 *   - wkv7_pool_create zero-fills the pool and waits for the device;
 *     wkv7_plan_create copies the plan with a synchronous copy;
 *   - wkv7_pool_destroy and wkv7_plan_destroy wait for all work on the
 *     device before freeing (releasing device or pinned memory waits for
 *     the whole device on this runtime in any case), as does
 *     wkv7_sessions_destroy;
 *   - a call that stages host metadata (wkv7_forward, wkv7_forward_noalloc,
 *     wkv7_fork, wkv7_migrate, wkv7_reset, and wkv7_hibernate/wkv7_resume
 *     of scattered slots) uses the pool's eight pinned staging buffers in
 *     turn; when the buffer's previous copy (eight staged calls earlier)
 *     has not yet run, the call waits on the host for that copy alone.
 * Nothing else waits: wkv7_forward_plan, wkv7_snapshot, and hibernate or
 * resume of runs of slots only enqueue. A buffer a call outgrows (staging,
 * segment buffers) is not freed but kept until wkv7_pool_destroy, and its
 * replacement is allocated with hipMalloc, which does not wait.
 */
#ifndef WKV7_H
#define WKV7_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t wkv7_status;

enum {
  WKV7_OK = 0,
  WKV7_ERR_INVALID_ARG = -1,    /* null pointer, bad size, bad cu_seqlens */
  WKV7_ERR_OUT_OF_RANGE = -2,   /* a slot id outside [0, n_slots) */
  WKV7_ERR_DUPLICATE_SLOT = -3, /* a slot named twice where it would race */
  WKV7_ERR_POOL_FULL = -4,      /* fewer free slots than requested */
  WKV7_ERR_UNSUPPORTED = -5,    /* N != 64, unknown dtype or option */
  WKV7_ERR_OOM = -6,            /* device or pinned host allocation failed */
  WKV7_ERR_HIP = -7             /* a HIP runtime call failed */
};

/* dtype of r, w, k, v, a, b. The state and o are always float32. */
enum { WKV7_F32 = 0, WKV7_BF16 = 1 };

/* options for wkv7_pool_set_option */
enum {
  /* Sequences with at least this many tokens take the chunked-prefill
   * kernel; shorter ones (including every decode token) take the
   * sequential kernel. Default 32; must be >= 1. The choice depends on the
   * sequence length only, so a slot's result never depends on the rest of
   * the batch (the sequential kernel's variants for few and for many
   * sequences compute the same bits). The chunked kernel runs a chunk token
   * by token when its decay exceeds the range of its scaled operands, so
   * both paths accept any w in (0, 1]. */
  WKV7_OPT_PREFILL_MIN_LEN = 1,
  /* Operand precision of the chunked kernel for bf16 inputs. 0 (default):
   * the key-side Gram products use split bf16 (hi + lo) operands and the
   * value-side products single fp16 operands (the state and intermediates
   * scaled by powers of two), about 3e-3 of max|err|/rms(o) on the
   * workloads' inputs. 1: every product uses split bf16 operands, about
   * 1e-4, in about 1.5 times the time (the value-side products take three
   * matrix-core operations each). fp32 inputs always use 1. */
  WKV7_OPT_CHUNK_PRECISE = 2,
  /* Segment-parallel prefill, for batches with few long sequences (the
   * chunked kernel runs one workgroup per (sequence, head), so a handful of
   * sequences leaves most of the GPU idle). 0 (default): off. s > 0 (a
   * multiple of 32, at least 64): every sequence of at least 2 s tokens
   * (any input type and CHUNK_PRECISE) is cut into segments of s tokens that
   * run in parallel: each segment's transition and zero-start state, a
   * short scan chaining the segments' states (the recurrence is affine in
   * the state), then every segment again from its true initial state. About
   * three times the arithmetic, so it pays only while the (sequence, head)
   * count is well below the CU count. The split depends on the sequence's
   * own length only; results agree with the unsplit run to rounding, not
   * bit for bit. */
  WKV7_OPT_SEGMENT_LEN = 3
};

typedef struct wkv7_pool wkv7_pool;

/* Message for the calling thread's last failed call ("" if none). The
 * string stays valid until the thread's next libwkv7 call. */
const char* wkv7_last_error(void);

/* Library version as major*10000 + minor*100 + patch. */
int32_t wkv7_version(void);

/* create — allocate a pool of n_slots slots of H heads of N x N float32 on
 * the current device, zero-filled (synchronously), plus pinned staging for
 * per-call metadata. The pool owns that memory. n_slots >= 1, H >= 1,
 * N == 64 (else WKV7_ERR_UNSUPPORTED). *out receives the handle. */
wkv7_status wkv7_pool_create(int32_t n_slots, int32_t H, int32_t N,
                             wkv7_pool** out);

/* destroy — wait for all work on the pool's device (so the pool's work on
 * every stream has finished), then free everything the pool owns (page
 * "RWKV-X Architecture", section "Adapter API": the state's free call; page
 * "Virtual Memory for KV Cache and Model Weights": memory is released only
 * after the transfers that use it have finished). Plans made for the pool
 * must be destroyed first. A NULL pool is a no-op. */
wkv7_status wkv7_pool_destroy(wkv7_pool* pool);

/* Bytes in one slot image: H*N*N*4 (0 for NULL). */
size_t wkv7_slot_bytes(const wkv7_pool* pool);

/* Device address of slot 0 (the pool is float32 [n_slots][H][N][N]).
 * Borrowed; for inspection by tests and benchmarks. */
void* wkv7_pool_state_ptr(wkv7_pool* pool);

/* Shape of the pool; any out pointer may be NULL. */
wkv7_status wkv7_pool_shape(const wkv7_pool* pool, int32_t* n_slots,
                            int32_t* H, int32_t* N);

/* The HIP device that holds the pool's memory and runs its launches (the
 * device current at wkv7_pool_create). The input, output and buffer
 * pointers of every call on the pool must be memory of this device; the
 * library cannot check a raw device pointer's device, so a binding that
 * holds typed tensors checks it (the Python binding does). */
wkv7_status wkv7_pool_device(const wkv7_pool* pool, int32_t* device);

/* Set a pool option (see WKV7_OPT_*). */
wkv7_status wkv7_pool_set_option(wkv7_pool* pool, int32_t opt, int64_t val);

/* admission — take n free slot ids from the host free list into ids_out
 * (host array of n) (page "Virtual Memory for KV Cache and Model Weights":
 * admitting a request needs a free recurrent-state slot besides its KV
 * blocks; page "wkvm: state-slot inference for RWKV, GDN and Mamba
 * hybrids", section "The allocation unit wkvm changes": the fixed-size slot
 * is the unit a request is given). WKV7_ERR_POOL_FULL if fewer than n are
 * free; then nothing is taken. Allocation does not clear the slots (see
 * wkv7_reset). Host only; no device work. */
wkv7_status wkv7_slot_alloc(wkv7_pool* pool, int32_t n, int32_t* ids_out);

/* Return n allocated ids (host array) to the free list (the same passages:
 * a finished request gives its slot back). Every id must be allocated and
 * appear once, else nothing is freed. Host only; no device work. */
wkv7_status wkv7_slot_free(wkv7_pool* pool, const int32_t* ids, int32_t n);

/* forward — run the recurrence for a packed batch of sequences.
 *
 * slot_ids[n_seqs] and cu_seqlens[n_seqs+1] are HOST int32 arrays;
 * cu_seqlens[0] == 0 and it is non-decreasing. Sequence s starts from the
 * state in slot slot_ids[s], consumes tokens cu_seqlens[s]..cu_seqlens[s+1]-1
 * of r,w,k,v,a,b (device, [T_tot][H][N], dtype WKV7_F32 or WKV7_BF16), writes
 * those rows of o (device, float32 [T_tot][H][N]) and leaves its final state
 * in the slot. A zero-length sequence is a no-op. Slots not named are not
 * touched. Any slot id in range is accepted, allocated or not.
 *
 * Errors: WKV7_ERR_OUT_OF_RANGE (an id outside the pool),
 * WKV7_ERR_DUPLICATE_SLOT (an id named twice), WKV7_ERR_INVALID_ARG (null
 * or misaligned pointers with T_tot > 0, bad cu_seqlens, n_seqs < 0),
 * WKV7_ERR_UNSUPPORTED (dtype). The host arrays may be reused as soon as
 * the call returns (they are staged); the device arrays must stay alive
 * until the stream has passed the call. With WKV7_OPT_SEGMENT_LEN on, a
 * batch that needs more segment buffers than any before on this pool gets
 * new, larger ones (hipMalloc; WKV7_ERR_OOM if that fails); the old ones
 * are kept until the pool is destroyed. */
wkv7_status wkv7_forward(wkv7_pool* pool, const int32_t* slot_ids,
                         const int32_t* cu_seqlens, int32_t n_seqs,
                         int32_t dtype, const void* r, const void* w,
                         const void* k, const void* v, const void* a,
                         const void* b, float* o, void* stream);

/* forward without allocation — for callers that cannot allocate device or
 * pinned memory during the call (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation). The same validation,
 * errors, kernels and results, bit for bit, as wkv7_forward on the same
 * arguments; the difference is where the kernels' scratch lives.
 *
 * The work description and, with WKV7_OPT_SEGMENT_LEN on, the segment
 * buffers (three H*N*N float32 blocks per segment) go into one static
 * device array of 32 MiB that the library holds on every GPU it runs on
 * until the process ends (its address is looked up once per device, at the
 * first pool creation there). The work description (16 bytes per
 * non-empty sequence, plus 32 bytes per segment and per split sequence when
 * segments are on) may take at most 64 KiB of it, and both parts together
 * at most 32 MiB; a larger batch fails with WKV7_ERR_INVALID_ARG before any
 * device work. The work description is copied in through one of the
 * pool's pinned staging buffers, preallocated at pool creation; the call
 * waits on the host only when that buffer's previous copy (eight calls
 * earlier) has not yet run. The call itself makes no device, pinned or
 * runtime allocation.
 *
 * Every call on a GPU, from any pool, uses that GPU's one array, which keeps
 * the last call's contents: calls on one GPU must be ordered (one stream,
 * or events); calls that overlap on one GPU race and give wrong results.
 * Nothing in the array needs to start at zero. */
wkv7_status wkv7_forward_noalloc(wkv7_pool* pool, const int32_t* slot_ids,
                                 const int32_t* cu_seqlens, int32_t n_seqs,
                                 int32_t dtype, const void* r, const void* w,
                                 const void* k, const void* v, const void* a,
                                 const void* b, float* o, void* stream);

/* plans — the metadata of a batch, validated once and kept on the device,
 * for callers that run the same batch layout step after step (steady-state
 * decode) or capture steps into a HIP graph. Page "rvLLM", section "What
 * actually makes B=1 fast": per-step synchronous metadata uploads serialise
 * the host against the GPU, and graphing the decode loop removes them;
 * section "Correctness discipline": a captured graph binds a frozen
 * metadata layout. */
typedef struct wkv7_plan wkv7_plan;

/* Validate slot_ids[n_seqs] and cu_seqlens[n_seqs+1] (host arrays) exactly
 * as wkv7_forward does, with the same errors, split the sequences between
 * the kernels (using the pool's PREFILL_MIN_LEN now) and copy the work list
 * into device memory owned by the plan. The copy is synchronous, so the
 * host arrays may be reused at once. *out receives the plan, which belongs
 * to `pool` and must be destroyed before it. */
wkv7_status wkv7_plan_create(wkv7_pool* pool, const int32_t* slot_ids,
                             const int32_t* cu_seqlens, int32_t n_seqs,
                             wkv7_plan** out);

/* Token rows (T_tot = cu_seqlens[n_seqs]) a forward with this plan reads
 * from r..b and writes to o; 0 for NULL. */
int64_t wkv7_plan_tokens(const wkv7_plan* plan);

/* forward with a plan — the same computation, with the same results bit for
 * bit, as wkv7_forward on the plan's slot_ids and cu_seqlens. It only checks
 * the pointers and dtype (as wkv7_forward) and enqueues the kernels on
 * `stream`: no allocation, no host-to-device copy, no event and no host
 * wait, so it may be captured into a HIP graph. The plan's device memory
 * must stay alive until the stream (or every launch of a graph that
 * captured the call) has passed it. WKV7_ERR_INVALID_ARG if the plan was
 * made for another pool. The chunked kernel's precision is the pool's
 * CHUNK_PRECISE at the time of the call. */
wkv7_status wkv7_forward_plan(wkv7_pool* pool, const wkv7_plan* plan,
                              int32_t dtype, const void* r, const void* w,
                              const void* k, const void* v, const void* a,
                              const void* b, float* o, void* stream);

/* Wait for all work on the plan's device (a plan's launches record no
 * event, so this is how work that used it is known to be done), then free
 * the plan. A NULL plan is a no-op. */
wkv7_status wkv7_plan_destroy(wkv7_plan* plan);

/* snapshot — copy slot `slot` (slot_bytes) into caller-owned device memory
 * dst_device, bit-exact (page "Virtual Memory for KV Cache and Model
 * Weights": a recoverable linear-state checkpoint). */
wkv7_status wkv7_snapshot(wkv7_pool* pool, int32_t slot, void* dst_device,
                          void* stream);

/* fork — pool[dst[i]] <- pool[src[i]] for i < n (host arrays), bit-exact
 * (page "wkvm: state-slot inference for RWKV, GDN and Mamba hybrids",
 * section "The allocation unit wkvm changes": fork is one of the slot
 * verbs; continuing a fork equals continuing its parent). dst ids must be
 * distinct and disjoint from src ids (WKV7_ERR_DUPLICATE_SLOT otherwise);
 * src ids may repeat. */
wkv7_status wkv7_fork(wkv7_pool* pool, const int32_t* src, const int32_t* dst,
                      int32_t n, void* stream);

/* reset — zero-fill n slots (host array of distinct ids) (page "RWKV-X
 * Architecture", section "Dual State": resetting a session zeroes its
 * recurrent state). */
wkv7_status wkv7_reset(wkv7_pool* pool, const int32_t* ids, int32_t n,
                       void* stream);

/* hibernate — copy n slots (host array of ids; repeats allowed) into
 * caller-owned host memory host_dst as n consecutive slot images,
 * bit-exact. host_dst must be pinned (page-locked, e.g. hipHostMalloc) and
 * must stay alive and untouched until the stream has passed the call (page
 * "Virtual Memory for KV Cache and Model Weights": blocks stay retained
 * until their transfers finish). bytes >= n*slot_bytes, else
 * WKV7_ERR_INVALID_ARG. The slots stay valid on the device.
 * Ids that form at least four runs of consecutive slots go through a
 * device staging buffer of the pool (at most 64 MiB, allocated on first
 * use, kept until the pool is destroyed; WKV7_ERR_OOM if that fails): a
 * kernel gathers up to 64 MiB of slots and one DMA moves them, so
 * scattered slots cross PCIe at the rate of one large copy. Fewer runs
 * take one DMA per run. */
wkv7_status wkv7_hibernate(wkv7_pool* pool, const int32_t* ids, int32_t n,
                           void* host_dst, size_t bytes, void* stream);

/* resume — copy n consecutive slot images from src (pinned host memory or
 * device memory, e.g. a snapshot) into slots ids[0..n) (distinct),
 * bit-exact (page "wkvm: state-slot inference for RWKV, GDN and Mamba
 * hybrids", section "The allocation unit wkvm changes": resume is the verb
 * that brings a hibernated slot back; page "Virtual Memory for KV Cache and
 * Model Weights": offloaded state is loaded back from host memory). bytes >= n*slot_bytes, else WKV7_ERR_INVALID_ARG. src must
 * stay alive until the stream has passed the call. Scattered ids (at
 * least four runs) take the staging path described under hibernate; a
 * 16-byte-aligned src in device memory of the pool's device is instead
 * scattered into the slots by one kernel, without staging. */
wkv7_status wkv7_resume(wkv7_pool* pool, const int32_t* ids, int32_t n,
                        const void* src, size_t bytes, void* stream);

/* live-migrate — copy n slots from pool `src` (ids src_ids, host array,
 * repeats allowed) into pool `dst` (ids dst_ids, host array, distinct),
 * bit-exact, on `stream` (page "wkvm: state-slot inference for RWKV, GDN
 * and Mamba hybrids", section "The allocation unit wkvm changes": the slot
 * verbs include live-migrate). Both pools must have the same H and N
 * (else WKV7_ERR_UNSUPPORTED) and live on the same device (pools on two
 * devices: WKV7_ERR_UNSUPPORTED; peer migration is not built). With
 * src == dst this is wkv7_fork. The source slots are left as they were
 * (freeing them is the caller's wkv7_slot_free); work on the two pools on
 * other streams must be ordered by the caller. */
wkv7_status wkv7_migrate(wkv7_pool* src, const int32_t* src_ids,
                         wkv7_pool* dst, const int32_t* dst_ids, int32_t n,
                         void* stream);

/* Slot images outside a pool (hibernated to host memory, sent to another
 * process or a later library version) are described by a versioned 64-byte
 * header, written in front of the n_slots consecutive images it describes
 * (the layout wkv7_hibernate writes and wkv7_resume reads). Little-endian;
 * reserved fields are zero. */
#define WKV7_IMAGE_MAGIC "WKV7SLOT"
enum { WKV7_IMAGE_VERSION = 1 };

typedef struct {
  char magic[8];          /* WKV7_IMAGE_MAGIC, no terminator */
  uint32_t version;       /* WKV7_IMAGE_VERSION */
  uint32_t header_bytes;  /* sizeof(wkv7_image_header) = 64 */
  uint32_t H, N;          /* heads and head size of every image */
  uint32_t state_dtype;   /* WKV7_F32 */
  uint32_t n_slots;       /* images that follow the header */
  uint64_t slot_bytes;    /* H*N*N*4, bytes of one image */
  uint64_t reserved[3];   /* zero */
} wkv7_image_header;

/* Fill *hdr for n_slots images of H heads of N x N float32 (N must be 64,
 * else WKV7_ERR_UNSUPPORTED). Host only. */
wkv7_status wkv7_image_header_init(wkv7_image_header* hdr, int32_t H,
                                   int32_t N, int32_t n_slots);

/* Check that *hdr describes slot images this library can resume into slots
 * of H heads of N x N: WKV7_ERR_INVALID_ARG for a bad magic, non-zero
 * reserved fields or an inconsistent header, WKV7_ERR_UNSUPPORTED for
 * another version or another slot shape. Host only. */
wkv7_status wkv7_image_header_check(const wkv7_image_header* hdr, int32_t H,
                                    int32_t N);

/* INT8 projections — the step upstream of the recurrence in decode (page
 * "RWKV-X Architecture", section "INT8 Quantization"): each row of a linear
 * projection's weights [out][in] is quantized symmetrically with its own
 * scale, the input is quantized once, and every output is an integer dot
 * product times the two scales.
 *
 * quantize — per-row symmetric INT8 codes of x [rows][cols] (device, dtype
 * WKV7_F32 or WKV7_BF16, row-major): scale[r] = max_c |x[r][c]| / 127 and
 * q[r][c] = round(x[r][c] / scale[r]), both in IEEE float32 with C roundf
 * rounding (halves away from zero), so the codes are reproducible bit for
 * bit; a row of zeros gets scale 0 and codes 0. q (int8 [rows][cols]) and
 * scale (float32 [rows]) are device arrays owned by the caller. Inputs must
 * be finite (other values give unspecified codes). Used for weight rows
 * once and for the input rows (one per token) of every call. */
wkv7_status wkv7_q8_quantize(const void* x, int32_t dtype, int64_t rows,
                             int64_t cols, int8_t* q, float* scale,
                             void* stream);

/* matmul — y[b][o] = (sum_i wq[o][i] * xq[b][i]) * w_scale[o] * x_scale[b]
 * for B input rows (tokens) and `out` output rows: wq int8 [out][in] and
 * w_scale float32 [out] from wkv7_q8_quantize of the weights, xq int8
 * [B][in] and x_scale float32 [B] from wkv7_q8_quantize of the inputs, y
 * float32 [B][out]; all device memory owned by the caller, wq, w_scale, xq
 * and y 16-byte aligned. The integer sums are exact (int32). in must be a
 * multiple of 64 and out of 16 (else WKV7_ERR_UNSUPPORTED). Stacking the
 * weights of several projections (r, w, k, v, a, b) into one [6C][C] matrix
 * runs them in one call. */
wkv7_status wkv7_q8_matmul(const int8_t* wq, const float* w_scale,
                           int64_t out, int64_t in, const int8_t* xq,
                           const float* x_scale, int64_t B, float* y,
                           void* stream);

/* linear — quantize the inputs and multiply: xq, x_scale = wkv7_q8_quantize
 * of x [B][in] (dtype WKV7_F32 or WKV7_BF16) and y = wkv7_q8_matmul of wq,
 * w_scale with them, the same bits as the two calls (page "RWKV-X
 * Architecture", section "INT8 Quantization": the input is quantized once
 * and every output row is an integer dot product, rescaled). For at most
 * four tokens with in <= 2048 (a decode step's projections) it is one
 * launch, which saves the separate quantization launch; otherwise the two.
 * xq int8 [B][in] and x_scale float32 [B] are outputs owned by the caller;
 * wq, w_scale, x, xq and y 16-byte aligned; in a multiple of 64, out of 16
 * (else WKV7_ERR_UNSUPPORTED); inputs finite. */
wkv7_status wkv7_q8_linear(const int8_t* wq, const float* w_scale,
                           int64_t out, int64_t in, const void* x,
                           int32_t dtype, int64_t B, int8_t* xq,
                           float* x_scale, float* y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* WKV7_H */
