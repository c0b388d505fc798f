/*
 * gsz.h -- C ABI of libgsz: one rank's share of a synchronous data-parallel
 * training step with ZeRO-1/2 sharding, on one AMD Instinct MI355X (gfx950).
 *
 * The step, as the pages on data-parallel gradient synchronisation state it:
 *   1. pack per-parameter bf16 gradients into ~25 MB buckets in reverse layer
 *      order                                          (gsz_bucket_pack)
 *   2. the reduce-scatter half of a ring all-reduce: the fp32 mean of P rank
 *      contributions for the chunks this rank owns   (gsz_shard_reduce_mean)
 *   3. the squared-norm partial of the owned shard and the clip coefficient
 *      for clipping the global norm at max_norm     (gsz_shard_grad_sqnorm,
 *                                                    gsz_clip_coef)
 *   4. AdamW on the owned shard (fp32 master, m, v) writing bf16 parameters
 *      in all-gather layout                         (gsz_shard_adamw_step,
 *                                                    gsz_allgather_layout_write)
 *
 * Pages cited (title, section):
 *   "Data parallelism in depth" (infra-guide chapter 4.1)
 *   "Distributed Training: Data Parallel, Model Parallel and FSDP Strategies"
 *   "Data Parallelism: DDP, ZeRO and FSDP"
 *   "Data Parallelism: From Parameter Server to Ring All-Reduce"
 *
 * Conventions for every call:
 *   - Return value: GSZ_OK (0) or a negative gsz_status; gsz_last_error()
 *     (thread-local) describes the failure.  Arguments are validated before
 *     any work is enqueued, so an argument error enqueues nothing.  A call
 *     that issues several launches (a pack over more than 256 tensors, a
 *     reduce and its norm finalize) and gets GSZ_ERR_HIP from a later launch
 *     may leave the earlier ones enqueued.
 *   - Sizes are int64_t element counts.  bf16 values travel as uint16_t bit
 *     patterns.
 *   - "device" pointers are HIP device memory owned by the caller; "host"
 *     pointers are ordinary host memory read during the call only.  Device
 *     vector pointers must be 16-byte aligned (GSZ_ERR_MISALIGNED otherwise).
 *   - Device work is enqueued on the caller's hipStream_t (0 = the null
 *     stream) and is asynchronous; no call synchronises the host.
 *   - The library never allocates or frees device memory.  The plan's device
 *     tables (gsz_plan_device_bytes) and scratch space (gsz_workspace_bytes)
 *     live in buffers the caller provides.
 *   - Device calls refuse any device that is not gfx950 (GSZ_ERR_DEVICE).
 */
#ifndef GSZ_H
#define GSZ_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gsz_status {
    GSZ_OK = 0,
    GSZ_ERR_INVALID_ARG = -1,   /* null pointer, negative size, bad enum ...     */
    GSZ_ERR_MISALIGNED = -2,    /* a device pointer is not 16-byte aligned        */
    GSZ_ERR_SIZE = -3,          /* sizes disagree with the plan or a limit         */
    GSZ_ERR_BAD_RANK = -4,      /* owner rank outside [0, world_size)              */
    GSZ_ERR_PLAN_MISMATCH = -5, /* two ranks built different bucket plans          */
    GSZ_ERR_NOT_UPLOADED = -6,  /* plan has no device tables on the current device */
    GSZ_ERR_DEVICE = -7,        /* current device is not gfx950                    */
    GSZ_ERR_HIP = -8,           /* a HIP runtime call failed (text in last_error)  */
    GSZ_ERR_NO_MEMORY = -9      /* host allocation failed                          */
} gsz_status;

/* Largest number of simulated ranks one call accepts (contribution pointers
 * travel in the kernel argument block). */
#define GSZ_MAX_RANKS 256

/* Contribution layouts for gsz_shard_reduce_mean. */
#define GSZ_LAYOUT_BUCKET_FLAT 0    /* contrib[q]: rank q's whole bucket-major flat
                                       buffer (flat_len elements); the owner's chunk
                                       of bucket b is read at base_b + owner*C_b     */
#define GSZ_LAYOUT_SHARD_COMPACT 1  /* contrib[q]: the shard_len elements rank q
                                       sends to this owner, chunks in bucket order   */
#define GSZ_LAYOUT_RANK_INTERLEAVED 2
                                    /* contrib[0] (one pointer): a single receive
                                       buffer of P * ceil(S / 512) * 512 elements in
                                       which rank q's values for shard elements
                                       [512t, 512t + 512) sit at (t*P + q)*512 (the
                                       last tile's pieces are full slots, their
                                       tails unread); contrib[1..] are not read.
                                       One tile's P pieces are one contiguous
                                       stretch, so the reduce streams one buffer.   */
#define GSZ_INTERLEAVE_PIECE 512     /* elements per rank piece of the layout above */

typedef struct gsz_plan gsz_plan;

typedef struct gsz_plan_info {
    int32_t n_tensors;
    int32_t n_buckets;
    int32_t world_size;        /* P */
    int32_t align;             /* padding granule per rank, elements */
    int64_t bucket_cap_bytes;
    int64_t flat_len;          /* sum of padded bucket lengths */
    int64_t shard_len;         /* S = flat_len / P */
    int64_t n_params;          /* sum of tensor sizes */
    uint64_t hash;             /* FNV-1a 64 of the plan's canonical description */
} gsz_plan_info;

typedef struct gsz_bucket_info {
    int32_t first_tensor;      /* forward index of the bucket's first tensor; the
                                  bucket holds first_tensor, first_tensor-1, ...  */
    int32_t n_tensors;
    int64_t base;              /* flat offset of the bucket */
    int64_t n_elems;           /* gradient elements before padding */
    int64_t padded;            /* L_b, a multiple of world_size * align */
    int64_t chunk;             /* C_b = L_b / world_size */
    int64_t shard_off;         /* offset of this bucket's chunk inside every shard */
} gsz_bucket_info;

typedef struct gsz_adamw_hp {
    double lr;
    double beta1;
    double beta2;
    double eps;
    double weight_decay;
    int64_t step;              /* t >= 1: the exponent of this update's bias corrections */
} gsz_adamw_hp;

/* ---------------------------------------------------------------- plan --- */

/* Builds the bucket plan ("Data parallelism in depth" §4.2, The Bucket
 * mechanism; "Data Parallelism: DDP, ZeRO and FSDP", DDP section; "Data
 * Parallelism: From Parameter Server to Ring All-Reduce" §5).
 *   numel[n_tensors] (host): tensor sizes in forward (compute) order.
 * Tensors are taken in reverse order; each is appended to the open bucket,
 * which closes as soon as its bf16 byte size reaches bucket_cap_bytes; the
 * last bucket holds the rest.  A bucket of n elements is zero-padded to
 * L = ceil(n / (P*align)) * P*align; rank r owns chunk r (length L/P) of every
 * bucket and its shard is those chunks concatenated in bucket order.
 * Host only (no device call).  *out receives a plan owned by the caller;
 * release it with gsz_plan_destroy.  n_tensors may be 0; sizes may be 0.
 * GSZ_ERR_SIZE if the sizes add up to more than 2^48 elements. */
int gsz_plan_create(const int64_t* numel, int32_t n_tensors, int64_t bucket_cap_bytes,
                    int32_t world_size, int32_t align_elems, gsz_plan** out);

/* Frees the plan (host memory only; the device tables are the caller's
 * buffer).  NULL is accepted. */
int gsz_plan_destroy(gsz_plan* plan);

int gsz_plan_get_info(const gsz_plan* plan, gsz_plan_info* out);

/* Bucket b in bucket order (0 = the bucket holding the last forward tensors). */
int gsz_plan_bucket(const gsz_plan* plan, int32_t b, gsz_bucket_info* out);

/* Flat offset and bucket of forward tensor t. */
int gsz_plan_tensor(const gsz_plan* plan, int32_t t, int64_t* flat_offset, int32_t* bucket);

/* Every rank must issue its buckets in the same order ("Data Parallelism:
 * DDP, ZeRO and FSDP", DDP section; "Data parallelism in depth" §4.2 on
 * unused parameters).  Compares this plan's hash with a peer's:
 * GSZ_OK if equal, GSZ_ERR_PLAN_MISMATCH otherwise. */
int gsz_plan_check(const gsz_plan* plan, uint64_t peer_hash);

/* *out = bytes of device memory the plan's tables take (gsz_plan_upload):
 * per bucket {shard offset, flat base, chunk length}, per tensor {flat offset,
 * size, first pack tile}, per padded bucket {start, length}, and two lookup
 * tables of at most 2^16 cells (tile -> tensor, shard index -> bucket), 8
 * bytes per entry: at most 1,048,640 + 24 * n_tensors + 40 * n_buckets. */
int gsz_plan_device_bytes(const gsz_plan* plan, size_t* out);

/* Copies the plan's device tables into dev_tables (device memory on the
 * current device, owned by the caller, 16-byte aligned, at least
 * gsz_plan_device_bytes long), enqueued on `stream`; the source is the plan's
 * own host image, so the copy may complete after the call returns (the HIP
 * runtime may stage the pageable source before returning; nothing waits for
 * the device).  Every later device call that takes this plan reads the tables
 * there, on this device, and must be ordered after the copy (the same stream,
 * or an event).  The caller keeps dev_tables alive and unmodified while such
 * calls may run, and until it uploads the plan again (to another buffer or
 * device) or destroys it.  Not to be called while device calls on the same
 * plan are being issued from other threads (the plan is otherwise read-only
 * and may be shared between threads).  GSZ_ERR_SIZE if bytes is too small,
 * GSZ_ERR_MISALIGNED, GSZ_ERR_INVALID_ARG for a NULL buffer. */
int gsz_plan_upload(gsz_plan* plan, void* dev_tables, size_t bytes, hipStream_t stream);

/* ------------------------------------------------------------- ledger --- */

/* Model-state bytes per parameter per rank ("Data Parallelism: DDP, ZeRO and
 * FSDP", sections The memory ledger and The three stages): zero_stage 0 (DDP)
 * 16, 1: 4 + 12/P, 2: 2 + 14/P, 3: 16/P. */
int gsz_ledger_bytes_per_param(int32_t world_size, int32_t zero_stage, double* out);

/* *out = bytes of device scratch that gsz_shard_reduce_mean (n = the plan's
 * shard_len) or gsz_shard_grad_sqnorm (n = its element count) needs, per call
 * in flight: one fp64 partial per 2048 elements (at most 2^23 of them) plus
 * 1024 for the second stage of the fixed-order sum, i.e. 8 * (min(ceil(n /
 * 2048), 2^23) + 1024) with ceil(0 / 2048) taken as 1 (an upper bound: the
 * reduce of a large shard at P > 16 writes one partial per compute unit).
 * About 0.4% of the bytes of the fp32 values it reduces.  Needs no
 * initialisation.
 * GSZ_ERR_INVALID_ARG if n < 0 or out is NULL. */
int gsz_workspace_bytes(int64_t n, size_t* out);


/* -------------------------------------------------------------- steps --- */

/* Step 1: flat[base_b + ...] <- gradients of bucket b in bucket order, zero pads.
 *   grads (host array of n_tensors device pointers, forward order): tensor t
 *     holds numel[t] bf16 values; any alignment (unaligned tensors take a
 *     slower element path); NULL only when numel[t] == 0.
 *   flat (device, flat_len bf16, 16-byte aligned): written entirely.
 * Source: "Data parallelism in depth" §4.2; "Distributed Training ...",
 * section Inside DDP (25 MB buckets, gradient_as_bucket_view). */
int gsz_bucket_pack(const gsz_plan* plan, const uint16_t* const* grads, uint16_t* flat,
                    hipStream_t stream);

/* Step 2 (+ the squared-norm partial of step 3 when partial_out != NULL):
 *   g[i] = (((c[r+1] + c[r+2]) + ...) + c[r]) / P     in fp32, i in [0, S)
 * with c[q] the bf16 value rank q contributes for element i of owner r's shard
 * (indices mod P); each addition is an IEEE fp32 add, the division is exact
 * IEEE division.  This is the reduce-scatter of "Data Parallelism: From
 * Parameter Server to Ring All-Reduce" §5 (chunk c's partial sum starts at
 * rank c+1 and takes one fp32 addition per hop around the ring, ending at its
 * owner c), averaged as in "Data parallelism in depth" §2, accumulated in fp32 as in
 * "Distributed Training ...", section FSDP1 vs FSDP2 (reduce_dtype=fp32).
 *   contrib (host array of device pointers, 16-byte aligned): P buffers for
 *     GSZ_LAYOUT_BUCKET_FLAT (flat_len elements each) and
 *     GSZ_LAYOUT_SHARD_COMPACT (S each); one receive buffer for
 *     GSZ_LAYOUT_RANK_INTERLEAVED (P * ceil(S/512) * 512 elements).  The three
 *     layouts give the same g and partial bit for bit.
 *   g (device, S fp32): written.
 *   partial_out (device, one double, may be NULL): sum of g[i]^2 in fp64.
 *   ws (device, >= gsz_workspace_bytes): scratch, required if partial_out.
 * Deterministic: the same inputs give the same bits on the same device. */
int gsz_shard_reduce_mean(const gsz_plan* plan, int32_t owner,
                          const uint16_t* const* contrib, int32_t layout,
                          float* g, double* partial_out, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/* Step 3, standalone: *partial_out = sum_i g[i]^2 in fp64, i in [0, n)
 * (device pointers; ws as above).  Clipping at 1.0 by the global L2 norm:
 * "Distributed Training ...", section Inside DDP (clip_grad_norm_(..., 1.0)). */
int gsz_shard_grad_sqnorm(const float* g, int64_t n, double* partial_out, void* ws,
                          size_t ws_bytes, hipStream_t stream);

/* Step 3, finalize (one tiny kernel, no host sync):
 *   total = partials[0] + partials[1] + ... (fp64, rank order)
 *   norm  = fp32(sqrt(total));  coef = min(1, max_norm / (norm + 1e-6)) in fp32.
 *   partials (device, n_partials doubles); coef_out (device float);
 *   norm_out (device float, may be NULL); total_out (device double, may be NULL). */
int gsz_clip_coef(const double* partials, int32_t n_partials, float max_norm, float* coef_out,
                  float* norm_out, double* total_out, hipStream_t stream);

/* Step 4: AdamW on owner r's shard, in place, element by element in fp32 with
 * one IEEE rounding per operation and no fused multiply-add:
 *   gc = g*coef; m = b1*m + (1-b1)*gc; v = b2*v + (1-b2)*(gc*gc);
 *   u = (m/(1-b1^t)) / (sqrt(v/(1-b2^t)) + eps); theta = theta*(1-lr*wd) - lr*u;
 *   p = bf16(theta) (round to nearest even).
 * The fp32 constants are formed in double from hp and rounded once.
 * AdamW(lr=2e-4, weight_decay=0.1): "Distributed Training ...", section
 * Inside DDP; the owned-shard update and all-gather of updated parameters:
 * "Data Parallelism: DDP, ZeRO and FSDP", section The three stages.
 *   master, m, v, g (device, S fp32); coef (device float, from gsz_clip_coef).
 *   gathered (device, flat_len bf16, may be NULL): p written at
 *     base_b + r*C_b + j (all-gather layout); other elements untouched.
 *   shard_bf16 (device, S bf16, may be NULL): p in shard layout.
 *   At least one of gathered / shard_bf16 must be given. */
int gsz_shard_adamw_step(const gsz_plan* plan, int32_t owner, float* master, float* m, float* v,
                         const float* g, const float* coef, const gsz_adamw_hp* hp,
                         uint16_t* gathered, uint16_t* shard_bf16, hipStream_t stream);

/* All-gather layout writer: gathered[base_b + r*C_b + j] = shard[shard_off_b + j]
 * for every bucket b ("Data Parallelism: DDP, ZeRO and FSDP", section The three
 * stages; "Data Parallelism: From Parameter Server to Ring All-Reduce" §5,
 * all-gather).  shard_bf16 (device, S bf16); gathered (device, flat_len bf16). */
int gsz_allgather_layout_write(const gsz_plan* plan, int32_t owner, const uint16_t* shard_bf16,
                               uint16_t* gathered, hipStream_t stream);

/* --------------------------------------- gradient accumulation --- */

/* Gradient accumulation between synchronisations (the no_sync loop of
 * "Distributed Training: Data Parallel, Model Parallel and FSDP Strategies",
 * section Selecting and Tuning Your Strategy; gradients as views of the
 * buckets, section Inside DDP): for every tensor,
 *   flat[off_t + j] = bf16(f32(flat[off_t + j]) + f32(grads[t][j]))
 * (one fp32 add, rounded to nearest even).  Pads are not touched.  The first
 * micro-batch of a window is written with gsz_bucket_pack.  Arguments as for
 * gsz_bucket_pack. */
int gsz_bucket_accumulate(const gsz_plan* plan, const uint16_t* const* grads, uint16_t* flat,
                          hipStream_t stream);

/* The same accumulation into fp32 buckets (reduce_dtype = fp32: "Distributed
 * Training ...", section FSDP1 vs FSDP2 and DTensor).  flat32 (device,
 * flat_len fp32, 16-byte aligned) is the bucket-major buffer in fp32.
 *   gsz_bucket_pack_f32:        flat32[off_t + j] = f32(grads[t][j]) (exact), pads 0
 *                               (the first micro-batch of a window);
 *   gsz_bucket_accumulate_f32:  flat32[off_t + j] = flat32[off_t + j] + f32(grads[t][j])
 *                               (one fp32 add, nearest even); pads not touched.
 * grads as for gsz_bucket_pack.  The buffers then feed gsz_shard_reduce_mean_f32. */
int gsz_bucket_pack_f32(const gsz_plan* plan, const uint16_t* const* grads, float* flat32,
                        hipStream_t stream);
int gsz_bucket_accumulate_f32(const gsz_plan* plan, const uint16_t* const* grads, float* flat32,
                              hipStream_t stream);

/* --------------------------------------------- reduce-dtype variant --- */

/* gsz_shard_reduce_mean with bf16 partial sums on the wire ("Data Parallelism:
 * From Parameter Server to Ring All-Reduce" §8: the communication dtype changes
 * numerics): after every addition the partial sum is rounded to bf16 (nearest
 * even), as a ring carrying bf16 does; the owner's sum is divided by P in
 * fp32.  Same arguments and outputs as gsz_shard_reduce_mean. */
int gsz_shard_reduce_mean_bf16_wire(const gsz_plan* plan, int32_t owner,
                                    const uint16_t* const* contrib, int32_t layout, float* g,
                                    double* partial_out, void* ws, size_t ws_bytes,
                                    hipStream_t stream);

/* gsz_shard_reduce_mean without a workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The norm partials live in a fixed array
 * inside the library, one per device (8,396,800 bytes, held from the first
 * call on a device until the process ends), so shard_len may be at most 2^31
 * elements (GSZ_ERR_SIZE otherwise).  Arguments, outputs, results (bit for bit)
 * and errors otherwise as gsz_shard_reduce_mean.  Nothing needs clearing
 * between calls: every call writes the partials it reads.  Calls on the same
 * device share the array: calls that may overlap (different streams, or
 * different threads with no ordering between their streams) race and must be
 * serialised by the caller.  Allocates nothing; the first call on a device
 * looks up that device's copy of the array. */
int gsz_shard_reduce_mean_noalloc(const gsz_plan* plan, int32_t owner,
                                  const uint16_t* const* contrib, int32_t layout, float* g,
                                  double* partial_out, hipStream_t stream);

/* gsz_shard_reduce_mean over fp32 contributions (fp32 accumulation buckets,
 * fp32 on the wire; reduce_dtype = fp32, "Distributed Training ...", section
 * FSDP1 vs FSDP2 and DTensor): the same ring order
 * ((c_{r+1} + c_{r+2}) + ...) + c_r and division by P, the inputs taken as they
 * are.  contrib: P device pointers to fp32 buffers (flat_len for
 * GSZ_LAYOUT_BUCKET_FLAT, S for GSZ_LAYOUT_SHARD_COMPACT), or one fp32 receive
 * buffer of P * ceil(S/512) * 512 for GSZ_LAYOUT_RANK_INTERLEAVED; 16-byte aligned.
 * Other arguments, outputs and errors as gsz_shard_reduce_mean. */
int gsz_shard_reduce_mean_f32(const gsz_plan* plan, int32_t owner, const float* const* contrib,
                              int32_t layout, float* g, double* partial_out, void* ws,
                              size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------- unshard side and DDP --- */

/* Inverse of gsz_bucket_pack: params[t][j] = flat[off_t + j] for every tensor
 * (the reader of all-gathered parameters, "Data Parallelism: DDP, ZeRO and
 * FSDP", section How FSDP actually runs; the consumer side of ZeRO-1/2's
 * all-gather, section The three stages).  flat (device, flat_len bf16,
 * 16-byte aligned); params (host array of n_tensors device pointers, forward
 * order, any alignment; NULL only for empty tensors).  Pads are not read. */
int gsz_bucket_unpack(const gsz_plan* plan, const uint16_t* flat, uint16_t* const* params,
                      hipStream_t stream);

/* DDP / NO_SHARD all-reduce as local arithmetic ("Data parallelism in depth"
 * §4 and §5.1: all-reduce = reduce-scatter + all-gather; "Data Parallelism:
 * From Parameter Server to Ring All-Reduce" §5): g_flat[p] = the ring-order
 * mean of the P bucket-flat contributions at flat position p, where the ring
 * of chunk c ends at rank c -- so chunk c of g_flat is bit-identical to what
 * gsz_shard_reduce_mean gives owner c.  contrib (host array of P device
 * pointers, each flat_len bf16); g_flat (device, flat_len fp32).
 * partials (device, P doubles, may be NULL): partials[c] = the squared norm of
 * chunk-owner c's part of g_flat (fp64, as gsz_shard_reduce_mean's partial for
 * owner c), fused into the same pass, so gsz_clip_coef over them gives the
 * global clip coefficient with no separate norm pass.  ws/ws_bytes as for
 * gsz_shard_reduce_mean (gsz_workspace_bytes(shard_len)); required if partials. */
int gsz_allreduce_mean(const gsz_plan* plan, const uint16_t* const* contrib, float* g_flat,
                       double* partials, void* ws, size_t ws_bytes, hipStream_t stream);

/* The replicated (DDP) optimizer update: the AdamW of gsz_shard_adamw_step on
 * n contiguous elements, bf16 result written contiguously to out_bf16.
 * n must be a multiple of 8; all pointers device, 16-byte aligned. */
int gsz_adamw_step(float* master, float* m, float* v, const float* g, int64_t n,
                   const float* coef, const gsz_adamw_hp* hp, uint16_t* out_bf16,
                   hipStream_t stream);

/* ------------------------------------------------------------ errors --- */

const char* gsz_last_error(void);
const char* gsz_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* GSZ_H */
