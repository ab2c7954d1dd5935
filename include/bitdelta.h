/*
 * bitdelta.h - C ABI of libbitdelta, the MI355X (gfx950) BitDelta path.
 *
 * Method: the page "BitDelta: Tek bir GPU kümesinden 14 Zen modeli sunmak"
 * (hanzo.blog, 2026-02-28; Spanish translation on hanzo-blog.hanzo.app).
 * A fine-tuned weight W_ft is served as the shared base W_base plus a one-bit
 * code of its task vector: W_ft ~ W_base + alpha * sign(W_ft - W_base), with
 * alpha = mean|W_ft - W_base| (section "Matematiksel temel"), and the linear
 * layer y = x * (W_base + alpha * sign(Delta))^T is computed in one kernel
 * pass without writing the effective weight to memory (section "Sunum
 * mimarisi", the conceptual fused kernel).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers marked "device" are HIP device pointers; the caller allocates
 *   and owns every buffer.  The library allocates no memory and keeps no
 *   state between calls beyond cached device attributes; calls on different
 *   streams may run concurrently.
 * - bf16 values are passed as uint16_t bit patterns (the top half of an IEEE
 *   float32).
 * - Matrices are row-major: W [d_out, d_in], x [M, d_in], y [M, d_out].
 *   The page's activations [batch, seq, d_in] are passed flattened to
 *   [batch*seq, d_in].
 * - Packed signs: uint64 [d_out, d_in/64].  Element c of row r is bit
 *   (c mod 64) of word (c div 64) of row r, least significant bit first; bit
 *   value 1 means sign +1; sign(0) = +1.  On a little-endian machine the same
 *   bytes read as uint8/int8 [d_out, d_in/8], 8 signs per byte along the
 *   input dimension (section "Altyapı ayrıntıları": a 4096x4096 weight packs
 *   to 4096x512 bytes).  Exactly d_out*d_in/8 bytes.
 * - alpha: float32, one value (BITDELTA_ALPHA_PER_MATRIX) or d_out values
 *   (BITDELTA_ALPHA_PER_ROW, one per output dimension as the page stores it).
 * - stream: a hipStream_t passed as void*; NULL means the null stream.  All
 *   GPU work is enqueued on it asynchronously.  The returned status reports
 *   argument checks (done on the host before anything is enqueued) and
 *   launch errors only.
 * - Shapes: d_out >= 1, d_in >= 64 and d_in % 64 == 0, M >= 1.  d_out and
 *   M must each fit in a signed 32-bit int, d_in is at most 2^30, and
 *   d_out*d_in is below 2^40.
 * - Alignment: x, w_ft, w_base, packed and y must be 16-byte aligned.
 * - Outputs must not overlap inputs (checked: BITDELTA_ERR_OVERLAP).
 * - Data errors are encoded in values, never reported by status: a scope
 *   (row or matrix) whose delta is non-finite or has |delta| >= 2^15 gets
 *   alpha = NaN (bits 0x7FC00000); NaN alpha propagates to the outputs.
 */
#ifndef BITDELTA_H
#define BITDELTA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define BITDELTA_OK 0
#define BITDELTA_ERR_NULL 1      /* a required pointer is NULL */
#define BITDELTA_ERR_SHAPE 2     /* M, d_out or d_in out of range, d_in % 64 != 0 */
#define BITDELTA_ERR_ALIGN 3     /* a buffer is not 16-byte aligned */
#define BITDELTA_ERR_MODE 4      /* alpha_mode is not 0 or 1 */
#define BITDELTA_ERR_VARIANTS 5  /* n_variants outside [1, BITDELTA_MAX_VARIANTS] */
#define BITDELTA_ERR_WORKSPACE 6 /* workspace missing or smaller than required */
#define BITDELTA_ERR_HIP 7       /* the HIP runtime reported an error at launch */
#define BITDELTA_ERR_DEVICE 8    /* the current device is not a gfx950 GPU */
#define BITDELTA_ERR_OVERLAP 9   /* an output buffer overlaps an input buffer */
#define BITDELTA_ERR_CACHE 10    /* delta cache: parameter or variant out of range,
                                    or a call out of order */

/* alpha_mode values. */
#define BITDELTA_ALPHA_PER_MATRIX 0
#define BITDELTA_ALPHA_PER_ROW 1

/* Most variants one bitdelta_linear_multi call can address (their pointers
 * travel in the kernel arguments). */
#define BITDELTA_MAX_VARIANTS 64

/*
 * bitdelta_compress_workspace_size
 * Bytes of device workspace bitdelta_compress needs for this shape and mode:
 * 16 bytes per row in per-matrix mode (exact integer partial sums of the
 * scale, one per row), 0 in per-row mode.  Returns 0 for invalid arguments.
 */
size_t bitdelta_compress_workspace_size(int64_t d_out, int64_t d_in, int alpha_mode);

/*
 * bitdelta_compress - compress one fine-tuned weight matrix against its base.
 *
 * Computes Delta = W_ft - W_base (section "Matematiksel temel", Delta
 * equation) per element as one float32 subtraction of the widened bf16
 * values (round to nearest even, subnormals kept), writes sign(Delta) packed
 * as described above (section "Altyapı ayrıntıları"), and writes
 * alpha = mean|Delta| over each scope (section "Matematiksel temel", alpha
 * equation).  The mean is defined exactly: S = sum of floor(|d| * 2^48) as an
 * integer, alpha = S / (n * 2^48) rounded once to float32 (nearest, ties to
 * even), n the scope's element count.  The result does not depend on the
 * order of summation, so it is bit-reproducible.
 *
 *   w_ft, w_base  device, bf16 [d_out, d_in], read only
 *   packed        device, uint64 [d_out, d_in/64], written
 *   alpha         device, float32 [1] (per matrix) or [d_out] (per row), written
 *   workspace     device, >= bitdelta_compress_workspace_size(...) bytes, or
 *                 NULL when that size is 0; contents are scratch
 *   stream        hipStream_t or NULL
 * Returns BITDELTA_OK or an error status; nothing is enqueued on error.
 */
int bitdelta_compress(const uint16_t* w_ft, const uint16_t* w_base, int64_t d_out,
                      int64_t d_in, int alpha_mode, uint64_t* packed, float* alpha,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * bitdelta_compress_noalloc - bitdelta_compress for callers that cannot
 * allocate memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same computation and results, with
 * no workspace argument and no allocation of any kind.  In per-matrix mode
 * the per-row partial sums live in a scratch array of 4 MiB that the library
 * keeps on each GPU it runs on until the process ends, so d_out is limited to
 * 262144 rows there (BITDELTA_ERR_WORKSPACE beyond); per-row mode needs no
 * scratch and takes any shape bitdelta_compress takes.  All calls on one GPU
 * share that GPU's scratch: per-matrix calls that may overlap in time on one
 * GPU (different streams, or concurrent graph replays) race and must be
 * ordered by the caller.  Every partial sum a call reads was written by that
 * call, so nothing needs clearing between calls.
 * Arguments, layout, ownership and errors otherwise as bitdelta_compress;
 * BITDELTA_ERR_HIP if the scratch's device address cannot be obtained.
 */
int bitdelta_compress_noalloc(const uint16_t* w_ft, const uint16_t* w_base, int64_t d_out,
                              int64_t d_in, int alpha_mode, uint64_t* packed, float* alpha,
                              void* stream);

/*
 * bitdelta_linear - fused BitDelta linear for one variant:
 *   y[m, o] = sum_i x[m, i] * (W_base[o, i] + alpha_o * s[o, i]),   no bias
 * (section "Sunum mimarisi", the conceptual fused kernel; s from the packed
 * signs, alpha_o = alpha[o] per row or alpha[0] per matrix).  The effective
 * weight is never written to memory.  Accumulation is in float32, y is
 * rounded to bf16 (nearest even).  M <= 64 runs the decode-shaped kernel
 * (base and sign products on the matrix cores, one pass over W_base and the
 * packed signs); larger M runs the prefill GEMM, which rebuilds bf16 tiles of
 * W_eff in LDS.  Both address their tiles with 32-bit buffer offsets, which
 * limits d_in to 16777152 when M <= 64 and to 4194240 when M > 64
 * (BITDELTA_ERR_SHAPE beyond).
 *
 *   x       device, bf16 [M, d_in]
 *   w_base  device, bf16 [d_out, d_in]
 *   packed  device, uint64 [d_out, d_in/64]
 *   alpha   device, float32 [1] or [d_out]
 *   y       device, bf16 [M, d_out], written
 * Returns BITDELTA_OK or an error status; nothing is enqueued on error.
 */
int bitdelta_linear(const uint16_t* x, int64_t M, const uint16_t* w_base,
                    const uint64_t* packed, const float* alpha, int alpha_mode,
                    int64_t d_out, int64_t d_in, uint16_t* y, void* stream);

/*
 * bitdelta_linear_multi - one token batch that mixes variants of one base
 * (section "Sunum mimarisi": many variants' deltas served over one shared,
 * read-only base; section "Altyapı ayrıntıları": per-variant routing).
 * Token m uses variant v = variant_ids[m]:
 *   y[m] = x[m] * W_base^T + alpha_v (.) (x[m] * S_v^T)
 * and v = -1 selects the base model alone.  W_base is streamed once for all
 * tokens and each distinct variant's packed signs once.  An id outside
 * [-1, n_variants) makes that token's output row NaN (nothing out of bounds
 * is read).  Tokens are processed in groups of 64 (one pass over the weights
 * per group).  d_in is at most 16777152 (the decode-shaped kernel's 32-bit
 * buffer offsets; BITDELTA_ERR_SHAPE beyond).
 *
 *   x            device, bf16 [M, d_in]
 *   variant_ids  device, int32 [M]
 *   w_base       device, bf16 [d_out, d_in]
 *   n_variants   1 .. BITDELTA_MAX_VARIANTS
 *   packed       HOST array of n_variants device pointers, each uint64
 *                [d_out, d_in/64], none NULL
 *   alpha        HOST array of n_variants device pointers, float32 [1] or
 *                [d_out] each according to alpha_mode, none NULL
 *   y            device, bf16 [M, d_out], written
 * The host arrays are read during the call only.
 * Returns BITDELTA_OK or an error status; nothing is enqueued on error.
 */
int bitdelta_linear_multi(const uint16_t* x, int64_t M, const int32_t* variant_ids,
                          const uint16_t* w_base, int32_t n_variants,
                          const uint64_t* const* packed, const float* const* alpha,
                          int alpha_mode, int64_t d_out, int64_t d_in, uint16_t* y,
                          void* stream);

/*
 * bitdelta_reconstruct - the effective weight written out (unfused path):
 *   W_eff[o, i] = bf16(W_base[o, i] + alpha_o * s[o, i])
 * (section "Sunum mimarisi": the W_eff that the fused kernel keeps on chip;
 * a server without it writes W_eff to memory and then runs a standard
 * matmul; section "Matematiksel temel", W_ft ~ W_base + alpha*sign(Delta)).
 * Per element one float32 addition of W_base and +alpha_o or -alpha_o, then
 * rounding to bf16 (nearest even): the same values the prefill GEMM of
 * bitdelta_linear multiplies by.  A NaN alpha gives NaN weights in its scope.
 * Reads 2 + 1/8 bytes and writes 2 bytes per weight.
 *
 *   w_base  device, bf16 [d_out, d_in]
 *   packed  device, uint64 [d_out, d_in/64]
 *   alpha   device, float32 [1] or [d_out] (4-byte aligned)
 *   w_eff   device, bf16 [d_out, d_in], written; must not overlap the inputs
 * Returns BITDELTA_OK or an error status; nothing is enqueued on error.
 */
int bitdelta_reconstruct(const uint16_t* w_base, const uint64_t* packed, const float* alpha,
                         int alpha_mode, int64_t d_out, int64_t d_in, uint16_t* w_eff,
                         void* stream);

/*
 * Delta cache - which variant's packed delta lives in which device slot, and
 * the host-to-device loads that fill the slots (section "Altyapı
 * ayrıntıları": the cold-start paragraph, a delta that is not resident is
 * loaded into device memory on its first request and stays until evicted;
 * the eviction paragraph, least-recently-used eviction weighted by request
 * rate with the highest-rate variants pinned, the page pinning 6 of 14; the
 * routing paragraph, requests for a variant whose delta is loading wait for
 * that load instead of starting another).
 *
 * Policy, exactly:
 * - rate[v] counts requests for v; after every halve_every-th counted
 *   request all rates are halved (integer shift right); halve_every = 0
 *   never halves.  A request is counted first, then the halving applies.
 * - the n_pinned variants of highest rate (ties to the lower id) are pinned:
 *   a resident pinned variant is never evicted (no slot is reserved for a
 *   pinned variant that is not resident).
 * - a request for a resident variant is a HIT; for a variant whose load is in
 *   flight it is QUEUED (no second load); otherwise it is a LOAD into the
 *   lowest-numbered free slot, or into the slot of the evicted variant: the
 *   least recently requested variant that is resident, not pinned, not in
 *   use and not the one requested.  A variant is in use from each request
 *   that returned it until the matching release.  A variant still loading is
 *   never evicted.
 * - with no free slot and nothing to evict the request is FULL and changes
 *   no state (it is not counted); the caller retries later.
 *
 * A cache is a host object.  Without attached memory it runs the policy only
 * (bitdelta_cache_request / _loaded / _release: no HIP call at all).  With
 * memory attached (bitdelta_cache_attach) it moves the bytes itself
 * (bitdelta_cache_acquire / _release / _poll), and the policy-only calls
 * request and loaded are refused.  Calls on one cache are serialised by a
 * lock; the cache allocates host memory only (its state and, once memory is
 * attached, one HIP event per variant and per slot).
 */
typedef struct bitdelta_cache bitdelta_cache;

/* Request outcomes (action). */
#define BITDELTA_CACHE_HIT 0     /* resident and loaded: use the slot */
#define BITDELTA_CACHE_QUEUED 1  /* its load is in flight: wait for it */
#define BITDELTA_CACHE_LOAD 2    /* this request starts the load into the slot */
#define BITDELTA_CACHE_FULL 3    /* nothing can be evicted now; no state changed */

/* Variant states. */
#define BITDELTA_CACHE_ABSENT 0
#define BITDELTA_CACHE_LOADING 1
#define BITDELTA_CACHE_RESIDENT 2

/*
 * bitdelta_cache_create - a cache of n_slots slots for variants
 * 0 .. n_variants-1.  1 <= n_variants, n_slots <= 65536,
 * 0 <= n_pinned < n_slots, halve_every >= 0.  *out receives the cache (NULL
 * on error).  Returns BITDELTA_OK, BITDELTA_ERR_NULL or BITDELTA_ERR_CACHE.
 */
int bitdelta_cache_create(int32_t n_variants, int32_t n_slots, int32_t n_pinned,
                          int64_t halve_every, bitdelta_cache** out);

/* Frees the cache's host state and events (not the caller's memory).  Work
 * already enqueued keeps running.  NULL is ignored. */
void bitdelta_cache_destroy(bitdelta_cache* cache);

/*
 * bitdelta_cache_request - policy only (no memory attached): one request for
 * `variant`.  *action receives HIT, QUEUED, LOAD or FULL, *slot the slot
 * (-1 for FULL), *evicted the variant evicted by a LOAD or -1.  Except for
 * FULL the variant is in use until bitdelta_cache_release.  After a LOAD the
 * caller moves the bytes and reports it with bitdelta_cache_loaded.
 * Returns BITDELTA_ERR_CACHE for a variant out of range or a cache with
 * memory attached.
 */
int bitdelta_cache_request(bitdelta_cache* cache, int32_t variant, int32_t* action,
                           int32_t* slot, int32_t* evicted);

/* Policy only: the load of `variant` has finished (LOADING -> RESIDENT).
 * BITDELTA_ERR_CACHE if it is not loading or memory is attached. */
int bitdelta_cache_loaded(bitdelta_cache* cache, int32_t variant);

/*
 * bitdelta_cache_release - one use of `variant` ends.  With memory attached
 * an event is recorded on `stream` (a hipStream_t, NULL = null stream): a
 * later load into the variant's slot waits for it, so work enqueued on that
 * stream before the release still reads the old bytes.  A slot's releases
 * must come from one stream (or the caller orders its streams).  Without
 * memory `stream` is ignored.  BITDELTA_ERR_CACHE if the variant is not in use.
 */
int bitdelta_cache_release(bitdelta_cache* cache, int32_t variant, void* stream);

/* State (ABSENT / LOADING / RESIDENT), slot (-1 when absent) and current
 * rate of `variant`. */
int bitdelta_cache_state(bitdelta_cache* cache, int32_t variant, int32_t* state,
                         int32_t* slot, int64_t* rate);

/*
 * bitdelta_cache_attach - give the cache its memory, before any request.
 *   slots         HOST array of n_slots device pointers, each 16-byte
 *                 aligned, slot_bytes long, not overlapping
 *   sources       HOST array of n_variants host pointers: the bytes of each
 *                 variant's delta (its packed signs and alpha, in whatever
 *                 layout the caller reads them back from the slot); they
 *                 should be page-locked (hipHostMalloc) for the copy to run
 *                 asynchronously, and must stay valid while the cache lives
 *   source_bytes  HOST array of n_variants sizes, each <= slot_bytes
 * The current device becomes the cache's device.  Creates the events.
 * Returns BITDELTA_ERR_CACHE if a request was made already or a source is
 * larger than a slot, BITDELTA_ERR_ALIGN / _OVERLAP / _NULL for bad slots.
 */
int bitdelta_cache_attach(bitdelta_cache* cache, void* const* slots, size_t slot_bytes,
                          const void* const* sources, const size_t* source_bytes);

/*
 * bitdelta_cache_acquire - one request for `variant` that moves the bytes.
 * First finished loads are marked resident (their events polled), then the
 * request runs the policy.  LOAD: copy_stream waits for the slot's last
 * release event, the variant's source bytes are copied into the slot
 * (hipMemcpyAsync, host to device, on copy_stream) and the variant's load
 * event is recorded there.  LOAD and QUEUED: use_stream waits for that
 * event.  *slot_ptr receives the slot's device pointer (NULL for FULL):
 * kernels enqueued on use_stream after this call read the variant's bytes.
 * The current device must be the cache's (BITDELTA_ERR_DEVICE otherwise).
 * On BITDELTA_ERR_HIP nothing is left in use.
 */
int bitdelta_cache_acquire(bitdelta_cache* cache, int32_t variant, void* copy_stream,
                           void* use_stream, int32_t* action, void** slot_ptr,
                           int32_t* evicted);

/* Marks loads whose events have completed resident; *n_loaded (may be NULL)
 * receives how many.  BITDELTA_ERR_CACHE without attached memory. */
int bitdelta_cache_poll(bitdelta_cache* cache, int32_t* n_loaded);

/*
 * Router - decode batches fed from a request queue over a delta cache
 * (section "Altyapı ayrıntıları", the routing paragraph: requests are
 * tracked per variant and none waits behind a variant whose delta is
 * loading).  Exactly:
 * - bitdelta_router_submit appends a request (caller's id, variant in
 *   [-1, n_variants); -1 = the base model alone) to the queue;
 * - bitdelta_router_next_batch first registers every unregistered request
 *   with the cache, in arrival order: one cache request each (counted once);
 *   FULL leaves it unregistered for the next batch.  Without cache memory
 *   this is bitdelta_cache_request; with memory attached it is the request
 *   of bitdelta_cache_acquire, whose loads go on copy_stream and which makes
 *   no stream wait (finished loads are polled first).  A registered request
 *   is ready once its variant is resident; a base request is ready at once.
 *   The batch is the ready requests in arrival order, at most max_batch;
 *   they leave the queue.  ids, variants and slots (each >= max_batch
 *   entries, host) receive the batch's request ids, variants and slot
 *   numbers (-1 for base requests); *n its size (0 allowed).  With memory
 *   attached every slot of the batch holds its variant's bytes already.
 * - bitdelta_router_complete releases the variants of a served batch (the
 *   variants array as next_batch wrote it); with memory attached the
 *   releases record their events on use_stream.
 * The cache must outlive the router; router calls lock the router, then the
 * cache.  Returns BITDELTA_ERR_CACHE for a variant out of range,
 * max_batch < 1 or a release of a variant not in use.
 */
typedef struct bitdelta_router bitdelta_router;

int bitdelta_router_create(bitdelta_cache* cache, bitdelta_router** out);
void bitdelta_router_destroy(bitdelta_router* router);
int bitdelta_router_submit(bitdelta_router* router, int64_t request_id, int32_t variant);
int bitdelta_router_next_batch(bitdelta_router* router, int32_t max_batch, void* copy_stream,
                               int64_t* ids, int32_t* variants, int32_t* slots, int32_t* n);
int bitdelta_router_complete(bitdelta_router* router, int32_t n, const int32_t* variants,
                             void* use_stream);
/* Requests still queued (submitted, not yet in a batch). */
int bitdelta_router_pending(bitdelta_router* router, int32_t* n);

/*
 * MonoSoup merge - k fine-tuned checkpoints of one base merged through
 * rank-r truncations of their task vectors (section "MonoSoup": each
 * Delta_i = W_i - W_base is replaced by its rank-r truncated SVD tau_i and
 * W_merged = W_base + (1/k) sum_i tau_i).
 *
 * tau_i = Q_i (Delta_i^T Q_i)^T, where Q_i (orthonormal columns) comes from
 * orthogonal iteration started at omega: Q = orth(Delta omega), then
 * power_iters times Q = orth(Delta orth(Delta^T Q)).  This is the rank-r
 * truncation whenever sigma_r(Delta_i) > sigma_{r+1}(Delta_i), to within
 * about (sigma_{r+1}/sigma_r)^(2 power_iters + 1) relative times a factor
 * from the random start that grows like sqrt(r (d_out - r)); with no gap at r
 * the result is a rank-r approximation of the top subspace found.  Delta is
 * formed per element as one float32 subtraction of the bf16 values; sums are
 * float32 in a fixed order (deterministic).  Directions that vanish (a
 * Delta of rank below r, e.g. a checkpoint equal to the base) are dropped.
 *
 *   w_ft         HOST array of k device pointers, bf16 [d_out, d_in] each
 *   k            1 .. BITDELTA_MONOSOUP_MAX_CHECKPOINTS
 *   w_base       device, bf16 [d_out, d_in]; d_out at most 4194240 and d_in
 *                at most 16777152 (the general shape rules of this header
 *                apply otherwise)
 *   rank         1 .. min(BITDELTA_MONOSOUP_MAX_RANK, d_out, d_in)
 *   power_iters  0 .. BITDELTA_MONOSOUP_MAX_POWER_ITERS
 *   omega        device, float32 [d_in, rank], the caller's Gaussian start
 *                (the same start is used for every checkpoint)
 *   w_merged     device, bf16 [d_out, d_in], written: W_base + the mean,
 *                rounded to nearest even
 *   tau_mean     device, float32 [d_out, d_in], written, or NULL
 *   workspace    device, >= bitdelta_monosoup_workspace_size(...) bytes,
 *                16-byte aligned; contents are scratch
 * Returns BITDELTA_OK or an error status; nothing is enqueued on error.
 */
#define BITDELTA_MONOSOUP_MAX_RANK 32
#define BITDELTA_MONOSOUP_MAX_CHECKPOINTS 64
#define BITDELTA_MONOSOUP_MAX_POWER_ITERS 64

size_t bitdelta_monosoup_workspace_size(int64_t d_out, int64_t d_in, int32_t k, int32_t rank);
int bitdelta_monosoup_merge(const uint16_t* const* w_ft, int32_t k, const uint16_t* w_base,
                            int64_t d_out, int64_t d_in, int32_t rank, int32_t power_iters,
                            const float* omega, uint16_t* w_merged, float* tau_mean,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * Calibration probes - measured ceilings for the rooflines of the kernels
 * above (they compute nothing of the method).
 *
 * bitdelta_probe_stream_read reads `bytes` (a multiple of 16) of device
 * memory at src (16-byte aligned) once, with 16-byte loads: workgroup b of
 * `workgroups` (256 threads each) reads the b-th contiguous chunk.  sink is
 * device memory of 1024 bytes (4-byte aligned) that the kernel may write; its
 * contents mean nothing.  Time it to get the sustained HBM read rate.
 *
 * bitdelta_probe_mfma_bf16 runs `workgroups` workgroups of 4 waves; every
 * wave issues 8 * iters back-to-back v_mfma_f32_32x32x16_bf16 (8 independent
 * accumulator chains), 32768 flops each: 1048576 * workgroups * iters flops
 * in all.  sink as above.  Time it to get the sustained bf16 matrix-core rate.
 *
 * Both return BITDELTA_OK or an error status (BITDELTA_ERR_SHAPE for sizes
 * out of range); nothing is enqueued on error.
 */
int bitdelta_probe_stream_read(const void* src, size_t bytes, int32_t workgroups, uint32_t* sink,
                               void* stream);
int bitdelta_probe_mfma_bf16(int32_t workgroups, int32_t iters, float* sink, void* stream);

/* bitdelta_probe_decode_loads issues the single-variant decode's loads on a
 * 4096 x 4096 bf16 matrix without its arithmetic, so that the time of the
 * load pattern alone can be set beside the kernel's: 256 workgroups of 4
 * waves, 16 rows each, the 128-element blocks of a row round-robin over the
 * waves, two blocks of loads in flight per wave.  mode 0: contiguous 32 KB
 * per wave; 1: blocks of 16 consecutive rows x 256 bytes; 2: the same with
 * the rows interleaved as the decode kernel takes them; 3: mode 2 by buffer
 * loads to LDS; 4: mode 2 plus each block's sign words; 5: mode 3 plus the
 * sign words plus 1 KB of x per block.  w: 32 MiB (16-byte aligned),
 * signs: 2 MiB (4-byte aligned), x: 8 KiB (16-byte aligned), all read only
 * and all device memory owned by the caller; sink: 1024 bytes of device
 * memory that a chosen xor of the data would be written to (it never is
 * for data of real weights; the caller owns it).  Returns
 * BITDELTA_ERR_NULL, _MODE (mode outside 0..5), _ALIGN, _OVERLAP (sink
 * inside an input) or _HIP; computes nothing of the method. */
int bitdelta_probe_decode_loads(const void* w, const void* signs, const void* x, int32_t mode,
                                uint32_t* sink, void* stream);

/* Human-readable text of a status code (static storage, never NULL). */
const char* bitdelta_status_string(int status);

/*
 * bitdelta_ratio_to_f32_bits - host copy of the scale's final rounding step:
 * float32 bits of S / (n * 2^48) rounded to nearest, ties to even, where
 * S = s_hi * 2^64 + s_lo.  The device kernels use the same routine; it is
 * exported so the rounding can be checked without a GPU.  Returns 0 for
 * S = 0 and 0x7FC00000 for n = 0.
 */
uint32_t bitdelta_ratio_to_f32_bits(uint64_t s_hi, uint64_t s_lo, uint64_t n);

#ifdef __cplusplus
}
#endif

#endif /* BITDELTA_H */
