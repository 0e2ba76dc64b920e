/*
 * fastar.h -- C ABI of the FAST-AR attention step for AMD Instinct MI355X (gfx950).
 *
 * One autoregressive denoising step's attention over a bounded KV cache, as
 * described on the FAST-AR pages ("Fast Autoregressive Video Diffusion and
 * World Models with Temporal Cache Compression and Sparse Attention"; the
 * gist.science technical summary, "2. Core Components", and the FAST-AR blog
 * post, sections "1. TempCache", "2. AnnCA", "3. AnnSA").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer argument is a DEVICE pointer unless marked "host".
 *  - Tensors are dense and row-major: [H][N][d] means d is fastest, then N,
 *    then the head index H.  Heads are fully independent.
 *  - Element types: FASTAR_F32 (IEEE binary32) or FASTAR_BF16 (bfloat16 bits
 *    stored as uint16).  Hyperplanes are always fp32.  d is 64 or 128.
 *  - ``P`` is the number of hyperplanes; bucket ids are in [0, 2^P).  The
 *    bucketed calls accept P in [0, FASTAR_MAX_PLANES]; ``fastar_ann_hash``
 *    accepts P up to FASTAR_MAX_HASH_PLANES.  Id bits at or above P are
 *    ignored wherever ids are consumed.
 *  - ``stream`` is a hipStream_t (NULL = the default stream).  Every call only
 *    enqueues work on that stream and returns without synchronising the host;
 *    results are valid once the stream has reached that point.
 *  - The caller owns all memory: inputs, outputs, the cache and the scratch
 *    workspace.  The library allocates no device memory.  A workspace must be
 *    at least the size returned by the matching ``*_workspace`` query and is
 *    clobbered by the call; buffers must stay alive until the stream work has
 *    completed.  Calls on one stream are ordered; two calls that share a
 *    workspace or a cache must not run concurrently on different streams.
 *  - Arguments are validated on the host before anything is launched.  A
 *    negative status means nothing was enqueued and nothing was modified.
 *    FASTAR_EHIP reports a HIP launch error after validation; outputs (and,
 *    for fastar_tempcache_update, the cache) are then undefined.
 *  - Sizes are int32; every tensor must hold fewer than 2^31 elements, and
 *    one head's rows of a K or V tensor fewer than 2^32 bytes (FASTAR_EINVAL).
 *  - Pointers to d-wide tensors (activations, cache K/V, planes) must be
 *    16-byte aligned (FASTAR_EINVAL otherwise); a tensor with no elements
 *    may be passed as NULL.
 */
#ifndef FASTAR_H
#define FASTAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FASTAR_ABI_VERSION 3
#define FASTAR_MAX_PLANES 10      /* bucketed calls: at most 1024 buckets per head */
#define FASTAR_MAX_HASH_PLANES 16 /* ids are uint16 */
#define FASTAR_MAX_TABLES 8        /* multi-table AnnSA: tables * P <= 16 */
#define FASTAR_MAX_CODEWORDS 65536 /* quantization ids are uint16 */

typedef enum {
    FASTAR_OK = 0,
    FASTAR_EINVAL = -1,      /* null pointer, negative size, bad scalar (non-finite, scale <= 0) */
    FASTAR_EDTYPE = -2,      /* unknown dtype, or dtypes that must agree do not */
    FASTAR_ESHAPE = -3,      /* d not 64/128, P out of range, frame_len not dividing Nq, H mismatch */
    FASTAR_EWORKSPACE = -4,  /* workspace smaller than the query returned (or NULL with size > 0) */
    FASTAR_ECAPACITY = -5,   /* a chunk larger than the cache capacity */
    FASTAR_EHIP = -6,        /* HIP error while enqueueing */
    FASTAR_ESCRATCH = -7     /* the call needs more than the static scratch array holds */
} fastar_status;

typedef enum { FASTAR_F32 = 0, FASTAR_BF16 = 1 } fastar_dtype;

/* One attention layer's bounded KV cache, all heads.  The struct itself lives
 * in host memory; its array members are device pointers.
 *   k, v     [H][cap][d] of ``dtype``
 *   ids      [H][cap]  bucket id of the key held in each slot
 *   ts       [H][cap]  timestamp (step) at which each slot was written
 *   knorm    [H][cap]  fp32 norm |k| of the key held in each slot (the
 *                      TempCache cosine search divides by it)
 *   n_valid  [H]       number of valid slots; slots 0..n_valid[h]-1 are valid.
 *   count    [H][cap]  NULL, or the group size m >= 1 of each slot: the cache
 *                      is then a mean-merged cache (summary, Core Components
 *                      A, Lemma 5.1), whose slot j stands for m_j tokens that
 *                      share one key, with v_j their mean value.  Values below
 *                      1 are read as 1.
 * n_valid stays on the device so that a step never waits on the host; values
 * outside [0, cap] are clamped when read.  fastar_tempcache_update maintains
 * every field; a cache filled by other means gets ids and knorm from
 * fastar_ann_hash on its keys (and count = 1 for a fresh merged cache).
 * With count NULL the cache follows the replacement rule: a matched slot takes
 * the newest token, the other tokens that matched it are dropped. */
typedef struct {
    int32_t H;
    int32_t cap;
    int32_t d;
    int32_t dtype;            /* fastar_dtype of k and v */
    void* k;
    void* v;
    uint16_t* ids;
    int32_t* ts;
    int32_t* n_valid;
    float* knorm;
    int32_t* count;           /* NULL: replacement rule; else group sizes (mean merge) */
} fastar_cache;

/* Status name, e.g. "FASTAR_ESHAPE" (static storage, never NULL). */
const char* fastar_status_string(int32_t status);
int32_t fastar_abi_version(void);

/* ------------------------------------------------------------------------
 * ANN bucket ids (summary, Core Components A and B: queries and keys are
 * projected into a shared LSH space; read as random-hyperplane sign hashing).
 *
 *   ids[h][i] = sum_{p<P} [ <x[h][i], planes[h][p]> >= 0 ] << p
 *
 * x       [H][N][d] of ``dtype``      planes  [H][P][d] fp32
 * ids     [H][N] uint16 (output)
 * norms   [H][N] fp32 (output, may be NULL): |x[h][i]|, in the same pass
 * P in [0, 16]; P = 0 puts every token in bucket 0.  The projection is
 * accumulated in fp32; a projection within fp32 rounding of 0 may take either
 * sign.
 * ------------------------------------------------------------------------ */
fastar_status fastar_ann_hash(const void* x, int32_t dtype, int32_t H, int32_t N, int32_t d,
                              const float* planes, int32_t P, uint16_t* ids, float* norms,
                              void* stream);

/* Several token sets hashed with the same planes in one launch (a step's
 * queries and current keys, say): the same result as one fastar_ann_hash per
 * set.  ``x``, ``N``, ``ids`` and ``norms`` are HOST arrays of ``count``
 * entries holding device pointers and sizes; ``norms`` may be NULL or hold
 * NULL entries.  1 <= count <= FASTAR_HASH_BATCH; the sets share H, d, dtype
 * and the planes. */
#define FASTAR_HASH_BATCH 4
fastar_status fastar_ann_hash_batch(int32_t count, const void* const* x, const int32_t* N,
                                    uint16_t* const* ids, float* const* norms, int32_t dtype,
                                    int32_t H, int32_t d, const float* planes, int32_t P,
                                    void* stream);

/* ------------------------------------------------------------------------
 * Quantization bucket ids (summary, Core Components A and B name quantization
 * as the alternative ANN to LSH): each vector's bucket is its nearest codeword
 * of its head's codebook,
 *
 *   ids[h][i] = argmin_c |x[h][i] - codebook[h][c]|^2
 *             = argmax_c <x[h][i], codebook[h][c]> - |codebook[h][c]|^2 / 2
 *
 * with the lowest c on ties.
 * x        [H][N][d] of ``dtype``      codebook  [H][B][d] fp32
 * ids      [H][N] uint16 (output)      norms     [H][N] fp32 (output, may be NULL): |x|
 * 1 <= B <= FASTAR_MAX_CODEWORDS.  The inner products are fp32 sums on the
 * matrix cores; a runner-up within fp32 rounding of the best may be chosen.
 * The ids feed every bucketed call with P = ceil(log2 B) (B <= 2^FASTAR_MAX_PLANES
 * there).  How the codebook is obtained is the caller's choice.
 * ------------------------------------------------------------------------ */
fastar_status fastar_ann_quantize(const void* x, int32_t dtype, int32_t H, int32_t N, int32_t d,
                                  const float* codebook, int32_t B, uint16_t* ids, float* norms,
                                  void* stream);

/* Several token sets quantized with the same codebook in one launch (a
 * step's queries, current keys and prompt keys, say): the same result as one
 * fastar_ann_quantize per set.  Arguments as fastar_ann_hash_batch: ``x``,
 * ``N``, ``ids`` and ``norms`` are HOST arrays of ``count`` entries
 * (1 <= count <= FASTAR_HASH_BATCH) holding device pointers and sizes;
 * ``norms`` may be NULL or hold NULL entries; the sets share H, d, dtype and
 * the codebook. */
fastar_status fastar_ann_quantize_batch(int32_t count, const void* const* x, const int32_t* N,
                                        uint16_t* const* ids, float* const* norms, int32_t dtype,
                                        int32_t H, int32_t d, const float* codebook, int32_t B,
                                        void* stream);

/* ------------------------------------------------------------------------
 * Stable grouping of tokens by bucket -- the block-sparse layout AnnSA runs
 * on (summary, Core Components C).  Exposed for callers that reuse one
 * grouping across layers.
 *
 * ids   [H][N] uint16 (bits >= P ignored)
 * off   [H][2^P + 1] int32 (output): off[h][b] = #tokens of head h with id < b
 * perm  [H][N] int32 (output): perm[h][off[h][b] .. off[h][b+1]) = the token
 *       indices with id b, ascending.  Bit-exact and deterministic.
 * ------------------------------------------------------------------------ */
size_t fastar_bucket_sort_workspace(int32_t H, int32_t N, int32_t P);
fastar_status fastar_bucket_sort(const uint16_t* ids, int32_t H, int32_t N, int32_t P,
                                 int32_t* off, int32_t* perm, void* ws, size_t ws_bytes,
                                 void* stream);

/* ------------------------------------------------------------------------
 * AnnSA: bucket-restricted self-attention (blog, "3. AnnSA"; summary, Core
 * Components C).  Key context of head h = [cache slots 0..n_valid[h]-1 ;
 * the Ncur current keys in token order].  Query i attends to exactly the
 * context keys whose id equals q_ids[h][i]:
 *   out[h][i] = sum_j softmax_j(l_ij) v_j,   l_ij = scale * <q_i, k_j> + b_j,
 *   lse[h][i] = log sum_j exp(l_ij),
 * with out = 0 and lse = -inf when the bucket holds no key.  No causal mask.
 * b_j = 0, except for the slots of a mean-merged cache (cache->count set):
 * b_j = ln m_j, the group-size shift of Lemma 5.1 (summary, Core Components
 * A), which makes a slot of m identical keys attend like the m tokens.
 *
 * q         [H][Nq][d] of ``dtype``      q_ids [H][Nq] uint16
 * cache     host pointer, may be NULL (no cached keys); its H, d and dtype
 *           must equal the call's
 * k_cur, v_cur [H][Ncur][d] of ``dtype``, kcur_ids [H][Ncur]; Ncur may be 0
 * scale     softmax scale, finite and > 0; 1/sqrt(d) is the usual value
 * out       [H][Nq][d] of ``out_dtype`` (FASTAR_F32 or FASTAR_BF16)
 * lse       [H][Nq] fp32, may be NULL
 * best, best_cos  [H][Nq] int32 / fp32, may be NULL (both or neither): the
 *           same pass also returns TempCache's top-1 for each query -- the
 *           cached slot j < n_valid with ids[j] == q_ids[i] of largest
 *           cos(q_i, k_j) = <q_i,k_j> / (|q_i| knorm[j]) (ties: lowest slot;
 *           a zero norm gives 0), or -1 and -inf when the bucket holds no
 *           cached key -- ready to pass to fastar_tempcache_update as
 *           best_in/cos_in.
 * ws        workspace of fastar_annsa_workspace(H, Nq, cap, Ncur, P) bytes,
 *           cap = cache ? cache->cap : 0
 * Products are bf16 x bf16 (or fp32 x fp32) on the matrix cores with fp32
 * accumulation; softmax is fp32.
 * ------------------------------------------------------------------------ */
size_t fastar_annsa_workspace(int32_t H, int32_t Nq, int32_t cap, int32_t Ncur, int32_t P);
fastar_status fastar_annsa_forward(const void* q, const uint16_t* q_ids, int32_t H, int32_t Nq,
                                   int32_t d, int32_t dtype, const fastar_cache* cache,
                                   const void* k_cur, const void* v_cur, const uint16_t* kcur_ids,
                                   int32_t Ncur, int32_t P, float scale, void* out,
                                   int32_t out_dtype, float* lse, int32_t* best, float* best_cos,
                                   void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * AnnSA for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  The same
 * computation, arguments and results as fastar_annsa_forward, without the
 * workspace arguments: the library's own static device array of
 * FASTAR_STATIC_SCRATCH_BYTES serves as the workspace.  Each device the
 * library runs on holds its own copy of that array (reserved when the
 * library's code is loaded on the device, kept until the process ends); its
 * device address is resolved once per device, on the first call with that
 * device current, and the calling thread's current device must be the
 * stream's device.
 * Every call on one device uses the same array and leaves its contents there;
 * nothing in it needs to start at zero (a call writes every entry it reads
 * before reading it).  Two calls that overlap on one device -- on different
 * streams, or from different host threads -- race on the array: their
 * results are undefined.  Calls on one stream are ordered and safe.
 * Returns FASTAR_ESCRATCH, with nothing enqueued, when
 * fastar_annsa_workspace(H, Nq, cap, Ncur, P) exceeds the array; every other
 * status as fastar_annsa_forward.  Calls no allocating routine.
 * ------------------------------------------------------------------------ */
#define FASTAR_STATIC_SCRATCH_BYTES (16u << 20)
fastar_status fastar_annsa_forward_static(const void* q, const uint16_t* q_ids, int32_t H, int32_t Nq,
                                          int32_t d, int32_t dtype, const fastar_cache* cache,
                                          const void* k_cur, const void* v_cur, const uint16_t* kcur_ids,
                                          int32_t Ncur, int32_t P, float scale, void* out,
                                          int32_t out_dtype, float* lse, int32_t* best, float* best_cos,
                                          void* stream);

/* ------------------------------------------------------------------------
 * Multi-table AnnSA (blog, "3. AnnSA": a token may fall in several buckets;
 * summary, Core Components C).  The ids hold ``tables`` fields of P bits:
 * the bucket of a token in table t is (id >> (t*P)) & (2^P - 1) -- what
 * fastar_ann_hash returns for planes [H][tables*P][d] holding each table's P
 * planes in turn.  Query i attends to the union over tables of the context
 * keys sharing its bucket in that table, each key once:
 *   out[h][i] = sum_{j in U_i} softmax_j(l_ij) v_j,
 *   U_i = { j : some t has field_t(k_j) == field_t(q_i) },
 * l_ij, lse, the empty case, the mean-merge shift and the fused search
 * (now over U_i) as in fastar_annsa_forward, which is the case tables = 1.
 * 1 <= tables <= FASTAR_MAX_TABLES, P <= FASTAR_MAX_PLANES and
 * tables * P <= 16 (FASTAR_ESHAPE otherwise).  The cache's ids must hold the
 * same fields (fastar_tempcache_update copies a written token's id whole).
 * ws: fastar_annsa_multi_workspace(H, Nq, cap, Ncur, d, P, tables) bytes; it
 * also holds each query's running state between the per-table passes.
 * ------------------------------------------------------------------------ */
size_t fastar_annsa_multi_workspace(int32_t H, int32_t Nq, int32_t cap, int32_t Ncur, int32_t d,
                                    int32_t P, int32_t tables);
fastar_status fastar_annsa_multi_forward(const void* q, const uint16_t* q_ids, int32_t H, int32_t Nq,
                                         int32_t d, int32_t dtype, const fastar_cache* cache,
                                         const void* k_cur, const void* v_cur,
                                         const uint16_t* kcur_ids, int32_t Ncur, int32_t P,
                                         int32_t tables, float scale, void* out, int32_t out_dtype,
                                         float* lse, int32_t* best, float* best_cos, void* ws,
                                         size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * AnnCA: frame-relevant prompt pruning + cross-attention (blog, "2. AnnCA";
 * summary, Core Components B).  Queries are split into F = Nq / frame_len
 * frames.  For frame f, prompt token t is kept iff some query of the frame
 * shares its bucket; each query of the frame attends densely (softmax, scale)
 * over the kept tokens of its frame.  No kept token gives out = 0.
 *
 * q [H][Nq][d], q_ids [H][Nq]; kp, vp [H][L][d]; kp_ids [H][L]
 * out        [H][Nq][d] of ``out_dtype``
 * keep       [H][F][L] uint8 (0/1), may be NULL
 * keep_count [H][F] int32, may be NULL
 * frame_len must divide Nq.  L may be 0.  scale: finite and > 0.
 * ws: fastar_annca_workspace(...) bytes -- 0 when L <= 1024, where the
 * attention launch selects each frame's prompt tokens itself; a longer
 * prompt takes a separate selection launch and an [H][F][L] index list.
 * ------------------------------------------------------------------------ */
size_t fastar_annca_workspace(int32_t H, int32_t Nq, int32_t frame_len, int32_t L, int32_t P);
fastar_status fastar_annca_forward(const void* q, const uint16_t* q_ids, int32_t H, int32_t Nq,
                                   int32_t frame_len, int32_t d, int32_t dtype, const void* kp,
                                   const void* vp, const uint16_t* kp_ids, int32_t L, int32_t P,
                                   float scale, void* out, int32_t out_dtype, uint8_t* keep,
                                   int32_t* keep_count, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * TempCache commit of one chunk (blog, "1. TempCache"; summary, Core
 * Components A).  Per head, with n = n_valid[h] before the call:
 *  1. top-1: for each current token i, best[i] = the valid slot j < n with
 *     ids[j] == q_ids[i] maximising cos(q_i, k_j) = <q_i,k_j>/(|q_i| knorm[j])
 *     (ties: lowest j; a zero norm gives cosine 0); -1 and cos = -inf if the
 *     bucket has no slot.  Skipped when best_in and cos_in are given (then
 *     those are used -- e.g. fastar_annsa_forward's best/best_cos; a best_in
 *     value outside [0, n) means "no candidate").
 *  2. matched[i] = best[i] >= 0 && cos[i] >= tau.  Each matched slot is
 *     refreshed with the current token of largest index that matched it
 *     (k, v, id <- the token's k_cur, v_cur, kcur_id; ts <- step; knorm <-
 *     |k_cur|); the other
 *     tokens that matched the same slot are dropped (merged away).
 *     Mean-merged cache (cache->count set; Lemma 5.1, summary, Core
 *     Components A): every token that matched slot j joins its group instead
 *     -- with C_j those tokens and m_j the group size,
 *       v_j <- (m_j v_j + sum_{i in C_j} v_cur_i) / (m_j + |C_j|),
 *       m_j <- m_j + |C_j|,
 *     summed in fp32 in ascending token order and rounded once to the cache
 *     dtype; k, id, ts and knorm are refreshed as above.  Tokens written by
 *     step 3 start groups of size 1.
 *  3. the u unmatched tokens, in token order, fill slots n, n+1, ... up to
 *     cap, then the e = max(0, n + u - cap) non-refreshed slots with the
 *     smallest (ts, slot), taken in ascending slot order.
 *     n_valid[h] <- min(cap, n + u), so it never exceeds cap.
 *     order_in (may be NULL): fastar_tempcache_order's list for this cache
 *     and this N, made after the cache's last change; the evicted slots are
 *     then searched among those candidates only (same result, less work).
 *     A list from another cache state gives undefined slot choices (never
 *     an access outside the cache).
 * Outputs (each may be NULL):
 *   best [H][N] int32, best_cos [H][N] fp32 (step 1's result, or the inputs),
 *   dest [H][N] int32 (slot written by each token, -1 if dropped; in a
 *        mean-merged cache -1 marks a token folded into its slot's group
 *        without becoming its representative),
 *   evicted [H][N] int32 (replaced slots ascending, -1 padded),
 *   counts [H][5] int32 = {matched, refreshed, dropped, appended, evicted}.
 * Requires N <= cache->cap (else FASTAR_ECAPACITY) and a non-NaN tau.
 * q, k_cur, v_cur are [H][N][d] of cache->dtype; q_ids, kcur_ids [H][N].
 * Slot order, dest, evicted and counts are deterministic, and so are merged
 * values (a fixed summation order).
 * ------------------------------------------------------------------------ */
size_t fastar_tempcache_workspace(int32_t H, int32_t N, int32_t cap, int32_t P);
fastar_status fastar_tempcache_update(const fastar_cache* cache, const void* q,
                                      const uint16_t* q_ids, const void* k_cur, const void* v_cur,
                                      const uint16_t* kcur_ids, int32_t N, int32_t P, float tau,
                                      int32_t step, const int32_t* best_in, const float* cos_in,
                                      const int32_t* order_in, int32_t* best, float* best_cos,
                                      int32_t* dest, int32_t* evicted, int32_t* counts, void* ws,
                                      size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Eviction candidates of the next commit (blog, "1. TempCache": the least
 * recently refreshed entries leave a full cache first).  Per head, with
 * n = n_valid[h]: order[h][0 .. min(n, N)) = the min(n, N) slots of smallest
 * (ts, slot), in ascending slot order; order[h][min(n, N) .. N) = -1.
 * A commit of N tokens evicts only among these slots: each of its e evicted
 * slots is preceded in (ts, slot) order by fewer than e non-refreshed slots
 * and by at most r refreshed ones, and e + r <= N.  The list reads only ts
 * and n_valid, so it can be made on another stream while the step's
 * attention runs, then passed to fastar_tempcache_update as order_in.
 * order [H][N] int32 device buffer, written on ``stream``.  Requires
 * N <= cache->cap (else FASTAR_ECAPACITY).
 * ------------------------------------------------------------------------ */
fastar_status fastar_tempcache_order(const fastar_cache* cache, int32_t N, int32_t* order, void* stream);

/* ------------------------------------------------------------------------
 * Optional per-kernel timing, for measurement only.  While enabled, every
 * kernel the library enqueues is bracketed by HIP events on its own stream
 * (at most FASTAR_TIMER_MAX launches are recorded).  fastar_timer_stop waits
 * for those events, fills up to ``max`` entries (one per kernel name: the
 * number of launches and their summed duration in ms), returns the number of
 * distinct kernels, and disables timing.  The timer's state is per host
 * thread (it times the launches the calling thread enqueues); launches on a
 * stream that is being captured into a graph are not timed.  This is the
 * library's only state; every other call keeps none between calls.
 * ------------------------------------------------------------------------ */
#define FASTAR_TIMER_MAX 8192
typedef struct {
    char name[48];
    int32_t launches;
    float total_ms;
} fastar_kernel_time;
fastar_status fastar_timer_start(void);
int32_t fastar_timer_stop(fastar_kernel_time* out, int32_t max);

#ifdef __cplusplus
}
#endif

#endif /* FASTAR_H */
