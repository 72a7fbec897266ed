/*
 * pisa.h -- C ABI of libpisa.so: pyramid Top-K block selection for
 * block-sparse attention (the PISA selection stage) on AMD Instinct MI355X
 * (gfx950).
 *
 * The method (pages: "Block Sparse Attention with Log-Linear Complexity",
 * qqtang-code reading note, sections 3.1, 3.2, "Scoring: LogSumExp" and 4.1;
 * and the ai4snews summary "PISA cuts block-sparse attention selection to
 * O(N log N) with pyramid Top-K", second paragraph):
 *   - keys are mean-pooled into a pyramid: level 1 holds leaf blocks of C raw
 *     keys, every level above merges g=2 adjacent nodes, up to one root;
 *   - each query, per KV head, walks it from the root down: at every level
 *     only the children of the previous level's survivors are candidates; if
 *     there are at most K of them they all survive unscored, otherwise each is
 *     scored by the LogSumExp of the query's logits against its children's
 *     summaries (raw keys at the leaf level), summed over the query heads of
 *     the GQA group, and the K best survive; the leaf survivors are the
 *     selected key blocks;
 *   - decoding keeps the pyramid and, per new token, refreshes only the new
 *     token's leaf mean and the ancestors of that leaf before walking.
 *
 * Conventions fixed by this library where the pages are silent:
 *   logit = q.k / sqrt(d); level sizes M_1 = ceil(N/C), M_{l+1} = ceil(M_l/g)
 *   down to 1; a node that covers fewer raw keys than a full one (right edge)
 *   summarises the mean of the raw keys it covers; a node is eligible for
 *   query position t iff its first raw key index is <= t, and only eligible
 *   children enter a parent's LSE (raw keys > t are masked at the leaves);
 *   the at-most-K rule counts eligible candidates; query head h belongs to KV
 *   head h / (Hq/Hkv); equal scores rank the lower node index first; each
 *   output row lists the selected leaf indices in ascending order, padded
 *   with -1.
 *
 * Supported shapes: d = 64, C = 64, g = 2, 1 <= Hq/Hkv <= 16, 1 <= topk <= 32.
 * Other values return PISA_ERR_UNSUPPORTED before anything is launched.
 *
 * Memory: every pointer argument is DEVICE memory owned by the caller; the
 * library allocates nothing, keeps no global state and never synchronises
 * the stream. All work is enqueued asynchronously on `stream` (a hipStream_t;
 * NULL means the null stream). Arguments are validated on the host before any
 * launch; a launch failure returns PISA_ERR_HIP. Faults inside kernels
 * surface at the caller's next synchronisation. Values are not checked
 * (NaN/Inf inputs give unspecified indices).
 */
#ifndef PISA_H_
#define PISA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PISA_OK = 0,
    PISA_ERR_INVALID_ARG = -1,  /* null pointer, non-positive size, Hq % Hkv != 0, ... */
    PISA_ERR_UNSUPPORTED = -2,  /* d, C, g, group size or topk outside the supported set */
    PISA_ERR_WORKSPACE = -3,    /* workspace smaller than pisa_workspace_bytes() */
    PISA_ERR_CAPACITY = -4,     /* N (or n_before + 1) exceeds n_capacity */
    PISA_ERR_HIP = -5           /* a HIP launch reported an error */
} pisa_status;

typedef enum { PISA_DTYPE_F32 = 0, PISA_DTYPE_BF16 = 1 } pisa_dtype;

/* Candidate score, per query head over the candidate's eligible children's
 * logits z_1..z_m (child summaries; raw keys at the leaf level), summed over
 * the GQA group. Reading note "Block Sparse Attention with Log-Linear
 * Complexity", "Scoring: LogSumExp": the method's score is the LogSumExp;
 * dropping log m from its expansion around the mean of the z and truncating
 * gives the pages' two ablation scores, the mean (first order) and the mean
 * plus half the population variance (second order). */
typedef enum {
    PISA_SCORE_LSE = 0,            /* log sum exp(z) (the method) */
    PISA_SCORE_MEAN = 1,           /* mean(z) */
    PISA_SCORE_MEAN_HALF_VAR = 2   /* mean(z) + var(z) / 2, var over the m logits (1/m) */
} pisa_score;

/* Problem dimensions. dtype is the element type of q and k (both the same). */
typedef struct {
    int32_t B;      /* batch; B * Hkv <= 65535, else PISA_ERR_UNSUPPORTED */
    int32_t Hq;     /* query heads */
    int32_t Hkv;    /* key heads; Hq % Hkv == 0, group size GQ = Hq / Hkv */
    int32_t d;      /* head dimension (64) */
    int32_t C;      /* raw keys per leaf block (64) */
    int32_t g;      /* children per parent (2) */
    int32_t topk;   /* K: blocks kept per level and selected per query */
    int32_t dtype;  /* pisa_dtype of q and k */
    int32_t score;  /* pisa_score; other values return PISA_ERR_INVALID_ARG */
} pisa_dims;

/* Rows (nodes) per (batch, KV head) of a pyramid laid out for n_capacity
 * keys: sum over levels l >= 1 of M_l(n_capacity). Returns -1 on bad input. */
int64_t pisa_pyramid_nodes(const pisa_dims* dims, int64_t n_capacity);

/* Row offset of level l (1 = leaf blocks) inside one (batch, KV head) slab of
 * that layout; -1 if l is outside 1..L(n_capacity). */
int64_t pisa_level_offset(const pisa_dims* dims, int64_t n_capacity, int32_t level);

/* Bytes of the fp32 pyramid: B * Hkv * pisa_pyramid_nodes() * d * 4. */
size_t pisa_pyramid_bytes(const pisa_dims* dims, int64_t n_capacity);

/* Device workspace that pisa_select_prefill (is_decode = 0, N = sequence
 * length) or pisa_decode_update_select (is_decode = 1; N is ignored) needs for
 * a pyramid laid out for n_capacity keys. Returns 0 on bad input.
 * Prefill: scratch between the kernels of one call; its contents need not be
 * initialised and are meaningless after the call.
 * Decode with bf16 inputs: the workspace starts with one completion counter
 * per (batch, KV head) (8 * B * Hkv bytes), then one row of leaf scores per
 * (batch, KV head). Its contents need no initialisation: each counter carries
 * a tag that is distinct for every call (the library hands them out), and a
 * count left by another call, by a prefill call sharing the buffer or by stray
 * data is discarded. (Stray data equal to the call's own tag in the high half
 * of a counter, a 1-in-2^32 coincidence, is the only exception; zero-filled
 * memory never matches.) Steps sharing one workspace must be enqueued in order. */
size_t pisa_workspace_bytes(const pisa_dims* dims, int64_t N, int64_t n_capacity, int32_t is_decode);

/*
 * Builds the mean pyramid over keys 0..N-1 (reading note, section 3.1).
 *   k        [B, n_capacity, Hkv, d] of dims->dtype, row-major; rows >= N unused.
 *   pyramid  fp32 [B, Hkv, pisa_pyramid_nodes(n_capacity), d]; level l occupies
 *            rows pisa_level_offset(l) .. + M_l(N) - 1 of each (batch, head)
 *            slab; rows for nodes that do not exist at length N are not written.
 * Each node holds the fp32 mean of the raw keys it covers (leaf sums in fp32,
 * parents as count-weighted means of their children).
 */
int pisa_build_pyramid(const void* k, int64_t N, int64_t n_capacity, const pisa_dims* dims,
                       float* pyramid, void* stream);

/*
 * Prefill selection for every query position t in 0..N-1 (reading note,
 * sections 3.2, "Scoring: LogSumExp", 4.1).
 *   q        [B, N, Hq, d] of dims->dtype.
 *   k        [B, n_capacity, Hkv, d], the keys the pyramid was built from.
 *   pyramid  as written by pisa_build_pyramid for the same N and n_capacity.
 *   out_idx  int32 [B, N, Hkv, topk]: ascending leaf indices, -1 padded.
 *   workspace at least pisa_workspace_bytes(dims, N, n_capacity, 0) bytes of device memory.
 * bf16 inputs need B * N * Hkv * 2 * topk < 2^32 (the leaf stage numbers its
 * entries, one per walk and sibling pair of candidate leaves, in 32 bits): N up
 * to 8388607 keys at Hkv = 8, topk = 32. Beyond that the call returns
 * PISA_ERR_UNSUPPORTED and pisa_workspace_bytes returns 0.
 * Arithmetic: leaf scores use the exact bf16 (or fp32) q.k products accumulated
 * in fp32; upper-level scores multiply bf16 queries by the fp32 summaries held
 * as a hi + lo pair of bf16 values (relative error <= 2^-17 per element; fp32
 * inputs use fp32 summaries directly); LogSumExp in fp32.
 */
int pisa_select_prefill(const void* q, const void* k, const float* pyramid, int64_t N,
                        int64_t n_capacity, const pisa_dims* dims, int32_t* out_idx,
                        void* workspace, size_t ws_bytes, void* stream);

/*
 * Profiling variant of pisa_select_prefill: the same work, plus hipEventRecord
 * of caller-created hipEvent_t handles on `stream` at stage boundaries, so that
 * each stage's duration can be measured on the stream it runs on:
 *   stage_events[0]  before the upper-level walk (levels L .. 2),
 *   stage_events[1]  after it,
 *   stage_events[2]  before the leaf-level scoring kernel,
 *   stage_events[3]  after it.
 * stage_events may be NULL, and so may any entry (that event is skipped).
 */
int pisa_select_prefill_profiled(const void* q, const void* k, const float* pyramid, int64_t N,
                                 int64_t n_capacity, const pisa_dims* dims, int32_t* out_idx,
                                 void* workspace, size_t ws_bytes, void* stream,
                                 void* const* stage_events);

/*
 * One decoding step (ai4snews summary, second paragraph): appends k_new as key
 * n_before, refreshes the pyramid along the new key's leaf and its ancestors
 * only (nodes created by the new key included), then selects for the query
 * q_new at position t = n_before over n_before + 1 keys.
 *   q_new    [B, Hq, d]; k_new [B, Hkv, d] (dims->dtype).
 *   k_cache  [B, n_capacity, Hkv, d]; row n_before is written.
 *   pyramid  the pyramid of keys 0..n_before-1 (n_before >= 1) in the
 *            n_capacity layout; updated in place to cover n_before + 1 keys.
 *   out_idx  int32 [B, Hkv, topk]: ascending leaf indices, -1 padded.
 * The refreshed nodes are bitwise equal to what pisa_build_pyramid writes for
 * n_before + 1 keys. Steps on one pyramid must be enqueued in order.
 */
int pisa_decode_update_select(const void* q_new, const void* k_new, void* k_cache,
                              float* pyramid, int64_t n_before, int64_t n_capacity,
                              const pisa_dims* dims, int32_t* out_idx, void* workspace,
                              size_t ws_bytes, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): pisa_decode_update_select for bf16
 * inputs without a workspace argument. Its completion counters and leaf-score rows live in
 * a static device array of the library (1,081,344 bytes per GPU, held until the process
 * ends), whose address is taken once per device at the first call there; nothing in it
 * needs clearing (the counters are tagged per call, as in pisa_workspace_bytes). It
 * allocates nothing, launches nothing but the step, and calls no allocating routine.
 * Limits and errors: B * Hkv <= 4096 (else PISA_ERR_WORKSPACE); fp32 inputs return
 * PISA_ERR_UNSUPPORTED; otherwise as pisa_decode_update_select, whose selection and
 * refreshed pyramid it reproduces bit for bit.
 * Every call on one GPU shares that array: calls that overlap on one GPU (two streams or
 * host threads with steps in flight at the same time) race and give undefined results;
 * enqueue them on one stream, or order them.
 */
int pisa_decode_update_select_noalloc(const void* q_new, const void* k_new, void* k_cache, float* pyramid,
                                      int64_t n_before, int64_t n_capacity, const pisa_dims* dims,
                                      int32_t* out_idx, void* stream);

/* ------------------------------------------------------- attention (stage two)
 *
 * Reading note "Block Sparse Attention with Log-Linear Complexity", the two-stage
 * formulation it opens with: the second stage is attention limited to the raw
 * key/value rows of the blocks stage one picked. For query position t and query head h
 * (KV head j = h / (Hq/Hkv)): softmax of q.k / sqrt(d) over the keys <= t of the
 * blocks idx[b][t][j][0..topk-1] (entries < 0 or after t's block are skipped;
 * each block is counted as often as it appears), applied to those keys' value
 * rows.
 */

/* Device workspace of pisa_sparse_attention (0 on bad input): the value rows re-laid
 * as per-block tiles, B * Hkv * ceil(N / 64) * 64 * 64 bf16. */
size_t pisa_attention_workspace_bytes(const pisa_dims* dims, int64_t N, int64_t n_capacity);

/*
 * Attention over the selected blocks for every position t in 0..N-1 (bf16 only;
 * fp32 inputs return PISA_ERR_UNSUPPORTED).
 *   q    [B, N, Hq, d]; k, v [B, n_capacity, Hkv, d] (bf16).
 *   idx  int32 [B, N, Hkv, topk], as pisa_select_prefill writes it.
 *   out  fp32 [B, N, Hq, d].
 * Arithmetic: exact bf16 q.k products accumulated in fp32, base-2 online softmax in
 * fp32, probabilities as a bf16 hi + lo pair (2^-17 relative) times bf16 values on
 * the MFMA with fp32 accumulation.
 */
int pisa_sparse_attention(const void* q, const void* k, const void* v, const int32_t* idx, int64_t N,
                          int64_t n_capacity, const pisa_dims* dims, float* out, void* workspace,
                          size_t ws_bytes, void* stream);

/* ------------------------------------------------------------ packed documents
 *
 * Packed inputs (reading note "Block Sparse Attention with Log-Linear
 * Complexity", "Experiments: language modelling and downstream", the
 * continued-pretraining settings: packed inputs keep the document boundaries
 * and no document attends into another). D documents lie
 * end to end in T token rows; cu_seqlens is a DEVICE int32 array [D + 1]:
 * document i holds rows cu_seqlens[i] .. cu_seqlens[i+1] - 1, cu_seqlens[0] = 0,
 * cu_seqlens[D] = T, nondecreasing (empty documents allowed). Each document is
 * selected as a sequence of its own: its own pyramid over its own keys, query
 * positions and leaf indices counted from the document's first row. dims->B
 * must be 1 (INVALID_ARG otherwise). cu_seqlens values are read clamped into
 * [0, T]: an array that breaks the rules above gives unspecified selections,
 * but every access stays inside the buffers sized for T and D.
 *
 * Packed pyramid layout: fp32 [Hkv, pisa_pack_pyramid_rows(T, D), d]. Level l
 * (1 <= l <= L(T), L(T) the root level of T keys) is a region of
 * (T >> (5 + l)) + D + 1 rows starting at pisa_pack_level_offset(T, D, l); in
 * it, node i of document j's level l is row (cu_seqlens[j] >> (5 + l)) + j + i.
 * Rows no document owns are never written or read.
 */

/* Rows per KV head of the packed layout for T tokens in D documents (-1 on bad input). */
int64_t pisa_pack_pyramid_rows(const pisa_dims* dims, int64_t T, int64_t D);
/* First row of level `level`'s region (-1 on bad input or a level above L(T)). */
int64_t pisa_pack_level_offset(const pisa_dims* dims, int64_t T, int64_t D, int32_t level);
/* Bytes of the packed pyramid (0 on bad input). */
size_t pisa_pack_pyramid_bytes(const pisa_dims* dims, int64_t T, int64_t D);
/* Device workspace of pisa_select_prefill_packed (0 on bad input). */
size_t pisa_pack_workspace_bytes(const pisa_dims* dims, int64_t T, int64_t D);

/*
 * Builds every document's mean pyramid (section 3.1, per document) into the
 * packed layout. k: [T, Hkv, d] of dims->dtype (bf16 or fp32). Every node is
 * bitwise what pisa_build_pyramid writes for that document alone.
 */
int pisa_build_pyramid_packed(const void* k, const int32_t* cu_seqlens, int64_t D, int64_t T,
                              const pisa_dims* dims, float* pyramid, void* stream);

/*
 * Prefill selection for every row of a pack (bf16 only; fp32 returns
 * PISA_ERR_UNSUPPORTED, as does T with T * Hkv * 2 * topk >= 2^32).
 *   q        [T, Hq, d] bf16; k [T, Hkv, d] bf16, the keys the pyramid was built from.
 *   pyramid  as written by pisa_build_pyramid_packed for the same cu_seqlens.
 *   out_idx  int32 [T, Hkv, topk]: per row, its document's leaf indices,
 *            ascending, -1 padded (exactly what pisa_select_prefill gives for
 *            the document alone at B = 1).
 *   workspace at least pisa_pack_workspace_bytes(dims, T, D) bytes.
 */
int pisa_select_prefill_packed(const void* q, const void* k, const float* pyramid,
                               const int32_t* cu_seqlens, int64_t D, int64_t T,
                               const pisa_dims* dims, int32_t* out_idx, void* workspace,
                               size_t ws_bytes, void* stream);

/* Device workspace of pisa_decode_attention (0 on bad input): one completion counter per
 * (batch, KV head), 8 * B * Hkv bytes at its start, then the partial softmax states of the
 * call. Its contents need no initialisation (tagged counters, as in pisa_workspace_bytes).
 * Calls sharing one workspace must be enqueued in order. */
size_t pisa_decode_attention_workspace_bytes(const pisa_dims* dims);

/*
 * Attention of one decoding step (bf16 only), after pisa_decode_update_select has
 * selected the blocks for the query at position t = n_before:
 *   q_new   [B, Hq, d]; v_new [B, Hkv, d] or NULL: the new token's value row, written
 *           to row t of v_cache (pisa_decode_update_select writes only the key);
 *   k_cache, v_cache [B, n_capacity, Hkv, d], rows 0..t valid (row t of v_cache may be
 *           stale when v_new is given);
 *   idx     int32 [B, Hkv, topk] as pisa_decode_update_select writes it;
 *   out     fp32 [B, Hq, d].
 * For a few sequences the selected blocks are spread over ceil(topk / 4) workgroups per
 * (batch, KV head), whose partial softmax states the last one to finish merges; a batch
 * that would need more than 64 such workgroups runs one per (batch, KV head).
 * Either way the result is the attention over the selection (rounding of the merge aside).
 */
int pisa_decode_attention(const void* q_new, const void* v_new, const void* k_cache, void* v_cache,
                          const int32_t* idx, int64_t t, int64_t n_capacity, const pisa_dims* dims, float* out,
                          void* workspace, size_t ws_bytes, void* stream);

/* Device workspace of pisa_sparse_attention_packed (0 on bad input): the value rows as
 * per-block tiles in packed slots, Hkv * ((T >> 6) + D + 1) * 64 * 64 bf16. */
size_t pisa_pack_attention_workspace_bytes(const pisa_dims* dims, int64_t T, int64_t D);

/*
 * Attention over the selected blocks for every row of a pack (bf16 only): each row
 * attends over the keys <= its position of its own document's selected blocks, as
 * pisa_sparse_attention does for that document alone.
 *   q [T, Hq, d]; k, v [T, Hkv, d]; idx int32 [T, Hkv, topk] of document-local blocks
 *   (as pisa_select_prefill_packed writes them); out fp32 [T, Hq, d].
 */
int pisa_sparse_attention_packed(const void* q, const void* k, const void* v, const int32_t* idx,
                                 const int32_t* cu_seqlens, int64_t D, int64_t T, const pisa_dims* dims,
                                 float* out, void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------- flat stage-one selection
 *
 * The selection the pyramid replaces (reading note "Block Sparse Attention with
 * Log-Linear Complexity", "Background: two stages, and the bottleneck in the first";
 * ai4snews summary, first paragraph): every query scores every eligible leaf block's
 * mean-pooled summary and keeps the K best, with no hierarchy. Score of block b for
 * query position t and KV head j: the sum over the group's query heads h of
 * q_{t,h} . kbar_b / sqrt(d), kbar_b the mean of all the block's keys (level 1 of the
 * pyramid); block b is eligible iff b * C <= t; equal scores rank the lower block first.
 */

/* Device workspace of pisa_select_flat (0 on bad input): the leaf summaries as bf16
 * hi/lo planes, 2 * B * Hkv * ceil(N / 64) * 64 * 2 bytes. Contents need not be
 * initialised and are meaningless after the call. */
size_t pisa_flat_workspace_bytes(const pisa_dims* dims, int64_t N, int64_t n_capacity);

/*
 * Flat selection for every query position t in 0..N-1.
 *   q        [B, N, Hq, d] of dims->dtype (bf16 or fp32).
 *   pyramid  as written by pisa_build_pyramid for the same N and n_capacity (only level 1,
 *            the leaf means, is read).
 *   out_idx  int32 [B, N, Hkv, topk]: the K best eligible blocks in ascending order, -1
 *            padded (every eligible block when at most K are).
 *   workspace at least pisa_flat_workspace_bytes(dims, N, n_capacity) bytes.
 * dims->score is not used (this selector has the one score above).
 * Arithmetic: the group's query rows are summed in fp32; that sum and the leaf means are
 * each held as a hi + lo pair of bf16 values, whose three leading cross products are
 * accumulated in fp32 on the MFMA (scores within about 2^-16 relative of the exact dot
 * product). Errors: as pisa_select_prefill.
 */
int pisa_select_flat(const void* q, const float* pyramid, int64_t N, int64_t n_capacity, const pisa_dims* dims,
                     int32_t* out_idx, void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------- exact flat selection
 *
 * The selection the pyramid approximates, taken exactly (reading note "Block Sparse
 * Attention with Log-Linear Complexity", "Scoring: LogSumExp" and the accuracy comparison
 * of section 4.1): every eligible leaf block is scored as the walk scores a leaf candidate --
 * the sum over the group's query heads h of log sum_{s in block b, s <= t} exp(q_{t,h} . k_s
 * / sqrt(d)) over the block's raw keys -- and the K best are kept, with no hierarchy. Block b
 * is eligible iff b * C <= t; equal scores rank the lower block first. It is the ground truth
 * the pyramid walk's recall is measured against, at O(N^2) work.
 */

/* Device workspace of pisa_select_flat_exact (0 on bad input): every (position, eligible
 * leaf) score, fp32, B * Hkv * N * ceil(N / 64) * 4 bytes. Contents need not be initialised
 * and are meaningless after the call. */
size_t pisa_flat_exact_workspace_bytes(const pisa_dims* dims, int64_t N, int64_t n_capacity);

/*
 * Exact flat selection for every query position t in 0..N-1.
 *   q        [B, N, Hq, d] bf16.
 *   k        [B, n_capacity, Hkv, d] bf16 (the first N rows are read).
 *   out_idx  int32 [B, N, Hkv, topk]: the K best eligible blocks in ascending order, -1
 *            padded (every eligible block when at most K are).
 *   workspace at least pisa_flat_exact_workspace_bytes(dims, N, n_capacity) bytes.
 * dims->dtype must be PISA_DTYPE_BF16 and dims->score PISA_SCORE_LSE (else
 * PISA_ERR_UNSUPPORTED). Arithmetic: q.k on the MFMA in fp32 from the bf16 inputs, the
 * log-sum-exp in fp32 with base-2 exponentials, as the walk's leaf stage. Errors: as
 * pisa_select_prefill; also PISA_ERR_UNSUPPORTED when B * Hkv > 65535.
 */
int pisa_select_flat_exact(const void* q, const void* k, int64_t N, int64_t n_capacity, const pisa_dims* dims,
                           int32_t* out_idx, void* workspace, size_t ws_bytes, void* stream);

/* Static description of a status code. */
const char* pisa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* PISA_H_ */
