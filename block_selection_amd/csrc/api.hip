// api.hip -- the C ABI of libpisa.so (declared in include/pisa.h).
//
// Host side only: validates arguments, derives the pyramid geometry and
// enqueues the kernels on the caller's stream. No allocation, no
// synchronisation, no global state.
#include <limits.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "pisa.h"
#include "pisa_device.h"

namespace pisa {

template <typename KT>
__global__ void build_subtree_kernel(const KT*, Geom, Pack, float*);
__global__ void build_upper_kernel(Geom, Pack, float*);
template <typename KT>
__global__ void decode_refresh_kernel(const KT*, KT*, Geom, float*);
template <int S>
__global__ void decode_step_kernel(const uint16_t*, const uint16_t*, uint16_t*, float*, Geom, unsigned long long*,
                                   uint32_t, float*,
                                   int32_t*);
__global__ void split_planes_kernel(const float*, uint16_t*, int64_t);
template <int SLOTS, int S>
__global__ void walk_upper_f32_kernel(const float*, const float*, Geom, int64_t, int64_t, int32_t*, int32_t*);
template <int SLOTS, int S>
__global__ void walk_upper_delta_kernel(const uint16_t*, const uint16_t*, const uint16_t*, Geom, UpperCfg, int64_t,
                                        int64_t, int32_t*, int32_t*);
template <int SLOTS, int S>
__global__ void walk_upper_delta_pack_kernel(const uint16_t*, const uint16_t*, const uint16_t*, Geom, Pack, int,
                                             int32_t*, int32_t*);
__global__ void delta_planes_kernel(const float*, uint16_t*, Geom, Pack);
template <typename KT>
__global__ void leaf_walk_kernel(const KT*, const KT*, Geom, int64_t, int64_t, const int32_t*,
                                 const int32_t*, int32_t*);

template <int SL>
__global__ void bucket_pass_kernel(const int32_t*, const int32_t*, Geom, ClusterGeom, Pack, const int64_t*, int64_t,
                                   uint32_t*, const uint32_t*, const uint32_t*, uint2*, uint32_t*, int);
__global__ void pack_plan_kernel(Pack, int, int, int64_t*);
__global__ void plan_groups_kernel(const uint32_t*, Geom, ClusterGeom, Pack, const int64_t*, uint32_t, uint32_t,
                                   uint32_t*, uint32_t*, int4*, uint32_t*);
template <int S, bool kOneEach>
__global__ void leaf_cluster_kernel(const uint16_t*, const uint16_t*, Geom, ClusterGeom, Pack, int64_t,
                                    const int4*, uint32_t, const uint2*, uint32_t*, float*, float*);

__global__ void vt_tiles_kernel(const uint16_t*, Geom, Pack, int64_t, uint16_t*);
__global__ void sparse_attention_kernel(const uint16_t*, const uint16_t*, const uint16_t*, const int32_t*, Geom,
                                        Pack, int64_t, float*);
__global__ void decode_attention_kernel(const uint16_t*, const uint16_t*, const uint16_t*, uint16_t*, const int32_t*,
                                        Geom, int64_t, unsigned long long*, uint32_t, float*, float*);
__global__ void flat_planes_kernel(const float*, Geom, uint16_t*);
template <typename KT, int CAP>
__global__ void flat_select_kernel(const KT*, const uint16_t*, Geom, int32_t*);
__global__ void flat_exact_scores_kernel(const uint16_t*, const uint16_t*, Geom, float*);
__global__ void flat_exact_topk_kernel(const float*, Geom, int32_t*);
constexpr int kDecAttnBlocksPerGroup = 4;                          // wavefronts (blocks) per workgroup
// A decoding step (selection or attention) spreads each sequence's leaf or block work over
// several workgroups only while the whole grid stays within this many: past it the
// device-scope fences of the hand-over cost more than the spread saves (measured on
// MI355X, 32K keys, K = 32: the split wins up to 3-4 sequences x 2 KV heads).
constexpr int64_t kDecodeSplitMaxWorkgroups = 64;
constexpr int kDecAttnStateFloats = 2 * kMaxGroup + kMaxGroup * kD;  // one partial softmax state

// The kernels that score candidates are built once per candidate score (pisa_score);
// these pick the build for G.score.
template <int SLOTS>
static const void* upper_delta_fn(int score) {
    if (score == kScoreMean) return (const void*)walk_upper_delta_kernel<SLOTS, kScoreMean>;
    if (score == kScoreMeanHalfVar) return (const void*)walk_upper_delta_kernel<SLOTS, kScoreMeanHalfVar>;
    return (const void*)walk_upper_delta_kernel<SLOTS, kScoreLse>;
}
template <int SLOTS>
static const void* upper_pack_fn(int score) {
    if (score == kScoreMean) return (const void*)walk_upper_delta_pack_kernel<SLOTS, kScoreMean>;
    if (score == kScoreMeanHalfVar) return (const void*)walk_upper_delta_pack_kernel<SLOTS, kScoreMeanHalfVar>;
    return (const void*)walk_upper_delta_pack_kernel<SLOTS, kScoreLse>;
}
template <int SLOTS>
static const void* upper_f32_fn(int score) {
    if (score == kScoreMean) return (const void*)walk_upper_f32_kernel<SLOTS, kScoreMean>;
    if (score == kScoreMeanHalfVar) return (const void*)walk_upper_f32_kernel<SLOTS, kScoreMeanHalfVar>;
    return (const void*)walk_upper_f32_kernel<SLOTS, kScoreLse>;
}
static const void* leaf_cluster_fn(int score, bool one_each) {
    if (one_each) {
        if (score == kScoreMean) return (const void*)leaf_cluster_kernel<kScoreMean, true>;
        if (score == kScoreMeanHalfVar) return (const void*)leaf_cluster_kernel<kScoreMeanHalfVar, true>;
        return (const void*)leaf_cluster_kernel<kScoreLse, true>;
    }
    if (score == kScoreMean) return (const void*)leaf_cluster_kernel<kScoreMean, false>;
    if (score == kScoreMeanHalfVar) return (const void*)leaf_cluster_kernel<kScoreMeanHalfVar, false>;
    return (const void*)leaf_cluster_kernel<kScoreLse, false>;
}
static const void* decode_step_fn(int score) {
    if (score == kScoreMean) return (const void*)decode_step_kernel<kScoreMean>;
    if (score == kScoreMeanHalfVar) return (const void*)decode_step_kernel<kScoreMeanHalfVar>;
    return (const void*)decode_step_kernel<kScoreLse>;
}
template <int SLOTS>
__global__ void final_topk_kernel(const int32_t*, const int32_t*, const float*, Geom, int64_t, int32_t*);

constexpr size_t kAlign = 256;

// Tags of the split launches' completion counters: process-wide, distinct for every call
// (until 2^32 - 1 calls have been made), never 0.
static std::atomic<uint32_t> g_call_tag{0};
static uint32_t next_call_tag() {
    uint32_t t = g_call_tag.fetch_add(1u, std::memory_order_relaxed) + 1u;
    while (t == 0u) t = g_call_tag.fetch_add(1u, std::memory_order_relaxed) + 1u;
    return t;
}
// The leaf stage numbers its entries (one per walk and sibling pair of candidates, at most
// 2K per walk) and its (KV head, pair) groups in 32 bits: bf16 selection needs
// walks * 2K < 2^32 and Hkv * ceil(N / 128) < 2^31 (N positions per sequence).
static bool bf16_select_fits(const pisa_dims* d, int64_t walks, int64_t N) {
    return walks * 2 * d->topk < ((int64_t)1 << 32) &&
           (int64_t)d->Hkv * ((N + kGrpKeys - 1) / kGrpKeys) < ((int64_t)1 << 31);
}

static size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Positions per bucket range (log2): 1024, halved down to 64 while the call has fewer ranges
// than kRangeWorkgroups (one bucket-pass workgroup per CU of an MI355X), and doubled while
// the buckets (groups x ranges) would number more than kMaxBuckets (a very long call).
constexpr int64_t kRangeWorkgroups = 256;
constexpr int64_t kMaxBuckets = (int64_t)1 << 26;
static int range_log2(int64_t positions, int64_t groups) {
    int rl = kLog2RangeMax;
    while (rl > kLog2RangeMin && ((positions + ((int64_t)1 << rl) - 1) >> rl) < kRangeWorkgroups) --rl;
    while (groups * ((positions + ((int64_t)1 << rl) - 1) >> rl) > kMaxBuckets) ++rl;
    return rl;
}

// Workspace carve-up for `walks` walks over a pyramid of P rows per (batch, head).
struct Workspace {
    uint16_t* planes;    // [2][B*Hkv*P*64] bf16 hi/lo planes of the summaries (bf16 inputs only)
    uint16_t* dplanes;   // [B*Hkv*P*128] bf16: delta(c) = s(2c) - s(c) of levels >= 2, hi and lo split,
                         // 256 bytes per node, quarter-major inside each level (delta_planes_kernel)
    int32_t* cand;       // [walks][2K] leaf candidates
    int32_t* ncand;      // [walks]
    // clustered leaf scoring (prefill, bf16 inputs)
    float* score;        // [walks][2K]
    float* sink;         // [kLeafThreads] stores of lanes without a score
    uint32_t* counts;    // [nb] group-major: bucket (range r, group g) at g * NR + r
    uint32_t* offsets;   // [nb] offset of each bucket inside its group
    uint32_t* gbase;     // [ngroups] first entry of each group
    uint2* entries;      // [walks * 2K] incidences grouped by bucket
    int4* items;         // [item_cap] full items from the front, remainders from the back
    uint32_t item_cap;
    uint32_t* meta;      // [0] items, [1] entries, item-stream counters (kMetaWords)
    int64_t* cbase;      // [2D + 2] first count and first plan chunk of each document (packs only)
    // fused bf16 decoding step
    unsigned long long* done;   // [B*Hkv] tagged completion counters (any contents)
    float* leaf_score;   // [B*Hkv][64] leaf scores of one step
    ClusterGeom CG;
    bool clustered;
    size_t bytes;
};

// N positions per batch element (1 for a decoding step) over a pyramid of P rows.
static Workspace carve(const pisa_dims* d, int64_t N, int64_t P, bool decode, char* base) {
    Workspace w;
    memset(&w, 0, sizeof(w));
    const int64_t walks = (int64_t)d->B * (decode ? 1 : N) * d->Hkv;
    const int64_t cs = 2 * (int64_t)d->topk;
    size_t off = 0;
    auto take = [&](size_t bytes) -> char* {
        char* p = base ? base + off : nullptr;
        off = align_up(off + bytes);
        return p;
    };
    if (decode && d->dtype == PISA_DTYPE_BF16) {
        w.done = (unsigned long long*)take((size_t)d->B * d->Hkv * sizeof(unsigned long long));
        w.leaf_score = (float*)take((size_t)d->B * d->Hkv * 64 * sizeof(float));
        w.bytes = off;
        return w;
    }
    const size_t planes = (d->dtype == PISA_DTYPE_BF16) ? (size_t)2 * d->B * d->Hkv * P * kD * 2 : 0;
    w.planes = (uint16_t*)take(planes);
    w.dplanes = (uint16_t*)take(planes);
    w.cand = (int32_t*)take((size_t)walks * cs * sizeof(int32_t));
    w.ncand = (int32_t*)take((size_t)walks * sizeof(int32_t));
    const int64_t m1 = (N + kC - 1) / kC;
    const int64_t ngp = (m1 + kGrpLeaves - 1) / kGrpLeaves;
    // clustered leaf scoring for bf16 prefill (callers check bf16_select_fits first)
    w.clustered = !decode && d->dtype == PISA_DTYPE_BF16 && bf16_select_fits(d, walks, N);
    if (w.clustered) {
        w.CG.RL = range_log2((int64_t)d->B * N, (int64_t)d->B * d->Hkv * ngp);
        w.CG.NR = (int32_t)((N + ((int64_t)1 << w.CG.RL) - 1) >> w.CG.RL);
        w.CG.NGP = (int32_t)ngp;
        w.CG.ngroups = (int32_t)(d->B * d->Hkv * ngp);
        w.CG.nb = w.CG.ngroups * w.CG.NR;
        w.score = (float*)take((size_t)walks * cs * sizeof(float));
        w.sink = (float*)take((size_t)kLeafThreads * sizeof(float));
        w.counts = (uint32_t*)take((size_t)w.CG.nb * 4);
        w.offsets = (uint32_t*)take((size_t)w.CG.nb * 4);
        w.gbase = (uint32_t*)take((size_t)w.CG.ngroups * 4);
        w.entries = (uint2*)take((size_t)walks * cs * sizeof(uint2));
        w.item_cap = (uint32_t)(walks * cs / kItemMin + w.CG.ngroups + 1);
        w.items = (int4*)take((size_t)w.item_cap * sizeof(int4));
        w.meta = (uint32_t*)take(kMetaWords * sizeof(uint32_t));
    }
    w.bytes = off;
    return w;
}

// Packs of D documents over T tokens (bf16, clustered leaf scoring) on the packed layout
// of P rows per KV head.
static int64_t pack_count_bound(int Hkv, int64_t T, int64_t D, int rl) {
    // sum over documents of ceil(n/128) * ceil(n/R) <= sum (n/128 + 1)(n/R + 1)
    // <= T^2 / (128 R) + T/128 + T/R + D
    const int64_t R = (int64_t)1 << rl;
    return (int64_t)Hkv * (((T + kGrpKeys - 1) / kGrpKeys) * ((T + R - 1) / R) + T / kGrpKeys + T / R + D + 4);
}

static Workspace carve_pack(const pisa_dims* d, int64_t T, int64_t D, int64_t P, char* base) {
    Workspace w;
    memset(&w, 0, sizeof(w));
    const int64_t walks = T * d->Hkv;
    const int64_t cs = 2 * (int64_t)d->topk;
    size_t off = 0;
    auto take = [&](size_t bytes) -> char* {
        char* p = base ? base + off : nullptr;
        off = align_up(off + bytes);
        return p;
    };
    const size_t planes = (size_t)2 * d->Hkv * P * kD * 2;
    w.planes = (uint16_t*)take(planes);
    w.dplanes = (uint16_t*)take(planes);
    w.cand = (int32_t*)take((size_t)walks * cs * sizeof(int32_t));
    w.ncand = (int32_t*)take((size_t)walks * sizeof(int32_t));
    w.clustered = true;
    w.CG.NGP = (int32_t)((T >> (kLog2GrpKeys)) + D + 1);   // pair slots per KV head
    w.CG.RL = range_log2(T, (int64_t)d->Hkv * ((T + kGrpKeys - 1) / kGrpKeys) + D);
    w.CG.NR = (int32_t)((T >> w.CG.RL) + D + 1);        // range slots
    w.CG.ngroups = (int32_t)(d->Hkv * (int64_t)w.CG.NGP);
    const int64_t ncount = pack_count_bound(d->Hkv, T, D, w.CG.RL);
    w.CG.nb = 0;
    w.score = (float*)take((size_t)walks * cs * sizeof(float));
    w.sink = (float*)take((size_t)kLeafThreads * sizeof(float));
    w.counts = (uint32_t*)take((size_t)ncount * 4);
    w.offsets = (uint32_t*)take((size_t)ncount * 4);
    w.gbase = (uint32_t*)take((size_t)w.CG.ngroups * 4);
    w.entries = (uint2*)take((size_t)walks * cs * sizeof(uint2));
    w.item_cap = (uint32_t)(walks * cs / kItemMin + w.CG.ngroups + 1);
    w.items = (int4*)take((size_t)w.item_cap * sizeof(int4));
    w.meta = (uint32_t*)take(kMetaWords * sizeof(uint32_t));
    w.cbase = (int64_t*)take((size_t)(2 * D + 2) * sizeof(int64_t));
    w.bytes = off;
    return w;
}

// Level sizes for n keys: M[1] = ceil(n/64), M[l+1] = ceil(M[l]/2) until 1. Returns L.
static int level_sizes(int64_t n, int64_t M[kMaxLevels + 1]) {
    int64_t m = (n + kC - 1) / kC;
    int l = 1;
    for (;;) {
        M[l] = m;
        if (m == 1 || l == kMaxLevels) break;
        m = (m + 1) / 2;
        ++l;
    }
    return l;
}

static int check_dims(const pisa_dims* d) {
    if (!d) return PISA_ERR_INVALID_ARG;
    if (d->B < 1 || d->Hq < 1 || d->Hkv < 1 || d->topk < 1) return PISA_ERR_INVALID_ARG;
    if (d->Hq % d->Hkv != 0) return PISA_ERR_INVALID_ARG;
    if (d->dtype != PISA_DTYPE_F32 && d->dtype != PISA_DTYPE_BF16) return PISA_ERR_INVALID_ARG;
    if (d->score < PISA_SCORE_LSE || d->score > PISA_SCORE_MEAN_HALF_VAR) return PISA_ERR_INVALID_ARG;
    if (d->d != kD || d->C != kC || d->g != 2) return PISA_ERR_UNSUPPORTED;
    if (d->Hq / d->Hkv > kMaxGroup || d->topk > kMaxTopK) return PISA_ERR_UNSUPPORTED;
    if ((int64_t)d->B * d->Hkv > 65535) return PISA_ERR_UNSUPPORTED;   // one grid row per (batch, KV head)
    return PISA_OK;
}

// Geometry for n keys inside a layout sized for cap keys.
static int make_geom(const pisa_dims* d, int64_t n, int64_t cap, Geom* G) {
    if (n < 1 || cap < 1) return PISA_ERR_INVALID_ARG;
    if (n > cap) return PISA_ERR_CAPACITY;
    if (cap > (int64_t)INT_MAX) return PISA_ERR_UNSUPPORTED;
    memset(G, 0, sizeof(*G));
    int64_t Mc[kMaxLevels + 1] = {0}, Mn[kMaxLevels + 1] = {0};
    const int Lc = level_sizes(cap, Mc);
    const int Ln = level_sizes(n, Mn);
    int64_t off = 0;
    for (int l = 1; l <= Lc; ++l) { G->off[l] = off; off += Mc[l]; }
    G->P = off;
    for (int l = 1; l <= Ln; ++l) G->M[l] = (int32_t)Mn[l];
    G->L = Ln;
    G->N = n;
    G->cap = cap;
    G->B = d->B; G->Hq = d->Hq; G->Hkv = d->Hkv; G->GQ = d->Hq / d->Hkv; G->topk = d->topk;
    G->score = d->score;
    return PISA_OK;
}

// Packed layout for D documents over T tokens: level l (1 .. root_level(T)) has a region of
// (T >> (5 + l)) + D + 1 rows per KV head; G.M[l] holds the region sizes, G.P their total.
static int make_pack_geom(const pisa_dims* d, int64_t T, int64_t D, Geom* G) {
    if (T < 1 || D < 1) return PISA_ERR_INVALID_ARG;
    if (d->B != 1) return PISA_ERR_INVALID_ARG;
    if (T > (int64_t)INT_MAX / 2 || D > (int64_t)INT_MAX / 4) return PISA_ERR_UNSUPPORTED;
    if ((int64_t)d->Hkv * ((T >> (kLog2GrpKeys)) + D + 1) > (int64_t)INT_MAX) return PISA_ERR_UNSUPPORTED;
    memset(G, 0, sizeof(*G));
    const int L = root_level(T);
    int64_t off = 0;
    for (int l = 1; l <= L; ++l) {
        const int64_t R = (T >> (kLog2C + l - 1)) + D + 1;
        G->off[l] = off;
        G->M[l] = (int32_t)R;
        off += R;
    }
    G->P = off;
    G->L = L;
    G->N = T;
    G->cap = T;
    G->B = 1; G->Hq = d->Hq; G->Hkv = d->Hkv; G->GQ = d->Hq / d->Hkv; G->topk = d->topk;
    G->score = d->score;
    return PISA_OK;
}

static int launch_status() {
    return (hipGetLastError() == hipSuccess) ? PISA_OK : PISA_ERR_HIP;
}

template <typename KT>
static int build_impl(const KT* k, const Geom& G, const Pack& pk, float* pyr, hipStream_t s) {
    int64_t grid, ugrid;
    if (pk.cu) {
        grid = (int64_t)G.Hkv * ((pk.T >> 10) + pk.D + 1);   // (KV head, subtree slot)
        ugrid = (int64_t)pk.D * G.Hkv;
    } else {
        grid = (int64_t)G.B * G.Hkv * ((G.M[1] + 15) / 16);
        ugrid = (int64_t)G.B * G.Hkv;
    }
    if (grid > INT_MAX || ugrid > INT_MAX) return PISA_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(build_subtree_kernel<KT>, dim3((unsigned)grid), dim3(256), 0, s, k, G, pk, pyr);
    if (G.L > 5) hipLaunchKernelGGL(build_upper_kernel, dim3((unsigned)ugrid), dim3(1024), 0, s, G, pk, pyr);
    return launch_status();
}

// LDS staging of the delta-form walk of one batch element (the same plan the packed walk
// makes per document on the device).
static UpperCfg upper_cfg_delta(const Geom& G) {
    UpperCfg U;
    memset(&U, 0, sizeof(U));
    upper_cfg_for(batch_seg(G.N, 0), G.topk, U);
    return U;
}

template <int SLOTS>
static int launch_upper_delta(const uint16_t* q, const Geom& G, const UpperCfg& U, int64_t t0, int64_t NT,
                              const Workspace& W, int cus, hipStream_t s) {
    constexpr int WPW = 64 / SLOTS;
    constexpr int nwaves = kUpperThreads / 64;
    const int64_t groups = (NT + WPW - 1) / WPW;
    const int bh = G.B * G.Hkv;
    // one workgroup per CU (LDS-bound), a multiple of 8 so that XCDs split evenly
    int64_t need = (int64_t)bh * ((groups + nwaves - 1) / nwaves);
    int64_t nwg = need < cus ? need : cus;
    nwg = (nwg + 7) / 8 * 8;
    if (nwg < bh) nwg = bh;
    const size_t lds = (size_t)U.lds_nodes * kLdsNodeBytes;
    const void* fn = upper_delta_fn<SLOTS>(G.score);
    if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
        return PISA_ERR_HIP;
    const uint16_t* planes = W.planes;
    const uint16_t* dplanes = W.dplanes;
    void* args[] = {(void*)&q, (void*)&planes, (void*)&dplanes, (void*)&G, (void*)&U, (void*)&t0, (void*)&NT,
                    (void*)&W.cand, (void*)&W.ncand};
    if (hipLaunchKernel(fn, dim3((unsigned)nwg), dim3(kUpperThreads), args, lds, s) != hipSuccess)
        return PISA_ERR_HIP;
    return PISA_OK;
}

template <int SLOTS>
static int launch_upper_pack(const uint16_t* q, const Geom& G, const Pack& pk, const Workspace& W, int cus,
                             hipStream_t s) {
    constexpr int WPW = 64 / SLOTS;
    constexpr int nwaves = kUpperThreads / 64;
    const int64_t groups = (pk.T + WPW - 1) / WPW + pk.D;
    int64_t need = (int64_t)G.Hkv * ((groups + nwaves - 1) / nwaves);
    int64_t nwg = need < cus ? need : cus;
    nwg = (nwg + 7) / 8 * 8;
    if (nwg < G.Hkv) nwg = G.Hkv;
    // pieces of 512 tokens, fewer (down to 64) until every workgroup of a KV head has two
    const int64_t npeers = nwg / G.Hkv;
    int plog2 = 9;
    while (plog2 > 6 && ((pk.T + ((int64_t)1 << plog2) - 1) >> plog2) < 2 * npeers) --plog2;
    const size_t lds = (size_t)(kLdsDeltaBudgetNodes + 2 * G.topk) * kLdsNodeBytes;
    const void* fn = upper_pack_fn<SLOTS>(G.score);
    if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
        return PISA_ERR_HIP;
    const uint16_t* planes = W.planes;
    const uint16_t* dplanes = W.dplanes;
    void* args[] = {(void*)&q, (void*)&planes, (void*)&dplanes, (void*)&G, (void*)&pk, (void*)&plog2,
                    (void*)&W.cand, (void*)&W.ncand};
    if (hipLaunchKernel(fn, dim3((unsigned)nwg), dim3(kUpperThreads), args, lds, s) != hipSuccess)
        return PISA_ERR_HIP;
    return PISA_OK;
}

template <int SLOTS>
static int launch_upper_f32(const float* q, const float* pyr, const Geom& G, int64_t t0, int64_t NT,
                            const Workspace& W, int cus, hipStream_t s) {
    constexpr int WPW = 64 / SLOTS;
    constexpr int nwaves = kUpperThreads / 64;
    const int64_t groups = (NT + WPW - 1) / WPW;
    const int bh = G.B * G.Hkv;
    int64_t need = (int64_t)bh * ((groups + nwaves - 1) / nwaves);
    int64_t nwg = need < cus ? need : cus;
    nwg = (nwg + 7) / 8 * 8;
    if (nwg < bh) nwg = bh;
    void* args[] = {(void*)&q, (void*)&pyr, (void*)&G, (void*)&t0, (void*)&NT, (void*)&W.cand, (void*)&W.ncand};
    if (hipLaunchKernel(upper_f32_fn<SLOTS>(G.score), dim3((unsigned)nwg), dim3(kUpperThreads), args, 0, s) !=
        hipSuccess)
        return PISA_ERR_HIP;
    return PISA_OK;
}

static int device_cus(int* cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return PISA_ERR_HIP;
    if (hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return PISA_ERR_HIP;
    return PISA_OK;
}

// Leaf stage after the upper walk has recorded its incidences: bucket offsets and
// work items, entries grouped by bucket, clustered scoring, final top-K per walk.
static void mark(void* const* ev, int i, hipStream_t s) {
    if (ev && ev[i]) (void)hipEventRecord((hipEvent_t)ev[i], s);
}

// Resident workgroups per CU of each leaf-scoring kernel (a property of the code object,
// queried once per variant; 0 if the query fails).
static int leaf_blocks_per_cu(int score, bool one_each) {
    static std::atomic<int> cache[6] = {{-1}, {-1}, {-1}, {-1}, {-1}, {-1}};
    const int i = ((score == kScoreMean) ? 1 : (score == kScoreMeanHalfVar) ? 2 : 0) + (one_each ? 3 : 0);
    int v = cache[i].load(std::memory_order_relaxed);
    if (v < 0) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, leaf_cluster_fn(score, one_each), kLeafThreads, 0) !=
            hipSuccess)
            return 0;
        cache[i].store(v, std::memory_order_relaxed);
    }
    return v;
}

static int cluster_leaf_stage(const uint16_t* q, const uint16_t* k, const Geom& G, const Pack& pk, int64_t NT,
                              int32_t* out, const Workspace& W, int cus, hipStream_t s, void* const* ev) {
    const int64_t walks = (int64_t)G.B * NT * G.Hkv;
    const ClusterGeom& CG = W.CG;
    const int slots = 2 * G.topk;
    dim3 bgrid;
    size_t bins;
    if (pk.cu) {
        hipLaunchKernelGGL(pack_plan_kernel, dim3(1), dim3(1024), 0, s, pk, G.Hkv, (int)CG.RL, W.cbase);
        bgrid = dim3((unsigned)CG.NR, 1u);
        bins = (size_t)G.Hkv * ((pk.T + kGrpKeys - 1) / kGrpKeys);   // the longest document's groups
    } else {
        bgrid = dim3((unsigned)CG.NR, (unsigned)G.B);
        bins = (size_t)G.Hkv * CG.NGP;
    }
    bins = (bins < (size_t)kBinSlice ? bins : (size_t)kBinSlice) * sizeof(uint32_t);   // LDS bytes
    const int64_t* cbase = W.cbase;
    // items of L entries: kItemMax, halved (down to kItemMin) while the call's entries, about
    // K per walk, would make fewer than two items per wavefront the leaf stage keeps resident
    // (three per SIMD): a short call spreads its scoring over more wavefronts, at the price
    // of loading a pair's keys for fewer entries
    uint32_t L = kItemMax;
    while (L > (uint32_t)kItemMin && (int64_t)walks * G.topk < (int64_t)cus * 24 * L) L >>= 1;
    // plan workgroups: one per unit of 64 bins (a pack's units, at most Hkv (T / 128 + D) / 64
    // + D, are counted by its plan), the grid striding past 65536
    int64_t units = pk.cu ? (int64_t)G.Hkv * (pk.T / kGrpKeys + pk.D) / 64 + pk.D
                          : (int64_t)G.B * ((G.Hkv * (int64_t)CG.NGP + 63) / 64);
    const dim3 pgrid((unsigned)(units < 65536 ? units : 65536));
    for (int fill = 0; fill < 2; ++fill) {
        if (fill)
            hipLaunchKernelGGL(plan_groups_kernel, pgrid, dim3(64 * kPlanWaves), 0, s, W.counts, G, CG, pk, cbase, L, W.item_cap,
                               W.offsets, W.gbase, W.items, W.meta);
        if (slots <= 16)
            hipLaunchKernelGGL(bucket_pass_kernel<16>, bgrid, dim3(1024), bins, s, W.cand, W.ncand, G, CG, pk, cbase,
                               NT, W.counts, W.offsets, W.gbase, W.entries, W.meta, fill);
        else if (slots <= 32)
            hipLaunchKernelGGL(bucket_pass_kernel<32>, bgrid, dim3(1024), bins, s, W.cand, W.ncand, G, CG, pk, cbase,
                               NT, W.counts, W.offsets, W.gbase, W.entries, W.meta, fill);
        else
            hipLaunchKernelGGL(bucket_pass_kernel<64>, bgrid, dim3(1024), bins, s, W.cand, W.ncand, G, CG, pk, cbase,
                               NT, W.counts, W.offsets, W.gbase, W.entries, W.meta, fill);
    }
    // persistent wavefronts: as many workgroups as fit the CUs at once. A short call (at most
    // about two items of kItemMin entries per wavefront, counting K entries per walk) gives
    // each wavefront its first item without an atomic.
    const bool one_each = (int64_t)walks * G.topk <= (int64_t)cus * 12 * 2 * kItemMin;
    const void* leaf_fn = leaf_cluster_fn(G.score, one_each);
    const int per_cu = leaf_blocks_per_cu(G.score, one_each);
    if (per_cu < 1) return PISA_ERR_HIP;
    mark(ev, 2, s);
    {
        const int4* items = W.items;
        const uint2* entries = W.entries;
        void* args[] = {(void*)&q, (void*)&k, (void*)&G, (void*)&CG, (void*)&pk, (void*)&NT, (void*)&items,
                        (void*)&W.item_cap, (void*)&entries, (void*)&W.meta, (void*)&W.score, (void*)&W.sink};
        if (hipLaunchKernel(leaf_fn, dim3((unsigned)(cus * per_cu)), dim3(kLeafThreads), args, 0, s) != hipSuccess)
            return PISA_ERR_HIP;
    }
    mark(ev, 3, s);
    const int wpw = slots <= 16 ? 4 : (slots <= 32 ? 2 : 1);
    // workgroups of 4 wavefronts: one group of walks per wavefront while every wavefront can be
    // resident at once, else about kTopkBatch groups per wavefront trip
    const int64_t fgroups = (walks + wpw - 1) / wpw;
    int64_t fgrid = (fgroups + 3) / 4;
    if (fgroups > (int64_t)cus * 32) {
        fgrid = (fgroups + 4 * kTopkBatch - 1) / (4 * kTopkBatch);
        if (fgrid > (int64_t)cus * 16) fgrid = (int64_t)cus * 16;
    }
    if (slots <= 16)
        hipLaunchKernelGGL(final_topk_kernel<16>, dim3((unsigned)fgrid), dim3(256), 0, s, W.cand, W.ncand, W.score, G, NT, out);
    else if (slots <= 32)
        hipLaunchKernelGGL(final_topk_kernel<32>, dim3((unsigned)fgrid), dim3(256), 0, s, W.cand, W.ncand, W.score, G, NT, out);
    else
        hipLaunchKernelGGL(final_topk_kernel<64>, dim3((unsigned)fgrid), dim3(256), 0, s, W.cand, W.ncand, W.score, G, NT, out);
    return launch_status();
}

// Summary planes (the candidates' own rows, ragged children) and delta planes of a bf16
// walk over the pyramid of G (sequences: the batch elements, or the documents of pk).
static void plane_kernels(const float* pyr, const Geom& G, const Pack& pk, const Workspace& W, hipStream_t s) {
    const int64_t n = (int64_t)G.B * G.Hkv * G.P * kD;
    int64_t grid = (n + 255) / 256;
    if (grid > 8192) grid = 8192;
    hipLaunchKernelGGL(split_planes_kernel, dim3((unsigned)grid), dim3(256), 0, s, pyr, W.planes, n);
    if (pk.cu) {
        // documents average T/D tokens: about T/D * 64 / 64 delta elements per workgroup row
        int64_t dgrid = (pk.T / pk.D + 255) / 256;
        if (dgrid < 1) dgrid = 1;
        if (dgrid > 256) dgrid = 256;
        hipLaunchKernelGGL(delta_planes_kernel, dim3((unsigned)(pk.D * G.Hkv), (unsigned)dgrid), dim3(256), 0, s,
                           pyr, W.dplanes, G, pk);
        return;
    }
    int64_t drows = 0;
    for (int l = 2; l <= G.L; ++l) drows += G.M[l];
    int64_t dgrid = (drows * kD + 255) / 256;
    if (dgrid > 4096) dgrid = 4096;
    if (dgrid > 0)
        hipLaunchKernelGGL(delta_planes_kernel, dim3((unsigned)dgrid, (unsigned)(G.B * G.Hkv)), dim3(256), 0, s,
                           pyr, W.dplanes, G, pk);
}

template <typename KT>
static int select_impl(const KT* q, const KT* k, const float* pyr, const Geom& G, int64_t t0,
                       int64_t NT, int32_t* out, const Workspace& W, hipStream_t s, void* const* ev) {
    int rc, cus = 256;
    if ((rc = device_cus(&cus)) != PISA_OK) return rc;
    const int slots = 2 * G.topk;
    if constexpr (sizeof(KT) == 2) {
        plane_kernels(pyr, G, Pack{nullptr, 0, 0}, W, s);
        const UpperCfg U = upper_cfg_delta(G);
        mark(ev, 0, s);
        if (slots <= 16) rc = launch_upper_delta<16>(q, G, U, t0, NT, W, cus, s);
        else if (slots <= 32) rc = launch_upper_delta<32>(q, G, U, t0, NT, W, cus, s);
        else rc = launch_upper_delta<64>(q, G, U, t0, NT, W, cus, s);
    } else {
        mark(ev, 0, s);
        if (slots <= 16) rc = launch_upper_f32<16>(q, pyr, G, t0, NT, W, cus, s);
        else if (slots <= 32) rc = launch_upper_f32<32>(q, pyr, G, t0, NT, W, cus, s);
        else rc = launch_upper_f32<64>(q, pyr, G, t0, NT, W, cus, s);
    }
    if (rc != PISA_OK) return rc;
    mark(ev, 1, s);
    const int64_t walks = (int64_t)G.B * NT * G.Hkv;
    if constexpr (sizeof(KT) == 4) {
        // fp32 inputs: one wavefront per walk scores its leaf candidates from the raw keys
        int64_t grid = (walks + 3) / 4;
        if (grid > (1 << 22)) grid = 1 << 22;
        mark(ev, 2, s);
        hipLaunchKernelGGL(leaf_walk_kernel<KT>, dim3((unsigned)grid), dim3(256), 0, s, q, k, G, t0, NT,
                           W.cand, W.ncand, out);
        mark(ev, 3, s);
        return launch_status();
    } else {
        return cluster_leaf_stage(q, k, G, Pack{nullptr, 0, 0}, NT, out, W, cus, s, ev);
    }
}

// Packed documents, bf16: planes, the packed walk, clustered leaf scoring, final top-K.
static int select_pack_impl(const uint16_t* q, const uint16_t* k, const float* pyr, const Geom& G, const Pack& pk,
                            int32_t* out, const Workspace& W, hipStream_t s, void* const* ev) {
    int rc, cus = 256;
    if ((rc = device_cus(&cus)) != PISA_OK) return rc;
    const int slots = 2 * G.topk;
    plane_kernels(pyr, G, pk, W, s);
    mark(ev, 0, s);
    if (slots <= 16) rc = launch_upper_pack<16>(q, G, pk, W, cus, s);
    else if (slots <= 32) rc = launch_upper_pack<32>(q, G, pk, W, cus, s);
    else rc = launch_upper_pack<64>(q, G, pk, W, cus, s);
    if (rc != PISA_OK) return rc;
    mark(ev, 1, s);
    return cluster_leaf_stage(q, k, G, pk, pk.T, out, W, cus, s, ev);
}

}  // namespace pisa

using namespace pisa;

extern "C" {

int64_t pisa_pyramid_nodes(const pisa_dims* dims, int64_t n_capacity) {
    if (check_dims(dims) != PISA_OK || n_capacity < 1) return -1;
    int64_t M[kMaxLevels + 1] = {0};
    const int L = level_sizes(n_capacity, M);
    int64_t tot = 0;
    for (int l = 1; l <= L; ++l) tot += M[l];
    return tot;
}

int64_t pisa_level_offset(const pisa_dims* dims, int64_t n_capacity, int32_t level) {
    if (check_dims(dims) != PISA_OK || n_capacity < 1) return -1;
    int64_t M[kMaxLevels + 1] = {0};
    const int L = level_sizes(n_capacity, M);
    if (level < 1 || level > L) return -1;
    int64_t off = 0;
    for (int l = 1; l < level; ++l) off += M[l];
    return off;
}

size_t pisa_pyramid_bytes(const pisa_dims* dims, int64_t n_capacity) {
    const int64_t nodes = pisa_pyramid_nodes(dims, n_capacity);
    if (nodes < 0) return 0;
    return (size_t)dims->B * (size_t)dims->Hkv * (size_t)nodes * kD * sizeof(float);
}

size_t pisa_workspace_bytes(const pisa_dims* dims, int64_t N, int64_t n_capacity, int32_t is_decode) {
    if (check_dims(dims) != PISA_OK || n_capacity < 1 || (!is_decode && (N < 1 || N > n_capacity))) return 0;
    if (!is_decode && dims->dtype == PISA_DTYPE_BF16 && !bf16_select_fits(dims, (int64_t)dims->B * N * dims->Hkv, N))
        return 0;
    const int64_t P = pisa_pyramid_nodes(dims, n_capacity);
    return carve(dims, is_decode ? 1 : N, P, is_decode != 0, nullptr).bytes;
}

int pisa_build_pyramid(const void* k, int64_t N, int64_t n_capacity, const pisa_dims* dims,
                       float* pyramid, void* stream) {
    int rc = check_dims(dims);
    if (rc != PISA_OK) return rc;
    if (!k || !pyramid) return PISA_ERR_INVALID_ARG;
    Geom G;
    if ((rc = make_geom(dims, N, n_capacity, &G)) != PISA_OK) return rc;
    hipStream_t s = (hipStream_t)stream;
    const Pack none{nullptr, 0, 0};
    if (dims->dtype == PISA_DTYPE_BF16) return build_impl((const uint16_t*)k, G, none, pyramid, s);
    return build_impl((const float*)k, G, none, pyramid, s);
}

int pisa_select_prefill_profiled(const void* q, const void* k, const float* pyramid, int64_t N,
                                 int64_t n_capacity, const pisa_dims* dims, int32_t* out_idx,
                                 void* workspace, size_t ws_bytes, void* stream,
                                 void* const* stage_events) {
    int rc = check_dims(dims);
    if (rc != PISA_OK) return rc;
    if (!q || !k || !pyramid || !out_idx) return PISA_ERR_INVALID_ARG;
    Geom G;
    if ((rc = make_geom(dims, N, n_capacity, &G)) != PISA_OK) return rc;
    if (dims->dtype == PISA_DTYPE_BF16 && !bf16_select_fits(dims, (int64_t)dims->B * N * dims->Hkv, N))
        return PISA_ERR_UNSUPPORTED;
    const Workspace W = carve(dims, N, G.P, false, (char*)workspace);
    if (!workspace || ws_bytes < W.bytes) return PISA_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    if (dims->dtype == PISA_DTYPE_BF16)
        return select_impl((const uint16_t*)q, (const uint16_t*)k, pyramid, G, 0, N, out_idx, W, s, stage_events);
    return select_impl((const float*)q, (const float*)k, pyramid, G, 0, N, out_idx, W, s, stage_events);
}

int pisa_select_prefill(const void* q, const void* k, const float* pyramid, int64_t N,
                        int64_t n_capacity, const pisa_dims* dims, int32_t* out_idx,
                        void* workspace, size_t ws_bytes, void* stream) {
    return pisa_select_prefill_profiled(q, k, pyramid, N, n_capacity, dims, out_idx, workspace, ws_bytes,
                                        stream, nullptr);
}

// The bf16 decoding step: append, refresh, walk and leaf top-K in one launch, ceil(2K/8)
// workgroups per (batch, KV head) -- the last one to finish writes the selection -- or one
// per (batch, KV head) when that would make more than kDecodeSplitMaxWorkgroups. W holds the
// tagged completion counters (any contents) and the leaf-score rows.
static int launch_decode_bf16(const void* q_new, const void* k_new, void* k_cache, float* pyramid, const Geom& G,
                              const pisa_dims* dims, int32_t* out_idx, const Workspace& W, hipStream_t s) {
    const unsigned nbh = (unsigned)(dims->B * dims->Hkv);
    unsigned parts = (unsigned)((2 * dims->topk + 7) / 8);
    if ((int64_t)parts * nbh > kDecodeSplitMaxWorkgroups) parts = 1u;
    const uint16_t* qn = (const uint16_t*)q_new;
    const uint16_t* kn = (const uint16_t*)k_new;
    uint16_t* kc = (uint16_t*)k_cache;
    const uint32_t tag = next_call_tag();
    void* args[] = {(void*)&qn, (void*)&kn, (void*)&kc, (void*)&pyramid, (void*)&G, (void*)&W.done,
                    (void*)&tag, (void*)&W.leaf_score, (void*)&out_idx};
    if (hipLaunchKernel(decode_step_fn(G.score), dim3(parts, nbh), dim3(kDecodeThreads), args, 0, s) != hipSuccess)
        return PISA_ERR_HIP;
    return launch_status();
}

int pisa_decode_update_select(const void* q_new, const void* k_new, void* k_cache, float* pyramid,
                              int64_t n_before, int64_t n_capacity, const pisa_dims* dims,
                              int32_t* out_idx, void* workspace, size_t ws_bytes, void* stream) {
    int rc = check_dims(dims);
    if (rc != PISA_OK) return rc;
    if (!q_new || !k_new || !k_cache || !pyramid || !out_idx) return PISA_ERR_INVALID_ARG;
    if (n_before < 1) return PISA_ERR_INVALID_ARG;
    Geom G;
    if ((rc = make_geom(dims, n_before + 1, n_capacity, &G)) != PISA_OK) return rc;
    const Workspace W = carve(dims, 1, G.P, true, (char*)workspace);
    if (!workspace || ws_bytes < W.bytes) return PISA_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    const unsigned nbh = (unsigned)(dims->B * dims->Hkv);
    if (dims->dtype == PISA_DTYPE_BF16)
        return launch_decode_bf16(q_new, k_new, k_cache, pyramid, G, dims, out_idx, W, s);
    hipLaunchKernelGGL(decode_refresh_kernel<float>, dim3(nbh), dim3(64), 0, s,
                       (const float*)k_new, (float*)k_cache, G, pyramid);
    if ((rc = launch_status()) != PISA_OK) return rc;
    return select_impl((const float*)q_new, (const float*)k_cache, pyramid, G, n_before, 1, out_idx, W, s,
                       nullptr);
}

// ------------------------------------------------- decoding step without allocation --
// For callers that cannot allocate (graph capture, tight serving loops): the step's
// counters and leaf-score rows live in this file-scope device array, one copy per GPU,
// held until the process ends. Host code never passes `scratch` itself (its host-side
// name is not a device address): the first call on a device takes the array's address
// there with hipGetSymbolAddress and keeps it per device.
constexpr int64_t kNoAllocMaxBH = 4096;                                  // batch x KV heads
constexpr size_t kNoAllocCounterBytes = (size_t)kNoAllocMaxBH * sizeof(unsigned long long);
constexpr size_t kNoAllocBytes = kNoAllocCounterBytes + (size_t)kNoAllocMaxBH * 64 * sizeof(float);
static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

constexpr int kNoAllocMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kNoAllocMaxDevices];

// Device address of this device's scratch, taken at the first call on the device. Nothing
// in it needs clearing: the completion counters are tagged per call (arrive_last), and the
// leaf-score rows are written before they are read within a step.
static int noalloc_scratch(char** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return PISA_ERR_HIP;
    if (dev < 0 || dev >= kNoAllocMaxDevices) return PISA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return PISA_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = (char*)g_scratch_ptr[dev];
    return PISA_OK;
}

int pisa_decode_update_select_noalloc(const void* q_new, const void* k_new, void* k_cache, float* pyramid,
                                      int64_t n_before, int64_t n_capacity, const pisa_dims* dims,
                                      int32_t* out_idx, void* stream) {
    int rc = check_dims(dims);
    if (rc != PISA_OK) return rc;
    if (!q_new || !k_new || !k_cache || !pyramid || !out_idx) return PISA_ERR_INVALID_ARG;
    if (n_before < 1) return PISA_ERR_INVALID_ARG;
    if (dims->dtype != PISA_DTYPE_BF16) return PISA_ERR_UNSUPPORTED;
    if ((int64_t)dims->B * dims->Hkv > kNoAllocMaxBH) return PISA_ERR_WORKSPACE;   // beyond the static scratch
    Geom G;
    if ((rc = make_geom(dims, n_before + 1, n_capacity, &G)) != PISA_OK) return rc;
    hipStream_t s = (hipStream_t)stream;
    char* base = nullptr;
    if ((rc = noalloc_scratch(&base)) != PISA_OK) return rc;
    const Workspace W = carve(dims, 1, G.P, true, base);
    if (W.bytes > kNoAllocBytes) return PISA_ERR_WORKSPACE;
    return launch_decode_bf16(q_new, k_new, k_cache, pyramid, G, dims, out_idx, W, s);
}

// ------------------------------------------------------------- attention (stage two) --

// V tiles of the attention call: [B * Hkv][ceil(N / 64)][64 dims][64 keys] bf16.
static size_t attention_ws(const pisa_dims* d, int64_t N) {
    const int64_t nblk = (N + kC - 1) / kC;
    return align_up((size_t)d->B * d->Hkv * nblk * kD * kC * sizeof(uint16_t));
}

// V re-layout, then one wavefront per (position, KV head). nblk: tiles per (batch, KV head),
// or packed tile slots per KV head.
static int attention_impl(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* idx, const Geom& G,
                          const Pack& pk, int64_t nblk, float* out, uint16_t* vt, hipStream_t s) {
    const int64_t walks = (int64_t)G.B * G.N * G.Hkv;
    hipLaunchKernelGGL(vt_tiles_kernel, dim3((unsigned)nblk, (unsigned)(G.B * G.Hkv)), dim3(256), 0, s, v, G, pk,
                       nblk, vt);
    hipLaunchKernelGGL(sparse_attention_kernel, dim3((unsigned)((walks + 3) / 4)), dim3(256), 0, s, q, k,
                       (const uint16_t*)vt, idx, G, pk, nblk, out);
    return launch_status();
}

size_t pisa_attention_workspace_bytes(const pisa_dims* dims, int64_t N, int64_t n_capacity) {
    Geom G;
    if (check_dims(dims) != PISA_OK || make_geom(dims, N, n_capacity, &G) != PISA_OK) return 0;
    return attention_ws(dims, N);
}

int pisa_sparse_attention(const void* q, const void* k, const void* v, const int32_t* idx, int64_t N,
                          int64_t n_capacity, const pisa_dims* dims, float* out, void* workspace,
                          size_t ws_bytes, void* stream) {
    int rc = check_dims(dims);
    if (rc != PISA_OK) return rc;
    if (!q || !k || !v || !idx || !out) return PISA_ERR_INVALID_ARG;
    Geom G;
    if ((rc = make_geom(dims, N, n_capacity, &G)) != PISA_OK) return rc;
    if (dims->dtype != PISA_DTYPE_BF16) return PISA_ERR_UNSUPPORTED;
    const int64_t nblk = (N + kC - 1) / kC;
    const int64_t walks = (int64_t)dims->B * N * dims->Hkv;
    const int64_t grid = (walks + 3) / 4;
    if (grid > INT_MAX || nblk > INT_MAX) return PISA_ERR_UNSUPPORTED;
    if (!workspace || ws_bytes < attention_ws(dims, N)) return PISA_ERR_WORKSPACE;
    return attention_impl((const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, idx, G, Pack{nullptr, 0, 0},
                          nblk, out, (uint16_t*)workspace, (hipStream_t)stream);
}

// ------------------------------------------------------------------ packed documents --

static int check_pack(const pisa_dims* dims, int64_t T, int64_t D, Geom* G) {
    int rc = check_dims(dims);
    if (rc != PISA_OK) return rc;
    return make_pack_geom(dims, T, D, G);
}

int64_t pisa_pack_pyramid_rows(const pisa_dims* dims, int64_t T, int64_t D) {
    Geom G;
    if (check_pack(dims, T, D, &G) != PISA_OK) return -1;
    return G.P;
}

int64_t pisa_pack_level_offset(const pisa_dims* dims, int64_t T, int64_t D, int32_t level) {
    Geom G;
    if (check_pack(dims, T, D, &G) != PISA_OK || level < 1 || level > G.L) return -1;
    return G.off[level];
}

size_t pisa_pack_pyramid_bytes(const pisa_dims* dims, int64_t T, int64_t D) {
    Geom G;
    if (check_pack(dims, T, D, &G) != PISA_OK) return 0;
    return (size_t)dims->Hkv * (size_t)G.P * kD * sizeof(float);
}

size_t pisa_pack_workspace_bytes(const pisa_dims* dims, int64_t T, int64_t D) {
    Geom G;
    if (check_pack(dims, T, D, &G) != PISA_OK) return 0;
    return carve_pack(dims, T, D, G.P, nullptr).bytes;
}

int pisa_build_pyramid_packed(const void* k, const int32_t* cu_seqlens, int64_t D, int64_t T,
                              const pisa_dims* dims, float* pyramid, void* stream) {
    Geom G;
    int rc = check_pack(dims, T, D, &G);
    if (rc != PISA_OK) return rc;
    if (!k || !cu_seqlens || !pyramid) return PISA_ERR_INVALID_ARG;
    const Pack pk{cu_seqlens, (int32_t)D, T};
    hipStream_t s = (hipStream_t)stream;
    if (dims->dtype == PISA_DTYPE_BF16) return build_impl((const uint16_t*)k, G, pk, pyramid, s);
    return build_impl((const float*)k, G, pk, pyramid, s);
}

int pisa_select_prefill_packed(const void* q, const void* k, const float* pyramid, const int32_t* cu_seqlens,
                               int64_t D, int64_t T, const pisa_dims* dims, int32_t* out_idx,
                               void* workspace, size_t ws_bytes, void* stream) {
    Geom G;
    int rc = check_pack(dims, T, D, &G);
    if (rc != PISA_OK) return rc;
    if (!q || !k || !pyramid || !cu_seqlens || !out_idx) return PISA_ERR_INVALID_ARG;
    if (dims->dtype != PISA_DTYPE_BF16) return PISA_ERR_UNSUPPORTED;
    if (!bf16_select_fits(dims, T * dims->Hkv, T)) return PISA_ERR_UNSUPPORTED;
    const Workspace W = carve_pack(dims, T, D, G.P, (char*)workspace);
    if (!workspace || ws_bytes < W.bytes) return PISA_ERR_WORKSPACE;
    const Pack pk{cu_seqlens, (int32_t)D, T};
    return select_pack_impl((const uint16_t*)q, (const uint16_t*)k, pyramid, G, pk, out_idx, W,
                            (hipStream_t)stream, nullptr);
}

// Decoding-step attention workspace: one tagged completion counter per (batch, KV head)
// (any contents), then the partial states.
static size_t decode_attention_ws(const pisa_dims* d, size_t* counters) {
    const int64_t bh = (int64_t)d->B * d->Hkv;
    const int64_t parts = (d->topk + kDecAttnBlocksPerGroup - 1) / kDecAttnBlocksPerGroup;
    const size_t c = align_up((size_t)bh * sizeof(unsigned long long));
    if (counters) *counters = c;
    return c + align_up((size_t)bh * parts * kDecAttnStateFloats * sizeof(float));
}

size_t pisa_decode_attention_workspace_bytes(const pisa_dims* dims) {
    if (check_dims(dims) != PISA_OK) return 0;
    return decode_attention_ws(dims, nullptr);
}

int pisa_decode_attention(const void* q_new, const void* v_new, const void* k_cache, void* v_cache,
                          const int32_t* idx, int64_t t, int64_t n_capacity, const pisa_dims* dims, float* out,
                          void* workspace, size_t ws_bytes, void* stream) {
    int rc = check_dims(dims);
    if (rc != PISA_OK) return rc;
    if (!q_new || !k_cache || !v_cache || !idx || !out) return PISA_ERR_INVALID_ARG;
    if (t < 0) return PISA_ERR_INVALID_ARG;
    Geom G;
    if ((rc = make_geom(dims, t + 1, n_capacity, &G)) != PISA_OK) return rc;
    if (dims->dtype != PISA_DTYPE_BF16) return PISA_ERR_UNSUPPORTED;
    size_t cbytes = 0;
    if (!workspace || ws_bytes < decode_attention_ws(dims, &cbytes)) return PISA_ERR_WORKSPACE;
    // ceil(K/4) workgroups per (batch, KV head), or one when that would make more than
    // kDecodeSplitMaxWorkgroups
    unsigned parts = (unsigned)((dims->topk + kDecAttnBlocksPerGroup - 1) / kDecAttnBlocksPerGroup);
    if ((int64_t)parts * dims->B * dims->Hkv > kDecodeSplitMaxWorkgroups) parts = 1u;
    unsigned long long* done = (unsigned long long*)workspace;
    float* states = (float*)((char*)workspace + cbytes);
    hipLaunchKernelGGL(decode_attention_kernel, dim3(parts, (unsigned)(dims->B * dims->Hkv)),
                       dim3(64 * kDecAttnBlocksPerGroup), 0, (hipStream_t)stream, (const uint16_t*)q_new,
                       (const uint16_t*)v_new, (const uint16_t*)k_cache, (uint16_t*)v_cache, idx, G, t, done, next_call_tag(), states,
                       out);
    return launch_status();
}

// Packs: V tiles in the packed slots, (T >> 6) + D + 1 per KV head.
static int64_t pack_tile_slots(int64_t T, int64_t D) { return (T >> kLog2C) + D + 1; }

size_t pisa_pack_attention_workspace_bytes(const pisa_dims* dims, int64_t T, int64_t D) {
    Geom G;
    if (check_pack(dims, T, D, &G) != PISA_OK) return 0;
    return align_up((size_t)dims->Hkv * pack_tile_slots(T, D) * kD * kC * sizeof(uint16_t));
}

int pisa_sparse_attention_packed(const void* q, const void* k, const void* v, const int32_t* idx,
                                 const int32_t* cu_seqlens, int64_t D, int64_t T, const pisa_dims* dims,
                                 float* out, void* workspace, size_t ws_bytes, void* stream) {
    Geom G;
    int rc = check_pack(dims, T, D, &G);
    if (rc != PISA_OK) return rc;
    if (!q || !k || !v || !idx || !cu_seqlens || !out) return PISA_ERR_INVALID_ARG;
    if (dims->dtype != PISA_DTYPE_BF16) return PISA_ERR_UNSUPPORTED;
    const int64_t nslots = pack_tile_slots(T, D);
    if ((T * dims->Hkv + 3) / 4 > INT_MAX || nslots > INT_MAX || dims->Hkv > 65535) return PISA_ERR_UNSUPPORTED;
    if (!workspace || ws_bytes < pisa_pack_attention_workspace_bytes(dims, T, D)) return PISA_ERR_WORKSPACE;
    const Pack pk{cu_seqlens, (int32_t)D, T};
    return attention_impl((const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, idx, G, pk, nslots, out,
                          (uint16_t*)workspace, (hipStream_t)stream);
}

// ------------------------------------------------------- flat stage-one selection --

// hi/lo bf16 planes of the leaf means: 2 * B * Hkv * ceil(N / 64) rows of 64 elements.
static size_t flat_ws(const pisa_dims* d, int64_t N) {
    const int64_t m1 = (N + kC - 1) / kC;
    return align_up((size_t)2 * d->B * d->Hkv * m1 * kD * sizeof(uint16_t));
}

size_t pisa_flat_workspace_bytes(const pisa_dims* dims, int64_t N, int64_t n_capacity) {
    Geom G;
    if (check_dims(dims) != PISA_OK || make_geom(dims, N, n_capacity, &G) != PISA_OK) return 0;
    return flat_ws(dims, N);
}

int pisa_select_flat(const void* q, const float* pyramid, int64_t N, int64_t n_capacity, const pisa_dims* dims,
                     int32_t* out_idx, void* workspace, size_t ws_bytes, void* stream) {
    int rc = check_dims(dims);
    if (rc != PISA_OK) return rc;
    if (!q || !pyramid || !out_idx) return PISA_ERR_INVALID_ARG;
    Geom G;
    if ((rc = make_geom(dims, N, n_capacity, &G)) != PISA_OK) return rc;
    const int64_t waves = (int64_t)dims->B * dims->Hkv * ((N + 31) / 32);   // one per 32 positions
    if (waves > INT_MAX) return PISA_ERR_UNSUPPORTED;
    if (!workspace || ws_bytes < flat_ws(dims, N)) return PISA_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    uint16_t* planes = (uint16_t*)workspace;
    int64_t pgrid = ((int64_t)dims->B * dims->Hkv * G.M[1] * kD + 255) / 256;
    if (pgrid > 8192) pgrid = 8192;
    hipLaunchKernelGGL(flat_planes_kernel, dim3((unsigned)pgrid), dim3(256), 0, s, pyramid, G, planes);
    // a list holds the K best plus one tile (16) of new candidates
    const bool small = dims->topk <= 16;
    const dim3 grid((unsigned)waves), block(64);
    if (dims->dtype == PISA_DTYPE_BF16) {
        if (small) hipLaunchKernelGGL((flat_select_kernel<uint16_t, 32>), grid, block, 0, s, (const uint16_t*)q, planes, G, out_idx);
        else hipLaunchKernelGGL((flat_select_kernel<uint16_t, 64>), grid, block, 0, s, (const uint16_t*)q, planes, G, out_idx);
    } else {
        if (small) hipLaunchKernelGGL((flat_select_kernel<float, 32>), grid, block, 0, s, (const float*)q, planes, G, out_idx);
        else hipLaunchKernelGGL((flat_select_kernel<float, 64>), grid, block, 0, s, (const float*)q, planes, G, out_idx);
    }
    return launch_status();
}

// Exact flat selection: the score of every (position, eligible leaf), fp32, B * Hkv * N * M1.
static size_t flat_exact_ws(const pisa_dims* d, int64_t N) {
    const int64_t m1 = (N + kC - 1) / kC;
    return align_up((size_t)d->B * d->Hkv * N * m1 * sizeof(float));
}

size_t pisa_flat_exact_workspace_bytes(const pisa_dims* dims, int64_t N, int64_t n_capacity) {
    Geom G;
    if (check_dims(dims) != PISA_OK || make_geom(dims, N, n_capacity, &G) != PISA_OK) return 0;
    return flat_exact_ws(dims, N);
}

int pisa_select_flat_exact(const void* q, const void* k, int64_t N, int64_t n_capacity, const pisa_dims* dims,
                           int32_t* out_idx, void* workspace, size_t ws_bytes, void* stream) {
    int rc = check_dims(dims);
    if (rc != PISA_OK) return rc;
    if (!q || !k || !out_idx) return PISA_ERR_INVALID_ARG;
    if (dims->dtype != PISA_DTYPE_BF16 || dims->score != PISA_SCORE_LSE) return PISA_ERR_UNSUPPORTED;
    Geom G;
    if ((rc = make_geom(dims, N, n_capacity, &G)) != PISA_OK) return rc;
    const int64_t chunks = (N + kGrpKeys - 1) / kGrpKeys;             // 128 positions per chunk
    const int64_t tiles = chunks * (chunks + 1) / 2;                   // (chunk, sibling pair <= chunk)
    const int64_t walks = (int64_t)dims->B * N * dims->Hkv;
    if ((tiles + 3) / 4 > INT_MAX || (walks + 3) / 4 > INT_MAX || (int64_t)dims->B * dims->Hkv > 65535)
        return PISA_ERR_UNSUPPORTED;
    if (!workspace || ws_bytes < flat_exact_ws(dims, N)) return PISA_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    float* S = (float*)workspace;
    hipLaunchKernelGGL(flat_exact_scores_kernel, dim3((unsigned)((tiles + 3) / 4), (unsigned)(dims->B * dims->Hkv)), dim3(256),
                       0, s, (const uint16_t*)q, (const uint16_t*)k, G, S);
    hipLaunchKernelGGL(flat_exact_topk_kernel, dim3((unsigned)((walks + 3) / 4)), dim3(256), 0, s, S, G, out_idx);
    return launch_status();
}

const char* pisa_status_string(int status) {
    switch (status) {
        case PISA_OK: return "ok";
        case PISA_ERR_INVALID_ARG: return "invalid argument";
        case PISA_ERR_UNSUPPORTED: return "unsupported dimensions";
        case PISA_ERR_WORKSPACE: return "workspace too small";
        case PISA_ERR_CAPACITY: return "length exceeds capacity";
        case PISA_ERR_HIP: return "HIP launch error";
        default: return "unknown status";
    }
}

}  // extern "C"
