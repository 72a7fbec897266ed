// select.hip -- coarse-to-fine Top-K walk over the mean pyramid (gfx950).
//
// Reading note "Block Sparse Attention with Log-Linear Complexity":
//   section 3.2  -- the walk starts at the single coarsest node; at each finer
//                   level the candidates are the children of the survivors; a
//                   level with at most K candidates keeps them all unscored,
//                   otherwise the K best survive; the leaf survivors are the
//                   selected blocks;
//   "Scoring: LogSumExp" -- a candidate scores the LSE of the query's logits
//                   against its children's summaries (its raw keys at the leaf
//                   level, which gives the exact raw-key LSE);
//   section 4.1  -- the query heads of a GQA group add their scores and share
//                   one selection.
//
// One wavefront runs one walk (query position t, KV head). Lane layout of the
// 16x16 MFMA tiles: column n = lane % 16 is the query head of the group, and
// lane group gq = lane / 16 supplies one quarter of the d = 64 contraction. A
// result tile holds, in lane (gq, n), rows 4*gq .. 4*gq+3 for head n.
//   * upper levels: rows are the children of the candidates (two per candidate,
//     so a lane holds both children of two candidates), fp32 summaries times
//     fp32-widened queries on v_mfma_f32_16x16x4_f32;
//   * leaf level: rows are the raw keys of one candidate leaf (4 tiles of 16),
//     bf16 keys times bf16 queries on v_mfma_f32_16x16x32_bf16 (fp32 for fp32
//     inputs), exact products accumulated in fp32.
// LSE reductions run over the rows (in-lane, then xor 16/32), the group sum
// over the columns (xor 1..8). Top-K ranks scores by (higher score, lower index).
#include "pisa_device.h"

namespace pisa {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Query fragments of one walk: dims {8gq..8gq+7, 32+8gq..32+8gq+7} of head n.
template <typename KT>
struct QFrag;

template <>
struct QFrag<uint16_t> {
    bf16x8 lo, hi;     // bf16 MFMA B operand (two k-steps of 32)
    float f[16];       // the same 16 values widened to fp32
    __device__ void load(const uint16_t* qrow, bool valid, int gq) {
        u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
        if (valid) {
            a = *reinterpret_cast<const u32x4*>(qrow + 8 * gq);
            b = *reinterpret_cast<const u32x4*>(qrow + 32 + 8 * gq);
        }
        lo = __builtin_bit_cast(bf16x8, a);
        hi = __builtin_bit_cast(bf16x8, b);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(a[i] << 16);
            f[2 * i + 1] = __uint_as_float(a[i] & 0xffff0000u);
            f[8 + 2 * i] = __uint_as_float(b[i] << 16);
            f[8 + 2 * i + 1] = __uint_as_float(b[i] & 0xffff0000u);
        }
    }
};

template <>
struct QFrag<float> {
    float f[16];
    __device__ void load(const float* qrow, bool valid, int gq) {
        float a[8] = {0, 0, 0, 0, 0, 0, 0, 0}, b[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (valid) {
            load8_f32(qrow + 8 * gq, a);
            load8_f32(qrow + 32 + 8 * gq, b);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) { f[i] = a[i]; f[8 + i] = b[i]; }
    }
};

// fp32 tile: rows' 16 fp32 values (same dim order as QFrag::f) against the query.
__device__ inline f32x4 mfma_rows_f32(const float a[16], const float qf[16]) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 16; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], qf[s], acc, 0, 0, 0);
    return acc;
}

// Leaf-level tile of 16 raw keys starting at key `row0` (lane row = lane % 16).
template <typename KT>
__device__ inline f32x4 leaf_tile(const KT* kbase, int64_t row_stride, int64_t key,
                                  bool in_range, const QFrag<KT>& q, int gq);

template <>
__device__ inline f32x4 leaf_tile<uint16_t>(const uint16_t* kbase, int64_t row_stride, int64_t key,
                                            bool in_range, const QFrag<uint16_t>& q, int gq) {
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    if (in_range) {
        const uint16_t* row = kbase + key * row_stride;
        a = *reinterpret_cast<const u32x4*>(row + 8 * gq);
        b = *reinterpret_cast<const u32x4*>(row + 32 + 8 * gq);
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), q.lo, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, b), q.hi, acc, 0, 0, 0);
    return acc;
}

template <>
__device__ inline f32x4 leaf_tile<float>(const float* kbase, int64_t row_stride, int64_t key,
                                         bool in_range, const QFrag<float>& q, int gq) {
    float a[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) a[i] = 0.f;
    if (in_range) {
        const float* row = kbase + key * row_stride;
        load8_f32(row + 8 * gq, a);
        load8_f32(row + 32 + 8 * gq, a + 8);
    }
    return mfma_rows_f32(a, q.f);
}

// Sum over the group's heads (columns n < GQ) of a per-(lane group, head) value.
__device__ inline float group_sum(float v, int n, int GQ) {
    v = (n < GQ) ? v : 0.0f;
    v += xor_f(v, 1);
    v += xor_f(v, 2);
    v += xor_f(v, 4);
    v += xor_f(v, 8);
    return v;
}

// log(e^x + e^y) in natural-log units.
__device__ inline float log_add_exp(float x, float y) {
    const float m = fmaxf(x, y), d = fminf(x, y) - m;
    return m + kLn2 * __builtin_amdgcn_logf(1.0f + __builtin_amdgcn_exp2f(d * kLog2e));
}

// Scores of the candidates in lanes 0..nslots-1 (node index, -1 = empty) at level l >= 2.
template <typename KT>
__device__ inline float score_upper(const float* pyr_bh, const Geom& G, int l, int64_t t,
                                    int cand, int nslots, const QFrag<KT>& q, int lane) {
    const int n = lane & 15, gq = lane >> 4;
    const float inv_sqrt_d = 0.125f;
    const int lc = l - 1;                      // level of the children
    const int64_t Mc = G.M[lc];
    const float* base = pyr_bh + G.off[lc] * kD;
    float my = -INFINITY;
    const int ntiles = (2 * nslots + 15) / 16;
    for (int tau = 0; tau < ntiles; ++tau) {
        // A operand: child slot 16*tau + (lane % 16) = child (slot & 1) of candidate slot/2
        const int cs = 16 * tau + n;
        const int par = shfl_i(cand, cs >> 1);
        const int64_t child = (par >= 0) ? 2 * (int64_t)par + (cs & 1) : -1;
        const bool valid = child >= 0 && child < Mc && first_key(lc, child) <= t;
        float a[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) a[i] = 0.f;
        if (valid) {
            load8_f32(base + child * kD + 8 * gq, a);
            load8_f32(base + child * kD + 32 + 8 * gq, a + 8);
        }
        const f32x4 acc = mfma_rows_f32(a, q.f);
        // this lane holds child slots 16*tau + 4*gq + r: candidates 8*tau + 2*gq + {0, 1}
        float sc[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int ms = 8 * tau + 2 * gq + p;
            const int pp = shfl_i(cand, ms);
            const int64_t right = 2 * (int64_t)pp + 1;
            const bool has_right = pp >= 0 && right < Mc && first_key(lc, right) <= t;
            const float z0 = acc[2 * p] * inv_sqrt_d, z1 = acc[2 * p + 1] * inv_sqrt_d;
            const float lse = has_right ? log_add_exp(z0, z1) : z0;
            const float s = group_sum(lse, n, G.GQ);
            sc[p] = (pp >= 0) ? s : -INFINITY;
        }
        // lane m (candidate slot m) takes its score from lane group (m % 8) / 2
        const int src = 16 * ((lane & 7) >> 1);
        const float v0 = shfl_f(sc[0], src), v1 = shfl_f(sc[1], src);
        if ((lane >> 3) == tau) my = (lane & 1) ? v1 : v0;
    }
    return my;
}

// Score of one candidate leaf: exact LSE over its raw keys <= t, summed over the group.
template <typename KT>
__device__ inline float score_leaf(const KT* kbase, int64_t row_stride, const Geom& G, int64_t t,
                                   int64_t leaf, const QFrag<KT>& q, int lane) {
    const int n = lane & 15, gq = lane >> 4;
    const int64_t key0 = leaf * kC;
    f32x4 acc[4];
#pragma unroll
    for (int tau = 0; tau < 4; ++tau) {
        const int64_t key = key0 + 16 * tau + n;
        acc[tau] = leaf_tile<KT>(kbase, row_stride, key, key <= t, q, gq);
    }
    // lane holds keys key0 + 16*tau + 4*gq + r for head n
    const float c2 = 0.125f * kLog2e;
    float z[16];
    float mx = -INFINITY;
#pragma unroll
    for (int tau = 0; tau < 4; ++tau) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t key = key0 + 16 * tau + 4 * gq + r;
            const float v = (key <= t) ? acc[tau][r] * c2 : -INFINITY;
            z[4 * tau + r] = v;
            mx = fmaxf(mx, v);
        }
    }
    mx = fmaxf(mx, xor_f(mx, 16));
    mx = fmaxf(mx, xor_f(mx, 32));
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += __builtin_amdgcn_exp2f(z[i] - mx);
    s += xor_f(s, 16);
    s += xor_f(s, 32);
    const float lse = (mx + __builtin_amdgcn_logf(s)) * kLn2;
    return group_sum(lse, n, G.GQ);
}

// Keep the K best of the candidate slots (score desc, node asc); returns the survivors
// compacted into lanes 0..K-1 (-1 elsewhere).
__device__ inline int topk_survivors(float my, int cand, int nslots, int K, int lane) {
    int rank = 0;
    for (int j = 0; j < nslots; ++j) {
        const int nj = readlane_i(cand, j);
        const float sj = readlane_f(my, j);
        if (nj >= 0) rank += (sj > my || (sj == my && nj < cand)) ? 1 : 0;
    }
    const bool keep = cand >= 0 && rank < K;
    const int got = push_to_lane(keep ? rank : 63, cand);
    return (lane < K) ? got : -1;
}

// One walk for query position t, KV head kvh of batch element b. Writes K ascending
// leaf indices (-1 padded) to out_row.
template <typename KT>
__device__ void walk_one(const KT* __restrict__ qrow0, const KT* __restrict__ k,
                         const float* __restrict__ pyr, const Geom& G, int b, int kvh,
                         int64_t t, int32_t* __restrict__ out_row, int lane) {
    const int n = lane & 15, gq = lane >> 4;
    const int K = G.topk;
    QFrag<KT> q;
    q.load(qrow0 + (int64_t)n * kD, n < G.GQ, gq);
    const int bh = b * G.Hkv + kvh;
    const float* pyr_bh = pyr + (int64_t)bh * G.P * kD;
    const int64_t row_stride = (int64_t)G.Hkv * kD;
    const KT* kbase = k + ((int64_t)b * G.cap * G.Hkv + kvh) * kD;

    int surv = (lane == 0) ? 0 : -1;   // survivors of the level above, lanes 0..nsurv-1
    int nsurv = 1;
    for (int l = G.L; l >= 1; --l) {
        int cand;
        int nslots;
        if (l == G.L) {
            cand = (lane == 0) ? 0 : -1;   // the root covers key 0: always eligible
            nslots = 1;
        } else {
            nslots = 2 * nsurv;
            const int par = shfl_i(surv, lane >> 1);
            const int64_t child = 2 * (int64_t)par + (lane & 1);
            const bool ok = lane < nslots && par >= 0 && child < G.M[l] && first_key(l, child) <= t;
            cand = ok ? (int)child : -1;
        }
        const uint64_t vm = ballot(cand >= 0);
        const int ncand = __popcll(vm);
        if (ncand <= K) {
            // at most K candidates: all survive without scoring
            const int got = push_to_lane(cand >= 0 ? lanes_below(vm) : 63, cand);
            surv = (lane < ncand) ? got : -1;
            nsurv = ncand;
            continue;
        }
        float my;
        if (l >= 2) {
            my = score_upper<KT>(pyr_bh, G, l, t, cand, nslots, q, lane);
        } else {
            my = -INFINITY;
            for (int m = 0; m < nslots; ++m) {
                const int leaf = readlane_i(cand, m);
                if (leaf < 0) continue;
                const float s = score_leaf<KT>(kbase, row_stride, G, t, leaf, q, lane);
                if (lane == m) my = s;
            }
        }
        surv = topk_survivors(my, cand, nslots, K, lane);
        nsurv = K;
    }
    // ascending order, -1 padding
    int pos = 0;
    for (int j = 0; j < nsurv; ++j) {
        const int sj = readlane_i(surv, j);
        pos += (sj < surv) ? 1 : 0;
    }
    if (lane < nsurv) out_row[pos] = surv;
    else if (lane < K) out_row[lane] = -1;
}

// Walks w in [0, B*NT*Hkv): batch b, query row ti (position t0 + ti), KV head kvh, with
// kvh fastest. q holds NT rows of Hq heads per batch element; out has K entries per walk.
template <typename KT>
__global__ __launch_bounds__(256) void walk_kernel(const KT* __restrict__ q, const KT* __restrict__ k,
                                                   const float* __restrict__ pyr, Geom G,
                                                   int64_t t0, int64_t NT, int32_t* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int64_t total = (int64_t)G.B * NT * G.Hkv;
    const int64_t stride = (int64_t)gridDim.x * 4;
    for (int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); w < total; w += stride) {
        const int kvh = (int)(w % G.Hkv);
        const int64_t bt = w / G.Hkv;          // b * NT + ti
        const int64_t ti = bt % NT;
        const int b = (int)(bt / NT);
        const KT* qrow0 = q + (bt * G.Hq + (int64_t)kvh * G.GQ) * kD;
        walk_one<KT>(qrow0, k, pyr, G, b, kvh, t0 + ti, out + w * G.topk, lane);
    }
}

template __global__ void walk_kernel<uint16_t>(const uint16_t*, const uint16_t*, const float*, Geom,
                                               int64_t, int64_t, int32_t*);
template __global__ void walk_kernel<float>(const float*, const float*, const float*, Geom, int64_t,
                                            int64_t, int32_t*);

}  // namespace pisa
