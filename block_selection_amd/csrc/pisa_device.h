// pisa_device.h -- geometry and wavefront helpers shared by the gfx950 kernels.
//
// Pyramid geometry (reading note "Block Sparse Attention with Log-Linear
// Complexity", section 3.1): level 1 holds ceil(N/64) leaf blocks of 64 raw
// keys and every level above halves the node count (rounding up) until a
// single root remains. Node i of level l >= 1 covers raw keys
// [i * 64 * 2^(l-1), min((i+1) * 64 * 2^(l-1), N)).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pisa {

constexpr int kD = 64;          // head dimension
constexpr int kC = 64;          // raw keys per leaf block
constexpr int kLog2C = 6;
constexpr int kMaxLevels = 40;  // levels for up to 2^31 keys plus margin
constexpr int kMaxTopK = 32;    // 2*topk candidate slots fit one 64-lane wavefront
constexpr int kMaxGroup = 16;   // query heads per KV head: one 16-column MFMA tile

// Geometry of one call, passed by value to kernels.
struct Geom {
    int64_t N;                    // keys present
    int64_t cap;                  // key capacity (row stride of k per batch element)
    int64_t P;                    // pyramid rows per (batch, KV head) in the capacity layout
    int64_t off[kMaxLevels + 1];  // row offset of level l (capacity layout)
    int32_t M[kMaxLevels + 1];    // nodes at level l for N keys
    int32_t L;                    // root level for N keys
    int32_t B, Hq, Hkv, GQ, topk;
    int32_t score;                // candidate score: kScoreLse, kScoreMean or kScoreMeanHalfVar
};
constexpr int kScoreLse = 0, kScoreMean = 1, kScoreMeanHalfVar = 2;   // the values of pisa_score

// Raw keys covered by a full node of level l (l = 0: one key).
__host__ __device__ inline int64_t span_of(int l) { return l == 0 ? 1 : (int64_t)kC << (l - 1); }

// First raw key of node i at level l; a node is eligible for query t iff this is <= t.
__host__ __device__ inline int64_t first_key(int l, int64_t i) { return i * span_of(l); }

// Raw keys actually covered by node i of level l when n keys exist (0 if the node does not exist).
__host__ __device__ inline int64_t covered(int l, int64_t i, int64_t n) {
    const int64_t lo = first_key(l, i);
    if (lo >= n) return 0;
    const int64_t s = span_of(l);
    return (n - lo < s) ? (n - lo) : s;
}

// Root level of a sequence of n >= 1 keys: ceil(n/64) leaves, halved (rounding up) to 1.
__host__ __device__ inline int32_t root_level(int64_t n) {
    int64_t m = (n + kC - 1) / kC;
    int32_t l = 1;
    while (m > 1) {
        m = (m + 1) >> 1;
        ++l;
    }
    return l;
}

// One independent sequence of a call: a batch element, or one document of a pack.
// Level l of the sequence has M(l) = ceil(N / (64 * 2^(l-1))) nodes; node i sits at row
// off[l] + shift(l) + i of its KV head's pyramid region. A batch element has shift 0;
// document d of a pack, first token a, has shift (a >> (5 + l)) + d (the packed layout).
struct Seg {
    int64_t N;     // keys (and query positions) of the sequence; 0 for an empty document
    int64_t tk0;   // row of its key 0 in the key array (per batch element or pack)
    int64_t lsh;   // packed layout: first token of the document; 0 for a batch element
    int32_t ld;    // packed layout: index of the document; 0 for a batch element
    int32_t L;     // root level
    __host__ __device__ int32_t M(int l) const { return (int32_t)(((N - 1) >> (kLog2C + l - 1)) + 1); }
    __host__ __device__ int64_t shift(int l) const { return (lsh >> (kLog2C + l - 1)) + ld; }
};

__host__ __device__ inline Seg batch_seg(int64_t N, int64_t tk0) {
    Seg s;
    s.N = N;
    s.tk0 = tk0;
    s.lsh = 0;
    s.ld = 0;
    s.L = root_level(N);
    return s;
}

// Packed documents: D documents, document d at token rows [cu[d], cu[d+1]) of T. cu is
// read clamped into [0, T], so any array keeps every access inside the buffers sized for
// T and D (a cu that is not nondecreasing from 0 to T gives unspecified selections).
//
// Packed layout: per KV head, level l (1 <= l <= root_level(T)) has a region of
// R_l = (T >> (5 + l)) + D + 1 rows; document d's level-l nodes start at its row
// (cu[d] >> (5 + l)) + d. These starts increase with d by at least the node count, so the
// documents never overlap, and they are found from cu alone. The same "slot" rule at other
// granularities (2^s tokens: slot of (d, j) = (cu[d] >> s) + d + j) numbers per-document
// work units (16-leaf subtrees, sibling pairs of leaves, position ranges) in one flat space.
struct Pack {
    const int32_t* cu;
    int32_t D;
    int64_t T;
};

__device__ inline int64_t pack_cu(const Pack& p, int i) {
    const int64_t v = p.cu[i];
    return v < 0 ? 0 : (v > p.T ? p.T : v);
}

// Slots of granularity 2^s: the last document d with (cu[d] >> s) + d <= x.
__device__ inline int pack_find_slot(const Pack& p, int s, int64_t x) {
    int lo = 0, hi = p.D - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((pack_cu(p, mid) >> s) + mid <= x) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// The document holding token row x (the last d with cu[d] <= x).
__device__ inline int pack_find_token(const Pack& p, int64_t x) {
    int lo = 0, hi = p.D - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pack_cu(p, mid) <= x) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

__device__ inline Seg pack_seg(const Pack& p, int d) {
    const int64_t a = pack_cu(p, d), b = pack_cu(p, d + 1);
    Seg s;
    s.N = b > a ? b - a : 0;
    s.tk0 = a;
    s.lsh = a;
    s.ld = d;
    s.L = root_level(s.N > 0 ? s.N : 1);
    return s;
}

// Coarse candidate levels staged in LDS by the bf16 upper-level walk: levels
// j_lo..j_hi (none if j_lo > j_hi), node i of level j at LDS slot lds_first[j] + i, each
// slot holding the hi and lo bf16 planes of the node's delta row (kLdsNodeBytes, padded
// against bank conflicts).
constexpr int kLdsNodeBytes = 272;
constexpr int kUpperThreads = 1024;
constexpr int kLdsDeltaBudgetNodes = 504; // 504 * 272 B = 133.9 KiB
struct UpperCfg {
    int32_t j_lo, j_hi;
    int32_t lds_first[kMaxLevels + 1];
    int32_t lds_nodes;
    // summary (not delta) rows of level s_level at LDS slots s_first + i: the candidates of
    // the level where most walks start scoring (0: none staged)
    int32_t s_level, s_first;
};

// LDS staging of one sequence's walk: the delta rows of the candidate levels from the first
// level that can be scored (the highest with more than K nodes) downward while they fit
// kLdsDeltaBudgetNodes, then that level's summary rows (at most 2K). lds_nodes is at most
// kLdsDeltaBudgetNodes + 2K.
__host__ __device__ inline void upper_cfg_for(const Seg& sg, int topk, UpperCfg& U) {
    U.j_lo = 1;
    U.j_hi = 0;
    U.lds_nodes = 0;
    U.s_level = 0;
    U.s_first = 0;
    int top = 0;
    for (int l = sg.L; l >= 2; --l) {
        if (sg.M(l) > topk) {
            top = l;
            break;
        }
    }
    if (top < 2) return;
    int nodes = 0, j_lo = top + 1;
    while (j_lo - 1 >= 2 && nodes + sg.M(j_lo - 1) <= kLdsDeltaBudgetNodes) {
        --j_lo;
        nodes += sg.M(j_lo);
    }
    if (j_lo > top) return;
    U.j_lo = j_lo;
    U.j_hi = top;
    int slot = 0;
    for (int j = j_lo; j <= top; ++j) {
        U.lds_first[j] = slot;
        slot += sg.M(j);
    }
    U.s_level = top;
    U.s_first = slot;
    slot += sg.M(top);
    U.lds_nodes = slot;
}

// Clustered leaf scoring (prefill): incidences are bucketed by (batch, KV head, sibling
// pair of leaves, range of 2^RL query positions), so that each bucket is counted and
// filled by one workgroup and the entries of one (batch, KV head, pair) group are
// contiguous; work items hold at most kItemMax entries of one group, or fewer (down to
// kItemMin) when a call has too few entries to give every wavefront several items. Ranges
// hold 1024 positions, or fewer (down to 64) when a call has too few ranges to give every
// CU a workgroup.
constexpr int kGrpLeaves = 2;                      // one sibling pair of leaves per group
constexpr int kGrpKeys = kGrpLeaves * kC;          // 128 keys
constexpr int kLog2GrpKeys = kLog2C + 1;
constexpr int kLog2RangeMax = 10, kLog2RangeMin = 6;
constexpr int kItemMax = 128;                      // entries per work item
constexpr int kItemMin = 32;                       // ... of a call with few entries
constexpr int kLeafThreads = 256;                  // independent wavefronts, one work item each
constexpr int kBinSlice = 16384;                   // bucket-pass bins held in LDS at once (64 KiB)
constexpr int kBucketUnroll = 4;                   // rounds of walks per bucket-pass loop trip
constexpr int kPlanWaves = 16;                     // wavefronts of a plan workgroup
constexpr int kTopkBatch = 4;                      // groups of walks per final top-K wavefront trip
// meta words of the leaf stage: items at the front / back of the item array, entries
// placed, then kItemStreams item counters at meta[64 + 64 s], 256 bytes apart
constexpr int kMetaFront = 0, kMetaEntries = 1, kMetaBack = 2;
constexpr int kItemStreams = 8;
constexpr int kItemCounter0 = 64;
constexpr int kItemCounterStride = 64;
constexpr int kMetaWords = kItemCounter0 + kItemCounterStride * kItemStreams;
struct ClusterGeom {
    int32_t NR;      // position ranges per batch element (range slots of a pack)
    int32_t NGP;     // pair groups per KV head (pair slots of a pack)
    int32_t ngroups; // B * Hkv * NGP
    int32_t nb;      // buckets = ngroups * NR
    int32_t RL;      // log2 of the positions per range
};
// Fused decode step: workgroups of 8 wavefronts, ceil(2K / 8) per (batch, KV head).
constexpr int kDecodeThreads = 512;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// LDS pointer types (address space 3) so that LDS accesses compile to ds_* instructions
typedef __attribute__((address_space(3))) u32x4 lds_u32x4_t;
typedef __attribute__((address_space(3))) char lds_char_t;

__device__ inline float bf16_bits_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Raw buffer reads (gfx9 buffer resource, word 3 = 0x00020000): a wave-uniform base and
// range in scalar registers, a 32-bit per-lane byte offset, constant offsets folded into
// the instruction; reads at or past `bytes` return zero.
typedef __amdgpu_buffer_rsrc_t buf_rsrc_t;
__device__ inline buf_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ inline u32x4 load_b128(buf_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// Eight consecutive elements of a row as floats (bf16 or fp32 storage).
__device__ inline void load8_f32(const uint16_t* p, float v[8]) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
__device__ inline void load8_f32(const float* p, float v[8]) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
}

__device__ inline float shfl_f(float v, int src) { return __shfl(v, src, 64); }
__device__ inline int shfl_i(int v, int src) { return __shfl(v, src, 64); }
__device__ inline float xor_f(float v, int m) { return __shfl_xor(v, m, 64); }

__device__ inline float readlane_f(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}
__device__ inline int readlane_i(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }

__device__ inline uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// Completion counter of a split launch: one 64-bit word per (batch, KV head), the call's tag
// (never 0, unique per call) in the high half and the number of its workgroups that have
// finished in the low half. A workgroup arriving at a word whose tag is another call's
// discards the count it finds (stale, from another call, or stray data) and starts from
// zero, so the workgroup that sees `nparts` arrivals is this call's last whatever the word
// held before. One thread per workgroup calls this, after a device-scope fence.
__device__ inline bool arrive_last(unsigned long long* word, uint32_t tag, uint32_t nparts) {
    unsigned long long old = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (;;) {
        const uint32_t cnt = ((uint32_t)(old >> 32) == tag) ? (uint32_t)old : 0u;
        const unsigned long long nv = ((unsigned long long)tag << 32) | (unsigned long long)(cnt + 1u);
        const unsigned long long seen = atomicCAS(word, old, nv);
        if (seen == old) return cnt + 1u == nparts;
        old = seen;   // another workgroup arrived first: retry against what it wrote
    }
}

// Number of set bits of m below this lane.
__device__ inline int lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Lane i sends v to lane dst_i (all lanes active; each destination written at most once).
__device__ inline int push_to_lane(int dst, int v) { return __builtin_amdgcn_ds_permute(dst << 2, v); }

// Count-weighted mean of two children with explicit roundings, so that the
// full build and the decode refresh produce identical bits.
__device__ inline float parent_mean(float a, float ca, float b, float cb) {
    if (cb == 0.0f) return a;
    return __fdiv_rn(__fmaf_rn(ca, a, __fmul_rn(cb, b)), ca + cb);
}

}  // namespace pisa
