// Shared-prefix decode (pa_decode_shared_prefix in include/pa.h).
//
// Requests that begin with the same tokens point their block tables at the
// same physical blocks ("Paged attention in LLMs", "Sharing blocks"; forks
// for parallel samples or beams, MCQ page comparison table).  The attention
// of every request is still its own softmax over its own tokens; what the
// shared blocks allow is reading each shared key/value tile once for all the
// requests of a group instead of once per request.
//
// Two kernels:
//  - decode_prefix_kernel: one wave per (kv-head, partition of the shared
//    prefix, group).  The group's queries for that kv-head (group size x G
//    columns, up to 64, in 16-column matrix-core tiles) all attend over the
//    partition's tokens: each key/value step is loaded once and used by
//    every column tile.  Each (request, head) gets a partial (o, m, l).
//  - decode_suffix_kernel: one wave per (kv-head, partition of the rest,
//    request): the usual decode over the request's own tokens past the
//    prefix.  When those fit one partition (the common case for forks),
//    the wave folds the row's prefix partials into its own state and
//    writes the output rows.  Otherwise each partition leaves a partial
//    after the prefix ones and counts itself in; the wave that brings the
//    (request, kv-head) counter to the partition count merges the prefix
//    and suffix partials by the log-sum-exp rule,
//      M = max_j m_j,  w_j = l_j 2^(m_j - M),  out = sum w_j o_j / sum w_j,
//    and writes the rows.  The counters are cleared by the prefix kernel
//    (or a fill kernel when there is no prefix work), which runs first.
// The prefix is cut at a multiple of max(32, block_size) tokens so both
// parts start on a step and block boundary; the few tokens between that cut
// and the end of the shared blocks go with the suffix.

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "pa.h"
#include "pa_decode_common.h"

namespace pa {

// Tokens of the shared prefix that the prefix kernel covers.
template <int BS>
__device__ __forceinline__ int shared_tokens(int prefix_blocks) {
    constexpr int A = BS > 32 ? BS : 32;
    return (prefix_blocks * BS) / A * A;
}

// Attention over tokens [start, end) of the shared table row for NCT column
// tiles at once: every step's keys and values are loaded once and each tile
// computes its scores, softmax and PV from the same registers.
template <bool BF16, int D, int BS, int NCT>
__device__ __forceinline__ void attend_range_tiles(RunState<BF16, D, BS> (&S)[NCT],
                                                   const typename DecodeCfg<BF16, D, BS>::QRegs (&qr)[NCT],
                                                   const char* __restrict__ kbase, const char* __restrict__ vbase,
                                                   int64_t blk_bytes, const int32_t* __restrict__ trow, int num_blocks,
                                                   int start, int end, int L, int lane, int n, int j,
                                                   float scale_log2) {
    using C = DecodeCfg<BF16, D, BS>;
    for (int ctok = start; ctok < end; ctok += kTableChunk * BS) {
        const int cend = min(ctok + kTableChunk * BS, end);
        const int blk0 = ctok / BS;
        const int nblk = (cend - 1) / BS - blk0 + 1;
        const int32_t ent = (lane < nblk) ? trow[blk0 + lane] : 0;
        if (__any(lane < nblk && (ent < 0 || ent >= num_blocks))) {
#pragma unroll
            for (int t = 0; t < NCT; ++t) S[t].bad = true;
            return;
        }
        const int nst = (cend - ctok + C::STEP - 1) / C::STEP;
        StepRegs<BF16, D, BS> cur;
        issue_step<BF16, D, BS>(cur, kbase, vbase, blk_bytes, ent, blk0, nblk, ctok, L, n, j);
        int tok0 = ctok;
        for (int st = 0; st + 1 < nst; ++st, tok0 += C::STEP) {
            StepRegs<BF16, D, BS> nxt;
            issue_step<BF16, D, BS>(nxt, kbase, vbase, blk_bytes, ent, blk0, nblk, tok0 + C::STEP, L, n, j);
            __builtin_amdgcn_sched_barrier(0);  // loads stay ahead of the compute
#pragma unroll
            for (int t = 0; t < NCT; ++t)
                compute_step<BF16, D, BS>(cur, qr[t], S[t].m, S[t].l, S[t].acc, tok0, L, j, scale_log2);
            cur = nxt;
        }
#pragma unroll
        for (int t = 0; t < NCT; ++t)
            compute_step<BF16, D, BS>(cur, qr[t], S[t].m, S[t].l, S[t].acc, tok0, L, j, scale_log2);
    }
}

// Normalised partial (o, m, l) of one output row into slot `slot` of its
// P_max slots; a bad table entry makes it NaN.
template <bool BF16, int D, int BS>
__device__ __forceinline__ void store_partial(float* __restrict__ part_o, float* __restrict__ part_ml, int64_t row,
                                              int P_max, int slot, const RunState<BF16, D, BS>& S, int j) {
    using C = DecodeCfg<BF16, D, BS>;
    const int64_t prow = row * P_max + slot;
    const float inv = S.bad ? __builtin_nanf("") : 1.0f / S.l;
#pragma unroll
    for (int c = 0; c < C::NV; ++c) {
        const int d0 = 16 * c + 4 * j;
        *reinterpret_cast<f32x4*>(part_o + prow * D + d0) = S.acc[c] * inv;
    }
    if (j == 0) {
        part_ml[2 * prow] = S.bad ? 0.0f : S.m;
        part_ml[2 * prow + 1] = S.bad ? 1.0f : S.l;
    }
}

template <bool BF16, int D, int BS, int NCT>
__global__ __launch_bounds__(64) void decode_prefix_kernel(
    const void* __restrict__ q_, const void* __restrict__ kc_, const void* __restrict__ vc_,
    const int32_t* __restrict__ tables, const int32_t* __restrict__ groups,
    const int32_t* __restrict__ prefix_blocks, float* __restrict__ part_o, float* __restrict__ part_ml,
    int32_t* __restrict__ counters, int ncounters, int B, int Hq, int Hkv, int G, int max_blocks, int max_pre,
    int num_blocks, int max_group, int PS, int P_max, float scale_log2) {
    using C = DecodeCfg<BF16, D, BS>;
    const int g = blockIdx.x;
    const int p = blockIdx.y;
    const int gi = blockIdx.z;
    const int lane = threadIdx.x;
    const int n = lane & 15;
    const int j = lane >> 4;
    {
        // the suffix kernel's merge counters, cleared before it starts
        const int64_t wid = ((int64_t)blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
        const int64_t nwv = (int64_t)gridDim.x * gridDim.y * gridDim.z;
        for (int64_t i = wid * 64 + lane; i < ncounters; i += nwv * 64) counters[i] = 0;
    }
    const int s0 = groups[2 * gi];
    const int ns = groups[2 * gi + 1];
    if (s0 < 0 || ns < 1 || ns > B - s0) return;  // a malformed group has no prefix work
    const int pb = prefix_blocks[s0];
    if (pb <= 0 || pb > max_pre) return;  // the suffix kernel handles such rows
    const int T = shared_tokens<BS>(pb);
    const int start = p * PS;
    if (start >= T) return;
    const int end = min(start + PS, T);
    if (ns > max_group) {
        // larger than the launch was sized for: its rows' prefix partials are NaN
        for (int i = lane; i < ns * G; i += 64) {
            const int64_t prow = ((int64_t)(s0 + i / G) * Hq + g * G + i % G) * P_max + p;
            part_ml[2 * prow] = 0.0f;
            part_ml[2 * prow + 1] = 1.0f;
            for (int d = 0; d < D; ++d) part_o[prow * D + d] = __builtin_nanf("");
        }
        return;
    }
    const int ncol = ns * G;
    typename C::QRegs qr[NCT];
#pragma unroll
    for (int t = 0; t < NCT; ++t) {
        const int c = min(16 * t + n, ncol - 1);  // padding columns repeat the last one and are never stored
        const char* qp =
            reinterpret_cast<const char*>(q_) + ((int64_t)(s0 + c / G) * Hq + g * G + c % G) * D * C::ES;
#pragma unroll
        for (int k = 0; k < C::NKC; ++k) qr[t][k] = ld16(qp + (int64_t)(4 * k + j) * 16);
    }
    RunState<BF16, D, BS> S[NCT];
#pragma unroll
    for (int t = 0; t < NCT; ++t) run_init(S[t]);
    const int64_t blk_bytes = (int64_t)Hkv * C::TILE * C::ES;
    attend_range_tiles<BF16, D, BS, NCT>(S, qr, reinterpret_cast<const char*>(kc_) + (int64_t)g * C::TILE * C::ES,
                                         reinterpret_cast<const char*>(vc_) + (int64_t)g * C::TILE * C::ES, blk_bytes,
                                         tables + (int64_t)s0 * max_blocks, num_blocks, start, end, T, lane, n, j,
                                         scale_log2);
#pragma unroll
    for (int t = 0; t < NCT; ++t) {
        const int c = 16 * t + n;
        if (c < ncol)
            store_partial<BF16, D, BS>(part_o, part_ml, (int64_t)(s0 + c / G) * Hq + g * G + c % G, P_max, p, S[t],
                                       j);
    }
}

// Folding a row's partials (normalised o, m, l) into a running state S by
// the log-sum-exp rule, NU partials at a time: load() issues one batch's
// loads, add() folds the batch in.  Lane (n, j) holds its column's
// accumulator rows 16c + 4j ...
template <bool BF16, int D, int BS, int NU>
struct PartialBatch {
    float m[NU], l[NU];
    f32x4 o[NU][DecodeCfg<BF16, D, BS>::NV];

    __device__ __forceinline__ void load(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                                         int64_t base, int i0, int npre, int j) {
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int64_t pr = base + min(i0 + u, npre - 1);  // past the end: a valid partial, skipped in add()
            m[u] = part_ml[2 * pr];
            l[u] = part_ml[2 * pr + 1];
#pragma unroll
            for (int c = 0; c < DecodeCfg<BF16, D, BS>::NV; ++c)
                o[u][c] = *reinterpret_cast<const f32x4*>(part_o + pr * D + 16 * c + 4 * j);
        }
    }

    __device__ __forceinline__ void add(RunState<BF16, D, BS>& S, int count) const {
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            if (u >= count) break;
            const float M = fmaxf(S.m, m[u]);
            const float a = S.m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(S.m - M);
            const float w = l[u] * __builtin_amdgcn_exp2f(m[u] - M);
            S.l = S.l * a + w;
#pragma unroll
            for (int c = 0; c < DecodeCfg<BF16, D, BS>::NV; ++c) S.acc[c] = S.acc[c] * a + o[u][c] * w;
            S.m = M;
        }
    }
};

// Merge of output rows row0 .. row0 + G - 1 from their prefix partials
// [0, npre) and suffix partials [P_pre, P_pre + nsuf) (log-sum-exp rule),
// written by other waves of this launch or by the prefix kernel, read at the
// device-coherent level.
template <bool BF16, int D, int BS>
__device__ __forceinline__ void merge_row_partials(const float* __restrict__ part_o,
                                                   const float* __restrict__ part_ml, void* __restrict__ out_,
                                                   int64_t row0, int P_max, int npre, int P_pre, int nsuf, int n,
                                                   int j, int G) {
    using C = DecodeCfg<BF16, D, BS>;
    if (n >= G) return;
    const int64_t rbase = (row0 + n) * P_max;
    auto slot = [&](int i) { return rbase + (i < npre ? i : P_pre + (i - npre)); };
    const int np = npre + nsuf;
    float M = -INFINITY;
    for (int i = 0; i < np; ++i)
        M = fmaxf(M, coherent_load(reinterpret_cast<const uint64_t*>(part_ml + 2 * slot(i))).x);
    RunState<BF16, D, BS> Mg;
    run_init(Mg);
    Mg.m = M;
    for (int i = 0; i < np; ++i) {
        const float2 ml = coherent_load(reinterpret_cast<const uint64_t*>(part_ml + 2 * slot(i)));
        const float wt = ml.y * __builtin_amdgcn_exp2f(ml.x - M);
        Mg.l += wt;
        const uint64_t* po = reinterpret_cast<const uint64_t*>(part_o + slot(i) * D);
#pragma unroll
        for (int c = 0; c < C::NV; ++c) {
            const int e = (16 * c + 4 * j) / 2;
            const float2 lo = coherent_load(po + e), hi = coherent_load(po + e + 1);
            Mg.acc[c] += wt * f32x4{lo.x, lo.y, hi.x, hi.y};
        }
    }
    store_out<BF16, D, BS>(out_, row0, Mg, n, j, G);
}

template <bool BF16, int D, int BS>
__global__ __launch_bounds__(64) void decode_suffix_kernel(
    const void* __restrict__ q_, const void* __restrict__ kc_, const void* __restrict__ vc_,
    const int32_t* __restrict__ tables, const int32_t* __restrict__ lens, const int32_t* __restrict__ prefix_blocks,
    float* __restrict__ part_o, float* __restrict__ part_ml, int32_t* __restrict__ counters, void* __restrict__ out_,
    int Hq, int Hkv, int G, int max_blocks, int max_pre, int num_blocks, int PS, int P_pre, int P_max,
    float scale_log2) {
    using C = DecodeCfg<BF16, D, BS>;
    const int g = blockIdx.x;
    const int b = blockIdx.y;
    const int p = blockIdx.z;  // slowest: every request's first partition is dispatched first
    const int lane = threadIdx.x;
    const int n = lane & 15;
    const int j = lane >> 4;
    const int L = lens[b];
    const int pb = prefix_blocks[b];
    const int64_t row0 = (int64_t)b * Hq + g * G;
    if (L <= 0 || (int64_t)L > (int64_t)max_blocks * BS || pb < 0 || pb > max_pre || shared_tokens<BS>(pb) > L) {
        // empty request: zero rows; a length or prefix the table cannot hold: NaN rows
        if (p == 0) fill_rows<BF16, D>(out_, row0, G, L <= 0 ? 0.0f : __builtin_nanf(""), lane);
        return;
    }
    const int T = shared_tokens<BS>(pb);
    const int npre = (T + PS - 1) / PS;
    const int nsuf = (L - T + PS - 1) / PS;
    // own tokens in one partition (or none): this wave finishes the rows,
    // folding the prefix partials into its state
    const bool single = nsuf <= 1;
    if (single ? p > 0 : p >= nsuf) return;
    const int start = T + p * PS;
    const int end = min(start + PS, L);
    typename C::QRegs qr;
    load_q<BF16, D, BS>(qr, q_, row0 + n, n, j, G);
    RunState<BF16, D, BS> S;
    run_init(S);
    const int64_t blk_bytes = (int64_t)Hkv * C::TILE * C::ES;
    const char* kbase = reinterpret_cast<const char*>(kc_) + (int64_t)g * C::TILE * C::ES;
    const char* vbase = reinterpret_cast<const char*>(vc_) + (int64_t)g * C::TILE * C::ES;
    const int32_t* trow = tables + (int64_t)b * max_blocks;
    if (!single) {
        attend_chunk<BF16, D, BS>(S, qr, kbase, vbase, blk_bytes, trow, num_blocks, start, end, L, lane, n, j,
                                  scale_log2);
        // the partial at the device-coherent level, then the count
        if (n < G) {
            const int64_t prow = (row0 + n) * P_max + P_pre + p;
            const float inv = S.bad ? __builtin_nanf("") : 1.0f / S.l;
            uint64_t* po = reinterpret_cast<uint64_t*>(part_o + prow * D);
#pragma unroll
            for (int c = 0; c < C::NV; ++c) {
                const int e = (16 * c + 4 * j) / 2;
                coherent_store(po + e, S.acc[c][0] * inv, S.acc[c][1] * inv);
                coherent_store(po + e + 1, S.acc[c][2] * inv, S.acc[c][3] * inv);
            }
            if (j == 0)
                coherent_store(reinterpret_cast<uint64_t*>(part_ml + 2 * prow), S.bad ? 0.0f : S.m,
                               S.bad ? 1.0f : S.l);
        }
        __builtin_amdgcn_s_waitcnt(0);  // the stores are complete before the count
        int old = 0;
        if (lane == 0)
            old = __hip_atomic_fetch_add(counters + (int64_t)b * Hkv + g, 1, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
        old = __shfl(old, 0, 64);
        if (old == nsuf - 1) merge_row_partials<BF16, D, BS>(part_o, part_ml, out_, row0, P_max, npre, P_pre, nsuf,
                                                             n, j, G);
        return;
    }
    // The prefix partials start the state: the first batch's loads go out
    // with the table entries, so they cost no round trip of their own.  The
    // padding columns n >= G read row G - 1's partials and store nothing.
    constexpr int NU = 2;  // partials per batch (four would cost a wave per SIMD in float32)
    const int64_t base = (row0 + min(n, G - 1)) * P_max;
    PartialBatch<BF16, D, BS, NU> pb0;
    if (npre > 0) pb0.load(part_o, part_ml, base, 0, npre, j);
    auto fold = [&]() {
        if (npre <= 0) return;
        pb0.add(S, min(npre, NU));
        for (int i0 = NU; i0 < npre; i0 += NU) {
            PartialBatch<BF16, D, BS, NU> pbi;
            pbi.load(part_o, part_ml, base, i0, npre, j);
            pbi.add(S, min(npre - i0, NU));
        }
    };
    if (start < end)  // one table chunk: end - start <= PS <= kTableChunk * BS
        attend_chunk<BF16, D, BS>(S, qr, kbase, vbase, blk_bytes, trow, num_blocks, start, end, L, lane, n, j,
                                  scale_log2, fold);
    else
        fold();
    store_out<BF16, D, BS>(out_, row0, S, n, j, G);
}

// Clears the suffix kernel's merge counters when no prefix kernel runs (a
// fill kernel rather than a memset, so that a caller capturing the stream
// into a graph records a kernel node).
__global__ __launch_bounds__(256) void clear_counters_kernel(int32_t* __restrict__ c, int n) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) c[i] = 0;
}

}  // namespace pa

// ---------------------------------------------------------------------------- host side

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct SharedPlan {
    int64_t p_pre, p_suf, p_max;
};

inline SharedPlan shared_plan(int32_t block_size, int32_t max_blocks, int32_t max_prefix_blocks, int32_t ps) {
    SharedPlan pl;
    const int64_t a = block_size > 32 ? block_size : 32;
    const int64_t pre_tok = (int64_t)max_prefix_blocks * block_size / a * a;
    pl.p_pre = (pre_tok + ps - 1) / ps;
    pl.p_suf = ((int64_t)max_blocks * block_size + ps - 1) / ps;
    if (pl.p_suf < 1) pl.p_suf = 1;
    pl.p_max = pl.p_pre + pl.p_suf;
    return pl;
}

struct SharedLaunch {
    const void *q, *kc, *vc;
    const int32_t *tables, *lens, *groups, *pblk;
    void* out;
    float *po, *pml;
    int32_t* counters;  // one per (request, kv-head)
    int B, Hq, Hkv, max_blocks, max_pre, num_blocks, num_groups, max_group, PS, P_pre, P_max;
    float sl2;
    hipStream_t s;
};

template <bool BF16, int D, int BS, int NCT>
hipError_t launch_prefix(const SharedLaunch& a) {
    if (a.P_pre == 0 || a.num_groups == 0) return hipSuccess;
    hipLaunchKernelGGL((pa::decode_prefix_kernel<BF16, D, BS, NCT>),
                       dim3((unsigned)a.Hkv, (unsigned)a.P_pre, (unsigned)a.num_groups), dim3(64), 0, a.s, a.q, a.kc,
                       a.vc, a.tables, a.groups, a.pblk, a.po, a.pml, a.counters, a.B * a.Hkv, a.B, a.Hq, a.Hkv,
                       a.Hq / a.Hkv, a.max_blocks, a.max_pre, a.num_blocks, a.max_group, a.PS, a.P_max, a.sl2);
    return hipGetLastError();
}

// Query columns one prefix wave can hold: four 16-column tiles, except for
// float32 with head dim 128, whose four tiles of queries and accumulators
// would not fit the register file (two tiles there).
constexpr int max_columns(bool bf16, int head_dim) { return (!bf16 && head_dim == 128) ? 32 : 64; }

template <bool BF16, int D, int BS>
hipError_t launch_shared(const SharedLaunch& a) {
    const int cols = a.max_group * (a.Hq / a.Hkv);
    hipError_t e;
    if (cols <= 16)
        e = launch_prefix<BF16, D, BS, 1>(a);
    else if (cols <= 32 || max_columns(BF16, D) == 32)
        e = launch_prefix<BF16, D, BS, 2>(a);
    else
        e = launch_prefix<BF16, D, BS, max_columns(BF16, D) / 16>(a);
    if (e != hipSuccess) return e;
    const int P_suf = a.P_max - a.P_pre;
    if (P_suf > 1 && (a.P_pre == 0 || a.num_groups == 0)) {
        // no prefix launch to clear the counters (needed only when a request's
        // own tokens can span several partitions)
        const int nc = a.B * a.Hkv;
        hipLaunchKernelGGL(pa::clear_counters_kernel, dim3((unsigned)((nc + 255) / 256)), dim3(256), 0, a.s,
                           a.counters, nc);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((pa::decode_suffix_kernel<BF16, D, BS>), dim3((unsigned)a.Hkv, (unsigned)a.B, (unsigned)P_suf),
                       dim3(64), 0, a.s, a.q, a.kc, a.vc, a.tables, a.lens, a.pblk, a.po, a.pml, a.counters, a.out,
                       a.Hq, a.Hkv, a.Hq / a.Hkv, a.max_blocks, a.max_pre, a.num_blocks, a.PS, a.P_pre, a.P_max,
                       a.sl2);
    return hipGetLastError();
}

template <bool BF16, int D>
hipError_t shared_bs(int BS, const SharedLaunch& a) {
    switch (BS) {
        case 8: return launch_shared<BF16, D, 8>(a);
        case 16: return launch_shared<BF16, D, 16>(a);
        default: return launch_shared<BF16, D, 32>(a);
    }
}

}  // namespace

extern "C" size_t pa_decode_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                                          int32_t block_size, int32_t max_blocks_per_seq,
                                                          int32_t max_prefix_blocks, int32_t partition_size) {
    if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || block_size <= 0 || max_blocks_per_seq < 0 ||
        max_prefix_blocks < 0 || max_prefix_blocks > max_blocks_per_seq || partition_size <= 0)
        return 0;
    const SharedPlan pl = shared_plan(block_size, max_blocks_per_seq, max_prefix_blocks, partition_size);
    const size_t rows = (size_t)num_seqs * num_q_heads * (size_t)pl.p_max;
    // [pa_decode's counter region, left untouched | partials o | partials (m, l) |
    //  merge counters, one per (request, kv-head) <= num_q_heads per request]:
    // the same workspace can then serve pa_decode's balanced split as well
    return pa_decode_counter_bytes() + align_up(rows * head_dim * sizeof(float)) +
           align_up(rows * 2 * sizeof(float)) + align_up((size_t)num_seqs * num_q_heads * sizeof(int32_t));
}

extern "C" pa_status pa_decode_shared_prefix(const void* q, const void* k_cache, const void* v_cache,
                                             const int32_t* block_tables, const int32_t* seq_lens,
                                             int32_t num_kv_heads, float scale, void* out, void* stream,
                                             int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                             int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                                             pa_dtype dtype, const int32_t* groups,
                                             const int32_t* prefix_blocks, int32_t num_groups,
                                             int32_t max_group_size, int32_t max_prefix_blocks,
                                             int32_t partition_size, void* workspace, size_t workspace_bytes) {
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks < 0 || max_blocks_per_seq < 0 ||
        num_groups < 0 || max_group_size < 1 || max_prefix_blocks < 0 || max_prefix_blocks > max_blocks_per_seq ||
        !std::isfinite(scale))
        return PA_ERR_INVALID_ARG;
    if (num_q_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARG;
    if (dtype != PA_F32 && dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
    if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
    if (block_size != 8 && block_size != 16 && block_size != 32) return PA_ERR_UNSUPPORTED;
    const int G = num_q_heads / num_kv_heads;
    if (G > 16 || (int64_t)max_group_size * G > max_columns(dtype == PA_BF16, head_dim)) return PA_ERR_UNSUPPORTED;
    if (num_seqs > 65535 || num_kv_heads > 65535 || num_groups > 65535 || num_groups > num_seqs)
        return PA_ERR_UNSUPPORTED;
    if ((int64_t)max_blocks_per_seq * block_size > (int64_t)INT32_MAX / 2) return PA_ERR_UNSUPPORTED;
    if (partition_size <= 0 || partition_size % 32 != 0 || partition_size % block_size != 0 ||
        partition_size > 64 * block_size)
        return PA_ERR_UNSUPPORTED;
    if (num_seqs == 0) return PA_OK;
    if (!q || !k_cache || !v_cache || !block_tables || !seq_lens || !out || !prefix_blocks ||
        (num_groups > 0 && !groups))
        return PA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
        (reinterpret_cast<uintptr_t>(block_tables) & 3u) || (reinterpret_cast<uintptr_t>(seq_lens) & 3u) ||
        (reinterpret_cast<uintptr_t>(prefix_blocks) & 3u) || (reinterpret_cast<uintptr_t>(groups) & 3u))
        return PA_ERR_INVALID_ARG;
    const SharedPlan pl = shared_plan(block_size, max_blocks_per_seq, max_prefix_blocks, partition_size);
    if (pl.p_max > 65535) return PA_ERR_UNSUPPORTED;
    const size_t need = pa_decode_shared_prefix_workspace_bytes(num_seqs, num_q_heads, head_dim, block_size,
                                                               max_blocks_per_seq, max_prefix_blocks, partition_size);
    if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)))
        return PA_ERR_INVALID_ARG;
    const size_t rows = (size_t)num_seqs * num_q_heads * (size_t)pl.p_max;
    SharedLaunch a{};
    a.q = q;
    a.kc = k_cache;
    a.vc = v_cache;
    a.tables = block_tables;
    a.lens = seq_lens;
    a.groups = groups;
    a.pblk = prefix_blocks;
    a.out = out;
    char* parts = reinterpret_cast<char*>(workspace) + pa_decode_counter_bytes();
    a.po = reinterpret_cast<float*>(parts);
    a.pml = reinterpret_cast<float*>(parts + align_up(rows * head_dim * sizeof(float)));
    a.counters = reinterpret_cast<int32_t*>(parts + align_up(rows * head_dim * sizeof(float)) +
                                            align_up(rows * 2 * sizeof(float)));
    a.B = num_seqs;
    a.Hq = num_q_heads;
    a.Hkv = num_kv_heads;
    a.max_blocks = max_blocks_per_seq;
    a.max_pre = max_prefix_blocks;
    a.num_blocks = num_blocks;
    a.num_groups = num_groups;
    a.max_group = max_group_size;
    a.PS = partition_size;
    a.P_pre = (int)pl.p_pre;
    a.P_max = (int)pl.p_max;
    a.sl2 = (float)((double)scale * 1.4426950408889634);  // scale * log2(e)
    a.s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e;
    if (dtype == PA_BF16)
        e = head_dim == 128 ? shared_bs<true, 128>(block_size, a) : shared_bs<true, 64>(block_size, a);
    else
        e = head_dim == 128 ? shared_bs<false, 128>(block_size, a) : shared_bs<false, 64>(block_size, a);
    return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}
