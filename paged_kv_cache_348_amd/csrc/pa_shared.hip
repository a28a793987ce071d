// Shared-prefix decode (pa_decode_shared_prefix in include/pa.h).
//
// Requests that begin with the same tokens point their block tables at the
// same physical blocks ("Paged attention in LLMs", "Sharing blocks"; forks
// for parallel samples or beams, MCQ page comparison table).  The attention
// of every request is still its own softmax over its own tokens; what the
// shared blocks allow is reading each shared key/value tile once for all the
// requests of a group instead of once per request.
//
// Three kernels:
//  - decode_prefix_kernel: one wave per (kv-head, partition of the shared
//    prefix, group).  The group's queries for that kv-head (group size x G
//    columns, up to 64, in 16-column matrix-core tiles) all attend over the
//    partition's tokens: each key/value step is loaded once and used by
//    every column tile.  Each (request, head) gets a partial (o, m, l).
//  - decode_suffix_kernel: one wave per (kv-head, partition of the rest,
//    request): the usual decode over the request's own tokens past the
//    prefix, leaving partials after the prefix ones.
//  - merge_shared_kernel: log-sum-exp merge of a row's prefix and suffix
//    partials, M = max_j m_j, w_j = l_j 2^(m_j - M), out = sum w_j o_j / sum w_j.
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
    const int32_t* __restrict__ prefix_blocks, float* __restrict__ part_o, float* __restrict__ part_ml, int B, int Hq,
    int Hkv, int G, int max_blocks, int max_pre, int num_blocks, int max_group, int PS, int P_max, float scale_log2) {
    using C = DecodeCfg<BF16, D, BS>;
    const int g = blockIdx.x;
    const int p = blockIdx.y;
    const int gi = blockIdx.z;
    const int lane = threadIdx.x;
    const int n = lane & 15;
    const int j = lane >> 4;
    const int s0 = groups[2 * gi];
    const int ns = groups[2 * gi + 1];
    if (s0 < 0 || ns < 1 || ns > B - s0) return;  // a malformed group has no prefix work
    const int pb = prefix_blocks[s0];
    if (pb <= 0 || pb > max_pre) return;  // the suffix or merge kernel handles such rows
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

template <bool BF16, int D, int BS>
__global__ __launch_bounds__(64) void decode_suffix_kernel(
    const void* __restrict__ q_, const void* __restrict__ kc_, const void* __restrict__ vc_,
    const int32_t* __restrict__ tables, const int32_t* __restrict__ lens, const int32_t* __restrict__ prefix_blocks,
    float* __restrict__ part_o, float* __restrict__ part_ml, int Hq, int Hkv, int G, int max_blocks, int max_pre,
    int num_blocks, int PS, int P_pre, int P_max, float scale_log2) {
    using C = DecodeCfg<BF16, D, BS>;
    const int g = blockIdx.x;
    const int b = blockIdx.y;
    const int p = blockIdx.z;  // slowest: every request's first partition is dispatched first
    const int lane = threadIdx.x;
    const int n = lane & 15;
    const int j = lane >> 4;
    const int L = lens[b];
    const int pb = prefix_blocks[b];
    if (L <= 0 || (int64_t)L > (int64_t)max_blocks * BS || pb < 0 || pb > max_pre) return;  // merge writes the row
    const int T = shared_tokens<BS>(pb);
    if (T > L) return;
    const int start = T + p * PS;
    if (start >= L) return;
    const int end = min(start + PS, L);
    const int64_t row0 = (int64_t)b * Hq + g * G;
    typename C::QRegs qr;
    load_q<BF16, D, BS>(qr, q_, row0 + n, n, j, G);
    RunState<BF16, D, BS> S;
    run_init(S);
    const int64_t blk_bytes = (int64_t)Hkv * C::TILE * C::ES;
    attend_range<BF16, D, BS>(S, qr, reinterpret_cast<const char*>(kc_) + (int64_t)g * C::TILE * C::ES,
                              reinterpret_cast<const char*>(vc_) + (int64_t)g * C::TILE * C::ES, blk_bytes,
                              tables + (int64_t)b * max_blocks, num_blocks, start, end, L, lane, n, j, scale_log2);
    if (n < G) store_partial<BF16, D, BS>(part_o, part_ml, row0 + n, P_max, P_pre + p, S, j);
}

// One wave per output row (request b, query head h), four rows per
// workgroup: merges the request's prefix partials [0, npre) and its own
// partials [P_pre, P_pre + nsuf).  Lane i holds partial i's (m, l) of the
// current 64-partial window; each lane accumulates D / 64 dims, four
// partials' loads in flight at a time.
template <bool BF16, int D, int BS>
__global__ __launch_bounds__(256) void merge_shared_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_ml,
                                                           const int32_t* __restrict__ lens,
                                                           const int32_t* __restrict__ prefix_blocks,
                                                           void* __restrict__ out_, int B, int Hq, int max_blocks,
                                                           int max_pre, int PS, int P_pre, int P_max) {
    constexpr int PER = D / 64;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= (int64_t)B * Hq) return;
    const int b = (int)(row / Hq);
    const int L = lens[b];
    const int pb = prefix_blocks[b];
    const bool ok = L > 0 && (int64_t)L <= (int64_t)max_blocks * BS && pb >= 0 && pb <= max_pre &&
                    shared_tokens<BS>(pb) <= L;
    float res[PER];
    if (!ok) {
        // empty request: zero row; a length or prefix the table cannot hold: NaN row
#pragma unroll
        for (int e = 0; e < PER; ++e) res[e] = L <= 0 ? 0.0f : __builtin_nanf("");
    } else {
        const int T = shared_tokens<BS>(pb);
        const int npre = (T + PS - 1) / PS;
        const int np = npre + (L - T + PS - 1) / PS;
        const float* ml = part_ml + row * P_max * 2;
        const float* po = part_o + row * P_max * D + lane * PER;
        auto slot = [&](int i) { return i < npre ? i : P_pre + (i - npre); };
        float M = -INFINITY;
        for (int i = lane; i < np; i += 64) M = fmaxf(M, ml[2 * slot(i)]);
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, shfl_xor_f(M, o));
        float num[PER];
#pragma unroll
        for (int e = 0; e < PER; ++e) num[e] = 0.f;
        float den = 0.f;
        for (int w0 = 0; w0 < np; w0 += 64) {
            const int nw = min(64, np - w0);
            float wl = 0.f;
            if (lane < nw) {
                const int si = slot(w0 + lane);
                wl = ml[2 * si + 1] * __builtin_amdgcn_exp2f(ml[2 * si] - M);
            }
            den += wl;
            for (int i0 = 0; i0 < nw; i0 += 4) {
                float v[4][PER];
                float wt[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int i = min(i0 + u, nw - 1);  // past the end: a valid slot, weight 0
                    const float* src = po + (int64_t)slot(w0 + i) * D;
#pragma unroll
                    for (int e = 0; e < PER; ++e) v[u][e] = src[e];
                    const float wi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), i));
                    wt[u] = (i0 + u < nw) ? wi : 0.0f;
                }
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int e = 0; e < PER; ++e) num[e] += wt[u] * v[u][e];
            }
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) den += shfl_xor_f(den, o);
#pragma unroll
        for (int e = 0; e < PER; ++e) res[e] = num[e] / den;
    }
    if constexpr (BF16) {
        uint16_t* o = reinterpret_cast<uint16_t*>(out_) + row * D + lane * PER;
#pragma unroll
        for (int e = 0; e < PER; ++e) o[e] = (uint16_t)bf16_bits_rne(res[e]);
    } else {
        float* o = reinterpret_cast<float*>(out_) + row * D + lane * PER;
#pragma unroll
        for (int e = 0; e < PER; ++e) o[e] = res[e];
    }
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
    int B, Hq, Hkv, max_blocks, max_pre, num_blocks, num_groups, max_group, PS, P_pre, P_max;
    float sl2;
    hipStream_t s;
};

template <bool BF16, int D, int BS, int NCT>
hipError_t launch_prefix(const SharedLaunch& a) {
    if (a.P_pre == 0 || a.num_groups == 0) return hipSuccess;
    hipLaunchKernelGGL((pa::decode_prefix_kernel<BF16, D, BS, NCT>),
                       dim3((unsigned)a.Hkv, (unsigned)a.P_pre, (unsigned)a.num_groups), dim3(64), 0, a.s, a.q, a.kc,
                       a.vc, a.tables, a.groups, a.pblk, a.po, a.pml, a.B, a.Hq, a.Hkv, a.Hq / a.Hkv, a.max_blocks,
                       a.max_pre, a.num_blocks, a.max_group, a.PS, a.P_max, a.sl2);
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
    hipLaunchKernelGGL((pa::decode_suffix_kernel<BF16, D, BS>), dim3((unsigned)a.Hkv, (unsigned)a.B, (unsigned)P_suf),
                       dim3(64), 0, a.s, a.q, a.kc, a.vc, a.tables, a.lens, a.pblk, a.po, a.pml, a.Hq, a.Hkv,
                       a.Hq / a.Hkv, a.max_blocks, a.max_pre, a.num_blocks, a.PS, a.P_pre, a.P_max, a.sl2);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t rows = (int64_t)a.B * a.Hq;
    hipLaunchKernelGGL((pa::merge_shared_kernel<BF16, D, BS>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, a.s,
                       a.po, a.pml, a.lens, a.pblk, a.out, a.B, a.Hq, a.max_blocks, a.max_pre, a.PS, a.P_pre, a.P_max);
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
    // [pa_decode's counter region, left untouched | partials o | partials (m, l)]:
    // the same workspace can then serve pa_decode's balanced split as well
    return pa_decode_counter_bytes() + align_up(rows * head_dim * sizeof(float)) +
           align_up(rows * 2 * sizeof(float));
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
