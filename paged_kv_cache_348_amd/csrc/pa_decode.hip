// Paged single-query decode attention for gfx950 (pa_decode in include/pa.h).
//
// The pages describe the method; this is one gfx950 realisation of it:
//  - attention over a request's tokens is standard scaled dot-product
//    attention; only the storage is paged ("Paged Attention", chapter
//    introduction; PagedAttention MCQ page, code sketch);
//  - position pos is read from block table[pos / bs], offset pos % bs, and
//    the lookup sits inside the tile loop rather than in a separate gather
//    (MCQ page, code sketch and its closing remark).
//
// Work decomposition.  One 64-lane wave per (partition, kv-head, sequence).
// The wave walks its partition in steps of 32 tokens (bf16) or 16 tokens
// (f32).  Each step loads the keys and values of its tokens straight from
// the pool into registers with 16-byte loads whose per-lane placement is the
// matrix-core operand layout (the pool's tile layout is chosen for that,
// see include/pa.h), so no key or value passes through LDS: every element
// is used by exactly one lane.  The next step's loads are issued before the
// current step is computed.
//
// Per step, with the G query heads of the kv-head as the N columns of the
// matrix-core tile (padded to 16):
//   scores  S[token][head] = K[token][:] . q[head][:]   (MFMA, fp32 acc)
//   online softmax per head, in base 2 with scale*log2(e) folded into the
//   scores: m' = max(m, max S), alpha = 2^(m - m'), p = 2^(S - m'),
//   l = alpha l + sum p, acc = alpha acc
//   acc[d][head] += V^T[d][token] . p[token][head]        (MFMA, fp32 acc)
// The row/column maxima and sums across the four 16-lane groups use
// cross-lane shuffles.
//
// Matrix-core operand facts relied on (16x16 tiles, 64 lanes):
//  - lane l supplies row (l % 16) of A and column (l % 16) of B; the
//    contraction slots a lane supplies are set by l / 16 and the element
//    index, identically for A and B;
//  - lane l receives C[4 * (l / 16) + i][l % 16] in accumulator element i.
// Because A and B share the contraction-slot assignment, any placement of
// head-dim elements (for scores) or tokens (for PV) onto those slots is
// valid as long as both operands use it; the loads below pick placements
// that make every lane's 16 bytes contiguous in the pool.
//
// Long contexts: a sequence longer than one partition writes per-partition
// (o_j, m_j, l_j) to the workspace and merge_kernel combines them with the
// log-sum-exp rule.  m_j is kept in the base-2 scaled domain
// (m_j = max_p scale*log2(e)*score), so the merge weights are
// w_j = l_j * 2^(m_j - M).

#include <cmath>
#include <cstdint>

#include "pa.h"
#include "pa_device.h"

namespace pa {

constexpr int kTableChunk = 64;  // block-table entries held at once (one per lane)

template <bool BF16, int D, int BS>
struct DecodeCfg {
    static constexpr int ES = BF16 ? 2 : 4;            // element bytes
    static constexpr int X = 16 / ES;                   // elements per 16-byte chunk
    static constexpr int STEP = BF16 ? 32 : 16;         // tokens per loop step
    static constexpr int NT = BF16 ? 2 : 1;             // 16-row key tiles per step
    static constexpr int NKC = BF16 ? D / 32 : D / 16;  // 16-byte key loads per lane per tile
    static constexpr int NV = D / 16;                   // 16-byte value loads per lane per step
    static constexpr int VT = BF16 ? 8 : 4;             // tokens in one value load
    static constexpr int NE = STEP / BS > 0 ? STEP / BS : 1;  // table entries a step touches
    static constexpr int64_t TILE = (int64_t)D * BS;    // elements of one (block, head) tile
    static_assert(D % 32 == 0 && BS % 8 == 0, "shape");
};

template <bool BF16, int D, int BS>
struct StepRegs {
    u32x4 k[DecodeCfg<BF16, D, BS>::NT][DecodeCfg<BF16, D, BS>::NKC];
    u32x4 v[DecodeCfg<BF16, D, BS>::NV];
};

// Physical block holding token t of a step starting at tok0, from the
// step's table entries e[] (entry k covers tokens tok0/BS*BS + k*BS ...).
template <int NE, int BS>
__device__ __forceinline__ int32_t pick_block(const int32_t (&e)[NE], int t, int tok0) {
    if constexpr (NE == 1) {
        return e[0];
    } else {
        const int k = t / BS - tok0 / BS;
        int32_t r = e[0];
#pragma unroll
        for (int i = 1; i < NE; ++i) r = (k == i) ? e[i] : r;
        return r;
    }
}

template <bool BF16, int D, int BS>
__device__ __forceinline__ void issue_step(StepRegs<BF16, D, BS>& r, const char* __restrict__ kbase,
                                           const char* __restrict__ vbase, int64_t blk_bytes,
                                           int32_t ent, int blk0, int nblk, int tok0, int L, int n, int j) {
    using C = DecodeCfg<BF16, D, BS>;
    // table entries of the blocks this step touches (wave-uniform)
    int32_t e[C::NE];
    const int rel0 = tok0 / BS - blk0;
#pragma unroll
    for (int i = 0; i < C::NE; ++i) {
        const int rel = min(rel0 + i, nblk - 1);
        e[i] = lane_value(ent, rel);
    }
    const int last = L - 1;
#pragma unroll
    for (int t = 0; t < C::NT; ++t) {
        // key row n of tile t holds token: bf16 tile a 8*(n/4)+n%4, tile b +4; f32 token n
        int tok = BF16 ? tok0 + 8 * (n >> 2) + (n & 3) + 4 * t : tok0 + n;
        tok = min(tok, last);  // rows past the end read a valid slot and are masked later
        const int32_t phys = pick_block<C::NE, BS>(e, tok, tok0);
        const char* kp = kbase + (int64_t)phys * blk_bytes + (int64_t)(tok % BS) * 16;
#pragma unroll
        for (int c = 0; c < C::NKC; ++c) {
            const int chunk = 4 * c + j;  // 16-byte chunk of the head dim
            r.k[t][c] = ld16_stream(kp + (int64_t)chunk * BS * 16);
        }
    }
    // values: lane group j reads tokens [tok0 + VT*j, +VT) of head-dim row d
    int tv = tok0 + C::VT * j;
    tv = min(tv, last & ~(C::VT - 1));
    const int32_t pv = pick_block<C::NE, BS>(e, tv, tok0);
    const char* vp = vbase + (int64_t)pv * blk_bytes + (int64_t)(tv % BS) * C::ES;
#pragma unroll
    for (int c = 0; c < C::NV; ++c) {
        const int d = 16 * c + n;
        r.v[c] = ld16_stream(vp + (int64_t)d * BS * C::ES);
    }
}

__device__ __forceinline__ float wave_max16(float x) {
    // reduce over the four lanes l, l^16, l^32, l^48 (the same head column)
    x = fmaxf(x, shfl_xor_f(x, 16));
    x = fmaxf(x, shfl_xor_f(x, 32));
    return x;
}

__device__ __forceinline__ float wave_sum16(float x) {
    x += shfl_xor_f(x, 16);
    x += shfl_xor_f(x, 32);
    return x;
}

// One loop step: scores of the step's tokens for the G query heads, the
// online-softmax update and the PV accumulation.  Tokens at or past L are
// masked: their scores become -inf and their values are zeroed, since a
// stale or NaN value times a zero weight would still poison the sum.
template <bool BF16, int D, int BS>
__device__ __forceinline__ void compute_step(StepRegs<BF16, D, BS>& cur,
                                             const u32x4 (&qr)[DecodeCfg<BF16, D, BS>::NKC], float& m_run,
                                             float& l_run, f32x4 (&acc)[DecodeCfg<BF16, D, BS>::NV], int tok0,
                                             int L, int j, float scale_log2) {
    using C = DecodeCfg<BF16, D, BS>;
    const bool tail = tok0 + C::STEP > L;
    if constexpr (BF16) {
        // ---- scores: two 16-token tiles, rows 4j+i <-> tokens 8j+i (tile a), 8j+4+i (tile b)
        f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < C::NKC; ++c) {
            const bf16x8 qv = __builtin_bit_cast(bf16x8, qr[c]);
            sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur.k[0][c]), qv, sa,
                                                        0, 0, 0);
            sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur.k[1][c]), qv, sb,
                                                        0, 0, 0);
        }
        float s[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s[i] = sa[i] * scale_log2;
            s[4 + i] = sb[i] * scale_log2;
        }
        if (tail) {
            const int base = tok0 + 8 * j;
            uint32_t keep[4];
#pragma unroll
            for (int e = 0; e < 8; ++e) s[e] = (base + e < L) ? s[e] : -INFINITY;
#pragma unroll
            for (int w = 0; w < 4; ++w)
                keep[w] = ((base + 2 * w < L) ? 0x0000ffffu : 0u) | ((base + 2 * w + 1 < L) ? 0xffff0000u : 0u);
            // values of masked tokens may be NaN: zero them (p = 0 would not)
#pragma unroll
            for (int c = 0; c < C::NV; ++c)
                cur.v[c] = u32x4{cur.v[c][0] & keep[0], cur.v[c][1] & keep[1], cur.v[c][2] & keep[2],
                                 cur.v[c][3] & keep[3]};
        }
        float mx = s[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) mx = fmaxf(mx, s[e]);
        mx = wave_max16(mx);
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        float pe[8];
        float rs = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            pe[e] = __builtin_amdgcn_exp2f(s[e] - m_new);
            rs += pe[e];
        }
        rs = wave_sum16(rs);
        l_run = l_run * alpha + rs;
        m_run = m_new;
        const u32x4 pw = {pack_bf16x2(pe[0], pe[1]), pack_bf16x2(pe[2], pe[3]), pack_bf16x2(pe[4], pe[5]),
                          pack_bf16x2(pe[6], pe[7])};
        const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
        for (int c = 0; c < C::NV; ++c) {
            acc[c] *= alpha;
            acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur.v[c]), pb, acc[c],
                                                            0, 0, 0);
        }
    } else {
        // ---- scores: one 16-token tile, row 4j+i <-> token 4j+i
        f32x4 s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < C::NKC; ++c) {
            const f32x4 kf = __builtin_bit_cast(f32x4, cur.k[0][c]);
            const f32x4 qf = __builtin_bit_cast(f32x4, qr[c]);
#pragma unroll
            for (int e = 0; e < 4; ++e) s4 = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[e], qf[e], s4, 0, 0, 0);
        }
        float s[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) s[i] = s4[i] * scale_log2;
        if (tail) {
            const int base = tok0 + 4 * j;
#pragma unroll
            for (int i = 0; i < 4; ++i) s[i] = (base + i < L) ? s[i] : -INFINITY;
#pragma unroll
            for (int c = 0; c < C::NV; ++c)
                cur.v[c] = u32x4{base + 0 < L ? cur.v[c][0] : 0u, base + 1 < L ? cur.v[c][1] : 0u,
                                 base + 2 < L ? cur.v[c][2] : 0u, base + 3 < L ? cur.v[c][3] : 0u};
        }
        float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
        mx = wave_max16(mx);
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        float pe[4];
        float rs = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pe[i] = __builtin_amdgcn_exp2f(s[i] - m_new);
            rs += pe[i];
        }
        rs = wave_sum16(rs);
        l_run = l_run * alpha + rs;
        m_run = m_new;
#pragma unroll
        for (int c = 0; c < C::NV; ++c) {
            acc[c] *= alpha;
            const f32x4 vf = __builtin_bit_cast(f32x4, cur.v[c]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf[i], pe[i], acc[c], 0, 0, 0);
        }
    }}

template <bool BF16, int D, int BS>
__global__ __launch_bounds__(64) void decode_kernel(
    const void* __restrict__ q_, const void* __restrict__ kc_, const void* __restrict__ vc_,
    const int32_t* __restrict__ tables, const int32_t* __restrict__ lens, void* __restrict__ out_,
    float* __restrict__ part_o, float* __restrict__ part_ml, int Hq, int Hkv, int G, int max_blocks,
    int num_blocks, int PS, int P_max, float scale_log2) {
    using C = DecodeCfg<BF16, D, BS>;
    const int g = blockIdx.x;  // kv-head fastest: consecutive workgroups land on different XCDs
    const int p = blockIdx.y;
    const int b = blockIdx.z;
    const int lane = threadIdx.x;
    const int n = lane & 15;  // head column: query head g*G + n when n < G
    const int j = lane >> 4;  // lane group

    const int L = lens[b];
    const bool len_ok = L > 0 && (int64_t)L <= (int64_t)max_blocks * BS;
    const int nparts = len_ok ? (L + PS - 1) / PS : 1;
    if (p >= nparts) return;
    const bool direct = nparts == 1;
    const int h = g * G + n;

    if (!len_ok) {
        // empty sequence: zero row; a length the table cannot hold: NaN row
        const float fill = (L <= 0) ? 0.0f : __builtin_nanf("");
        for (int i = lane; i < G * D; i += 64) {
            const int64_t o = ((int64_t)b * Hq + g * G) * D + i;
            if constexpr (BF16)
                reinterpret_cast<uint16_t*>(out_)[o] = (uint16_t)bf16_bits_rne(fill);
            else
                reinterpret_cast<float*>(out_)[o] = fill;
        }
        return;
    }

    const int start = p * PS;
    const int end = min(start + PS, L);
    const int64_t blk_bytes = (int64_t)Hkv * C::TILE * C::ES;
    const char* kbase = reinterpret_cast<const char*>(kc_) + (int64_t)g * C::TILE * C::ES;
    const char* vbase = reinterpret_cast<const char*>(vc_) + (int64_t)g * C::TILE * C::ES;
    const int32_t* trow = tables + (int64_t)b * max_blocks;

    // query operand: lane holds 16-byte chunks 4*c + j of head n (zero for padding heads)
    u32x4 qr[C::NKC];
    {
        const char* qp = reinterpret_cast<const char*>(q_) + ((int64_t)b * Hq + h) * D * C::ES;
#pragma unroll
        for (int c = 0; c < C::NKC; ++c) {
            qr[c] = (n < G) ? ld16(qp + (int64_t)(4 * c + j) * 16) : u32x4{0u, 0u, 0u, 0u};
        }
    }

    float m_run = -INFINITY;
    float l_run = 0.0f;
    f32x4 acc[C::NV];
#pragma unroll
    for (int c = 0; c < C::NV; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    bool bad = false;

    for (int ctok = start; ctok < end; ctok += kTableChunk * BS) {
        const int cend = min(ctok + kTableChunk * BS, end);
        const int blk0 = ctok / BS;
        const int nblk = (cend - 1) / BS - blk0 + 1;
        const int32_t ent = (lane < nblk) ? trow[blk0 + lane] : 0;
        if (__any(lane < nblk && (ent < 0 || ent >= num_blocks))) {
            bad = true;
            break;
        }
        const int nst = (cend - ctok + C::STEP - 1) / C::STEP;
        // two-stage software pipeline: the next step's loads are in flight
        // while the current step is computed; the loop body issues them
        // unconditionally so the wait before each compute covers only the
        // current step's loads
        StepRegs<BF16, D, BS> cur;
        issue_step<BF16, D, BS>(cur, kbase, vbase, blk_bytes, ent, blk0, nblk, ctok, L, n, j);
        int tok0 = ctok;
        for (int st = 0; st + 1 < nst; ++st, tok0 += C::STEP) {
            StepRegs<BF16, D, BS> nxt;
            issue_step<BF16, D, BS>(nxt, kbase, vbase, blk_bytes, ent, blk0, nblk, tok0 + C::STEP, L, n, j);
            compute_step<BF16, D, BS>(cur, qr, m_run, l_run, acc, tok0, L, j, scale_log2);
            cur = nxt;
        }
        compute_step<BF16, D, BS>(cur, qr, m_run, l_run, acc, tok0, L, j, scale_log2);
    }

    if (n >= G) return;
    const float nanv = __builtin_nanf("");
    const float inv = bad ? nanv : 1.0f / l_run;
    if (direct) {
        const int64_t orow = ((int64_t)b * Hq + h) * D;
#pragma unroll
        for (int c = 0; c < C::NV; ++c) {
            const int d0 = 16 * c + 4 * j;
            if constexpr (BF16) {
                uint2 w;
                w.x = pack_bf16x2(acc[c][0] * inv, acc[c][1] * inv);
                w.y = pack_bf16x2(acc[c][2] * inv, acc[c][3] * inv);
                *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out_) + orow + d0) = w;
            } else {
                *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out_) + orow + d0) = acc[c] * inv;
            }
        }
    } else {
        const int64_t prow = ((int64_t)b * Hq + h) * P_max + p;
#pragma unroll
        for (int c = 0; c < C::NV; ++c) {
            const int d0 = 16 * c + 4 * j;
            *reinterpret_cast<f32x4*>(part_o + prow * D + d0) = acc[c] * inv;
        }
        if (j == 0) {
            part_ml[2 * prow] = bad ? 0.0f : m_run;
            part_ml[2 * prow + 1] = bad ? 1.0f : l_run;
        }
    }
}

// Log-sum-exp merge of per-partition results: one 256-lane workgroup per
// (query head, sequence); wave w takes partitions w, w+4, ...
template <bool BF16, int D>
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ part_o,
                                                    const float* __restrict__ part_ml,
                                                    const int32_t* __restrict__ lens, void* __restrict__ out_,
                                                    int Hq, int max_blocks, int BS, int PS, int P_max) {
    const int h = blockIdx.x;
    const int b = blockIdx.y;
    const int L = lens[b];
    if (L <= 0 || (int64_t)L > (int64_t)max_blocks * BS) return;  // written by the decode kernel
    const int np = (L + PS - 1) / PS;
    if (np <= 1) return;
    const int64_t row = (int64_t)b * Hq + h;
    const float* ml = part_ml + row * P_max * 2;
    const float* po = part_o + row * P_max * D;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;

    float M = -INFINITY;
    for (int i = lane; i < np; i += 64) M = fmaxf(M, ml[2 * i]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, shfl_xor_f(M, o));

    constexpr int PER = D / 64;
    float num[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) num[e] = 0.f;
    float den = 0.f;
    for (int i = w; i < np; i += 4) {
        const float wt = ml[2 * i + 1] * __builtin_amdgcn_exp2f(ml[2 * i] - M);
        den += wt;
#pragma unroll
        for (int e = 0; e < PER; ++e) num[e] += wt * po[(int64_t)i * D + lane * PER + e];
    }
    __shared__ float s_num[4][D];
    __shared__ float s_den[4];
#pragma unroll
    for (int e = 0; e < PER; ++e) s_num[w][lane * PER + e] = num[e];
    if (lane == 0) s_den[w] = den;
    __syncthreads();
    if (threadIdx.x < D) {
        const int d = threadIdx.x;
        const float total = s_den[0] + s_den[1] + s_den[2] + s_den[3];
        const float v = (s_num[0][d] + s_num[1][d] + s_num[2][d] + s_num[3][d]) / total;
        if constexpr (BF16)
            reinterpret_cast<uint16_t*>(out_)[row * D + d] = (uint16_t)bf16_bits_rne(v);
        else
            reinterpret_cast<float*>(out_)[row * D + d] = v;
    }
}

}  // namespace pa

// ---------------------------------------------------------------------------- host side

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Effective partition length and partition count for a call.
inline void partition_plan(int32_t block_size, int32_t max_blocks, int32_t partition_size, int64_t* ps,
                           int64_t* pmax) {
    const int64_t cap = (int64_t)max_blocks * block_size;
    if (partition_size == 0) {
        const int64_t whole = cap > 0 ? cap : 1;
        *ps = (whole + 31) / 32 * 32;
        *pmax = 1;
    } else {
        *ps = partition_size;
        *pmax = cap > 0 ? (cap + partition_size - 1) / partition_size : 1;
    }
}

template <bool BF16, int D, int BS>
hipError_t launch_decode(const void* q, const void* kc, const void* vc, const int32_t* tables,
                         const int32_t* lens, void* out, float* po, float* pml, int B, int Hq, int Hkv,
                         int max_blocks, int num_blocks, int PS, int P_max, float scale_log2,
                         hipStream_t stream) {
    dim3 grid((unsigned)Hkv, (unsigned)P_max, (unsigned)B);
    hipLaunchKernelGGL((pa::decode_kernel<BF16, D, BS>), grid, dim3(64), 0, stream, q, kc, vc, tables, lens, out,
                       po, pml, Hq, Hkv, Hq / Hkv, max_blocks, num_blocks, PS, P_max, scale_log2);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || P_max <= 1) return e;
    hipLaunchKernelGGL((pa::merge_kernel<BF16, D>), dim3((unsigned)Hq, (unsigned)B), dim3(256), 0, stream, po, pml,
                       lens, out, Hq, max_blocks, BS, PS, P_max);
    return hipGetLastError();
}

template <bool BF16, int D>
hipError_t dispatch_bs(int BS, const void* q, const void* kc, const void* vc, const int32_t* tables,
                       const int32_t* lens, void* out, float* po, float* pml, int B, int Hq, int Hkv,
                       int max_blocks, int num_blocks, int PS, int P_max, float sl2, hipStream_t s) {
    switch (BS) {
        case 8:
            return launch_decode<BF16, D, 8>(q, kc, vc, tables, lens, out, po, pml, B, Hq, Hkv, max_blocks,
                                             num_blocks, PS, P_max, sl2, s);
        case 16:
            return launch_decode<BF16, D, 16>(q, kc, vc, tables, lens, out, po, pml, B, Hq, Hkv, max_blocks,
                                              num_blocks, PS, P_max, sl2, s);
        default:
            return launch_decode<BF16, D, 32>(q, kc, vc, tables, lens, out, po, pml, B, Hq, Hkv, max_blocks,
                                              num_blocks, PS, P_max, sl2, s);
    }
}

}  // namespace

extern "C" size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                            int32_t block_size, int32_t max_blocks_per_seq,
                                            int32_t partition_size) {
    if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || block_size <= 0 || max_blocks_per_seq < 0 ||
        partition_size < 0)
        return 0;
    int64_t ps, pmax;
    partition_plan(block_size, max_blocks_per_seq, partition_size, &ps, &pmax);
    if (pmax <= 1) return 0;
    const size_t rows = (size_t)num_seqs * num_q_heads * (size_t)pmax;
    return align_up(rows * head_dim * sizeof(float)) + align_up(rows * 2 * sizeof(float));
}

extern "C" pa_status pa_decode(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, const int32_t* seq_lens, int32_t num_kv_heads,
                               float scale, void* out, void* stream, int32_t num_seqs, int32_t num_q_heads,
                               int32_t head_dim, int32_t block_size, int32_t num_blocks,
                               int32_t max_blocks_per_seq, pa_dtype dtype, int32_t partition_size,
                               void* workspace, size_t workspace_bytes) {
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks < 0 || max_blocks_per_seq < 0 ||
        partition_size < 0 || !std::isfinite(scale))
        return PA_ERR_INVALID_ARG;
    if (num_q_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARG;
    if (dtype != PA_F32 && dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
    if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
    if (block_size != 8 && block_size != 16 && block_size != 32) return PA_ERR_UNSUPPORTED;
    if (num_q_heads / num_kv_heads > 16) return PA_ERR_UNSUPPORTED;
    if (num_seqs > 65535 || num_kv_heads > 65535) return PA_ERR_UNSUPPORTED;
    if ((int64_t)max_blocks_per_seq * block_size > (int64_t)INT32_MAX / 2) return PA_ERR_UNSUPPORTED;
    if (partition_size > 0 &&
        (partition_size % 32 != 0 || partition_size % block_size != 0 || partition_size > 64 * block_size))
        return PA_ERR_UNSUPPORTED;
    if (num_seqs == 0) return PA_OK;
    if (!q || !k_cache || !v_cache || !block_tables || !seq_lens || !out) return PA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
        (reinterpret_cast<uintptr_t>(block_tables) & 3u) || (reinterpret_cast<uintptr_t>(seq_lens) & 3u))
        return PA_ERR_INVALID_ARG;

    int64_t ps, pmax;
    partition_plan(block_size, max_blocks_per_seq, partition_size, &ps, &pmax);
    if (pmax > 65535) return PA_ERR_UNSUPPORTED;
    float* po = nullptr;
    float* pml = nullptr;
    if (pmax > 1) {
        const size_t need = pa_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, block_size,
                                                      max_blocks_per_seq, partition_size);
        if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)))
            return PA_ERR_INVALID_ARG;
        const size_t rows = (size_t)num_seqs * num_q_heads * (size_t)pmax;
        po = reinterpret_cast<float*>(workspace);
        pml = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + align_up(rows * head_dim * sizeof(float)));
    }
    const float sl2 = (float)((double)scale * 1.4426950408889634);  // scale * log2(e)
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e;
    const int B = num_seqs, Hq = num_q_heads, Hkv = num_kv_heads, MB = max_blocks_per_seq, NB = num_blocks;
    const int PS = (int)ps, PM = (int)pmax;
    if (dtype == PA_BF16) {
        e = head_dim == 128 ? dispatch_bs<true, 128>(block_size, q, k_cache, v_cache, block_tables, seq_lens, out, po,
                                                     pml, B, Hq, Hkv, MB, NB, PS, PM, sl2, s)
                            : dispatch_bs<true, 64>(block_size, q, k_cache, v_cache, block_tables, seq_lens, out, po,
                                                    pml, B, Hq, Hkv, MB, NB, PS, PM, sl2, s);
    } else {
        e = head_dim == 128 ? dispatch_bs<false, 128>(block_size, q, k_cache, v_cache, block_tables, seq_lens, out,
                                                      po, pml, B, Hq, Hkv, MB, NB, PS, PM, sl2, s)
                            : dispatch_bs<false, 64>(block_size, q, k_cache, v_cache, block_tables, seq_lens, out, po,
                                                     pml, B, Hq, Hkv, MB, NB, PS, PM, sl2, s);
    }
    return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}
