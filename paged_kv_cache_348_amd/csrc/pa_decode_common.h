// Device building blocks of the decode kernels (gfx950): the per-step
// key/value loads in matrix-core operand order, the step compute (scores,
// online softmax, PV), the run over a token range, and the output and
// partial-result helpers.  Shared by pa_decode.hip and pa_shared.hip.
#pragma once

#include <cmath>
#include <cstdint>
#include <type_traits>

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
    static constexpr int VT = 4;                        // tokens in one value load (f32) / half-load (bf16)
    static constexpr int NE = STEP / BS > 0 ? STEP / BS : 1;  // table entries a step touches
    static constexpr int64_t TILE = (int64_t)D * BS;    // elements of one (block, head) tile
    typedef u32x4 QRegs[NKC];                           // query operand of one lane
    // bf16 with blocks of 16 or 32 tokens: values are stored with bits 2 and 3
    // of the in-block offset swapped, so a lane's 8 value tokens are one
    // 16-byte load (see the layout notes in include/pa.h)
    static constexpr bool VIL = BF16 && BS >= 16;
    static_assert(D % 32 == 0 && BS % 8 == 0, "shape");
};

template <bool BF16, int D, int BS>
struct StepRegs {
    u32x4 k[DecodeCfg<BF16, D, BS>::NT][DecodeCfg<BF16, D, BS>::NKC];
    u32x4 v[DecodeCfg<BF16, D, BS>::NV];
};

// Physical blocks of the (at most four) blocks one step touches, as four
// scalars (an array here would be turned into a per-lane indexed copy in
// scratch memory).
struct StepBlocks {
    int32_t e0, e1, e2, e3;
};

// Physical block holding token t of a step starting at tok0 (entry k covers
// tokens tok0/BS*BS + k*BS ...).  With four entries the lane's entry is
// fetched with a cross-lane read from lanes 0..3 (a chain of selects on a
// per-lane index would be turned into an indexed copy in scratch memory).
template <int NE, int BS>
__device__ __forceinline__ int32_t pick_block(const StepBlocks& e, int t, int tok0) {
    if constexpr (NE == 1) {
        return e.e0;
    } else if constexpr (NE == 2) {
        return (t / BS - tok0 / BS == 1) ? e.e1 : e.e0;
    } else {
        const int lane = threadIdx.x & 63;
        int32_t ev = e.e0;
        ev = (lane == 1) ? e.e1 : ev;
        ev = (lane == 2) ? e.e2 : ev;
        ev = (lane == 3) ? e.e3 : ev;
        return __shfl(ev, t / BS - tok0 / BS, 64);
    }
}

// Issue the loads of one step (tokens tok0 .. tok0 + STEP - 1, clamped to
// L - 1) given the physical blocks e[] of the step's blocks.
template <bool BF16, int D, int BS>
__device__ __forceinline__ void issue_step_e(StepRegs<BF16, D, BS>& r, const char* __restrict__ kbase,
                                             const char* __restrict__ vbase, int64_t blk_bytes, const StepBlocks& e,
                                             int tok0, int L, int n, int j);

template <bool BF16, int D, int BS>
__device__ __forceinline__ void issue_step(StepRegs<BF16, D, BS>& r, const char* __restrict__ kbase,
                                           const char* __restrict__ vbase, int64_t blk_bytes,
                                           int32_t ent, int blk0, int nblk, int tok0, int L, int n, int j) {
    using C = DecodeCfg<BF16, D, BS>;
    // table entries of the blocks this step touches (wave-uniform)
    const int rel0 = tok0 / BS - blk0;
    StepBlocks e;
    e.e0 = lane_value(ent, rel0);
    e.e1 = C::NE > 1 ? lane_value(ent, min(rel0 + 1, nblk - 1)) : 0;
    e.e2 = C::NE > 2 ? lane_value(ent, min(rel0 + 2, nblk - 1)) : 0;
    e.e3 = C::NE > 3 ? lane_value(ent, min(rel0 + 3, nblk - 1)) : 0;
    issue_step_e<BF16, D, BS>(r, kbase, vbase, blk_bytes, e, tok0, L, n, j);
}

template <bool BF16, int D, int BS>
__device__ __forceinline__ void issue_step_e(StepRegs<BF16, D, BS>& r, const char* __restrict__ kbase,
                                             const char* __restrict__ vbase, int64_t blk_bytes, const StepBlocks& e,
                                             int tok0, int L, int n, int j) {
    using C = DecodeCfg<BF16, D, BS>;
    const int last = L - 1;
#pragma unroll
    for (int t = 0; t < C::NT; ++t) {
        // key row n of tile t: with the interleaved value layout, step token
        // 16 (n / 8) + 8 t + n % 8, else 16 t + n.  Either way the rows a lane
        // group reads in one instruction are whole 128-byte lines of a chunk column.
        const int srow = C::VIL ? 16 * (n >> 3) + 8 * t + (n & 7) : 16 * t + n;
        const int tok = min(tok0 + srow, last);  // rows past the end read a valid slot, masked later
        const int32_t phys = pick_block<C::NE, BS>(e, tok, tok0);
        const char* kp = kbase + (int64_t)phys * blk_bytes + (int64_t)(tok % BS) * 16;
#pragma unroll
        for (int c = 0; c < C::NKC; ++c) {
            const int chunk = 4 * c + j;  // 16-byte chunk of the head dim
            r.k[t][c] = ld16_stream(kp + (int64_t)chunk * BS * 16);
        }
    }
    if constexpr (C::VIL) {
        // values: lane group j holds the scores of step tokens
        // 16 (j / 2) + 4 (j % 2) + {0..3} and the same + 8, which the
        // interleaved layout stores as the 8 slots from (tok0 + 8 j) % BS of
        // head-dim row d: one 16-byte load.  A group whose first token is past
        // the end has no valid token: it reads a group of the last token's
        // block instead (masked later).
        const int tv = (tok0 + 16 * (j >> 1) <= last) ? tok0 + 8 * j : (last & ~7);
        const char* vp = vbase + (int64_t)pick_block<C::NE, BS>(e, tv, tok0) * blk_bytes + (int64_t)(tv % BS) * 2;
#pragma unroll
        for (int c = 0; c < C::NV; ++c) {
            const int64_t d = 16 * c + n;
            r.v[c] = ld16_stream(vp + d * BS * 2);
        }
    } else if constexpr (BF16) {
        // values: lane group j reads tokens tok0 + 4j .. +3 (tile 0) and
        // tok0 + 16 + 4j .. +3 (tile 1) of head-dim row d, the tokens whose
        // scores it holds; one 8-byte load each
        const int ta = min(tok0 + 4 * j, last & ~3);
        const int tb = min(tok0 + 16 + 4 * j, last & ~3);
        const char* va = vbase + (int64_t)pick_block<C::NE, BS>(e, ta, tok0) * blk_bytes + (int64_t)(ta % BS) * 2;
        const char* vb = vbase + (int64_t)pick_block<C::NE, BS>(e, tb, tok0) * blk_bytes + (int64_t)(tb % BS) * 2;
#pragma unroll
        for (int c = 0; c < C::NV; ++c) {
            const int64_t d = 16 * c + n;
            const u32x2 lo = ld8_stream(va + d * BS * 2);
            const u32x2 hi = ld8_stream(vb + d * BS * 2);
            r.v[c] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
    } else {
        // values: lane group j reads tokens [tok0 + 4j, +4) of head-dim row d
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
}

// Two floats written / read as one 64-bit agent-scope atomic access: the
// access goes to the device-coherent level, so a wave on another XCD that
// reads it after a later counter update sees it.
__device__ __forceinline__ void coherent_store(uint64_t* p, float lo, float hi) {
    const uint64_t v = (uint64_t)__float_as_uint(lo) | ((uint64_t)__float_as_uint(hi) << 32);
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float2 coherent_load(const uint64_t* p) {
    const uint64_t v = __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return make_float2(__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32)));
}

// Reductions over the four lanes l, l^16, l^32, l^48 (one head column).
// gfx950's permlane swaps exchange 16-lane rows (and 32-lane halves)
// between two registers in the vector ALU, so no LDS crossbar operation
// (and no wait shared with scalar loads) is involved: after a swap of a
// value with itself, the two results hold x[l] and x[l ^ 16] (or x[l ^ 32])
// in every lane, in the same order in both partner lanes.
__device__ __forceinline__ float pair16_max(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair16_sum(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair32_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float wave_max16(float x) { return pair32_max(pair16_max(x)); }
__device__ __forceinline__ float wave_sum16(float x) { return pair32_sum(pair16_sum(x)); }

// Online-softmax reference update with lazy rescaling.  The running
// reference m (per head column) only moves when a step's maximum exceeds it
// by more than kLazyRescale (base 2): then l and the accumulators are scaled
// by 2^(m_old - m_new) and m takes the new maximum.  Otherwise the step's
// probabilities 2^(s - m) stay below 2^kLazyRescale (256: exact range in
// bfloat16 and float32) and no rescale is spent.  Any reference gives the
// same final acc / l; partial results carry their reference as m.  The
// branch is taken by the whole wave (a ballot), on a run's first step with a
// visible key (m = -inf before it).
constexpr float kLazyRescale = 8.0f;

template <int NV>
__device__ __forceinline__ void rescale(float& m_run, float& l_run, f32x4 (&acc)[NV], float mx) {
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kLazyRescale)) {
        const float m_new = fmaxf(m_run, mx);
        // a column with no visible key yet (causal runs) keeps m = -inf and l = acc = 0
        const float alpha = m_new == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int c = 0; c < NV; ++c) acc[c] *= alpha;
        m_run = m_new;
    }
}

// One loop step: scores of the step's tokens for the G query heads, the
// online-softmax update and the PV accumulation.  Tokens at or past L are
// masked: their scores become -inf and their values are zeroed, since a
// stale or NaN value times a zero weight would still poison the sum.
// CAUSAL: each lane's column has its own key limit Lcol <= L (a query token
// sees the keys up to its own position); Lmin is the smallest limit of the
// wave's columns, so steps wholly below it skip the masking.  Values are
// still zeroed only at or past L (everything below L is stored data).
// FMA_EXP (bfloat16, scale_log2 > 0 only): the scores stay unscaled, their
// maximum is scaled once, and each probability is 2^fma(s, scale_log2, -m):
// the same running maximum (rounding is monotonic for a positive factor)
// for one instruction per score instead of two.
template <bool BF16, int D, int BS, bool CAUSAL = false, bool FMA_EXP = false>
__device__ __forceinline__ void compute_step(StepRegs<BF16, D, BS>& cur,
                                             const u32x4 (&qr)[DecodeCfg<BF16, D, BS>::NKC], float& m_run,
                                             float& l_run, f32x4 (&acc)[DecodeCfg<BF16, D, BS>::NV], int tok0,
                                             int L, int j, float scale_log2, int Lcol = 0, int Lmin = 0) {
    using C = DecodeCfg<BF16, D, BS>;
    const int Ls = CAUSAL ? Lcol : L;  // score limit of this lane's column
    const bool tail = tok0 + C::STEP > (CAUSAL ? Lmin : L);
    if constexpr (BF16) {
        // ---- scores: two 16-token tiles (rows as in issue_step_e); lane (n, j)
        // receives rows 4j+i of tile a and of tile b
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
            s[i] = FMA_EXP ? sa[i] : sa[i] * scale_log2;
            s[4 + i] = FMA_EXP ? sb[i] : sb[i] * scale_log2;
        }
        if (tail) {
            // element e of the lane's scores / value operand is token tok(e)
            // element e (score and value operand) of lane group j is step token
            // tok(e); tile 1 holds the second four
            auto tok = [&](int e) {
                return C::VIL ? tok0 + 16 * (j >> 1) + 4 * (j & 1) + (e & 3) + 8 * (e >> 2)
                              : tok0 + 4 * j + (e & 3) + 16 * (e >> 2);
            };
            uint32_t keep[4];
#pragma unroll
            for (int e = 0; e < 8; ++e) s[e] = (tok(e) < Ls) ? s[e] : -INFINITY;
#pragma unroll
            for (int w = 0; w < 4; ++w)
                keep[w] = ((tok(2 * w) < L) ? 0x0000ffffu : 0u) | ((tok(2 * w + 1) < L) ? 0xffff0000u : 0u);
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
        if constexpr (FMA_EXP) mx *= scale_log2;
        rescale<C::NV>(m_run, l_run, acc, mx);
        // causal: a run cut mid-sequence can start with steps whose keys are all
        // past a column's position; that column keeps m = -inf and gets p = 0
        const float mref = (CAUSAL && m_run == -INFINITY) ? 0.0f : m_run;
        float pe[8];
        float rs = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            pe[e] = __builtin_amdgcn_exp2f(FMA_EXP ? __builtin_fmaf(s[e], scale_log2, -mref) : s[e] - mref);
            rs += pe[e];
        }
        rs = wave_sum16(rs);
        l_run += rs;
        const u32x4 pw = {pack_bf16x2(pe[0], pe[1]), pack_bf16x2(pe[2], pe[3]), pack_bf16x2(pe[4], pe[5]),
                          pack_bf16x2(pe[6], pe[7])};
        const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
        for (int c = 0; c < C::NV; ++c)
            acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur.v[c]), pb, acc[c],
                                                            0, 0, 0);
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
            for (int i = 0; i < 4; ++i) s[i] = (base + i < Ls) ? s[i] : -INFINITY;
#pragma unroll
            for (int c = 0; c < C::NV; ++c)
                cur.v[c] = u32x4{base + 0 < L ? cur.v[c][0] : 0u, base + 1 < L ? cur.v[c][1] : 0u,
                                 base + 2 < L ? cur.v[c][2] : 0u, base + 3 < L ? cur.v[c][3] : 0u};
        }
        float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
        mx = wave_max16(mx);
        rescale<C::NV>(m_run, l_run, acc, mx);
        const float mref = (CAUSAL && m_run == -INFINITY) ? 0.0f : m_run;  // as in the bf16 path
        float pe[4];
        float rs = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pe[i] = __builtin_amdgcn_exp2f(s[i] - mref);
            rs += pe[i];
        }
        rs = wave_sum16(rs);
        l_run += rs;
#pragma unroll
        for (int c = 0; c < C::NV; ++c) {
            const f32x4 vf = __builtin_bit_cast(f32x4, cur.v[c]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf[i], pe[i], acc[c], 0, 0, 0);
        }
    }
}

// Running state of one wave over a run of tokens of one (sequence, kv-head):
// online-softmax maximum and sum per head column, the unnormalised PV
// accumulator, and whether a bad block-table entry was met.
template <bool BF16, int D, int BS>
struct RunState {
    float m;
    float l;
    f32x4 acc[DecodeCfg<BF16, D, BS>::NV];
    bool bad;
};

template <bool BF16, int D, int BS>
__device__ __forceinline__ void run_init(RunState<BF16, D, BS>& S) {
    S.m = -INFINITY;
    S.l = 0.0f;
#pragma unroll
    for (int c = 0; c < DecodeCfg<BF16, D, BS>::NV; ++c) S.acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    S.bad = false;
}

// Query operand of kv-head g's G query heads: lane (n, j) holds 16-byte
// chunks 4c + j of head g*G + n (zero for the padding columns n >= G).
template <bool BF16, int D, int BS>
__device__ __forceinline__ void load_q(typename DecodeCfg<BF16, D, BS>::QRegs& qr, const void* __restrict__ q_,
                                       int64_t row, int n, int j, int G) {
    using C = DecodeCfg<BF16, D, BS>;
    const char* qp = reinterpret_cast<const char*>(q_) + row * D * C::ES;
#pragma unroll
    for (int c = 0; c < C::NKC; ++c) qr[c] = (n < G) ? ld16(qp + (int64_t)(4 * c + j) * 16) : u32x4{0u, 0u, 0u, 0u};
}

struct NoHook {
    __device__ __forceinline__ void operator()() const {}
};

// Attention over tokens [ctok, cend) of one sequence (cend - ctok <=
// kTableChunk * BS, cend <= L) for one kv-head: the chunk's block-table
// entries are read once (one per lane, read back with readlane) and the
// tokens are streamed in steps through a two-stage load pipeline.  The loop
// body issues the next step's loads unconditionally, so the wait before each
// compute covers only the current step's loads.  hook() runs after the
// table entries have arrived and before the first step's loads are issued:
// work on loads the caller issued before the call costs no round trip of
// its own there.  Returns false (S.bad set, nothing read) on an entry
// outside the pool.
template <bool BF16, int D, int BS, class Hook = NoHook>
__device__ __forceinline__ bool attend_chunk(RunState<BF16, D, BS>& S,
                                             const u32x4 (&qr)[DecodeCfg<BF16, D, BS>::NKC],
                                             const char* __restrict__ kbase, const char* __restrict__ vbase,
                                             int64_t blk_bytes, const int32_t* __restrict__ trow, int num_blocks,
                                             int ctok, int cend, int L, int lane, int n, int j, float scale_log2,
                                             Hook&& hook = Hook{}) {
    using C = DecodeCfg<BF16, D, BS>;
    const int blk0 = ctok / BS;
    const int nblk = (cend - 1) / BS - blk0 + 1;
    const int32_t ent = (lane < nblk) ? trow[blk0 + lane] : 0;
    const bool bad = __any(lane < nblk && (ent < 0 || ent >= num_blocks));
    if constexpr (!std::is_same_v<std::decay_t<Hook>, NoHook>) {
        hook();
        __builtin_amdgcn_sched_barrier(0);  // the hook's registers die before the first step's are allocated
    }
    if (bad) {
        S.bad = true;
        return false;
    }
    const int nst = (cend - ctok + C::STEP - 1) / C::STEP;
    StepRegs<BF16, D, BS> cur;
    issue_step<BF16, D, BS>(cur, kbase, vbase, blk_bytes, ent, blk0, nblk, ctok, L, n, j);
    int tok0 = ctok;
    for (int st = 0; st + 1 < nst; ++st, tok0 += C::STEP) {
        StepRegs<BF16, D, BS> nxt;
        issue_step<BF16, D, BS>(nxt, kbase, vbase, blk_bytes, ent, blk0, nblk, tok0 + C::STEP, L, n, j);
        __builtin_amdgcn_sched_barrier(0);  // loads stay ahead of the compute
        compute_step<BF16, D, BS>(cur, qr, S.m, S.l, S.acc, tok0, L, j, scale_log2);
        cur = nxt;
    }
    compute_step<BF16, D, BS>(cur, qr, S.m, S.l, S.acc, tok0, L, j, scale_log2);
    return true;
}

// Attention over tokens [start, end) of one sequence (0 <= start < end <= L)
// for one kv-head, walking the block table in chunks of kTableChunk entries.
template <bool BF16, int D, int BS>
__device__ __forceinline__ void attend_range(RunState<BF16, D, BS>& S,
                                             const u32x4 (&qr)[DecodeCfg<BF16, D, BS>::NKC],
                                             const char* __restrict__ kbase, const char* __restrict__ vbase,
                                             int64_t blk_bytes, const int32_t* __restrict__ trow, int num_blocks,
                                             int start, int end, int L, int lane, int n, int j, float scale_log2) {
    for (int ctok = start; ctok < end; ctok += kTableChunk * BS)
        if (!attend_chunk<BF16, D, BS>(S, qr, kbase, vbase, blk_bytes, trow, num_blocks, ctok,
                                       min(ctok + kTableChunk * BS, end), L, lane, n, j, scale_log2))
            return;
}

// Normalise and store the G output rows of one (sequence, kv-head) starting
// at row `row0` of out; a bad table entry gives NaN rows.
template <bool BF16, int D, int BS>
__device__ __forceinline__ void store_out(void* __restrict__ out_, int64_t row0, const RunState<BF16, D, BS>& S,
                                          int n, int j, int G) {
    using C = DecodeCfg<BF16, D, BS>;
    if (n >= G) return;
    const float inv = S.bad ? __builtin_nanf("") : 1.0f / S.l;
    const int64_t orow = (row0 + n) * D;
#pragma unroll
    for (int c = 0; c < C::NV; ++c) {
        const int d0 = 16 * c + 4 * j;
        if constexpr (BF16) {
            uint2 w;
            w.x = pack_bf16x2(S.acc[c][0] * inv, S.acc[c][1] * inv);
            w.y = pack_bf16x2(S.acc[c][2] * inv, S.acc[c][3] * inv);
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out_) + orow + d0) = w;
        } else {
            *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out_) + orow + d0) = S.acc[c] * inv;
        }
    }
}

// Fill `nrows` output rows from `row0` with v (zero rows for empty
// sequences, NaN rows for lengths the block table cannot hold).
template <bool BF16, int D>
__device__ __forceinline__ void fill_rows(void* __restrict__ out_, int64_t row0, int nrows, float v, int lane) {
    for (int i = lane; i < nrows * D; i += 64) {
        const int64_t o = row0 * D + i;
        if constexpr (BF16)
            reinterpret_cast<uint16_t*>(out_)[o] = (uint16_t)bf16_bits_rne(v);
        else
            reinterpret_cast<float*>(out_)[o] = v;
    }
}

}  // namespace pa
