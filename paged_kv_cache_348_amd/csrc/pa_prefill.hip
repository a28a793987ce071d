// Multi-token query over the paged cache (pa_prefill in include/pa.h):
// prefill, chunked prefill and speculative verification all attend a run of
// new query tokens of a request to its cached keys and values with a causal
// mask.  The new tokens' keys and values are in the cache already (written
// with pa_cache_write, as the cache grows by the tokens a step adds: "Paged
// attention in LLMs", "The cache being stored"); query token i of a request
// with L cached tokens and M new ones sits at position L - M + i and sees the
// keys at positions 0 .. L - M + i.  The attention is the standard scaled
// dot-product over those keys, reached through the block table (MCQ page,
// code sketch: the lookup inside the tile loop).
//
// One wave per (kv-head, tile of query tokens, request).  The tile's query
// columns are (token, head) pairs, token-major: QT tokens x G heads, up to
// 64 columns in 16-column matrix-core tiles (32 for float32 with head dim
// 128).  The wave streams the request's keys and values from position 0 to
// its last token's position once for all columns — the same step loop as the
// decode kernels — and each lane masks the keys past its own column's
// position.
//
// Key partitions: when a launch would hold few waves (short chunks of a
// batch), its time is the longest request's walk over all its keys.  Then
// the keys are cut into partitions of kSplitTokens; one wave per (kv-head,
// query tile, partition, request) leaves a partial (normalised o, running
// maximum m, sum l) per query row, and a merge kernel combines a row's
// partials by the log-sum-exp rule.  A column with no visible key in a
// partition leaves m = -inf, l = 0: weight 0 in the merge.

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "pa.h"
#include "pa_decode_common.h"

namespace pa {

template <bool BF16, int D>
__device__ __forceinline__ void store_row(void* __restrict__ out_, int64_t row, const f32x4 (&acc)[D / 16], float inv,
                                          int j) {
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
        const int d0 = 16 * c + 4 * j;
        if constexpr (BF16) {
            uint2 w;
            w.x = pack_bf16x2(acc[c][0] * inv, acc[c][1] * inv);
            w.y = pack_bf16x2(acc[c][2] * inv, acc[c][3] * inv);
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out_) + row * D + d0) = w;
        } else {
            *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out_) + row * D + d0) = acc[c] * inv;
        }
    }
}

// Key partitions (see above): rows x P partials (o: D floats, (m, l)).
struct KeySplit {
    int PS;  // tokens per partition; 0: no split
    int P;   // partitions per row (grid y = query tiles x P)
    float* o;
    float* ml;
};

template <bool BF16, int D, int BS, int NCT>
__global__ __launch_bounds__(64) void prefill_kernel(const void* __restrict__ q_, const void* __restrict__ kc_,
                                                     const void* __restrict__ vc_, const int32_t* __restrict__ tables,
                                                     const int32_t* __restrict__ lens,
                                                     const int32_t* __restrict__ q_start, void* __restrict__ out_,
                                                     int T, int Hq, int Hkv, int G, int QT, int max_q,
                                                     int max_blocks, int num_blocks, float scale_log2, KeySplit ks) {
    using C = DecodeCfg<BF16, D, BS>;
    const int g = blockIdx.x;
    const int qt = blockIdx.y / ks.P;
    const int p = blockIdx.y % ks.P;
    const int b = blockIdx.z;
    const int lane = threadIdx.x;
    const int n = lane & 15;
    const int j = lane >> 4;
    const int t0 = q_start[b];
    const int t1 = q_start[b + 1];
    if (t0 < 0 || t1 > T || t1 < t0) return;  // malformed query offsets: the request writes nothing
    const int M = t1 - t0;
    const int L = lens[b];
    if (M > max_q || M > L || (int64_t)L > (int64_t)max_blocks * BS) {
        // more query tokens than the launch bound or than cached tokens, or a
        // length the table cannot hold: tile 0 writes NaN in all the request's rows
        if (qt != 0 || p != 0) return;
        for (int64_t i = lane; i < (int64_t)M * G * D; i += 64) {
            const int c = (int)(i / D);
            const int64_t row = (int64_t)(t0 + c / G) * Hq + g * G + c % G;
            if constexpr (BF16)
                reinterpret_cast<uint16_t*>(out_)[row * D + i % D] = (uint16_t)bf16_bits_rne(__builtin_nanf(""));
            else
                reinterpret_cast<float*>(out_)[row * D + i % D] = __builtin_nanf("");
        }
        return;
    }
    const int q0 = qt * QT;
    if (q0 >= M) return;
    const int nq = min(QT, M - q0);  // query tokens of this tile
    const int ncol = nq * G;
    const int pos0 = L - M + q0;  // position of the tile's first query token
    const int Lend = pos0 + nq;   // keys the tile needs: [0, Lend)
    const int kstart = p * ks.PS; // this wave's keys: [kstart, kend)
    if (kstart >= Lend) return;
    const int kend = ks.PS ? min(kstart + ks.PS, Lend) : Lend;

    typename C::QRegs qr[NCT];
    int Lcol[NCT];
#pragma unroll
    for (int t = 0; t < NCT; ++t) {
        const int c = min(16 * t + n, ncol - 1);  // padding columns repeat the last one and are never stored
        const char* qp = reinterpret_cast<const char*>(q_) + ((int64_t)(t0 + q0 + c / G) * Hq + g * G + c % G) * D * C::ES;
#pragma unroll
        for (int k = 0; k < C::NKC; ++k) qr[t][k] = ld16(qp + (int64_t)(4 * k + j) * 16);
        Lcol[t] = min(pos0 + c / G + 1, kend);
    }
    RunState<BF16, D, BS> S[NCT];
#pragma unroll
    for (int t = 0; t < NCT; ++t) run_init(S[t]);

    const int64_t blk_bytes = (int64_t)Hkv * C::TILE * C::ES;
    const char* kbase = reinterpret_cast<const char*>(kc_) + (int64_t)g * C::TILE * C::ES;
    const char* vbase = reinterpret_cast<const char*>(vc_) + (int64_t)g * C::TILE * C::ES;
    const int32_t* trow = tables + (int64_t)b * max_blocks;
    bool bad = false;
    for (int ctok = kstart; ctok < kend; ctok += kTableChunk * BS) {
        const int cend = min(ctok + kTableChunk * BS, kend);
        const int blk0 = ctok / BS;
        const int nblk = (cend - 1) / BS - blk0 + 1;
        const int32_t ent = (lane < nblk) ? trow[blk0 + lane] : 0;
        if (__any(lane < nblk && (ent < 0 || ent >= num_blocks))) {
            bad = true;
            break;
        }
        const int nst = (cend - ctok + C::STEP - 1) / C::STEP;
        StepRegs<BF16, D, BS> cur;
        issue_step<BF16, D, BS>(cur, kbase, vbase, blk_bytes, ent, blk0, nblk, ctok, kend, n, j);
        int tok0 = ctok;
        for (int st = 0; st + 1 < nst; ++st, tok0 += C::STEP) {
            StepRegs<BF16, D, BS> nxt;
            issue_step<BF16, D, BS>(nxt, kbase, vbase, blk_bytes, ent, blk0, nblk, tok0 + C::STEP, kend, n, j);
            __builtin_amdgcn_sched_barrier(0);  // loads stay ahead of the compute
#pragma unroll
            for (int t = 0; t < NCT; ++t)
                compute_step<BF16, D, BS, true>(cur, qr[t], S[t].m, S[t].l, S[t].acc, tok0, kend, j, scale_log2,
                                                Lcol[t], min(pos0 + (16 * t) / G + 1, kend));
            cur = nxt;
        }
#pragma unroll
        for (int t = 0; t < NCT; ++t)
            compute_step<BF16, D, BS, true>(cur, qr[t], S[t].m, S[t].l, S[t].acc, tok0, kend, j, scale_log2,
                                            Lcol[t], min(pos0 + (16 * t) / G + 1, kend));
    }
    if (ks.PS == 0 || Lend <= ks.PS) {
        // no split, or the tile's keys fit partition 0 (p = 0 here): the rows
        // themselves, which the merge leaves alone
#pragma unroll
        for (int t = 0; t < NCT; ++t) {
            const int c = 16 * t + n;
            if (c < ncol) {
                const int64_t row = (int64_t)(t0 + q0 + c / G) * Hq + g * G + c % G;
                store_row<BF16, D>(out_, row, S[t].acc, bad ? __builtin_nanf("") : 1.0f / S[t].l, j);
            }
        }
        return;
    }
    // key partitions: the partial of each row
#pragma unroll
    for (int t = 0; t < NCT; ++t) {
        const int c = 16 * t + n;
        if (c < ncol) {
            const int64_t row = (int64_t)(t0 + q0 + c / G) * Hq + g * G + c % G;
            const int64_t slot = row * ks.P + p;
            const bool seen = S[t].l > 0.0f;  // a visible key in this partition
            const float inv = bad ? __builtin_nanf("") : (seen ? 1.0f / S[t].l : 0.0f);
#pragma unroll
            for (int cc = 0; cc < C::NV; ++cc)
                *reinterpret_cast<f32x4*>(ks.o + slot * D + 16 * cc + 4 * j) = S[t].acc[cc] * inv;
            if (j == 0) {
                ks.ml[2 * slot] = bad ? 0.0f : (seen ? S[t].m : -INFINITY);
                ks.ml[2 * slot + 1] = bad ? 1.0f : S[t].l;
            }
        }
    }
}

// The merge, on the tile kernel's grid (kv-head, query tile, request) with
// 16 waves per workgroup, one query row per wave at a time: the same checks
// as the tile kernel decide which tiles it wrote partials for (error rows are
// its NaN rows, and a tile whose keys fit one partition its finished rows,
// both left alone here) and over how many partitions.
template <bool BF16, int D>
__global__ __launch_bounds__(1024) void prefill_merge_kernel(const float* __restrict__ part_o,
                                                            const float* __restrict__ part_ml,
                                                            const int32_t* __restrict__ lens,
                                                            const int32_t* __restrict__ q_start,
                                                            void* __restrict__ out_, int T, int Hq, int G, int QT,
                                                            int max_q, int max_blocks, int BS, int PS, int P) {
    constexpr int PER = D / 64;
    const int g = blockIdx.x;
    const int qt = blockIdx.y;
    const int b = blockIdx.z;
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int t0 = q_start[b];
    const int t1 = q_start[b + 1];
    if (t0 < 0 || t1 > T || t1 < t0) return;
    const int M = t1 - t0;
    const int L = lens[b];
    if (M > max_q || M > L || (int64_t)L > (int64_t)max_blocks * BS) return;
    const int q0 = qt * QT;
    if (q0 >= M) return;
    const int nq = min(QT, M - q0);
    const int Lend = L - M + q0 + nq;
    const int np = (Lend + PS - 1) / PS;  // partitions the tile's waves wrote
    if (np < 2) return;
    for (int c = wv; c < nq * G; c += 16) {
        const int64_t row = (int64_t)(t0 + q0 + c / G) * Hq + g * G + c % G;
        const float* ml = part_ml + row * P * 2;
        const float* po = part_o + row * P * D + lane * PER;
        float Mx = -INFINITY;
        for (int i = 0; i < np; ++i) Mx = fmaxf(Mx, ml[2 * i]);
        float num[PER];
#pragma unroll
        for (int e = 0; e < PER; ++e) num[e] = 0.0f;
        float den = 0.0f;
        for (int i = 0; i < np; ++i) {
            const float w = ml[2 * i + 1] * __builtin_amdgcn_exp2f(ml[2 * i] - Mx);  // m = -inf: weight 0
            den += w;
#pragma unroll
            for (int e = 0; e < PER; ++e) num[e] += w * po[(int64_t)i * D + e];
        }
        const float inv = 1.0f / den;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const int d = lane * PER + e;
            if constexpr (BF16)
                reinterpret_cast<uint16_t*>(out_)[row * D + d] = (uint16_t)bf16_bits_rne(num[e] * inv);
            else
                reinterpret_cast<float*>(out_)[row * D + d] = num[e] * inv;
        }
    }
}

// ---------------------------------------------------------------------------- workgroup tiles (bfloat16)
//
// Long chunks.  A workgroup of NW waves takes NW consecutive wave tiles of
// query tokens of one (kv-head, request): each wave holds NCT 16-column
// matrix-core tiles of (token, head) columns, as in prefill_kernel, and the
// workgroup walks the keys once for all of them, up to its last token's
// position.  Every 32-token step of keys and values is copied from the pool
// into a four-slot LDS ring by direct global-to-LDS loads (no staging
// registers), each wave moving its own 1 KiB pieces, four steps ahead of
// the step whose slot they refill; the waves read their operands from the
// ring in the order prefill_kernel reads them from the pool.  One barrier
// per step makes the step two ahead visible and frees the slot just read.
// A step's keys and values are read from the pool once per workgroup
// instead of once per wave, and two workgroups fit a CU (two waves per
// SIMD, at most 256 registers each), so one wave's softmax work overlaps
// the other's matrix-core work.

// Largest batch whose workgroups are dispatched longest request first (at
// most one request per lane of a workgroup).
constexpr int kFlashOrderMax = 256;

// s_waitcnt immediate (gfx9 encoding) that waits for at most n outstanding
// vector-memory loads and leaves the export and LDS/scalar counters alone.
constexpr int vmcnt_only(int n) { return (n & 0xf) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8); }

// Workgroup barrier of the LDS ring: this wave's direct loads but the last
// IN_FLIGHT have landed, then every wave meets.  A __syncthreads() would
// add a workgroup release fence, which waits for every direct load still
// landing (they count as LDS stores); the compiler fences here only keep
// the compiler from moving memory accesses across the barrier.
template <int IN_FLIGHT>
__device__ __forceinline__ void ring_barrier() {
    __builtin_amdgcn_s_waitcnt(vmcnt_only(IN_FLIGHT));
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <int D, int BS, int NW>
struct FlashCfg {
    static constexpr int NSLOT = 4;          // ring slots: two steps resident, two in flight
    static constexpr int TILE = D * BS * 2;  // bytes of one (block, head) tile
    static constexpr int PAD = 128;          // LDS gap after each tile (the two tiles a lane group reads differ in bank)
    static constexpr int TSTRIDE = TILE + PAD;
    static constexpr int NE = 32 / BS;       // blocks of one step
    static constexpr int SLOT = NE * TSTRIDE;  // LDS bytes of a step's keys (or values)
    static constexpr int NLD = 32 * D * 2 / (1024 * NW);  // 16-byte pieces per lane of a step's keys
    static_assert(NLD >= 1 && NLD * 1024 * NW == 32 * D * 2 && TILE % 1024 == 0,
                  "the waves' pieces cover a step, and one wave's piece lies in one tile");
    // piece i of wave w: bytes [1024 (w + NW i), +1024) of the step's keys
    // (values), in tile blk(w, i) of the step
    __device__ static int blk(int w, int i) { return 1024 * (w + NW * i) / TILE; }
    __device__ static int inner(int w, int i) { return 1024 * (w + NW * i) - blk(w, i) * TILE; }
};

// LDS byte offsets (within a slot's key or value region) of a lane's
// operands, the same for every step: step token s of the slot is token
// s % BS of the slot's tile s / BS, and the placement is issue_step_e's.
// No token is clamped: every slot is written in full, every read stays in
// its slot, and tokens past the keys are masked by the step compute (scores
// -inf, values zeroed bitwise).
template <int D, int BS, int TSTRIDE>
struct FlashOffsets {
    using C = DecodeCfg<true, D, BS>;
    int k[C::NT];  // key tile t: + (4 c) BS 16 for chunk group c
    int va, vb;    // values: + d BS 2 for head-dim row d (vb: second 8-byte half, blocks of 8)
    __device__ void init(int n, int j) {
#pragma unroll
        for (int t = 0; t < C::NT; ++t) {
            const int srow = C::VIL ? 16 * (n >> 3) + 8 * t + (n & 7) : 16 * t + n;
            k[t] = (srow / BS) * TSTRIDE + (srow % BS) * 16 + j * BS * 16;
        }
        if constexpr (C::VIL) {
            va = (8 * j / BS) * TSTRIDE + (8 * j % BS) * 2 + n * BS * 2;
            vb = 0;
        } else {
            va = (4 * j / BS) * TSTRIDE + (4 * j % BS) * 2 + n * BS * 2;
            vb = ((16 + 4 * j) / BS) * TSTRIDE + ((16 + 4 * j) % BS) * 2 + n * BS * 2;
        }
    }
};

// A step's keys (both 16-token tiles) and values from a ring slot, in the
// matrix-core operand order.
template <int D, int BS, int TSTRIDE>
__device__ __forceinline__ void flash_read_keys(u32x4 (&k)[2][D / 32], const char* sk,
                                                const FlashOffsets<D, BS, TSTRIDE>& o) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int c = 0; c < D / 32; ++c) k[t][c] = *reinterpret_cast<const u32x4*>(sk + o.k[t] + 4 * c * BS * 16);
}

template <int D, int BS, int TSTRIDE>
__device__ __forceinline__ void flash_read_values(u32x4 (&v)[D / 16], const char* sv,
                                                  const FlashOffsets<D, BS, TSTRIDE>& o) {
    using C = DecodeCfg<true, D, BS>;
    if constexpr (C::VIL) {
#pragma unroll
        for (int c = 0; c < C::NV; ++c) v[c] = *reinterpret_cast<const u32x4*>(sv + o.va + 16 * c * BS * 2);
    } else {
#pragma unroll
        for (int c = 0; c < C::NV; ++c) {
            const u32x2 lo = *reinterpret_cast<const u32x2*>(sv + o.va + 16 * c * BS * 2);
            const u32x2 hi = *reinterpret_cast<const u32x2*>(sv + o.vb + 16 * c * BS * 2);
            v[c] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
    }
}

// Maximum of non-NaN floats as one v_max_f32 / v_max3_f32 (the compiler's
// fmaxf would canonicalise each operand first).  Vector ALU only.
__device__ __forceinline__ float vmax(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
__device__ __forceinline__ float vmax3(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// Step token held in element e (scores and value operand) of lane group j.
template <int BS>
__device__ __forceinline__ int flash_tok(int tok0, int j, int e) {
    return BS >= 16 ? tok0 + 16 * (j >> 1) + 4 * (j & 1) + (e & 3) + 8 * (e >> 2)
                    : tok0 + 4 * j + (e & 3) + 16 * (e >> 2);
}

// Scores of one 16-column tile for a step's 32 keys (unscaled): sa for the
// keys of tile 0, sb for tile 1, lane (n, j) holding rows 4 j .. 4 j + 3.
template <int D>
__device__ __forceinline__ void flash_scores(f32x4& sa, f32x4& sb, const u32x4 (&k)[2][D / 32],
                                             const u32x4 (&q)[D / 32]) {
    sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k[0][0]), __builtin_bit_cast(bf16x8, q[0]),
                                                 f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k[1][0]), __builtin_bit_cast(bf16x8, q[0]),
                                                 f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
    for (int c = 1; c < D / 32; ++c) {
        const bf16x8 qv = __builtin_bit_cast(bf16x8, q[c]);
        sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k[0][c]), qv, sa, 0, 0, 0);
        sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k[1][c]), qv, sb, 0, 0, 0);
    }
}

// Online-softmax state of one tile for the workgroup kernel: the running
// reference m (base 2, scaled), the lane's share of the softmax sum (its
// own keys' probabilities; the column's total is the sum over its four
// lanes, taken once at the end: a rescale multiplies every share by the
// same factor), the accumulators, and two values cached from m: thr, the
// unscaled score above which a probability could exceed 2^kLazyRescale
// (thr = (m + kLazyRescale) / scale_log2), and negm = -m (0 while m = -inf).
template <int D>
struct FlashState {
    float m, l, thr, negm;
    f32x4 acc[D / 16];
};

template <int D>
__device__ __forceinline__ void flash_state_init(FlashState<D>& S) {
    S.m = -INFINITY;
    S.l = 0.0f;
    S.thr = -INFINITY;
    S.negm = 0.0f;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) S.acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// Online-softmax update and PV of all NCT tiles of a wave from their step
// scores (already masked: -inf past each column's limit): the method of
// compute_step (base 2, lazy rescale), with the scale folded into the
// exponent argument (scale_log2 > 0).  The references move only when some
// lane of some tile holds a score above its column's cached threshold (one
// ballot per step for all tiles), so most steps take no cross-lane maximum
// and no cross-lane sum; when one does, every tile moves its reference to
// its running maximum (a move that lazy rescaling would have skipped is
// still exact: the reference only has to keep the scores seen so far at
// most kLazyRescale above it).  v: the step's values, already zeroed at or
// past the keys' end.
template <int D, int NCT>
__device__ __forceinline__ void flash_softmax_pv_all(FlashState<D> (&S)[NCT], const float (&s)[NCT][8],
                                                     const u32x4 (&v)[D / 16], float sl2) {
    float lm[NCT];
    bool up = false;
#pragma unroll
    for (int t = 0; t < NCT; ++t) {
        lm[t] = vmax3(vmax3(s[t][0], s[t][1], s[t][2]), vmax3(s[t][3], s[t][4], s[t][5]), vmax(s[t][6], s[t][7]));
        up = up || lm[t] > S[t].thr;
    }
    if (__builtin_amdgcn_ballot_w64(up)) {
#pragma unroll
        for (int t = 0; t < NCT; ++t) {
            const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(lm[t]), __float_as_uint(lm[t]), false, false);
            float mx = vmax(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
            const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
            mx = vmax(__uint_as_float(r32[0]), __uint_as_float(r32[1])) * sl2;
            const float m_new = vmax(S[t].m, mx);
            const float alpha = m_new == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(S[t].m - m_new);
            S[t].l *= alpha;
#pragma unroll
            for (int c = 0; c < D / 16; ++c) S[t].acc[c] *= alpha;
            S[t].m = m_new;
            S[t].thr = (m_new + kLazyRescale) / sl2;
            S[t].negm = m_new == -INFINITY ? 0.0f : -m_new;
        }
    }
#pragma unroll
    for (int t = 0; t < NCT; ++t) {
        float pe[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pe[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][e], sl2, S[t].negm));
        S[t].l += ((pe[0] + pe[1]) + (pe[2] + pe[3])) + ((pe[4] + pe[5]) + (pe[6] + pe[7]));
        const u32x4 pw = {pack_bf16x2(pe[0], pe[1]), pack_bf16x2(pe[2], pe[3]), pack_bf16x2(pe[4], pe[5]),
                          pack_bf16x2(pe[6], pe[7])};
        const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
        for (int c = 0; c < D / 16; ++c)
            S[t].acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v[c]), pb, S[t].acc[c], 0, 0, 0);
    }
}

template <int D, int BS, int NW, int NCT>
struct FlashWave {
    using C = DecodeCfg<true, D, BS>;
    using F = FlashCfg<D, BS, NW>;
    // the ring: NSLOT slots of [keys SLOT | values SLOT], each its own LDS
    // array, so the compiler can tell a slot's reads from the direct loads
    // still landing in the other slots and does not wait for those
    char* r0;
    char* r1;
    char* r2;
    char* r3;
    const char* kbase;
    const char* vbase;
    const int32_t* trow;
    uint32_t blk_bytes;  // bytes of one block (all kv-heads) in a pool
    FlashOffsets<D, BS, F::TSTRIDE> off;
    int num_blocks, lastb, nst, kend, w, lane, n, j;
    float sl2;
    int bad;  // a table entry outside the pool was met (wave-uniform)
    int Lcol[NCT], Lmin[NCT];
    int toff[8];  // step token of each score element, less the step's first token
    u32x4 qr[NCT][C::NKC];
    FlashState<D> S[NCT];

    template <int SL>
    __device__ __forceinline__ char* slot_keys() {
        static_assert(F::NSLOT == 4 && SL >= 0 && SL < 4, "four ring slots");
        return SL == 0 ? r0 : SL == 1 ? r1 : SL == 2 ? r2 : r3;
    }

    // Table entry of this wave's piece i of step y (wave-uniform: a scalar
    // load; steps past the keys repeat the last block).
    __device__ __forceinline__ int32_t entry(int y, int i) { return trow[min(y * 32 / BS + F::blk(w, i), lastb)]; }

    // Copy this wave's pieces of step y (entries e[]) from the pool into its
    // ring slot, straight into LDS (no registers): each instruction moves
    // 1 KiB, 16 bytes per lane at consecutive addresses on both sides.
    template <int SL>
    __device__ __forceinline__ void issue(const int32_t (&e)[F::NLD]) {
        char* sk = slot_keys<SL>();
        const uint32_t lane_off = 16u * (uint32_t)lane;
#pragma unroll
        for (int i = 0; i < F::NLD; ++i) {
            const bool ok = e[i] >= 0 && e[i] < num_blocks;
            bad |= ok ? 0 : 1;  // scalar: e[i] comes from a scalar load
            // wave-uniform piece base (scalar registers) + the lane's 16 bytes
            const uint64_t o = (uint64_t)(uint32_t)(ok ? e[i] : 0) * blk_bytes + (uint32_t)F::inner(w, i);
            const int lo = F::blk(w, i) * F::TSTRIDE + F::inner(w, i);
            __builtin_amdgcn_global_load_lds((kbase + o) + lane_off,
                                             (__attribute__((address_space(3))) void*)(sk + lo), 16, 0, 0);
            __builtin_amdgcn_global_load_lds((vbase + o) + lane_off,
                                             (__attribute__((address_space(3))) void*)(sk + F::SLOT + lo), 16, 0, 0);
        }
    }

    // Iteration x: step x + 1's scores into `nxt` (their matrix-core work
    // runs while this step's softmax goes on), step x's softmax and PV from
    // `cur`, then the ring turn: wait for step x + 2's pieces, one barrier
    // (step x + 2 visible to every wave, slot x free), step x + 4's pieces
    // into slot x.  Memory operations are the same on every path (past the
    // keys the entries repeat the last block), so each wait leaves the later
    // step's loads in flight.
    // (x is in slot SL = x % 4)
    template <int SL>
    __device__ __forceinline__ void iter(int x, f32x4 (&cur)[NCT][2], f32x4 (&nxt)[NCT][2]) {
        int32_t e[F::NLD];
#pragma unroll
        for (int i = 0; i < F::NLD; ++i) e[i] = entry(x + 4, i);
        u32x4 k[2][C::NKC];
        flash_read_keys<D, BS, F::TSTRIDE>(k, slot_keys<(SL + 1) % 4>(), off);
#pragma unroll
        for (int t = 0; t < NCT; ++t) flash_scores<D>(nxt[t][0], nxt[t][1], k, qr[t]);
        if (x < nst) {
            u32x4 v[C::NV];
            flash_read_values<D, BS, F::TSTRIDE>(v, slot_keys<SL>() + F::SLOT, off);
            const int tok0 = 32 * x;
            float sc[NCT][8];
#pragma unroll
            for (int t = 0; t < NCT; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    sc[t][e] = cur[t][0][e];
                    sc[t][4 + e] = cur[t][1][e];
                }
            // One scalar test for every tail: Lmin[0] is the smallest key limit
            // of the wave's columns and kend bounds them all, so a step with no
            // limit inside it needs no mask and no value zeroing.  Masking a
            // tile whose limits all lie past the step changes nothing.
            if (tok0 + 32 > Lmin[0]) {
                if (tok0 + 32 > kend) {  // the last step: values at or past the keys' end may be anything
                    const int vl = kend - tok0;
                    uint32_t keep[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        keep[q] = (toff[2 * q] < vl ? 0x0000ffffu : 0u) | (toff[2 * q + 1] < vl ? 0xffff0000u : 0u);
#pragma unroll
                    for (int c = 0; c < C::NV; ++c)
                        v[c] = u32x4{v[c][0] & keep[0], v[c][1] & keep[1], v[c][2] & keep[2], v[c][3] & keep[3]};
                }
#pragma unroll
                for (int t = 0; t < NCT; ++t) {
                    const int lim = Lcol[t] - tok0;
#pragma unroll
                    for (int e = 0; e < 8; ++e) sc[t][e] = toff[e] < lim ? sc[t][e] : -INFINITY;
                }
            }
            flash_softmax_pv_all<D, NCT>(S, sc, v, sl2);
        }
        // step x + 2's pieces have landed once at most step x + 3's (2 NLD
        // loads) are outstanding; the barrier makes every wave's visible and
        // tells every wave that slot x (read above, its values consumed by the
        // PV products, and one iteration ago) is free
        ring_barrier<2 * F::NLD>();
        issue<SL>(e);
    }
};

template <int D, int BS, int NW, int NCT, int WPE>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(WPE)))
void prefill_flash_kernel(const void* __restrict__ q_, const void* __restrict__ kc_, const void* __restrict__ vc_,
                          const int32_t* __restrict__ tables, const int32_t* __restrict__ lens,
                          const int32_t* __restrict__ q_start, void* __restrict__ out_, int T, int Hq, int Hkv,
                          int G, int QTw, int max_q, int max_blocks, int num_blocks, float scale_log2) {
    using C = DecodeCfg<true, D, BS>;
    using F = FlashCfg<D, BS, NW>;
    using W_t = FlashWave<D, BS, NW, NCT>;
    __shared__ __attribute__((aligned(16))) char ring0[2 * F::SLOT];
    __shared__ __attribute__((aligned(16))) char ring1[2 * F::SLOT];
    __shared__ __attribute__((aligned(16))) char ring2[2 * F::SLOT];
    __shared__ __attribute__((aligned(16))) char ring3[2 * F::SLOT];
    __shared__ int s_bad;
    __shared__ int s_len[kFlashOrderMax];
    __shared__ int s_req, s_t0, s_t1;
    const int g = blockIdx.x;
    const int qt = blockIdx.y;
    const int tid = threadIdx.x;
    // Longest requests first: a workgroup walks its request's keys, so with
    // more workgroups than the CUs hold at once, a long request dispatched
    // last sets the end.  Workgroups are dispatched in index order, so
    // blockIdx.z is taken as a rank in length order (longest first, ties in
    // index order) for batches of up to kFlashOrderMax requests; each
    // workgroup finds the request of its rank (a strict order: exactly one
    // request has it).  Larger batches keep the index order.
    static_assert(kFlashOrderMax <= 64 * NW, "one request per lane");
    int b = blockIdx.z;
    int t0, t1, L;
    const int B = (int)gridDim.z;
    if (B <= kFlashOrderMax) {
        // one round trip: every request's length and query offsets at once
        int my_t0 = 0, my_t1 = 0;
        if (tid < B) {
            s_len[tid] = lens[tid];
            my_t0 = q_start[tid];
            my_t1 = q_start[tid + 1];
        }
        __syncthreads();
        if (tid < B) {
            const int lt = s_len[tid];
            int rank = 0;
            for (int u = 0; u < B; ++u) {
                const int lu = s_len[u];
                rank += (lu > lt || (lu == lt && u < tid)) ? 1 : 0;
            }
            if (rank == b) {
                s_req = tid;
                s_t0 = my_t0;
                s_t1 = my_t1;
            }
        }
        __syncthreads();
        // wave-uniform (the same LDS words for every lane): the table row and
        // the entry loads stay scalar
        b = __builtin_amdgcn_readfirstlane(s_req);
        t0 = __builtin_amdgcn_readfirstlane(s_t0);
        t1 = __builtin_amdgcn_readfirstlane(s_t1);
        L = __builtin_amdgcn_readfirstlane(s_len[b]);
    } else {
        t0 = q_start[b];
        t1 = q_start[b + 1];
        L = lens[b];
    }
    if (t0 < 0 || t1 > T || t1 < t0) return;  // malformed query offsets: the request writes nothing
    const int M = t1 - t0;
    if (M > max_q || M > L || (int64_t)L > (int64_t)max_blocks * BS) {
        // as prefill_kernel: the first tile writes NaN in all the request's rows
        if (qt != 0) return;
        for (int64_t i = tid; i < (int64_t)M * G * D; i += 64 * NW) {
            const int c = (int)(i / D);
            const int64_t row = (int64_t)(t0 + c / G) * Hq + g * G + c % G;
            reinterpret_cast<uint16_t*>(out_)[row * D + i % D] = (uint16_t)bf16_bits_rne(__builtin_nanf(""));
        }
        return;
    }
    const int QTW = QTw * NW;  // query tokens of the workgroup
    const int q0 = qt * QTW;
    if (q0 >= M) return;
    const int kend = L - M + q0 + min(QTW, M - q0);  // keys of the workgroup: [0, kend)

    W_t W;
    W.r0 = ring0;
    W.r1 = ring1;
    W.r2 = ring2;
    W.r3 = ring3;
    W.w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: entry loads and piece bases go scalar
    W.lane = tid & 63;
    W.n = W.lane & 15;
    W.j = W.lane >> 4;
    W.blk_bytes = (uint32_t)Hkv * C::TILE * C::ES;
    W.off.init(W.n, W.j);
#pragma unroll
    for (int e = 0; e < 8; ++e) W.toff[e] = flash_tok<BS>(0, W.j, e);
    W.kbase = reinterpret_cast<const char*>(kc_) + (int64_t)g * C::TILE * C::ES;
    W.vbase = reinterpret_cast<const char*>(vc_) + (int64_t)g * C::TILE * C::ES;
    W.trow = tables + (int64_t)b * max_blocks;
    W.num_blocks = num_blocks;
    W.kend = kend;
    W.lastb = (kend - 1) / BS;
    W.nst = (kend + 31) / 32;
    W.sl2 = scale_log2;
    W.bad = 0;
    if (tid == 0) s_bad = 0;

    // this wave's query tokens and columns (padding columns repeat the last
    // real one; a wave past the request's tokens computes column 0's and
    // stores nothing)
    const int qw = q0 + W.w * QTw;                 // first query token of the wave
    const int nqw = max(0, min(QTw, M - qw));      // its tokens
    const int ncol = nqw * G;
    const int pos0 = L - M + qw;
#pragma unroll
    for (int t = 0; t < NCT; ++t) {
        const int c = max(0, min(16 * t + W.n, ncol - 1));
        const int tok = nqw > 0 ? qw + c / G : q0;
        const int head = nqw > 0 ? c % G : 0;
        const char* qp = reinterpret_cast<const char*>(q_) + ((int64_t)(t0 + tok) * Hq + g * G + head) * D * 2;
#pragma unroll
        for (int k = 0; k < C::NKC; ++k) W.qr[t][k] = ld16(qp + (int64_t)(4 * k + W.j) * 16);
        W.Lcol[t] = min(L - M + tok + 1, kend);
        // smallest key limit of the tile's columns, wave-uniform so the tail
        // test is a scalar branch (a wave past the request's tokens: every
        // step is a tail, each lane masked by its own limit)
        W.Lmin[t] = __builtin_amdgcn_readfirstlane(nqw > 0 ? min(pos0 + (16 * t) / G + 1, kend) : 0);
        flash_state_init(W.S[t]);
    }

    // prologue: steps 0 .. 3 into slots 0 .. 3; wait for 0 and 1 (2 and 3
    // stay in flight); step 0's scores
    {
        int32_t e[F::NSLOT][F::NLD];
#pragma unroll
        for (int y = 0; y < F::NSLOT; ++y)
#pragma unroll
            for (int i = 0; i < F::NLD; ++i) e[y][i] = W.entry(y, i);
        W.template issue<0>(e[0]);
        W.template issue<1>(e[1]);
        W.template issue<2>(e[2]);
        W.template issue<3>(e[3]);
    }
    ring_barrier<2 * 2 * F::NLD>();
    f32x4 SA[NCT][2], SB[NCT][2];
    {
        u32x4 k[2][C::NKC];
        flash_read_keys<D, BS, F::TSTRIDE>(k, W.template slot_keys<0>(), W.off);
#pragma unroll
        for (int t = 0; t < NCT; ++t) flash_scores<D>(SA[t][0], SA[t][1], k, W.qr[t]);
    }
    // steps in fours (one per ring slot; the score buffers swap roles
    // without a copy); the last round's iterations past the keys only keep
    // the ring turning in step
    const int nst = W.nst;
    for (int x = 0; x < nst; x += 4) {
        W.template iter<0>(x, SA, SB);
        W.template iter<1>(x + 1, SB, SA);
        W.template iter<2>(x + 2, SA, SB);
        W.template iter<3>(x + 3, SB, SA);
    }
    // every wave's outstanding ring loads land before the workgroup ends
    __builtin_amdgcn_s_waitcnt(vmcnt_only(0));

    if (W.bad) s_bad = 1;
    __syncthreads();
    const bool bad = s_bad != 0;
#pragma unroll
    for (int t = 0; t < NCT; ++t) {
        const float l = wave_sum16(W.S[t].l);  // the column's sum over its four lanes
        const int c = 16 * t + W.n;
        if (c < ncol) {
            const int64_t row = (int64_t)(t0 + qw + c / G) * Hq + g * G + c % G;
            store_row<true, D>(out_, row, W.S[t].acc, bad ? __builtin_nanf("") : 1.0f / l, W.j);
        }
    }
}

}  // namespace pa

// ---------------------------------------------------------------------------- host side

// The balanced split of the decode (pa_decode.hip) serves multi-token
// queries whose M * G columns fit one wave (up to 16).
namespace pa_internal {
size_t multi_balanced_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t max_query_len);
pa_status multi_balanced_launch(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                                const int32_t* seq_lens, const int32_t* query_start, int32_t num_kv_heads, float scale,
                                void* out, void* stream, int32_t num_seqs, int32_t num_query_tokens,
                                int32_t num_q_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                int32_t max_blocks_per_seq, pa_dtype dtype, void* workspace);
}  // namespace pa_internal

namespace {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Query columns one wave holds: four 16-column tiles, two for float32 with
// head dim 128 (four would not fit the register file).
constexpr int max_columns(bool bf16, int head_dim) { return (!bf16 && head_dim == 128) ? 32 : 64; }

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Key partitions (prefill_kernel): used when the query-tile launch would hold
// fewer than kSplitWaves waves and the longest table spans two partitions or
// more.  Measured on MI355X (Llama-3-8B-shaped batch, 64 requests of 512 to
// 4,096 tokens, GQA 4): with 8 or 16 new tokens each the tile launch has 512
// waves and its time is the 4,096-token requests' walk over all their keys;
// partitions of 2,048 keys took it from 147 to 117 us (8 new tokens) and from
// 252 to 164 us (16); 512 and 1,024 keys did less well.  From 32 new tokens
// (1,024 waves) on, the partials' traffic costs more than the split saves.
constexpr int kSplitTokens = 2048;
constexpr int64_t kSplitWaves = 1024;
constexpr size_t kSplitMaxBytes = size_t(1) << 30;

struct SplitPlan {
    int P;  // partitions per row (0: no split)
    size_t o_off, ml_off, bytes;
};

// Workspace: [pa_decode's counter region, left untouched | o: rows x P x D |
// (m, l): rows x P x 2], rows = query tokens x query heads.
inline SplitPlan split_plan(int64_t B, int64_t T, int Hq, int Hkv, int D, int G, int maxc, int bs,
                            int64_t max_blocks, int max_q) {
    SplitPlan sp{0, 0, 0, 0};
    const int QT = maxc / G;
    const int64_t waves = (int64_t)Hkv * B * ((max_q + QT - 1) / QT);
    const int64_t P = (max_blocks * bs + kSplitTokens - 1) / kSplitTokens;
    if (waves >= kSplitWaves || P < 2 || T <= 0) return sp;
    const size_t rows = (size_t)T * Hq;
    sp.o_off = pa_decode_counter_bytes();
    sp.ml_off = sp.o_off + align_up(rows * (size_t)P * D * sizeof(float));
    sp.bytes = sp.ml_off + align_up(rows * (size_t)P * 2 * sizeof(float));
    if (sp.bytes > kSplitMaxBytes) return SplitPlan{0, 0, 0, 0};
    sp.P = (int)P;
    return sp;
}

struct PrefillLaunch {
    const void *q, *kc, *vc;
    const int32_t *tables, *lens, *qs;
    void* out;
    int T, B, Hq, Hkv, G, QT, max_q, n_tiles, max_blocks, num_blocks;
    float sl2;
    hipStream_t s;
    pa::KeySplit ks;
};

template <bool BF16, int D, int BS, int NCT>
hipError_t launch_prefill(const PrefillLaunch& a) {
    hipLaunchKernelGGL((pa::prefill_kernel<BF16, D, BS, NCT>),
                       dim3((unsigned)a.Hkv, (unsigned)(a.n_tiles * a.ks.P), (unsigned)a.B), dim3(64), 0, a.s, a.q,
                       a.kc, a.vc, a.tables, a.lens, a.qs, a.out, a.T, a.Hq, a.Hkv, a.G, a.QT, a.max_q, a.max_blocks,
                       a.num_blocks, a.sl2, a.ks);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.ks.PS == 0) return e;
    hipLaunchKernelGGL((pa::prefill_merge_kernel<BF16, D>), dim3((unsigned)a.Hkv, (unsigned)a.n_tiles, (unsigned)a.B),
                       dim3(1024), 0, a.s, a.ks.o, a.ks.ml, a.lens, a.qs, a.out, a.T, a.Hq, a.G, a.QT, a.max_q,
                       a.max_blocks, BS, a.ks.PS, a.ks.P);
    return hipGetLastError();
}

// Workgroup tiles for bfloat16 chunks (prefill_flash_kernel): kFlashCols
// columns per wave, two waves per SIMD (the register budget that allows),
// kFlashWaves waves per workgroup.  Measured on MI355X (512 new tokens per
// request, Llama-3-8B shape): 64 columns at one wave per SIMD and eight
// waves per workgroup were both slower.
constexpr int kFlashCols = 32;
constexpr int kFlashWavesPerSimd = 2;
constexpr int kFlashWaves = 4;

template <int D, int BS>
hipError_t launch_flash(const PrefillLaunch& a) {
    constexpr int NW = kFlashWaves;
    const int QTw = kFlashCols / a.G;
    const int QTW = QTw * NW;
    hipLaunchKernelGGL((pa::prefill_flash_kernel<D, BS, NW, kFlashCols / 16, kFlashWavesPerSimd>),
                       dim3((unsigned)a.Hkv, (unsigned)((a.max_q + QTW - 1) / QTW), (unsigned)a.B), dim3(64 * NW), 0,
                       a.s, a.q, a.kc, a.vc, a.tables, a.lens, a.qs, a.out, a.T, a.Hq, a.Hkv, a.G, QTw, a.max_q,
                       a.max_blocks, a.num_blocks, a.sl2);
    return hipGetLastError();
}

// Blocks of 8 with head dim 128 do not fit two waves per SIMD without
// spilling inside the step loop; that shape keeps the query-tile kernel.
inline bool flash_fits(int D, int BS) { return !(D == 128 && BS == 8); }

template <int D>
hipError_t flash_bs(int BS, const PrefillLaunch& a) {
    switch (BS) {
        case 8:
            if constexpr (D != 128) return launch_flash<D, 8>(a);
            return hipErrorInvalidValue;  // not reached: flash_fits
        case 16: return launch_flash<D, 16>(a);
        default: return launch_flash<D, 32>(a);
    }
}

template <bool BF16, int D, int BS>
hipError_t prefill_cols(int cols, const PrefillLaunch& a) {
    if (cols <= 16) return launch_prefill<BF16, D, BS, 1>(a);
    if (cols <= 32 || max_columns(BF16, D) == 32) return launch_prefill<BF16, D, BS, 2>(a);
    return launch_prefill<BF16, D, BS, max_columns(BF16, D) / 16>(a);
}

template <bool BF16, int D>
hipError_t prefill_bs(int BS, int cols, const PrefillLaunch& a) {
    switch (BS) {
        case 8: return prefill_cols<BF16, D, 8>(cols, a);
        case 16: return prefill_cols<BF16, D, 16>(cols, a);
        default: return prefill_cols<BF16, D, 32>(cols, a);
    }
}

}  // namespace

extern "C" size_t pa_prefill_workspace_bytes(int32_t num_seqs, int32_t num_query_tokens, int32_t num_q_heads,
                                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                             int32_t max_blocks_per_seq, int32_t max_query_len) {
    if (num_seqs <= 0 || num_query_tokens <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
        num_q_heads % num_kv_heads || head_dim <= 0 || block_size <= 0 || max_blocks_per_seq < 0 ||
        max_query_len <= 0)
        return 0;
    const size_t bal =
        pa_internal::multi_balanced_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_query_len);
    if (bal) return bal;
    const int G = num_q_heads / num_kv_heads;
    return split_plan(num_seqs, num_query_tokens, num_q_heads, num_kv_heads, head_dim, G,
                      max_columns(true, head_dim), block_size, max_blocks_per_seq, max_query_len)
        .bytes;
}

extern "C" pa_status pa_prefill(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                                const int32_t* seq_lens, const int32_t* query_start, int32_t num_kv_heads, float scale,
                                void* out, void* stream, int32_t num_seqs, int32_t num_query_tokens,
                                int32_t num_q_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                int32_t max_blocks_per_seq, pa_dtype dtype, int32_t max_query_len, void* workspace,
                                size_t workspace_bytes) {
    if (num_seqs < 0 || num_query_tokens < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks < 0 ||
        max_blocks_per_seq < 0 || max_query_len < 0 || !std::isfinite(scale))
        return PA_ERR_INVALID_ARG;
    if (num_q_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARG;
    if (dtype != PA_F32 && dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
    if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
    if (block_size != 8 && block_size != 16 && block_size != 32) return PA_ERR_UNSUPPORTED;
    const int G = num_q_heads / num_kv_heads;
    const int maxc = max_columns(dtype == PA_BF16, head_dim);
    if (G > 16) return PA_ERR_UNSUPPORTED;
    if (num_seqs > 65535 || num_kv_heads > 65535) return PA_ERR_UNSUPPORTED;
    if ((int64_t)max_blocks_per_seq * block_size > (int64_t)INT32_MAX / 2) return PA_ERR_UNSUPPORTED;
    if (num_seqs == 0 || num_query_tokens == 0 || max_query_len == 0) return PA_OK;
    if (!q || !k_cache || !v_cache || !block_tables || !seq_lens || !query_start || !out) return PA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
        (reinterpret_cast<uintptr_t>(block_tables) & 3u) || (reinterpret_cast<uintptr_t>(seq_lens) & 3u) ||
        (reinterpret_cast<uintptr_t>(query_start) & 3u))
        return PA_ERR_INVALID_ARG;
    // verification-sized chunks: the balanced split (every request's tokens
    // fit one wave's columns) when the caller brings its workspace
    const size_t wneed = pa_internal::multi_balanced_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                                     max_query_len);
    if (wneed && workspace) {
        if (workspace_bytes < wneed || (reinterpret_cast<uintptr_t>(workspace) & 255u)) return PA_ERR_INVALID_ARG;
        return pa_internal::multi_balanced_launch(q, k_cache, v_cache, block_tables, seq_lens, query_start,
                                                  num_kv_heads, scale, out, stream, num_seqs, num_query_tokens,
                                                  num_q_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                                                  dtype, workspace);
    }
    PrefillLaunch a{};
    a.q = q;
    a.kc = k_cache;
    a.vc = v_cache;
    a.tables = block_tables;
    a.lens = seq_lens;
    a.qs = query_start;
    a.out = out;
    a.T = num_query_tokens;
    a.B = num_seqs;
    a.Hq = num_q_heads;
    a.Hkv = num_kv_heads;
    a.G = G;
    a.QT = maxc / G;  // query tokens per wave
    a.max_q = max_query_len;
    const int qt_used = std::min(a.QT, (int)max_query_len);
    a.n_tiles = (max_query_len + a.QT - 1) / a.QT;
    a.max_blocks = max_blocks_per_seq;
    a.num_blocks = num_blocks;
    a.sl2 = (float)((double)scale * 1.4426950408889634);  // scale * log2(e)
    a.s = reinterpret_cast<hipStream_t>(stream);
    // key partitions when the launch is small, with the caller's workspace
    a.ks = pa::KeySplit{0, 1, nullptr, nullptr};
    const SplitPlan sp = split_plan(num_seqs, num_query_tokens, num_q_heads, num_kv_heads, head_dim, G,
                                    max_columns(true, head_dim), block_size, max_blocks_per_seq, max_query_len);
    if (sp.P && workspace) {
        if (workspace_bytes < sp.bytes || (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)))
            return PA_ERR_INVALID_ARG;
        char* w = reinterpret_cast<char*>(workspace);
        a.ks = pa::KeySplit{kSplitTokens, sp.P, reinterpret_cast<float*>(w + sp.o_off),
                            reinterpret_cast<float*>(w + sp.ml_off)};
    }
    if ((int64_t)a.n_tiles * a.ks.P > 65535) return PA_ERR_UNSUPPORTED;
    const int cols = qt_used * G;
    hipError_t e;
    // (the workgroup kernel folds the scale into its exponent argument, which
    // needs a positive scale; other scales take the query tiles)
    if (dtype == PA_BF16 && a.ks.PS == 0 && flash_fits(head_dim, block_size) && a.sl2 > 0.0f &&
        (int64_t)max_query_len * G >= (int64_t)kFlashCols * kFlashWaves) {
        // chunks that fill a workgroup's tiles: workgroup tiles sharing each step through LDS
        e = head_dim == 128 ? flash_bs<128>(block_size, a) : flash_bs<64>(block_size, a);
        return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
    }
    if (dtype == PA_BF16)
        e = head_dim == 128 ? prefill_bs<true, 128>(block_size, cols, a) : prefill_bs<true, 64>(block_size, cols, a);
    else
        e = head_dim == 128 ? prefill_bs<false, 128>(block_size, cols, a) : prefill_bs<false, 64>(block_size, cols, a);
    return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}
