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
// Work decomposition.  A 64-lane wave attends over a run of tokens of one
// (sequence, kv-head) pair for all G query heads of that kv-head.  It walks
// the run in steps of 32 tokens (bf16) or 16 tokens (f32).  Each step loads
// the keys and values of its tokens straight from the pool into registers
// with 16-byte non-temporal loads whose per-lane placement is the
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
// Which runs the waves take:
//  - single pass: one wave per (sequence, kv-head);
//  - fixed partitions: one wave per (kv-head, partition, sequence); each
//    partition leaves (o_j, m_j, l_j) in the workspace and merge_kernel
//    combines them with the log-sum-exp rule
//      M = max_j m_j,  w_j = l_j 2^(m_j - M),  out = sum_j w_j o_j / sum_j w_j
//    (m_j is kept in the base-2 scaled domain, max_p scale*log2(e)*score);
//  - balanced split: a fixed grid of waves, each taking an equal share of
//    all the token steps of the batch (decode_balanced_kernel), with the
//    pieces of a cut (sequence, kv-head) merged by the same rule inside the
//    kernel.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "pa.h"
#include "pa_decode_common.h"

namespace pa {

// ---------------------------------------------------------------------------- fixed partitions

// One wave per (kv-head, partition, sequence).  A sequence that fits one
// partition is written directly; otherwise each partition writes its
// normalised output o_j, maximum m_j and sum l_j for merge_kernel.
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
    const int64_t row0 = (int64_t)b * Hq + g * G;
    if (!len_ok) {
        fill_rows<BF16, D>(out_, row0, G, L <= 0 ? 0.0f : __builtin_nanf(""), lane);
        return;
    }
    const int start = p * PS;
    const int end = min(start + PS, L);
    const int64_t blk_bytes = (int64_t)Hkv * C::TILE * C::ES;
    u32x4 qr[C::NKC];
    load_q<BF16, D, BS>(qr, q_, row0 + n, n, j, G);
    RunState<BF16, D, BS> S;
    run_init(S);
    attend_range<BF16, D, BS>(S, qr, reinterpret_cast<const char*>(kc_) + (int64_t)g * C::TILE * C::ES,
                              reinterpret_cast<const char*>(vc_) + (int64_t)g * C::TILE * C::ES, blk_bytes,
                              tables + (int64_t)b * max_blocks, num_blocks, start, end, L, lane, n, j, scale_log2);
    if (nparts == 1) {
        store_out<BF16, D, BS>(out_, row0, S, n, j, G);
        return;
    }
    if (n >= G) return;
    const float inv = S.bad ? __builtin_nanf("") : 1.0f / S.l;
    const int64_t prow = (row0 + n) * P_max + p;
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

// Log-sum-exp merge of per-partition results: one 256-lane workgroup per
// (query head, sequence).  A lane owns four consecutive head-dim elements of
// one partition row at a time (D / 4 lanes per row, so 1024 / D rows side by
// side) and takes NR rows per loop trip with all their loads issued
// together.  The launch picks NR from the partition bound: 16 when rows can
// have many partitions (a 512-token split of 131,072 tokens at D = 128 in
// two trips; few, long workgroups), 4 or 1 when they have few (many short
// workgroups, which need the smaller register count to share a CU, and
// loads past the last partition would only repeat it).  Each
// row group keeps its own running maximum (rescaling its sums when a trip
// raises it), so no pass over the maxima comes first; the row groups'
// (maximum, sum, weighted output) meet in LDS.
template <int NR, int D>
__device__ __forceinline__ void merge_trips(const float* __restrict__ ml, const float* __restrict__ po, int np,
                                            int rg, int c, int RG, float& m, float& den, f32x4& num) {
    for (int i0 = rg; i0 < np; i0 += NR * RG) {
        float2 w[NR];
        f32x4 o[NR];
#pragma unroll
        for (int u = 0; u < NR; ++u) {
            const int i = min(i0 + u * RG, np - 1);  // past the last partition: a valid row, skipped below
            w[u] = *reinterpret_cast<const float2*>(ml + 2 * i);
            o[u] = *reinterpret_cast<const f32x4*>(po + (int64_t)i * D + 4 * c);
        }
        float tm = -INFINITY;
#pragma unroll
        for (int u = 0; u < NR; ++u)
            if (i0 + u * RG < np) tm = fmaxf(tm, w[u].x);
        const float mn = fmaxf(m, tm);
        const float a = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - mn);
        den *= a;
        num *= a;
        m = mn;
#pragma unroll
        for (int u = 0; u < NR; ++u) {
            if (i0 + u * RG < np) {
                const float wt = w[u].y * __builtin_amdgcn_exp2f(w[u].x - m);
                den += wt;
                num += wt * o[u];
            }
        }
    }
}

template <bool BF16, int D, int NR>
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ part_o,
                                                    const float* __restrict__ part_ml,
                                                    const int32_t* __restrict__ lens, void* __restrict__ out_,
                                                    int Hq, int max_blocks, int BS, int PS, int P_max) {
    constexpr int LPR = D / 4;     // lanes per partition row
    constexpr int RG = 256 / LPR;  // partition rows side by side
    const int h = blockIdx.x;
    const int b = blockIdx.y;
    const int L = lens[b];
    if (L <= 0 || (int64_t)L > (int64_t)max_blocks * BS) return;  // written by the decode kernel
    const int np = (L + PS - 1) / PS;
    if (np <= 1) return;
    const int64_t row = (int64_t)b * Hq + h;
    const float* ml = part_ml + row * P_max * 2;
    const float* po = part_o + row * P_max * D;
    const int t = threadIdx.x;
    const int rg = t / LPR;
    const int c = t % LPR;

    float m = -INFINITY;  // this row group's running maximum
    f32x4 num = {0.f, 0.f, 0.f, 0.f};
    float den = 0.f;
    merge_trips<NR, D>(ml, po, np, rg, c, RG, m, den, num);
    __shared__ f32x4 s_num[RG][LPR];
    __shared__ float s_den[RG], s_m[RG];
    s_num[rg][c] = num;
    if (c == 0) {
        s_den[rg] = den;
        s_m[rg] = m;
    }
    __syncthreads();
    if (t < LPR) {
        float M = s_m[0];
#pragma unroll
        for (int r = 1; r < RG; ++r) M = fmaxf(M, s_m[r]);
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        float total = 0.f;
#pragma unroll
        for (int r = 0; r < RG; ++r) {
            // a row group with no partition (np < RG) has m = -inf and zero sums
            const float f = s_m[r] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(s_m[r] - M);
            v += f * s_num[r][t];
            total += f * s_den[r];
        }
        v = v / total;
        if constexpr (BF16) {
            const uint32_t lo = pack_bf16x2(v[0], v[1]);
            const uint32_t hi = pack_bf16x2(v[2], v[3]);
            *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(out_) + row * D + 4 * t) = u32x2{lo, hi};
        } else {
            *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out_) + row * D + 4 * t) = v;
        }
    }
}

// ---------------------------------------------------------------------------- balanced split

constexpr int kBalancedMaxSeqs = 1024;   // sequences a balanced call may hold
constexpr int kBalancedMaxWaves = 2048;  // waves (and partial-slot pairs) of a balanced call
constexpr int kBalancedWavesPerGroup = 2;  // waves of a balanced workgroup (independent, one LDS table each)

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int64_t wave_incl_scan(int64_t v, int lane) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int64_t t = __shfl_up(v, o, 64);
        if (lane >= o) v += t;
    }
    return v;
}

// Wave-uniform copies (values read from LDS land in vector registers; the
// loop state derived from them is kept in scalar registers this way).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uniform64(int64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Wave (of nw) whose step range holds global step x; wave w covers
// [S*w/nw, S*(w+1)/nw).
__device__ __forceinline__ int wave_of_step(int64_t x, int64_t S, int nw) {
    return (int)(((x + 1) * nw - 1) / S);
}

// A wave's position in the global step order (all fields wave-uniform).
struct StepCursor {
    int b;    // sequence
    int g;    // kv-head
    int ls;   // step within the (sequence, kv-head) segment
    int nst;  // steps of that segment
    int L;    // length of sequence b
    int t0;   // multi-token query: first query row of sequence b
    int M;    // multi-token query: its query tokens (the last M of its L)
};

// Advance one step, skipping sequences without steps.  Called only while
// a next step exists, so a later sequence with steps exists too.
template <bool MULTI>
__device__ __forceinline__ void cursor_next(StepCursor& c, const int32_t* s_steps, const int32_t* s_len,
                                            const int32_t* s_qs, int Hkv) {
    if (++c.ls < c.nst) return;
    c.ls = 0;
    if (++c.g < Hkv) return;
    c.g = 0;
    do {
        ++c.b;
    } while (uniform(s_steps[c.b]) == 0);
    c.nst = uniform(s_steps[c.b]);
    c.L = uniform(s_len[c.b]);
    if constexpr (MULTI) {
        c.t0 = uniform(s_qs[c.b]);
        c.M = uniform(s_qs[c.b + 1]) - c.t0;
    }
}

// Output row of column n of segment (b, g): head g*G + n for a decode; for a
// multi-token query, columns are (token, head) pairs, token-major.
template <bool MULTI>
__device__ __forceinline__ int64_t col_row(int b, int g, int t0, int n, int Hq, int G) {
    if constexpr (MULTI)
        return (int64_t)(t0 + n / G) * Hq + g * G + n % G;
    else
        return (int64_t)b * Hq + g * G + n;
}

// What the load stage of a step needs: its sequence length and the
// physical blocks of its tokens.  The table entries are read with scalar
// loads (wave-uniform addresses); their wait counter is shared only with
// the rare LDS reads of the step cursor.  An entry outside the pool is
// replaced by block 0 (so no load leaves the pool) and flags the step.
struct StepInfo {
    StepBlocks e;
    int L;
    bool bad;
};

template <bool BF16, int D, int BS>
__device__ __forceinline__ void fetch_step(StepInfo& f, const StepCursor& c, const int32_t* __restrict__ tables,
                                           int max_blocks, int num_blocks) {
    using C = DecodeCfg<BF16, D, BS>;
    const int32_t* trow = tables + (int64_t)c.b * max_blocks;
    const int blk = c.ls * C::STEP / BS;
    const int lastb = (c.L - 1) / BS;
    bool bad = false;
    auto entry = [&](int i) {
        const int32_t v = trow[min(blk + i, lastb)];
        const bool ok = v >= 0 && v < num_blocks;
        bad |= !ok;
        return ok ? v : 0;
    };
    f.e.e0 = entry(0);
    f.e.e1 = C::NE > 1 ? entry(1) : 0;
    f.e.e2 = C::NE > 2 ? entry(2) : 0;
    f.e.e3 = C::NE > 3 ? entry(3) : 0;
    f.L = c.L;
    f.bad = bad;
}

// Query operand loaded by every lane: the padding columns n >= G repeat
// head G-1.  Their scores, softmax statistics and outputs stay in their own
// columns and are never stored, and the loaded registers are used as they
// arrive (touching them here would make this stage wait for the load).
template <bool BF16, int D, int BS, bool MULTI>
__device__ __forceinline__ void load_q_all(typename DecodeCfg<BF16, D, BS>::QRegs& qr, const void* __restrict__ q_,
                                           const StepCursor& c, int Hq, int n, int j, int G, int qi, int qh) {
    using C = DecodeCfg<BF16, D, BS>;
    int64_t row;
    if constexpr (MULTI)  // column (qi, qh) = (n / G, n % G); past the last token: the last column
        row = (int64_t)(c.t0 + min(qi, c.M - 1)) * Hq + c.g * G + (qi < c.M ? qh : G - 1);
    else
        row = (int64_t)c.b * Hq + c.g * G + min(n, G - 1);
    const char* qp = reinterpret_cast<const char*>(q_) + row * D * C::ES;
#pragma unroll
    for (int c = 0; c < C::NKC; ++c) qr[c] = ld16(qp + (int64_t)(4 * c + j) * 16);
}

// A cut (sequence, kv-head) whose piece this wave left in a partial slot.
struct CutPiece {
    bool valid;
    int b, g;
    int64_t seg0, seg1;  // the segment's global steps [seg0, seg1)
    int t0, M;           // multi-token query: the segment's rows
};

// The counter of a cut segment and the waves holding its pieces: one
// counter per cut segment, named by the first wave holding a piece of it (a
// wave is the first of at most one cut segment: the last one that starts in
// it), so the names never collide, whatever the batch.
struct CutCount {
    int32_t* cnt;
    int w0, w1;
};
__device__ __forceinline__ CutCount cut_count(const CutPiece& cp, int32_t* __restrict__ counters, int64_t S, int nw) {
    const int w0 = wave_of_step(cp.seg0, S, nw);
    return CutCount{counters + w0, w0, wave_of_step(cp.seg1 - 1, S, nw)};
}

// Merge every piece of a cut segment (log-sum-exp rule) and write its rows:
// the pieces' (m, l) and values are loaded two pieces at a time, all loads
// of a pair in flight together, with a running maximum over the pairs
// (a segment has two pieces unless it spans more than two waves).  Called
// by the wave whose count-in completed the segment.
template <bool BF16, int D, int BS, bool MULTI>
__device__ __forceinline__ void merge_cut(const CutPiece& cp, const CutCount& cc, const float* __restrict__ slot_o,
                                          const float* __restrict__ slot_ml, void* __restrict__ out_, int64_t S, int nw,
                                          int Hq, int G, int n, int j) {
    using C = DecodeCfg<BF16, D, BS>;
    const int SC = MULTI ? 16 : G;          // columns per partial slot
    const int ncol = MULTI ? cp.M * G : G;  // columns with an output row
    if (n >= ncol) return;
    RunState<BF16, D, BS> Mg;
    Mg.m = -INFINITY;
    Mg.l = 0.0f;
    Mg.bad = false;
#pragma unroll
    for (int c = 0; c < C::NV; ++c) Mg.acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    // the first wave's piece sits in its second slot when the segment starts
    // inside that wave (the other waves' pieces begin their ranges)
    const int first_slot = cp.seg0 != S * cc.w0 / nw ? 1 : 0;
    for (int k0 = cc.w0; k0 <= cc.w1; k0 += 2) {
        float2 ml[2];
        f32x4 o[2][C::NV];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int k = min(k0 + u, cc.w1);  // a lone last piece loads twice, counted once
            const int64_t sk = 2 * (int64_t)k + (k == cc.w0 ? first_slot : 0);
            ml[u] = coherent_load(reinterpret_cast<const uint64_t*>(slot_ml + (sk * SC + n) * 2));
            const uint64_t* po = reinterpret_cast<const uint64_t*>(slot_o + (sk * SC + n) * D);
#pragma unroll
            for (int c = 0; c < C::NV; ++c) {
                const int e = (16 * c + 4 * j) / 2;
                const float2 lo = coherent_load(po + e), hi = coherent_load(po + e + 1);
                o[u][c] = f32x4{lo.x, lo.y, hi.x, hi.y};
            }
        }
        const bool two = k0 + 1 <= cc.w1;
        const float mb = two ? fmaxf(ml[0].x, ml[1].x) : ml[0].x;
        if (mb > Mg.m) {  // every piece has a visible key, so mb is finite
            const float alpha = Mg.m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(Mg.m - mb);
            Mg.l *= alpha;
#pragma unroll
            for (int c = 0; c < C::NV; ++c) Mg.acc[c] *= alpha;
            Mg.m = mb;
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            if (u == 1 && !two) break;
            const float wt = __builtin_amdgcn_exp2f(ml[u].x - Mg.m);
            Mg.l += wt * ml[u].y;
#pragma unroll
            for (int c = 0; c < C::NV; ++c) Mg.acc[c] += wt * o[u][c];
        }
    }
    store_out<BF16, D, BS>(out_, col_row<MULTI>(cp.b, cp.g, cp.t0, n, Hq, G) - n, Mg, n, j, ncol);
}

// Finish the piece whose last step was just computed: a whole segment is
// written out; a cut one leaves its partial in slot (w, 0) if it is the
// wave's first piece, else (w, 1), and is remembered for counting in.
template <bool BF16, int D, int BS, bool MULTI>
__device__ __forceinline__ void finish_piece(const RunState<BF16, D, BS>& St, const StepCursor& cc, bool seg_begin,
                                             bool& first_piece, CutPiece& cut0, CutPiece& cut1,
                                             const int64_t* s_first, float* __restrict__ slot_o,
                                             float* __restrict__ slot_ml, void* __restrict__ out_, int w, int Hq,
                                             int G, int n, int j) {
    using C = DecodeCfg<BF16, D, BS>;
    const int SC = MULTI ? 16 : G;          // columns per partial slot
    const int ncol = MULTI ? cc.M * G : G;  // columns with an output row
    const bool complete = seg_begin && cc.ls == cc.nst - 1;
    if (complete) {
        store_out<BF16, D, BS>(out_, col_row<MULTI>(cc.b, cc.g, cc.t0, n, Hq, G) - n, St, n, j, ncol);
    } else {
        const int64_t slot = 2 * (int64_t)w + (first_piece ? 0 : 1);
        if (n < ncol) {
            uint64_t* po = reinterpret_cast<uint64_t*>(slot_o + (slot * SC + n) * D);
#pragma unroll
            for (int c = 0; c < C::NV; ++c) {
                const f32x4 a = St.bad ? f32x4{NAN, NAN, NAN, NAN} : St.acc[c];
                const int e = (16 * c + 4 * j) / 2;
                coherent_store(po + e, a[0], a[1]);
                coherent_store(po + e + 1, a[2], a[3]);
            }
            if (j == 0)
                coherent_store(reinterpret_cast<uint64_t*>(slot_ml + (slot * SC + n) * 2), St.bad ? 0.0f : St.m,
                               St.bad ? 1.0f : St.l);
        }
        const int64_t seg0 = uniform64(s_first[cc.b]) + (int64_t)cc.g * cc.nst;
        const CutPiece cp = {true, cc.b, cc.g, seg0, seg0 + cc.nst, cc.t0, cc.M};
        if (first_piece)
            cut0 = cp;
        else
            cut1 = cp;
    }
    first_piece = false;
}

// The decode step's new tokens for the fused append (pa_decode_append):
// row b of k / v ([B][Hkv][D]) is sequence b's token at position L_b - 1,
// stored to slot slots[b] (skipped outside [0, total_slots)) by the launch
// that attends over it.
struct AppendArgs {
    const char* k;
    const char* v;
    const int64_t* slots;
    char* kc;
    char* vc;
    int64_t total_slots;
};

// One wave's state in the balanced kernel and its pipeline stages.  For
// compute step x an iteration (1) issues the key/value/query loads of step
// x+1 with the table entries fetched one iteration earlier, (2) fetches the
// entries of step x+2 with scalar loads and (3) computes step x.  A piece
// ends where its segment ends or at the wave's last step.
template <bool BF16, int D, int BS, bool MULTI, bool APPEND>
struct BalancedWave {
    using C = DecodeCfg<BF16, D, BS>;
    AppendArgs ap;  // APPEND: the new tokens
    const int32_t* s_qs;  // multi-token query: query_start in LDS
    int qi, qh;           // multi-token query: this lane's column as (token n / G, head n % G)
    const void* q_;
    const char* kc;
    const char* vc;
    const int32_t* tables;
    const int64_t* s_first;
    const int32_t* s_steps;
    const int32_t* s_len;
    void* out_;
    float* slot_o;
    float* slot_ml;
    int Hq, Hkv, G, max_blocks, num_blocks;
    float scale_log2;
    int w, n, j;
    int64_t wend;
    int64_t blk_bytes;
    StepCursor cc, ci;  // steps x (compute) and x+1 (issue)
    StepInfo fe;        // fetched table entries of step x+1 (of x+2 after the fetch stage)
    bool bad_c, bad_i;  // bad table entry in step x / x+1
    RunState<BF16, D, BS> St;
    bool seg_begin, first_piece;
    CutPiece cut0, cut1;

    __device__ __forceinline__ void issue(StepRegs<BF16, D, BS>& buf, typename C::QRegs& q, const StepCursor& c,
                                          const StepInfo& f) {
        const int64_t hb = (int64_t)c.g * C::TILE * C::ES;
        issue_step_e<BF16, D, BS>(buf, kc + hb, vc + hb, blk_bytes, f.e, c.ls * C::STEP, c.L, n, j);
        load_q_all<BF16, D, BS, MULTI>(q, q_, c, Hq, n, j, G, qi, qh);
    }

    // step x0 loaded into (buf, q); entries of x0+1 fetched
    __device__ __forceinline__ void prologue(StepRegs<BF16, D, BS>& buf, typename C::QRegs& q, int64_t x0) {
        StepInfo f0;
        fetch_step<BF16, D, BS>(f0, cc, tables, max_blocks, num_blocks);
        bad_c = f0.bad;
        issue(buf, q, cc, f0);
        ci = cc;
        if (x0 + 1 < wend) {
            cursor_next<MULTI>(ci, s_steps, s_len, s_qs, Hkv);
            fetch_step<BF16, D, BS>(fe, ci, tables, max_blocks, num_blocks);
        }
    }

    __device__ __forceinline__ void compute(StepRegs<BF16, D, BS>& buf, const typename C::QRegs& q) {
        if constexpr (APPEND) {
            // the cache holds positions 0 .. L - 2; position L - 1 (not read
            // from the cache, which this launch is writing) is added after the
            // segment's last step.  A step with no cached position (the one
            // step of a length-1 sequence, or a last step starting at L - 1)
            // is skipped: a piece starting there keeps m = -inf, l = 0, acc = 0.
            if (cc.ls * C::STEP < cc.L - 1)
                compute_step<BF16, D, BS>(buf, q, St.m, St.l, St.acc, cc.ls * C::STEP, cc.L - 1, j, scale_log2);
        } else if constexpr (MULTI) {
            // column n is query token n / G at position L - M + n / G: it sees keys up to there
            const int lim = cc.L - cc.M + 1;
            compute_step<BF16, D, BS, true>(buf, q, St.m, St.l, St.acc, cc.ls * C::STEP, cc.L, j, scale_log2,
                                            lim + min(qi, cc.M - 1), lim);
        } else {
            compute_step<BF16, D, BS>(buf, q, St.m, St.l, St.acc, cc.ls * C::STEP, cc.L, j, scale_log2);
        }
        St.bad |= bad_c;
    }

    // The new token's key chunks (4c + j) and value rows (16c + 4j ..) of
    // segment (b, g) for this lane.  Loaded before the next step's loads, so
    // waiting for them leaves those in flight.
    struct NewRow {
        u32x4 k[C::NKC];
        u32x4 v[C::NV];  // bf16: the low half of each holds the lane's 4 values
    };
    __device__ __forceinline__ void load_new(NewRow& r) {
        const int64_t row = ((int64_t)cc.b * Hkv + cc.g) * D * C::ES;
#pragma unroll
        for (int c = 0; c < C::NKC; ++c) r.k[c] = ld16(ap.k + row + (int64_t)(4 * c + j) * 16);
#pragma unroll
        for (int c = 0; c < C::NV; ++c) {
            const int d0 = 16 * c + 4 * j;
            if constexpr (BF16) {
                const u32x2 w = *reinterpret_cast<const u32x2*>(ap.v + row + (int64_t)d0 * 2);
                r.v[c] = u32x4{w[0], w[1], 0u, 0u};
            } else {
                r.v[c] = ld16(ap.v + row + (int64_t)d0 * 4);
            }
        }
    }

    // Position L - 1 of segment (b, g) from the new tokens' rows: its score
    // for each head column (lane group j holds chunks 4c + j of the query
    // and of the key), then one online-softmax update with its value row.
    __device__ __forceinline__ void add_new(const typename C::QRegs& q, const NewRow& nr) {
        float part = 0.0f;
#pragma unroll
        for (int c = 0; c < C::NKC; ++c) {
            const u32x4 kv = nr.k[c];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if constexpr (BF16) {  // two bfloat16 per word, widened exactly
                    part = fmaf(__uint_as_float(q[c][e] << 16), __uint_as_float(kv[e] << 16), part);
                    part = fmaf(__uint_as_float(q[c][e] & 0xffff0000u), __uint_as_float(kv[e] & 0xffff0000u), part);
                } else {
                    part = fmaf(__uint_as_float(q[c][e]), __uint_as_float(kv[e]), part);
                }
            }
        }
        const float sc = wave_sum16(part) * scale_log2;
        const float m_new = fmaxf(St.m, sc);
        const float alpha = m_new == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(St.m - m_new);
        const float p = __builtin_amdgcn_exp2f(sc - m_new);
        St.l = St.l * alpha + p;
        St.m = m_new;
#pragma unroll
        for (int c = 0; c < C::NV; ++c) {  // the lane's accumulator rows 16c + 4j ..
            const u32x4 w = nr.v[c];
            f32x4 vf;
            if constexpr (BF16)
                vf = f32x4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u), __uint_as_float(w[1] << 16),
                           __uint_as_float(w[1] & 0xffff0000u)};
            else
                vf = __builtin_bit_cast(f32x4, w);
            St.acc[c] = St.acc[c] * alpha + p * vf;
        }
    }

    __device__ __forceinline__ void finish() {
        finish_piece<BF16, D, BS, MULTI>(St, cc, seg_begin, first_piece, cut0, cut1, s_first, slot_o, slot_ml, out_, w, Hq,
                                  G, n, j);
    }

    // one iteration for compute step x (x + 1 < wend): load into (bl, ql), compute (bc, qc)
    __device__ __forceinline__ void iter(StepRegs<BF16, D, BS>& bl, typename C::QRegs& ql,
                                         StepRegs<BF16, D, BS>& bc, const typename C::QRegs& qc, int64_t x) {
        const bool seg_end = cc.ls == cc.nst - 1;
        NewRow nr;
        if constexpr (APPEND)
            if (seg_end) load_new(nr);
        issue(bl, ql, ci, fe);
        bad_i = fe.bad;
        StepCursor cf = ci;
        if (x + 2 < wend) {
            cursor_next<MULTI>(cf, s_steps, s_len, s_qs, Hkv);
            fetch_step<BF16, D, BS>(fe, cf, tables, max_blocks, num_blocks);
        }
        // keep the compiler from hoisting the compute (and its wait) above the loads
        __builtin_amdgcn_sched_barrier(0);
        compute(bc, qc);
        if (seg_end) {
            if constexpr (APPEND) add_new(qc, nr);
            finish();
        }
        cc = ci;
        bad_c = bad_i;
        ci = cf;
        if (cc.ls == 0) {
            run_init(St);
            seg_begin = true;
        }
    }

    // the wave's last step
    __device__ __forceinline__ void last(StepRegs<BF16, D, BS>& bc, const typename C::QRegs& qc) {
        if constexpr (APPEND) {
            NewRow nr;
            const bool seg_end = cc.ls == cc.nst - 1;
            if (seg_end) load_new(nr);
            compute(bc, qc);
            if (seg_end) add_new(qc, nr);
        } else {
            compute(bc, qc);
        }
        finish();
    }
};

// The fused append's stores: wave w stores (sequence, kv-head) rows w,
// w + grid, ... of the new tokens (lane c: 16-byte chunk c of the key and of
// the value) in the layout pa_cache_write uses, non-temporally.  Nothing in
// the launch reads those slots, so a wave issues them after all its own
// work and never waits for them: issued earlier, they would hold up the
// wave's next load wait (loads and stores complete in issue order), and the
// partial-line value stores are slow to complete.
template <int ES, int D, int BS>
__device__ __forceinline__ void append_rows(const AppendArgs& ap, int w, int nwaves, int rows, int Hkv,
                                            int lane) {
    constexpr int NCH = D * ES / 16;  // 16-byte chunks of a key row
    for (int r = w; r < rows; r += nwaves) {
        const int64_t sl = ap.slots[r / Hkv];
        if (lane < NCH && sl >= 0 && sl < ap.total_slots) {
            const int64_t src = (int64_t)r * D * ES + (int64_t)lane * 16;
            store_token_chunk<ES, true>(ap.kc, ap.vc, sl, r % Hkv, lane, Hkv, D, BS, ld16(ap.k + src),
                                        ld16(ap.v + src));
        }
    }
}

// Balanced split ("stream-K" over the attention's token steps).
//
// The work is the sequence of segments (b, g), b-major, each of
// ceil(L_b / STEP) steps.  Wave w of nw takes the global steps
// [S*w/nw, S*(w+1)/nw), so every wave reads the same number of key/value
// bytes whatever the length mix.  The wave runs one three-stage pipeline
// over all its steps, across segment boundaries: at step x it reads the
// table entries of step x+2, issues the key/value/query loads of step x+1
// and computes step x, so a new segment costs no extra memory round trip.
// A segment wholly inside the wave is written directly.  A segment cut by
// a wave boundary leaves one partial (unnormalised accumulator, running
// maximum and sum) per piece in the workspace; after its loop each wave
// counts its cut pieces in, and the wave that completes a segment's count
// merges its pieces, writes the rows and puts the counter back to zero.
// No wave waits for another.
// MULTI: a multi-token query (query_start given): segment (b, g) has the
// M_b * G columns (token, head) of sequence b's M_b new tokens, M_b * G <= 16,
// each masked causally at its own position.
// APPEND (decode only): the launch also stores the decode step's new tokens
// (ap) in their slots and attends to position L_b - 1 from ap's rows, so it
// never reads the slots it writes.
template <bool BF16, int D, int BS, bool MULTI, bool APPEND = false>
__global__ __launch_bounds__(64 * kBalancedWavesPerGroup) void decode_balanced_kernel(
    const void* __restrict__ q_, const void* __restrict__ kc_, const void* __restrict__ vc_,
    const int32_t* __restrict__ tables, const int32_t* __restrict__ lens, void* __restrict__ out_,
    float* __restrict__ slot_o, float* __restrict__ slot_ml, int32_t* __restrict__ counters, int B, int Hq,
    int Hkv, int G, int max_blocks, int num_blocks, float scale_log2, const int32_t* __restrict__ q_start, int T,
    AppendArgs ap) {
    using C = DecodeCfg<BF16, D, BS>;
    static_assert(!(MULTI && APPEND), "the fused append is a decode");
    // each wave of the workgroup has its own copy of the tables
    constexpr int WPG = kBalancedWavesPerGroup;
    __shared__ int64_t s_first_g[WPG][kBalancedMaxSeqs];  // global step where sequence b's segments start
    __shared__ int32_t s_steps_g[WPG][kBalancedMaxSeqs];  // steps per segment of sequence b (0: no work)
    __shared__ int32_t s_len_g[WPG][kBalancedMaxSeqs];    // length of sequence b
    __shared__ int32_t s_qs_g[WPG][MULTI ? kBalancedMaxSeqs + 1 : 1];  // multi-token query: query_start
    const int sub = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int64_t* s_first = s_first_g[sub];
    int32_t* s_steps = s_steps_g[sub];
    int32_t* s_len = s_len_g[sub];
    int32_t* s_qs = s_qs_g[sub];
    const int lane = threadIdx.x & 63;
    const int n = lane & 15;
    const int j = lane >> 4;
    const int w = blockIdx.x * WPG + sub;  // this wave
    const int nwaves = gridDim.x * WPG;

    // 1. step counts of every sequence and their prefix sums (each wave
    //    computes the same table; the length loads are issued together)
    constexpr int NCH = kBalancedMaxSeqs / 64;
    int32_t lv[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int b = 64 * c + lane;
        lv[c] = (b < B) ? lens[b] : 0;
    }
    int64_t S = 0;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        if (64 * c >= B) break;
        const int b = 64 * c + lane;
        const int L = lv[c];
        bool ok = b < B && L > 0 && (int64_t)L <= (int64_t)max_blocks * BS;
        if constexpr (MULTI) {
            // M new tokens at the end of the L cached ones, M * G columns at most 16
            const int t0 = b < B ? q_start[b] : 0, t1 = b < B ? q_start[b + 1] : 0;
            const int M = t1 - t0;
            ok = ok && t0 >= 0 && t1 <= T && M >= 1 && M <= L && M * G <= 16;
            if (b < B) {
                s_qs[b] = t0;
                if (b == B - 1) s_qs[B] = t1;
            }
        }
        const int st = ok ? (L + C::STEP - 1) / C::STEP : 0;
        const int64_t v = (int64_t)st * Hkv;
        const int64_t incl = wave_incl_scan(v, lane);
        if (b < B) {
            s_first[b] = S + incl - v;
            s_steps[b] = st;
            s_len[b] = L;
        }
        S += __shfl(incl, 63, 64);
    }
    S = uniform64(S);
    __syncthreads();

    // 2. rows no segment covers: empty sequences (zeros) and lengths the
    //    table cannot hold (NaN)
    for (int b = w; b < B; b += nwaves) {
        if (s_steps[b] == 0) {
            const int L = lens[b];
            if constexpr (MULTI) {
                // rows of a request that cannot be served (more new tokens than
                // cached ones or than the columns hold, or a bad length): NaN;
                // malformed query offsets: nothing is written
                const int t0 = q_start[b], t1 = q_start[b + 1];
                if (t0 >= 0 && t1 <= T && t1 > t0)
                    fill_rows<BF16, D>(out_, (int64_t)t0 * Hq, (t1 - t0) * Hq, __builtin_nanf(""), lane);
            } else {
                fill_rows<BF16, D>(out_, (int64_t)b * Hq, Hq, L <= 0 ? 0.0f : __builtin_nanf(""), lane);
            }
        }
    }
    const int nw = (int)min((int64_t)nwaves, S);
    if (w >= nw) {
        if constexpr (APPEND) append_rows<C::ES, D, BS>(ap, w, nwaves, B * Hkv, Hkv, lane);
        return;
    }
    const int64_t wbeg = S * w / nw;
    const int64_t wend = S * (w + 1) / nw;

    // 3. cursor at step wbeg: the last b with s_first[b] <= wbeg holds it
    int lo = 0, hi = B - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (uniform64(s_first[mid]) <= wbeg) lo = mid;
        else hi = mid - 1;
    }
    StepCursor cc;
    cc.b = uniform(lo);
    cc.nst = uniform(s_steps[cc.b]);
    cc.L = uniform(s_len[cc.b]);
    cc.t0 = 0;
    cc.M = 1;
    if constexpr (MULTI) {
        cc.t0 = uniform(s_qs[cc.b]);
        cc.M = uniform(s_qs[cc.b + 1]) - cc.t0;
    }
    {
        const int64_t off = wbeg - uniform64(s_first[cc.b]);
        cc.g = (int)(off / cc.nst);
        cc.ls = (int)(off % cc.nst);
    }

    // 4. the pipeline: stage buffers A and B alternate, so no loaded
    //    register is ever copied (a copy would have to wait for its load)
    BalancedWave<BF16, D, BS, MULTI, APPEND> W;
    W.ap = ap;
    W.s_qs = s_qs;
    W.qi = MULTI ? n / G : 0;
    W.qh = MULTI ? n % G : 0;
    W.q_ = q_;
    W.kc = reinterpret_cast<const char*>(kc_);
    W.vc = reinterpret_cast<const char*>(vc_);
    W.tables = tables;
    W.s_first = s_first;
    W.s_steps = s_steps;
    W.s_len = s_len;
    W.out_ = out_;
    W.slot_o = slot_o;
    W.slot_ml = slot_ml;
    W.Hq = Hq;
    W.Hkv = Hkv;
    W.G = G;
    W.max_blocks = max_blocks;
    W.num_blocks = num_blocks;
    W.scale_log2 = scale_log2;
    W.w = w;
    W.n = n;
    W.j = j;
    W.wend = wend;
    W.blk_bytes = (int64_t)Hkv * C::TILE * C::ES;
    W.cc = cc;
    W.seg_begin = cc.ls == 0;
    W.first_piece = true;
    W.cut0 = CutPiece{false, 0, 0, 0, 0, 0, 0};
    W.cut1 = CutPiece{false, 0, 0, 0, 0, 0, 0};
    run_init(W.St);

    StepRegs<BF16, D, BS> bufA, bufB;
    typename C::QRegs qA, qB;
    W.prologue(bufA, qA, wbeg);
    int64_t x = wbeg;
    for (; x + 2 < wend; x += 2) {
        W.iter(bufB, qB, bufA, qA, x);
        W.iter(bufA, qA, bufB, qB, x + 1);
    }
    if (x + 1 < wend) {
        W.iter(bufB, qB, bufA, qA, x);
        W.last(bufB, qB);
    } else {
        W.last(bufA, qA);
    }
    const CutPiece cut0 = W.cut0, cut1 = W.cut1;

    // 5. count the cut pieces in (their partials must be at the coherent
    //    level first), both counts in one round trip; the wave that completes
    //    a segment's count merges its pieces and puts the counter back to zero
    if (cut0.valid || cut1.valid) {
        __builtin_amdgcn_s_waitcnt(0);
        const CutCount k0 = cut_count(cut0, counters, S, nw), k1 = cut_count(cut1, counters, S, nw);
        int old0 = -1, old1 = -1;
        if (lane == 0) {
            if (cut0.valid) old0 = __hip_atomic_fetch_add(k0.cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (cut1.valid) old1 = __hip_atomic_fetch_add(k1.cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        old0 = __shfl(old0, 0, 64);
        old1 = __shfl(old1, 0, 64);
        const bool mine0 = cut0.valid && old0 == k0.w1 - k0.w0;
        const bool mine1 = cut1.valid && old1 == k1.w1 - k1.w0;
        // one inlined copy of the merge serves both cut pieces
#pragma unroll 1
        for (int q = 0; q < 2; ++q) {
            if (!(q == 0 ? mine0 : mine1)) continue;
            const CutPiece cp = q == 0 ? cut0 : cut1;
            const CutCount kq = q == 0 ? k0 : k1;
            merge_cut<BF16, D, BS, MULTI>(cp, kq, slot_o, slot_ml, out_, S, nw, Hq, G, n, j);
            if (lane == 0) __hip_atomic_store(kq.cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    // 6. the new tokens' stores, last: nothing in the launch waits for them
    if constexpr (APPEND) append_rows<C::ES, D, BS>(ap, w, nwaves, B * Hkv, Hkv, lane);
}

// Zero n 32-bit words (a fill kernel rather than a memset, so that a caller
// capturing the stream into a graph records a kernel node).
__global__ __launch_bounds__(256) void zero_words_kernel(int32_t* __restrict__ p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

// Scratch of pa_decode_append_noalloc: the balanced split's merge counters
// and cut-piece partials for callers that cannot allocate.  Every GPU the
// library runs on holds its own copy until the process ends.  Host code
// never uses this name as an address: it takes each device's address of
// the array from hipGetSymbolAddress (see noalloc_scratch below).
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

}  // namespace pa

// ---------------------------------------------------------------------------- host side

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Workspace layout (every mode): [counters | partials].  The counter region
// (one int32 per wave of a balanced call) comes first and has one size for
// every call, so that other modes and other batch sizes never overwrite it.
inline size_t counter_bytes() { return align_up((size_t)pa::kBalancedMaxWaves * sizeof(int32_t)); }

// Effective partition length and partition count of the fixed-partition modes.
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

// Waves of a balanced call: kWavesPerCU per compute unit of the current device,
// launched kBalancedWavesPerGroup to a workgroup.  Measured on MI355X
// (Llama-3-8B-shaped batch): 2 per CU reads fastest; 4 is ~3 % slower and
// more than 4 no longer fit in one round.  Two waves per workgroup instead
// of one ran 0.3-0.6 % faster in every paired run (the Llama-3-8B and
// 70B shapes, with and without the fused append).
constexpr int kWavesPerCU = 2;
int balanced_waves() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (!cached[dev]) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        cached[dev] = std::min(pa::kBalancedMaxWaves, kWavesPerCU * cus) / pa::kBalancedWavesPerGroup *
                      pa::kBalancedWavesPerGroup;
    }
    return cached[dev];
}

// Device address of the no-alloc scratch on the current device, set up on
// the first call there: hipGetSymbolAddress with that device current, then
// the counter region cleared by a fill kernel on the caller's stream (the
// balanced split leaves its counters zero after every call, so once is
// enough).  Null on failure.
char* noalloc_scratch(hipStream_t stream) {
    static std::mutex mu;
    static char* addr[64] = {nullptr};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(pa::scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return nullptr;
        }
        const int64_t words = (int64_t)(counter_bytes() / sizeof(int32_t));
        hipLaunchKernelGGL(pa::zero_words_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, stream,
                           reinterpret_cast<int32_t*>(p), words);
        if (hipGetLastError() != hipSuccess) return nullptr;
        addr[dev] = reinterpret_cast<char*>(p);
    }
    return addr[dev];
}

struct Launch {
    const void *q, *kc, *vc;
    const int32_t *tables, *lens;
    void* out;
    float *po, *pml;
    int32_t* counters;
    int B, Hq, Hkv, max_blocks, num_blocks, PS, P_max;
    bool balanced;
    const int32_t* q_start;  // set: a multi-token query on the balanced split (T query rows)
    int T;
    float sl2;
    hipStream_t stream;
    bool append;  // the fused append (balanced split): ap holds the new tokens
    pa::AppendArgs ap;
};

template <bool BF16, int D, int BS>
hipError_t launch_decode(const Launch& a) {
    const int G = a.Hq / a.Hkv;
    if (a.balanced) {
        if (a.q_start)
            hipLaunchKernelGGL((pa::decode_balanced_kernel<BF16, D, BS, true>), dim3((unsigned)(balanced_waves() / pa::kBalancedWavesPerGroup)),
                               dim3(64 * pa::kBalancedWavesPerGroup), 0, a.stream, a.q, a.kc, a.vc, a.tables, a.lens, a.out, a.po, a.pml,
                               a.counters, a.B, a.Hq, a.Hkv, G, a.max_blocks, a.num_blocks, a.sl2, a.q_start, a.T,
                               pa::AppendArgs{});
        else if (a.append)
            hipLaunchKernelGGL((pa::decode_balanced_kernel<BF16, D, BS, false, true>), dim3((unsigned)(balanced_waves() / pa::kBalancedWavesPerGroup)),
                               dim3(64 * pa::kBalancedWavesPerGroup), 0, a.stream, a.q, a.kc, a.vc, a.tables, a.lens, a.out, a.po, a.pml,
                               a.counters, a.B, a.Hq, a.Hkv, G, a.max_blocks, a.num_blocks, a.sl2, nullptr, 0, a.ap);
        else
            hipLaunchKernelGGL((pa::decode_balanced_kernel<BF16, D, BS, false>), dim3((unsigned)(balanced_waves() / pa::kBalancedWavesPerGroup)),
                               dim3(64 * pa::kBalancedWavesPerGroup), 0, a.stream, a.q, a.kc, a.vc, a.tables, a.lens, a.out, a.po, a.pml,
                               a.counters, a.B, a.Hq, a.Hkv, G, a.max_blocks, a.num_blocks, a.sl2, nullptr, 0,
                               pa::AppendArgs{});
        return hipGetLastError();
    }
    dim3 grid((unsigned)a.Hkv, (unsigned)a.P_max, (unsigned)a.B);
    hipLaunchKernelGGL((pa::decode_kernel<BF16, D, BS>), grid, dim3(64), 0, a.stream, a.q, a.kc, a.vc, a.tables,
                       a.lens, a.out, a.po, a.pml, a.Hq, a.Hkv, G, a.max_blocks, a.num_blocks, a.PS, a.P_max, a.sl2);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.P_max <= 1) return e;
    constexpr int RG = 256 / (D / 4);  // partition rows a merge workgroup holds side by side
    const dim3 mg((unsigned)a.Hq, (unsigned)a.B);
    if (a.P_max <= RG)
        hipLaunchKernelGGL((pa::merge_kernel<BF16, D, 1>), mg, dim3(256), 0, a.stream, a.po, a.pml, a.lens, a.out,
                           a.Hq, a.max_blocks, BS, a.PS, a.P_max);
    else if (a.P_max <= 4 * RG)
        hipLaunchKernelGGL((pa::merge_kernel<BF16, D, 4>), mg, dim3(256), 0, a.stream, a.po, a.pml, a.lens, a.out,
                           a.Hq, a.max_blocks, BS, a.PS, a.P_max);
    else
        hipLaunchKernelGGL((pa::merge_kernel<BF16, D, 16>), mg, dim3(256), 0, a.stream, a.po, a.pml, a.lens, a.out,
                           a.Hq, a.max_blocks, BS, a.PS, a.P_max);
    return hipGetLastError();
}

template <bool BF16, int D>
hipError_t dispatch_bs(int BS, const Launch& a) {
    switch (BS) {
        case 8: return launch_decode<BF16, D, 8>(a);
        case 16: return launch_decode<BF16, D, 16>(a);
        default: return launch_decode<BF16, D, 32>(a);
    }
}

}  // namespace

extern "C" size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                            int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                                            int32_t partition_size) {
    if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads || head_dim <= 0 ||
        block_size <= 0 || max_blocks_per_seq < 0 || partition_size < PA_PARTITION_BALANCED)
        return 0;
    const size_t cnt = counter_bytes();
    if (partition_size == PA_PARTITION_BALANCED) {
        const size_t slots = 2 * (size_t)pa::kBalancedMaxWaves * (size_t)(num_q_heads / num_kv_heads);
        return cnt + align_up(slots * head_dim * sizeof(float)) + align_up(slots * 2 * sizeof(float));
    }
    int64_t ps, pmax;
    partition_plan(block_size, max_blocks_per_seq, partition_size, &ps, &pmax);
    if (pmax <= 1) return 0;
    const size_t rows = (size_t)num_seqs * num_q_heads * (size_t)pmax;
    return cnt + align_up(rows * head_dim * sizeof(float)) + align_up(rows * 2 * sizeof(float));
}

// pa_decode, and with `ap` the fused append (pa_decode_append) on the balanced split.
static pa_status decode_impl(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                             const int32_t* seq_lens, int32_t num_kv_heads, float scale, void* out, void* stream,
                             int32_t num_seqs, int32_t num_q_heads, int32_t head_dim, int32_t block_size,
                             int32_t num_blocks, int32_t max_blocks_per_seq, pa_dtype dtype, int32_t partition_size,
                             void* workspace, size_t workspace_bytes, const pa::AppendArgs* ap,
                             bool noalloc = false) {
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks < 0 || max_blocks_per_seq < 0 ||
        partition_size < PA_PARTITION_BALANCED || !std::isfinite(scale))
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
    const bool balanced = partition_size == PA_PARTITION_BALANCED;
    if (balanced && num_seqs > pa::kBalancedMaxSeqs) return PA_ERR_UNSUPPORTED;
    if (num_seqs == 0) return PA_OK;
    if (!q || !k_cache || !v_cache || !block_tables || !seq_lens || !out) return PA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
        (reinterpret_cast<uintptr_t>(block_tables) & 3u) || (reinterpret_cast<uintptr_t>(seq_lens) & 3u))
        return PA_ERR_INVALID_ARG;
    if (ap && (!ap->k || !ap->v || !ap->slots || !aligned16(ap->k) || !aligned16(ap->v) ||
               (reinterpret_cast<uintptr_t>(ap->slots) & 7u)))
        return PA_ERR_INVALID_ARG;

    int64_t ps = 0, pmax = 1;
    if (!balanced) {
        partition_plan(block_size, max_blocks_per_seq, partition_size, &ps, &pmax);
        if (pmax > 65535) return PA_ERR_UNSUPPORTED;
    }
    Launch a{};
    if (noalloc) {
        // the library's own scratch (pa_decode_append_noalloc): partials are
        // indexed by wave, two slots of G rows per wave of the launch, so
        // the size follows the device's wave count, not the batch
        if (!balanced) return PA_ERR_INVALID_ARG;
        const size_t rows = 2 * (size_t)balanced_waves() * (size_t)(num_q_heads / num_kv_heads);
        const size_t o_bytes = align_up(rows * (size_t)head_dim * sizeof(float));
        if (counter_bytes() + o_bytes + align_up(rows * 2 * sizeof(float)) > pa::kNoAllocScratchBytes)
            return PA_ERR_UNSUPPORTED;
        char* base = noalloc_scratch(reinterpret_cast<hipStream_t>(stream));
        if (!base) return PA_ERR_LAUNCH;
        a.counters = reinterpret_cast<int32_t*>(base);
        a.po = reinterpret_cast<float*>(base + counter_bytes());
        a.pml = reinterpret_cast<float*>(base + counter_bytes() + o_bytes);
    } else if (balanced || pmax > 1) {
        const size_t need = pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                                      max_blocks_per_seq, partition_size);
        if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)))
            return PA_ERR_INVALID_ARG;
        char* ws = reinterpret_cast<char*>(workspace);
        const size_t cnt = counter_bytes();
        const size_t rows = balanced ? 2 * (size_t)pa::kBalancedMaxWaves * (size_t)(num_q_heads / num_kv_heads)
                                     : (size_t)num_seqs * num_q_heads * (size_t)pmax;
        a.counters = reinterpret_cast<int32_t*>(ws);
        a.po = reinterpret_cast<float*>(ws + cnt);
        a.pml = reinterpret_cast<float*>(ws + cnt + align_up(rows * head_dim * sizeof(float)));
    }
    a.q = q;
    a.kc = k_cache;
    a.vc = v_cache;
    a.tables = block_tables;
    a.lens = seq_lens;
    a.out = out;
    a.B = num_seqs;
    a.Hq = num_q_heads;
    a.Hkv = num_kv_heads;
    a.max_blocks = max_blocks_per_seq;
    a.num_blocks = num_blocks;
    a.PS = (int)ps;
    a.P_max = (int)pmax;
    a.balanced = balanced;
    a.sl2 = (float)((double)scale * 1.4426950408889634);  // scale * log2(e)
    a.stream = reinterpret_cast<hipStream_t>(stream);
    a.append = ap != nullptr;
    if (ap) a.ap = *ap;
    hipError_t e;
    if (dtype == PA_BF16)
        e = head_dim == 128 ? dispatch_bs<true, 128>(block_size, a) : dispatch_bs<true, 64>(block_size, a);
    else
        e = head_dim == 128 ? dispatch_bs<false, 128>(block_size, a) : dispatch_bs<false, 64>(block_size, a);
    return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

extern "C" pa_status pa_decode(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, const int32_t* seq_lens, int32_t num_kv_heads,
                               float scale, void* out, void* stream, int32_t num_seqs, int32_t num_q_heads,
                               int32_t head_dim, int32_t block_size, int32_t num_blocks,
                               int32_t max_blocks_per_seq, pa_dtype dtype, int32_t partition_size,
                               void* workspace, size_t workspace_bytes) {
    return decode_impl(q, k_cache, v_cache, block_tables, seq_lens, num_kv_heads, scale, out, stream, num_seqs,
                       num_q_heads, head_dim, block_size, num_blocks, max_blocks_per_seq, dtype, partition_size,
                       workspace, workspace_bytes, nullptr);
}

extern "C" pa_status pa_decode_append(const void* q, const void* k, const void* v, const int64_t* slot_mapping,
                                      void* k_cache, void* v_cache, const int32_t* block_tables,
                                      const int32_t* seq_lens, int32_t num_kv_heads, float scale, void* out,
                                      void* stream, int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                      int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                                      pa_dtype dtype, void* workspace, size_t workspace_bytes) {
    if (num_blocks < 0 || block_size <= 0) return PA_ERR_INVALID_ARG;
    pa::AppendArgs ap{reinterpret_cast<const char*>(k), reinterpret_cast<const char*>(v), slot_mapping,
                      reinterpret_cast<char*>(k_cache), reinterpret_cast<char*>(v_cache),
                      (int64_t)num_blocks * block_size};
    return decode_impl(q, k_cache, v_cache, block_tables, seq_lens, num_kv_heads, scale, out, stream, num_seqs,
                       num_q_heads, head_dim, block_size, num_blocks, max_blocks_per_seq, dtype,
                       PA_PARTITION_BALANCED, workspace, workspace_bytes, &ap);
}

extern "C" pa_status pa_decode_append_noalloc(const void* q, const void* k, const void* v,
                                              const int64_t* slot_mapping, void* k_cache, void* v_cache,
                                              const int32_t* block_tables, const int32_t* seq_lens,
                                              int32_t num_kv_heads, float scale, void* out, void* stream,
                                              int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                              int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                                              pa_dtype dtype) {
    if (num_blocks < 0 || block_size <= 0) return PA_ERR_INVALID_ARG;
    pa::AppendArgs ap{reinterpret_cast<const char*>(k), reinterpret_cast<const char*>(v), slot_mapping,
                      reinterpret_cast<char*>(k_cache), reinterpret_cast<char*>(v_cache),
                      (int64_t)num_blocks * block_size};
    return decode_impl(q, k_cache, v_cache, block_tables, seq_lens, num_kv_heads, scale, out, stream, num_seqs,
                       num_q_heads, head_dim, block_size, num_blocks, max_blocks_per_seq, dtype,
                       PA_PARTITION_BALANCED, nullptr, 0, &ap, true);
}

// ---- multi-token query on the balanced split (pa_prefill's path for
// requests whose new tokens fit one wave's 16 columns: M * G <= 16)
namespace pa_internal {

size_t multi_balanced_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t max_query_len) {
    if (num_seqs <= 0 || num_seqs > pa::kBalancedMaxSeqs || num_kv_heads <= 0 || num_q_heads % num_kv_heads ||
        head_dim <= 0 || max_query_len <= 0 || (int64_t)max_query_len * (num_q_heads / num_kv_heads) > 16)
        return 0;
    const size_t slots = 2 * (size_t)pa::kBalancedMaxWaves * 16;
    return counter_bytes() + align_up(slots * head_dim * sizeof(float)) +
           align_up(slots * 2 * sizeof(float));
}

// Arguments are validated by the caller (pa_prefill); the workspace holds at
// least multi_balanced_workspace_bytes().
pa_status multi_balanced_launch(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                                const int32_t* seq_lens, const int32_t* query_start, int32_t num_kv_heads, float scale,
                                void* out, void* stream, int32_t num_seqs, int32_t num_query_tokens,
                                int32_t num_q_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                int32_t max_blocks_per_seq, pa_dtype dtype, void* workspace) {
    Launch a{};
    char* ws = reinterpret_cast<char*>(workspace);
    const size_t cnt = counter_bytes();
    const size_t slots = 2 * (size_t)pa::kBalancedMaxWaves * 16;
    a.counters = reinterpret_cast<int32_t*>(ws);
    a.po = reinterpret_cast<float*>(ws + cnt);
    a.pml = reinterpret_cast<float*>(ws + cnt + align_up(slots * head_dim * sizeof(float)));
    a.q = q;
    a.kc = k_cache;
    a.vc = v_cache;
    a.tables = block_tables;
    a.lens = seq_lens;
    a.out = out;
    a.B = num_seqs;
    a.Hq = num_q_heads;
    a.Hkv = num_kv_heads;
    a.max_blocks = max_blocks_per_seq;
    a.num_blocks = num_blocks;
    a.PS = 0;
    a.P_max = 1;
    a.balanced = true;
    a.q_start = query_start;
    a.T = num_query_tokens;
    a.sl2 = (float)((double)scale * 1.4426950408889634);  // scale * log2(e)
    a.stream = reinterpret_cast<hipStream_t>(stream);
    hipError_t e;
    if (dtype == PA_BF16)
        e = head_dim == 128 ? dispatch_bs<true, 128>(block_size, a) : dispatch_bs<true, 64>(block_size, a);
    else
        e = head_dim == 128 ? dispatch_bs<false, 128>(block_size, a) : dispatch_bs<false, 64>(block_size, a);
    return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // namespace pa_internal

extern "C" size_t pa_decode_counter_bytes(void) { return counter_bytes(); }
