// Cache append (pa_cache_write) and whole-block copy (pa_copy_blocks).
//
// The cache grows by one token's keys and values per step, and each token
// lands in the slot its request's block table gives it ("Paged attention in
// LLMs", "The cache being stored"; PagedAttention MCQ page, code sketch).
// A shared block is copied whole before a request writes into it (MCQ page,
// comparison table, "Copy on write blocks").
//
// Pool tile layout (include/pa.h): keys [head_dim/X][block_size][X], values
// [head_dim][block_size] per (block, kv-head), X = 16 bytes of elements; bf16
// values in blocks of 16 or 32 tokens sit at the in-block offset with bits 2
// and 3 swapped.
// One thread moves one 16-byte chunk of a token's key (a 16-byte store) and
// the same chunk of its value (X element stores, block_size apart).

#include <cstdint>

#include "pa.h"
#include "pa_device.h"

namespace pa {

template <int ES, bool NT>
__global__ __launch_bounds__(256) void cache_write_kernel(const char* __restrict__ k, const char* __restrict__ v,
                                                          const int64_t* __restrict__ slots, char* __restrict__ kc,
                                                          char* __restrict__ vc, int64_t n_chunks, int Hkv, int D,
                                                          int BS, int64_t total_slots) {
    constexpr int X = 16 / ES;
    const int C = D / X;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= n_chunks) return;
    const int c = (int)(idx % C);
    const int64_t th = idx / C;  // token * Hkv + head
    const int h = (int)(th % Hkv);
    const int64_t t = th / Hkv;
    // the token's chunks are loaded together with its slot (their addresses
    // do not depend on it), so the launch waits one memory round trip
    const int64_t src = (th * D + (int64_t)c * X) * ES;
    const u32x4 kv = ld16(k + src);
    const u32x4 vv = ld16(v + src);
    const int64_t s = slots[t];
    if (s < 0 || s >= total_slots) return;
    store_token_chunk<ES, NT>(kc, vc, s, h, c, Hkv, D, BS, kv, vv);
}

// ---------------------------------------------------------------------------- bulk append
//
// An append of many tokens (a prefill) mostly fills whole blocks: BS
// consecutive tokens whose slots are one block's slots in order.  For such a
// block the (block, head) tiles of keys and values are written whole, as
// consecutive 16-byte stores in tile order, so every store fills its share
// of whole cache lines; the per-token path above writes each token's 16-byte
// key chunks BS * 16 bytes apart and its values as 2-byte stores, leaving L2
// to merge partial lines.
//
// A workgroup takes a window of W consecutive tokens of one kv-head.  It
// owns every full block whose first token lies in the window (reading up to
// BS - 1 tokens past it), and every token of the window that belongs to no
// full block (written one token at a time, as above).  A token of a full
// block whose first token lies in an earlier window is that window's.
// The slots and every row the workgroup may write are loaded in one round
// trip (all loads in flight at once) and the rows staged through LDS; the
// LDS row stride has 16 bytes of padding, so the tile-order reads of 16 lanes (one
// token each) fall in different banks.
template <int ES, int D, int BS>
struct BulkCfg {
    static constexpr int ROW = D * ES;          // bytes of one token's key (or value) row of one head
    static constexpr int RS = ROW + 16;         // LDS row stride
    static constexpr int CH = ROW / 16;         // 16-byte chunks of a row
    static constexpr int W = 16384 / ROW;       // tokens of a window (16 KiB of keys)
    static constexpr int ROWS = W + BS - 1;     // + the rest of a full block starting in the window
    static constexpr int NS = W + 2 * (BS - 1);  // slots held: tokens t0 - (BS-1) .. t0 + W + BS - 2
    static constexpr int X = 16 / ES;           // elements of a 16-byte piece
    static constexpr int PIECES = D * BS * ES / 16;  // 16-byte pieces of a (block, head) tile
    static constexpr int PR = BS * ES / 16;     // 16-byte pieces of one value row of a tile
    static_assert(W % BS == 0 && W <= 256, "window");
};

template <int ES, int D, int BS>
__global__ __launch_bounds__(256) void cache_write_bulk_kernel(const char* __restrict__ k,
                                                               const char* __restrict__ v,
                                                               const int64_t* __restrict__ slots,
                                                               char* __restrict__ kc, char* __restrict__ vc,
                                                               int64_t T, int Hkv, int64_t total_slots) {
    using C = BulkCfg<ES, D, BS>;
    __shared__ __align__(16) char lk[C::ROWS * C::RS];
    __shared__ __align__(16) char lv[C::ROWS * C::RS];
    __shared__ int64_t ls[C::NS];
    __shared__ int lead[C::W / BS];    // window positions of the full blocks it owns
    __shared__ int scat[C::W];         // window positions of its single tokens
    __shared__ int n_lead, n_scat;
    const int tid = threadIdx.x;
    // workgroup id = window * Hkv + kv-head: consecutive windows of one head
    // are Hkv ids apart, so with the ids dealt round-robin over the XCDs they
    // share an XCD (and its L2) whenever Hkv is a multiple of the XCD count,
    // and the BS - 1 rows a workgroup reads past its window are read from L2
    // by the next one
    const int h = (int)(blockIdx.x % (unsigned)Hkv);
    const int64_t t0 = (int64_t)(blockIdx.x / (unsigned)Hkv) * C::W;

    if (tid == 0) {
        n_lead = 0;
        n_scat = 0;
    }
    // one round trip: the window's slots (with the BS - 1 before and after it)
    // and every row the workgroup may write, its window's and the BS - 1
    // after it where a full block starting in the window can end (those are
    // the next workgroup's first rows, read at about the same time)
    static_assert(C::NS <= 256, "one slot per lane");
    int64_t my_sl = -1;
    if (tid < C::NS) {
        const int64_t t = t0 - (BS - 1) + tid;
        if (t >= 0 && t < T) my_sl = slots[t];
    }
    {
        constexpr int NP = (C::ROWS * C::CH + 255) / 256;  // 16-byte pieces per lane
        u32x4 kr[NP], vr[NP];
        // every load in flight at once, none under a branch: the piece index
        // is clamped to the last piece (a repeat of its load and LDS write)
        // and the row to the last token (rows past it are never read)
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const int p = min(tid + 256 * i, C::ROWS * C::CH - 1);
            const int r = p / C::CH, c = p % C::CH;
            const int64_t src = (min(t0 + r, T - 1) * Hkv + h) * (int64_t)C::ROW + c * 16;
            kr[i] = ld16(k + src);
            vr[i] = ld16(v + src);
        }
        if (tid < C::NS) ls[tid] = (my_sl >= 0 && my_sl < total_slots) ? my_sl : -1;
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const int p = min(tid + 256 * i, C::ROWS * C::CH - 1);
            const int r = p / C::CH, c = p % C::CH;
            *reinterpret_cast<u32x4*>(lk + r * C::RS + c * 16) = kr[i];
            *reinterpret_cast<u32x4*>(lv + r * C::RS + c * 16) = vr[i];
        }
    }
    __syncthreads();

    // slot index i = window position + BS - 1; a full block starts there when
    // its slot is a block's first and the next BS - 1 tokens take the next slots
    auto full_from = [&](int i) {
        const int64_t s0 = ls[i];
        if (s0 < 0 || s0 % BS != 0) return false;
#pragma unroll
        for (int q = 1; q < BS; ++q)
            if (ls[i + q] != s0 + q) return false;
        return true;
    };
    if (tid < C::W && t0 + tid < T) {
        const int64_t s = ls[tid + BS - 1];
        if (s >= 0) {
            const int off = (int)(s % BS);
            if (full_from(tid - off + BS - 1)) {  // in a full block
                if (off == 0) lead[atomicAdd(&n_lead, 1)] = tid;  // ... whose first token is this one: owned here
            } else {
                scat[atomicAdd(&n_scat, 1)] = tid;
            }
        }
    }
    __syncthreads();

    // full blocks: both tiles whole, piece p of the tile at byte 16 p
    const int nl = n_lead;
    for (int li = 0; li < nl; ++li) {
        const int j = lead[li];
        const int64_t blk = ls[j + BS - 1] / BS;
        const int64_t tile = (blk * Hkv + h) * (int64_t)D * BS * ES;  // byte offset of the (block, head) tile
        for (int p = tid; p < C::PIECES; p += 256) {
            // keys [D/X][BS][X]: piece p = (chunk p / BS, token p % BS)
            const int c = p / BS, off = p % BS;
            st16_stream(kc + tile + (int64_t)p * 16, *reinterpret_cast<const u32x4*>(lk + (j + off) * C::RS + c * 16));
            // values [D][BS]: piece p = (row p / PR, positions X (p % PR) ..)
            const int d = p / C::PR, pos0 = (p % C::PR) * C::X;
            u32x4 out;
            if constexpr (ES == 2) {
                uint32_t w[4];
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    // position pos holds the token of offset pos with bits 2 and 3
                    // swapped (blocks of 16 or 32; the swap is its own inverse)
                    auto tok = [&](int pos) {
                        return BS >= 16 ? (pos & ~12) | ((pos & 4) << 1) | ((pos & 8) >> 1) : pos;
                    };
                    const uint16_t lo = *reinterpret_cast<const uint16_t*>(lv + (j + tok(pos0 + e)) * C::RS + d * 2);
                    const uint16_t hi =
                        *reinterpret_cast<const uint16_t*>(lv + (j + tok(pos0 + e + 1)) * C::RS + d * 2);
                    w[e / 2] = (uint32_t)lo | ((uint32_t)hi << 16);
                }
                out = u32x4{w[0], w[1], w[2], w[3]};
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) out[e] = *reinterpret_cast<const uint32_t*>(lv + (j + pos0 + e) * C::RS + d * 4);
            }
            st16_stream(vc + tile + (int64_t)p * 16, out);
        }
    }

    // tokens in no full block: one token at a time
    const int ns = n_scat;
    for (int p = tid; p < ns * C::CH; p += 256) {
        const int r = scat[p / C::CH], c = p % C::CH;
        store_token_chunk<ES, false>(kc, vc, ls[r + BS - 1], h, c, Hkv, D, BS,
                                     *reinterpret_cast<const u32x4*>(lk + r * C::RS + c * 16),
                                     *reinterpret_cast<const u32x4*>(lv + r * C::RS + c * 16));
    }
}

__global__ __launch_bounds__(256) void copy_blocks_kernel(char* __restrict__ kc, char* __restrict__ vc,
                                                          const int32_t* __restrict__ pairs, int64_t block_bytes,
                                                          int num_blocks) {
    const int pi = blockIdx.y;
    const int32_t src = pairs[2 * pi];
    const int32_t dst = pairs[2 * pi + 1];
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
    const int64_t nvec = block_bytes / 16;
    const int64_t so = (int64_t)src * block_bytes, dO = (int64_t)dst * block_bytes;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += (int64_t)gridDim.x * blockDim.x) {
        st16(kc + dO + i * 16, ld16(kc + so + i * 16));
        st16(vc + dO + i * 16, ld16(vc + so + i * 16));
    }
}

// Whole-block copies from one pool to another of the same block shape (a
// device pool and a pinned host pool when a request is swapped out or back
// in).  Pair p copies block pairs[p][0] of the source to block pairs[p][1]
// of the destination, keys and values; workgroup row y takes pairs y,
// y + gridDim.y, ...
__global__ __launch_bounds__(256) void swap_blocks_kernel(const char* __restrict__ sk, const char* __restrict__ sv,
                                                          char* __restrict__ dk, char* __restrict__ dv,
                                                          const int32_t* __restrict__ pairs, int num_pairs,
                                                          int64_t block_bytes, int src_blocks, int dst_blocks) {
    const int64_t nvec = block_bytes / 16;
    for (int pi = blockIdx.y; pi < num_pairs; pi += gridDim.y) {
        const int32_t src = pairs[2 * pi];
        const int32_t dst = pairs[2 * pi + 1];
        if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) continue;
        const int64_t so = (int64_t)src * block_bytes, dO = (int64_t)dst * block_bytes;
        for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec;
             i += (int64_t)gridDim.x * blockDim.x) {
            st16(dk + dO + i * 16, ld16(sk + so + i * 16));
            st16(dv + dO + i * 16, ld16(sv + so + i * 16));
        }
    }
}

}  // namespace pa

namespace {
inline bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// pa_cache_write launches of up to this many tokens (a decode step's batch)
// store non-temporally; larger ones (prefill appends) through write-back.
constexpr int32_t kNonTemporalMaxTokens = 4096;

// Address a kernel can use for p: device memory as is, pinned host memory
// (hipHostMalloc) through its device mapping; anything else (pageable host
// memory, unknown pointers) gives nullptr.
inline const void* device_view(const void* p) {
    hipPointerAttribute_t at;
    if (hipPointerGetAttributes(&at, p) != hipSuccess) {
        (void)hipGetLastError();  // clear the sticky error a failed query leaves
        return nullptr;
    }
    if (at.type == hipMemoryTypeDevice) return p;
    if (at.type == hipMemoryTypeHost && at.devicePointer) return at.devicePointer;
    return nullptr;
}

inline pa_status check_pool(int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                            pa_dtype dtype) {
    if (num_kv_heads <= 0 || num_blocks < 0) return PA_ERR_INVALID_ARG;
    if (dtype != PA_F32 && dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
    if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
    if (block_size != 8 && block_size != 16 && block_size != 32) return PA_ERR_UNSUPPORTED;
    return PA_OK;
}
}  // namespace

namespace {
template <int ES, int D, int BS>
pa_status launch_bulk_t(const char* kp, const char* vp, const int64_t* slots, char* kcp, char* vcp, int64_t T,
                        int Hkv, int64_t total_slots, hipStream_t s) {
    using C = pa::BulkCfg<ES, D, BS>;
    const int64_t nwg = ((T + C::W - 1) / C::W) * Hkv;  // (window, kv-head) workgroups
    if (nwg > 2147483647LL) return PA_ERR_UNSUPPORTED;
    const dim3 grid((unsigned)nwg);
    hipLaunchKernelGGL((pa::cache_write_bulk_kernel<ES, D, BS>), grid, dim3(256), 0, s, kp, vp, slots, kcp, vcp, T, Hkv,
                       total_slots);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

template <int ES, int D>
pa_status launch_bulk_d(int bs, const char* kp, const char* vp, const int64_t* slots, char* kcp, char* vcp,
                        int64_t T, int Hkv, int64_t total_slots, hipStream_t s) {
    switch (bs) {
        case 8: return launch_bulk_t<ES, D, 8>(kp, vp, slots, kcp, vcp, T, Hkv, total_slots, s);
        case 16: return launch_bulk_t<ES, D, 16>(kp, vp, slots, kcp, vcp, T, Hkv, total_slots, s);
        default: return launch_bulk_t<ES, D, 32>(kp, vp, slots, kcp, vcp, T, Hkv, total_slots, s);
    }
}

// Arguments were validated by pa_cache_write.
pa_status launch_bulk(pa_dtype dtype, int head_dim, int bs, const char* kp, const char* vp, const int64_t* slots,
                      char* kcp, char* vcp, int64_t T, int Hkv, int64_t total_slots, hipStream_t s) {
    if (dtype == PA_BF16)
        return head_dim == 128 ? launch_bulk_d<2, 128>(bs, kp, vp, slots, kcp, vcp, T, Hkv, total_slots, s)
                               : launch_bulk_d<2, 64>(bs, kp, vp, slots, kcp, vcp, T, Hkv, total_slots, s);
    return head_dim == 128 ? launch_bulk_d<4, 128>(bs, kp, vp, slots, kcp, vcp, T, Hkv, total_slots, s)
                           : launch_bulk_d<4, 64>(bs, kp, vp, slots, kcp, vcp, T, Hkv, total_slots, s);
}
}  // namespace

extern "C" pa_status pa_cache_write(const void* k, const void* v, const int64_t* slot_mapping, void* k_cache,
                                    void* v_cache, int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t block_size, int32_t num_blocks, pa_dtype dtype, void* stream) {
    if (num_tokens < 0) return PA_ERR_INVALID_ARG;
    pa_status st = check_pool(num_kv_heads, head_dim, block_size, num_blocks, dtype);
    if (st != PA_OK) return st;
    if (num_tokens == 0) return PA_OK;
    if (!k || !v || !slot_mapping || !k_cache || !v_cache) return PA_ERR_INVALID_ARG;
    if (!al16(k) || !al16(v) || !al16(k_cache) || !al16(v_cache) || (reinterpret_cast<uintptr_t>(slot_mapping) & 7u))
        return PA_ERR_INVALID_ARG;
    const int es = dtype == PA_BF16 ? 2 : 4;
    const int64_t chunks = (int64_t)num_tokens * num_kv_heads * (head_dim * es / 16);
    const int64_t grid = (chunks + 255) / 256;
    if (grid > 2147483647LL) return PA_ERR_UNSUPPORTED;
    const int64_t total_slots = (int64_t)num_blocks * block_size;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const char* kp = reinterpret_cast<const char*>(k);
    const char* vp = reinterpret_cast<const char*>(v);
    char* kcp = reinterpret_cast<char*>(k_cache);
    char* vcp = reinterpret_cast<char*>(v_cache);
    // decode-sized appends (about one token per block) store non-temporally,
    // one thread per 16-byte chunk; bulk appends write whole tiles
    if (num_tokens > kNonTemporalMaxTokens) {
        return launch_bulk(dtype, head_dim, block_size, kp, vp, slot_mapping, kcp, vcp, num_tokens, num_kv_heads,
                           total_slots, s);
    }
    const bool nt = true;
    if (dtype == PA_BF16) {
        if (nt)
            hipLaunchKernelGGL((pa::cache_write_kernel<2, true>), dim3((unsigned)grid), dim3(256), 0, s, kp, vp,
                               slot_mapping, kcp, vcp, chunks, num_kv_heads, head_dim, block_size, total_slots);
        else
            hipLaunchKernelGGL((pa::cache_write_kernel<2, false>), dim3((unsigned)grid), dim3(256), 0, s, kp, vp,
                               slot_mapping, kcp, vcp, chunks, num_kv_heads, head_dim, block_size, total_slots);
    } else {
        if (nt)
            hipLaunchKernelGGL((pa::cache_write_kernel<4, true>), dim3((unsigned)grid), dim3(256), 0, s, kp, vp,
                               slot_mapping, kcp, vcp, chunks, num_kv_heads, head_dim, block_size, total_slots);
        else
            hipLaunchKernelGGL((pa::cache_write_kernel<4, false>), dim3((unsigned)grid), dim3(256), 0, s, kp, vp,
                               slot_mapping, kcp, vcp, chunks, num_kv_heads, head_dim, block_size, total_slots);
    }
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

extern "C" pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int32_t num_pairs,
                                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                    pa_dtype dtype, void* stream) {
    if (num_pairs < 0) return PA_ERR_INVALID_ARG;
    pa_status st = check_pool(num_kv_heads, head_dim, block_size, num_blocks, dtype);
    if (st != PA_OK) return st;
    if (num_pairs == 0) return PA_OK;
    if (!k_cache || !v_cache || !pairs) return PA_ERR_INVALID_ARG;
    if (!al16(k_cache) || !al16(v_cache) || (reinterpret_cast<uintptr_t>(pairs) & 3u)) return PA_ERR_INVALID_ARG;
    if (num_pairs > 65535) return PA_ERR_UNSUPPORTED;
    const int es = dtype == PA_BF16 ? 2 : 4;
    const int64_t block_bytes = (int64_t)num_kv_heads * head_dim * block_size * es;
    int64_t gx = (block_bytes / 16 + 255) / 256;
    if (gx > 64) gx = 64;
    hipLaunchKernelGGL(pa::copy_blocks_kernel, dim3((unsigned)gx, (unsigned)num_pairs), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), reinterpret_cast<char*>(k_cache),
                       reinterpret_cast<char*>(v_cache), pairs, block_bytes, num_blocks);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

extern "C" pa_status pa_swap_blocks(const void* src_k, const void* src_v, int32_t src_num_blocks, void* dst_k,
                                    void* dst_v, int32_t dst_num_blocks, const int32_t* pairs, int32_t num_pairs,
                                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, pa_dtype dtype,
                                    void* stream) {
    if (num_pairs < 0 || src_num_blocks < 0) return PA_ERR_INVALID_ARG;
    pa_status st = check_pool(num_kv_heads, head_dim, block_size, dst_num_blocks, dtype);
    if (st != PA_OK) return st;
    if (num_pairs == 0) return PA_OK;
    if (!src_k || !src_v || !dst_k || !dst_v || !pairs) return PA_ERR_INVALID_ARG;
    if (!al16(src_k) || !al16(src_v) || !al16(dst_k) || !al16(dst_v) || (reinterpret_cast<uintptr_t>(pairs) & 3u))
        return PA_ERR_INVALID_ARG;
    const void* sk = device_view(src_k);
    const void* sv = device_view(src_v);
    const void* dk = device_view(dst_k);
    const void* dv = device_view(dst_v);
    const void* pp = device_view(pairs);
    if (!sk || !sv || !dk || !dv || !pp) return PA_ERR_INVALID_ARG;  // pageable or unknown memory
    const int es = dtype == PA_BF16 ? 2 : 4;
    const int64_t block_bytes = (int64_t)num_kv_heads * head_dim * block_size * es;
    int64_t gx = (block_bytes / 16 + 255) / 256;
    if (gx > 64) gx = 64;
    const int gy = num_pairs < 65535 ? num_pairs : 65535;
    hipLaunchKernelGGL(pa::swap_blocks_kernel, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), reinterpret_cast<const char*>(sk),
                       reinterpret_cast<const char*>(sv), reinterpret_cast<char*>(const_cast<void*>(dk)),
                       reinterpret_cast<char*>(const_cast<void*>(dv)), reinterpret_cast<const int32_t*>(pp), num_pairs,
                       block_bytes, src_num_blocks, dst_num_blocks);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}
