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
    // bulk appends through write-back (see store_token_chunk)
    const bool nt = num_tokens <= kNonTemporalMaxTokens;
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
