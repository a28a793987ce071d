// Device-side helpers shared by the libpa kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 16-byte global load / store (one global_load_dwordx4 / global_store_dwordx4).
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// 16-byte streaming load: marked non-temporal, for data read once (the
// K/V pool during decode), so it does not displace reusable lines.
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// 8-byte streaming load (same policy).
__device__ __forceinline__ u32x2 ld8_stream(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
}

// 16-byte streaming store: marked non-temporal, for pool tiles written once
// and not read again soon.
__device__ __forceinline__ void st16_stream(void* p, u32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// float -> bfloat16 bits, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// Two floats -> two bfloat16 in one word (lo in the low half), round to
// nearest even: gfx950's packed conversion instruction (a NaN stays a NaN).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

__device__ __forceinline__ float shfl_xor_f(float x, int mask) { return __shfl_xor(x, mask, 64); }

// Store 16-byte chunk c (head-dim elements c*X .. c*X + X - 1, X = 16 / ES)
// of one token's key (kv) and value (vv) for kv-head h into slot s of a pool
// of blocks of BS tokens, in the pool's tile layout: keys [D/X][BS][X],
// values [D][BS] per (block, head), bf16 values in blocks of 16 or 32 at the
// in-block offset with bits 2 and 3 swapped.  One key store, X value stores.
// NT: non-temporal stores, for launches that write one token per block (a
// decode step): its scattered value stores are partial lines, which leave
// sooner this way than through write-back at the end of the kernel
// (measured: the two-call decode step 104.2 -> 101.3 us, the one-launch step
// 99.6 -> 98.5 us).  Appends of many tokens per block keep write-back stores,
// which L2 merges into whole lines (with NT a bulk append of 139k tokens took
// 8.1 ms instead of 1.2 ms).
template <int ES, bool NT>
__device__ __forceinline__ void store_token_chunk(char* __restrict__ kc, char* __restrict__ vc, int64_t s, int h,
                                                  int c, int Hkv, int D, int BS, u32x4 kv, u32x4 vv) {
    constexpr int X = 16 / ES;
    const int64_t blk = s / BS;
    const int off = (int)(s % BS);
    const int64_t tile = (blk * Hkv + h) * (int64_t)D * BS;  // element offset of the (block, head) tile
    u32x4* kp = reinterpret_cast<u32x4*>(kc + (tile + ((int64_t)c * BS + off) * X) * ES);
    if constexpr (NT)
        __builtin_nontemporal_store(kv, kp);
    else
        *kp = kv;
    if constexpr (ES == 2) {
        const int vpos = BS >= 16 ? (off & ~12) | ((off & 4) << 1) | ((off & 8) >> 1) : off;
        uint16_t* vt = reinterpret_cast<uint16_t*>(vc) + tile + (int64_t)c * X * BS + vpos;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint16_t x = (uint16_t)(vv[e >> 1] >> (16 * (e & 1)));
            if constexpr (NT)
                __builtin_nontemporal_store(x, vt + (int64_t)e * BS);
            else
                vt[(int64_t)e * BS] = x;
        }
    } else {
        uint32_t* vt = reinterpret_cast<uint32_t*>(vc) + tile + (int64_t)c * X * BS + off;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if constexpr (NT)
                __builtin_nontemporal_store(vv[e], vt + (int64_t)e * BS);
            else
                vt[(int64_t)e * BS] = vv[e];
        }
    }
}

// Wave-uniform copy of a lane's value (v_readlane_b32).
__device__ __forceinline__ int32_t lane_value(int32_t v, int lane) {
    return __builtin_amdgcn_readlane(v, lane);
}

}  // namespace pa
