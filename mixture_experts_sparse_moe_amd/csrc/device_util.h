// Small device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// silu(z) = z / (1 + e^-z), with the hardware reciprocal (about 1 ulp)
__device__ __forceinline__ float silu_f32(float z) {
    return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// Reinterpret 16 bytes as 8 bf16 MFMA operands.
__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) {
    return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// LDS destination operand of the direct-to-LDS loads (global_load_lds).
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Swizzle of LDS rows of 128 bytes (8 chunks of 16 B): chunk c of row r sits
// at c ^ swz(r), so 16-byte reads of one chunk in 32 consecutive rows hit
// distinct banks.
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// s_waitcnt immediate (gfx9 encoding: vmcnt bits [3:0] and [15:14], expcnt
// [6:4], lgkmcnt [11:8]) waiting for vmcnt <= n only.
constexpr int wait_vmcnt(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
// ... and for lgkmcnt == 0 as well (every LDS access of the wave done).
constexpr int wait_vmcnt_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }

// The tile height of the routed GEMMs of a layer with several M tiles per
// expert, from the experts' rows n_e = offsets[e + 1] - offsets[e]: true
// (288-row tiles) if their gate/up tiles take fewer rounds of the persistent
// grid than 256-row tiles would, a 288-row round weighing 9/8 of a 256-row
// one (its rows).  Rounds = ceil(M tiles x tiles_n / slots).  Every wave
// computes it on its own from the same integers, so all the kernels of a call
// agree.  Mixtral prefill (982-1068 rows per expert): 14 rounds against 16,
// 288; Hunyuan-A13B (Zipf-skewed, 199-6363 rows): 25 against 27, 256.
__device__ __forceinline__ bool tall_tiles_chosen(const int32_t* offsets, int E, int tiles_n, int slots) {
    int t256 = 0, t288 = 0;
    for (int e = (int)(threadIdx.x & 63); e < E; e += 64) {
        const int n = offsets[e + 1] - offsets[e];
        t256 += (n + 255) / 256;
        t288 += (n + 287) / 288;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        t256 += __shfl_xor(t256, o, 64);
        t288 += __shfl_xor(t288, o, 64);
    }
    t256 = __builtin_amdgcn_readfirstlane(t256);
    t288 = __builtin_amdgcn_readfirstlane(t288);
    const int64_t r256 = ((int64_t)t256 * tiles_n + slots - 1) / slots;
    const int64_t r288 = ((int64_t)t288 * tiles_n + slots - 1) / slots;
    return 9 * r288 < 8 * r256;
}

}  // namespace moe
