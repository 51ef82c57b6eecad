// Gate-weighted combine back into token order ("8.6 Mixture of Experts" sec.
// 2, boxed MoE(x) = sum_e g_e f_e(x); sec. 4.1 adds the shared expert with
// weight 1):
//   y[t] = sum_{j<k} w[t,j] * expert_out[pair_pos[t*k + j]]  (+ shared[t])
// One workgroup per token row (and, in bf16, per 2048 columns), fp32 sums in
// slot order j = 0..k-1, then the shared row, then rounding.  Each y row is
// written exactly once: no atomics, deterministic.  bf16 rows move as 16-byte
// vectors (8 elements per lane).
// When the down projection was computed in K ranges, expert_out (and shared)
// hold one bf16 slice per range; a row is the fp32 sum of its slices in slice
// order, taken before the gate weight.  A pair with pair_pos -1 (dropped for
// capacity, "8.6 Mixture of Experts", sec. 3.2) contributes nothing.
#include "device_util.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kThreads = 256;

// expert_out, the shared rows and y are each touched once: non-temporal
// 16-byte loads and stores, which keep them from displacing other lines in
// the caches (DeepSeek-V3 combine 238 -> 211 us, Hunyuan-A13B 117 -> 101 us)
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_nt16(const uint16_t* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void store_nt16(uint16_t* p, uint4 q) {
    u32x4_t v;
    v.x = q.x;
    v.y = q.y;
    v.z = q.z;
    v.w = q.w;
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
}

__device__ __forceinline__ void add_bf16x8(uint4 q, float* r) {
    const uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r[2 * i] += bf16_to_f32((uint16_t)(u[i] & 0xFFFF));
        r[2 * i + 1] += bf16_to_f32((uint16_t)(u[i] >> 16));
    }
}

// 8 bf16 elements at p, summed in fp32 over `slices` slices `stride` apart
// (slice order).
__device__ __forceinline__ void load_row_sum(const uint16_t* p, int slices, int64_t stride, float* r) {
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = 0.0f;
    for (int sl = 0; sl < slices; ++sl) add_bf16x8(load_nt16(p + sl * stride), r);
}

// Workgroup (t, c): token t, vectors c*256 .. c*256 + 255 of 8 elements.  The
// loads of JB = 8 / S rows' slices are issued together, then added in the
// fixed order: slices of a row in slice order, rows in slot order.
template <int S>
__global__ __launch_bounds__(kThreads) void combine_bf16_kernel(CombineArgs a) {
    constexpr int JB = 8 / S;
    // launched beside the combine of the other tile height's K split: run only
    // if the device-side choice of the routed GEMMs' tile height is this one
    if (a.choice.offsets &&
        tall_tiles_chosen(a.choice.offsets, a.choice.E, a.choice.tiles_n, a.choice.slots) != (a.choice.rows == 288))
        return;
    const int t = blockIdx.x;
    __shared__ int s_pos[16];
    __shared__ float s_w[16];
    if (threadIdx.x < a.k) {
        s_pos[threadIdx.x] = a.pair_pos[(int64_t)t * a.k + threadIdx.x];
        s_w[threadIdx.x] = a.weights[(int64_t)t * a.k + threadIdx.x];
    }
    __syncthreads();
    const uint16_t* O = static_cast<const uint16_t*>(a.expert_out);
    const uint16_t* Sh = static_cast<const uint16_t*>(a.shared);
    uint16_t* Y = static_cast<uint16_t*>(a.y);
    const int v = blockIdx.y * kThreads + threadIdx.x;
    if (v >= a.d / 8) return;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int j0 = 0; j0 < a.k; j0 += JB) {
        uint4 q[JB][S];
#pragma unroll
        for (int jj = 0; jj < JB; ++jj)
#pragma unroll
            for (int sl = 0; sl < S; ++sl)
                if (j0 + jj < a.k && s_pos[j0 + jj] >= 0)
                    q[jj][sl] = load_nt16(O + sl * a.part_stride + (int64_t)s_pos[j0 + jj] * a.d + v * 8);
#pragma unroll
        for (int jj = 0; jj < JB; ++jj) {
            if (j0 + jj >= a.k) break;
            if (s_pos[j0 + jj] < 0) continue;       // dropped for capacity: contributes nothing
            float row[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
            for (int sl = 0; sl < S; ++sl) add_bf16x8(q[jj][sl], row);
            const float wj = s_w[j0 + jj];
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = fmaf(wj, row[i], acc[i]);
        }
    }
    if (Sh) {
        float row[8];
        load_row_sum(Sh + (int64_t)t * a.d + v * 8, a.shared_splitk, a.shared_stride, row);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += row[i];
    }
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    store_nt16(Y + (int64_t)t * a.d + v * 8, o);
}

__global__ __launch_bounds__(kThreads) void combine_f32_kernel(CombineArgs a) {
    const int t = blockIdx.x;
    const float* O = static_cast<const float*>(a.expert_out);
    const float* S = static_cast<const float*>(a.shared);
    float* Y = static_cast<float*>(a.y);
    for (int c = threadIdx.x; c < a.d; c += kThreads) {
        float acc = 0.0f;
        for (int j = 0; j < a.k; ++j) {
            const int pos = a.pair_pos[(int64_t)t * a.k + j];
            if (pos < 0) continue;                  // dropped for capacity
            acc = fmaf(a.weights[(int64_t)t * a.k + j], O[(int64_t)pos * a.d + c], acc);
        }
        if (S) acc += S[(int64_t)t * a.d + c];
        Y[(int64_t)t * a.d + c] = acc;
    }
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, bool bf16, hipStream_t s) {
    if (a.T == 0) return hipSuccess;
    if (!bf16) {
        hipLaunchKernelGGL(combine_f32_kernel, dim3(a.T), dim3(kThreads), 0, s, a);
        return hipGetLastError();
    }
    const dim3 grid(a.T, (a.d / 8 + kThreads - 1) / kThreads);
    switch (a.splitk) {
        case 1: hipLaunchKernelGGL(combine_bf16_kernel<1>, grid, dim3(kThreads), 0, s, a); break;
        case 2: hipLaunchKernelGGL(combine_bf16_kernel<2>, grid, dim3(kThreads), 0, s, a); break;
        case 4: hipLaunchKernelGGL(combine_bf16_kernel<4>, grid, dim3(kThreads), 0, s, a); break;
        case 8: hipLaunchKernelGGL(combine_bf16_kernel<8>, grid, dim3(kThreads), 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace moe
