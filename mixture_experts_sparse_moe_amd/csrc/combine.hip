// Gate-weighted combine back into token order ("8.6 Mixture of Experts" sec.
// 2, boxed MoE(x) = sum_e g_e f_e(x); sec. 4.1 adds the shared expert with
// weight 1):
//   y[t] = sum_{j<k} w[t,j] * expert_out[pair_pos[t*k + j]]  (+ shared[t])
// One workgroup per token row, fp32 sums in slot order j = 0..k-1, then the
// shared row, then rounding.  Each y row is written exactly once: no atomics,
// deterministic.  bf16 rows move as 16-byte vectors (8 elements per lane).
// When the down projection was computed in K ranges, expert_out (and shared)
// hold one bf16 slice per range; a row is the fp32 sum of its slices in slice
// order, taken before the gate weight.
#include "device_util.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kThreads = 256;

// 8 bf16 elements at p, summed in fp32 over `slices` slices `stride` apart.
__device__ __forceinline__ void load_row_sum(const uint16_t* p, int slices, int64_t stride, float* r) {
    const uint4 q = *reinterpret_cast<const uint4*>(p);
    const uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r[2 * i] = bf16_to_f32((uint16_t)(u[i] & 0xFFFF));
        r[2 * i + 1] = bf16_to_f32((uint16_t)(u[i] >> 16));
    }
    for (int sl = 1; sl < slices; ++sl) {
        const uint4 e = *reinterpret_cast<const uint4*>(p + sl * stride);
        const uint32_t w[4] = {e.x, e.y, e.z, e.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            r[2 * i] += bf16_to_f32((uint16_t)(w[i] & 0xFFFF));
            r[2 * i + 1] += bf16_to_f32((uint16_t)(w[i] >> 16));
        }
    }
}

__global__ __launch_bounds__(kThreads) void combine_bf16_kernel(CombineArgs a) {
    const int t = blockIdx.x;
    __shared__ int s_pos[16];
    __shared__ float s_w[16];
    if (threadIdx.x < a.k) {
        s_pos[threadIdx.x] = a.pair_pos[(int64_t)t * a.k + threadIdx.x];
        s_w[threadIdx.x] = a.weights[(int64_t)t * a.k + threadIdx.x];
    }
    __syncthreads();
    const uint16_t* O = static_cast<const uint16_t*>(a.expert_out);
    const uint16_t* S = static_cast<const uint16_t*>(a.shared);
    uint16_t* Y = static_cast<uint16_t*>(a.y);
    const int nvec = a.d / 8;
    for (int v = threadIdx.x; v < nvec; v += kThreads) {
        float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int j = 0; j < a.k; ++j) {
            float row[8];
            load_row_sum(O + (int64_t)s_pos[j] * a.d + v * 8, a.splitk, a.part_stride, row);
            const float wj = s_w[j];
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = fmaf(wj, row[i], acc[i]);
        }
        if (S) {
            float row[8];
            load_row_sum(S + (int64_t)t * a.d + v * 8, a.shared_splitk, a.shared_stride, row);
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] += row[i];
        }
        uint4 o;
        o.x = pack_bf16x2(acc[0], acc[1]);
        o.y = pack_bf16x2(acc[2], acc[3]);
        o.z = pack_bf16x2(acc[4], acc[5]);
        o.w = pack_bf16x2(acc[6], acc[7]);
        *reinterpret_cast<uint4*>(Y + (int64_t)t * a.d + v * 8) = o;
    }
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
            acc = fmaf(a.weights[(int64_t)t * a.k + j], O[(int64_t)pos * a.d + c], acc);
        }
        if (S) acc += S[(int64_t)t * a.d + c];
        Y[(int64_t)t * a.d + c] = acc;
    }
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, bool bf16, hipStream_t s) {
    if (a.T == 0) return hipSuccess;
    if (bf16) hipLaunchKernelGGL(combine_bf16_kernel, dim3(a.T), dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL(combine_f32_kernel, dim3(a.T), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
