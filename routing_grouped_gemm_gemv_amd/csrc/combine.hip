// Weighted combine: the final reduction of the layer.
//
// The RL-Kernel roadmap ("DSV4 Flash MoE Train-Inference Consistency
// Roadmap", Problem 3: Final Reduction Is The Core Drift Point) makes the
// combine order, accumulator dtype and downcast point part of the contract,
// and arXiv 2607.28097 ("From Expert Reduction to Behavioral Divergence",
// Abstract) shows that operand conversion, accumulator precision and
// reduction order each change observable results.  This kernel fixes all
// three: for every kept token and hidden element,
//     acc = +0.0f
//     acc = fl32(acc + fl32(w_j * f32(y_j)))   for j in ascending expert id
//     acc = fl32(acc + f32(shared))            if a shared expert is present
//     out = bf16_rne(acc)  or  acc
// with every multiply and add rounded on its own (contraction to FMA is off
// for this file), so the result is a function of the K expert outputs and
// weights only.  The pass is HBM-bound: each thread streams 16-byte chunks of
// the K expert-output rows of its token.
#include "common.hpp"
#include "kernels.hpp"

#pragma clang fp contract(off)

namespace moe {

constexpr int kCombineThreads = 256;
constexpr int kMaxK = 16;

template <typename Tin>
struct Vec8;
template <>
struct Vec8<uint16_t> {
    static __device__ __forceinline__ void load(const uint16_t* p, float* v) {
        const u32x4 u = *reinterpret_cast<const u32x4*>(p);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    }
};
template <>
struct Vec8<float> {
    static __device__ __forceinline__ void load(const float* p, float* v) {
        const float4 a = *reinterpret_cast<const float4*>(p);
        const float4 b = *reinterpret_cast<const float4*>(p + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
};

template <typename Tin, bool OUT_BF16>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const Tin* __restrict__ y, const int32_t* __restrict__ inv_pos, const float* __restrict__ w,
    const Tin* __restrict__ shared, int64_t T, int D, int K, void* __restrict__ out) {
    const int64_t t = blockIdx.x;
    int64_t pos[kMaxK];
    float wt[kMaxK];
    bool kept = false;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
        pos[j] = -1;
        wt[j] = 0.0f;
        if (j < K) {
            pos[j] = inv_pos[t * K + j];
            wt[j] = w[t * K + j];
            kept = kept || pos[j] >= 0;
        }
    }
    for (int d0 = threadIdx.x * 8; d0 < D; d0 += kCombineThreads * 8) {
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
        if (kept) {
#pragma unroll
            for (int j = 0; j < kMaxK; ++j) {
                if (j >= K || pos[j] < 0) continue;
                float v[8];
                Vec8<Tin>::load(y + pos[j] * D + d0, v);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float prod = wt[j] * v[i];
                    acc[i] = acc[i] + prod;
                }
            }
            if (shared != nullptr) {
                float v[8];
                Vec8<Tin>::load(shared + t * D + d0, v);
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] = acc[i] + v[i];
            }
        }
        if (OUT_BF16) {
            uint32_t pk[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                pk[i] = static_cast<uint32_t>(f32_to_bf16(acc[2 * i])) |
                        (static_cast<uint32_t>(f32_to_bf16(acc[2 * i + 1])) << 16);
            *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + t * D + d0) = u32x4{pk[0], pk[1], pk[2], pk[3]};
        } else {
            float* o = static_cast<float*>(out) + t * D + d0;
            *reinterpret_cast<float4*>(o) = make_float4(acc[0], acc[1], acc[2], acc[3]);
            *reinterpret_cast<float4*>(o + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
        }
    }
}

hipError_t launch_combine(const void* y, const int32_t* inv_pos, const float* w, const void* shared,
                          int64_t T, int D, int K, int dtype, int out_dtype, void* out, hipStream_t stream) {
    const unsigned grid = static_cast<unsigned>(T);
    if (dtype == 0) {
        const uint16_t* yy = static_cast<const uint16_t*>(y);
        const uint16_t* ss = static_cast<const uint16_t*>(shared);
        if (out_dtype == 0) combine_kernel<uint16_t, true><<<grid, kCombineThreads, 0, stream>>>(yy, inv_pos, w, ss, T, D, K, out);
        else combine_kernel<uint16_t, false><<<grid, kCombineThreads, 0, stream>>>(yy, inv_pos, w, ss, T, D, K, out);
    } else {
        const float* yy = static_cast<const float*>(y);
        const float* ss = static_cast<const float*>(shared);
        if (out_dtype == 0) combine_kernel<float, true><<<grid, kCombineThreads, 0, stream>>>(yy, inv_pos, w, ss, T, D, K, out);
        else combine_kernel<float, false><<<grid, kCombineThreads, 0, stream>>>(yy, inv_pos, w, ss, T, D, K, out);
    }
    return hipGetLastError();
}

}  // namespace moe
