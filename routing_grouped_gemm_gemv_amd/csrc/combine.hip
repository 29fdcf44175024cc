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
// weights only.  The order-invariant mode forms the same products in float64,
// where they are exact (float32 x bf16 or float32 x float32 needs at most 48
// significant bits), sums them and the shared term in float64 in the same
// order and rounds once; while that sum is exact, every order of the terms
// gives the same bits.  The pass is HBM-bound: each thread streams 16-byte
// chunks of the K expert-output rows of its token.  Every operand is read
// once and the output written once, so all of them bypass the caches
// (non-temporal loads and stores).
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
        const u32x4 u = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
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
        const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
        const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4));
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
};

// Eight consecutive elements loaded raw, so that the loads of all K rows can
// be in flight together, and widened to float32 where they are used.
template <typename Tin>
struct Raw8;
template <>
struct Raw8<uint16_t> {
    u32x4 u;
    static __device__ __forceinline__ Raw8 load(const uint16_t* p) {
        return Raw8{__builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p))};
    }
    static __device__ __forceinline__ Raw8 zero() { return Raw8{u32x4{0u, 0u, 0u, 0u}}; }
    __device__ __forceinline__ void widen(float* v) const {
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    }
};
template <>
struct Raw8<float> {
    f32x4 a, b;
    static __device__ __forceinline__ Raw8 load(const float* p) {
        return Raw8{__builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p)),
                    __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4))};
    }
    static __device__ __forceinline__ Raw8 zero() { return Raw8{f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}}; }
    __device__ __forceinline__ void widen(float* v) const {
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
};

// float64 -> bf16 with one rounding (nearest-even): the float64 value is first
// narrowed to float32 rounding to odd (truncate, then set the last bit if
// anything was dropped), which keeps enough bits that the final float32 ->
// bf16 rounding to nearest-even is the correct rounding of the float64 value.
__device__ __forceinline__ uint16_t f64_to_bf16(double d) {
    float f = static_cast<float>(d);
    if (static_cast<double>(f) != d) {
        uint32_t b = __float_as_uint(f);
        if (fabs(static_cast<double>(f)) > fabs(d)) b -= 1;  // rounded away from zero: step back
        f = __uint_as_float(b | 1u);
    }
    return f32_to_bf16(f);
}

template <bool OUT_BF16>
__device__ __forceinline__ void store8(void* out, int64_t idx, const float (&acc)[8]) {
    if (OUT_BF16) {
        uint32_t pk[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            pk[i] = static_cast<uint32_t>(f32_to_bf16(acc[2 * i])) |
                    (static_cast<uint32_t>(f32_to_bf16(acc[2 * i + 1])) << 16);
        __builtin_nontemporal_store(u32x4{pk[0], pk[1], pk[2], pk[3]},
                                    reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + idx));
    } else {
        float* o = static_cast<float*>(out) + idx;
        __builtin_nontemporal_store(f32x4{acc[0], acc[1], acc[2], acc[3]}, reinterpret_cast<f32x4*>(o));
        __builtin_nontemporal_store(f32x4{acc[4], acc[5], acc[6], acc[7]}, reinterpret_cast<f32x4*>(o + 4));
    }
}

template <bool OUT_BF16>
__device__ __forceinline__ void store8(void* out, int64_t idx, const double (&acc)[8]) {
    if (OUT_BF16) {
        uint32_t pk[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            pk[i] = static_cast<uint32_t>(f64_to_bf16(acc[2 * i])) |
                    (static_cast<uint32_t>(f64_to_bf16(acc[2 * i + 1])) << 16);
        __builtin_nontemporal_store(u32x4{pk[0], pk[1], pk[2], pk[3]},
                                    reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + idx));
    } else {
        float f[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = static_cast<float>(acc[i]);
        float* o = static_cast<float*>(out) + idx;
        __builtin_nontemporal_store(f32x4{f[0], f[1], f[2], f[3]}, reinterpret_cast<f32x4*>(o));
        __builtin_nontemporal_store(f32x4{f[4], f[5], f[6], f[7]}, reinterpret_cast<f32x4*>(o + 4));
    }
}

// Acc: float (the float32 fold) or double (the order-invariant sum)
template <typename Tin, bool OUT_BF16, typename Acc>
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
        Acc acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = Acc(0);
        if (kept) {
#pragma unroll
            for (int j = 0; j < kMaxK; ++j) {
                if (j >= K || pos[j] < 0) continue;
                float v[8];
                Vec8<Tin>::load(y + pos[j] * D + d0, v);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const Acc prod = static_cast<Acc>(wt[j]) * static_cast<Acc>(v[i]);
                    acc[i] = acc[i] + prod;
                }
            }
            if (shared != nullptr) {
                float v[8];
                Vec8<Tin>::load(shared + t * D + d0, v);
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] = acc[i] + static_cast<Acc>(v[i]);
            }
        }
        store8<OUT_BF16>(out, t * D + d0, acc);
    }
}

// The same fold for batches of fewer than kCombineLargeT tokens: all K row
// loads of a 16-byte chunk are issued before the first is used (the kernel
// above waits for each row in turn).  Measured on the workloads' shapes: this
// kernel is faster up to 16384 tokens (4096 x 4096, top-1: 18.5 -> 13.7 us;
// 8192 x 2048, top-8: 56 -> 53 us; 16384 x 2048, top-10: 144 -> 142 us) and
// 2% slower at 32768 x 4096, top-6 (378 -> 386 us), where the kernel above
// stays.  The
// fold runs over KC slots, K rounded up to a compiled size, with weight +0
// and zero data past K and in slots without a row: that adds +0 to an
// accumulator that cannot be -0 (it starts at +0, and round-to-nearest
// returns +0, not -0, for +0 + -0 and for two terms that cancel), so every
// bit is the same as the kernel above, which skips those slots.
constexpr int64_t kCombineLargeT = 16385;

template <typename Tin, bool OUT_BF16, typename Acc, int KC>
__global__ __launch_bounds__(kCombineThreads) void combine_small_kernel(
    const Tin* __restrict__ y, const int32_t* __restrict__ inv_pos, const float* __restrict__ w,
    const Tin* __restrict__ shared, int64_t T, int D, int K, void* __restrict__ out) {
    const int64_t t = blockIdx.x;
    int64_t pos[KC];
    float wt[KC];
    bool kept = false;
#pragma unroll
    for (int j = 0; j < KC; ++j) {
        pos[j] = -1;
        wt[j] = 0.0f;
        if (j < K) {
            pos[j] = inv_pos[t * K + j];
            // a slot without a row (-1) takes weight +0 and zero data below:
            // it adds +0, which leaves the bits of skipping it
            wt[j] = pos[j] >= 0 ? w[t * K + j] : 0.0f;
            kept = kept || pos[j] >= 0;
        }
    }
    for (int d0 = threadIdx.x * 8; d0 < D; d0 += kCombineThreads * 8) {
        Acc acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = Acc(0);
        if (kept) {
            Raw8<Tin> r[KC];
#pragma unroll
            for (int j = 0; j < KC; ++j)
                r[j] = pos[j] >= 0 ? Raw8<Tin>::load(y + pos[j] * D + d0) : Raw8<Tin>::zero();
            const Raw8<Tin> rs = shared != nullptr ? Raw8<Tin>::load(shared + t * D + d0) : Raw8<Tin>::zero();
#pragma unroll
            for (int j = 0; j < KC; ++j) {
                float v[8];
                r[j].widen(v);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const Acc prod = static_cast<Acc>(wt[j]) * static_cast<Acc>(v[i]);
                    acc[i] = acc[i] + prod;
                }
            }
            if (shared != nullptr) {
                float v[8];
                rs.widen(v);
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] = acc[i] + static_cast<Acc>(v[i]);
            }
        }
        store8<OUT_BF16>(out, t * D + d0, acc);
    }
}

// The large-batch fold with bf16 operands and K <= 8: two tokens per
// 256-thread workgroup, 128 threads per token, and each thread takes four
// 16-byte chunks of its token (1024 elements apart) per round, so the K + 1
// row loads of all four chunks are in flight before the first fold.  Slots
// are padded to KC as in combine_small_kernel (weight +0, zero data), which
// leaves every bit of the fold.  At 32768 x 4096, top-6 with a shared expert
// this is 376 -> 361 us against combine_kernel (one token per workgroup,
// rows loaded one after another); one token per 128- or 512-thread
// workgroup, four tokens per workgroup and persistent grids were all slower.
constexpr int kPairTokThreads = 128;  // threads per token
constexpr int kPairChunks = 4;        // 16-byte chunks per thread per round

template <bool OUT_BF16, typename Acc, int KC>
__global__ __launch_bounds__(2 * kPairTokThreads) void combine_pair_kernel(
    const uint16_t* __restrict__ y, const int32_t* __restrict__ inv_pos, const float* __restrict__ w,
    const uint16_t* __restrict__ shared, int64_t T, int D, int K, void* __restrict__ out) {
    // the token of this wave's half (waves 0-1: the first, 2-3: the second),
    // wave-uniform, so its slots come through scalar loads
    const int half = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x)) / kPairTokThreads;
    const int64_t t = 2 * static_cast<int64_t>(blockIdx.x) + half;
    if (t >= T) return;  // the second half of the last workgroup when T is odd
    int64_t pos[KC];
    float wt[KC];
    bool kept = false;
    int32_t p32[KC];
#pragma unroll
    for (int j = 0; j < KC; ++j) {  // unconditional loads (slots past K reread slot K - 1), all in flight together
        const int64_t i = t * K + (j < K ? j : K - 1);
        p32[j] = inv_pos[i];
        wt[j] = w[i];
    }
    __builtin_amdgcn_sched_barrier(0);  // no use of a slot before every slot's loads are issued
#pragma unroll
    for (int j = 0; j < KC; ++j) {
        pos[j] = j < K ? p32[j] : -1;
        wt[j] = pos[j] >= 0 ? wt[j] : 0.0f;
        kept = kept || pos[j] >= 0;
    }
    const int d_lane = (threadIdx.x % kPairTokThreads) * 8;
    for (int base = 0; base < D; base += kPairChunks * kPairTokThreads * 8) {
        Raw8<uint16_t> r[kPairChunks][KC], rs[kPairChunks];
#pragma unroll
        for (int c = 0; c < kPairChunks; ++c) {
            const int d = base + c * kPairTokThreads * 8 + d_lane;
            const bool live = kept && d < D;
#pragma unroll
            for (int j = 0; j < KC; ++j)
                r[c][j] = live && pos[j] >= 0 ? Raw8<uint16_t>::load(y + pos[j] * D + d) : Raw8<uint16_t>::zero();
            rs[c] = live && shared != nullptr ? Raw8<uint16_t>::load(shared + t * D + d) : Raw8<uint16_t>::zero();
        }
#pragma unroll
        for (int c = 0; c < kPairChunks; ++c) {
            const int d = base + c * kPairTokThreads * 8 + d_lane;
            if (d >= D) continue;
            Acc acc[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = Acc(0);
            if (kept) {
#pragma unroll
                for (int j = 0; j < KC; ++j) {
                    float v[8];
                    r[c][j].widen(v);
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const Acc prod = static_cast<Acc>(wt[j]) * static_cast<Acc>(v[i]);
                        acc[i] = acc[i] + prod;
                    }
                }
                if (shared != nullptr) {
                    float v[8];
                    rs[c].widen(v);
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[i] = acc[i] + static_cast<Acc>(v[i]);
                }
            }
            store8<OUT_BF16>(out, t * D + d, acc);
        }
    }
}

template <typename Tin, bool OUT_BF16, typename Acc>
static void launch_combine_t(const void* y, const int32_t* inv_pos, const float* w, const void* shared, int64_t T,
                             int D, int K, void* out, hipStream_t stream) {
    const unsigned grid = static_cast<unsigned>(T);
    const Tin* yy = static_cast<const Tin*>(y);
    const Tin* ss = static_cast<const Tin*>(shared);
    if (T >= kCombineLargeT) {
        if constexpr (sizeof(Tin) == 2) {
            if (K <= 8) {
                const unsigned g2 = static_cast<unsigned>((T + 1) / 2);
#define MOE_COMBINE_PAIR(KC) \
    combine_pair_kernel<OUT_BF16, Acc, KC><<<g2, 2 * kPairTokThreads, 0, stream>>>(yy, inv_pos, w, ss, T, D, K, out)
                if (K <= 1) MOE_COMBINE_PAIR(1);
                else if (K <= 2) MOE_COMBINE_PAIR(2);
                else if (K <= 4) MOE_COMBINE_PAIR(4);
                else if (K <= 6) MOE_COMBINE_PAIR(6);
                else MOE_COMBINE_PAIR(8);
#undef MOE_COMBINE_PAIR
                return;
            }
        }
        combine_kernel<Tin, OUT_BF16, Acc><<<grid, kCombineThreads, 0, stream>>>(yy, inv_pos, w, ss, T, D, K, out);
        return;
    }
#define MOE_COMBINE_SMALL(KC) \
    combine_small_kernel<Tin, OUT_BF16, Acc, KC><<<grid, kCombineThreads, 0, stream>>>(yy, inv_pos, w, ss, T, D, K, out)
    if (K <= 1) MOE_COMBINE_SMALL(1);
    else if (K <= 2) MOE_COMBINE_SMALL(2);
    else if (K <= 4) MOE_COMBINE_SMALL(4);
    else if (K <= 6) MOE_COMBINE_SMALL(6);
    else if (K <= 8) MOE_COMBINE_SMALL(8);
    else if (K <= 10) MOE_COMBINE_SMALL(10);
    else if (K <= 12) MOE_COMBINE_SMALL(12);
    else MOE_COMBINE_SMALL(kMaxK);
#undef MOE_COMBINE_SMALL
}

hipError_t launch_combine(const void* y, const int32_t* inv_pos, const float* w, const void* shared,
                          int64_t T, int D, int K, int dtype, int out_dtype, int mode, void* out, hipStream_t stream) {
#define MOE_COMBINE(TIN, BF16OUT, ACC) launch_combine_t<TIN, BF16OUT, ACC>(y, inv_pos, w, shared, T, D, K, out, stream)
    if (dtype == 0) {
        if (mode == 0) {
            if (out_dtype == 0) MOE_COMBINE(uint16_t, true, float);
            else MOE_COMBINE(uint16_t, false, float);
        } else {
            if (out_dtype == 0) MOE_COMBINE(uint16_t, true, double);
            else MOE_COMBINE(uint16_t, false, double);
        }
    } else {
        if (mode == 0) {
            if (out_dtype == 0) MOE_COMBINE(float, true, float);
            else MOE_COMBINE(float, false, float);
        } else {
            if (out_dtype == 0) MOE_COMBINE(float, true, double);
            else MOE_COMBINE(float, false, double);
        }
    }
#undef MOE_COMBINE
    return hipGetLastError();
}

}  // namespace moe
