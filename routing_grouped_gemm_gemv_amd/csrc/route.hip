// Routing: router logits, scores, selection bias, top-k ids and weights.
//
// What is computed follows the RL-Kernel roadmap "DSV4 Flash MoE
// Train-Inference Consistency Roadmap" (Problem 1: Routing Is A Discrete
// Decision: logits from hidden states, score, top-k with an explicit
// tie-break) and the router commit notes of SpecForge pull request #1003
// (a selection bias shifts only which experts are picked; the weights come
// from the unbiased scores; weights renormalised unless disabled, then scaled
// by route_scale).
//
// Precision: a top-k decision is discrete, so the logits are accumulated far
// more accurately than the score margins that decide it.  In bf16 mode the
// GEMM runs on MFMA with fp32 accumulation over chunks of 64 products, and the
// chunk sums are added in float64; in fp32 mode each logit is a float64 FMA
// chain (the fp32 x fp32 products are exact in float64).  Scores, choices and
// weights are then float64; the weights are rounded once to float32.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// ---------------------------------------------------------------------------
// router logits, bf16 operands: 64 tokens x 64 experts per workgroup
// ---------------------------------------------------------------------------
constexpr int kRtTok = 64;
constexpr int kRtExp = 64;
constexpr int kRtK = 64;  // k per chunk: fp32 partial sums of 64 products, then float64

__global__ __launch_bounds__(256) void router_logits_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int64_t T, int D, int E,
    double* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) uint8_t sx[kRtTok * 128];
    __shared__ __attribute__((aligned(16))) uint8_t sw[kRtExp * 128];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kRtTok;
    const int e0 = blockIdx.y * kRtExp;

    double acc64[4][4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc64[nb][i] = 0.0;

    for (int k0 = 0; k0 < D; k0 += kRtK) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int row = p * 32 + (tid >> 3);
            const int ch = tid & 7;
            u32x4 vx = u32x4{0u, 0u, 0u, 0u};
            u32x4 vw = u32x4{0u, 0u, 0u, 0u};
            const int64_t tr = t0 + row;
            if (tr < T) vx = *reinterpret_cast<const u32x4*>(x + tr * D + k0 + ch * 8);
            const int er = e0 + row;
            if (er < E) vw = *reinterpret_cast<const u32x4*>(w + static_cast<int64_t>(er) * D + k0 + ch * 8);
            const int off = row * 128 + ((ch ^ (row & 7)) << 4);
            *reinterpret_cast<u32x4*>(sx + off) = vx;
            *reinterpret_cast<u32x4*>(sw + off) = vw;
        }
        __syncthreads();
        f32x4 acc[4];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int ch = 4 * s + (lane >> 4);
            const int ar = wv * 16 + (lane & 15);
            const u32x4 a = *reinterpret_cast<const u32x4*>(sx + ar * 128 + ((ch ^ (ar & 7)) << 4));
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                const int br = nb * 16 + (lane & 15);
                const u32x4 b = *reinterpret_cast<const u32x4*>(sw + br * 128 + ((ch ^ (br & 7)) << 4));
                acc[nb] = mfma_bf16(a, b, acc[nb]);
            }
        }
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc64[nb][i] += static_cast<double>(acc[nb][i]);
        __syncthreads();
    }
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
        const int e = e0 + nb * 16 + (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t t = t0 + wv * 16 + 4 * (lane >> 4) + i;
            if (t < T && e < E) out[t * E + e] = acc64[nb][i];
        }
    }
}

// ---------------------------------------------------------------------------
// router logits, fp32 operands: float64 FMA chains, 16 tokens x 16 experts
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void router_logits_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ w, int64_t T, int D, int E,
    double* __restrict__ out) {
    __shared__ float sx[16][65];
    __shared__ float sw[16][65];
    const int tid = threadIdx.x;
    const int ty = tid >> 4, tx = tid & 15;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * 16;
    const int e0 = blockIdx.y * 16;
    double acc = 0.0;
    for (int k0 = 0; k0 < D; k0 += 64) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int idx = tid + 256 * q;
            const int r = idx >> 6, c = idx & 63;
            sx[r][c] = (t0 + r < T) ? x[(t0 + r) * D + k0 + c] : 0.f;
            sw[r][c] = (e0 + r < E) ? w[static_cast<int64_t>(e0 + r) * D + k0 + c] : 0.f;
        }
        __syncthreads();
#pragma unroll 8
        for (int c = 0; c < 64; ++c)
            acc = fma(static_cast<double>(sx[ty][c]), static_cast<double>(sw[tx][c]), acc);
        __syncthreads();
    }
    const int64_t t = t0 + ty;
    const int e = e0 + tx;
    if (t < T && e < E) out[t * E + e] = acc;
}

// ---------------------------------------------------------------------------
// scores + selection bias + wavefront top-k + weights: one wave per token
// ---------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
    const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(v)), CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(v >> 32)), CTRL, 0xF, 0xF, false);
    return (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo);
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
    const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v)), l);
    const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v >> 32)), l);
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ double readlane_f64(double v, int l) {
    return __longlong_as_double(static_cast<long long>(readlane_u64(static_cast<uint64_t>(__double_as_longlong(v)), l)));
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Maximum over the wave.  Within each row of 16 lanes: quad_perm [1,0,3,2] and
// [2,3,0,1] make every quad uniform, row_half_mirror pairs each quad with the
// other quad of its half-row and row_mirror pairs the two half-rows.  The four
// row results are then combined through readlane, so the result is uniform.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t k) {
    k = umax64(k, dpp_u64<0xB1>(k));   // quad_perm(1,0,3,2)
    k = umax64(k, dpp_u64<0x4E>(k));   // quad_perm(2,3,0,1)
    k = umax64(k, dpp_u64<0x141>(k));  // row_half_mirror
    k = umax64(k, dpp_u64<0x140>(k));  // row_mirror
    return umax64(umax64(readlane_u64(k, 0), readlane_u64(k, 16)),
                  umax64(readlane_u64(k, 32), readlane_u64(k, 48)));
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
    return __longlong_as_double(static_cast<long long>(dpp_u64<CTRL>(static_cast<uint64_t>(__double_as_longlong(v)))));
}

__device__ __forceinline__ double wave_max_f64(double v) {
    v = fmax(v, dpp_f64<0xB1>(v));
    v = fmax(v, dpp_f64<0x4E>(v));
    v = fmax(v, dpp_f64<0x141>(v));
    v = fmax(v, dpp_f64<0x140>(v));
    return fmax(fmax(readlane_f64(v, 0), readlane_f64(v, 16)), fmax(readlane_f64(v, 32), readlane_f64(v, 48)));
}

// Sum over the wave in one fixed order; every lane ends with the same bits.
__device__ __forceinline__ double wave_sum_f64(double v) {
    v = v + dpp_f64<0xB1>(v);
    v = v + dpp_f64<0x4E>(v);
    v = v + dpp_f64<0x141>(v);
    v = v + dpp_f64<0x140>(v);
    return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

// Key ordering (choice descending, id ascending) as one unsigned integer:
// the order-preserving image of the float64 choice (with -0 taken as +0),
// its low 10 bits replaced by 1023 - id.  Equal choices therefore compare by
// id, lowest first.  Choices that differ only below the 42nd significant bit
// (relative 2^-42) also compare by id; such margins are far below both the
// accuracy of the logits and the near-tie exemption.  0 is never a valid key.
__device__ __forceinline__ uint64_t choice_key(double c, int e) {
    if (c == 0.0) c = 0.0;
    const uint64_t b = static_cast<uint64_t>(__double_as_longlong(c));
    const uint64_t ord = (b >> 63) ? ~b : (b | 0x8000000000000000ull);
    return (ord & ~0x3FFull) | static_cast<uint64_t>(1023 - e);
}

// Scores, choice and weights of one token whose float64 logits the wave holds,
// E/64 (rounded up) per lane: lane l holds experts l, l + 64, ...  Writes the
// K ids in ascending order and their weights (ids -1, weights 0 if masked).
template <int EPL>
__device__ __forceinline__ void topk_token(const double (&lg)[EPL], int64_t t, int E, int K, int score,
                                           int renorm, double route_scale, const float* __restrict__ bias,
                                           bool kept, int32_t* __restrict__ ids_out, float* __restrict__ w_out) {
    const int lane = lane_id();
    if (!kept) {
        if (lane < K) {
            ids_out[t * K + lane] = -1;
            w_out[t * K + lane] = 0.f;
        }
        return;
    }
    bool ok[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) ok[i] = lane + 64 * i < E;

    double s[EPL];
    if (score == 0) {  // softmax over the experts
        double m = -1.7976931348623157e308;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (ok[i]) m = fmax(m, lg[i]);
        m = wave_max_f64(m);
        double part = 0.0;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            s[i] = ok[i] ? exp(lg[i] - m) : 0.0;
            part += s[i];
        }
        const double z = wave_sum_f64(part);
#pragma unroll
        for (int i = 0; i < EPL; ++i) s[i] = s[i] / z;
    } else {  // logistic sigmoid of each logit
#pragma unroll
        for (int i = 0; i < EPL; ++i) s[i] = ok[i] ? 1.0 / (1.0 + exp(-lg[i])) : 0.0;
    }

    uint64_t key[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        double c = s[i];
        if (bias != nullptr && ok[i]) c += static_cast<double>(bias[e]);
        key[i] = ok[i] ? choice_key(c, e) : 0ull;
    }

    // K rounds of wave argmax; lane r keeps the r-th pick
    int my_e = -1;
    double my_s = 0.0;
    for (int r = 0; r < K; ++r) {
        uint64_t best = key[0];
#pragma unroll
        for (int i = 1; i < EPL; ++i) best = umax64(best, key[i]);
        const uint64_t win = wave_max_u64(best);
        const int ew = 1023 - static_cast<int>(win & 0x3FFull);
        const int owner = ew & 63;
        const int slot = ew >> 6;
        double sw = 0.0;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            if (lane == owner && i == slot) {
                sw = s[i];
                key[i] = 0ull;
            }
        }
        sw = readlane_f64(sw, owner);
        if (lane == r) {
            my_e = ew;
            my_s = sw;
        }
    }

    // ascending id order: rank of each pick among the K picks (ids are distinct)
    int rank = 0;
    for (int i = 0; i < K; ++i) {
        const int ei = __builtin_amdgcn_readlane(my_e, i);
        rank += (lane < K && ei < my_e) ? 1 : 0;
    }
    double den = 1.0;
    if (renorm) {
        den = 0.0;
        for (int r = 0; r < K; ++r) {
            const uint64_t holder_mask = __ballot(lane < K && rank == r);
            const int holder = __builtin_ctzll(holder_mask);
            den += readlane_f64(my_s, holder);
        }
    }
    if (lane < K) {
        const double wv = renorm ? (my_s / den) * route_scale : my_s * route_scale;
        ids_out[t * K + rank] = my_e;
        w_out[t * K + rank] = static_cast<float>(wv);
    }
}

template <int EPL>
__global__ __launch_bounds__(256) void topk_kernel(
    const double* __restrict__ logits, int64_t T, int E, int K, int score, int renorm,
    double route_scale, const float* __restrict__ bias, const uint8_t* __restrict__ mask,
    float* __restrict__ logits_out, int32_t* __restrict__ ids_out, float* __restrict__ w_out) {
    const int lane = lane_id();
    const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (t >= T) return;  // uniform per wave

    double lg[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        lg[i] = e < E ? logits[t * E + e] : 0.0;
        if (logits_out && e < E) logits_out[t * E + e] = static_cast<float>(lg[i]);
    }
    const bool kept = (mask == nullptr) || (mask[t] != 0);
    topk_token<EPL>(lg, t, E, K, score, renorm, route_scale, bias, kept, ids_out, w_out);
}

// ---------------------------------------------------------------------------
// fused routing, bf16 operands: logits of TB tokens x all experts in one
// workgroup, kept in LDS as float64, then top-k per token from LDS.
// The hidden rows are read from memory once and the logits never leave the
// chip.  Each logit is computed exactly as router_logits_bf16_kernel does
// (two MFMA k=32 steps into a zeroed fp32 accumulator per 64-wide k chunk,
// chunks added in float64 in k order), so both paths give the same bits.
// ---------------------------------------------------------------------------
// TBB: 16-token blocks per workgroup; NBW: 16-expert blocks per wave (4 waves).
template <int TBB, int NBW>
struct RouteTile {
    static constexpr int TB = 16 * TBB;        // tokens per workgroup
    static constexpr int EMAX = 64 * NBW;      // experts per workgroup
    static constexpr int EPL = EMAX / 64;      // experts per lane in the top-k
    static constexpr int ROWS = TB + EMAX;     // rows staged per 64-wide k chunk
    static constexpr int STAGE = ROWS * 128;   // bytes per chunk
    static constexpr int LOGB = TB * EMAX * 8; // float64 logits
    static constexpr int SMEM = (2 * STAGE > LOGB) ? 2 * STAGE : LOGB;
    static constexpr int LOADS = ROWS * 8 / 256;  // 16-byte loads per thread per chunk
    static_assert(ROWS % 32 == 0, "staging must divide over 256 threads");
};

template <int TBB, int NBW>
__global__ __launch_bounds__(256) void route_fused_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int64_t T, int D, int E, int K,
    int score, int renorm, double route_scale, const float* __restrict__ bias,
    const uint8_t* __restrict__ mask, float* __restrict__ logits_out, int32_t* __restrict__ ids_out,
    float* __restrict__ w_out) {
    using RT = RouteTile<TBB, NBW>;
    __shared__ __attribute__((aligned(16))) uint8_t smem[RT::SMEM];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * RT::TB;

    // staging: row r < TB is hidden row t0 + r, row TB + j is router row j
    const uint8_t* src[RT::LOADS];
    int dst[RT::LOADS];
#pragma unroll
    for (int j = 0; j < RT::LOADS; ++j) {
        const int q = tid + 256 * j;
        const int row = q >> 3, ch = q & 7;
        dst[j] = row * 128 + ((ch ^ (row & 7)) << 4);
        const uint8_t* p = nullptr;
        if (row < RT::TB) {
            if (t0 + row < T) p = reinterpret_cast<const uint8_t*>(x + (t0 + row) * D) + ch * 16;
        } else if (row - RT::TB < E) {
            p = reinterpret_cast<const uint8_t*>(w + static_cast<int64_t>(row - RT::TB) * D) + ch * 16;
        }
        src[j] = p;
    }
    u32x4 stg[RT::LOADS];
    auto fetch = [&](int k0) {
#pragma unroll
        for (int j = 0; j < RT::LOADS; ++j)
            stg[j] = src[j] ? *reinterpret_cast<const u32x4*>(src[j] + 2 * k0) : u32x4{0u, 0u, 0u, 0u};
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int j = 0; j < RT::LOADS; ++j)
            *reinterpret_cast<u32x4*>(smem + buf * RT::STAGE + dst[j]) = stg[j];
    };

    double acc64[TBB][NBW][4];
#pragma unroll
    for (int a = 0; a < TBB; ++a)
#pragma unroll
        for (int b = 0; b < NBW; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc64[a][b][i] = 0.0;

    const int nchunks = D / 64;
    fetch(0);
    store(0);
    __syncthreads();
    for (int c = 0; c < nchunks; ++c) {
        const int buf = c & 1;
        if (c + 1 < nchunks) fetch((c + 1) * 64);
        const uint8_t* sb = smem + buf * RT::STAGE;
        f32x4 acc[TBB][NBW];
#pragma unroll
        for (int a = 0; a < TBB; ++a)
#pragma unroll
            for (int b = 0; b < NBW; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int ch = 4 * s + (lane >> 4);
            u32x4 af[TBB];
#pragma unroll
            for (int a = 0; a < TBB; ++a) {
                const int r = a * 16 + (lane & 15);
                af[a] = *reinterpret_cast<const u32x4*>(sb + r * 128 + ((ch ^ (r & 7)) << 4));
            }
#pragma unroll
            for (int b = 0; b < NBW; ++b) {
                const int r = RT::TB + wv * (16 * NBW) + b * 16 + (lane & 15);
                const u32x4 bf = *reinterpret_cast<const u32x4*>(sb + r * 128 + ((ch ^ (r & 7)) << 4));
#pragma unroll
                for (int a = 0; a < TBB; ++a) acc[a][b] = mfma_bf16(af[a], bf, acc[a][b]);
            }
        }
#pragma unroll
        for (int a = 0; a < TBB; ++a)
#pragma unroll
            for (int b = 0; b < NBW; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc64[a][b][i] += static_cast<double>(acc[a][b][i]);
        if (c + 1 < nchunks) store(buf ^ 1);
        __syncthreads();
    }

    // logits to LDS: [TB][EMAX] float64 (the staging buffers are dead)
    double* lgs = reinterpret_cast<double*>(smem);
#pragma unroll
    for (int a = 0; a < TBB; ++a)
#pragma unroll
        for (int b = 0; b < NBW; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tl = a * 16 + 4 * (lane >> 4) + i;
                const int e = wv * (16 * NBW) + b * 16 + (lane & 15);
                lgs[tl * RT::EMAX + e] = acc64[a][b][i];
            }
    __syncthreads();

    for (int tl = wv; tl < RT::TB; tl += 4) {
        const int64_t t = t0 + tl;
        if (t >= T) break;  // uniform per wave
        double lg[RT::EPL];
#pragma unroll
        for (int i = 0; i < RT::EPL; ++i) {
            const int e = lane + 64 * i;
            lg[i] = lgs[tl * RT::EMAX + e];
            if (logits_out && e < E) logits_out[t * E + e] = static_cast<float>(lg[i]);
        }
        const bool kept = (mask == nullptr) || (mask[t] != 0);
        topk_token<RT::EPL>(lg, t, E, K, score, renorm, route_scale, bias, kept, ids_out, w_out);
    }
}

hipError_t launch_router_logits(const void* x, const void* router, int64_t T, int D, int E,
                                int dtype, double* logits64, hipStream_t stream) {
    if (dtype == 0) {
        dim3 grid(static_cast<unsigned>((T + kRtTok - 1) / kRtTok), static_cast<unsigned>((E + kRtExp - 1) / kRtExp));
        router_logits_bf16_kernel<<<grid, 256, 0, stream>>>(static_cast<const uint16_t*>(x),
                                                            static_cast<const uint16_t*>(router), T, D, E, logits64);
    } else {
        dim3 grid(static_cast<unsigned>((T + 15) / 16), static_cast<unsigned>((E + 15) / 16));
        router_logits_f32_kernel<<<grid, 256, 0, stream>>>(static_cast<const float*>(x),
                                                           static_cast<const float*>(router), T, D, E, logits64);
    }
    return hipGetLastError();
}

hipError_t launch_topk(const double* logits64, int64_t T, int E, int K, int score, int renorm,
                       float route_scale, const float* bias, const uint8_t* mask,
                       float* logits_out, int32_t* ids, float* w, hipStream_t stream) {
    const unsigned grid = static_cast<unsigned>((T + 3) / 4);
    const double rs = static_cast<double>(route_scale);
#define MOE_TOPK(EPL)                                                                                   \
    topk_kernel<EPL><<<grid, 256, 0, stream>>>(logits64, T, E, K, score, renorm, rs, bias, mask, \
                                                logits_out, ids, w)
    if (E <= 64) MOE_TOPK(1);
    else if (E <= 128) MOE_TOPK(2);
    else if (E <= 256) MOE_TOPK(4);
    else if (E <= 512) MOE_TOPK(8);
    else MOE_TOPK(16);
#undef MOE_TOPK
    return hipGetLastError();
}

bool route_fused(int E, int dtype) { return dtype == 0 && E <= 512; }

hipError_t launch_route(const void* x, const void* router, int64_t T, int D, int E, int K, int dtype,
                        int score, int renorm, float route_scale, const float* bias, const uint8_t* mask,
                        double* logits64, float* logits_out, int32_t* ids, float* w, hipStream_t stream) {
    if (!route_fused(E, dtype)) {
        hipError_t err = launch_router_logits(x, router, T, D, E, dtype, logits64, stream);
        if (err != hipSuccess) return err;
        return launch_topk(logits64, T, E, K, score, renorm, route_scale, bias, mask, logits_out, ids, w, stream);
    }
    const double rs = static_cast<double>(route_scale);
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    const uint16_t* wb = static_cast<const uint16_t*>(router);
#define MOE_ROUTE(TBB, NBW)                                                                              \
    route_fused_bf16_kernel<TBB, NBW><<<static_cast<unsigned>((T + 16 * TBB - 1) / (16 * TBB)), 256, 0, \
                                         stream>>>(xb, wb, T, D, E, K, score, renorm, rs, bias, mask,      \
                                                   logits_out, ids, w)
    if (E <= 64) MOE_ROUTE(4, 1);
    else if (E <= 128) MOE_ROUTE(4, 2);
    else if (E <= 256) MOE_ROUTE(4, 4);
    else MOE_ROUTE(2, 8);
#undef MOE_ROUTE
    return hipGetLastError();
}

}  // namespace moe
