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
// GEMM runs on MFMA with fp32 accumulation over chunks of 256 products (the
// last chunk may hold 64, 128 or 192), and the chunk sums are added in
// float64; in fp32
// mode each logit is a float64 FMA chain (the fp32 x fp32 products are exact
// in float64).  Scores, choices and weights are then float64 (the softmax
// normaliser sums float32 exponentials in float64); the weights are rounded
// once to float32.
#include "common.hpp"
#include "kernels.hpp"
#include "permute_block.hpp"

#include <type_traits>

namespace moe {

// ---------------------------------------------------------------------------
// router logits, bf16 operands: 64 tokens x 64 experts per workgroup
// ---------------------------------------------------------------------------
constexpr int kRtTok = 64;
constexpr int kRtExp = 64;
constexpr int kRtK = 64;  // k per LDS stage; fp32 partial sums span four stages (256 products)
// the small-batch router runs while T * E is at most this (each of its waves
// re-reads 16 hidden rows and 16 router rows, so its traffic grows with T * E;
// measured crossover with the fused router on the Qwen3-30B- and DSV4-like layers)
constexpr int64_t kRouteSmallTE = int64_t{1} << 18;
constexpr int64_t kTopkPermuteT = 8;  // moe_forward fuses top-k and permute up to this many tokens

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
    f32x4 acc[4];

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
        if ((k0 & 255) == 0) {
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
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
        if ((k0 & 255) == 192 || k0 + kRtK == D) {
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc64[nb][i] += static_cast<double>(acc[nb][i]);
        }
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
// given != nullptr replays routing: the K experts are given[t*K .. t*K+K-1]
// instead of the K largest choices (a token whose given ids are not K
// distinct ids in [0, E) is treated as masked); the weights still come from
// this token's scores.
// Score of one logit, float64: the logistic sigmoid (score 1) or
// sqrtsoftplus (score 2), sqrt(log(1 + e^l)) written as
// sqrt(max(l, 0) + log1p(e^-|l|)), which does not overflow.
__device__ __forceinline__ double elem_score(double l, int score) {
    if (score == 2) return sqrt(fmax(l, 0.0) + log1p(exp(-fabs(l))));
    return 1.0 / (1.0 + exp(-l));
}

// (a, b), a >= b: the two largest of this lane's and the other set's pair
// (the sets are disjoint)
__device__ __forceinline__ void top2_merge(double& a, double& b, double a2, double b2) {
    const double lo = fmax(fmin(a, a2), fmax(b, b2));
    a = fmax(a, a2);
    b = lo;
}
// The two largest values over the wave (uniform result).  Every step pairs
// lanes whose sets of values are disjoint, as a top-2 merge needs.
__device__ __forceinline__ void wave_top2_f64(double& a, double& b) {
    top2_merge(a, b, dpp_f64<0xB1>(a), dpp_f64<0xB1>(b));    // quad_perm(1,0,3,2)
    top2_merge(a, b, dpp_f64<0x4E>(a), dpp_f64<0x4E>(b));    // quad_perm(2,3,0,1)
    top2_merge(a, b, dpp_f64<0x141>(a), dpp_f64<0x141>(b));  // row_half_mirror
    top2_merge(a, b, dpp_f64<0x140>(a), dpp_f64<0x140>(b));  // row_mirror
    double ra = readlane_f64(a, 0), rb = readlane_f64(b, 0);
    top2_merge(ra, rb, readlane_f64(a, 16), readlane_f64(b, 16));
    top2_merge(ra, rb, readlane_f64(a, 32), readlane_f64(b, 32));
    top2_merge(ra, rb, readlane_f64(a, 48), readlane_f64(b, 48));
    a = ra;
    b = rb;
}

template <int EPL>
__device__ __forceinline__ void topk_token(const double (&lg)[EPL], int64_t t, int E, int K, int score,
                                           int renorm, double route_scale, const float* __restrict__ bias,
                                           bool kept, int32_t* __restrict__ ids_out, float* __restrict__ w_out,
                                           const int32_t* __restrict__ given, int n_group, int topk_group) {
    const int lane = lane_id();
    if (given != nullptr && kept) {
        const int g = lane < K ? given[t * K + lane] : 0;
        bool bad = lane < K && (g < 0 || g >= E);
        for (int i = 0; i < K; ++i) {
            const int gi = __builtin_amdgcn_readlane(g, i);
            bad = bad | (lane < K && i != lane && gi == g);
        }
        kept = __ballot(bad) == 0ull;
    }
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
    } else {  // sigmoid or sqrtsoftplus of each logit
#pragma unroll
        for (int i = 0; i < EPL; ++i) s[i] = ok[i] ? elem_score(lg[i], score) : 0.0;
    }

    uint64_t key[EPL];
    double ch[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        double c = s[i];
        if (bias != nullptr && ok[i]) c += static_cast<double>(bias[e]);
        ch[i] = c;
        key[i] = ok[i] ? choice_key(c, e) : 0ull;
    }

    // Group-limited select: group g holds experts g*gs .. g*gs+gs-1; its
    // score is the sum of its two largest choices; the topk_group best
    // groups are kept (ties to the lower group id) and the others' experts
    // leave the race.
    if (given == nullptr && n_group > 1) {
        const int gs = E / n_group;
        double gsc = 0.0;  // lane g: the score of group g
        for (int g = 0; g < n_group; ++g) {
            double a = -INFINITY, b = -INFINITY;
#pragma unroll
            for (int i = 0; i < EPL; ++i) {
                if (ok[i] && (lane + 64 * i) / gs == g) {
                    const double v = ch[i];
                    if (v > a) {
                        b = a;
                        a = v;
                    } else if (v > b) {
                        b = v;
                    }
                }
            }
            wave_top2_f64(a, b);
            if (lane == g) gsc = a + b;
        }
        uint64_t gkey = lane < n_group ? choice_key(gsc, lane) : 0ull;
        uint64_t keep = 0ull;
        for (int r = 0; r < topk_group; ++r) {
            const uint64_t win = wave_max_u64(gkey);
            const int g = 1023 - static_cast<int>(win & 0x3FFull);
            keep |= 1ull << g;
            if (lane == g) gkey = 0ull;
        }
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (ok[i] && ((keep >> ((lane + 64 * i) / gs)) & 1ull) == 0ull) key[i] = 0ull;
    }

    // K rounds of wave argmax; lane r keeps the r-th pick
    int my_e = -1;
    double my_s = 0.0;
    for (int r = 0; r < K; ++r) {
        int ew;
        if (given != nullptr) {
            ew = given[t * K + r];
        } else {
            uint64_t best = key[0];
#pragma unroll
            for (int i = 1; i < EPL; ++i) best = umax64(best, key[i]);
            const uint64_t win = wave_max_u64(best);
            ew = 1023 - static_cast<int>(win & 0x3FFull);
        }
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

// ---- sixteen lanes per token ------------------------------------------------
// The same selection for four tokens per wave: row r (lanes 16r .. 16r+15)
// takes one token, lane j of the row holds experts j, j + 16, ...  The row
// reductions use the first four DPP steps of the wave reductions above, which
// leave every lane of the row with the row's result.
__device__ __forceinline__ uint64_t row_max_u64(uint64_t k) {
    k = umax64(k, dpp_u64<0xB1>(k));
    k = umax64(k, dpp_u64<0x4E>(k));
    k = umax64(k, dpp_u64<0x141>(k));
    return umax64(k, dpp_u64<0x140>(k));
}
__device__ __forceinline__ double row_max_f64(double v) {
    v = fmax(v, dpp_f64<0xB1>(v));
    v = fmax(v, dpp_f64<0x4E>(v));
    v = fmax(v, dpp_f64<0x141>(v));
    return fmax(v, dpp_f64<0x140>(v));
}
__device__ __forceinline__ double row_sum_f64(double v) {
    v = v + dpp_f64<0xB1>(v);
    v = v + dpp_f64<0x4E>(v);
    v = v + dpp_f64<0x141>(v);
    return v + dpp_f64<0x140>(v);
}
// value of lane src (an absolute lane index) to the calling lane
__device__ __forceinline__ int lane_get(int v, int src) { return __builtin_amdgcn_ds_bpermute(src << 2, v); }
__device__ __forceinline__ double lane_get_f64(double v, int src) {
    const uint64_t b = static_cast<uint64_t>(__double_as_longlong(v));
    const uint32_t lo = static_cast<uint32_t>(lane_get(static_cast<int>(static_cast<uint32_t>(b)), src));
    const uint32_t hi = static_cast<uint32_t>(lane_get(static_cast<int>(static_cast<uint32_t>(b >> 32)), src));
    return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

template <int CTRL>
__device__ __forceinline__ int dpp_i32(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true);
}
__device__ __forceinline__ float row_max_f32(float v) {
    v = fmaxf(v, __int_as_float(dpp_i32<0xB1>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_i32<0x4E>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_i32<0x141>(__float_as_int(v))));
    return fmaxf(v, __int_as_float(dpp_i32<0x140>(__float_as_int(v))));
}
// inclusive prefix sum over the 16 lanes of a row (row_shr 1, 2, 4, 8)
__device__ __forceinline__ int row_scan_i32(int v) {
    v += dpp_i32<0x111>(v);
    v += dpp_i32<0x112>(v);
    v += dpp_i32<0x114>(v);
    return v + dpp_i32<0x118>(v);
}
__device__ __forceinline__ int row_max_i32(int v) {
    v = max(v, dpp_i32<0xB1>(v));
    v = max(v, dpp_i32<0x4E>(v));
    v = max(v, dpp_i32<0x141>(v));
    return max(v, dpp_i32<0x140>(v));
}

// How many lanes of this lane's row hold a value v below x (the other 15
// lanes through row rotations).
template <int S>
__device__ __forceinline__ void count_step(int v, int x, int& n) {
    n += dpp_i32<0x120 + S>(v) < x ? 1 : 0;  // row_ror:S
}
__device__ __forceinline__ int row_count_below(int v, int x) {
    int n = 0;
    count_step<1>(v, x, n);
    count_step<2>(v, x, n);
    count_step<3>(v, x, n);
    count_step<4>(v, x, n);
    count_step<5>(v, x, n);
    count_step<6>(v, x, n);
    count_step<7>(v, x, n);
    count_step<8>(v, x, n);
    count_step<9>(v, x, n);
    count_step<10>(v, x, n);
    count_step<11>(v, x, n);
    count_step<12>(v, x, n);
    count_step<13>(v, x, n);
    count_step<14>(v, x, n);
    count_step<15>(v, x, n);
    return n;
}

// The picks of P rows (lane r of a row holds its r-th pick: my_e, my_s) in
// ascending id order with their weights, to ids_out / w_out.  The
// renormalising sum adds the picks' scores in ascending id order, through
// the wave's scratch (the rows16_select slots, free again by now).
// ids_lds, if given, receives the ids too (at the same index as ids_out).
template <int P>
__device__ __forceinline__ void write_picks16(const int (&my_e)[P], const double (&my_s)[P], const int64_t (&t)[P],
                                              const bool (&live)[P], const bool (&kept)[P], int K, int renorm,
                                              double route_scale, int32_t* __restrict__ ids_out,
                                              float* __restrict__ w_out, lds_u8* scr, int* ids_lds = nullptr) {
    const int lane = lane_id();
    const int j = lane & 15;
    const int row = lane >> 4;
    int rank[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        // ascending id order: rank of each pick among the row's K picks (K <= 16)
        // (every lane takes part in the rotations; lanes past K hold no pick)
        const int below = row_count_below(j < K ? my_e[p] : 0x7FFFFFFF, my_e[p]);
        rank[p] = j < K ? below : 0;
        if (renorm && j < K)
            *reinterpret_cast<__attribute__((address_space(3))) double*>(scr + ((p * 4 + row) * 32 + rank[p]) * 16) =
                my_s[p];
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int p = 0; p < P; ++p) {
        double den = 1.0;
        if (renorm) {
            den = 0.0;
            for (int r = 0; r < K; ++r)
                den += *reinterpret_cast<const __attribute__((address_space(3))) double*>(scr + ((p * 4 + row) * 32 + r) *
                                                                                           16);
        }
        if (live[p] && j < K) {
            if (kept[p]) {
                const double wv = renorm ? (my_s[p] / den) * route_scale : my_s[p] * route_scale;
                ids_out[t[p] * K + rank[p]] = my_e[p];
                w_out[t[p] * K + rank[p]] = static_cast<float>(wv);
                if (ids_lds != nullptr) ids_lds[t[p] * K + rank[p]] = my_e[p];
            } else {
                ids_out[t[p] * K + j] = -1;
                w_out[t[p] * K + j] = 0.f;
                if (ids_lds != nullptr) ids_lds[t[p] * K + j] = -1;
            }
        }
    }
    __builtin_amdgcn_wave_barrier();  // the scratch is read before the next use
}

// ---- top-k of one token per row of sixteen lanes ------------------------------
// Every routing path of a layer with at most 512 experts (with group-limited
// select: groups of 16 to 128 experts, at most 16 groups) selects through the
// functions below (the fused router, the top-k kernel, the decode top-k +
// permute kernel and replay), so a token's ids and weights are the same bits
// whichever kernel runs and whatever the batch.  Row r of a wave (lanes 16r .. 16r+15) takes one token; lane j of
// the row covers experts j, j + 16, ... (EPL16 slots, those past E unused).
// The float64 logits are read through lg_of(p, e): the logit of expert e of
// the row's p-th token, from LDS or from memory.
//
// Scores: sigmoid and sqrtsoftplus per logit in float64 (elem_score).
// Softmax: m = the token's largest logit; z = the sum over its experts of
// float64(expf(float32(l - m))), each lane adding its slots in order and the
// row then adding the lanes in a fixed pairwise tree; an expert's score is
// exp(l - m) / z in float64.  The float32 exponentials put z within about
// 1e-7 relative of the float64 sum; z scales every score of the token alike,
// so it moves a weight by at most that much and decides no pick whose choice
// margin is larger.
template <int EPL16, typename LG>
__device__ __forceinline__ void row_softmax(LG lg_of, int p, int E, double& m, double& z) {
    const int j = lane_id() & 15;
    double mx = -1.7976931348623157e308;
#pragma unroll 4
    for (int i = 0; i < EPL16; ++i)
        if (j + 16 * i < E) mx = fmax(mx, lg_of(p, j + 16 * i));
    m = row_max_f64(mx);
    double part = 0.0;
#pragma unroll 4
    for (int i = 0; i < EPL16; ++i)
        if (j + 16 * i < E) part += static_cast<double>(__expf(static_cast<float>(lg_of(p, j + 16 * i) - m)));
    z = row_sum_f64(part);
}

__device__ __forceinline__ double row_score(double l, int score, double m, double z) {
    return score == 0 ? exp(l - m) / z : elem_score(l, score);
}

// scratch of rows16_select per wave: 4 rows x 32 slots x 16 bytes for each of
// the P tokens per row, then one slot per lane that takes the compaction's
// stores of non-candidates (so that no store needs a branch)
constexpr int kRowScr = 4 * 32 * 16;
constexpr int kDumpScr = 64 * 16;

// The selection bias of this lane's experts j, j + 16, ... (0 without a
// bias or past E); the same for every token, so loaded once per kernel.
template <int EPL16>
__device__ __forceinline__ void load_bias16(const float* __restrict__ bias, int E, float (&bv)[EPL16]) {
    const int j = lane_id() & 15;
#pragma unroll
    for (int i = 0; i < EPL16; ++i) bv[i] = (bias != nullptr && j + 16 * i < E) ? bias[j + 16 * i] : 0.0f;
}

// Rank of key a among the 2 x 16 keys (k0, k1) of this lane's row: how many
// of them are larger.  The keys of a row are distinct or zero.
template <int S>
__device__ __forceinline__ void rank_step(uint64_t k0, uint64_t k1, int& r0, int& r1) {
    const uint64_t o0 = dpp_u64<0x120 + S>(k0);  // row_ror:S
    const uint64_t o1 = dpp_u64<0x120 + S>(k1);
    r0 += (o0 > k0 ? 1 : 0) + (o1 > k0 ? 1 : 0);
    r1 += (o0 > k1 ? 1 : 0) + (o1 > k1 ? 1 : 0);
}
__device__ __forceinline__ void row_ranks(uint64_t k0, uint64_t k1, int& r0, int& r1) {
    r0 = k1 > k0 ? 1 : 0;
    r1 = k0 > k1 ? 1 : 0;
    rank_step<1>(k0, k1, r0, r1);
    rank_step<2>(k0, k1, r0, r1);
    rank_step<3>(k0, k1, r0, r1);
    rank_step<4>(k0, k1, r0, r1);
    rank_step<5>(k0, k1, r0, r1);
    rank_step<6>(k0, k1, r0, r1);
    rank_step<7>(k0, k1, r0, r1);
    rank_step<8>(k0, k1, r0, r1);
    rank_step<9>(k0, k1, r0, r1);
    rank_step<10>(k0, k1, r0, r1);
    rank_step<11>(k0, k1, r0, r1);
    rank_step<12>(k0, k1, r0, r1);
    rank_step<13>(k0, k1, r0, r1);
    rank_step<14>(k0, k1, r0, r1);
    rank_step<15>(k0, k1, r0, r1);
}
// the same with one key per lane (the row's candidates fit its 16 lanes)
template <int S>
__device__ __forceinline__ void rank_step1(uint64_t k0, int& r0) {
    r0 += dpp_u64<0x120 + S>(k0) > k0 ? 1 : 0;  // row_ror:S
}
__device__ __forceinline__ int row_rank1(uint64_t k0) {
    int r0 = 0;
    rank_step1<1>(k0, r0);
    rank_step1<2>(k0, r0);
    rank_step1<3>(k0, r0);
    rank_step1<4>(k0, r0);
    rank_step1<5>(k0, r0);
    rank_step1<6>(k0, r0);
    rank_step1<7>(k0, r0);
    rank_step1<8>(k0, r0);
    rank_step1<9>(k0, r0);
    rank_step1<10>(k0, r0);
    rank_step1<11>(k0, r0);
    rank_step1<12>(k0, r0);
    rank_step1<13>(k0, r0);
    rank_step1<14>(k0, r0);
    rank_step1<15>(k0, r0);
    return r0;
}

// The compacted candidates of each row (slot k: logit, id, bias) get their
// float64 score and choice key, H slots per lane (lane j takes slots j and
// j + 16); each candidate's rank among its row's candidates (how many keys
// are larger) places the K best at slots 0 .. K-1 (score, id).  One slot per
// lane when no row of the wave has more than 16 candidates; both give the
// same placement.
template <int H, int P>
__device__ __forceinline__ void rows16_place(lds_u8* scr, const int (&n_row)[P], const double (&m)[P],
                                             const double (&z)[P], int score, int K) {
    const int lane = lane_id();
    const int j = lane & 15;
    const int row = lane >> 4;
    uint64_t key[P][H];
    double sc[P][H];
    int ce[P][H];
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
        for (int h = 0; h < H; ++h) {
            key[p][h] = 0ull;
            sc[p][h] = 0.0;
            ce[p][h] = 0;
            const int slot = j + 16 * h;
            if (slot < n_row[p]) {
                const u32x4 rec = *reinterpret_cast<lds_u32x4*>(scr + ((p * 4 + row) * 32 + slot) * 16);
                const double l =
                    __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(rec[1]) << 32) | rec[0]));
                ce[p][h] = static_cast<int>(rec[2]);
                sc[p][h] = row_score(l, score, m[p], z[p]);
                const double c = sc[p][h] + static_cast<double>(__uint_as_float(rec[3]));
                key[p][h] = choice_key(c, ce[p][h]);
            }
        }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int p = 0; p < P; ++p) {
        int rk[H];
        if constexpr (H == 2) row_ranks(key[p][0], key[p][1], rk[0], rk[1]);
        else rk[0] = row_rank1(key[p][0]);
#pragma unroll
        for (int h = 0; h < H; ++h) {
            if (j + 16 * h < n_row[p] && rk[h] < K) {
                const uint64_t sb = static_cast<uint64_t>(__double_as_longlong(sc[p][h]));
                const u32x4 rec = {static_cast<uint32_t>(sb), static_cast<uint32_t>(sb >> 32),
                                   static_cast<uint32_t>(ce[p][h]), 0u};
                *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(scr + ((p * 4 + row) * 32 + rk[h]) * 16) =
                    rec;
            }
        }
    }
}

// The K largest choices (score + bias, ties to the lower id) of the P tokens
// of this lane's row; lane r < K of the row receives one pick and its score
// (the picks in descending choice order).  Every choice is first evaluated in
// float32 (within about 1e-6 + 1e-7 |c| of its float64 value, far inside the
// margin below).  mu, the K-th largest of the 16 lanes' largest float32
// choices, is at most the K-th largest float32 choice (K lanes hold one
// >= mu), so every expert the float64 choice can pick has a float32 choice
// >= mu - margin.  Those candidates (at most 32 per row) are compacted
// through the wave's LDS scratch (16 bytes per slot: logit, id, bias; P x 4
// rows x 32 slots), get their float64 choice key, and each candidate's rank
// among its row's candidates (how many keys are larger) places the K best.
// A wave with a live row of more than 32 candidates (or K > 32) runs K rounds
// of row argmax over every expert's float64 choice instead, rereading the
// logits through lg_of; both give the same bits.  Every lane of the wave must
// call this.
template <int EPL16, int P, typename LG>
__device__ __forceinline__ void rows16_select(LG lg_of, const bool (&live)[P], int E, int K, int score,
                                              const float* __restrict__ bias, const float (&bv)[EPL16], lds_u8* scr,
                                              int (&my_e)[P], double (&my_s)[P]) {
    const int lane = lane_id();
    const int j = lane & 15;
    const int row = lane >> 4;
    double lg[P][EPL16];
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
        for (int i = 0; i < EPL16; ++i) lg[p][i] = j + 16 * i < E ? lg_of(p, j + 16 * i) : 0.0;

    double m[P], z[P];
    uint32_t cm[P];  // candidate slots of this lane, one bit per slot
    int off[P], n_row[P];
    bool over = K > 32;
#pragma unroll
    for (int p = 0; p < P; ++p) {
        float c32[EPL16];
        m[p] = 0.0;
        z[p] = 1.0;
        if (score == 0) {
            // the softmax of row_softmax, from registers
            double mx = -1.7976931348623157e308;
#pragma unroll
            for (int i = 0; i < EPL16; ++i)
                if (j + 16 * i < E) mx = fmax(mx, lg[p][i]);
            m[p] = row_max_f64(mx);
            double part = 0.0;
#pragma unroll
            for (int i = 0; i < EPL16; ++i) {
                c32[i] = 0.0f;
                if (j + 16 * i < E) {
                    c32[i] = __expf(static_cast<float>(lg[p][i] - m[p]));
                    part += static_cast<double>(c32[i]);
                }
            }
            z[p] = row_sum_f64(part);
            const float rz = static_cast<float>(1.0 / z[p]);
#pragma unroll
            for (int i = 0; i < EPL16; ++i) c32[i] = j + 16 * i < E ? c32[i] * rz + bv[i] : -INFINITY;
        } else if (score == 2) {  // one loop per score: no branch per slot
#pragma unroll
            for (int i = 0; i < EPL16; ++i) {
                const float l = static_cast<float>(lg[p][i]);
                const float sc32 = sqrtf(fmaxf(l, 0.0f) + log1pf(__expf(-fabsf(l))));
                c32[i] = j + 16 * i < E ? sc32 + bv[i] : -INFINITY;
            }
        } else {
#pragma unroll
            for (int i = 0; i < EPL16; ++i) {
                const float l = static_cast<float>(lg[p][i]);
                const float sc32 = __builtin_amdgcn_rcpf(1.0f + __expf(-l));
                c32[i] = j + 16 * i < E ? sc32 + bv[i] : -INFINITY;
            }
        }
        float v = -INFINITY;
#pragma unroll
        for (int i = 0; i < EPL16; ++i) v = fmaxf(v, c32[i]);
        float mu = -INFINITY;
        for (int r = 0; r < K; ++r) {
            mu = row_max_f32(v);
            v = v == mu ? -INFINITY : v;  // equal lane maxima go together: mu only gets smaller
        }
        const float thr = mu - (1e-5f + 1e-6f * fabsf(mu));
        cm[p] = 0u;
#pragma unroll
        for (int i = 0; i < EPL16; ++i)
            if (live[p] && c32[i] >= thr) cm[p] |= 1u << i;
        const int nl = __builtin_popcount(cm[p]);
        const int incl = row_scan_i32(nl);
        off[p] = incl - nl;
        n_row[p] = row_max_i32(incl);
        over = over || n_row[p] > 32;
    }

    if (__ballot(over) == 0ull) {
        // candidate k of row r of token p at slot (p, r, k): logit, id, bias;
        // every slot of the lane is stored, the non-candidates to the lane's
        // dump slot
        const int dump = (P * 4 * 32 + lane) * 16;
#pragma unroll
        for (int p = 0; p < P; ++p) {
            int k = off[p];
#pragma unroll
            for (int i = 0; i < EPL16; ++i) {
                const bool c = (cm[p] >> i) & 1u;
                const uint64_t lb = static_cast<uint64_t>(__double_as_longlong(lg[p][i]));
                const u32x4 rec = {static_cast<uint32_t>(lb), static_cast<uint32_t>(lb >> 32),
                                   static_cast<uint32_t>(j + 16 * i), __float_as_uint(bv[i])};
                *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(scr + (c ? ((p * 4 + row) * 32 + k) * 16
                                                                                       : dump)) = rec;
                k += c ? 1 : 0;
            }
        }
        __builtin_amdgcn_wave_barrier();
        bool wide = false;
#pragma unroll
        for (int p = 0; p < P; ++p) wide = wide || n_row[p] > 16;
        if (__ballot(wide) == 0ull) rows16_place<1, P>(scr, n_row, m, z, score, K);
        else rows16_place<2, P>(scr, n_row, m, z, score, K);
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int p = 0; p < P; ++p) {
            my_e[p] = -1;
            my_s[p] = 0.0;
            if (j < K && live[p]) {
                const u32x4 rec = *reinterpret_cast<lds_u32x4*>(scr + ((p * 4 + row) * 32 + j) * 16);
                my_s[p] = __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(rec[1]) << 32) | rec[0]));
                my_e[p] = static_cast<int>(rec[2]);
            }
        }
        __builtin_amdgcn_wave_barrier();
        return;
    }

    // round r picks the largest key below the previous pick's (keys are
    // distinct: their low bits hold the id)
    auto key_of = [&](int p, int e) {
        const double c = row_score(lg_of(p, e), score, m[p], z[p]) +
                         (bias != nullptr ? static_cast<double>(bias[e]) : 0.0);
        return choice_key(c, e);
    };
#pragma unroll 1
    for (int p = 0; p < P; ++p) {
        my_e[p] = -1;
        uint64_t prev = ~0ull;
        for (int r = 0; r < K; ++r) {
            uint64_t best = 0ull;
#pragma unroll 1
            for (int i = 0; i < EPL16; ++i) {
                if (j + 16 * i < E) {
                    const uint64_t k = key_of(p, j + 16 * i);
                    if (k < prev) best = umax64(best, k);
                }
            }
            prev = row_max_u64(best);
            if (j == r) my_e[p] = 1023 - static_cast<int>(prev & 0x3FFull);
        }
        // rows past the batch pick nothing meaningful and read expert 0
        const int e = (live[p] && my_e[p] >= 0 && my_e[p] < E) ? my_e[p] : 0;
        my_s[p] = j < K ? row_score(lg_of(p, e), score, m[p], z[p]) : 0.0;
    }
}

// Group-limited select in a row of sixteen lanes, the selection of
// topk_token's group stage: experts form n_group groups of 16 SP consecutive
// ids (group g: slots g SP .. g SP + SP - 1 of every lane), a group's score
// is the sum of its two largest float64 choices, the topk_group best groups
// are kept (ties to the lower group id), and K rounds of row argmax over the
// kept experts' keys pick the experts; lane r of the row receives the r-th
// pick and its score.  Every choice is evaluated in float64 (the group sums
// need the exact two largest of every group).  Every lane of the wave must
// call this.
__device__ __forceinline__ void row_top2_f64(double& a, double& b) {
    top2_merge(a, b, dpp_f64<0xB1>(a), dpp_f64<0xB1>(b));    // quad_perm(1,0,3,2)
    top2_merge(a, b, dpp_f64<0x4E>(a), dpp_f64<0x4E>(b));    // quad_perm(2,3,0,1)
    top2_merge(a, b, dpp_f64<0x141>(a), dpp_f64<0x141>(b));  // row_half_mirror
    top2_merge(a, b, dpp_f64<0x140>(a), dpp_f64<0x140>(b));  // row_mirror
}

// lane g of the row receives the score of group g (groups of SP slots)
template <int EPL16, int SP>
__device__ __forceinline__ void group_scores16(const double (&ch)[EPL16], int E, double& gsc) {
    static_assert(EPL16 % SP == 0 && EPL16 / SP <= 16, "groups of whole slots, at most one per lane");
    const int j = lane_id() & 15;
#pragma unroll
    for (int g = 0; g < EPL16 / SP; ++g) {
        double a = -INFINITY, b = -INFINITY;
#pragma unroll
        for (int k = 0; k < SP; ++k) {
            const int i = g * SP + k;
            if (j + 16 * i < E) {
                const double v = ch[i];
                if (v > a) {
                    b = a;
                    a = v;
                } else if (v > b) {
                    b = v;
                }
            }
        }
        row_top2_f64(a, b);
        if (j == g) gsc = a + b;
    }
}

// slots per lane of one group (16 SP experts) where the sixteen-lane group
// select applies, else 0: groups of 16, 32, 64 or 128 experts, at most 16
// groups
__host__ __device__ inline int grouped16_sp(int E, int n_group) {
    if (n_group <= 1 || E % n_group != 0 || n_group > 16) return 0;
    const int gs = E / n_group;
    return (gs == 16 || gs == 32 || gs == 64 || gs == 128) ? gs / 16 : 0;
}

template <int EPL16, typename LG>
__device__ __forceinline__ void rows16_grouped(LG lg_of, int E, int K, int score, const float (&bv)[EPL16],
                                               int n_group, int topk_group, int& my_e, double& my_s) {
    const int lane = lane_id();
    const int j = lane & 15;
    const int rbase = lane & 48;
    double lg[EPL16];
#pragma unroll
    for (int i = 0; i < EPL16; ++i) lg[i] = j + 16 * i < E ? lg_of(0, j + 16 * i) : 0.0;
    double m = 0.0, z = 1.0;
    if (score == 0) {  // the softmax of row_softmax, from registers
        double mx = -1.7976931348623157e308;
#pragma unroll
        for (int i = 0; i < EPL16; ++i)
            if (j + 16 * i < E) mx = fmax(mx, lg[i]);
        m = row_max_f64(mx);
        double part = 0.0;
#pragma unroll
        for (int i = 0; i < EPL16; ++i)
            if (j + 16 * i < E) part += static_cast<double>(__expf(static_cast<float>(lg[i] - m)));
        z = row_sum_f64(part);
    }
    double sc[EPL16], ch[EPL16];
    uint64_t key[EPL16];
#pragma unroll
    for (int i = 0; i < EPL16; ++i) {
        const int e = j + 16 * i;
        sc[i] = e < E ? row_score(lg[i], score, m, z) : 0.0;
    }
#pragma unroll
    for (int i = 0; i < EPL16; ++i) {
        const int e = j + 16 * i;
        ch[i] = sc[i] + static_cast<double>(bv[i]);
        key[i] = e < E ? choice_key(ch[i], e) : 0ull;
    }
    const int sp = grouped16_sp(E, n_group);
    double gsc = 0.0;
    if (sp == 1) {
        if constexpr (EPL16 <= 16) group_scores16<EPL16, 1>(ch, E, gsc);
    } else if (sp == 2) {
        group_scores16<EPL16, 2>(ch, E, gsc);
    } else if (sp == 4) {
        if constexpr (EPL16 >= 4) group_scores16<EPL16, 4>(ch, E, gsc);
    } else {
        if constexpr (EPL16 >= 8) group_scores16<EPL16, 8>(ch, E, gsc);
    }
    uint64_t gkey = j < n_group ? choice_key(gsc, j) : 0ull;
    uint32_t keep = 0u;
    for (int r = 0; r < topk_group; ++r) {
        const uint64_t win = row_max_u64(gkey);
        const int g = 1023 - static_cast<int>(win & 0x3FFull);
        keep |= 1u << g;
        if (j == g) gkey = 0ull;
    }
    const int sh = sp == 1 ? 0 : sp == 2 ? 1 : sp == 4 ? 2 : 3;  // slot i lies in group i >> sh
#pragma unroll
    for (int i = 0; i < EPL16; ++i)
        if (((keep >> (i >> sh)) & 1u) == 0u) key[i] = 0ull;
    // K rounds of row argmax; lane r keeps the r-th pick
    my_e = -1;
    my_s = 0.0;
    for (int r = 0; r < K; ++r) {
        uint64_t best = key[0];
#pragma unroll
        for (int i = 1; i < EPL16; ++i) best = umax64(best, key[i]);
        const uint64_t win = row_max_u64(best);
        const int ew = 1023 - static_cast<int>(win & 0x3FFull);
        const int owner = ew & 15;
        const int slot = ew >> 4;
        double sw = 0.0;
#pragma unroll
        for (int i = 0; i < EPL16; ++i) {
            if (j == owner && i == slot) {
                sw = sc[i];
                key[i] = 0ull;
            }
        }
        sw = lane_get_f64(sw, rbase + owner);
        if (j == r) {
            my_e = ew;
            my_s = sw;
        }
    }
}

// Replay: lane j < K of the row takes the given id given[t * K + j]; a token
// whose K given ids are not distinct ids in [0, E) is dropped (kept false).
// The scores are those of rows16_select.  Every lane of the wave must call
// this.
template <int EPL16, int P, typename LG>
__device__ __forceinline__ void rows16_given(LG lg_of, const int64_t (&t)[P], const bool (&live)[P], int E, int K,
                                             int score, const int32_t* __restrict__ given, bool (&kept)[P],
                                             int (&my_e)[P], double (&my_s)[P]) {
    const int lane = lane_id();
    const int j = lane & 15;
    const int rbase = lane & 48;
#pragma unroll
    for (int p = 0; p < P; ++p) {
        double m = 0.0, z = 1.0;
        if (score == 0) row_softmax<EPL16>(lg_of, p, E, m, z);
        const bool mine = live[p] && j < K;
        const int g = mine ? given[t[p] * K + j] : 0;
        bool bad = mine && (g < 0 || g >= E);
        for (int i = 0; i < K; ++i) {
            const int gi = lane_get(g, rbase + i);
            bad = bad || (mine && i != j && gi == g);
        }
        kept[p] = kept[p] && ((__ballot(bad) >> rbase) & 0xFFFFull) == 0ull;
        my_e[p] = -1;
        my_s[p] = 0.0;
        if (kept[p] && j < K) {
            my_e[p] = g;
            my_s[p] = row_score(lg_of(p, g), score, m, z);
        }
    }
}

template <int EPL>
__global__ __launch_bounds__(256) void topk_kernel(
    const double* __restrict__ logits, int64_t T, int E, int K, int score, int renorm,
    double route_scale, const float* __restrict__ bias, const uint8_t* __restrict__ mask,
    float* __restrict__ logits_out, int32_t* __restrict__ ids_out, float* __restrict__ w_out,
    const int32_t* __restrict__ given, int n_group, int topk_group) {
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
    topk_token<EPL>(lg, t, E, K, score, renorm, route_scale, bias, kept, ids_out, w_out, given, n_group, topk_group);
}

// Decode-sized batches in moe_forward: the top-k of every token and the
// dispatch permutation in one workgroup, one launch instead of two.  Wave w
// takes tokens w, w + 4, ... and picks exactly as topk_kernel does; the
// barrier makes the ids visible to the workgroup, and the permutation
// follows from LDS (permute_small, the rows of the multi-block path).
template <int EPL>
__global__ __launch_bounds__(256) void topk_permute_kernel(
    const double* __restrict__ logits, int64_t T, int E, int K, int score, int renorm, double route_scale,
    const float* __restrict__ bias, const uint8_t* __restrict__ mask, float* __restrict__ logits_out,
    int32_t* __restrict__ ids_out, float* __restrict__ w_out, const int32_t* __restrict__ given, int n_group,
    int topk_group, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm_token, int32_t* __restrict__ inv_pos) {
    const int lane = lane_id();
    const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    for (int64_t t = wv; t < T; t += 4) {
        double lg[EPL];
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane + 64 * i;
            lg[i] = e < E ? logits[t * E + e] : 0.0;
            if (logits_out && e < E) logits_out[t * E + e] = static_cast<float>(lg[i]);
        }
        const bool kept = (mask == nullptr) || (mask[t] != 0);
        topk_token<EPL>(lg, t, E, K, score, renorm, route_scale, bias, kept, ids_out, w_out, given, n_group,
                        topk_group);
    }
    __syncthreads();  // every token's ids written and visible to the workgroup
    __shared__ int pairs[kSmallPairs];  // T * K <= 8 * 16 pairs
    if (threadIdx.x < T * K) pairs[threadIdx.x] = ids_out[threadIdx.x];
    __syncthreads();
    permute_small(pairs, static_cast<int>(T * K), K, E, counts, offsets, perm_token, inv_pos);
}


// The top-k of 16 tokens per 256-thread workgroup, one per row of sixteen
// lanes (E <= 512; GRP: group-limited select, rows16_grouped).
template <int EPL16, bool GRP = false>
__global__ __launch_bounds__(256) void topk_rows16_kernel(
    const double* __restrict__ logits, int64_t T, int E, int K, int score, int renorm, double route_scale,
    const float* __restrict__ bias, const uint8_t* __restrict__ mask, float* __restrict__ logits_out,
    int32_t* __restrict__ ids_out, float* __restrict__ w_out, const int32_t* __restrict__ given, int n_group,
    int topk_group) {
    __shared__ __attribute__((aligned(16))) uint8_t scr_raw[4 * (kRowScr + kDumpScr)];
    const int j = lane_id() & 15;
    const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    int64_t t[1];
    bool live[1], kept[1];
    t[0] = static_cast<int64_t>(blockIdx.x) * 16 + (threadIdx.x >> 4);
    live[0] = t[0] < T;
    // rows past T read token T-1 (their picks are not written)
    const double* row_lg = logits + (live[0] ? t[0] : T - 1) * E;
    auto lg_of = [&](int, int e) { return row_lg[e]; };
    if (logits_out && live[0])
        for (int e = j; e < E; e += 16) logits_out[t[0] * E + e] = static_cast<float>(row_lg[e]);
    kept[0] = live[0] && ((mask == nullptr) || (mask[t[0]] != 0));
    int my_e[1];
    double my_s[1];
    lds_u8* scr = (lds_u8*)(scr_raw) + wv * (kRowScr + kDumpScr);
    if (given != nullptr) {
        rows16_given<EPL16, 1>(lg_of, t, live, E, K, score, given, kept, my_e, my_s);
    } else {
        float bv[EPL16];
        load_bias16<EPL16>(bias, E, bv);
        if constexpr (GRP) rows16_grouped<EPL16>(lg_of, E, K, score, bv, n_group, topk_group, my_e[0], my_s[0]);
        else rows16_select<EPL16, 1>(lg_of, live, E, K, score, bias, bv, scr, my_e, my_s);
    }
    write_picks16<1>(my_e, my_s, t, live, kept, K, renorm, route_scale, ids_out, w_out, scr);
}

// topk_permute_kernel for layers whose top-k runs in rows of sixteen lanes:
// 16 tokens per pass, the picks kept in LDS as well, then the permutation of
// every pair from there (T * K <= 8 * 16 pairs: permute_small).
template <int EPL16, bool GRP = false>
__global__ __launch_bounds__(256) void topk_permute_rows16_kernel(
    const double* __restrict__ logits, int64_t T, int E, int K, int score, int renorm, double route_scale,
    const float* __restrict__ bias, const uint8_t* __restrict__ mask, float* __restrict__ logits_out,
    int32_t* __restrict__ ids_out, float* __restrict__ w_out, const int32_t* __restrict__ given, int n_group,
    int topk_group, int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ perm_token,
    int32_t* __restrict__ inv_pos) {
    __shared__ __attribute__((aligned(16))) uint8_t scr_raw[4 * (kRowScr + kDumpScr)];
    __shared__ int pairs[kSmallPairs];
    const int j = lane_id() & 15;
    const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    lds_u8* scr = (lds_u8*)(scr_raw) + wv * (kRowScr + kDumpScr);
    float bv[EPL16];
    load_bias16<EPL16>(given == nullptr ? bias : nullptr, E, bv);
    for (int64_t tb = 0; tb < T; tb += 16) {
        int64_t t[1];
        bool live[1], kept[1];
        t[0] = tb + (threadIdx.x >> 4);
        live[0] = t[0] < T;
        const double* row_lg = logits + (live[0] ? t[0] : T - 1) * E;
        auto lg_of = [&](int, int e) { return row_lg[e]; };
        if (logits_out && live[0])
            for (int e = j; e < E; e += 16) logits_out[t[0] * E + e] = static_cast<float>(row_lg[e]);
        kept[0] = live[0] && ((mask == nullptr) || (mask[t[0]] != 0));
        int my_e[1];
        double my_s[1];
        if (given != nullptr) {
            rows16_given<EPL16, 1>(lg_of, t, live, E, K, score, given, kept, my_e, my_s);
        } else {
            if constexpr (GRP) rows16_grouped<EPL16>(lg_of, E, K, score, bv, n_group, topk_group, my_e[0], my_s[0]);
            else rows16_select<EPL16, 1>(lg_of, live, E, K, score, bias, bv, scr, my_e, my_s);
        }
        write_picks16<1>(my_e, my_s, t, live, kept, K, renorm, route_scale, ids_out, w_out, scr, pairs);
    }
    __syncthreads();  // every pick in LDS
    permute_small(pairs, static_cast<int>(T * K), K, E, counts, offsets, perm_token, inv_pos);
}

// ---------------------------------------------------------------------------
// fused routing, bf16 operands: logits of TB tokens x all experts in one
// workgroup, kept in LDS as float64, then top-k per token from LDS.
// The hidden rows are read from memory once and the logits never leave the
// chip.  Each logit is computed exactly as router_logits_bf16_kernel does
// (MFMA k=32 steps into an fp32 accumulator zeroed every 256 k, the 256-wide
// partial sums added in float64 in k order), so both paths give the same bits.
// The chunks stream through two LDS stages filled by global_load_lds_dwordx4
// (8 rows x 128 bytes per instruction, the 16-byte chunks of a row XOR-
// swizzled by row % 8), so loads run a whole chunk ahead of the MFMAs.
// ---------------------------------------------------------------------------
// TBB: 16-token blocks per workgroup; NBW: 16-expert blocks per wave (4 waves).
// Hidden rows stream from memory through a ring of XS stages (loads run XS-1
// chunks ahead); router rows, read by every workgroup and so mostly served
// from L2, through a ring of WS stages.
template <int TBB, int NBW>
struct RouteTile {
    static constexpr int TB = 16 * TBB;        // tokens per workgroup
    static constexpr int EMAX = 64 * NBW;      // experts per workgroup
    static constexpr int EPL = EMAX / 64;      // experts per lane in the top-k
    static constexpr int XSTAGE = TB * 128;    // bytes of hidden rows per 64-wide k chunk
    static constexpr int WSTAGE = EMAX * 128;  // bytes of router rows per chunk
    static constexpr int XS = (TB >= 128 || EMAX > 256) ? 4 : 8;
    static constexpr int WS = (3 * WSTAGE + XS * XSTAGE <= 160 * 1024) ? 3 : 2;
    static constexpr int WOFF = XS * XSTAGE;   // LDS offset of the router ring
    static constexpr int RING = WOFF + WS * WSTAGE;
    static constexpr int TBP_MAX = EMAX > 256 ? 32 : 64;
    static constexpr int TBP = TB < TBP_MAX ? TB : TBP_MAX;  // tokens whose logits are in LDS at a time
    static constexpr int LOGB = TBP * EMAX * 8; // float64 logits of one pass
    static constexpr int SCRB = 4 * (2 * kRowScr + kDumpScr);  // top-k scratch: 4 waves, up to 2 tokens per row
    static constexpr int SMEM = RING > LOGB + SCRB ? RING : LOGB + SCRB;
    static constexpr int XPER = TB / 32;       // 8-row DMA instructions per wave per chunk
    static constexpr int WPER = EMAX / 32;
    static_assert(TB % 32 == 0 && EMAX % 32 == 0, "8-row DMA groups over 4 waves");
    // the stage wait counts on hidden chunk st being older than router chunk st
    static_assert(XS > WS, "hidden rows run further ahead than router rows");
    static_assert(SMEM <= 160 * 1024, "LDS");
};

// Top-k of the TBP tokens starting at token tp whose float64 logits are in
// lgs ([TBP][EMAX]); scr: the candidate slots of the screened selection.
// LAST: no other pass's logits are held in registers any more.
template <typename RT, bool GRP, bool LAST>
__device__ __forceinline__ void route_topk_pass(const __attribute__((address_space(3))) double* lgs, lds_u8* scr_base,
                                                int64_t tp, int64_t T, int E, int K, int score, int renorm,
                                                double route_scale, const float* __restrict__ bias,
                                                const float (&bv)[RT::EMAX / 16], int n_group, int topk_group,
                                                const uint8_t* __restrict__ mask, float* __restrict__ logits_out,
                                                int32_t* __restrict__ ids_out, float* __restrict__ w_out) {
    const int lane = lane_id();
    const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const int64_t t0 = tp;
    // P tokens per row of sixteen lanes at a time: two where registers allow
    // (during the first pass of a 128-token tile the other pass's logits are
    // still held in registers; its last pass has them free)
    constexpr int EPL16 = RT::EMAX / 16;
    constexpr int P = ((RT::TB > RT::TBP && !LAST) || EPL16 > 16) ? 1 : 2;
    static_assert(RT::TBP % (16 * P) == 0, "tokens per wave pass");
    if constexpr (GRP) {  // group-limited select: one token per row at a time
        lds_u8* scr = scr_base + wv * (P * kRowScr + kDumpScr);
        for (int tb = 4 * wv; tb < RT::TBP; tb += 16) {
            const int tl = tb + (lane >> 4);
            int64_t t[1];
            bool live[1], kept[1];
            t[0] = t0 + tl;
            live[0] = t[0] < T;
            if (logits_out && live[0])
                for (int e = lane & 15; e < E; e += 16)
                    logits_out[t[0] * E + e] = static_cast<float>(lgs[tl * RT::EMAX + e]);
            kept[0] = live[0] && ((mask == nullptr) || (mask[t[0]] != 0));
            auto lg_of = [&](int, int e) { return lgs[tl * RT::EMAX + e]; };
            int my_e[1];
            double my_s[1];
            if constexpr (EPL16 > 16) {
                float bvi[EPL16];
                load_bias16<EPL16>(bias, E, bvi);
                rows16_grouped<EPL16>(lg_of, E, K, score, bvi, n_group, topk_group, my_e[0], my_s[0]);
            } else {
                rows16_grouped<EPL16>(lg_of, E, K, score, bv, n_group, topk_group, my_e[0], my_s[0]);
            }
            write_picks16<1>(my_e, my_s, t, live, kept, K, renorm, route_scale, ids_out, w_out, scr);
        }
    } else {
    for (int tb = 4 * P * wv; tb < RT::TBP; tb += 16 * P) {
        int64_t t[P];
        int tl[P];
        bool live[P], kept[P];
#pragma unroll
        for (int p = 0; p < P; ++p) {
            tl[p] = tb + 4 * p + (lane >> 4);
            t[p] = t0 + tl[p];
            live[p] = t[p] < T;
            if (logits_out && live[p])
                for (int e = lane & 15; e < E; e += 16)
                    logits_out[t[p] * E + e] = static_cast<float>(lgs[tl[p] * RT::EMAX + e]);
            kept[p] = live[p] && ((mask == nullptr) || (mask[t[p]] != 0));
        }
        auto lg_of = [&](int p, int e) { return lgs[tl[p] * RT::EMAX + e]; };
        int my_e[P];
        double my_s[P];
        lds_u8* scr = scr_base + wv * (P * kRowScr + kDumpScr);
        if constexpr (EPL16 > 16) {  // 32 bias registers held across the pass would spill
            float bvi[EPL16];
            load_bias16<EPL16>(bias, E, bvi);
            rows16_select<EPL16, P>(lg_of, live, E, K, score, bias, bvi, scr, my_e, my_s);
        } else {
            rows16_select<EPL16, P>(lg_of, live, E, K, score, bias, bv, scr, my_e, my_s);
        }
        write_picks16<P>(my_e, my_s, t, live, kept, K, renorm, route_scale, ids_out, w_out, scr);
    }
    }
}

// TOPK false: the same k loop, and the float64 logits go to logits64 [T][E]
// instead of the top-k (the logits of the two-kernel paths: group-limited
// select, replay, the backward's recompute).
template <int TBB, int NBW, bool TOPK = true, bool GRP = false>
__global__ __launch_bounds__(256) void route_fused_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int64_t T, int D, int E, int K,
    int score, int renorm, double route_scale, const float* __restrict__ bias,
    const uint8_t* __restrict__ mask, float* __restrict__ logits_out, int32_t* __restrict__ ids_out,
    float* __restrict__ w_out, int n_group, int topk_group, double* __restrict__ logits64) {
    using RT = RouteTile<TBB, NBW>;
    __shared__ __attribute__((aligned(1024))) uint8_t smem_raw[RT::SMEM];
    lds_u8* smem = (lds_u8*)(smem_raw);  // the array lives in LDS: an address-space cast
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * RT::TB;
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(smem));

    // DMA sources.  Each instruction moves 8 rows x 128 bytes; lane l lands
    // on row l / 8 at physical chunk l % 8 and fetches logical chunk
    // (l % 8) ^ (row % 8).  Hidden rows past T repeat row T-1 and router rows
    // past E repeat row E-1; their logits are never used.  Hidden-row offsets
    // are relative to the workgroup's first row, so they stay below TB*D*2.
    // Chunks past the end re-fetch the last chunk into a stage nothing reads
    // again, so every chunk issues the same instructions (uniform waits).
    const uint8_t* xb = reinterpret_cast<const uint8_t*>(x + t0 * D);
    const uint8_t* wb = reinterpret_cast<const uint8_t*>(w);
    const uint32_t row_bytes = static_cast<uint32_t>(D) * 2;
    const int chunk = (lane & 7) ^ (lane >> 3);
    const int ns = D / 64;
    // DMA i of this wave for hidden chunk st / router chunk st
    auto issue_x1 = [&](int st, int i) {
        const int c = st < ns ? st : ns - 1;
        const uint32_t kb = static_cast<uint32_t>(c) * 128 + chunk * 16;
        const uint32_t dst = lds0 + (st % RT::XS) * RT::XSTAGE;
        const int q = wv * RT::XPER + i;
        int64_t rr = 8 * q + (lane >> 3);
        if (t0 + rr >= T) rr = T - 1 - t0;
        dma16(xb, static_cast<uint32_t>(rr) * row_bytes + kb, dst + q * 1024);
    };
    auto issue_w1 = [&](int st, int i) {
        const int c = st < ns ? st : ns - 1;
        const uint32_t kb = static_cast<uint32_t>(c) * 128 + chunk * 16;
        const uint32_t dst = lds0 + RT::WOFF + (st % RT::WS) * RT::WSTAGE;
        const int q = wv * RT::WPER + i;
        int er = 8 * q + (lane >> 3);
        if (er >= E) er = E - 1;
        dma16(wb, static_cast<uint32_t>(er) * row_bytes + kb, dst + q * 1024);
    };
    double acc64[TBB][NBW][4];
#pragma unroll
    for (int a = 0; a < TBB; ++a)
#pragma unroll
        for (int b = 0; b < NBW; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc64[a][b][i] = 0.0;
    f32x4 acc[TBB][NBW];

    // fragment of half j of a chunk: logical chunk 4j + lane/16 of row
    // lane%16 (+16 per block), stored at chunk ^ (lane % 8)
    const int xo0 = ((lane >> 4) ^ (lane & 7)) << 4;
    const int xo1 = ((4 + (lane >> 4)) ^ (lane & 7)) << 4;
    const int arow = (lane & 15) * 128;
    const int brow = (wv * (16 * NBW) + (lane & 15)) * 128;

    // Chunk st needs hidden stage st and router stage st.  During chunk t,
    // after its barrier and spread over its MFMAs (a burst of DMAs would
    // stall the wave's issue), the DMAs of router chunk t+WS-1 and hidden
    // chunk t+XS-1 are issued (in that order) into the buffers chunk t-1
    // used; the router
    // chunk a step needs was issued WS-1 steps earlier, and only its own
    // step's hidden DMAs and the WS-2 later steps' DMAs are younger.
    constexpr int kWaitN = RT::XPER + (RT::WS - 2) * (RT::WPER + RT::XPER);
    for (int j = 0; j < RT::XS - 1; ++j)
#pragma unroll
        for (int i = 0; i < RT::XPER; ++i) issue_x1(j, i);
    for (int j = 0; j < RT::WS - 1; ++j)
#pragma unroll
        for (int i = 0; i < RT::WPER; ++i) issue_w1(j, i);
    wait_vmem<0>();
    // one k64 stage: wait, barrier, next DMAs, two MFMA k=32 steps into acc
    auto stage = [&](int st) {
        if (st > 0) wait_vmem<kWaitN>();
        __syncthreads();  // chunk st visible; every wave is done with chunk st-1
        const lds_u8* xs = smem + (st % RT::XS) * RT::XSTAGE;
        const lds_u8* ws = smem + RT::WOFF + (st % RT::WS) * RT::WSTAGE;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int xoj = j == 0 ? xo0 : xo1;
            u32x4 af[TBB];
#pragma unroll
            for (int a = 0; a < TBB; ++a) af[a] = *reinterpret_cast<lds_u32x4*>(xs + arow + a * 16 * 128 + xoj);
#pragma unroll
            for (int b = 0; b < NBW; ++b) {
                const u32x4 bf = *reinterpret_cast<lds_u32x4*>(ws + brow + b * 16 * 128 + xoj);
#pragma unroll
                for (int a = 0; a < TBB; ++a) acc[a][b] = mfma_bf16(af[a], bf, acc[a][b]);
                // this stage's DMAs spread over its MFMA groups, router rows first
                constexpr int kQ = RT::WPER + RT::XPER;
                constexpr int kSlots = 2 * NBW;
                const int slot = j * NBW + b;
#pragma unroll
                for (int q = slot * kQ / kSlots; q < (slot + 1) * kQ / kSlots; ++q) {
                    if (q < RT::WPER) issue_w1(st + RT::WS - 1, q);
                    else issue_x1(st + RT::XS - 1, q - RT::WPER);
                }
            }
        }
    };
    // 256-wide partial sums: four stages per fp32 accumulation, then float64
    for (int st = 0; st < ns; st += 4) {
#pragma unroll
        for (int a = 0; a < TBB; ++a)
#pragma unroll
            for (int b = 0; b < NBW; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
        stage(st);
        if (st + 1 < ns) stage(st + 1);
        if (st + 2 < ns) stage(st + 2);
        if (st + 3 < ns) stage(st + 3);
#pragma unroll
        for (int a = 0; a < TBB; ++a)
#pragma unroll
            for (int b = 0; b < NBW; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc64[a][b][i] += static_cast<double>(acc[a][b][i]);
    }
    wait_vmem<0>();
    __syncthreads();  // the stages are dead: the logits take their place

    // Logits to LDS, TBP tokens per pass ([TBP][EMAX] float64), and the
    // top-k of those tokens from there.
    __attribute__((address_space(3))) double* lgs = (__attribute__((address_space(3))) double*)(smem);
    float bv[RT::EMAX / 16];  // (loaded per token block instead past 256 experts)
    load_bias16<RT::EMAX / 16>(RT::EMAX > 256 ? nullptr : bias, E, bv);
    constexpr int NP = RT::TB / RT::TBP;  // passes
    static_assert(NP == 1 || NP == 2, "one or two top-k passes per tile");
    auto pass = [&](auto hc) {
        constexpr int h = decltype(hc)::value;
        if (h > 0) __syncthreads();  // the previous pass is done with its logits
#pragma unroll
        for (int a = 0; a < TBB; ++a) {
            if (a * 16 / RT::TBP != h) continue;
#pragma unroll
            for (int b = 0; b < NBW; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tl = a * 16 + 4 * (lane >> 4) + i - h * RT::TBP;
                    const int e = wv * (16 * NBW) + b * 16 + (lane & 15);
                    lgs[tl * RT::EMAX + e] = acc64[a][b][i];
                }
        }
        __syncthreads();
        const int64_t tp = t0 + h * RT::TBP;  // first token of the pass
        if constexpr (!TOPK) {
            // the pass's logits to memory, consecutive threads on consecutive logits
            const int rows = static_cast<int>(min(static_cast<int64_t>(RT::TBP), T - tp));
            for (int c = static_cast<int>(threadIdx.x); c < rows * E; c += 256) {
                const int r = c / E, e = c - r * E;
                logits64[(tp + r) * E + e] = lgs[r * RT::EMAX + e];
            }
        } else {
            route_topk_pass<RT, GRP, h == NP - 1>(lgs, smem + RT::LOGB, tp, T, E, K, score, renorm, route_scale, bias,
                                                  bv, n_group, topk_group, mask, logits_out, ids_out, w_out);
        }
    };
    pass(std::integral_constant<int, 0>{});
    if constexpr (NP > 1) pass(std::integral_constant<int, 1>{});
}

// ---------------------------------------------------------------------------
// router logits for decode-sized batches: one workgroup per 16 tokens x 16
// experts, operand fragments loaded straight from memory, kRdU 32-wide k
// steps (one 256-product chunk) in flight per wave.  The same MFMA chain,
// chunking (float32 over 256 products, then float64 in k order) and
// 16-aligned token and expert blocks as the kernels above, so the same bits.
// ---------------------------------------------------------------------------
constexpr int kRdU = 8;

// The chunks of a 16 x 16 block are spread over kSplitW waves: each wave
// computes one 256-product chunk per round (all of its loads in flight, the
// float32 MFMA chain from zero), the chunks meet in LDS, and each output adds
// them in float64 in chunk order.  A decode-sized batch has few blocks, so a
// wave per block walking the chunks one after another would wait for D/256
// dependent memory round trips; here there are D/(256 SW): SW = 16 waves when
// D > 2048 (one round for the 4096-wide layers), else 8.  Which wave computes
// a chunk changes no bit.
template <int SW>
__global__ __launch_bounds__(64 * SW) void router_logits_split_kernel(const uint16_t* __restrict__ x,
                                                                   const uint16_t* __restrict__ w, int64_t T, int D,
                                                                   int E, double* __restrict__ out) {
    constexpr int kSplitW = SW;
    __shared__ __attribute__((aligned(16))) float part[kSplitW][64][4];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * 16;
    const int e0 = blockIdx.y * 16;
    int64_t tr = t0 + (lane & 15);
    if (tr > T - 1) tr = T - 1;  // rows past T repeat row T-1; never stored
    int er = e0 + (lane & 15);
    if (er > E - 1) er = E - 1;
    const int kq = 8 * (lane >> 4);
    const uint16_t* xp = x + tr * D + kq;
    const uint16_t* wp = w + static_cast<int64_t>(er) * D + kq;
    const int S = D / 32;
    const int nc = (S + kRdU - 1) / kRdU;  // 256-product chunks (the last may be short)
    double acc64 = 0.0;                    // output (tid / 4, element tid % 4) of the MFMA layout
    for (int c0 = 0; c0 < nc; c0 += kSplitW) {
        const int c = c0 + wv;
        if (c < nc) {  // uniform per wave
            const int s0 = c * kRdU;
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
            if (s0 + kRdU <= S) {
                // a full chunk: no branch between the loads and their MFMAs,
                // so the compiler cannot sink a load down to its use
                u32x4 a[kRdU], b[kRdU];
#pragma unroll
                for (int u = 0; u < kRdU; ++u) {
                    a[u] = *reinterpret_cast<const u32x4*>(xp + 32 * (s0 + u));
                    b[u] = *reinterpret_cast<const u32x4*>(wp + 32 * (s0 + u));
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int u = 0; u < kRdU; ++u) acc = mfma_bf16(a[u], b[u], acc);
            } else {
                for (int st = s0; st < S; ++st)  // the short last chunk when D % 256 != 0
                    acc = mfma_bf16(*reinterpret_cast<const u32x4*>(xp + 32 * st),
                                    *reinterpret_cast<const u32x4*>(wp + 32 * st), acc);
            }
            *reinterpret_cast<f32x4*>(&part[wv][lane][0]) = acc;
        }
        __syncthreads();
        if (tid < 256) {
            const int n = nc - c0 < kSplitW ? nc - c0 : kSplitW;
            for (int j = 0; j < n; ++j) acc64 += static_cast<double>(part[j][tid >> 2][tid & 3]);
        }
        __syncthreads();
    }
    if (tid < 256) {
        const int l = tid >> 2;
        const int e = e0 + (l & 15);
        const int64_t t = t0 + 4 * (l >> 4) + (tid & 3);
        if (t < T && e < E) out[t * E + e] = acc64;
    }
}

// whether the decode-sized router (small logits kernel + top-k kernel) runs:
// small batches, and with at most 16 experts up to 8192 tokens, where the
// fused router's 64-expert waves would mostly compute clamped rows (top-1
// draft layer, E = 8, T = 4096: 21.5 -> 15.3 us; at T = 16384 the fused
// router is faster again, 33.5 against 36.2 us)
static bool route_small(int64_t T, int E, int dtype) {
    return dtype == 0 && (T <= 1024 || (E <= 16 && T <= 8192)) && T * E <= kRouteSmallTE;
}

// The fused router's workgroup tile for T tokens and E <= 512 experts: TBB
// 16-token blocks, NBW 16-expert blocks per wave.  Larger token tiles cut the
// router-matrix traffic per token once there are enough of them to give every
// CU one; smaller ones keep every CU busy on shorter batches.  The logits and
// picks do not depend on the tile.
static void route_tile(int64_t T, int E, int& tbb, int& nbw) {
    const int64_t cus = compute_units();
    const bool wide = T >= 64 * cus;
    if (E <= 64) { tbb = wide ? 4 : 2; nbw = 1; }
    else if (E <= 128) { tbb = wide ? 4 : 2; nbw = 2; }
    else if (E <= 256) { tbb = T >= 128 * cus ? 8 : 4; nbw = 4; }
    else { tbb = wide ? 4 : 2; nbw = 8; }
}

hipError_t launch_router_logits(const void* x, const void* router, int64_t T, int D, int E,
                                int dtype, double* logits64, hipStream_t stream) {
    if (dtype == 0 && E <= 512 && !route_small(T, E, dtype)) {
        // the fused router's k loop, logits to memory
        int tbb = 0, nbw = 0;
        route_tile(T, E, tbb, nbw);
        // (the 128-token tile of this variant spills inside its k loop, where
        // a reload waits for every DMA in flight: 64-token tiles instead)
        if (tbb == 8) tbb = 4;
        const uint16_t* xb = static_cast<const uint16_t*>(x);
        const uint16_t* wb = static_cast<const uint16_t*>(router);
#define MOE_LOGITS(TBB, NBW)                                                                                  \
    route_fused_bf16_kernel<TBB, NBW, false><<<static_cast<unsigned>((T + 16 * TBB - 1) / (16 * TBB)), 256, 0, \
                                                stream>>>(xb, wb, T, D, E, 0, 0, 0, 0.0, nullptr, nullptr,      \
                                                          nullptr, nullptr, nullptr, 1, 1, logits64)
        if (tbb == 4 && nbw == 1) MOE_LOGITS(4, 1);
        else if (tbb == 2 && nbw == 1) MOE_LOGITS(2, 1);
        else if (tbb == 4 && nbw == 2) MOE_LOGITS(4, 2);
        else if (tbb == 2 && nbw == 2) MOE_LOGITS(2, 2);
        else if (tbb == 4 && nbw == 4) MOE_LOGITS(4, 4);
        else if (tbb == 4 && nbw == 8) MOE_LOGITS(4, 8);
        else MOE_LOGITS(2, 8);
#undef MOE_LOGITS
        return hipGetLastError();
    }
    if (route_small(T, E, dtype)) {
        dim3 grid(static_cast<unsigned>((T + 15) / 16), static_cast<unsigned>((E + 15) / 16));
        const uint16_t* xb = static_cast<const uint16_t*>(x);
        const uint16_t* wb = static_cast<const uint16_t*>(router);
        if (D > 2048) router_logits_split_kernel<16><<<grid, 64 * 16, 0, stream>>>(xb, wb, T, D, E, logits64);
        else router_logits_split_kernel<8><<<grid, 64 * 8, 0, stream>>>(xb, wb, T, D, E, logits64);
        return hipGetLastError();
    }
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

// whether a layer's top-k runs in rows of sixteen lanes (rows16_select or
// rows16_grouped, and rows16_given) on every path, or one token per wave
// (topk_token) on every path
static bool topk_rows16(int E, int n_group) { return E <= 512 && (n_group <= 1 || grouped16_sp(E, n_group) > 0); }

hipError_t launch_topk(const double* logits64, int64_t T, int E, int K, int score, int renorm,
                       float route_scale, int n_group, int topk_group, const float* bias, const uint8_t* mask,
                       float* logits_out, int32_t* ids, float* w, hipStream_t stream, const int32_t* given) {
    const double rs = static_cast<double>(route_scale);
    if (topk_rows16(E, n_group)) {
        const unsigned grid = static_cast<unsigned>((T + 15) / 16);
#define MOE_TOPK16_G(EPL16, GRP)                                                                              \
    topk_rows16_kernel<EPL16, GRP><<<grid, 256, 0, stream>>>(logits64, T, E, K, score, renorm, rs, bias, mask, \
                                                              logits_out, ids, w, given, n_group, topk_group)
#define MOE_TOPK16(EPL16)                                                        \
    do {                                                                         \
        if (n_group > 1 && given == nullptr) MOE_TOPK16_G(EPL16, true);          \
        else MOE_TOPK16_G(EPL16, false);                                         \
    } while (0)
        if (E <= 64) MOE_TOPK16(4);
        else if (E <= 128) MOE_TOPK16(8);
        else if (E <= 256) MOE_TOPK16(16);
        else MOE_TOPK16(32);
#undef MOE_TOPK16
#undef MOE_TOPK16_G
        return hipGetLastError();
    }
    const unsigned grid = static_cast<unsigned>((T + 3) / 4);
#define MOE_TOPK(EPL)                                                                                   \
    topk_kernel<EPL><<<grid, 256, 0, stream>>>(logits64, T, E, K, score, renorm, rs, bias, mask, \
                                                logits_out, ids, w, given, n_group, topk_group)
    if (E <= 64) MOE_TOPK(1);
    else if (E <= 128) MOE_TOPK(2);
    else if (E <= 256) MOE_TOPK(4);
    else if (E <= 512) MOE_TOPK(8);
    else MOE_TOPK(16);
#undef MOE_TOPK
    return hipGetLastError();
}

bool route_permute_fused(int64_t T) { return T >= 1 && T <= kTopkPermuteT; }

hipError_t launch_route_permute(const void* x, const void* router, int64_t T, int D, int E, int K, int dtype,
                                int score, int renorm, float route_scale, int n_group, int topk_group,
                                const float* bias, const int32_t* given, const uint8_t* mask, double* logits64,
                                float* logits_out, int32_t* ids, float* w, int32_t* counts, int32_t* offsets,
                                int32_t* perm_token, int32_t* inv_pos, hipStream_t stream) {
    hipError_t err = launch_router_logits(x, router, T, D, E, dtype, logits64, stream);
    if (err != hipSuccess) return err;
    const double rs = static_cast<double>(route_scale);  // one workgroup: T * K <= 8 * 16 pairs
    if (topk_rows16(E, n_group)) {
#define MOE_TOPK16_PERMUTE_G(EPL16, GRP)                                                                     \
    topk_permute_rows16_kernel<EPL16, GRP><<<1, 256, 0, stream>>>(logits64, T, E, K, score, renorm, rs, bias,  \
                                                                  mask, logits_out, ids, w, given, n_group,    \
                                                                  topk_group, counts, offsets, perm_token,     \
                                                                  inv_pos)
#define MOE_TOPK16_PERMUTE(EPL16)                                                \
    do {                                                                         \
        if (n_group > 1 && given == nullptr) MOE_TOPK16_PERMUTE_G(EPL16, true);  \
        else MOE_TOPK16_PERMUTE_G(EPL16, false);                                 \
    } while (0)
        if (E <= 64) MOE_TOPK16_PERMUTE(4);
        else if (E <= 128) MOE_TOPK16_PERMUTE(8);
        else if (E <= 256) MOE_TOPK16_PERMUTE(16);
        else MOE_TOPK16_PERMUTE(32);
#undef MOE_TOPK16_PERMUTE
#undef MOE_TOPK16_PERMUTE_G
        return hipGetLastError();
    }
#define MOE_TOPK_PERMUTE(EPL)                                                                               \
    topk_permute_kernel<EPL><<<1, 256, 0, stream>>>(logits64, T, E, K, score, renorm, rs, bias, mask,      \
                                                    logits_out, ids, w, given, n_group, topk_group, counts, \
                                                    offsets, perm_token, inv_pos)
    if (E <= 64) MOE_TOPK_PERMUTE(1);
    else if (E <= 128) MOE_TOPK_PERMUTE(2);
    else if (E <= 256) MOE_TOPK_PERMUTE(4);
    else if (E <= 512) MOE_TOPK_PERMUTE(8);
    else MOE_TOPK_PERMUTE(16);
#undef MOE_TOPK_PERMUTE
    return hipGetLastError();
}

// (group-limited select in the fused kernel up to 256 experts: past that its
// float64 choices of every slot, next to the other pass's logits, spill into
// the k loop; the two-kernel path takes those layers)
bool route_fused(int E, int dtype, int n_group) {
    return dtype == 0 && E <= 512 && (n_group <= 1 || (E <= 256 && grouped16_sp(E, n_group) > 0));
}

hipError_t launch_route(const void* x, const void* router, int64_t T, int D, int E, int K, int dtype,
                        int score, int renorm, float route_scale, int n_group, int topk_group, const float* bias,
                        const uint8_t* mask, double* logits64, float* logits_out, int32_t* ids, float* w,
                        hipStream_t stream) {
    if (!route_fused(E, dtype, n_group) || route_small(T, E, dtype)) {
        hipError_t err = launch_router_logits(x, router, T, D, E, dtype, logits64, stream);
        if (err != hipSuccess) return err;
        return launch_topk(logits64, T, E, K, score, renorm, route_scale, n_group, topk_group, bias, mask,
                           logits_out, ids, w, stream, nullptr);
    }
    const double rs = static_cast<double>(route_scale);
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    const uint16_t* wb = static_cast<const uint16_t*>(router);
#define MOE_ROUTE_G(TBB, NBW, GRP)                                                                          \
    route_fused_bf16_kernel<TBB, NBW, true, GRP><<<static_cast<unsigned>((T + 16 * TBB - 1) / (16 * TBB)), 256, \
                                                   0, stream>>>(xb, wb, T, D, E, K, score, renorm, rs, bias, mask, \
                                                                logits_out, ids, w, n_group, topk_group, nullptr)
#define MOE_ROUTE(TBB, NBW)                                 \
    do {                                                    \
        if (n_group > 1) MOE_ROUTE_G(TBB, NBW, true);       \
        else MOE_ROUTE_G(TBB, NBW, false);                  \
    } while (0)
    int tbb = 0, nbw = 0;
    route_tile(T, E, tbb, nbw);
    if (tbb == 4 && nbw == 1) MOE_ROUTE(4, 1);
    else if (tbb == 2 && nbw == 1) MOE_ROUTE(2, 1);
    else if (tbb == 4 && nbw == 2) MOE_ROUTE(4, 2);
    else if (tbb == 2 && nbw == 2) MOE_ROUTE(2, 2);
    else if (tbb == 8 && nbw == 4) MOE_ROUTE(8, 4);
    else if (tbb == 4 && nbw == 4) MOE_ROUTE(4, 4);
    else if (tbb == 4 && nbw == 8) MOE_ROUTE(4, 8);
    else MOE_ROUTE(2, 8);
#undef MOE_ROUTE
#undef MOE_ROUTE_G
    return hipGetLastError();
}

hipError_t launch_route_replay(const void* x, const void* router, int64_t T, int D, int E, int K, int dtype,
                               int score, int renorm, float route_scale, int n_group, const int32_t* given,
                               const uint8_t* mask, double* logits64, float* logits_out, int32_t* ids, float* w,
                               hipStream_t stream) {
    hipError_t err = launch_router_logits(x, router, T, D, E, dtype, logits64, stream);
    if (err != hipSuccess) return err;
    // n_group only picks the top-k code the layer's forward runs (so a
    // replayed token gets the forward's weight bits); given ids skip the
    // group-limited select itself
    return launch_topk(logits64, T, E, K, score, renorm, route_scale, n_group, 1, nullptr, mask, logits_out, ids, w,
                       stream, given);
}

}  // namespace moe
