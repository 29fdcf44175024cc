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
// in float64).  Scores, choices and weights are then float64; the weights are
// rounded once to float32.
#include "common.hpp"
#include "kernels.hpp"
#include "permute_block.hpp"

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

// The picks of P rows (lane r of a row holds its r-th pick: my_e, my_s) in
// ascending id order with their weights, to ids_out / w_out.
template <int P>
__device__ __forceinline__ void write_picks16(const int (&my_e)[P], const double (&my_s)[P], const int64_t (&t)[P],
                                              const bool (&live)[P], const bool (&kept)[P], int K, int renorm,
                                              double route_scale, int32_t* __restrict__ ids_out,
                                              float* __restrict__ w_out) {
    const int lane = lane_id();
    const int j = lane & 15;
    const int rbase = lane & 48;
#pragma unroll
    for (int p = 0; p < P; ++p) {
        // ascending id order: rank of each pick among the row's K picks
        int rank = 0;
        for (int i = 0; i < K; ++i) {
            const int ei = lane_get(my_e[p], rbase + i);
            rank += (j < K && ei < my_e[p]) ? 1 : 0;
        }
        double den = 1.0;
        if (renorm) {
            den = 0.0;
            for (int r = 0; r < K; ++r) {
                const uint64_t holders = __ballot(j < K && rank == r);
                const int holder = __builtin_ctzll((holders >> rbase) & 0xFFFFull) + rbase;
                den += lane_get_f64(my_s[p], holder);
            }
        }
        if (live[p] && j < K) {
            if (kept[p]) {
                const double wv = renorm ? (my_s[p] / den) * route_scale : my_s[p] * route_scale;
                ids_out[t[p] * K + rank] = my_e[p];
                w_out[t[p] * K + rank] = static_cast<float>(wv);
            } else {
                ids_out[t[p] * K + j] = -1;
                w_out[t[p] * K + j] = 0.f;
            }
        }
    }
}

// Elementwise scores (sigmoid, sqrtsoftplus), screened: the same picks and
// scores as select_rows16, with float64 scores computed only for the few
// experts that can be picked.  Every choice c = score(l) + bias is first
// evaluated in float32 (c32, within about 1e-6 + 1e-7 |c| of the float64
// value, far inside the margin below).
// mu, the K-th largest of the 16 lanes' largest c32, is at most the K-th
// largest c32 (K lanes hold a value >= mu), so every expert the float64
// choice can pick has c32 >= mu - margin.  Those candidates are compacted
// one per lane through the wave's LDS scratch (16 bytes per slot, P x 64
// slots), get their float64 choice exactly as select_rows16 computes it, and
// K rounds of row argmax pick among them.  Returns false, with no picks,
// when a row of the wave has more than 16 candidates.
template <int EPL16, int P>
__device__ __forceinline__ bool select_rows16_screened(const double (&lg)[P][EPL16], int E, int K, int score,
                                                       const float* __restrict__ bias, lds_u8* scr, int (&my_e)[P],
                                                       double (&my_s)[P]) {
    const int lane = lane_id();
    const int j = lane & 15;
    const int row = lane >> 4;
    bool ok[EPL16];
    float bv[EPL16];
#pragma unroll
    for (int i = 0; i < EPL16; ++i) {
        ok[i] = j + 16 * i < E;
        bv[i] = (bias != nullptr && ok[i]) ? bias[j + 16 * i] : 0.0f;
    }
    uint32_t cm[P];  // candidate bits over i
    int off[P], n_row[P];
    bool over = false;
#pragma unroll
    for (int p = 0; p < P; ++p) {
        float c32[EPL16];
#pragma unroll
        for (int i = 0; i < EPL16; ++i) {
            const float l = static_cast<float>(lg[p][i]);
            float sc32;
            if (score == 2) sc32 = sqrtf(fmaxf(l, 0.0f) + log1pf(__expf(-fabsf(l))));
            else sc32 = __builtin_amdgcn_rcpf(1.0f + __expf(-l));
            c32[i] = ok[i] ? sc32 + bv[i] : -INFINITY;
        }
        float m[EPL16];
#pragma unroll
        for (int i = 0; i < EPL16; ++i) m[i] = c32[i];
#pragma unroll
        for (int w = EPL16 / 2; w >= 1; w /= 2)
#pragma unroll
            for (int i = 0; i < w; ++i) m[i] = fmaxf(m[i], m[i + w]);
        float v = m[0], mu = -INFINITY;
        for (int r = 0; r < K; ++r) {
            mu = row_max_f32(v);
            v = v == mu ? -INFINITY : v;  // equal lane maxima go together: mu only gets smaller
        }
        const float thr = mu - (1e-5f + 1e-6f * fabsf(mu));
        cm[p] = 0u;
#pragma unroll
        for (int i = 0; i < EPL16; ++i)
            if (ok[i] && c32[i] >= thr) cm[p] |= 1u << i;
        const int nl = __builtin_popcount(cm[p]);
        const int incl = row_scan_i32(nl);
        off[p] = incl - nl;
        n_row[p] = row_max_i32(incl);
        over = over || n_row[p] > 16;
    }
    if (__ballot(over) != 0) return false;

    // compaction: candidate k of row r of pass p at slot (p, r, k)
#pragma unroll
    for (int p = 0; p < P; ++p) {
        int k = off[p];
#pragma unroll
        for (int i = 0; i < EPL16; ++i) {
            if ((cm[p] >> i) & 1u) {
                lds_u8* sl = scr + ((p * 4 + row) * 16 + k) * 16;
                *reinterpret_cast<__attribute__((address_space(3))) double*>(sl) = lg[p][i];
                *reinterpret_cast<__attribute__((address_space(3))) int*>(sl + 8) = j + 16 * i;
                *reinterpret_cast<__attribute__((address_space(3))) float*>(sl + 12) = bv[i];
                ++k;
            }
        }
    }
    uint64_t key[P];
    double sc[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        key[p] = 0ull;
        sc[p] = 0.0;
        if (j < n_row[p]) {
            const lds_u8* sl = scr + ((p * 4 + row) * 16 + j) * 16;
            const double l = *reinterpret_cast<const __attribute__((address_space(3))) double*>(sl);
            const int e = *reinterpret_cast<const __attribute__((address_space(3))) int*>(sl + 8);
            const float b = *reinterpret_cast<const __attribute__((address_space(3))) float*>(sl + 12);
            sc[p] = elem_score(l, score);
            double c = sc[p];
            if (bias != nullptr) c += static_cast<double>(b);
            key[p] = choice_key(c, e);
        }
    }

    // K rounds of row argmax over the candidates; lane r keeps the r-th pick
#pragma unroll
    for (int p = 0; p < P; ++p) {
        my_e[p] = -1;
        my_s[p] = 0.0;
    }
    for (int r = 0; r < K; ++r) {
        uint64_t win[P];
#pragma unroll
        for (int p = 0; p < P; ++p) win[p] = row_max_u64(key[p]);
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const bool mine = key[p] == win[p];
            const double sw = row_max_f64(mine ? sc[p] : -1.0);
            if (mine) key[p] = 0ull;
            if (j == r) {
                my_e[p] = 1023 - static_cast<int>(win[p] & 0x3FFull);
                my_s[p] = sw;
            }
        }
    }
    return true;
}

// P tokens per row of 16 lanes: token t[p] of this lane's row, whose float64
// logits the row holds (EPL16 per lane: experts j, j + 16, ... for lane j of
// the row).  The P tokens are independent and handled side by side, so their
// dependent chains (row reductions, K argmax rounds) overlap.  Every lane of
// the wave must call it (rows whose token does not exist pass live = false
// and write nothing).  Same arithmetic as topk_token except the order of the
// softmax sums across lanes.
template <int EPL16, int P>
__device__ __forceinline__ void select_rows16(const double (&lg)[P][EPL16], int E, int K, int score,
                                              const float* __restrict__ bias, int (&my_e)[P], double (&my_s)[P]) {
    const int lane = lane_id();
    const int j = lane & 15;
    bool ok[EPL16];
#pragma unroll
    for (int i = 0; i < EPL16; ++i) ok[i] = j + 16 * i < E;

    double s[P][EPL16];
    if (score == 0) {
        double m[P];
#pragma unroll
        for (int p = 0; p < P; ++p) {
            m[p] = -1.7976931348623157e308;
#pragma unroll
            for (int i = 0; i < EPL16; ++i)
                if (ok[i]) m[p] = fmax(m[p], lg[p][i]);
        }
#pragma unroll
        for (int p = 0; p < P; ++p) m[p] = row_max_f64(m[p]);
        double part[P];
#pragma unroll
        for (int p = 0; p < P; ++p) {
            part[p] = 0.0;
#pragma unroll
            for (int i = 0; i < EPL16; ++i) {
                s[p][i] = ok[i] ? exp(lg[p][i] - m[p]) : 0.0;
                part[p] += s[p][i];
            }
        }
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const double z = row_sum_f64(part[p]);
#pragma unroll
            for (int i = 0; i < EPL16; ++i) s[p][i] = s[p][i] / z;
        }
    } else {
#pragma unroll
        for (int p = 0; p < P; ++p)
#pragma unroll
            for (int i = 0; i < EPL16; ++i) s[p][i] = ok[i] ? elem_score(lg[p][i], score) : 0.0;
    }

    uint64_t key[P][EPL16];
#pragma unroll
    for (int i = 0; i < EPL16; ++i) {
        const int e = j + 16 * i;
        const double b = (bias != nullptr && ok[i]) ? static_cast<double>(bias[e]) : 0.0;
#pragma unroll
        for (int p = 0; p < P; ++p) {
            double c = s[p][i];
            if (bias != nullptr && ok[i]) c += b;
            key[p][i] = ok[i] ? choice_key(c, e) : 0ull;
        }
    }

    // K rounds of row argmax; lane r of the row keeps the r-th pick
#pragma unroll
    for (int p = 0; p < P; ++p) {
        my_e[p] = -1;
        my_s[p] = 0.0;
    }
    for (int r = 0; r < K; ++r) {
        uint64_t win[P];
#pragma unroll
        for (int p = 0; p < P; ++p) {
            uint64_t m[EPL16];  // the lane's largest key, as a tree
#pragma unroll
            for (int i = 0; i < EPL16; ++i) m[i] = key[p][i];
#pragma unroll
            for (int w = EPL16 / 2; w >= 1; w /= 2)
#pragma unroll
                for (int i = 0; i < w; ++i) m[i] = umax64(m[i], m[i + w]);
            win[p] = m[0];
        }
#pragma unroll
        for (int p = 0; p < P; ++p) win[p] = row_max_u64(win[p]);
        double sw[P];
        int ew[P];
#pragma unroll
        for (int p = 0; p < P; ++p) {
            ew[p] = 1023 - static_cast<int>(win[p] & 0x3FFull);
            const int owner = ew[p] & 15;
            const int slot = ew[p] >> 4;
            sw[p] = -1.0;  // scores are >= 0: the row max picks the owner's value
#pragma unroll
            for (int i = 0; i < EPL16; ++i) {
                if (j == owner && i == slot) {
                    sw[p] = s[p][i];
                    key[p][i] = 0ull;
                }
            }
        }
#pragma unroll
        for (int p = 0; p < P; ++p) {
            sw[p] = row_max_f64(sw[p]);
            if (j == r) {
                my_e[p] = ew[p];
                my_s[p] = sw[p];
            }
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
// follows as permute_single_kernel computes it.
template <int EPL>
__global__ __launch_bounds__(256) void topk_permute_kernel(
    const double* __restrict__ logits, int64_t T, int E, int K, int score, int renorm, double route_scale,
    const float* __restrict__ bias, const uint8_t* __restrict__ mask, float* __restrict__ logits_out,
    int32_t* __restrict__ ids_out, float* __restrict__ w_out, const int32_t* __restrict__ given, int n_group,
    int topk_group, int ppb, int id_bits, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
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
    permute_one_block(ids_out, T * K, K, E, ppb, id_bits, counts, offsets, perm_token, inv_pos);
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
    static constexpr int SCRB = 4 * 2 * 64 * 16;  // top-k candidate slots: 4 waves x 2 passes x 64
    static constexpr int SMEM = RING > LOGB + SCRB ? RING : LOGB + SCRB;
    static constexpr int XPER = TB / 32;       // 8-row DMA instructions per wave per chunk
    static constexpr int WPER = EMAX / 32;
    static_assert(TB % 32 == 0 && EMAX % 32 == 0, "8-row DMA groups over 4 waves");
    static_assert(SMEM <= 160 * 1024, "LDS");
};

// Top-k of the TBP tokens starting at token tp whose float64 logits are in
// lgs ([TBP][EMAX]); scr: the candidate slots of the screened selection.
template <typename RT>
__device__ __forceinline__ void route_topk_pass(const __attribute__((address_space(3))) double* lgs, lds_u8* scr_base,
                                                int64_t tp, int64_t T, int E, int K, int score, int renorm,
                                                double route_scale, const float* __restrict__ bias,
                                                const uint8_t* __restrict__ mask, float* __restrict__ logits_out,
                                                int32_t* __restrict__ ids_out, float* __restrict__ w_out) {
    const int lane = lane_id();
    const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const int64_t t0 = tp;
    if constexpr (RT::EMAX <= 256) {
        // P tokens per row of sixteen lanes at a time
        constexpr int EPL16 = RT::EMAX / 16;
        // two tokens per row where registers allow; the 128-token tile holds
        // the other pass's logits in registers meanwhile
        constexpr int P = RT::TB > RT::TBP ? 1 : 2;
        static_assert(RT::TBP % (16 * P) == 0, "tokens per wave pass");
        for (int tb = 4 * P * wv; tb < RT::TBP; tb += 16 * P) {
            double lg[P][EPL16];
            int64_t t[P];
            bool live[P], kept[P];
#pragma unroll
            for (int p = 0; p < P; ++p) {
                const int tl = tb + 4 * p + (lane >> 4);
                t[p] = t0 + tl;
                live[p] = t[p] < T;
#pragma unroll
                for (int i = 0; i < EPL16; ++i) {
                    const int e = (lane & 15) + 16 * i;
                    lg[p][i] = lgs[tl * RT::EMAX + e];
                    if (logits_out && live[p] && e < E) logits_out[t[p] * E + e] = static_cast<float>(lg[p][i]);
                }
                kept[p] = live[p] && ((mask == nullptr) || (mask[t[p]] != 0));
            }
            lds_u8* scr = scr_base + wv * (P * 64 * 16);
            int my_e[P];
            double my_s[P];
            if (score == 0 || !select_rows16_screened<EPL16, P>(lg, E, K, score, bias, scr, my_e, my_s))
                select_rows16<EPL16, P>(lg, E, K, score, bias, my_e, my_s);
            write_picks16<P>(my_e, my_s, t, live, kept, K, renorm, route_scale, ids_out, w_out);
        }
    } else {
        for (int tl = wv; tl < RT::TBP; tl += 4) {
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
            topk_token<RT::EPL>(lg, t, E, K, score, renorm, route_scale, bias, kept, ids_out, w_out, nullptr, 1, 1);
        }
    }
}

template <int TBB, int NBW>
__global__ __launch_bounds__(256) void route_fused_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int64_t T, int D, int E, int K,
    int score, int renorm, double route_scale, const float* __restrict__ bias,
    const uint8_t* __restrict__ mask, float* __restrict__ logits_out, int32_t* __restrict__ ids_out,
    float* __restrict__ w_out) {
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
#pragma unroll
    for (int h = 0; h < RT::TB / RT::TBP; ++h) {
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
        route_topk_pass<RT>(lgs, smem + RT::LOGB, tp, T, E, K, score, renorm, route_scale, bias, mask, logits_out,
                            ids_out, w_out);
    }
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
// dependent memory round trips; here there are D/2048.
constexpr int kSplitW = 8;

__global__ __launch_bounds__(64 * kSplitW) void router_logits_split_kernel(const uint16_t* __restrict__ x,
                                                                        const uint16_t* __restrict__ w, int64_t T,
                                                                        int D, int E, double* __restrict__ out) {
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

// whether the decode-sized router (small logits kernel + top-k kernel) runs
static bool route_small(int64_t T, int E, int dtype) {
    return dtype == 0 && T <= 1024 && T * E <= kRouteSmallTE;
}

hipError_t launch_router_logits(const void* x, const void* router, int64_t T, int D, int E,
                                int dtype, double* logits64, hipStream_t stream) {
    if (route_small(T, E, dtype)) {
        dim3 grid(static_cast<unsigned>((T + 15) / 16), static_cast<unsigned>((E + 15) / 16));
        router_logits_split_kernel<<<grid, 64 * kSplitW, 0, stream>>>(
            static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(router), T, D, E, logits64);
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

hipError_t launch_topk(const double* logits64, int64_t T, int E, int K, int score, int renorm,
                       float route_scale, int n_group, int topk_group, const float* bias, const uint8_t* mask,
                       float* logits_out, int32_t* ids, float* w, hipStream_t stream, const int32_t* given) {
    const unsigned grid = static_cast<unsigned>((T + 3) / 4);
    const double rs = static_cast<double>(route_scale);
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
    const PermutePlan pl = permute_plan(T * K, E);  // one block: T * K <= 8 * 16 pairs
    const double rs = static_cast<double>(route_scale);
#define MOE_TOPK_PERMUTE(EPL)                                                                               \
    topk_permute_kernel<EPL><<<1, 256, 0, stream>>>(logits64, T, E, K, score, renorm, rs, bias, mask,      \
                                                    logits_out, ids, w, given, n_group, topk_group,         \
                                                    pl.pairs_per_block, pl.id_bits, counts, offsets, perm_token, \
                                                    inv_pos)
    if (E <= 64) MOE_TOPK_PERMUTE(1);
    else if (E <= 128) MOE_TOPK_PERMUTE(2);
    else if (E <= 256) MOE_TOPK_PERMUTE(4);
    else if (E <= 512) MOE_TOPK_PERMUTE(8);
    else MOE_TOPK_PERMUTE(16);
#undef MOE_TOPK_PERMUTE
    return hipGetLastError();
}

bool route_fused(int E, int dtype, int n_group) { return dtype == 0 && E <= 512 && n_group <= 1; }

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
#define MOE_ROUTE(TBB, NBW)                                                                              \
    route_fused_bf16_kernel<TBB, NBW><<<static_cast<unsigned>((T + 16 * TBB - 1) / (16 * TBB)), 256, 0, \
                                         stream>>>(xb, wb, T, D, E, K, score, renorm, rs, bias, mask,      \
                                                   logits_out, ids, w)
    // Larger token tiles cut the router-matrix traffic per token once there
    // are enough of them to give every CU one; smaller ones keep every CU
    // busy on shorter batches.  The logits and picks do not depend on the
    // tile.
    const bool wide = T >= 64 * static_cast<int64_t>(compute_units());
    if (E <= 64 && wide) MOE_ROUTE(4, 1);
    else if (E <= 64) MOE_ROUTE(2, 1);
    else if (E <= 128 && wide) MOE_ROUTE(4, 2);
    else if (E <= 128) MOE_ROUTE(2, 2);
    else if (E <= 256 && T >= 128 * static_cast<int64_t>(compute_units())) MOE_ROUTE(8, 4);
    else if (E <= 256) MOE_ROUTE(4, 4);
    else if (T >= 64 * static_cast<int64_t>(compute_units())) MOE_ROUTE(4, 8);
    else MOE_ROUTE(2, 8);
#undef MOE_ROUTE
    return hipGetLastError();
}

hipError_t launch_route_replay(const void* x, const void* router, int64_t T, int D, int E, int K, int dtype,
                               int score, int renorm, float route_scale, const int32_t* given,
                               const uint8_t* mask, double* logits64, float* logits_out, int32_t* ids, float* w,
                               hipStream_t stream) {
    hipError_t err = launch_router_logits(x, router, T, D, E, dtype, logits64, stream);
    if (err != hipSuccess) return err;
    return launch_topk(logits64, T, E, K, score, renorm, route_scale, 1, 1, nullptr, mask, logits_out, ids, w,
                       stream, given);
}

}  // namespace moe
