// Backward of the sparse-MoE layer: the gradients of the hidden states and of
// every weight, given the gradient G of the layer output.
//
// The RL-Kernel roadmap ("DSV4 Flash MoE Train-Inference Consistency
// Roadmap": the scope list and the issue-bucket table) puts forward +
// backward with a deterministic reduction order in scope, without formulas.
// Read as the gradients of this library's forward with the top-k selection
// fixed and the bf16 rounding points passed straight through.  Every sum runs
// in a fixed order without atomics, so repeated runs give the same bits, and
// the gradient of a token's hidden state does not depend on the other tokens.
//
// Steps (P routed pairs, rows in the forward's expert order; bf16 operands,
// float32 accumulation):
//   combine_bwd   dY[p] = bf16(w * G[t]);  dw[t, j] = <G[t], y[p]> (float64)
//   gemm          H = X W1_e^T, rows gathered (float32, recomputed)
//   gemm          dA = dY W2_e (float32)
//   swiglu_bwd    A = bf16(silu(g) u) as the forward formed it;
//                 dH = bf16([dA u silu'(g), dA silu(g)])
//   gemm          dW2_e = dY_e^T A_e, K-grouped (float32)
//   gemm          dXp = dH W1_e (float32)
//   gemm          dW1_e = dH_e^T X_e, K-grouped, rows gathered
//   (the same for the shared expert, with dY = G on every kept token)
//   router_bwd    dl[t, e] from dw through the weights and the score (bf16)
//   gemm          dx_r = dl W_r;  gemm  dW_r = dl^T x (K-grouped, one group)
//   dx_assemble   dx[t] = sum_j dXp[p_j] (ascending expert id) + dX_shared[t] + dx_r[t]
#include "common.hpp"
#include "kernels.hpp"

#include <math.h>

namespace moe {

// ===========================================================================
// Generic grouped GEMM for the backward: C[m][n] = sum_k A(m, k) B(k, n),
// bf16 operands, float32 accumulation and output.
//
// A is stored [M rows][K] (K contiguous) or, AT, [K rows][M]; B is stored
// [N rows][K] or, BT, [K rows][N].  Groups split either M (the routed rows of
// an expert; B is the expert's matrix) or, GK, K (an expert's rows are the
// reduction; C is the expert's matrix).  A 128 x 128 tile per 256-thread
// workgroup, four waves of 64 x 64 (MFMA 16x16x32 bf16), 64-wide k stages
// staged through registers into two LDS buffers laid out as the forward
// kernels lay them out ([row][64 k], 16-byte chunk c of row r at c ^ (r % 8)).
// An operand stored [K][X] is loaded as 8 k-rows x 4 columns per thread and
// transposed in registers before its LDS write.  Each output element is one
// MFMA chain over its k range in ascending order: no split-K, no atomics.
// ===========================================================================
constexpr int kBT = 128;                 // tile rows and columns
constexpr int kBK = 64;                  // k per stage
constexpr int kRowB = 128;               // LDS bytes per tile row (64 bf16)
constexpr int kOpB = kBT * kRowB;        // one operand's stage: 16 KiB
constexpr int kStageB = 2 * kOpB;        // 32 KiB

struct BwdOperand {
    const uint16_t* base;    // bf16 elements
    int64_t ld;              // elements between stored rows
    int64_t gstride;         // elements between the groups' matrices (0: one matrix)
    const int32_t* gather;   // index map of the stored rows (m rows of A; k rows of BT), or null
};

struct BwdGemm {
    BwdOperand a, b;
    float* c;
    int64_t ldc;
    int64_t c_gstride;          // GK: elements between the groups' outputs
    const int32_t* offsets;     // row ranges of the G groups [G + 1], or null: one group [0, rows)
    const int32_t* tile_start;  // !GK: m-tile prefix over the groups [G + 1] (null with one group)
    int G;
    int rows;                   // the one-group row count
    int M, N, K;                // !GK: N, K fixed (M from the groups); GK: M, N fixed
    int kb_valid;               // !GK, BT: B rows k >= kb_valid read as zero
    int m_valid;                // GK: output rows m >= m_valid are not stored (A may be wider)
};

// m-tile prefix over groups of 128-row tiles (one workgroup of 1024 threads)
__global__ __launch_bounds__(1024) void bwd_tile_prefix_kernel(const int32_t* __restrict__ offsets, int G,
                                                               int32_t* __restrict__ ts) {
    __shared__ int part[1024];
    const int tid = threadIdx.x;
    int v = 0;
    if (tid < G) v = (offsets[tid + 1] - offsets[tid] + kBT - 1) / kBT;
    part[tid] = v;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {
        const int u = tid >= d ? part[tid - d] : 0;
        __syncthreads();
        part[tid] += u;
        __syncthreads();
    }
    if (tid < G) ts[tid + 1] = part[tid];
    if (tid == 0) ts[0] = 0;
}

// 4 bf16 of 8 k-rows (v[r] = columns c..c+3 of row r) -> 8 k of each column
__device__ __forceinline__ void transpose_8x4(const u32x2 (&v)[8], u32x4 (&t)[4]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t lo = (c < 2) ? v[2 * q].x : v[2 * q].y;
            const uint32_t hi = (c < 2) ? v[2 * q + 1].x : v[2 * q + 1].y;
            w[q] = (c & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
        }
        t[c] = u32x4{w[0], w[1], w[2], w[3]};
    }
}

template <bool AT, bool BT, bool GK>
__global__ __launch_bounds__(256) void bwd_gemm_kernel(BwdGemm p) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem_raw[2 * kStageB];
    lds_u8* smem = (lds_u8*)(smem_raw);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv >> 1;
    const int wn = wv & 1;

    // ---- the tile -------------------------------------------------------------
    int g = 0;
    int64_t m0 = 0;
    int mrows = 0;
    int kbeg = 0, kend = p.K;
    const int n0 = blockIdx.x * kBT;
    const int ncols = min(kBT, p.N - n0);
    if (!GK) {
        const int L = blockIdx.y;
        if (p.offsets == nullptr) {
            m0 = static_cast<int64_t>(L) * kBT;
            if (m0 >= p.rows) return;
            mrows = min(kBT, p.rows - static_cast<int>(m0));
        } else {
            if (L >= p.tile_start[p.G]) return;
            int lo = 0, hi = p.G - 1;  // last group whose first tile is <= L
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (p.tile_start[mid] <= L) lo = mid; else hi = mid - 1;
            }
            g = lo;
            m0 = p.offsets[g] + static_cast<int64_t>(L - p.tile_start[g]) * kBT;
            mrows = min(static_cast<int64_t>(kBT), static_cast<int64_t>(p.offsets[g + 1]) - m0);
        }
    } else {
        g = blockIdx.z;
        m0 = static_cast<int64_t>(blockIdx.y) * kBT;
        mrows = min(kBT, p.m_valid - static_cast<int>(m0));
        kbeg = p.offsets ? p.offsets[g] : 0;
        kend = p.offsets ? p.offsets[g + 1] : p.rows;
    }
    const int ns = (kend - kbeg + kBK - 1) / kBK;

    const uint16_t* abase = p.a.base;
    const uint16_t* bbase = p.b.base + (GK ? 0 : static_cast<int64_t>(g) * p.b.gstride);
    const int kb_lim = GK ? kend : (BT ? p.kb_valid : kend);

    // ---- staging: each thread's share of one stage ------------------------------
    // K-major operand: rows (tid / 8) + 32 i, 16-byte chunk tid % 8.
    // Stored [K][X]: k rows 8 (tid / 32) + r, columns 4 (tid % 32) .. + 3.
    const int km_chunk = tid & 7;
    const int km_row = tid >> 3;
    const int tr_col = 4 * (tid & 31);
    const int tr_ko = tid >> 5;
    u32x4 ra[4], rb[4];
    u32x2 ta[8], tb[8];

    auto load_stage = [&](int s) {
        const int k0 = kbeg + s * kBK;
        if (!AT) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = km_row + 32 * i;
                const int rr = r < mrows ? r : mrows - 1;  // rows past the tile repeat its last; never stored
                int64_t row = m0 + rr;
                if (p.a.gather) row = p.a.gather[row];
                ra[i] = *reinterpret_cast<const u32x4*>(abase + row * p.a.ld + k0 + 8 * km_chunk);
            }
        } else {
            const int col = static_cast<int>(m0) + tr_col < p.M ? static_cast<int>(m0) + tr_col : p.M - 4;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const int k = k0 + 8 * tr_ko + r;
                ta[r] = u32x2{0u, 0u};
                if (k < kend) ta[r] = *reinterpret_cast<const u32x2*>(abase + static_cast<int64_t>(k) * p.a.ld + col);
            }
        }
        if (!BT) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = km_row + 32 * i;
                const int rr = r < ncols ? r : ncols - 1;
                rb[i] = *reinterpret_cast<const u32x4*>(bbase + static_cast<int64_t>(n0 + rr) * p.b.ld + k0 +
                                                        8 * km_chunk);
            }
        } else {
            const int col = n0 + tr_col < p.N ? n0 + tr_col : p.N - 4;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const int k = k0 + 8 * tr_ko + r;
                tb[r] = u32x2{0u, 0u};
                if (k < kb_lim && k < kend) {
                    int64_t row = k;
                    if (GK && p.b.gather) row = p.b.gather[k];
                    tb[r] = *reinterpret_cast<const u32x2*>(bbase + row * p.b.ld + col);
                }
            }
        }
    };
    auto store_stage = [&](int buf) {
        lds_u8* sa = smem + buf * kStageB;
        lds_u8* sb = sa + kOpB;
        if (!AT) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = km_row + 32 * i;
                *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(sa + r * kRowB +
                                                                             ((km_chunk ^ (r & 7)) << 4)) = ra[i];
            }
        } else {
            u32x4 t[4];
            transpose_8x4(ta, t);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int r = tr_col + c;
                *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(sa + r * kRowB +
                                                                             ((tr_ko ^ (r & 7)) << 4)) = t[c];
            }
        }
        if (!BT) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = km_row + 32 * i;
                *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(sb + r * kRowB +
                                                                             ((km_chunk ^ (r & 7)) << 4)) = rb[i];
            }
        } else {
            u32x4 t[4];
            transpose_8x4(tb, t);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int r = tr_col + c;
                *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(sb + r * kRowB +
                                                                             ((tr_ko ^ (r & 7)) << 4)) = t[c];
            }
        }
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // fragment of half j of a stage: logical chunk 4j + lane/16 of row lane%16
    // (+16 per block), at chunk ^ (lane % 8)
    const int xo0 = ((lane >> 4) ^ (lane & 7)) << 4;
    const int xo1 = ((4 + (lane >> 4)) ^ (lane & 7)) << 4;
    const int a_frag = (wm * 64 + (lane & 15)) * kRowB;
    const int b_frag = kOpB + (wn * 64 + (lane & 15)) * kRowB;

    if (ns > 0) {
        load_stage(0);
        store_stage(0);
        __syncthreads();
        for (int s = 0; s < ns; ++s) {
            if (s + 1 < ns) load_stage(s + 1);  // global loads in flight over this stage's MFMAs
            const lds_u8* st = smem + (s & 1) * kStageB;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int xo = j == 0 ? xo0 : xo1;
                u32x4 af[4], bf[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    af[i] = *reinterpret_cast<lds_u32x4*>(st + a_frag + i * 16 * kRowB + xo);
                    bf[i] = *reinterpret_cast<lds_u32x4*>(st + b_frag + i * 16 * kRowB + xo);
                }
#pragma unroll
                for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                    for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = mfma_bf16(bf[nb], af[mb], acc[mb][nb]);
            }
            if (s + 1 < ns) store_stage((s + 1) & 1);  // that buffer was last read in stage s-1
            __syncthreads();
        }
    }

    // ---- output: lane holds row (lane % 16) x 4 consecutive columns per block ----
    float* cb = p.c + (GK ? static_cast<int64_t>(g) * p.c_gstride : 0);
    const int c4 = 4 * (lane >> 4);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
        const int m = wm * 64 + mb * 16 + (lane & 15);
        if (m >= mrows) continue;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            const int n = wn * 64 + nb * 16 + c4;
            if (n < ncols)
                *reinterpret_cast<f32x4*>(cb + (m0 + m) * p.ldc + n0 + n) = acc[mb][nb];
        }
    }
}

// ===========================================================================
// Per-token and elementwise steps
// ===========================================================================
constexpr int kBwdThreads = 256;
constexpr int kBwdMaxK = 16;

// dY[p] = bf16(fl32(w * G[t])) for each pick; dw[t, j] = <G[t], y[p]> summed in
// float64 (every product of two bf16 values is exact there) in a fixed order:
// each thread its 16-byte chunks in order, then a fixed tree over the
// workgroup.  gs (optional): G with masked rows zeroed, the shared expert's dY.
__global__ __launch_bounds__(kBwdThreads) void combine_bwd_kernel(
    const uint16_t* __restrict__ G, const uint16_t* __restrict__ y, const int32_t* __restrict__ inv_pos,
    const float* __restrict__ w, const uint8_t* __restrict__ mask, int64_t T, int D, int K,
    uint16_t* __restrict__ dY, double* __restrict__ dw, uint16_t* __restrict__ gs) {
    __shared__ double red[kBwdThreads];
    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x;
    const bool kept = mask == nullptr || mask[t] != 0;
    for (int j = 0; j < K; ++j) {
        const int64_t pos = kept ? inv_pos[t * K + j] : -1;
        const float wt = w[t * K + j];
        double part = 0.0;
        if (pos >= 0) {
            for (int d0 = tid * 8; d0 < D; d0 += kBwdThreads * 8) {
                const u32x4 gv = *reinterpret_cast<const u32x4*>(G + t * D + d0);
                const u32x4 yv = *reinterpret_cast<const u32x4*>(y + pos * D + d0);
                const uint32_t ga[4] = {gv.x, gv.y, gv.z, gv.w};
                const uint32_t ya[4] = {yv.x, yv.y, yv.z, yv.w};
                uint32_t o[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float g0 = __uint_as_float(ga[i] << 16), g1 = __uint_as_float(ga[i] & 0xFFFF0000u);
                    const float y0 = __uint_as_float(ya[i] << 16), y1 = __uint_as_float(ya[i] & 0xFFFF0000u);
                    part += static_cast<double>(g0) * static_cast<double>(y0);
                    part += static_cast<double>(g1) * static_cast<double>(y1);
                    const float p0 = wt * g0, p1 = wt * g1;
                    o[i] = static_cast<uint32_t>(f32_to_bf16(p0)) | (static_cast<uint32_t>(f32_to_bf16(p1)) << 16);
                }
                *reinterpret_cast<u32x4*>(dY + pos * D + d0) = u32x4{o[0], o[1], o[2], o[3]};
            }
        }
        red[tid] = part;
        __syncthreads();
        for (int h = kBwdThreads / 2; h > 0; h >>= 1) {
            if (tid < h) red[tid] += red[tid + h];
            __syncthreads();
        }
        if (tid == 0) dw[t * K + j] = pos >= 0 ? red[0] : 0.0;
        __syncthreads();
    }
    if (gs != nullptr) {
        for (int d0 = tid * 8; d0 < D; d0 += kBwdThreads * 8) {
            const u32x4 gv = kept ? *reinterpret_cast<const u32x4*>(G + t * D + d0) : u32x4{0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4*>(gs + t * D + d0) = gv;
        }
    }
}

// SwiGLU backward over rows [0, *rows_dev or rows): H [rows, 2I] float32 (gate
// columns, then up), dA [rows, I] float32 -> dH [rows, 2I] bf16 and the
// forward's activation A [rows, I] bf16.  Eight columns per thread.
__global__ __launch_bounds__(kBwdThreads) void swiglu_bwd_kernel(
    const float* __restrict__ H, const float* __restrict__ dA, const int32_t* __restrict__ rows_dev, int64_t rows,
    int I, uint16_t* __restrict__ dH, uint16_t* __restrict__ A) {
    const int64_t r = blockIdx.x;
    const int64_t nrows = rows_dev ? *rows_dev : rows;
    if (r >= nrows) return;
    const int i0 = (blockIdx.y * kBwdThreads + threadIdx.x) * 8;
    if (i0 >= I) return;
    const float* hg = H + r * 2 * I + i0;
    const float* hu = hg + I;
    const float* da = dA + r * I + i0;
    uint32_t og[4], ou[4], oa[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        float vg[2], vu[2], va[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float g = hg[2 * q + h], u = hu[2 * q + h], d = da[2 * q + h];
            const float sg = 1.0f / (1.0f + expf(-g));
            const float silu = g * sg;
            const float dsilu = sg * (1.0f + g * (1.0f - sg));
            vg[h] = d * u * dsilu;
            vu[h] = d * silu;
            va[h] = silu_mul_fast(g, u);
        }
        og[q] = static_cast<uint32_t>(f32_to_bf16(vg[0])) | (static_cast<uint32_t>(f32_to_bf16(vg[1])) << 16);
        ou[q] = static_cast<uint32_t>(f32_to_bf16(vu[0])) | (static_cast<uint32_t>(f32_to_bf16(vu[1])) << 16);
        oa[q] = static_cast<uint32_t>(f32_to_bf16(va[0])) | (static_cast<uint32_t>(f32_to_bf16(va[1])) << 16);
    }
    *reinterpret_cast<u32x4*>(dH + r * 2 * I + i0) = u32x4{og[0], og[1], og[2], og[3]};
    *reinterpret_cast<u32x4*>(dH + r * 2 * I + I + i0) = u32x4{ou[0], ou[1], ou[2], ou[3]};
    *reinterpret_cast<u32x4*>(A + r * I + i0) = u32x4{oa[0], oa[1], oa[2], oa[3]};
}

// float64 score of one logit (softmax handled by the caller)
__device__ __forceinline__ double bwd_elem_score(double l, int score) {
    if (score == 2) return sqrt(fmax(l, 0.0) + log1p(exp(-fabs(l))));
    return 1.0 / (1.0 + exp(-l));
}

// Router backward, one wave per token: dl[t, e] = d(score_e)/d(l) applied to
// ds, where ds comes from dw through the weights (renormalised over the K
// picks or not, times route_scale).  Float64 throughout; dl is stored as a
// bf16 operand [T, ldl] with zeros past E and for masked tokens.
__global__ __launch_bounds__(256) void router_bwd_kernel(
    const double* __restrict__ logits, const int32_t* __restrict__ ids, const double* __restrict__ dw,
    const uint8_t* __restrict__ mask, int64_t T, int E, int K, int score, int renorm, double route_scale,
    uint16_t* __restrict__ dl, int ldl) {
    const int lane = threadIdx.x & 63;
    const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (t >= T) return;  // uniform per wave
    const bool kept = (mask == nullptr || mask[t] != 0) && ids[t * K] >= 0;
    constexpr int kEPL = 16;  // E <= 1024
    double s[kEPL], lg[kEPL];
    const int epl = (E + 63) / 64;
    double m = -1.7976931348623157e308, z = 0.0;
    for (int i = 0; i < kEPL; ++i) {
        const int e = lane + 64 * i;
        lg[i] = (i < epl && e < E && kept) ? logits[t * E + e] : 0.0;
        if (i < epl && e < E) m = fmax(m, lg[i]);
    }
    if (score == 0) {
        for (int off = 32; off > 0; off >>= 1) m = fmax(m, __shfl_xor(m, off));
        double part = 0.0;
        for (int i = 0; i < kEPL; ++i) {
            const int e = lane + 64 * i;
            s[i] = (i < epl && e < E) ? exp(lg[i] - m) : 0.0;
            part += s[i];
        }
        z = part;
        for (int off = 32; off > 0; off >>= 1) z += __shfl_xor(z, off);
        for (int i = 0; i < kEPL; ++i) s[i] = s[i] / z;
    } else {
        for (int i = 0; i < kEPL; ++i) {
            const int e = lane + 64 * i;
            s[i] = (i < epl && e < E) ? bwd_elem_score(lg[i], score) : 0.0;
        }
    }
    // the picks' scores and weight gradients (uniform)
    double sp[kBwdMaxK], dwp[kBwdMaxK];
    int ep[kBwdMaxK];
    double Z = 0.0, sdw = 0.0;
    for (int j = 0; j < K; ++j) {
        ep[j] = kept ? ids[t * K + j] : 0;
        const int owner = ep[j] & 63, slot = ep[j] >> 6;
        double v = 0.0;
        for (int i = 0; i < kEPL; ++i)
            if (i == slot) v = s[i];
        sp[j] = __shfl(v, owner);
        dwp[j] = kept ? dw[t * K + j] : 0.0;
        Z += sp[j];
        sdw += dwp[j] * sp[j];
    }
    // ds of each pick, and sum_j ds_j s_j for the softmax
    double dsp[kBwdMaxK];
    double dss = 0.0;
    for (int j = 0; j < K; ++j) {
        dsp[j] = renorm ? route_scale / Z * (dwp[j] - sdw / Z) : route_scale * dwp[j];
        dss += dsp[j] * sp[j];
    }
    for (int i = 0; i < kEPL; ++i) {
        if (i >= epl) break;  // ldl = 64 * epl
        const int e = lane + 64 * i;
        double ds = 0.0;
        for (int j = 0; j < K; ++j)
            if (ep[j] == e) ds = dsp[j];
        double d = 0.0;
        if (kept && e < E) {
            if (score == 0) d = s[i] * (ds - dss);
            else if (score == 1) d = ds * s[i] * (1.0 - s[i]);
            else d = s[i] > 0.0 ? ds * (1.0 / (1.0 + exp(-lg[i]))) / (2.0 * s[i]) : 0.0;
        }
        if (e < ldl) dl[t * ldl + e] = f32_to_bf16(static_cast<float>(d));
    }
}

// dx[t] = fl32 fold over the picks in ascending expert id of dXp[p_j], then
// + dXs[t] (shared) + dxr[t] (router); zero for masked tokens.
__global__ __launch_bounds__(kBwdThreads) void dx_assemble_kernel(
    const float* __restrict__ dXp, const int32_t* __restrict__ inv_pos, const float* __restrict__ dXs,
    const float* __restrict__ dxr, const uint8_t* __restrict__ mask, int64_t T, int D, int K,
    float* __restrict__ dx) {
    const int64_t t = blockIdx.x;
    const bool kept = mask == nullptr || mask[t] != 0;
    for (int d0 = threadIdx.x * 4; d0 < D; d0 += kBwdThreads * 4) {
        f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
        if (kept) {
            for (int j = 0; j < K; ++j) {
                const int64_t pos = inv_pos[t * K + j];
                if (pos >= 0) a = a + *reinterpret_cast<const f32x4*>(dXp + pos * D + d0);
            }
            if (dXs) a = a + *reinterpret_cast<const f32x4*>(dXs + t * D + d0);
            a = a + *reinterpret_cast<const f32x4*>(dxr + t * D + d0);
        }
        *reinterpret_cast<f32x4*>(dx + t * D + d0) = a;
    }
}

// ===========================================================================
// launcher
// ===========================================================================
template <bool AT, bool BT, bool GK>
static hipError_t gemm(const BwdGemm& p, int m_tiles, int groups_z, hipStream_t stream) {
    dim3 grid(static_cast<unsigned>((p.N + kBT - 1) / kBT), static_cast<unsigned>(m_tiles),
              static_cast<unsigned>(groups_z));
    bwd_gemm_kernel<AT, BT, GK><<<grid, 256, 0, stream>>>(p);
    return hipGetLastError();
}

static BwdOperand op(const void* base, int64_t ld, int64_t gstride = 0, const int32_t* gather = nullptr) {
    return BwdOperand{static_cast<const uint16_t*>(base), ld, gstride, gather};
}

size_t backward_ws_bytes(int64_t T, int D, int E, int K, int I, int Is) {
    const int64_t P = T * K;
    const int64_t rows2 = P * 2 * I > T * 2 * static_cast<int64_t>(Is) ? P * 2 * I : T * 2 * static_cast<int64_t>(Is);
    const int64_t rows1 = P * I > T * static_cast<int64_t>(Is) ? P * I : T * static_cast<int64_t>(Is);
    const int64_t Epad = (E + 63) / 64 * 64;
    size_t b = 0;
    auto take = [&](size_t n) { b += (n + 255) & ~static_cast<size_t>(255); };
    take(sizeof(double) * T * E);        // logits
    take(sizeof(double) * P);            // dw
    take(2 * static_cast<size_t>(P) * D);  // dY
    take(2 * static_cast<size_t>(T) * D);  // dYs
    take(4 * static_cast<size_t>(rows2));  // H
    take(4 * static_cast<size_t>(rows1));  // dA
    take(2 * static_cast<size_t>(rows2));  // dH
    take(2 * static_cast<size_t>(rows1));  // A
    take(4 * static_cast<size_t>(P) * D);  // dXp
    take(4 * static_cast<size_t>(T) * D);  // dXs
    take(4 * static_cast<size_t>(T) * D);  // dxr
    take(2 * static_cast<size_t>(T) * Epad);  // dl
    take(sizeof(int32_t) * (E + 1));     // tile prefix
    return b;
}

hipError_t launch_backward(const BwdArgs& a, hipStream_t stream) {
    const int64_t T = a.T;
    const int D = a.D, E = a.E, K = a.K, I = a.I, Is = a.Is;
    const int64_t P = T * K;
    const int64_t rows2 = P * 2 * I > T * 2 * static_cast<int64_t>(Is) ? P * 2 * I : T * 2 * static_cast<int64_t>(Is);
    const int64_t rows1 = P * I > T * static_cast<int64_t>(Is) ? P * I : T * static_cast<int64_t>(Is);
    const int Epad = (E + 63) / 64 * 64;
    uint8_t* w = static_cast<uint8_t*>(a.ws);
    size_t off = 0;
    auto take = [&](size_t n) {
        void* q = w + off;
        off += (n + 255) & ~static_cast<size_t>(255);
        return q;
    };
    double* logits = static_cast<double*>(take(sizeof(double) * T * E));
    double* dw = static_cast<double*>(take(sizeof(double) * P));
    uint16_t* dY = static_cast<uint16_t*>(take(2 * static_cast<size_t>(P) * D));
    uint16_t* dYs = static_cast<uint16_t*>(take(2 * static_cast<size_t>(T) * D));
    float* H = static_cast<float*>(take(4 * static_cast<size_t>(rows2)));
    float* dA = static_cast<float*>(take(4 * static_cast<size_t>(rows1)));
    uint16_t* dH = static_cast<uint16_t*>(take(2 * static_cast<size_t>(rows2)));
    uint16_t* Aact = static_cast<uint16_t*>(take(2 * static_cast<size_t>(rows1)));
    float* dXp = static_cast<float*>(take(4 * static_cast<size_t>(P) * D));
    float* dXs = static_cast<float*>(take(4 * static_cast<size_t>(T) * D));
    float* dxr = static_cast<float*>(take(4 * static_cast<size_t>(T) * D));
    uint16_t* dl = static_cast<uint16_t*>(take(2 * static_cast<size_t>(T) * Epad));
    int32_t* ts = static_cast<int32_t*>(take(sizeof(int32_t) * (E + 1)));

    hipError_t err;
    if ((err = launch_router_logits(a.x, a.router, T, D, E, 0, logits, stream)) != hipSuccess) return err;
    combine_bwd_kernel<<<static_cast<unsigned>(T), kBwdThreads, 0, stream>>>(
        static_cast<const uint16_t*>(a.dout), static_cast<const uint16_t*>(a.y), a.inv_pos, a.topk_w, a.mask, T, D,
        K, dY, dw, Is > 0 ? dYs : nullptr);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    bwd_tile_prefix_kernel<<<1, 1024, 0, stream>>>(a.offsets, E, ts);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    const int mt_routed = static_cast<int>((P + kBT - 1) / kBT) + E;

    // routed experts
    BwdGemm g{};
    g.offsets = a.offsets;
    g.tile_start = ts;
    g.G = E;
    // H = X_e W1_e^T (rows gathered)
    g.a = op(a.x, D, 0, a.perm_token);
    g.b = op(a.gate_up, D, static_cast<int64_t>(2) * I * D);
    g.c = H; g.ldc = 2 * I; g.N = 2 * I; g.K = D; g.kb_valid = D;
    if ((err = gemm<false, false, false>(g, mt_routed, 1, stream)) != hipSuccess) return err;
    // dA = dY W2_e
    g.a = op(dY, D);
    g.b = op(a.down, I, static_cast<int64_t>(D) * I);
    g.c = dA; g.ldc = I; g.N = I; g.K = D; g.kb_valid = D;
    if ((err = gemm<false, true, false>(g, mt_routed, 1, stream)) != hipSuccess) return err;
    {
        dim3 grid(static_cast<unsigned>(P), static_cast<unsigned>((I / 8 + kBwdThreads - 1) / kBwdThreads));
        swiglu_bwd_kernel<<<grid, kBwdThreads, 0, stream>>>(H, dA, a.offsets + E, P, I, dH, Aact);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    // dXp = dH W1_e
    g.a = op(dH, 2 * I);
    g.b = op(a.gate_up, D, static_cast<int64_t>(2) * I * D);
    g.c = dXp; g.ldc = D; g.N = D; g.K = 2 * I; g.kb_valid = 2 * I;
    if ((err = gemm<false, true, false>(g, mt_routed, 1, stream)) != hipSuccess) return err;
    // dW2_e = dY_e^T A_e
    BwdGemm k{};
    k.offsets = a.offsets;
    k.G = E;
    k.a = op(dY, D);
    k.b = op(Aact, I);
    k.c = a.d_down; k.ldc = I; k.c_gstride = static_cast<int64_t>(D) * I; k.M = D; k.N = I; k.m_valid = D;
    if ((err = gemm<true, true, true>(k, (D + kBT - 1) / kBT, E, stream)) != hipSuccess) return err;
    // dW1_e = dH_e^T X_e (rows gathered)
    k.a = op(dH, 2 * I);
    k.b = op(a.x, D, 0, a.perm_token);
    k.c = a.d_gate_up; k.ldc = D; k.c_gstride = static_cast<int64_t>(2) * I * D; k.M = 2 * I; k.N = D;
    k.m_valid = 2 * I;
    if ((err = gemm<true, true, true>(k, (2 * I + kBT - 1) / kBT, E, stream)) != hipSuccess) return err;

    // shared expert: one group of T rows, dY = G on kept tokens
    if (Is > 0) {
        const int mt = static_cast<int>((T + kBT - 1) / kBT);
        BwdGemm s{};
        s.G = 1;
        s.rows = static_cast<int>(T);
        s.a = op(a.x, D);
        s.b = op(a.gate_up_shared, D);
        s.c = H; s.ldc = 2 * Is; s.N = 2 * Is; s.K = D; s.kb_valid = D;
        if ((err = gemm<false, false, false>(s, mt, 1, stream)) != hipSuccess) return err;
        s.a = op(dYs, D);
        s.b = op(a.down_shared, Is);
        s.c = dA; s.ldc = Is; s.N = Is; s.K = D; s.kb_valid = D;
        if ((err = gemm<false, true, false>(s, mt, 1, stream)) != hipSuccess) return err;
        dim3 grid(static_cast<unsigned>(T), static_cast<unsigned>((Is / 8 + kBwdThreads - 1) / kBwdThreads));
        swiglu_bwd_kernel<<<grid, kBwdThreads, 0, stream>>>(H, dA, nullptr, T, Is, dH, Aact);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        s.a = op(dH, 2 * Is);
        s.b = op(a.gate_up_shared, D);
        s.c = dXs; s.ldc = D; s.N = D; s.K = 2 * Is; s.kb_valid = 2 * Is;
        if ((err = gemm<false, true, false>(s, mt, 1, stream)) != hipSuccess) return err;
        BwdGemm sk{};
        sk.G = 1;
        sk.rows = static_cast<int>(T);
        sk.a = op(dYs, D);
        sk.b = op(Aact, Is);
        sk.c = a.d_down_shared; sk.ldc = Is; sk.M = D; sk.N = Is; sk.m_valid = D;
        if ((err = gemm<true, true, true>(sk, (D + kBT - 1) / kBT, 1, stream)) != hipSuccess) return err;
        sk.a = op(dH, 2 * Is);
        sk.b = op(a.x, D);
        sk.c = a.d_gate_up_shared; sk.ldc = D; sk.M = 2 * Is; sk.N = D; sk.m_valid = 2 * Is;
        if ((err = gemm<true, true, true>(sk, (2 * Is + kBT - 1) / kBT, 1, stream)) != hipSuccess) return err;
    }

    // router
    router_bwd_kernel<<<static_cast<unsigned>((T + 3) / 4), 256, 0, stream>>>(
        logits, a.topk_ids, dw, a.mask, T, E, K, a.score, a.renorm, static_cast<double>(a.route_scale), dl, Epad);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    {
        const int mt = static_cast<int>((T + kBT - 1) / kBT);
        BwdGemm r{};
        r.G = 1;
        r.rows = static_cast<int>(T);
        r.a = op(dl, Epad);
        r.b = op(a.router, D);
        r.c = dxr; r.ldc = D; r.N = D; r.K = Epad; r.kb_valid = E;
        if ((err = gemm<false, true, false>(r, mt, 1, stream)) != hipSuccess) return err;
        BwdGemm rk{};
        rk.G = 1;
        rk.rows = static_cast<int>(T);
        rk.a = op(dl, Epad);
        rk.b = op(a.x, D);
        rk.c = a.d_router; rk.ldc = D; rk.M = Epad; rk.N = D; rk.m_valid = E;
        if ((err = gemm<true, true, true>(rk, (E + kBT - 1) / kBT, 1, stream)) != hipSuccess) return err;
    }
    dx_assemble_kernel<<<static_cast<unsigned>(T), kBwdThreads, 0, stream>>>(dXp, a.inv_pos, Is > 0 ? dXs : nullptr,
                                                                             dxr, a.mask, T, D, K, a.dx);
    return hipGetLastError();
}

}  // namespace moe
