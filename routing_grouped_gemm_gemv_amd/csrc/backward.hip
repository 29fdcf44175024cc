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
//   gather        Xp = x[perm] (the routed rows in expert order)
//   gemm          dA = dY W2_e (float32)
//   gemm          H = Xp W1_e^T recomputed in float32, never stored: its
//                 epilogue forms A = bf16(silu(g) u) as the forward formed it
//                 and dH = bf16([dA u silu'(g), dA silu(g)])
//   gemm          dW2_e = dY_e^T A_e, K-grouped (float32)
//   gemm          dXp = dH W1_e (float32)
//   gemm          dW1_e = dH_e^T Xp_e, K-grouped
//   (the same for the shared expert, with dY = G on every kept token)
//   router_bwd    dl[t, e] from dw through the weights and the score (bf16)
//   gemm          dx_r = dl W_r;  gemm  dW_r = dl^T x (K-grouped, one group)
//   dx_assemble   dx[t] = sum_j dXp[p_j] (ascending expert id) + dX_shared[t] + dx_r[t]
#include "common.hpp"
#include "kernels.hpp"

#include <math.h>

namespace moe {

// ===========================================================================
// Grouped GEMM for the backward: C[m][n] = sum_k A(m, k) B(k, n), bf16
// operands, float32 accumulation and output.
//
// A is stored [M rows][K] (K contiguous) or, AT, [K rows][M]; B is stored
// [N rows][K] or, BT, [K rows][N].  Groups split either M (the routed rows of
// an expert; B is the expert's matrix) or, GK, K (an expert's rows are the
// reduction; C is the expert's matrix).  256 x 256 tiles, four waves of
// 128 x 128 (MFMA 16x16x32 bf16), 64-wide k stages moved global -> LDS by
// DMA into two buffers, the next stage in flight over the current one's
// MFMAs.  Each output element is one MFMA chain over its k range in
// ascending order: no split-K, no atomics.
//
// LDS layouts of one operand's stage (32 KiB):
//  * K-major: 256 rows of 64 k (128 B); 16-byte chunk c of row r at
//    c ^ (r % 8).  A fragment (16 rows x 8 k per lane) is one 16-byte read.
//  * [K][X]: 64 k-rows of 256 x-values (512 B); the 32-byte block of 16
//    x-values p of k-row k at p ^ h(k), h(k) = (k % 4) + 4 ((k / 8) % 2), so
//    that the 16 k-rows one transposed read touches fall on distinct banks.
//    A fragment is two ds_read_b64_tr_b16: in each 16-lane block, lane i
//    receives element i % 4 of the 8 bytes that lane 4j + i / 4 addresses, as
//    its element j; a lane that addresses x-values 4 (s % 4) .. + 3 of k-row
//    k0 + s / 4 (s its index in the block) hands lane i the four k of x-value
//    i, which is the MFMA operand layout.
// ===========================================================================
constexpr int kT = 256;                  // tile rows and columns
constexpr int kSK = 64;                  // k per stage
constexpr int kOpB = 32768;              // one operand's stage
constexpr int kStageB = 2 * kOpB;
constexpr int kZeroTail = 1024;          // zero bytes after each K-grouped A operand

typedef short bwd_v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bwd_v4s lds_v4s;

struct BwdOperand {
    const uint16_t* base;    // bf16 elements
    int64_t ld;              // elements between stored rows
    int64_t gstride;         // elements between the groups' matrices (0: one matrix)
};

struct BwdGemm {
    BwdOperand a, b;
    float* c;
    int64_t ldc;
    int64_t c_gstride;          // GK: elements between the groups' outputs
    const int32_t* offsets;     // row ranges of the G groups [G + 1], or null: one group [0, rows)
    const int32_t* tile_start;  // !GK: m-tile prefix over the groups [G + 1] (null with one group)
    const uint16_t* a_zero;     // GK: kZeroTail zero bytes after A's buffer (A's k-rows past a group read these)
    int G;
    int rows;                   // the one-group row count
    int M, N, K;                // !GK: N, K fixed (M from the groups); GK: M, N fixed
    int kb_valid;               // !GK: B k-rows >= kb_valid are clamped (A is zero there)
    int m_valid;                // GK: output rows m >= m_valid are not stored
    // SW (gate/up recompute with the SwiGLU backward in the epilogue): B is
    // the expert's W1 [2I][D]; a tile takes gate rows c and up rows I + c of
    // 128 columns c; dA [rows][I] float32 in, dH [rows][2I] and A [rows][I] bf16 out
    int I;
    const float* da;
    uint16_t* dh;
    uint16_t* act;
};

// two floats -> two bf16 (round to nearest even) in one word, low first
__device__ __forceinline__ uint32_t bwd_pack_bf16(float lo, float hi) {
    return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// SwiGLU backward of one element: the forward's activation a = bf16(silu(g) u)
// (the same expression the forward's epilogue evaluates) and the gate and up
// gradients dg = dA u silu'(g), du = dA silu(g), float32.
__device__ __forceinline__ void swiglu_grad(float g, float u, float d, float& dg, float& du, float& a) {
    const float sg = 1.0f / (1.0f + expf(-g));
    const float silu = g * sg;
    const float dsilu = sg * (1.0f + g * (1.0f - sg));
    dg = d * u * dsilu;
    du = d * silu;
    a = silu_mul_fast(g, u);
}

// m-tile prefix over groups of kT-row tiles (one workgroup of 1024 threads)
__global__ __launch_bounds__(1024) void bwd_tile_prefix_kernel(const int32_t* __restrict__ offsets, int G,
                                                               int32_t* __restrict__ ts) {
    __shared__ int part[1024];
    const int tid = threadIdx.x;
    int v = 0;
    if (tid < G) v = (offsets[tid + 1] - offsets[tid] + kT - 1) / kT;
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

template <bool AT, bool BT, bool GK, bool SW = false>
__global__ __launch_bounds__(256) void bwd_gemm_kernel(BwdGemm p) {
    static_assert(!SW || (!AT && !BT && !GK), "the SwiGLU epilogue is for the M-grouped K-major gate/up GEMM");
    __shared__ __attribute__((aligned(1024))) uint8_t smem_raw[2 * kStageB + 8192];  // stages; the output staging needs 128 x 1040 B
    lds_u8* smem = (lds_u8*)(smem_raw);
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(smem));
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv >> 1;
    const int wn = wv & 1;

    // ---- the tile (XCD-aware: consecutive tiles on one XCD) ---------------------
    const int ntn = SW ? (p.I + 127) / 128 : (p.N + kT - 1) / kT;
    const int64_t L = xcd_remap(blockIdx.x, gridDim.x);
    int g = 0, mt = 0, nt = 0;
    int64_t m0 = 0;     // !GK: first row of the tile
    int mrows = 0;      // !GK: valid rows of the tile
    int kbeg = 0, kend = p.K;
    if (!GK) {
        if (p.offsets == nullptr) {
            const int mtn = (p.rows + kT - 1) / kT;
            if (L >= static_cast<int64_t>(mtn) * ntn) return;
            nt = static_cast<int>(L / mtn);
            mt = static_cast<int>(L % mtn);
            m0 = static_cast<int64_t>(mt) * kT;
            mrows = min(kT, p.rows - static_cast<int>(m0));
        } else {
            if (L >= static_cast<int64_t>(p.tile_start[p.G]) * ntn) return;
            int lo = 0, hi = p.G - 1;  // last group whose first tile is <= L
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (static_cast<int64_t>(p.tile_start[mid]) * ntn <= L) lo = mid; else hi = mid - 1;
            }
            g = lo;
            const int mtn = p.tile_start[g + 1] - p.tile_start[g];
            const int loc = static_cast<int>(L - static_cast<int64_t>(p.tile_start[g]) * ntn);
            nt = loc / mtn;
            mt = loc % mtn;
            m0 = p.offsets[g] + static_cast<int64_t>(mt) * kT;
            mrows = min(static_cast<int64_t>(kT), static_cast<int64_t>(p.offsets[g + 1]) - m0);
        }
    } else {
        const int mtn = (p.M + kT - 1) / kT;
        const int per = mtn * ntn;
        if (L >= static_cast<int64_t>(per) * p.G) return;
        g = static_cast<int>(L / per);
        const int loc = static_cast<int>(L % per);
        mt = loc / ntn;
        nt = loc % ntn;
        kbeg = p.offsets ? p.offsets[g] : 0;
        kend = p.offsets ? p.offsets[g + 1] : p.rows;
    }
    const int n0 = nt * kT;
    const int ns = (kend - kbeg + kSK - 1) / kSK;

    // ---- operand bases (wave-uniform) and per-lane DMA offsets --------------------
    // K-major: instruction q of wave w fills rows 64 w + 8 q + lane / 8 at
    // physical chunk lane % 8 with logical chunk (lane % 8) ^ (lane / 8).
    // [K][X]: instruction q of wave w fills k-rows 8 q + 2 w + lane / 32 at
    // physical chunk lane % 32 (block (lane % 32) / 2).
    const uint8_t* abase;
    const uint8_t* bbase;
    if (!GK) {
        abase = reinterpret_cast<const uint8_t*>(p.a.base + m0 * p.a.ld);
        bbase = reinterpret_cast<const uint8_t*>(p.b.base + static_cast<int64_t>(g) * p.b.gstride);
    } else {
        abase = reinterpret_cast<const uint8_t*>(p.a.base + static_cast<int64_t>(kbeg) * p.a.ld);
        bbase = reinterpret_cast<const uint8_t*>(p.b.base + static_cast<int64_t>(kbeg) * p.b.ld);
    }
    const uint32_t lda2 = static_cast<uint32_t>(p.a.ld) * 2;
    const uint32_t ldb2 = static_cast<uint32_t>(p.b.ld) * 2;
    const int km_chunk = (lane & 7) ^ (lane >> 3);
    const int km_row = 64 * wv + (lane >> 3);          // + 8 q
    const int tx_row = 2 * wv + (lane >> 5);           // + 8 q
    const int tx_pc = lane & 31;
    // [K][X] x offset (bytes) of instruction parity qp, clamped to the operand's width
    auto tx_x = [&](int qp, int x0, int xlim) -> uint32_t {
        const int h = ((2 * wv + (lane >> 5)) & 3) | (qp << 2);
        const int c = 2 * ((tx_pc >> 1) ^ h) + (tx_pc & 1);
        int x = x0 + 8 * c;
        if (x > xlim - 8) x = xlim - 8;
        return static_cast<uint32_t>(x) * 2;
    };
    const int m_tile0 = GK ? mt * kT : 0;
    const uint32_t ax0 = AT ? tx_x(0, m_tile0, p.M) : 0u, ax1 = AT ? tx_x(1, m_tile0, p.M) : 0u;
    const uint32_t bx0 = BT ? tx_x(0, n0, p.N) : 0u, bx1 = BT ? tx_x(1, n0, p.N) : 0u;
    const uint32_t a_zero_off =
        GK ? static_cast<uint32_t>(reinterpret_cast<const uint8_t*>(p.a_zero) - abase) + 16 * tx_pc : 0u;
    const int klen = kend - kbeg;
    const int kb_lim = GK ? klen : p.kb_valid;
    // K-major rows: lane base and the clamp to the last valid row (rows past
    // the group repeat its last row and are never stored)
    const uint32_t a_km = static_cast<uint32_t>(km_row) * lda2 + km_chunk * 16;
    const uint32_t a_km_lim = static_cast<uint32_t>(mrows - 1) * lda2 + km_chunk * 16;
    // SW: tile row r of B is gate row c = 128 nt + r % 128 (waves 0, 1) or the
    // matching up row I + c (waves 2, 3); columns past I repeat I - 1 (never stored)
    const int b_row0 = SW ? (wv < 2 ? 0 : p.I) + nt * 128 + 64 * (wv & 1) + (lane >> 3) : n0 + km_row;
    const int b_rowlim = SW ? (wv < 2 ? p.I : 2 * p.I) - 1 : p.N - 1;
    const uint32_t b_km = static_cast<uint32_t>(b_row0) * ldb2 + km_chunk * 16;
    const uint32_t b_km_lim = static_cast<uint32_t>(b_rowlim) * ldb2 + km_chunk * 16;

    auto dma = [&](int st, uint32_t stage_off, int q) {
        const int s = st < ns ? st : ns - 1;  // past the end: reload the last stage (never read)
        if (q < 8) {  // A
            const uint32_t dst = lds0 + stage_off + static_cast<uint32_t>(q * 4 + wv) * 1024u;
            if (!AT) {
                uint32_t v = a_km;
                asm volatile("" : "+v"(v));  // recomputed per DMA, not held for every q
                v = min(v + static_cast<uint32_t>(8 * q) * lda2, a_km_lim);
                dma16(abase, v + static_cast<uint32_t>(s) * 128u,
                      lds0 + stage_off + static_cast<uint32_t>(64 * wv + 8 * q) * 128u);
            } else {
                const int k = s * kSK + 8 * q + tx_row;
                const uint32_t off = k < klen ? static_cast<uint32_t>(k) * lda2 + ((q & 1) ? ax1 : ax0) : a_zero_off;
                dma16(abase, off, dst);
            }
        } else {      // B
            const int qb = q - 8;
            const uint32_t dst = lds0 + stage_off + kOpB + static_cast<uint32_t>(qb * 4 + wv) * 1024u;
            if (!BT) {
                uint32_t v = b_km;
                asm volatile("" : "+v"(v));
                v = min(v + static_cast<uint32_t>(8 * qb) * ldb2, b_km_lim);
                dma16(bbase, v + static_cast<uint32_t>(s) * 128u,
                      lds0 + stage_off + kOpB + static_cast<uint32_t>(64 * wv + 8 * qb) * 128u);
            } else {
                int k = s * kSK + 8 * qb + tx_row;
                if (k >= kb_lim) k = kb_lim - 1;  // A is zero there
                dma16(bbase, static_cast<uint32_t>(k) * ldb2 + ((qb & 1) ? bx1 : bx0), dst);
            }
        }
    };

    // ---- fragment reads ----------------------------------------------------------
    // K-major: sub-step j reads logical chunk 4 j + lane / 16 of row lane % 16.
    const int xo0 = ((lane >> 4) ^ (lane & 7)) << 4;
    const int xo1 = ((4 + (lane >> 4)) ^ (lane & 7)) << 4;
    // [K][X]: lane (block b, index s) reads k-row 32 j + 8 b + 4 h + s / 4,
    // x-values 16 t + 4 (s % 4) .. + 3, at block t ^ hl.
    const int tb = lane >> 4, ts_ = lane & 15;
    const int hl = (ts_ >> 2) | ((tb & 1) << 2);
    const int tx_base = (8 * tb + (ts_ >> 2)) * 512 + 8 * (ts_ & 3);
    auto frag = [&](uint32_t stage_off, int j, int op, int t) -> u32x4 {
        // op 0: A block t (rows 16 t of the wave's 128), op 1: B block t
        // (SW: gate blocks 4 wn + t, then the matching up blocks 8 + 4 wn + t)
        const int wblk = op == 0 ? wm * 8 + t : (SW ? (t < 4 ? 4 * wn + t : 4 + 4 * wn + t) : wn * 8 + t);
        const lds_u8* st = smem + stage_off + (op == 0 ? 0 : kOpB);
        const bool tr = op == 0 ? AT : BT;
        if (!tr) {
            return *reinterpret_cast<lds_u32x4*>(st + (wblk * 16 + (lane & 15)) * 128 + (j == 0 ? xo0 : xo1));
        } else {
            const lds_u8* q = st + tx_base + 32 * j * 512 + (((wblk & 8) | ((wblk & 7) ^ hl)) << 5);
            const bwd_v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(q));
            const bwd_v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(q + 4 * 512));
            const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
            return u32x4{l2.x, l2.y, h2.x, h2.y};
        }
    };

    f32x4 acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // f[0..7]: A blocks, f[8..15]: B blocks of one 32-wide sub-step.  One
    // sub-step: 64 MFMAs, the next sub-step's 16 fragments read in its first
    // half, and (do_dma) the 16 DMAs of stage dst spread over it.
    auto sub = [&](const u32x4 (&f)[16], u32x4 (&nx)[16], uint32_t rs, int rj, bool do_dma, int dst, uint32_t ds) {
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int nb = 4 * h; nb < 4 * h + 4; ++nb) acc[mb][nb] = mfma_bf16(f[8 + nb], f[mb], acc[mb][nb]);
                const int q = 2 * mb + h;
                if (q < 8) {
                    nx[2 * q] = frag(rs, rj, (2 * q) >> 3, (2 * q) & 7);
                    nx[2 * q + 1] = frag(rs, rj, (2 * q + 1) >> 3, (2 * q + 1) & 7);
                }
                if (do_dma) dma(dst, ds, q);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    if (ns > 0) {
#pragma unroll
        for (int q = 0; q < 16; ++q) dma(0, 0, q);
#pragma unroll
        for (int q = 0; q < 16; ++q) dma(1, kStageB, q);
        wait_vmem<16>();
        __syncthreads();
        u32x4 f0[16], f1[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) f0[k] = frag(0, 0, k >> 3, k & 7);
        for (int st = 0; st < ns; ++st) {
            const uint32_t cur = static_cast<uint32_t>(st & 1) * kStageB;
            const uint32_t nxt = static_cast<uint32_t>((st + 1) & 1) * kStageB;
            // first half: fragments of this stage's second half
            sub(f0, f1, cur, 1, false, 0, 0);
            // stage st+1 has landed and every wave is done with stage st
            wait_vmem<0>();
            __syncthreads();
            __builtin_amdgcn_sched_barrier(0);
            // second half: fragments of the next stage's first half; stage st+2 into this buffer
            sub(f1, f0, nxt, 0, true, st + 2, cur);
        }
        wait_vmem<0>();
    }

    if constexpr (SW) {
        // ---- SwiGLU backward epilogue: acc[mb][nb] (gate) and acc[mb][nb + 4]
        // (up) hold the same (row, column); dH gate and up halves, then A, each
        // staged through LDS (256 rows x 272 B) and stored as whole 256-byte rows.
        constexpr int kSR = 272;
        const int c4 = 4 * (lane >> 4);
        const int cl0 = 64 * wn + c4;  // tile column of block 0
        auto put = [&](int buf, int mb, int nb, uint32_t lo, uint32_t hi) {
            *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(
                smem + buf * 256 * kSR + (wm * 128 + mb * 16 + (lane & 15)) * kSR + (cl0 + nb * 16) * 2) = u32x2{lo, hi};
        };
        auto drain = [&](int buf, uint16_t* base, int64_t ld) {
            const int cc = nt * 128 + 8 * (lane & 15);
            for (int r = 4 * wv + (lane >> 4); r < kT; r += 16) {
                const u32x4 v = *reinterpret_cast<lds_u32x4*>(smem + buf * 256 * kSR + r * kSR + 16 * (lane & 15));
                if (r < mrows && cc < p.I)
                    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(base + (m0 + r) * ld + cc));
            }
        };
        __syncthreads();  // every wave is done with the stages
        uint32_t apk[8][4][2];  // A, packed, until the dH tiles have left LDS
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) {
            const int m = wm * 128 + mb * 16 + (lane & 15);
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                const int c = nt * 128 + cl0 + nb * 16;
                f32x4 d = f32x4{0.f, 0.f, 0.f, 0.f};
                if (m < mrows && c < p.I) d = *reinterpret_cast<const f32x4*>(p.da + (m0 + m) * p.I + c);
                float dg[4], du[4], av[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) swiglu_grad(acc[mb][nb][i], acc[mb][nb + 4][i], d[i], dg[i], du[i], av[i]);
                put(0, mb, nb, bwd_pack_bf16(dg[0], dg[1]), bwd_pack_bf16(dg[2], dg[3]));
                put(1, mb, nb, bwd_pack_bf16(du[0], du[1]), bwd_pack_bf16(du[2], du[3]));
                apk[mb][nb][0] = bwd_pack_bf16(av[0], av[1]);
                apk[mb][nb][1] = bwd_pack_bf16(av[2], av[3]);
            }
            __builtin_amdgcn_sched_barrier(0);  // one row block's dA loads live at a time
        }
        __syncthreads();
        drain(0, p.dh, 2 * static_cast<int64_t>(p.I));
        drain(1, p.dh + p.I, 2 * static_cast<int64_t>(p.I));
        __syncthreads();
#pragma unroll
        for (int mb = 0; mb < 8; ++mb)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) put(0, mb, nb, apk[mb][nb][0], apk[mb][nb][1]);
        __syncthreads();
        drain(0, p.act, p.I);
        return;
    }

    // ---- output: through LDS, 128 rows at a time (row stride padded by 16
    // bytes against bank conflicts), so that each store writes one whole
    // 1 KiB output row; streaming (non-temporal) stores ---------------------------
    float* cb = p.c + (GK ? static_cast<int64_t>(g) * p.c_gstride : 0);
    const int c4 = 4 * (lane >> 4);
    const int mlim = GK ? p.m_valid - mt * kT : mrows;
    const int64_t row0 = GK ? static_cast<int64_t>(mt) * kT : m0;
    const int ncols = min(kT, p.N - n0);
    constexpr int kOR = 1040;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        __syncthreads();
        if (wm == half) {
#pragma unroll
            for (int mb = 0; mb < 8; ++mb)
#pragma unroll
                for (int nb = 0; nb < 8; ++nb)
                    *reinterpret_cast<__attribute__((address_space(3))) f32x4*>(
                        smem + (mb * 16 + (lane & 15)) * kOR + (wn * 128 + nb * 16 + c4) * 4) = acc[mb][nb];
        }
        __syncthreads();
        for (int r = wv; r < 128; r += 4) {
            const int row = half * 128 + r;
            const f32x4 v = *reinterpret_cast<__attribute__((address_space(3))) f32x4*>(smem + r * kOR + lane * 16);
            if (row < mlim && 4 * lane < ncols) __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(cb + (row0 + row) * p.ldc + n0 + 4 * lane));
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

// rows p < *count of x gathered by perm: xp[p] = x[perm[p]] (16 bytes per thread)
__global__ __launch_bounds__(kBwdThreads) void gather_rows_kernel(const uint16_t* __restrict__ x,
                                                                  const int32_t* __restrict__ perm,
                                                                  const int32_t* __restrict__ count, int D,
                                                                  uint16_t* __restrict__ xp) {
    const int64_t p = blockIdx.x;
    if (p >= *count) return;
    const int64_t t = perm[p];
    for (int d0 = threadIdx.x * 8; d0 < D; d0 += kBwdThreads * 8)
        *reinterpret_cast<u32x4*>(xp + p * D + d0) = *reinterpret_cast<const u32x4*>(x + t * D + d0);
}

// K-slices of a single-group weight-gradient GEMM: off[i] = min(i * len, rows)
__global__ void split_bounds_kernel(int32_t* __restrict__ off, int S, int rows, int len) {
    const int i = threadIdx.x;
    if (i <= S) off[i] = min(i * len, rows);
}

// out[m][n] = sum over s = 0..S-1, in that order, of part[s][m][n] (float32);
// m < M rows of N columns, four columns per thread
__global__ __launch_bounds__(kBwdThreads) void sum_slices_kernel(const float* __restrict__ part, int S, int64_t M,
                                                                 int N, float* __restrict__ out) {
    const int64_t i = (static_cast<int64_t>(blockIdx.x) * kBwdThreads + threadIdx.x) * 4;
    const int64_t mn = M * N;
    if (i >= mn) return;
    f32x4 a = *reinterpret_cast<const f32x4*>(part + i);
    for (int s = 1; s < S; ++s) a = a + *reinterpret_cast<const f32x4*>(part + s * mn + i);
    __builtin_nontemporal_store(a, reinterpret_cast<f32x4*>(out + i));
}

// n 16-byte words of zeros at each of up to four addresses
__global__ void zero_tails_kernel(uint8_t* a, uint8_t* b, uint8_t* c, uint8_t* d, int n) {
    const int i = threadIdx.x;
    uint8_t* dst[4] = {a, b, c, d};
    for (int k = 0; k < 4; ++k)
        if (dst[k] != nullptr && i < n) reinterpret_cast<u32x4*>(dst[k])[i] = u32x4{0u, 0u, 0u, 0u};
}

// n4 groups of four float32 zeros
__global__ __launch_bounds__(256) void zero_f32x4_kernel(float* __restrict__ p, int64_t n4) {
    const int64_t step = static_cast<int64_t>(gridDim.x) * 256;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n4; i += step)
        reinterpret_cast<f32x4*>(p)[i] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// ===========================================================================
// launcher
// ===========================================================================
// tiles: an upper bound of the tile count (padded to a multiple of 8 for the
// XCD mapping; tiles past the real count exit at once)
template <bool AT, bool BT, bool GK, bool SW = false>
static hipError_t gemm(const BwdGemm& p, int64_t tiles, hipStream_t stream) {
    if (tiles <= 0) return hipSuccess;
    const int64_t n = (tiles + 7) / 8 * 8;
    bwd_gemm_kernel<AT, BT, GK, SW><<<dim3(static_cast<unsigned>(n)), 256, 0, stream>>>(p);
    return hipGetLastError();
}

static BwdOperand op(const void* base, int64_t ld, int64_t gstride = 0) {
    return BwdOperand{static_cast<const uint16_t*>(base), ld, gstride};
}

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

namespace {
struct BwdLayout {
    size_t logits, dw, dY, dYs, dA, dH, Aact, xp, dXp, dXs, dxr, dl, ts, slices, bounds, total;
};

// K-slices of a single-group weight-gradient GEMM with `tiles` output tiles
// over `rows` rows: enough slices to give 256 workgroups, each slice at least
// 1024 rows, at most 64.  A function of the shape only, so the summation
// order (and the bits) never depend on the device.
int wgrad_slices(int64_t tiles, int64_t rows) {
    int64_t s = (256 + tiles - 1) / tiles;
    const int64_t by_rows = rows / 1024;
    if (s > by_rows) s = by_rows;
    if (s > 64) s = 64;
    return s < 1 ? 1 : static_cast<int>(s);
}
BwdLayout bwd_layout(int64_t T, int D, int E, int K, int I, int Is) {
    const int64_t P = T * K;
    const int64_t rows2 = P * 2 * I > T * 2 * static_cast<int64_t>(Is) ? P * 2 * I : T * 2 * static_cast<int64_t>(Is);
    const int64_t rows1 = P * I > T * static_cast<int64_t>(Is) ? P * I : T * static_cast<int64_t>(Is);
    const int64_t Epad = (E + 63) / 64 * 64;
    BwdLayout l{};
    size_t b = 0;
    auto take = [&](size_t n) {
        const size_t at = b;
        b += (n + 255) & ~static_cast<size_t>(255);
        return at;
    };
    l.logits = take(sizeof(double) * T * E);
    l.dw = take(sizeof(double) * P);
    l.dY = take(2 * static_cast<size_t>(P) * D + kZeroTail);      // zero tail: K-grouped A operand
    l.dYs = take(2 * static_cast<size_t>(T) * D + kZeroTail);
    l.dA = take(4 * static_cast<size_t>(rows1));
    l.dH = take(2 * static_cast<size_t>(rows2) + kZeroTail);
    l.Aact = take(2 * static_cast<size_t>(rows1));
    l.xp = take(2 * static_cast<size_t>(P) * D);
    l.dXp = take(4 * static_cast<size_t>(P) * D);
    l.dXs = take(4 * static_cast<size_t>(T) * D);
    l.dxr = take(4 * static_cast<size_t>(T) * D);
    l.dl = take(2 * static_cast<size_t>(T) * Epad + kZeroTail);
    l.ts = take(sizeof(int32_t) * (E + 1));
    // partial sums of the sliced weight gradients (shared down, shared gate_up, router)
    size_t sl = 0;
    auto need = [&](int64_t M, int64_t N) {
        const int S = wgrad_slices(cdiv(M, kT) * cdiv(N, kT), T);
        if (S > 1) sl = std::max(sl, static_cast<size_t>(S) * M * N * 4);
    };
    if (Is > 0) {
        need(D, Is);
        need(2 * static_cast<int64_t>(Is), D);
    }
    need(E, D);
    l.slices = take(sl);
    l.bounds = take(sizeof(int32_t) * 65);
    l.total = b;
    return l;
}
}  // namespace

size_t backward_ws_bytes(int64_t T, int D, int E, int K, int I, int Is) { return bwd_layout(T, D, E, K, I, Is).total; }

bool backward_fits_dma(int64_t T, int D, int K, int I, int Is) {
    // every DMA-staged buffer (and its zero tail) spans less than 4 GiB: the
    // GEMMs address it with 32-bit offsets from a group's first row
    const int64_t P = T * K;
    const int64_t lim = (int64_t{1} << 32) - 2 * kZeroTail;
    const int64_t w = 2 * I > D ? 2 * I : D;
    const int64_t ws = 2 * Is > D ? 2 * Is : D;
    return 2 * P * w < lim && 2 * T * ws < lim;
}

hipError_t launch_backward(const BwdArgs& a, hipStream_t stream) {
    const int64_t T = a.T;
    const int D = a.D, E = a.E, K = a.K, I = a.I, Is = a.Is;
    const int64_t P = T * K;
    const int Epad = (E + 63) / 64 * 64;
    const BwdLayout lo = bwd_layout(T, D, E, K, I, Is);
    uint8_t* w = static_cast<uint8_t*>(a.ws);
    double* logits = reinterpret_cast<double*>(w + lo.logits);
    double* dw = reinterpret_cast<double*>(w + lo.dw);
    uint16_t* dY = reinterpret_cast<uint16_t*>(w + lo.dY);
    uint16_t* dYs = reinterpret_cast<uint16_t*>(w + lo.dYs);
    float* dA = reinterpret_cast<float*>(w + lo.dA);
    uint16_t* dH = reinterpret_cast<uint16_t*>(w + lo.dH);
    uint16_t* Aact = reinterpret_cast<uint16_t*>(w + lo.Aact);
    uint16_t* xp = reinterpret_cast<uint16_t*>(w + lo.xp);
    float* dXp = reinterpret_cast<float*>(w + lo.dXp);
    float* dXs = reinterpret_cast<float*>(w + lo.dXs);
    float* dxr = reinterpret_cast<float*>(w + lo.dxr);
    uint16_t* dl = reinterpret_cast<uint16_t*>(w + lo.dl);
    int32_t* ts = reinterpret_cast<int32_t*>(w + lo.ts);
    float* slices = reinterpret_cast<float*>(w + lo.slices);
    int32_t* bounds = reinterpret_cast<int32_t*>(w + lo.bounds);
    const int64_t rows2 = P * 2 * I > T * 2 * static_cast<int64_t>(Is) ? P * 2 * I : T * 2 * static_cast<int64_t>(Is);
    // the zero tails sit right after each buffer's rows
    uint8_t* z_dY = reinterpret_cast<uint8_t*>(dY) + 2 * static_cast<size_t>(P) * D;
    uint8_t* z_dYs = reinterpret_cast<uint8_t*>(dYs) + 2 * static_cast<size_t>(T) * D;
    uint8_t* z_dH = reinterpret_cast<uint8_t*>(dH) + 2 * static_cast<size_t>(rows2);
    uint8_t* z_dl = reinterpret_cast<uint8_t*>(dl) + 2 * static_cast<size_t>(T) * Epad;

    hipError_t err;
    // A single-group weight gradient (K = the T rows).  With few output tiles
    // its rows are cut into wgrad_slices() slices of a multiple of 64 rows,
    // each slice's float32 partial written on its own, then summed in slice
    // order: a fixed order for a given shape.
    auto wgrad = [&](BwdGemm k1, float* out) -> hipError_t {
        const int64_t tiles = cdiv(k1.M, kT) * cdiv(k1.N, kT);
        const int S = wgrad_slices(tiles, k1.rows);
        if (S == 1) {
            k1.c = out;
            return gemm<true, true, true>(k1, tiles, stream);
        }
        const int len = static_cast<int>(cdiv(cdiv(k1.rows, S), kSK) * kSK);
        split_bounds_kernel<<<1, 65, 0, stream>>>(bounds, S, k1.rows, len);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        k1.offsets = bounds;
        k1.G = S;
        k1.c = slices;
        k1.ldc = k1.N;
        k1.c_gstride = static_cast<int64_t>(k1.m_valid) * k1.N;
        if ((e = gemm<true, true, true>(k1, tiles * S, stream)) != hipSuccess) return e;
        const int64_t mn4 = static_cast<int64_t>(k1.m_valid) * k1.N / 4;
        sum_slices_kernel<<<static_cast<unsigned>(cdiv(mn4, kBwdThreads)), kBwdThreads, 0, stream>>>(
            slices, S, k1.m_valid, k1.N, out);
        return hipGetLastError();
    };
    zero_tails_kernel<<<1, kZeroTail / 16, 0, stream>>>(z_dY, z_dYs, z_dH, z_dl, kZeroTail / 16);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if ((err = launch_router_logits(a.x, a.router, T, D, E, 0, logits, stream)) != hipSuccess) return err;
    combine_bwd_kernel<<<static_cast<unsigned>(T), kBwdThreads, 0, stream>>>(
        static_cast<const uint16_t*>(a.dout), static_cast<const uint16_t*>(a.y), a.inv_pos, a.topk_w, a.mask, T, D,
        K, dY, dw, Is > 0 ? dYs : nullptr);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    bwd_tile_prefix_kernel<<<1, 1024, 0, stream>>>(a.offsets, E, ts);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    gather_rows_kernel<<<static_cast<unsigned>(P), kBwdThreads, 0, stream>>>(
        static_cast<const uint16_t*>(a.x), a.perm_token, a.offsets + E, D, xp);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    const int64_t mt_routed = cdiv(P, kT) + E;  // bound on the routed m-tiles

    // routed experts
    BwdGemm g{};
    g.offsets = a.offsets;
    g.tile_start = ts;
    g.G = E;
    // dA = dY W2_e
    g.a = op(dY, D);
    g.b = op(a.down, I, static_cast<int64_t>(D) * I);
    g.c = dA; g.ldc = I; g.N = I; g.K = D; g.kb_valid = D;
    if ((err = gemm<false, true, false>(g, mt_routed * cdiv(g.N, kT), stream)) != hipSuccess) return err;
    // H = Xp W1_e^T recomputed, and from it and dA: dH and A
    g.a = op(xp, D);
    g.b = op(a.gate_up, D, static_cast<int64_t>(2) * I * D);
    g.c = nullptr; g.N = 2 * I; g.K = D; g.kb_valid = D;
    g.I = I; g.da = dA; g.dh = dH; g.act = Aact;
    if ((err = gemm<false, false, false, true>(g, mt_routed * cdiv(I, 128), stream)) != hipSuccess) return err;
    // dXp = dH W1_e
    g.a = op(dH, 2 * I);
    g.b = op(a.gate_up, D, static_cast<int64_t>(2) * I * D);
    g.c = dXp; g.ldc = D; g.N = D; g.K = 2 * I; g.kb_valid = 2 * I;
    if ((err = gemm<false, true, false>(g, mt_routed * cdiv(g.N, kT), stream)) != hipSuccess) return err;
    // dW2_e = dY_e^T A_e
    BwdGemm k{};
    k.offsets = a.offsets;
    k.G = E;
    k.a = op(dY, D);
    k.a_zero = reinterpret_cast<const uint16_t*>(z_dY);
    k.b = op(Aact, I);
    k.c = a.d_down; k.ldc = I; k.c_gstride = static_cast<int64_t>(D) * I; k.M = D; k.N = I; k.m_valid = D;
    if ((err = gemm<true, true, true>(k, E * cdiv(k.M, kT) * cdiv(k.N, kT), stream)) != hipSuccess) return err;
    // dW1_e = dH_e^T Xp_e
    k.a = op(dH, 2 * I);
    k.a_zero = reinterpret_cast<const uint16_t*>(z_dH);
    k.b = op(xp, D);
    k.c = a.d_gate_up; k.ldc = D; k.c_gstride = static_cast<int64_t>(2) * I * D; k.M = 2 * I; k.N = D;
    k.m_valid = 2 * I;
    if ((err = gemm<true, true, true>(k, E * cdiv(k.M, kT) * cdiv(k.N, kT), stream)) != hipSuccess) return err;

    // shared expert: one group of T rows, dY = G on kept tokens
    if (Is > 0) {
        BwdGemm s{};
        s.G = 1;
        s.rows = static_cast<int>(T);
        s.a = op(dYs, D);
        s.b = op(a.down_shared, Is);
        s.c = dA; s.ldc = Is; s.N = Is; s.K = D; s.kb_valid = D;
        if ((err = gemm<false, true, false>(s, cdiv(T, kT) * cdiv(s.N, kT), stream)) != hipSuccess) return err;
        s.a = op(a.x, D);
        s.b = op(a.gate_up_shared, D);
        s.c = nullptr; s.N = 2 * Is; s.K = D; s.kb_valid = D;
        s.I = Is; s.da = dA; s.dh = dH; s.act = Aact;
        if ((err = gemm<false, false, false, true>(s, cdiv(T, kT) * cdiv(Is, 128), stream)) != hipSuccess) return err;
        s.a = op(dH, 2 * Is);
        s.b = op(a.gate_up_shared, D);
        s.c = dXs; s.ldc = D; s.N = D; s.K = 2 * Is; s.kb_valid = 2 * Is;
        if ((err = gemm<false, true, false>(s, cdiv(T, kT) * cdiv(s.N, kT), stream)) != hipSuccess) return err;
        BwdGemm sk{};
        sk.G = 1;
        sk.rows = static_cast<int>(T);
        sk.a = op(dYs, D);
        sk.a_zero = reinterpret_cast<const uint16_t*>(z_dYs);
        sk.b = op(Aact, Is);
        sk.ldc = Is; sk.M = D; sk.N = Is; sk.m_valid = D;
        if ((err = wgrad(sk, a.d_down_shared)) != hipSuccess) return err;
        sk.a = op(dH, 2 * Is);
        sk.a_zero = reinterpret_cast<const uint16_t*>(z_dH);
        sk.b = op(a.x, D);
        sk.ldc = D; sk.M = 2 * Is; sk.N = D; sk.m_valid = 2 * Is;
        if ((err = wgrad(sk, a.d_gate_up_shared)) != hipSuccess) return err;
    }

    // router
    router_bwd_kernel<<<static_cast<unsigned>((T + 3) / 4), 256, 0, stream>>>(
        logits, a.topk_ids, dw, a.mask, T, E, K, a.score, a.renorm, static_cast<double>(a.route_scale), dl, Epad);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    {
        BwdGemm r{};
        r.G = 1;
        r.rows = static_cast<int>(T);
        r.a = op(dl, Epad);
        r.b = op(a.router, D);
        r.c = dxr; r.ldc = D; r.N = D; r.K = Epad; r.kb_valid = E;
        if ((err = gemm<false, true, false>(r, cdiv(T, kT) * cdiv(r.N, kT), stream)) != hipSuccess) return err;
        BwdGemm rk{};
        rk.G = 1;
        rk.rows = static_cast<int>(T);
        rk.a = op(dl, Epad);
        rk.a_zero = reinterpret_cast<const uint16_t*>(z_dl);
        rk.b = op(a.x, D);
        rk.ldc = D; rk.M = Epad; rk.N = D; rk.m_valid = E;
        if ((err = wgrad(rk, a.d_router)) != hipSuccess) return err;
    }
    dx_assemble_kernel<<<static_cast<unsigned>(T), kBwdThreads, 0, stream>>>(dXp, a.inv_pos, Is > 0 ? dXs : nullptr,
                                                                             dxr, a.mask, T, D, K, a.dx);
    return hipGetLastError();
}

// An empty batch: every weight gradient is a sum over no tokens, so zeros.
hipError_t launch_backward_empty(const BwdArgs& a, hipStream_t stream) {
    const int64_t D = a.D;
    struct { float* p; int64_t n; } bufs[5] = {
        {a.d_router, a.E * D},
        {a.d_gate_up, a.E * 2 * a.I * D},
        {a.d_down, a.E * D * a.I},
        {a.Is > 0 ? a.d_gate_up_shared : nullptr, 2 * a.Is * D},
        {a.Is > 0 ? a.d_down_shared : nullptr, D * a.Is},
    };
    for (const auto& b : bufs) {
        if (b.p == nullptr || b.n == 0) continue;
        const int64_t n4 = b.n / 4;  // D is a multiple of 64
        const int64_t blocks = (n4 + 255) / 256;
        zero_f32x4_kernel<<<static_cast<unsigned>(blocks < 4096 ? blocks : 4096), 256, 0, stream>>>(b.p, n4);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

}  // namespace moe
