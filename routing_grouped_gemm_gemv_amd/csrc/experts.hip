// Routed (and shared) expert MLPs as a pair of grouped GEMMs on MFMA.
//
// The expert boundary of the RL-Kernel roadmap ("DSV4 Flash MoE
// Train-Inference Consistency Roadmap", Problem 2: gate_and_up -> down, with
// the accumulation dtype and the rounding points part of the contract) and the
// grouped-GEMM experts of SpecForge pull request #1003 ("Design notes"):
//
//   gate_up kernel:  h = x[src(p)] . W1[g]^T over the rows p of group g,
//                    epilogue a = silu(h_gate) * h_up (fp32), stored in the
//                    operand dtype (bf16 rounds to nearest even);
//   down kernel:     y[p] = a[p] . W2[g]^T, stored in the operand dtype.
//
// Batch invariance.  Every output element is one accumulator chain: one MFMA
// instruction shape per operand dtype (16x16x32 bf16, or 16x16x4 f32), the
// reduction dimension walked upward in fixed steps from a zero accumulator,
// no split-K.  Tile and grid shapes only decide which workgroup owns an
// element, never how it is summed, so an element's bits do not depend on how
// many rows its expert received, where in a tile its row sits, or on T.
//
// bf16 kernel: 256 x 256 output tile per 256-thread workgroup (4 waves as
// 2 x 2, 128 x 128 per wave: 64 accumulator blocks of 16 x 16).  The k
// dimension advances in 64-element slices (128 bytes per row) double-buffered
// in 128 KiB of LDS.  Slices are fetched with global_load_lds_dwordx4, which
// writes each lane's 16 bytes straight into LDS at (wave base + 16 * lane):
// the XOR swizzle of the 16-byte chunks of a row (chunk ^ row % 8, which makes
// the MFMA fragment reads conflict-free) is therefore applied to the global
// addresses each lane fetches.  The next slice is in flight while the current
// one is multiplied.  For gate_up the 256 weight rows of a tile are 128 gate
// rows and the matching 128 up rows, so the SwiGLU epilogue pairs registers
// of the same wave.
//
// fp32 kernel (the fp32-operand mode): 128 x 128 tiles staged through
// registers, 16x16x4 f32 MFMA.
//
// Tiles are ordered (group, n-tile, m-tile) and each XCD receives a
// contiguous range of them, so the m-tiles sharing a weight slice meet in
// one L2.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kRowBytes = 128;  // bytes of one tile row per k slice

struct GemmParams {
    const void* a;             // gate_up: x [*, Kd] (rows via perm); down: act [rows, Kd]
    const int32_t* perm;       // gate_up: perm_token or nullptr (identity)
    const int32_t* offsets;    // [G+1] or nullptr (one group of ident_rows rows)
    const int32_t* tile_start; // [G+1] m-tile prefix sums (with offsets)
    int64_t ident_rows;
    int G;
    int Kd;                    // reduction length
    const void* w;             // [G, Nw, Kd]
    int64_t w_group_stride;    // Nw * Kd elements
    int I;                     // gate_up: intermediate size (first up row); down: unused
    int n_tiles;               // output column tiles per group
    void* out;
    int ldo;                   // columns of the output (I for gate_up, D for down)
};

__global__ __launch_bounds__(1024) void build_tiles_kernel(const int32_t* __restrict__ offsets, int G, int bm,
                                                           int32_t* __restrict__ tile_start) {
    __shared__ int part[1024];
    const int tid = threadIdx.x;
    // G <= 1024: one group per thread
    int mt = 0;
    if (tid < G) mt = (offsets[tid + 1] - offsets[tid] + bm - 1) / bm;
    part[tid] = mt;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {
        const int v = tid >= d ? part[tid - d] : 0;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    if (tid < G) tile_start[tid] = part[tid] - mt;
    if (tid == G - 1) tile_start[G] = part[tid];
}

struct TileCoord {
    int g;
    int64_t m0;
    int rows;
    int n;
};

// Which tile this workgroup owns; false if none (grid padding).
template <int BM>
__device__ __forceinline__ bool locate_tile(const GemmParams& p, TileCoord& tc) {
    int64_t total;
    if (p.offsets == nullptr) total = ((p.ident_rows + BM - 1) / BM) * p.n_tiles;
    else total = static_cast<int64_t>(p.tile_start[p.G]) * p.n_tiles;
    const int64_t padded = (total + 7) & ~static_cast<int64_t>(7);
    if (static_cast<int64_t>(blockIdx.x) >= padded) return false;
    const int64_t L = xcd_remap(blockIdx.x, padded);
    if (L >= total) return false;
    if (p.offsets == nullptr) {
        const int64_t mt = (p.ident_rows + BM - 1) / BM;
        tc.g = 0;
        tc.n = static_cast<int>(L / mt);
        tc.m0 = (L % mt) * BM;
        const int64_t left = p.ident_rows - tc.m0;
        tc.rows = left < BM ? static_cast<int>(left) : BM;
    } else {
        int lo = 0, hi = p.G - 1;  // last g with tile_start[g] * n_tiles <= L
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (static_cast<int64_t>(p.tile_start[mid]) * p.n_tiles <= L) lo = mid; else hi = mid - 1;
        }
        tc.g = lo;
        const int ts = p.tile_start[lo];
        const int mtg = p.tile_start[lo + 1] - ts;
        const int64_t local = L - static_cast<int64_t>(ts) * p.n_tiles;
        tc.n = static_cast<int>(local / mtg);
        const int m = static_cast<int>(local % mtg);
        tc.m0 = p.offsets[lo] + static_cast<int64_t>(m) * BM;
        const int left = p.offsets[lo + 1] - static_cast<int>(tc.m0);
        tc.rows = left < BM ? left : BM;
    }
    return true;
}

__device__ __forceinline__ int swz(int row, int chunk) { return row * kRowBytes + ((chunk ^ (row & 7)) << 4); }

__device__ __forceinline__ float silu_mul(float g, float u) { return (g / (1.0f + expf(-g))) * u; }

// ===========================================================================
// bf16 operands: 256 x 256 tiles, direct-to-LDS slices
// ===========================================================================
constexpr int kBM2 = 256;
constexpr int kBN2 = 256;
constexpr int kStage2 = (kBM2 + kBN2) * kRowBytes;  // 64 KiB: one A and one B slice

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

// 16 bytes per lane from global memory into LDS at wave_base + 16 * lane
__device__ __forceinline__ void dma16(const void* g, uint8_t* wave_base) {
    __builtin_amdgcn_global_load_lds((gbl_void_t*)g, (lds_void_t*)wave_base, 16, 0, 0);
}

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x3F70); }  // vmcnt(0)

template <bool GATE_UP>
__global__ __launch_bounds__(256) void grouped_gemm_bf16_kernel(GemmParams p) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kStage2];

    TileCoord tc;
    if (!locate_tile<kBM2>(p, tc)) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int wm = wv >> 1;
    const int wn = wv & 1;

    // ---- per-lane sources of the 8 + 8 DMA instructions of this wave ------
    // Instruction i fills rows wv*64 + 8i .. +7 of the A and B slices; lane l
    // lands on row (l / 8) of that group at physical chunk l % 8, so it fetches
    // logical chunk (l % 8) ^ (row % 8).
    // Byte offsets fit 32 bits: x, the activations and one group's weights are
    // each below 4 GiB (checked by the launcher), so the DMA addresses are a
    // uniform base plus one 32-bit offset per instruction.
    const uint8_t* __restrict__ abase = static_cast<const uint8_t*>(p.a);
    const uint8_t* __restrict__ wbase =
        static_cast<const uint8_t*>(p.w) + static_cast<int64_t>(tc.g) * p.w_group_stride * 2;
    const int chunk = (lane & 7) ^ ((lane >> 3) & 7);
    uint32_t aoff[8], boff[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = wv * 64 + 8 * i + (lane >> 3);
        const int rr = r < tc.rows ? r : tc.rows - 1;  // rows past the group repeat its last row; never stored
        int64_t src = tc.m0 + rr;
        if (GATE_UP && p.perm != nullptr) src = p.perm[src];
        aoff[i] = static_cast<uint32_t>(src * p.Kd * 2 + chunk * 16);
        int wrow;
        if (GATE_UP) {
            int c = tc.n * 128 + (r & 127);  // gate row; the matching up row is I + c
            if (c >= p.I) c = p.I - 1;       // I % 128 == 64: last tile half full
            wrow = r < 128 ? c : p.I + c;
        } else {
            wrow = tc.n * kBN2 + r;
            if (wrow >= p.ldo) wrow = p.ldo - 1;
        }
        boff[i] = static_cast<uint32_t>(static_cast<int64_t>(wrow) * p.Kd * 2 + chunk * 16);
    }
    uint8_t* const a_dst = smem + wv * 64 * kRowBytes;
    uint8_t* const b_dst = smem + kBM2 * kRowBytes + wv * 64 * kRowBytes;

    // LDS byte offsets of this lane's MFMA fragments: block b adds b * 16 rows;
    // the swizzle term depends only on the lane (row % 8 == lane % 8)
    const int a_frag = (wm * 128 + (lane & 15)) * kRowBytes;
    const int b_frag = ((GATE_UP ? wn * 64 : wn * 128) + (lane & 15)) * kRowBytes;
    auto b_row_off = [&](int b) {
        if (GATE_UP) return (b < 4 ? b * 16 : 128 + (b - 4) * 16) * kRowBytes;
        return b * 16 * kRowBytes;
    };

    f32x4 acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = p.Kd / 64;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        dma16(abase + aoff[i], a_dst + i * 8 * kRowBytes);
        dma16(wbase + boff[i], b_dst + i * 8 * kRowBytes);
    }
    wait_vmem();
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) {
            const int st = (cur ^ 1) * kStage2;
            const int kb = (kt + 1) * 128;  // bytes
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                dma16(abase + (aoff[i] + kb), a_dst + st + i * 8 * kRowBytes);
                dma16(wbase + (boff[i] + kb), b_dst + st + i * 8 * kRowBytes);
            }
        }
        const uint8_t* sa = smem + cur * kStage2;
        const uint8_t* sb = sa + kBM2 * kRowBytes;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int xo = ((4 * s + (lane >> 4)) ^ (lane & 7)) << 4;
            u32x4 af[8], bf[8];
#pragma unroll
            for (int b = 0; b < 8; ++b) af[b] = *reinterpret_cast<const u32x4*>(sa + a_frag + xo + b * 16 * kRowBytes);
#pragma unroll
            for (int b = 0; b < 8; ++b) bf[b] = *reinterpret_cast<const u32x4*>(sb + b_frag + xo + b_row_off(b));
#pragma unroll
            for (int mb = 0; mb < 8; ++mb)
#pragma unroll
                for (int nb = 0; nb < 8; ++nb) acc[mb][nb] = mfma_bf16(af[mb], bf[nb], acc[mb][nb]);
        }
        wait_vmem();
        __syncthreads();
    }

    // ---- epilogue ---------------------------------------------------------
    uint16_t* __restrict__ out = static_cast<uint16_t*>(p.out);
    if (GATE_UP) {
#pragma unroll
        for (int mb = 0; mb < 8; ++mb)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                const int col = tc.n * 128 + wn * 64 + nb * 16 + (lane & 15);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = wm * 128 + mb * 16 + 4 * (lane >> 4) + i;
                    if (row < tc.rows && col < p.I)
                        out[(tc.m0 + row) * p.ldo + col] = f32_to_bf16(silu_mul(acc[mb][nb][i], acc[mb][nb + 4][i]));
                }
            }
    } else {
#pragma unroll
        for (int mb = 0; mb < 8; ++mb)
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) {
                const int col = tc.n * kBN2 + wn * 128 + nb * 16 + (lane & 15);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = wm * 128 + mb * 16 + 4 * (lane >> 4) + i;
                    if (row < tc.rows && col < p.ldo) out[(tc.m0 + row) * p.ldo + col] = f32_to_bf16(acc[mb][nb][i]);
                }
            }
    }
}

// ===========================================================================
// fp32 operands: 128 x 128 tiles through registers, 16x16x4 f32 MFMA
// ===========================================================================
constexpr int kBM1 = 128;
constexpr int kBN1 = 128;
constexpr int kTile1 = (kBM1 + kBN1) * kRowBytes;

template <bool GATE_UP>
__global__ __launch_bounds__(256) void grouped_gemm_f32_kernel(GemmParams p) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kTile1];

    TileCoord tc;
    if (!locate_tile<kBM1>(p, tc)) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int wm = wv >> 1;
    const int wn = wv & 1;

    const float* __restrict__ asrc = static_cast<const float*>(p.a);
    const float* __restrict__ wsrc = static_cast<const float*>(p.w) + static_cast<int64_t>(tc.g) * p.w_group_stride;
    const int ch = tid & 7;
    const float* aptr[4];
    const float* bptr[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int r = q * 32 + (tid >> 3);
        const int rr = r < tc.rows ? r : tc.rows - 1;
        int64_t src = tc.m0 + rr;
        if (GATE_UP && p.perm != nullptr) src = p.perm[src];
        aptr[q] = asrc + src * p.Kd + ch * 4;
        int wrow;
        if (GATE_UP) {
            int c = tc.n * 64 + (r & 63);
            if (c >= p.I) c = p.I - 1;
            wrow = r < 64 ? c : p.I + c;
        } else {
            wrow = tc.n * kBN1 + r;
            if (wrow >= p.ldo) wrow = p.ldo - 1;
        }
        bptr[q] = wsrc + static_cast<int64_t>(wrow) * p.Kd + ch * 4;
    }

    int brow[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
        if (GATE_UP) brow[nb] = (nb < 2 ? wn * 32 + nb * 16 : 64 + wn * 32 + (nb - 2) * 16) + (lane & 15);
        else brow[nb] = wn * 64 + nb * 16 + (lane & 15);
    }
    int sto[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) sto[q] = swz(q * 32 + (tid >> 3), ch);

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 ra[4], rb[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        ra[q] = *reinterpret_cast<const u32x4*>(aptr[q]);
        rb[q] = *reinterpret_cast<const u32x4*>(bptr[q]);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        *reinterpret_cast<u32x4*>(smem + sto[q]) = ra[q];
        *reinterpret_cast<u32x4*>(smem + kBM1 * kRowBytes + sto[q]) = rb[q];
    }
    __syncthreads();

    const int nk = p.Kd / 32;
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) {
            const int k1 = (kt + 1) * 32;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                ra[q] = *reinterpret_cast<const u32x4*>(aptr[q] + k1);
                rb[q] = *reinterpret_cast<const u32x4*>(bptr[q] + k1);
            }
        }
        const uint8_t* sa = smem + cur * kTile1;
        const uint8_t* sb = sa + kBM1 * kRowBytes;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int c = 4 * s + (lane >> 4);
            u32x4 af[4], bf[4];
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
                af[mb] = *reinterpret_cast<const u32x4*>(sa + swz(wm * 64 + mb * 16 + (lane & 15), c));
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) bf[nb] = *reinterpret_cast<const u32x4*>(sb + swz(brow[nb], c));
            // four K=4 steps; in step q every lane group supplies element q of its chunk
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                    for (int nb = 0; nb < 4; ++nb)
                        acc[mb][nb] = mfma_f32(__uint_as_float(af[mb][q]), __uint_as_float(bf[nb][q]), acc[mb][nb]);
        }
        if (more) {
            uint8_t* da = smem + (cur ^ 1) * kTile1;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                *reinterpret_cast<u32x4*>(da + sto[q]) = ra[q];
                *reinterpret_cast<u32x4*>(da + kBM1 * kRowBytes + sto[q]) = rb[q];
            }
        }
        __syncthreads();
    }

    float* __restrict__ out = static_cast<float*>(p.out);
    if (GATE_UP) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                const int col = tc.n * 64 + wn * 32 + nb * 16 + (lane & 15);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = wm * 64 + mb * 16 + 4 * (lane >> 4) + i;
                    if (row < tc.rows && col < p.I)
                        out[(tc.m0 + row) * p.ldo + col] = silu_mul(acc[mb][nb][i], acc[mb][nb + 2][i]);
                }
            }
    } else {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                const int col = tc.n * kBN1 + wn * 64 + nb * 16 + (lane & 15);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = wm * 64 + mb * 16 + 4 * (lane >> 4) + i;
                    if (row < tc.rows && col < p.ldo) out[(tc.m0 + row) * p.ldo + col] = acc[mb][nb][i];
                }
            }
    }
}

static size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

size_t experts_ws_bytes(int64_t rows_max, int G, int I, int dtype) {
    const size_t eb = dtype == 0 ? 2 : 4;
    return align256(sizeof(int32_t) * (G + 1)) + align256(static_cast<size_t>(rows_max) * I * eb);
}

hipError_t launch_experts(const void* x, int64_t x_rows, const int32_t* perm_token, const int32_t* offsets, int G,
                          int64_t rows_max, int D, int I, int dtype, const void* gate_up, const void* down,
                          void* y, void* ws, hipStream_t stream) {
    const bool bf16 = dtype == 0;
    const int BM = bf16 ? kBM2 : kBM1;
    const int gate_cols = bf16 ? 128 : 64;   // gate (and up) rows per gate_up tile
    const int down_cols = bf16 ? kBN2 : kBN1;
    int32_t* tile_start = static_cast<int32_t*>(ws);
    void* act = static_cast<uint8_t*>(ws) + align256(sizeof(int32_t) * (G + 1));
    if (offsets != nullptr) {
        build_tiles_kernel<<<1, 1024, 0, stream>>>(offsets, G, BM, tile_start);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    // upper bound of m-tiles: every group adds at most one partial tile
    const int64_t mt_max = (rows_max + BM - 1) / BM + (offsets != nullptr ? G : 0);

    GemmParams p1{};
    p1.a = x;
    p1.perm = perm_token;
    p1.offsets = offsets;
    p1.tile_start = offsets != nullptr ? tile_start : nullptr;
    p1.ident_rows = rows_max;
    p1.G = G;
    p1.Kd = D;
    p1.w = gate_up;
    p1.w_group_stride = static_cast<int64_t>(2) * I * D;
    p1.I = I;
    p1.n_tiles = (I + gate_cols - 1) / gate_cols;
    p1.out = act;
    p1.ldo = I;
    const int64_t nwg1 = ((mt_max * p1.n_tiles) + 7) & ~static_cast<int64_t>(7);

    GemmParams p2 = p1;
    p2.a = act;
    p2.perm = nullptr;
    p2.Kd = I;
    p2.w = down;
    p2.w_group_stride = static_cast<int64_t>(D) * I;
    p2.n_tiles = (D + down_cols - 1) / down_cols;
    p2.out = y;
    p2.ldo = D;
    const int64_t nwg2 = ((mt_max * p2.n_tiles) + 7) & ~static_cast<int64_t>(7);

    if (bf16) {
        // the bf16 kernel addresses x, the activations and one group's weights
        // with 32-bit byte offsets
        const int64_t lim = static_cast<int64_t>(1) << 32;
        if (static_cast<int64_t>(2) * I * D * 2 >= lim || rows_max * I * 2 >= lim || x_rows * D * 2 >= lim)
            return hipErrorInvalidValue;
        grouped_gemm_bf16_kernel<true><<<static_cast<unsigned>(nwg1), 256, 0, stream>>>(p1);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        grouped_gemm_bf16_kernel<false><<<static_cast<unsigned>(nwg2), 256, 0, stream>>>(p2);
    } else {
        grouped_gemm_f32_kernel<true><<<static_cast<unsigned>(nwg1), 256, 0, stream>>>(p1);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        grouped_gemm_f32_kernel<false><<<static_cast<unsigned>(nwg2), 256, 0, stream>>>(p2);
    }
    return hipGetLastError();
}

}  // namespace moe
