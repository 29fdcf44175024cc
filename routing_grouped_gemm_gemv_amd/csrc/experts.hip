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
// instruction shape (16x16x32 bf16, or 16x16x4 f32), the reduction dimension
// walked upward in fixed steps from a zero accumulator, no split-K.  Tile and
// grid shapes only decide which workgroup owns an element, never how it is
// summed, so an element's bits do not depend on how many rows its expert
// received, where in a tile its row sits, or on T.
//
// Tiling: 128 x 128 output tile per 256-thread workgroup (4 waves as 2 x 2,
// 64 x 64 per wave), 128-byte-deep k slices double-buffered in LDS with the
// 16-byte chunks of each row XOR-swizzled by the row index, global loads for
// the next slice in flight while the current one is multiplied.  For gate_up
// the 128 weight rows of a tile are 64 gate rows and the 64 matching up rows,
// so the SwiGLU epilogue pairs registers of the same wave.  Tiles are ordered
// (group, n-tile, m-tile) and each XCD receives a contiguous range of them,
// so the m-tiles that share a weight slice run on one L2.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kRowBytes = 128;                      // bytes of one tile row per k slice
constexpr int kTileBytes = (kBM + kBN) * kRowBytes;  // A + B slice

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
    int I;                     // gate_up: first up row; down: unused
    int n_tiles;               // output column tiles per group
    void* out;
    int ldo;
};

__global__ __launch_bounds__(1024) void build_tiles_kernel(const int32_t* __restrict__ offsets, int G,
                                                           int32_t* __restrict__ tile_start) {
    __shared__ int part[1024];
    const int tid = threadIdx.x;
    // G <= 1024: one group per thread
    int mt = 0;
    if (tid < G) mt = (offsets[tid + 1] - offsets[tid] + kBM - 1) / kBM;
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

template <bool BF16>
struct Elem;
template <>
struct Elem<true> {
    typedef uint16_t T;
    static constexpr int kPerChunk = 8;   // 16 bytes
    static constexpr int kSlice = 64;     // k per 128-byte row
};
template <>
struct Elem<false> {
    typedef float T;
    static constexpr int kPerChunk = 4;
    static constexpr int kSlice = 32;
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * kRowBytes + ((chunk ^ (row & 7)) << 4); }

template <bool GATE_UP, bool BF16>
__global__ __launch_bounds__(256) void grouped_gemm_kernel(GemmParams p) {
    typedef typename Elem<BF16>::T T;
    constexpr int EPC = Elem<BF16>::kPerChunk;
    constexpr int SLICE = Elem<BF16>::kSlice;
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kTileBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int wm = wv >> 1;
    const int wn = wv & 1;

    // ---- which tile -------------------------------------------------------
    int64_t total;
    if (p.offsets == nullptr) {
        total = ((p.ident_rows + kBM - 1) / kBM) * p.n_tiles;
    } else {
        total = static_cast<int64_t>(p.tile_start[p.G]) * p.n_tiles;
    }
    const int64_t padded = (total + 7) & ~static_cast<int64_t>(7);
    if (static_cast<int64_t>(blockIdx.x) >= padded) return;
    const int64_t L = xcd_remap(blockIdx.x, padded);
    if (L >= total) return;

    int g = 0;
    int64_t m0;
    int rows;
    int n;
    if (p.offsets == nullptr) {
        const int64_t mt = (p.ident_rows + kBM - 1) / kBM;
        n = static_cast<int>(L / mt);
        const int64_t m = L % mt;
        m0 = m * kBM;
        const int64_t left = p.ident_rows - m0;
        rows = left < kBM ? static_cast<int>(left) : kBM;
    } else {
        int lo = 0, hi = p.G - 1;  // last g with tile_start[g] * n_tiles <= L
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (static_cast<int64_t>(p.tile_start[mid]) * p.n_tiles <= L) lo = mid; else hi = mid - 1;
        }
        g = lo;
        const int ts = p.tile_start[g];
        const int mtg = p.tile_start[g + 1] - ts;
        const int64_t local = L - static_cast<int64_t>(ts) * p.n_tiles;
        n = static_cast<int>(local / mtg);
        const int m = static_cast<int>(local % mtg);
        const int o0 = p.offsets[g];
        m0 = o0 + static_cast<int64_t>(m) * kBM;
        const int left = p.offsets[g + 1] - static_cast<int>(m0);
        rows = left < kBM ? left : kBM;
    }

    // ---- per-thread global source pointers (4 A rows, 4 B rows) ------------
    const T* __restrict__ asrc = static_cast<const T*>(p.a);
    const T* __restrict__ wsrc = static_cast<const T*>(p.w) + static_cast<int64_t>(g) * p.w_group_stride;
    const int ch = tid & 7;
    const T* aptr[4];
    const T* bptr[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int r = q * 32 + (tid >> 3);
        const int rr = r < rows ? r : rows - 1;  // rows past the group repeat its last row; never stored
        int64_t src = m0 + rr;
        if (GATE_UP && p.perm != nullptr) src = p.perm[src];
        aptr[q] = asrc + src * p.Kd + ch * EPC;
        int wrow;
        if (GATE_UP) wrow = r < 64 ? n * 64 + r : p.I + n * 64 + (r - 64);
        else wrow = n * kBN + r < p.ldo ? n * kBN + r : p.ldo - 1;  // D % 128 == 64: last tile half full
        bptr[q] = wsrc + static_cast<int64_t>(wrow) * p.Kd + ch * EPC;
    }

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    int brow[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
        if (GATE_UP) brow[nb] = (nb < 2 ? wn * 32 + nb * 16 : 64 + wn * 32 + (nb - 2) * 16) + (lane & 15);
        else brow[nb] = wn * 64 + nb * 16 + (lane & 15);
    }
    // LDS byte offsets this thread stores its four A and four B chunks to
    int sto[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) sto[q] = swz(q * 32 + (tid >> 3), ch);

    u32x4 ra[4], rb[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        ra[q] = *reinterpret_cast<const u32x4*>(aptr[q]);
        rb[q] = *reinterpret_cast<const u32x4*>(bptr[q]);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        *reinterpret_cast<u32x4*>(smem + sto[q]) = ra[q];
        *reinterpret_cast<u32x4*>(smem + kBM * kRowBytes + sto[q]) = rb[q];
    }
    __syncthreads();

    const int nk = p.Kd / SLICE;
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) {
            const int k1 = (kt + 1) * SLICE;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                ra[q] = *reinterpret_cast<const u32x4*>(aptr[q] + k1);
                rb[q] = *reinterpret_cast<const u32x4*>(bptr[q] + k1);
            }
        }
        const uint8_t* sa = smem + cur * kTileBytes;
        const uint8_t* sb = sa + kBM * kRowBytes;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int c = 4 * s + (lane >> 4);
            u32x4 af[4], bf[4];
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
                af[mb] = *reinterpret_cast<const u32x4*>(sa + swz(wm * 64 + mb * 16 + (lane & 15), c));
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) bf[nb] = *reinterpret_cast<const u32x4*>(sb + swz(brow[nb], c));
            if (BF16) {
#pragma unroll
                for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                    for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = mfma_bf16(af[mb], bf[nb], acc[mb][nb]);
            } else {
                // four K=4 steps; in step q every lane group supplies element q of its chunk
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                        for (int nb = 0; nb < 4; ++nb) {
                            const float av = __uint_as_float(af[mb][q]);
                            const float bv = __uint_as_float(bf[nb][q]);
                            acc[mb][nb] = mfma_f32(av, bv, acc[mb][nb]);
                        }
            }
        }
        if (more) {
            uint8_t* da = smem + (cur ^ 1) * kTileBytes;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                *reinterpret_cast<u32x4*>(da + sto[q]) = ra[q];
                *reinterpret_cast<u32x4*>(da + kBM * kRowBytes + sto[q]) = rb[q];
            }
        }
        __syncthreads();
    }

    // ---- epilogue ---------------------------------------------------------
    T* __restrict__ out = static_cast<T*>(p.out);
    if (GATE_UP) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                const int col = n * 64 + wn * 32 + nb * 16 + (lane & 15);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = wm * 64 + mb * 16 + 4 * (lane >> 4) + i;
                    if (row < rows) {
                        const float hg = acc[mb][nb][i];
                        const float hu = acc[mb][nb + 2][i];
                        const float a = (hg / (1.0f + expf(-hg))) * hu;
                        T* dst = out + (m0 + row) * p.ldo + col;
                        if (BF16) *reinterpret_cast<uint16_t*>(dst) = f32_to_bf16(a);
                        else *reinterpret_cast<float*>(dst) = a;
                    }
                }
            }
    } else {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                const int col = n * kBN + wn * 64 + nb * 16 + (lane & 15);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = wm * 64 + mb * 16 + 4 * (lane >> 4) + i;
                    if (row < rows && col < p.ldo) {
                        T* dst = out + (m0 + row) * p.ldo + col;
                        if (BF16) *reinterpret_cast<uint16_t*>(dst) = f32_to_bf16(acc[mb][nb][i]);
                        else *reinterpret_cast<float*>(dst) = acc[mb][nb][i];
                    }
                }
            }
    }
}

static size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

size_t experts_ws_bytes(int64_t rows_max, int G, int I, int dtype) {
    const size_t eb = dtype == 0 ? 2 : 4;
    return align256(sizeof(int32_t) * (G + 1)) + align256(static_cast<size_t>(rows_max) * I * eb);
}

hipError_t launch_experts(const void* x, const int32_t* perm_token, const int32_t* offsets, int G,
                          int64_t rows_max, int D, int I, int dtype, const void* gate_up, const void* down,
                          void* y, void* ws, hipStream_t stream) {
    int32_t* tile_start = static_cast<int32_t*>(ws);
    void* act = static_cast<uint8_t*>(ws) + align256(sizeof(int32_t) * (G + 1));
    if (offsets != nullptr) {
        build_tiles_kernel<<<1, 1024, 0, stream>>>(offsets, G, tile_start);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    // upper bound of m-tiles: every group adds at most one partial tile
    const int64_t mt_max = offsets != nullptr ? (rows_max + kBM - 1) / kBM + G : (rows_max + kBM - 1) / kBM;

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
    p1.n_tiles = I / 64;
    p1.out = act;
    p1.ldo = I;
    const int64_t nwg1 = ((mt_max * p1.n_tiles) + 7) & ~static_cast<int64_t>(7);

    GemmParams p2 = p1;
    p2.a = act;
    p2.perm = nullptr;
    p2.Kd = I;
    p2.w = down;
    p2.w_group_stride = static_cast<int64_t>(D) * I;
    p2.n_tiles = (D + kBN - 1) / kBN;
    p2.out = y;
    p2.ldo = D;
    const int64_t nwg2 = ((mt_max * p2.n_tiles) + 7) & ~static_cast<int64_t>(7);

    if (dtype == 0) {
        grouped_gemm_kernel<true, true><<<static_cast<unsigned>(nwg1), 256, 0, stream>>>(p1);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        grouped_gemm_kernel<false, true><<<static_cast<unsigned>(nwg2), 256, 0, stream>>>(p2);
    } else {
        grouped_gemm_kernel<true, false><<<static_cast<unsigned>(nwg1), 256, 0, stream>>>(p1);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        grouped_gemm_kernel<false, false><<<static_cast<unsigned>(nwg2), 256, 0, stream>>>(p2);
    }
    return hipGetLastError();
}

}  // namespace moe
