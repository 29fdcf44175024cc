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

// M0 is reserved to the compiler; the DMA asm below sets it on purpose
#pragma clang diagnostic ignored "-Winline-asm"

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

// silu(g) * u with the hardware exponential and reciprocal (about 2 ulp in
// float32); used where the activation is then rounded to bf16
__device__ __forceinline__ float silu_mul_fast(float g, float u) {
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// ===========================================================================
// bf16 operands: 256 x 256 tiles, direct-to-LDS slices, 5-stage pipeline
// ===========================================================================
constexpr int kBM2 = 256;
constexpr int kBN2 = 256;
constexpr int kSlice2 = 32;                         // k per slice
constexpr int kRow2 = kSlice2 * 2;                  // 64 bytes per tile row per slice
constexpr int kStage2 = (kBM2 + kBN2) * kRow2;      // 32 KiB: one A and one B slice
constexpr int kStages2 = 5;                         // 160 KiB of LDS
constexpr int kDmaPerSlice2 = 8;                    // DMA instructions per wave per slice

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

// 16 bytes per lane from global memory (base + 32-bit per-lane offset) into
// LDS at wave_base + 16 * lane: global_load_lds_dwordx4 with M0 holding the
// wave's LDS base.  It is issued from inline asm on purpose: the compiler's
// wait-count tracking of LDS DMA cannot tell the stages of this pipeline
// apart and would drain every DMA in flight before each fragment read.  The
// instruction has no destination register; completion is awaited with the
// explicit vmcnt waits of the pipeline, and no other code in these kernels
// uses M0.
__device__ __forceinline__ void dma16(const uint8_t* gbase, uint32_t voff, uint8_t* wave_base) {
    const uint32_t lds = __builtin_amdgcn_readfirstlane(
        static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)wave_base)));
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(lds), "v"(voff), "s"(gbase)
                 : "memory", "m0");
}

// s_waitcnt with vmcnt(n) and the other counters left alone
constexpr int vmcnt_imm(int n) { return 0x3F70 | (n & 15) | (((n >> 4) & 3) << 14); }
template <int N>
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(vmcnt_imm(N)); }

// Chunk swizzle of a 64-byte row (four 16-byte chunks): chunk ^ ((row / 2) % 4).
// The eight lanes of a ds_read_b128 group read rows r..r+7 at one logical
// chunk; the swizzle spreads them over all 32 banks.
__device__ __forceinline__ int swz64(int row, int chunk) { return row * kRow2 + ((chunk ^ ((row >> 1) & 3)) << 4); }

template <bool GATE_UP>
__global__ __launch_bounds__(256) void grouped_gemm_bf16_kernel(GemmParams p) {
    // one array per stage: with compile-time stage indices the compiler can
    // tell that a DMA in flight to one stage never aliases reads of another
    __shared__ __attribute__((aligned(1024))) uint8_t lds0[kStage2];
    __shared__ __attribute__((aligned(1024))) uint8_t lds1[kStage2];
    __shared__ __attribute__((aligned(1024))) uint8_t lds2[kStage2];
    __shared__ __attribute__((aligned(1024))) uint8_t lds3[kStage2];
    __shared__ __attribute__((aligned(1024))) uint8_t lds4[kStage2];
    auto stage = [&](int st) -> uint8_t* {
        return st == 0 ? lds0 : st == 1 ? lds1 : st == 2 ? lds2 : st == 3 ? lds3 : lds4;
    };

    TileCoord tc;
    if (!locate_tile<kBM2>(p, tc)) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int wm = wv >> 1;
    const int wn = wv & 1;

    // ---- per-lane sources of the 4 + 4 DMA instructions of this wave ------
    // Instruction i fills rows wv*64 + 16i .. +15 of the A (or B) slice; lane l
    // lands on row l / 4 of that group at physical chunk l % 4, so it fetches
    // the logical chunk (l % 4) ^ ((row / 2) % 4).  Byte offsets fit 32 bits:
    // x, the activations and one group's weights are each below 4 GiB
    // (checked by the launcher).
    const uint8_t* __restrict__ abase = static_cast<const uint8_t*>(p.a);
    const uint8_t* __restrict__ wbase =
        static_cast<const uint8_t*>(p.w) + static_cast<int64_t>(tc.g) * p.w_group_stride * 2;
    const int chunk = (lane & 3) ^ ((lane >> 3) & 3);
    uint32_t aoff[4], boff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = wv * 64 + 16 * i + (lane >> 2);
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
    const int a_dst = wv * 64 * kRow2;
    const int b_dst = kBM2 * kRow2 + wv * 64 * kRow2;

    // LDS byte offsets of this lane's MFMA fragments: block b adds b * 16 rows,
    // and the swizzle term depends only on the lane (row % 16 == lane % 16)
    const int xo = ((lane >> 4) ^ ((lane >> 1) & 3)) << 4;
    const int a_frag = (wm * 128 + (lane & 15)) * kRow2 + xo;
    const int b_frag = kBM2 * kRow2 + ((GATE_UP ? wn * 64 : wn * 128) + (lane & 15)) * kRow2 + xo;
    auto b_row_off = [&](int b) {
        if (GATE_UP) return (b < 4 ? b * 16 : 128 + (b - 4) * 16) * kRow2;
        return b * 16 * kRow2;
    };

    f32x4 acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // DMA instruction q (0..3: A rows, 4..7: B rows) of slice kt into stage
    // kt % 5.  Slices past the end re-fetch the last slice: every step then
    // issues the same eight instructions (uniform waits, no tail code), and
    // the stage they land in is never read for results again.
    const int nk = p.Kd / kSlice2;
    auto dma = [&](int kt, int st, int q) {
        uint8_t* sb = stage(st);
        const uint32_t kb = static_cast<uint32_t>(kt < nk ? kt : nk - 1) * kRow2;
        if (q < 4) dma16(abase, aoff[q] + kb, sb + a_dst + q * 16 * kRow2);
        else dma16(wbase, boff[q - 4] + kb, sb + b_dst + (q - 4) * 16 * kRow2);
    };
    // Fragment k of the slice in stage st, in the order the MFMAs consume
    // them: A block 0, B blocks 0..7, then A blocks 1..7.
    auto frag = [&](int st, int k) -> u32x4 {
        const uint8_t* base = stage(st);
        if (k == 0) return *reinterpret_cast<const u32x4*>(base + a_frag);
        if (k <= 8) return *reinterpret_cast<const u32x4*>(base + b_frag + b_row_off(k - 1));
        return *reinterpret_cast<const u32x4*>(base + a_frag + (k - 8) * 16 * kRow2);
    };

    // Pipeline.  Slice kt lives in stage kt % 5.  At the top of step kt the
    // fragments of slice kt are in registers (f) and the DMAs of slices
    // kt+1 .. kt+4 are in flight.  The step waits for slice kt+1 only (the 24
    // younger DMA instructions may stay outstanding), then a barrier makes it
    // visible and proves every wave has read slice kt, whose stage then
    // receives slice kt+5.  The 64 MFMAs of slice kt run with the 16 fragment
    // reads of slice kt+1 spread through them (one per 4 MFMAs) and the 8 DMA
    // instructions in their first half.
    auto step = [&](int kt, int st, const u32x4 (&f)[16], u32x4 (&g)[16]) {
        wait_vmem<(kStages2 - 2) * kDmaPerSlice2>();
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        const int gst = st + 1 == kStages2 ? 0 : st + 1;
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) {
            const u32x4 a = mb == 0 ? f[0] : f[8 + mb];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int nb = 4 * h; nb < 4 * h + 4; ++nb) acc[mb][nb] = mfma_bf16(a, f[1 + nb], acc[mb][nb]);
                // first half of the step: two fragment reads and one DMA per 4
                // MFMAs, so the reads have landed before the next barrier
                const int q = 2 * mb + h;
                if (q < 8) {
                    g[2 * q] = frag(gst, 2 * q);
                    g[2 * q + 1] = frag(gst, 2 * q + 1);
                    dma(kt + kStages2, st, q);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

#pragma unroll
    for (int j = 0; j < kStages2; ++j)
#pragma unroll
        for (int q = 0; q < kDmaPerSlice2; ++q) dma(j, j, q);
    wait_vmem<(kStages2 - 1) * kDmaPerSlice2>();
    __syncthreads();
    u32x4 f0[16], f1[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) f0[k] = frag(0, k);
    // Ten steps per trip, so that stage indices (kt % 5) and the register
    // sets (kt % 2) are compile-time constants; then the tail (nk is even).
    int kt = 0;
    for (; kt + 10 <= nk; kt += 10) {
#pragma unroll
        for (int j = 0; j < 10; j += 2) {
            step(kt + j, j % kStages2, f0, f1);
            step(kt + j + 1, (j + 1) % kStages2, f1, f0);
        }
    }
    for (; kt < nk; kt += 2) {
        step(kt, kt % kStages2, f0, f1);
        step(kt + 1, (kt + 1) % kStages2, f1, f0);
    }
    wait_vmem<0>();

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
                        out[(tc.m0 + row) * p.ldo + col] = f32_to_bf16(silu_mul_fast(acc[mb][nb][i], acc[mb][nb + 4][i]));
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
