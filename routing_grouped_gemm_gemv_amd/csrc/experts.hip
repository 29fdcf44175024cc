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
// 2 x 2, 128 x 128 per wave: 64 accumulator blocks of 16 x 16); the last
// <= 128 rows of a group form 128 x 512 tail tiles (4 waves as 1 x 4).  The
// k dimension advances in 64-element stages (128 bytes per row), two stages
// in LDS.  Stages are fetched with global_load_lds_dwordx4, which writes each
// lane's 16 bytes straight into LDS at (wave base + 16 * lane), 8 rows x 128
// bytes per instruction, so every 128-byte line of an operand row is fetched
// whole; the XOR swizzle of the 16-byte chunks of a row (chunk ^ row % 8,
// which keeps the MFMA fragment reads conflict-free) is applied to the global
// addresses each lane fetches.  The MFMAs step through each stage in two
// 32-wide halves with the fragments of the next half read ahead.  For
// gate_up the weight rows of a tile are gate rows and the matching up rows,
// so the SwiGLU epilogue pairs registers of the same wave.  The epilogue
// stages the bf16 tile in LDS and stores whole rows in 16-byte pieces; the
// first stage of the workgroup's next tile is fetched meanwhile, so a tile
// starts with its operands already on the way.
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
    const int32_t* tile_start; // fp32 kernel: [G+1] m-tile prefix sums (with offsets)
    const u32x4* tiles;        // bf16 kernel: tile descriptors in grouped order
    int32_t* ctl;              // bf16 kernel: tile count and work-queue counters of this GEMM
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


// two floats -> two bf16 (round to nearest even), low half first
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// ===========================================================================
// bf16 operands: direct-to-LDS stages of 64-wide k
// ===========================================================================
constexpr int kLds2 = 160 * 1024;



// Tiles of one group of c rows.  Full tiles are 256 rows x one n-tile.  When
// the number of n-tiles is even, the last c % 256 rows, if at most 128, form
// tail tiles of 128 rows x two n-tiles (the same work per wave as a full
// tile), which halves the rows a group pads on average.
struct GroupTiles {
    int full;   // 256-row m-tiles
    int tail;   // 1 if a 128-row tail exists
};
__host__ __device__ __forceinline__ GroupTiles group_tiles(int c, int n_tiles) {
    GroupTiles t;
    const int r = c & 255;
    if ((n_tiles & 1) == 0 && r > 0 && r <= 128) {
        t.full = c >> 8;
        t.tail = 1;
    } else {
        t.full = (c + 255) >> 8;
        t.tail = 0;
    }
    return t;
}
__host__ __device__ __forceinline__ int tiles_of(int c, int n_tiles) {
    const GroupTiles t = group_tiles(c, n_tiles);
    return t.tail ? (n_tiles >> 1) * (2 * t.full + 1) : n_tiles * t.full;
}

struct Tile2 {
    int g;
    int64_t m0;
    int rows;
    int n;      // first n-tile
    bool tail;  // 128 rows x two n-tiles
};

// Tile `local` of a group of c rows.  Order inside a group: for each pair of
// n-tiles, the full tiles of the first n-tile (m fastest), those of the
// second, then the pair's tail tile, so the tail reads weight slices its
// group's full tiles have just used.
__host__ __device__ __forceinline__ void decode_tile(int c, int n_tiles, int64_t local, int& n, int& m, bool& tail) {
    const GroupTiles gt = group_tiles(c, n_tiles);
    tail = false;
    if (gt.tail) {
        const int per_pair = 2 * gt.full + 1;
        const int j = static_cast<int>(local / per_pair);
        const int rem = static_cast<int>(local % per_pair);
        if (rem < 2 * gt.full) {
            n = 2 * j + rem / gt.full;
            m = rem % gt.full;
        } else {
            n = 2 * j;
            m = gt.full;
            tail = true;
        }
    } else {
        n = static_cast<int>(local / gt.full);
        m = static_cast<int>(local % gt.full);
    }
}

__device__ __forceinline__ u32x4 tile_desc(int g, int64_t m0, int rows, int n, bool tail) {
    return u32x4{static_cast<uint32_t>(g), static_cast<uint32_t>(m0), static_cast<uint32_t>(rows),
                 static_cast<uint32_t>(n) | (tail ? 0x10000u : 0u)};
}

// Control block of one GEMM launch: the tile count, then one work-queue
// counter per XCD, each on its own 128-byte line.
constexpr int kCtlInts = 8 * 32 + 32;
__host__ __device__ __forceinline__ int ctl_queue(int x) { return 32 + 32 * x; }

// Tile descriptors of both GEMMs (gate_up and down have different n-tiles) in
// grouped order, the tile counts, and zeroed queue counters.  offsets ==
// nullptr means one group of ident_rows rows.  Each block rebuilds the tile
// prefix sums of the groups in LDS and fills a strided share of both tables.
__global__ __launch_bounds__(1024) void build_tile_table_kernel(const int32_t* __restrict__ offsets, int G,
                                                                int ident_rows, int nt1, int nt2,
                                                                u32x4* __restrict__ desc1, int cap1,
                                                                u32x4* __restrict__ desc2, int cap2,
                                                                int32_t* __restrict__ ctl1, int32_t* __restrict__ ctl2) {
    __shared__ int part1[1024];
    __shared__ int part2[1024];
    __shared__ int off[1025];
    const int tid = threadIdx.x;
    int a = 0, b = 0;
    if (tid < G) {
        const int o0 = offsets ? offsets[tid] : 0;
        const int o1 = offsets ? offsets[tid + 1] : ident_rows;
        off[tid] = o0;
        if (tid == G - 1) off[G] = o1;
        const int c = o1 - o0;
        a = tiles_of(c, nt1);
        b = tiles_of(c, nt2);
    }
    part1[tid] = a;
    part2[tid] = b;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {
        const int v1 = tid >= d ? part1[tid - d] : 0;
        const int v2 = tid >= d ? part2[tid - d] : 0;
        __syncthreads();
        part1[tid] += v1;
        part2[tid] += v2;
        __syncthreads();
    }
    // exclusive starts: part[g] - tiles(g); total = part[G - 1]
    const int total1 = part1[G - 1], total2 = part2[G - 1];
    if (blockIdx.x == 0 && tid < kCtlInts) {
        ctl1[tid] = tid == 0 ? total1 : 0;
        ctl2[tid] = tid == 0 ? total2 : 0;
    }
    for (int t = 0; t < 2; ++t) {
        const int* part = t == 0 ? part1 : part2;
        const int nt = t == 0 ? nt1 : nt2;
        const int total = t == 0 ? total1 : total2;
        const int cap = t == 0 ? cap1 : cap2;
        u32x4* desc = t == 0 ? desc1 : desc2;
        for (int L = blockIdx.x * 1024 + tid; L < total && L < cap; L += gridDim.x * 1024) {
            // last g whose exclusive start is <= L (empty groups share a start)
            int lo = 0, hi = G - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                const int st = mid == 0 ? 0 : part[mid - 1];
                if (st <= L) lo = mid; else hi = mid - 1;
            }
            const int g = lo;
            const int st = g == 0 ? 0 : part[g - 1];
            const int c = off[g + 1] - off[g];
            int n, m;
            bool tail;
            decode_tile(c, nt, L - st, n, m, tail);
            const int left = c - m * 256;
            desc[L] = tile_desc(g, static_cast<int64_t>(off[g]) + static_cast<int64_t>(m) * 256,
                                left < 256 ? left : 256, n, tail);
        }
    }
}

// Descriptor of tile L.  L is uniform over the workgroup and the table is
// written by an earlier launch, so it comes through the scalar data cache
// (no vector-memory wait, which would also wait for the output stores of
// the tile before).
__device__ __forceinline__ Tile2 load_tile(const GemmParams& p, int L) {
    typedef const __attribute__((address_space(4))) u32x4 const_u32x4;
    const u32x4 d = ((const_u32x4*)p.tiles)[L];
    Tile2 t;
    t.g = static_cast<int>(d.x);
    t.m0 = static_cast<int64_t>(d.y);
    t.rows = static_cast<int>(d.z);
    t.n = static_cast<int>(d.w & 0xFFFFu);
    t.tail = (d.w >> 16) != 0;
    return t;
}

// Work queues.  The tiles in grouped order are cut into 8 contiguous ranges,
// one per XCD (workgroup b runs on XCD b % 8), so tiles that share operands
// run in one L2.  A workgroup takes the next tile of its own range with an
// atomic increment and, once that range is used up, of the others in turn.
// Which workgroup computes a tile never changes its result.
struct Queues {
    int total;
    int per;  // tiles per range
};
__device__ __forceinline__ int queue_tile(const Queues& qs, int q, int i) {
    const int L = q * qs.per + i;
    return (i < qs.per && L < qs.total) ? L : -1;
}
// Next tile for the calling wave starting at range q (updated), or -1.  Lane
// 0 performs the atomics; the result is uniform over the wave.
__device__ __forceinline__ int take_tile(int32_t* ctl, const Queues& qs, int& q) {
    for (int k = 0; k < 8; ++k) {
        int i = 0;
        if (lane_id() == 0) i = __hip_atomic_fetch_add(ctl + ctl_queue(q), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        i = __builtin_amdgcn_readfirstlane(i);
        const int L = queue_tile(qs, q, i);
        if (L >= 0) return L;
        q = (q + 1) & 7;
    }
    return -1;
}

// Lane index computed where it is used: the asm keeps the compiler from
// hoisting per-lane addresses out of the persistent loop and holding
// (spilling) them across the k loop.
__device__ __forceinline__ int fresh_lane() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

// Stages.  A tile is BM rows x BN weight rows (gate_up: BN/2 gate rows and
// the matching BN/2 up rows); stage st holds k = 64 st .. 64 st + 63 of all of
// them, 128 bytes a row.  Each DMA instruction moves 8 rows x 128 bytes: lane
// l lands on row l / 8 of its 8-row group at physical chunk l % 8 and fetches
// logical chunk (l % 8) ^ (row % 8).  Byte offsets fit 32 bits: x, the
// activations and one group's weights are each below 4 GiB (checked by the
// launcher).
template <int BM, int BN>
struct StageShape {
    static constexpr int kBytes = (BM + BN) * kRowBytes;
    static constexpr int kDmaA = BM / 32;  // 8-row DMA instructions per wave per stage
    static constexpr int kDma = BM / 32 + BN / 32;
};

// Gate_up: the byte offset of the x row (plus the lane's chunk) behind each
// of the lane's BM / 32 A rows, through the permutation when there is one;
// computed once per tile ahead of its first stage.  Rows past the group
// repeat its last row and are never stored.
template <int BM>
__device__ __forceinline__ void a_offsets(const GemmParams& p, const Tile2& tc, int lane, int wv, uint32_t (&aoff)[8]) {
    const int chunk = (lane & 7) ^ (lane >> 3);
    const uint32_t row_bytes = static_cast<uint32_t>(p.Kd) * 2;
    const int ra = wv * (BM / 4) + (lane >> 3);
    uint32_t row[BM / 32];
    if (p.perm != nullptr) {
#pragma unroll
        for (int i = 0; i < BM / 32; ++i) {
            const int r = ra + 8 * i;
            row[i] = static_cast<uint32_t>(p.perm[tc.m0 + (r < tc.rows ? r : tc.rows - 1)]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < BM / 32; ++i) {
            const int r = ra + 8 * i;
            row[i] = static_cast<uint32_t>(tc.m0 + (r < tc.rows ? r : tc.rows - 1));
        }
    }
#pragma unroll
    for (int i = 0; i < BM / 32; ++i) aoff[i] = row[i] * row_bytes + chunk * 16;
}

// DMA number dq of the calling wave for stage st of tile tc into the stage
// buffer at LDS byte stage_off; stages past the end fetch the last one again.
template <bool GATE_UP, int BM, int BN>
__device__ __forceinline__ void stage_dma(const GemmParams& p, const Tile2& tc, const uint32_t (&aoff)[8], int lane,
                                          int wv, uint32_t lds0, int st, uint32_t stage_off, int dq) {
    constexpr int kDmaA = StageShape<BM, BN>::kDmaA;
    const int chunk = (lane & 7) ^ (lane >> 3);
    const uint32_t row_bytes = static_cast<uint32_t>(p.Kd) * 2;
    const int ns = p.Kd / 64;
    const uint32_t kb = static_cast<uint32_t>(st < ns ? st : ns - 1) * kRowBytes;
    if (dq < kDmaA) {
        uint32_t off;
        if (GATE_UP) {
            off = aoff[dq];
        } else {
            const int r = wv * (BM / 4) + (lane >> 3) + 8 * dq;
            const int rr = r < tc.rows ? r : tc.rows - 1;
            off = static_cast<uint32_t>(tc.m0 + rr) * row_bytes + chunk * 16;
        }
        dma16(static_cast<const uint8_t*>(p.a), off + kb, lds0 + stage_off + (wv * (BM / 4) + 8 * dq) * kRowBytes);
    } else {
        const int r = wv * (BN / 4) + (lane >> 3) + 8 * (dq - kDmaA);
        int wrow;
        if (GATE_UP) {
            int c = tc.n * 128 + (r % (BN / 2));  // gate row; the matching up row is I + c
            if (c >= p.I) c = p.I - 1;           // I % 128 == 64: last tile half full
            wrow = r < BN / 2 ? c : p.I + c;
        } else {
            wrow = tc.n * 256 + r;
            if (wrow >= p.ldo) wrow = p.ldo - 1;
        }
        const uint8_t* wbase = static_cast<const uint8_t*>(p.w) + static_cast<int64_t>(tc.g) * p.w_group_stride * 2;
        dma16(wbase, static_cast<uint32_t>(wrow) * row_bytes + chunk * 16 + kb,
              lds0 + stage_off + (BM + wv * (BN / 4) + 8 * (dq - kDmaA)) * kRowBytes);
    }
}

// Every DMA of stage st (0 or 1) of tile tc, of either shape, into stage
// buffer st; for gate_up, first the tile's A row offsets (st == 0).
template <bool GATE_UP>
__device__ __forceinline__ void first_stage(const GemmParams& p, const Tile2& tc, uint32_t (&aoff)[8], int lane, int wv,
                                            uint32_t lds0, int st) {
    if (tc.tail) {
        using S = StageShape<128, 512>;
        if (GATE_UP && st == 0) a_offsets<128>(p, tc, lane, wv, aoff);
#pragma unroll
        for (int dq = 0; dq < S::kDma; ++dq)
            stage_dma<GATE_UP, 128, 512>(p, tc, aoff, lane, wv, lds0, st, st * S::kBytes, dq);
    } else {
        using S = StageShape<256, 256>;
        if (GATE_UP && st == 0) a_offsets<256>(p, tc, lane, wv, aoff);
#pragma unroll
        for (int dq = 0; dq < S::kDma; ++dq)
            stage_dma<GATE_UP, 256, 256>(p, tc, aoff, lane, wv, lds0, st, st * S::kBytes, dq);
    }
}

// LDS byte that carries the next tile's index from wave 0 to the others:
// past stage 0 of either tile shape and below every output staging area.
constexpr int kNextWord = StageShape<128, 512>::kBytes;
static_assert(StageShape<256, 256>::kBytes <= kNextWord, "LDS");

// Output stores of one tile per thread: gate_up 64 KB, down 128 KB, in
// 16-byte pieces over 256 threads.  Every one is issued (rows and columns
// outside the output are dropped by the buffer range check), so the number in
// flight behind a tile is this constant.
template <bool GATE_UP>
constexpr int kTileStores = GATE_UP ? 16 : 32;

// One tile: k loop, epilogue, and the start of the next tile.
//
// On entry stages 0 and 1 of tc are in flight (issued by the tile before, or
// before the first tile); after a tile (after_tile) that tile's output stores
// were issued between them.  The k loop steps through each stage in two
// 32-wide MFMA sub-steps with one wait + barrier per stage.
//
// Epilogue: the bf16 output is staged in LDS above kNextWord and stored in
// 16-byte pieces of whole rows (down: in two halves, one after the other).
// Meanwhile stage 0 of the next tile is fetched below kNextWord, and stage 1
// once every wave is done with the staging area.  Returns the next tile's
// index (uniform; -1 when none is left) with tn and naoff its descriptor and
// (gate_up) A row offsets.
template <bool GATE_UP, int BM, int BN>
__device__ __forceinline__ int tile_pipeline(const GemmParams& p, const Tile2& tc, const uint32_t (&aoff)[8],
                                             lds_u8* smem, int wv, bool after_tile, const Queues& qs, int& q,
                                             Tile2& tn, uint32_t (&naoff)[8]) {
    using S = StageShape<BM, BN>;
    constexpr int kWN = BM == 256 ? 2 : 4;
    constexpr int kRow = kRowBytes;
    constexpr int kStage = S::kBytes;
    constexpr int kDma = S::kDma;
    constexpr int kStores = kTileStores<GATE_UP>;
    static_assert(2 * kStage <= kLds2, "LDS");
    static_assert(kDma <= 32, "DMA issue slots");
    static_assert(kStores + kDma <= 63, "vmcnt");

    const int lane = fresh_lane();
    const int tid = wv * 64 + lane;
    const int wm = wv / kWN;
    const int wn = wv % kWN;
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(smem));

    // fragment of sub-step j (k 32j .. 32j+31 of the stage): logical chunk
    // 4j + lane/16 of row lane%16 (+ 16 per block), physical chunk ^ (lane % 8)
    const int xo0 = (((lane >> 4)) ^ (lane & 7)) << 4;
    const int xo1 = ((4 + (lane >> 4)) ^ (lane & 7)) << 4;
    const int a_frag = (wm * 128 + (lane & 15)) * kRow;
    const int b_frag = BM * kRow + ((GATE_UP ? wn * 64 : wn * 128) + (lane & 15)) * kRow;
    auto b_row_off = [&](int b) {
        if (GATE_UP) return (b < 4 ? b * 16 : BN / 2 + (b - 4) * 16) * kRow;
        return b * 16 * kRow;
    };

    f32x4 acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int ns = p.Kd / 64;  // stages of the k loop
    auto dma = [&](int st, uint32_t stage_off, int dq) {
        stage_dma<GATE_UP, BM, BN>(p, tc, aoff, lane, wv, lds0, st, stage_off, dq);
    };
    auto frag = [&](uint32_t stage_off, int xo, int k) -> u32x4 {
        const lds_u8* st = smem + stage_off;
        if (k == 0) return *reinterpret_cast<lds_u32x4*>(st + a_frag + xo);
        if (k <= 8) return *reinterpret_cast<lds_u32x4*>(st + b_frag + b_row_off(k - 1) + xo);
        return *reinterpret_cast<lds_u32x4*>(st + a_frag + (k - 8) * 16 * kRow + xo);
    };
    // one 32-wide sub-step: 64 MFMAs on f, the 16 fragment reads of the next
    // sub-step (stage rs, half xo) in the first half, and DO_DMA: this
    // stage's DMAs spread over the sub-step
    auto sub = [&](const u32x4 (&f)[16], u32x4 (&g)[16], uint32_t rs, int xo, bool do_dma, int dst, uint32_t ds) {
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) {
            const u32x4 a = mb == 0 ? f[0] : f[8 + mb];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int nb = 4 * h; nb < 4 * h + 4; ++nb) acc[mb][nb] = mfma_bf16(f[1 + nb], a, acc[mb][nb]);
                const int qq = 2 * mb + h;
                if (qq < 8) {
                    g[2 * qq] = frag(rs, xo, 2 * qq);
                    g[2 * qq + 1] = frag(rs, xo, 2 * qq + 1);
                }
                if (do_dma) {
                    constexpr int kPer = (kDma + 15) / 16;  // DMAs per 4 MFMAs
#pragma unroll
                    for (int u = 0; u < kPer; ++u)
                        if (qq * kPer + u < kDma) dma(dst, ds, qq * kPer + u);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    // stage 0 has landed once at most stage 1 (and, after a tile, its
    // stores) is still in flight
    if (after_tile) wait_vmem<kStores + kDma>();
    else wait_vmem<kDma>();
    __syncthreads();
    u32x4 f0[16], f1[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) f0[k] = frag(0, xo0, k);
    for (int st = 0; st < ns; ++st) {
        const uint32_t cur = static_cast<uint32_t>(st & 1) * kStage;
        const uint32_t nxt = static_cast<uint32_t>((st + 1) & 1) * kStage;
        // first half of the stage: fragments of its second half
        sub(f0, f1, cur, xo1, false, 0, 0);
        // stage st+1 has landed and every wave is done with stage st
        wait_vmem<0>();
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        // second half: fragments of the next stage's first half; stage st+2 into stage st's buffer
        sub(f1, f0, nxt, xo0, true, st + 2, cur);
    }
    wait_vmem<0>();
    __syncthreads();


    // Output pieces of PR rows x PC columns: gate_up one piece, down two
    // (the row halves of a 256-row tile, the column halves of a tail tile).
    constexpr int NC = GATE_UP ? BN / 2 : BN;
    constexpr int kPieces = GATE_UP ? 1 : 2;
    constexpr int PR = GATE_UP ? BM : 128;
    constexpr int PC = GATE_UP ? NC : 256;
    constexpr bool kSplitRows = !GATE_UP && BM == 256;
    constexpr int kOutRow = PC * 2 + 16;
    constexpr int kStg = kLds2 - PR * kOutRow;
    static_assert(kStg >= kNextWord + 16, "LDS");
    static_assert(kPieces * PR * PC * 2 == kStores * 256 * 16, "stores per thread");
    const int my_piece = GATE_UP ? 0 : (kSplitRows ? wm : (wn >> 1));
    const int lrow0 = (kSplitRows ? 0 : wm * 128) + (lane & 15);
    const int lcol0 = (GATE_UP ? wn * 64 : (kSplitRows ? wn : (wn & 1)) * 128) + 4 * (lane >> 4);
    auto stage_out = [&]() {
        if (GATE_UP) {
#pragma unroll
            for (int mb = 0; mb < 8; ++mb)
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) {
                    const uint32_t w0 = pack_bf16(silu_mul_fast(acc[mb][nb][0], acc[mb][nb + 4][0]),
                                                  silu_mul_fast(acc[mb][nb][1], acc[mb][nb + 4][1]));
                    const uint32_t w1 = pack_bf16(silu_mul_fast(acc[mb][nb][2], acc[mb][nb + 4][2]),
                                                  silu_mul_fast(acc[mb][nb][3], acc[mb][nb + 4][3]));
                    const int off = kStg + (lrow0 + mb * 16) * kOutRow + (lcol0 + nb * 16) * 2;
                    *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(smem + off) = u32x2{w0, w1};
                }
        } else {
#pragma unroll
            for (int mb = 0; mb < 8; ++mb)
#pragma unroll
                for (int nb = 0; nb < 8; ++nb) {
                    const uint32_t w0 = pack_bf16(acc[mb][nb][0], acc[mb][nb][1]);
                    const uint32_t w1 = pack_bf16(acc[mb][nb][2], acc[mb][nb][3]);
                    const int off = kStg + (lrow0 + mb * 16) * kOutRow + (lcol0 + nb * 16) * 2;
                    *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(smem + off) = u32x2{w0, w1};
                }
        }
    };
    // the tile's rows through a buffer resource: rows at or past tc.rows fall
    // outside its range, columns past the output are sent outside it
    constexpr int kChunks = PC / 8;
    constexpr int kRowsPerPass = 256 / kChunks;
    const int col_lim = GATE_UP ? p.I : p.ldo;
    const int ch = tid % kChunks;
    const int r0 = tid / kChunks;
    uint8_t* obase = static_cast<uint8_t*>(p.out) + tc.m0 * p.ldo * 2;
    const __amdgpu_buffer_rsrc_t orsrc =
        __builtin_amdgcn_make_buffer_rsrc(obase, static_cast<short>(0), tc.rows * p.ldo * 2, 0x00020000);
    auto store_piece = [&](int h) {
        const int col = (GATE_UP ? tc.n * 128 : tc.n * 256) + (GATE_UP || kSplitRows ? 0 : 256 * h) + ch * 8;
        const int rb = kSplitRows ? 128 * h : 0;
#pragma unroll
        for (int i = 0; i < PR / kRowsPerPass; ++i) {
            const int r = r0 + i * kRowsPerPass;
            const u32x4 v = *reinterpret_cast<lds_u32x4*>(smem + kStg + r * kOutRow + ch * 16);
            const uint32_t off = col < col_lim ? static_cast<uint32_t>((rb + r) * p.ldo + col) * 2u : 0x80000000u;
            __builtin_amdgcn_raw_buffer_store_b128(v, orsrc, off, 0, 0);
        }
    };

    // the next tile: wave 0 claims the next one of its queue range while
    // its output is staged (or, with that range used up, takes one from the
    // others) and leaves the index in LDS for the other waves
    int ticket = 0;
    if (wv == 0 && lane == 0)
        ticket = __hip_atomic_fetch_add(p.ctl + ctl_queue(q), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (my_piece == 0) stage_out();
    if (wv == 0) {
        int nx = queue_tile(qs, q, __builtin_amdgcn_readfirstlane(ticket));
        if (nx < 0) {
            q = (q + 1) & 7;
            nx = take_tile(p.ctl, qs, q);
        }
        if (lane == 0) *reinterpret_cast<__attribute__((address_space(3))) int*>(smem + kNextWord) = nx;
    }
    __syncthreads();
    const int next = __builtin_amdgcn_readfirstlane(*reinterpret_cast<__attribute__((address_space(3))) int*>(smem + kNextWord));
    if (next >= 0) {
        tn = load_tile(p, next);
        first_stage<GATE_UP>(p, tn, naoff, lane, wv, lds0, 0);
    }
    store_piece(0);
    if (kPieces == 2) {
        __syncthreads();
        if (my_piece == 1) stage_out();
        __syncthreads();
        store_piece(1);
    }
    // every wave is done with the staging area (and with the next index)
    __syncthreads();
    if (next >= 0) first_stage<GATE_UP>(p, tn, naoff, lane, wv, lds0, 1);
    return next;
}

// Value of wave 0 to every wave of the workgroup (through LDS word 0, before
// any stage is fetched).
__device__ __forceinline__ int broadcast_from_wave0(lds_u8* smem, int v) {
    __syncthreads();
    if (threadIdx.x == 0) *reinterpret_cast<__attribute__((address_space(3))) int*>(smem) = v;
    __syncthreads();
    const int r = *reinterpret_cast<__attribute__((address_space(3))) int*>(smem);
    __syncthreads();
    return r;
}

// Persistent: one workgroup per CU takes tiles from the work queues until
// none are left; each tile claims the next one while it runs and starts
// fetching it while its own output is stored.
template <bool GATE_UP>
__global__ __launch_bounds__(256) void grouped_gemm_bf16_kernel(GemmParams p) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kLds2];
    lds_u8* lds = (lds_u8*)(smem);  // the array lives in LDS: an address-space cast
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    Queues qs;
    qs.total = p.ctl[0];
    qs.per = (qs.total + 7) >> 3;
    int q = blockIdx.x & 7;
    int L = -1;
    if (wv == 0) L = take_tile(p.ctl, qs, q);
    L = __builtin_amdgcn_readfirstlane(broadcast_from_wave0(lds, L));
    if (L < 0) return;
    Tile2 tc = load_tile(p, L);
    uint32_t aoff[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
    {
        const int lane = fresh_lane();
        const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
        first_stage<GATE_UP>(p, tc, aoff, lane, wv, lds0, 0);
        first_stage<GATE_UP>(p, tc, aoff, lane, wv, lds0, 1);
    }
    bool after_tile = false;
    for (;;) {
        Tile2 tn;
        uint32_t naoff[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
        int next;
        if (tc.tail) next = tile_pipeline<GATE_UP, 128, 512>(p, tc, aoff, lds, wv, after_tile, qs, q, tn, naoff);
        else next = tile_pipeline<GATE_UP, 256, 256>(p, tc, aoff, lds, wv, after_tile, qs, q, tn, naoff);
        if (next < 0) break;
        tc = tn;
#pragma unroll
        for (int i = 0; i < 8; ++i) aoff[i] = naoff[i];
        after_tile = true;
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

// Workgroups of the bf16 GEMMs: an upper bound of their tiles (every group
// adds at most one partial m-tile; a tail tile stands in for one), rounded up
// to a multiple of 8 for the XCD mapping.
static void bf16_grid(int64_t rows_max, int G, bool grouped, int D, int I, int64_t& nwg1, int64_t& nwg2) {
    const int64_t mt_max = (rows_max + 255) / 256 + (grouped ? G : 0);
    nwg1 = ((mt_max * ((I + 127) / 128)) + 7) & ~static_cast<int64_t>(7);
    nwg2 = ((mt_max * ((D + 255) / 256)) + 7) & ~static_cast<int64_t>(7);
}

constexpr size_t kCtlBytes = 2 * kCtlInts * sizeof(int32_t);

// CUs of the current device (queried once per device)
int compute_units() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

size_t experts_ws_bytes(int64_t rows_max, int G, int D, int I, int dtype) {
    const size_t eb = dtype == 0 ? 2 : 4;
    size_t tables = align256(2 * sizeof(int32_t) * (G + 1));
    if (dtype == 0) {
        int64_t nwg1, nwg2;
        bf16_grid(rows_max, G, true, D, I, nwg1, nwg2);
        tables = align256(kCtlBytes + static_cast<size_t>(nwg1 + nwg2) * sizeof(u32x4));
    }
    return tables + align256(static_cast<size_t>(rows_max) * I * eb);
}

hipError_t launch_experts(const void* x, int64_t x_rows, const int32_t* perm_token, const int32_t* offsets, int G,
                          int64_t rows_max, int D, int I, int dtype, const void* gate_up, const void* down,
                          void* y, void* ws, hipStream_t stream) {
    const bool bf16 = dtype == 0;
    const size_t ws_total = experts_ws_bytes(rows_max, G, D, I, dtype);
    void* act = static_cast<uint8_t*>(ws) + (ws_total - align256(static_cast<size_t>(rows_max) * I * (bf16 ? 2 : 4)));

    GemmParams p1{};
    p1.a = x;
    p1.perm = perm_token;
    p1.offsets = offsets;
    p1.ident_rows = rows_max;
    p1.G = G;
    p1.Kd = D;
    p1.w = gate_up;
    p1.w_group_stride = static_cast<int64_t>(2) * I * D;
    p1.I = I;
    p1.out = act;
    p1.ldo = I;
    GemmParams p2 = p1;
    p2.a = act;
    p2.perm = nullptr;
    p2.Kd = I;
    p2.w = down;
    p2.w_group_stride = static_cast<int64_t>(D) * I;
    p2.out = y;
    p2.ldo = D;

    hipError_t err;
    if (bf16) {
        // the bf16 kernel addresses x, the activations and one group's weights
        // with 32-bit byte offsets
        const int64_t lim = static_cast<int64_t>(1) << 32;
        if (static_cast<int64_t>(2) * I * D * 2 >= lim || rows_max * I * 2 >= lim || x_rows * D * 2 >= lim)
            return hipErrorInvalidValue;
        p1.n_tiles = (I + 127) / 128;
        p2.n_tiles = (D + 255) / 256;
        int64_t nwg1, nwg2;
        bf16_grid(rows_max, G, offsets != nullptr, D, I, nwg1, nwg2);
        int32_t* ctl1 = static_cast<int32_t*>(ws);
        int32_t* ctl2 = ctl1 + kCtlInts;
        u32x4* d1 = reinterpret_cast<u32x4*>(static_cast<uint8_t*>(ws) + kCtlBytes);
        u32x4* d2 = d1 + nwg1;
        const int64_t most = nwg1 > nwg2 ? nwg1 : nwg2;
        const unsigned blocks = static_cast<unsigned>((most + 2047) / 2048);
        build_tile_table_kernel<<<blocks, 1024, 0, stream>>>(offsets, offsets ? G : 1, static_cast<int>(rows_max),
                                                            p1.n_tiles, p2.n_tiles, d1, static_cast<int>(nwg1), d2,
                                                            static_cast<int>(nwg2), ctl1, ctl2);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        p1.tiles = d1;
        p2.tiles = d2;
        p1.ctl = ctl1;
        p2.ctl = ctl2;
        // one workgroup per CU (each holds all of a CU's LDS), a multiple of 8
        const int slots = (compute_units() + 7) & ~7;
        const unsigned g1 = static_cast<unsigned>(nwg1 < slots ? nwg1 : slots);
        const unsigned g2 = static_cast<unsigned>(nwg2 < slots ? nwg2 : slots);
        grouped_gemm_bf16_kernel<true><<<g1, 256, 0, stream>>>(p1);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        grouped_gemm_bf16_kernel<false><<<g2, 256, 0, stream>>>(p2);
        return hipGetLastError();
    }
    int32_t* ts1 = static_cast<int32_t*>(ws);
    p1.n_tiles = (I + 63) / 64;
    p2.n_tiles = (D + kBN1 - 1) / kBN1;
    if (offsets != nullptr) {
        build_tiles_kernel<<<1, 1024, 0, stream>>>(offsets, G, kBM1, ts1);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        p1.tile_start = ts1;
        p2.tile_start = ts1;
    }
    const int64_t mt_max = (rows_max + kBM1 - 1) / kBM1 + (offsets != nullptr ? G : 0);
    const int64_t nwg1 = ((mt_max * p1.n_tiles) + 7) & ~static_cast<int64_t>(7);
    const int64_t nwg2 = ((mt_max * p2.n_tiles) + 7) & ~static_cast<int64_t>(7);
    grouped_gemm_f32_kernel<true><<<static_cast<unsigned>(nwg1), 256, 0, stream>>>(p1);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    grouped_gemm_f32_kernel<false><<<static_cast<unsigned>(nwg2), 256, 0, stream>>>(p2);
    return hipGetLastError();
}

}  // namespace moe
