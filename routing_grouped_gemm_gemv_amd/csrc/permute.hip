// Dispatch: per-expert counts, offsets and a stable token permutation.
//
// The dispatch boundary of the RL-Kernel roadmap ("DSV4 Flash MoE
// Train-Inference Consistency Roadmap", Problem 2: the token-to-expert map,
// valid token counts and padding provenance) as a stable counting sort of the
// T*K (token, slot) pairs by expert id.  No atomics, global or LDS: every
// count is produced by exactly one lane, so the result is the same on every
// run.
//
//   pass 1 (count):   each block takes a contiguous range of pairs; each wave
//                     walks 64-pair segments of its sub-range and, with a
//                     ballot per id bit, finds for every lane the lanes holding
//                     the same expert (a "match mask").  The lowest such lane
//                     adds the popcount to the wave's LDS histogram row.
//   pass 2 (scan):    over more than kScanInScatter blocks, one workgroup per
//                     expert scans that expert's block counts: the expert's
//                     count and, per block, the pairs of the expert in
//                     earlier blocks.  Up to kScanInScatter blocks, each
//                     block of pass 3 sums the few counts it needs itself.
//   pass 3 (scatter): each block scans the expert counts (the offsets; block
//                     0 stores them), recomputes its wave histograms, turns
//                     them into per-wave bases, and walks its segments again;
//                     a pair's row is its wave base plus the pairs of the same
//                     expert in earlier segments plus its rank in the segment.
//
// Pairs of one expert therefore keep their flat (token, slot) order, and since
// a token lists distinct experts, tokens ascend within every expert.
#include "common.hpp"
#include "kernels.hpp"
#include "permute_block.hpp"

namespace moe {


PermutePlan permute_plan(int64_t P, int E) {
    PermutePlan pl;
    int64_t ppb = 2048;
    // keep the scan's (expert, block) table small
    while ((P + ppb - 1) / ppb > 1024) ppb *= 2;
    pl.pairs_per_block = static_cast<int>(ppb);
    pl.blocks = static_cast<int>(P > 0 ? (P + ppb - 1) / ppb : 1);
    int bits = 0;
    while ((1 << bits) < E) ++bits;
    pl.id_bits = bits;
    return pl;
}

static_assert(kPermWaves == 4, "the count pass stores a block's wave counts as one int4 per expert");

// Workspace of the multi-block path, in int32: block histogram [E][blocks]
// (an expert's counts contiguous, for the scan), block bases [E][blocks], then
// (from a 16-byte boundary) the wave histograms [blocks][E][kPermWaves] (a
// block's counts contiguous, for its scatter pass).
static int64_t wave_hist_at(int64_t eb) { return (2 * eb + 3) & ~static_cast<int64_t>(3); }

size_t permute_ws_bytes(int64_t P, int E) {
    const PermutePlan pl = permute_plan(P, E);
    const int64_t eb = static_cast<int64_t>(E) * pl.blocks;
    return sizeof(int32_t) * static_cast<size_t>(wave_hist_at(eb) + kPermWaves * eb);
}

// Up to this many blocks the scatter pass sums the block counts itself (one
// launch fewer); above it, the per-expert loop of loads costs more than the
// separate scan launch.
constexpr int kScanInScatter = 64;



__global__ __launch_bounds__(256) void permute_count_kernel(
    const int32_t* __restrict__ ids, int64_t P, int E, int ppb, int nblocks, int id_bits,
    int32_t* __restrict__ block_hist, int32_t* __restrict__ wave_hist) {
    __shared__ int hist[kPermWaves][kMaxExperts];
    const int tid = threadIdx.x;
    const int wv = tid >> 6;
    for (int i = tid; i < kPermWaves * E; i += 256) hist[i / E][i % E] = 0;
    __syncthreads();
    const int64_t base = static_cast<int64_t>(blockIdx.x) * ppb;
    const int per_wave = ppb / kPermWaves;
    wave_histogram(ids, P, E, base + wv * per_wave, base + (wv + 1) * per_wave, id_bits, hist[wv]);
    __syncthreads();
    for (int e = tid; e < E; e += 256) {
        block_hist[static_cast<int64_t>(e) * nblocks + blockIdx.x] = hist[0][e] + hist[1][e] + hist[2][e] + hist[3][e];
        reinterpret_cast<int4*>(wave_hist)[static_cast<int64_t>(blockIdx.x) * E + e] =
            int4{hist[0][e], hist[1][e], hist[2][e], hist[3][e]};
    }
}

// Exclusive scan of one expert's block counts (workgroup e scans row e of
// block_hist, at most 1024 blocks); counts[e] is the row total.
__global__ __launch_bounds__(256) void permute_scan_kernel(
    const int32_t* __restrict__ block_hist, int nblocks, int32_t* __restrict__ block_base,
    int32_t* __restrict__ counts) {
    __shared__ int part[256];
    const int tid = threadIdx.x;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * nblocks;
    int v[4];
    int sum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int b = 4 * tid + j;
        v[j] = b < nblocks ? block_hist[row + b] : 0;
        sum += v[j];
    }
    part[tid] = sum;
    __syncthreads();
    for (int d = 1; d < 256; d <<= 1) {
        const int u = tid >= d ? part[tid - d] : 0;
        __syncthreads();
        part[tid] += u;
        __syncthreads();
    }
    int run = part[tid] - sum;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int b = 4 * tid + j;
        if (b < nblocks) block_base[row + b] = run;
        run += v[j];
    }
    if (tid == 255) counts[blockIdx.x] = part[255];
}

// Exclusive scan of the E expert counts (in LDS) into offs[0..E] (256 threads).
__device__ __forceinline__ void scan_counts(const int* counts, int E, int* offs, int* part) {
    const int tid = threadIdx.x;
    int v[4];
    int sum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = 4 * tid + j;
        v[j] = e < E ? counts[e] : 0;
        sum += v[j];
    }
    part[tid] = sum;
    __syncthreads();
    for (int d = 1; d < 256; d <<= 1) {
        const int u = tid >= d ? part[tid - d] : 0;
        __syncthreads();
        part[tid] += u;
        __syncthreads();
    }
    int run = part[tid] - sum;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = 4 * tid + j;
        if (e < E) offs[e] = run;
        run += v[j];
    }
    if (tid == 255) offs[E] = part[255];
    __syncthreads();
}

// block_base == nullptr: the block sums its counts from block_hist (and
// block 0 stores the expert counts); else block_base and counts come from
// permute_scan_kernel.  The per-wave counts of the block come from the count
// pass (wave_hist), so the ids are walked once here.
__global__ __launch_bounds__(256) void permute_scatter_kernel(
    const int32_t* __restrict__ ids, int64_t P, int K, int E, int ppb, int nblocks, int id_bits,
    const int32_t* __restrict__ block_hist, const int32_t* __restrict__ block_base,
    const int32_t* __restrict__ wave_hist, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm_token, int32_t* __restrict__ inv_pos) {
    __shared__ int hist[kPermWaves][kMaxExperts];
    __shared__ int offs[kMaxExperts + 1];
    __shared__ int cnt[kMaxExperts];    // pairs of each expert
    __shared__ int before[kMaxExperts]; // pairs of each expert in earlier blocks
    __shared__ int part[256];
    const int tid = threadIdx.x;
    const int wv = tid >> 6;
    for (int e = tid; e < E; e += 256) {
        const int4 h = reinterpret_cast<const int4*>(wave_hist)[static_cast<int64_t>(blockIdx.x) * E + e];
        hist[0][e] = h.x;
        hist[1][e] = h.y;
        hist[2][e] = h.z;
        hist[3][e] = h.w;
    }
    if (block_base == nullptr) {
        // row e of block_hist: expert e's pairs per block, in block order
        for (int e = tid; e < E; e += 256) {
            const int32_t* row = block_hist + static_cast<int64_t>(e) * nblocks;
            int pre = 0, tot = 0;
#pragma unroll 8
            for (int b = 0; b < nblocks; ++b) {
                const int v = row[b];
                pre += b < static_cast<int>(blockIdx.x) ? v : 0;
                tot += v;
            }
            cnt[e] = tot;
            before[e] = pre;
            if (blockIdx.x == 0) counts[e] = tot;
        }
    } else {
        for (int e = tid; e < E; e += 256) {
            cnt[e] = counts[e];
            before[e] = block_base[static_cast<int64_t>(e) * nblocks + blockIdx.x];
        }
    }
    __syncthreads();
    scan_counts(cnt, E, offs, part);
    if (blockIdx.x == 0)
        for (int e = tid; e <= E; e += 256) offsets[e] = offs[e];
    const int64_t base = static_cast<int64_t>(blockIdx.x) * ppb;
    const int per_wave = ppb / kPermWaves;
    const int64_t w_begin = base + wv * per_wave;
    const int64_t w_end = w_begin + per_wave;
    // per-wave base rows: block base of the expert plus earlier waves' pairs
    for (int e = tid; e < E; e += 256) {
        int run = offs[e] + before[e];
#pragma unroll
        for (int w = 0; w < kPermWaves; ++w) {
            const int h = hist[w][e];
            hist[w][e] = run;
            run += h;
        }
    }
    __syncthreads();
    wave_scatter(ids, P, K, E, w_begin, w_end, id_bits, hist[wv], perm_token, inv_pos);
}

// All three passes in one workgroup when every pair fits one block (the
// block's base rows are zero), for decode-sized batches: one launch instead
// of three, the same rows.  Up to 256 pairs the ids go to LDS once and
// permute_small places them.
__global__ __launch_bounds__(256) void permute_single_kernel(
    const int32_t* __restrict__ ids, int64_t P, int K, int E, int ppb, int id_bits, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm_token, int32_t* __restrict__ inv_pos) {
    if (P <= kSmallPairs) {  // uniform
        __shared__ int pairs[kSmallPairs];
        if (threadIdx.x < P) pairs[threadIdx.x] = ids[threadIdx.x];
        __syncthreads();
        permute_small(pairs, static_cast<int>(P), K, E, counts, offsets, perm_token, inv_pos);
        return;
    }
    permute_one_block(ids, P, K, E, ppb, id_bits, counts, offsets, perm_token, inv_pos);
}

hipError_t launch_permute(const int32_t* ids, int64_t T, int K, int E, int32_t* ws_i32,
                          int32_t* counts, int32_t* offsets, int32_t* perm_token, int32_t* inv_pos,
                          hipStream_t stream) {
    const int64_t P = T * K;
    const PermutePlan pl = permute_plan(P, E);
    if (pl.blocks == 1) {
        permute_single_kernel<<<1, 256, 0, stream>>>(ids, P, K, E, pl.pairs_per_block, pl.id_bits, counts, offsets,
                                                     perm_token, inv_pos);
        return hipGetLastError();
    }
    const int64_t eb = static_cast<int64_t>(E) * pl.blocks;
    int32_t* block_hist = ws_i32;
    int32_t* block_base = nullptr;
    int32_t* wave_hist = ws_i32 + wave_hist_at(eb);  // 16-byte aligned, as the workspace is
    permute_count_kernel<<<pl.blocks, 256, 0, stream>>>(ids, P, E, pl.pairs_per_block, pl.blocks, pl.id_bits,
                                                       block_hist, wave_hist);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (pl.blocks > kScanInScatter) {
        block_base = ws_i32 + eb;
        permute_scan_kernel<<<E, 256, 0, stream>>>(block_hist, pl.blocks, block_base, counts);
        err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    permute_scatter_kernel<<<pl.blocks, 256, 0, stream>>>(ids, P, K, E, pl.pairs_per_block, pl.blocks,
                                                         pl.id_bits, block_hist, block_base, wave_hist, counts,
                                                         offsets, perm_token, inv_pos);
    return hipGetLastError();
}

}  // namespace moe
