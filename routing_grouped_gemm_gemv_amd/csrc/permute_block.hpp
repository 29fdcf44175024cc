// Device side of the dispatch permutation shared by the permute kernels and
// the decode-sized fused top-k + permute kernel: a stable counting sort of
// the (token, slot) pairs by expert id, with no atomics (every count comes
// from exactly one lane), so every run gives the same rows.
#pragma once
#include "common.hpp"

namespace moe {

constexpr int kPermWaves = 4;
constexpr int kMaxExperts = 1024;

// lanes of this wave whose id equals mine (valid lanes only)
__device__ __forceinline__ uint64_t match_mask(int e, bool valid, int id_bits) {
    uint64_t m = __ballot(valid);
    for (int b = 0; b < id_bits; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t bm = __ballot(bit);
        m &= bit ? bm : ~bm;
    }
    return m;
}

// A wave walks its sub-range in 64-pair segments, kSegBatch of them per
// round of loads: the ids of a round are loaded at once (clamped, in-bounds,
// unconditional loads, so all of them are in flight together) and then the
// segments are taken one after another as before.  Sub-ranges are multiples
// of 64 * kSegBatch pairs.
constexpr int kSegBatch = 8;

__device__ __forceinline__ void load_segments(const int32_t* __restrict__ ids, int64_t P, int64_t seg0,
                                              int (&ev)[kSegBatch]) {
    const int lane = lane_id();
#pragma unroll
    for (int s = 0; s < kSegBatch; ++s) {
        const int64_t p = seg0 + 64 * s + lane;
        ev[s] = ids[p < P ? p : P - 1];  // pairs past P are never used
    }
}

// Fill hist[w][*] with the per-expert pair counts of wave w's sub-range.  An
// id outside [0, E) (the -1 of a masked slot, or a caller's out-of-range id)
// marks a slot without a row.
__device__ __forceinline__ void wave_histogram(const int32_t* __restrict__ ids, int64_t P, int E, int64_t w_begin,
                                               int64_t w_end, int id_bits, int* hist_row) {
    const int lane = lane_id();
    const uint64_t lt = (1ull << lane) - 1ull;
    for (int64_t seg0 = w_begin; seg0 < w_end; seg0 += 64 * kSegBatch) {
        int ev[kSegBatch];
        load_segments(ids, P, seg0, ev);
#pragma unroll
        for (int s = 0; s < kSegBatch; ++s) {
            const int64_t p = seg0 + 64 * s + lane;
            const int e = (p < w_end && p < P) ? ev[s] : -1;
            const bool valid = e >= 0 && e < E;
            const uint64_t m = match_mask(valid ? e : 0, valid, id_bits);
            if (valid && (m & lt) == 0ull) hist_row[e] += __popcll(m);
        }
    }
}

// The scatter of wave w's sub-range: row[e] holds the next row of expert e
// for this wave.
__device__ __forceinline__ void wave_scatter(const int32_t* __restrict__ ids, int64_t P, int K, int E, int64_t w_begin,
                                             int64_t w_end, int id_bits, int* row, int32_t* __restrict__ perm_token,
                                             int32_t* __restrict__ inv_pos) {
    const int lane = lane_id();
    const uint64_t lt = (1ull << lane) - 1ull;
    for (int64_t seg0 = w_begin; seg0 < w_end; seg0 += 64 * kSegBatch) {
        int ev[kSegBatch];
        load_segments(ids, P, seg0, ev);
#pragma unroll
        for (int s = 0; s < kSegBatch; ++s) {
            const int64_t p = seg0 + 64 * s + lane;
            const bool in = p < w_end && p < P;
            const int e = in ? ev[s] : -1;
            const bool valid = e >= 0 && e < E;
            const uint64_t m = match_mask(valid ? e : 0, valid, id_bits);
            if (valid) {
                const int pos = row[e] + __popcll(m & lt);
                perm_token[pos] = static_cast<int32_t>(p / K);
                inv_pos[p] = pos;
            } else if (in) {
                inv_pos[p] = -1;
            }
            __builtin_amdgcn_wave_barrier();
            if (valid && (m & lt) == 0ull) row[e] += __popcll(m);
            __builtin_amdgcn_wave_barrier();
        }
    }
}

// Counts, offsets and the permutation of all P pairs in one workgroup of
// 256 threads (P at most ppb: every pair in one block, whose base rows are
// zero): the three passes of the multi-block path one after another.
__device__ __forceinline__ void permute_one_block(const int32_t* __restrict__ ids, int64_t P, int K, int E, int ppb,
                                                  int id_bits, int32_t* __restrict__ counts,
                                                  int32_t* __restrict__ offsets, int32_t* __restrict__ perm_token,
                                                  int32_t* __restrict__ inv_pos) {
    __shared__ int hist[kPermWaves][kMaxExperts];
    __shared__ int offs[kMaxExperts + 1];
    __shared__ int part[256];
    const int tid = threadIdx.x;
    const int wv = tid >> 6;
    for (int i = tid; i < kPermWaves * E; i += 256) hist[i / E][i % E] = 0;
    __syncthreads();
    const int per_wave = ppb / kPermWaves;
    const int64_t w_begin = static_cast<int64_t>(wv) * per_wave;
    const int64_t w_end = w_begin + per_wave;
    wave_histogram(ids, P, E, w_begin, w_end, id_bits, hist[wv]);
    __syncthreads();
    // counts, then their exclusive scan into offs[0..E]
    int v[4];
    int sum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = 4 * tid + j;
        v[j] = e < E ? hist[0][e] + hist[1][e] + hist[2][e] + hist[3][e] : 0;
        if (e < E) counts[e] = v[j];
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
    for (int e = tid; e <= E; e += 256) offsets[e] = offs[e];
    // per-wave base rows, then the scatter of the three-kernel path
    for (int e = tid; e < E; e += 256) {
        int r = offs[e];
#pragma unroll
        for (int w = 0; w < kPermWaves; ++w) {
            const int h = hist[w][e];
            hist[w][e] = r;
            r += h;
        }
    }
    __syncthreads();
    wave_scatter(ids, P, K, E, w_begin, w_end, id_bits, hist[wv], perm_token, inv_pos);
}

// The permutation of at most 256 pairs in one 256-thread workgroup, thread p
// taking pair p, from ids already in LDS (pairs[0 .. P)): each thread walks
// every pair once, counting those of its expert and those of its expert
// before it; the first pair of each expert stores the count; a block scan of
// the counts (four consecutive experts per thread) gives the offsets, and a
// pair's row is its expert's offset plus the pairs of that expert before it
// (token order within an expert, as in the multi-block path).  No atomics.
// Every thread of the workgroup must call this.
constexpr int kSmallPairs = 256;

__device__ __forceinline__ void permute_small(const int* pairs, int P, int K, int E, int32_t* __restrict__ counts,
                                              int32_t* __restrict__ offsets, int32_t* __restrict__ perm_token,
                                              int32_t* __restrict__ inv_pos) {
    __shared__ int cnt[kMaxExperts];
    __shared__ int wsum[kPermWaves];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    for (int e = tid; e < E; e += 256) cnt[e] = 0;
    const int ep = tid < P ? pairs[tid] : -1;
    const bool valid = ep >= 0 && ep < E;
    int before = 0, same = 0;
    for (int q = 0; q < P; ++q) {
        const int eq = pairs[q];
        before += (eq == ep && q < tid) ? 1 : 0;
        same += eq == ep ? 1 : 0;
    }
    __syncthreads();  // cnt zeroed
    if (valid && before == 0) cnt[ep] = same;
    __syncthreads();
    int c[4];
    int local = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = 4 * tid + j;
        c[j] = e < E ? cnt[e] : 0;
        local += c[j];
    }
    int incl = local;  // inclusive scan over the wave
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int v = __shfl_up(incl, d);
        if (lane >= d) incl += v;
    }
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    int run = incl - local;
    for (int w = 0; w < wv; ++w) run += wsum[w];
    __syncthreads();  // every count read before the offsets replace them
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = 4 * tid + j;
        if (e < E) {
            counts[e] = c[j];
            offsets[e] = run;
            cnt[e] = run;
        }
        run += c[j];
    }
    if (tid == 255) offsets[E] = run;
    __syncthreads();
    if (tid < P) {
        if (valid) {
            const int pos = cnt[ep] + before;
            perm_token[pos] = tid / K;
            inv_pos[tid] = pos;
        } else {
            inv_pos[tid] = -1;
        }
    }
}

}  // namespace moe
