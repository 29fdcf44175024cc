// Expert MLP for few rows per expert (decode-sized batches): the same
// grouped gate_up + SwiGLU and down products as the tiled kernels, laid out
// for weight streaming instead of operand reuse.
//
// With a handful of routed rows per expert, the 256-row tiles of the grouped
// GEMM give each expert's weight slice to one CU and leave most CUs idle,
// while the work is bound by reading the touched experts' weights once.
// Here one wave computes up to 64 rows (four 16-row blocks) of one expert
// against one 16-column slice of its weights, so the weights of even a single
// routed token are streamed by hundreds of waves at once, and an expert's
// weights are read once per 64 of its rows.  Every output element is the same
// MFMA chain as in the tiled kernels (v_mfma_f32_16x16x32_bf16 over k in
// ascending 32-wide steps from zero, rows in 16-row blocks counted from the
// expert's first row, columns in 16-column blocks) and the same epilogue
// rounding, so both paths give the same bits and the choice between them
// (made from the shape alone) does not change any result.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kSkRows = 64;  // rows of a unit: up to four 16-row MFMA blocks, one weight stream

struct SkinnyParams {
    const uint16_t* a;          // rows: x (gathered through perm) or the activations
    const int32_t* perm;        // row -> x row, or null (identity)
    const int32_t* offsets;     // [G + 1] row ranges, or null: one group of ident_rows rows
    const int32_t* u_start;     // [G + 1] prefix of the groups' 64-row units
    int G;
    int ident_rows;
    int Kd;                     // reduction length (D for gate_up, I for down)
    const uint16_t* w;          // the groups' weight matrices [.][Kd], w_group_stride apart
    int64_t w_group_stride;
    int I;                      // gate_up: up rows start at I
    int N;                      // output columns (I for gate_up, D for down)
    uint16_t* out;              // [rows][N] bf16
};

// u_start[g] = sum over earlier groups of ceil(rows / 64); u_start[G] = total
__global__ __launch_bounds__(1024) void skinny_prefix_kernel(const int32_t* __restrict__ offsets, int G,
                                                             int ident_rows, int32_t* __restrict__ u_start) {
    __shared__ int part[1024];
    const int tid = threadIdx.x;
    int v = 0;
    if (tid < G) {
        const int c = offsets ? offsets[tid + 1] - offsets[tid] : ident_rows;
        v = (c + kSkRows - 1) / kSkRows;
    }
    part[tid] = v;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {
        const int u = tid >= d ? part[tid - d] : 0;
        __syncthreads();
        part[tid] += u;
        __syncthreads();
    }
    if (tid < G) u_start[tid + 1] = part[tid];
    if (tid == 0) u_start[0] = 0;
}

// The k loop of one wave over RB row blocks (nb of them valid, uniform) with
// U 32-wide steps of loads issued before their MFMAs.
template <bool GATE_UP, int RB, int U>
__device__ __forceinline__ void skinny_loop(const uint16_t* const (&ap)[4], const uint16_t* bp, const uint16_t* cp,
                                            int S, int nb, f32x4 (&acc)[4], f32x4 (&acc_u)[4]) {
    for (int s0 = 0; s0 < S; s0 += U) {
        u32x4 a[U][RB], b[U], c[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int s = s0 + u < S ? s0 + u : S - 1;
            b[u] = *reinterpret_cast<const u32x4*>(bp + 32 * s);
            if (GATE_UP) c[u] = *reinterpret_cast<const u32x4*>(cp + 32 * s);
#pragma unroll
            for (int r = 0; r < RB; ++r)
                if (r < nb) a[u][r] = *reinterpret_cast<const u32x4*>(ap[r] + 32 * s);
        }
        __builtin_amdgcn_sched_barrier(0);  // every load of the batch is in flight before the first MFMA
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (s0 + u >= S) break;  // uniform
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                if (r >= nb) break;  // uniform
                acc[r] = mfma_bf16(b[u], a[u][r], acc[r]);
                if (GATE_UP) acc_u[r] = mfma_bf16(c[u], a[u][r], acc_u[r]);
            }
        }
    }
}

// One wave per (group, 16-column slice, 64-row unit); the units and slices of
// a group run on consecutive workgroups.
template <bool GATE_UP>
__global__ __launch_bounds__(64) void skinny_kernel(SkinnyParams p) {
    const int lane = threadIdx.x;
    const int ns = p.N / 16;  // column slices
    const int64_t L = blockIdx.x;
    if (L >= static_cast<int64_t>(p.u_start[p.G]) * ns) return;
    int lo = 0, hi = p.G - 1;  // last group whose first unit is <= L
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (static_cast<int64_t>(p.u_start[mid]) * ns <= L) lo = mid; else hi = mid - 1;
    }
    const int g = lo;
    const int nu = p.u_start[g + 1] - p.u_start[g];
    const int loc = static_cast<int>(L - static_cast<int64_t>(p.u_start[g]) * ns);
    const int slice = loc / nu;
    const int unit = loc % nu;
    const int o0 = p.offsets ? p.offsets[g] : 0;
    const int o1 = p.offsets ? p.offsets[g + 1] : p.ident_rows;
    const int r0 = o0 + kSkRows * unit;               // first row of the unit
    const int nb = min(4, (o1 - r0 + 15) / 16);      // valid 16-row blocks (uniform)

    // operand rows: row r0 + 16 r + lane % 16 of block r (rows past the group
    // repeat its last row and are never stored); weight row n (and I + n)
    const int kq = 8 * (lane >> 4);  // this lane's 8 k of each 32-wide step
    const uint16_t* ap[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        int row = r0 + 16 * r + (lane & 15);
        if (row > o1 - 1) row = o1 - 1;
        const int64_t arow = p.perm ? p.perm[row] : row;
        ap[r] = p.a + arow * p.Kd + kq;
    }
    const int n = 16 * slice + (lane & 15);
    const uint16_t* wg = p.w + static_cast<int64_t>(g) * p.w_group_stride;
    const uint16_t* bp = wg + static_cast<int64_t>(n) * p.Kd + kq;
    const uint16_t* cp = GATE_UP ? wg + static_cast<int64_t>(p.I + n) * p.Kd + kq : bp;

    f32x4 acc[4], acc_u[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = acc_u[r] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int S = p.Kd / 32;
    if (nb == 1) skinny_loop<GATE_UP, 1, 8>(ap, bp, cp, S, nb, acc, acc_u);
    else skinny_loop<GATE_UP, 4, 4>(ap, bp, cp, S, nb, acc, acc_u);

    // lane holds row r0 + 16 r + lane % 16 and the 4 columns 16 slice + 4 (lane / 16) + i
    const int col = 16 * slice + 4 * (lane >> 4);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int orow = r0 + 16 * r + (lane & 15);
        if (r >= nb || orow >= o1) continue;
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = GATE_UP ? silu_mul_fast(acc[r][i], acc_u[r][i]) : acc[r][i];
        const uint32_t w0 = static_cast<uint32_t>(f32_to_bf16(v[0])) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
        const uint32_t w1 = static_cast<uint32_t>(f32_to_bf16(v[2])) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16);
        *reinterpret_cast<u32x2*>(p.out + static_cast<int64_t>(orow) * p.N + col) = u32x2{w0, w1};
    }
}

bool experts_use_skinny(int64_t rows_max, int G, int dtype) {
    // bf16 operands and decode-sized batches: at most 4 rows per expert on
    // average (measured crossover with the tiled kernels on the Qwen3-30B-
    // and DeepSeek-V4-like layers), or at most 64 rows of a single group (the
    // shared expert, which the tiled kernels give only its n-tiles)
    if (dtype != 0) return false;
    return G > 1 ? rows_max <= static_cast<int64_t>(4) * G : rows_max <= 64;
}

hipError_t launch_experts_skinny(const void* x, const int32_t* perm_token, const int32_t* offsets, int G,
                                 int64_t rows_max, int D, int I, const void* gate_up, const void* down, void* y,
                                 void* ws, hipStream_t stream) {
    // the workspace of launch_experts: u_start in its table area at the
    // front, the activations [rows_max][I] where the tiled path keeps them
    const size_t ws_total = experts_ws_bytes(rows_max, G, D, I, 0);
    const size_t act_bytes = (static_cast<size_t>(rows_max) * I * 2 + 255) & ~static_cast<size_t>(255);
    int32_t* u_start = static_cast<int32_t*>(ws);
    uint16_t* act = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(ws) + (ws_total - act_bytes));
    const int ident_rows = static_cast<int>(rows_max);
    skinny_prefix_kernel<<<1, 1024, 0, stream>>>(offsets, G, ident_rows, u_start);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    // units: at most ceil(rows / 64) + G, times the column slices
    const int64_t blocks = (rows_max + kSkRows - 1) / kSkRows + G;
    SkinnyParams p{};
    p.perm = perm_token;
    p.offsets = offsets;
    p.u_start = u_start;
    p.G = G;
    p.ident_rows = ident_rows;
    p.a = static_cast<const uint16_t*>(x);
    p.Kd = D;
    p.w = static_cast<const uint16_t*>(gate_up);
    p.w_group_stride = static_cast<int64_t>(2) * I * D;
    p.I = I;
    p.N = I;
    p.out = act;
    skinny_kernel<true><<<static_cast<unsigned>(blocks * (I / 16)), 64, 0, stream>>>(p);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    p.a = act;
    p.perm = nullptr;
    p.Kd = I;
    p.w = static_cast<const uint16_t*>(down);
    p.w_group_stride = static_cast<int64_t>(D) * I;
    p.N = D;
    p.out = static_cast<uint16_t*>(y);
    skinny_kernel<false><<<static_cast<unsigned>(blocks * (D / 16)), 64, 0, stream>>>(p);
    return hipGetLastError();
}

}  // namespace moe
