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
    int G;                      // at most 1024
    int ident_rows;
    int Kd;                     // reduction length (D for gate_up, I for down)
    const uint16_t* w;          // the groups' weight matrices [.][Kd], w_group_stride apart
    int64_t w_group_stride;
    int I;                      // gate_up: up rows start at I
    int N;                      // output columns (I for gate_up, D for down)
    uint16_t* out;              // [rows][N] bf16
};

// Work item L of a launch: unit `unit` (64 rows) of group g against column
// slice `slice`, items in group order, the units of a slice consecutive.  The
// wave finds it from the offsets alone, with one round of loads: lane l holds
// the row counts of groups [l*gpl, (l+1)*gpl), a wave scan of their unit
// counts gives each group's first item, and the lane whose range holds L
// hands (g, rows of g) to the others.  Returns false when L is past the last
// item.
__device__ __forceinline__ bool skinny_locate(const SkinnyParams& p, int64_t L, int ns, int& g, int& o0, int& o1,
                                              int& slice, int& unit) {
    const int lane = lane_id();
    if (p.offsets == nullptr) {  // one group of ident_rows rows
        const int nu = (p.ident_rows + kSkRows - 1) / kSkRows;
        if (L >= static_cast<int64_t>(nu) * ns) return false;
        g = 0;
        o0 = 0;
        o1 = p.ident_rows;
        slice = static_cast<int>(L / nu);
        unit = static_cast<int>(L % nu);
        return true;
    }
    constexpr int kMaxPer = 16;  // groups per lane: G <= 1024
    const int gpl = (p.G + 63) / 64;
    const int ga = lane * gpl;
    int beg[kMaxPer], cnt[kMaxPer];
#pragma unroll
    for (int k = 0; k < kMaxPer; ++k) {
        // every load in bounds (a clamped group) and unconditional, so all of
        // them are in flight together
        int gi = ga + k;
        if (gi > p.G - 1) gi = p.G - 1;
        beg[k] = p.offsets[gi];
        cnt[k] = p.offsets[gi + 1];
    }
    int local = 0;
#pragma unroll
    for (int k = 0; k < kMaxPer; ++k) {
        const bool own = k < gpl && ga + k < p.G;
        cnt[k] = own ? cnt[k] - beg[k] : 0;
        local += (cnt[k] + kSkRows - 1) / kSkRows;
    }
    int incl = local;  // inclusive wave scan of the unit counts
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int v = __shfl_up(incl, d);
        if (lane >= d) incl += v;
    }
    const int total = __shfl(incl, 63);
    if (L >= static_cast<int64_t>(total) * ns) return false;
    int u0 = incl - local;  // first unit of this lane's first group
    bool found = false;
    int fg = 0, fb = 0, fc = 0, floc = 0, fnu = 1;
#pragma unroll
    for (int k = 0; k < kMaxPer; ++k) {
        const int nu = (cnt[k] + kSkRows - 1) / kSkRows;
        const int64_t first = static_cast<int64_t>(u0) * ns;
        if (nu > 0 && L >= first && L < first + static_cast<int64_t>(nu) * ns) {
            found = true;
            fg = ga + k;
            fb = beg[k];
            fc = cnt[k];
            floc = static_cast<int>(L - first);
            fnu = nu;
        }
        u0 += nu;
    }
    const uint64_t who = __ballot(found);
    const int src = __builtin_ctzll(who);  // exactly one lane: L < total
    g = __shfl(fg, src);
    o0 = __shfl(fb, src);
    o1 = o0 + __shfl(fc, src);
    const int loc = __shfl(floc, src);
    const int nu = __shfl(fnu, src);
    slice = loc / nu;
    unit = loc % nu;
    return true;
}

// The k loop of one wave over RB row blocks (nb of them valid, uniform):
// batches of U 32-wide steps, double-buffered, so the loads of the next
// batch are in flight while the MFMAs of the current one run; the last
// S % U steps follow on their own.  Operand pointers advance per batch and
// each load is an immediate offset from them.  The MFMAs take the steps in
// ascending order, as in a plain loop.
template <int RB, int U>
__device__ __forceinline__ void skinny_loop(const uint16_t* const (&ap)[4], const uint16_t* bp, int S, int nb,
                                            f32x4 (&acc)[4]) {
    const uint16_t* aq[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) aq[r] = ap[r];
    const uint16_t* bq = bp;
    u32x4 a0[U][RB], b0[U], a1[U][RB], b1[U];
    auto load = [&](u32x4 (&a)[U][RB], u32x4 (&b)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            b[u] = *reinterpret_cast<const u32x4*>(bq + 32 * u);
#pragma unroll
            for (int r = 0; r < RB; ++r) a[u][r] = *reinterpret_cast<const u32x4*>(aq[r] + 32 * u);
        }
        bq += 32 * U;
#pragma unroll
        for (int r = 0; r < RB; ++r) aq[r] += 32 * U;
    };
    auto mma = [&](const u32x4 (&a)[U][RB], const u32x4 (&b)[U], int n) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (u >= n) break;  // uniform
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                if (r >= nb) break;  // uniform
                acc[r] = mfma_bf16(b[u], a[u][r], acc[r]);
            }
        }
    };
    const int full = S / U;
    if (full > 0) {
        load(a0, b0);  // batch 0
        int i = 0;     // batch i is in a0
        for (; i + 2 < full; i += 2) {
            load(a1, b1);
            __builtin_amdgcn_sched_barrier(0);
            mma(a0, b0, U);
            load(a0, b0);
            __builtin_amdgcn_sched_barrier(0);
            mma(a1, b1, U);
        }
        if (i + 1 < full) {
            load(a1, b1);
            __builtin_amdgcn_sched_barrier(0);
            mma(a0, b0, U);
            mma(a1, b1, U);
        } else {
            mma(a0, b0, U);
        }
    }
    const int rem = S - full * U;
    if (rem > 0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (u >= rem) break;  // uniform
            b0[u] = *reinterpret_cast<const u32x4*>(bq + 32 * u);
#pragma unroll
            for (int r = 0; r < RB; ++r) a0[u][r] = *reinterpret_cast<const u32x4*>(aq[r] + 32 * u);
        }
        mma(a0, b0, rem);
    }
}

// One wave per (group, 16-column slice, 64-row unit); the units and slices of
// a group run on consecutive workgroups.
// Blocks below `split` work on problem p0, the others on p1 (the routed
// experts and the shared expert of one layer in one launch: both are weight
// streams too short to fill the chip on their own).
// gate_up: two waves per work item, wave 0 streaming the gate rows and wave 1
// the up rows (each the same MFMA chain as one wave doing both), the up
// accumulators meeting the gate ones in LDS for the epilogue: twice the waves
// in flight for the same weight stream.
template <bool GATE_UP>
__global__ __launch_bounds__(GATE_UP ? 128 : 64) void skinny_kernel(SkinnyParams p0, SkinnyParams p1, int64_t split) {
    const int lane = threadIdx.x & 63;
    const int half = GATE_UP ? static_cast<int>(threadIdx.x >> 6) : 0;  // gate_up: 0 gate rows, 1 up rows
    const bool second = static_cast<int64_t>(blockIdx.x) >= split;
    const SkinnyParams p = second ? p1 : p0;
    const int64_t L = second ? static_cast<int64_t>(blockIdx.x) - split : static_cast<int64_t>(blockIdx.x);
    const int ns = p.N / 16;  // column slices
    int g, o0, o1, slice, unit;
    if (!skinny_locate(p, L, ns, g, o0, o1, slice, unit)) return;
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
    const uint16_t* bp = wg + static_cast<int64_t>(half * p.I + n) * p.Kd + kq;

    f32x4 acc[4], acc_u[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = acc_u[r] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int S = p.Kd / 32;
    if (nb == 1) skinny_loop<1, 8>(ap, bp, S, nb, acc);
    else skinny_loop<4, 4>(ap, bp, S, nb, acc);
    if (GATE_UP) {
        __shared__ f32x4 up_acc[4][64];
        if (half == 1) {
#pragma unroll
            for (int r = 0; r < 4; ++r) up_acc[r][lane] = acc[r];
        }
        __syncthreads();
        if (half == 1) return;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc_u[r] = up_acc[r][lane];
    }

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

// One token: the down projections of its K routed experts (and of the
// shared expert) and the combine, in one launch.  Workgroup n takes output
// columns 16 n .. 16 n + 15; its wave j < K computes pick j's 16 columns
// exactly as skinny_kernel<false> does (its group holds one row, so every
// MFMA row is that row; the same chain over I in ascending 32-wide steps),
// stores them to y as bf16 and hands them to LDS; wave K does the shared
// expert's.  Wave 0 then folds them as the combine does: from +0, in pick
// order (ascending expert id) fl32(w_j * f32(y_j)), then f32(shared), no
// fused multiply-add, one rounding to bf16 (or the float32 sum); a token
// with no pick gives +0.  The same bits as the down launch followed by the
// combine, one launch and one pass over y fewer.
// NW waves: 8 (two per SIMD, 256 registers each, k batches of U = 8 steps) or
// 16 (four per SIMD, 128 registers, batches of U = 4 steps: the same MFMA
// chain, k ascending).
constexpr int kDecodeWaves = 16;

template <int NW, int U>
__global__ __launch_bounds__(64 * NW) void skinny_down_combine_kernel(
    SkinnyParams rp, SkinnyParams sp, int K, const int32_t* __restrict__ ids, const int32_t* __restrict__ inv_pos,
    const float* __restrict__ w, int out_f32, void* __restrict__ out) {
    __shared__ float red[NW][16];
    const int lane = threadIdx.x & 63;
    const int j = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const int slice = blockIdx.x;
    const bool shared_wave = j == K;
    const SkinnyParams& p = shared_wave ? sp : rp;
    int row = 0;   // the pick's row of the activations and of y
    int g = 0;     // its expert
    bool live = true;
    if (!shared_wave) {
        row = inv_pos[j];
        g = ids[j];
        live = row >= 0 && g >= 0;
    }
    if (live) {
        const int kq = 8 * (lane >> 4);
        const uint16_t* ap[4];
        ap[0] = p.a + static_cast<int64_t>(row) * p.Kd + kq;
        ap[1] = ap[2] = ap[3] = ap[0];
        const int n = 16 * slice + (lane & 15);
        const uint16_t* bp = p.w + static_cast<int64_t>(g) * p.w_group_stride + static_cast<int64_t>(n) * p.Kd + kq;
        f32x4 acc[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
        skinny_loop<1, U>(ap, bp, p.Kd / 32, 1, acc);
        // lanes 0, 16, 32, 48 hold the row's columns 16 slice + 4 (lane / 16) + i
        if ((lane & 15) == 0) {
            const int c = 4 * (lane >> 4);
            uint16_t b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                b[i] = f32_to_bf16(acc[0][i]);
                red[j][c + i] = bf16_to_f32(b[i]);
            }
            const uint32_t w0 = static_cast<uint32_t>(b[0]) | (static_cast<uint32_t>(b[1]) << 16);
            const uint32_t w1 = static_cast<uint32_t>(b[2]) | (static_cast<uint32_t>(b[3]) << 16);
            *reinterpret_cast<u32x2*>(p.out + static_cast<int64_t>(row) * p.N + 16 * slice + c) = u32x2{w0, w1};
        }
    }
    __syncthreads();
    if (j == 0 && lane < 16) {
#pragma clang fp contract(off)
        const int col = 16 * slice + lane;
        float acc = 0.0f;
        bool kept = false;
        for (int q = 0; q < K; ++q) {
            if (inv_pos[q] < 0 || ids[q] < 0) continue;
            kept = true;
            const float prod = w[q] * red[q][lane];
            acc = acc + prod;
        }
        if (kept && sp.w != nullptr) acc = acc + red[K][lane];
        if (!kept) acc = 0.0f;
        if (out_f32) static_cast<float*>(out)[col] = acc;
        else static_cast<uint16_t*>(out)[col] = f32_to_bf16(acc);
    }
}

bool decode_combine_fits(int64_t T, int K, bool shared) { return T == 1 && K + (shared ? 1 : 0) <= kDecodeWaves; }

bool experts_use_skinny(int64_t rows_max, int G, int dtype) {
    // bf16 operands and decode-sized batches: at most 4 rows per expert on
    // average (measured crossover with the tiled kernels on the Qwen3-30B-
    // and DeepSeek-V4-like layers), or at most 64 rows of a single group (the
    // shared expert, which the tiled kernels give only its n-tiles)
    if (dtype != 0) return false;
    return G > 1 ? rows_max <= static_cast<int64_t>(4) * G : rows_max <= 64;
}

// The two products of one expert MLP problem and their grid bounds.
struct SkinnyProblem {
    SkinnyParams gu, dn;
    int64_t units;  // upper bound of the 64-row units
};

static SkinnyProblem skinny_problem(const void* x, const int32_t* perm_token, const int32_t* offsets, int G,
                                    int64_t rows_max, int D, int I, const void* gate_up, const void* down, void* y,
                                    uint16_t* act) {
    SkinnyProblem pr;
    // a group of c rows has ceil(c / 64) <= c / 64 + 1 units, and at most
    // min(G, rows) groups are non-empty
    const int64_t groups = offsets ? (rows_max < G ? rows_max : G) : 1;
    pr.units = (rows_max + kSkRows - 1) / kSkRows + groups;
    SkinnyParams p{};
    p.perm = perm_token;
    p.offsets = offsets;
    p.G = offsets ? G : 1;
    p.ident_rows = static_cast<int>(rows_max);
    p.a = static_cast<const uint16_t*>(x);
    p.Kd = D;
    p.w = static_cast<const uint16_t*>(gate_up);
    p.w_group_stride = static_cast<int64_t>(2) * I * D;
    p.I = I;
    p.N = I;
    p.out = act;
    pr.gu = p;
    p.a = act;
    p.perm = nullptr;
    p.Kd = I;
    p.w = static_cast<const uint16_t*>(down);
    p.w_group_stride = static_cast<int64_t>(D) * I;
    p.N = D;
    p.out = static_cast<uint16_t*>(y);
    pr.dn = p;
    return pr;
}

static uint16_t* skinny_act(void* ws, int64_t rows_max, int G, int D, int I) {
    // the workspace of launch_experts: the activations [rows_max][I] where
    // the tiled path keeps them
    const size_t ws_total = experts_ws_bytes(rows_max, G, D, I, 0);
    const size_t act_bytes = (static_cast<size_t>(rows_max) * I * 2 + 255) & ~static_cast<size_t>(255);
    return reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(ws) + (ws_total - act_bytes));
}

hipError_t launch_experts_skinny(const void* x, const int32_t* perm_token, const int32_t* offsets, int G,
                                 int64_t rows_max, int D, int I, const void* gate_up, const void* down, void* y,
                                 void* ws, hipStream_t stream) {
    const SkinnyProblem a = skinny_problem(x, perm_token, offsets, G, rows_max, D, I, gate_up, down, y,
                                           skinny_act(ws, rows_max, G, D, I));
    const int64_t b1 = a.units * (I / 16), b2 = a.units * (D / 16);
    skinny_kernel<true><<<static_cast<unsigned>(b1), 128, 0, stream>>>(a.gu, a.gu, b1);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    skinny_kernel<false><<<static_cast<unsigned>(b2), 64, 0, stream>>>(a.dn, a.dn, b2);
    return hipGetLastError();
}

hipError_t launch_experts_skinny_pair(const void* x, const int32_t* perm_token, const int32_t* offsets, int G,
                                      int64_t rows_max, int D, int I, const void* gate_up, const void* down, void* y,
                                      void* ws, int64_t rows_s, int Is, const void* gate_up_s, const void* down_s,
                                      void* y_s, void* act_s, hipStream_t stream) {
    const SkinnyProblem a = skinny_problem(x, perm_token, offsets, G, rows_max, D, I, gate_up, down, y,
                                           skinny_act(ws, rows_max, G, D, I));
    const SkinnyProblem b = skinny_problem(x, nullptr, nullptr, 1, rows_s, D, Is, gate_up_s, down_s, y_s,
                                           static_cast<uint16_t*>(act_s));
    const int64_t a1 = a.units * (I / 16), a2 = a.units * (D / 16);
    const int64_t n1 = a1 + b.units * (Is / 16), n2 = a2 + b.units * (D / 16);
    skinny_kernel<true><<<static_cast<unsigned>(n1), 128, 0, stream>>>(a.gu, b.gu, a1);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    skinny_kernel<false><<<static_cast<unsigned>(n2), 64, 0, stream>>>(a.dn, b.dn, a2);
    return hipGetLastError();
}

// One token (decode_combine_fits): the gate_up launch of launch_experts_skinny
// or launch_experts_skinny_pair, then skinny_down_combine_kernel in place of
// the down launch and the combine.  y, y_s and act_s as there; ids, inv_pos
// and w the pick's ids, rows and weights; out [D] bf16 or float32.
hipError_t launch_experts_decode_combine(const void* x, const int32_t* perm_token, const int32_t* offsets, int G,
                                         int K, int D, int I, const void* gate_up, const void* down, void* y,
                                         void* ws, int Is, const void* gate_up_s, const void* down_s, void* y_s,
                                         void* act_s, const int32_t* ids, const int32_t* inv_pos, const float* w,
                                         int out_f32, void* out, hipStream_t stream) {
    const SkinnyProblem a = skinny_problem(x, perm_token, offsets, G, K, D, I, gate_up, down, y,
                                           skinny_act(ws, K, G, D, I));
    SkinnyParams sdn{};  // no shared expert: w stays null
    if (Is > 0) {
        const SkinnyProblem b = skinny_problem(x, nullptr, nullptr, 1, 1, D, Is, gate_up_s, down_s, y_s,
                                               static_cast<uint16_t*>(act_s));
        const int64_t a1 = a.units * (I / 16);
        const int64_t n1 = a1 + b.units * (Is / 16);
        skinny_kernel<true><<<static_cast<unsigned>(n1), 128, 0, stream>>>(a.gu, b.gu, a1);
        sdn = b.dn;
    } else {
        const int64_t b1 = a.units * (I / 16);
        skinny_kernel<true><<<static_cast<unsigned>(b1), 128, 0, stream>>>(a.gu, a.gu, b1);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int waves = K + (Is > 0 ? 1 : 0);
    const unsigned grid = static_cast<unsigned>(D / 16);
    if (waves <= 8)
        skinny_down_combine_kernel<8, 8><<<grid, 64 * waves, 0, stream>>>(a.dn, sdn, K, ids, inv_pos, w, out_f32, out);
    else
        skinny_down_combine_kernel<16, 4><<<grid, 64 * waves, 0, stream>>>(a.dn, sdn, K, ids, inv_pos, w, out_f32, out);
    return hipGetLastError();
}

}  // namespace moe
