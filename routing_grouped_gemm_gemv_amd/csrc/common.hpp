// Shared device helpers of the MoE library (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// 16 bytes as a native vector (HIP's uint4 struct defeats scalar replacement of arrays)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    __bf16 h = static_cast<__bf16>(f);
    return __builtin_bit_cast(uint16_t, h);
}

// v_mfma_f32_16x16x32_bf16: D[16x16] = A[16x32] * B[32x16] + C.
// Lane l supplies row (l % 16) of A and column (l % 16) of B, each with the
// eight k values 8*(l/16) .. 8*(l/16)+7; it receives D[4*(l/16) + i][l % 16].
// silu(g) * u with the hardware exponential and reciprocal (about 2 ulp in
// float32); used where the activation is then rounded to bf16 (the
// gate_up epilogue, and the backward pass recomputing the same activation)
__device__ __forceinline__ float silu_mul_fast(float g, float u) {
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// v_mfma_f32_16x16x4_f32: lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16].
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Map a workgroup id so that consecutive logical ids run on the same XCD.
// Workgroups are dispatched round-robin over the 8 XCDs; with a grid padded to
// a multiple of 8, XCD x then receives the contiguous logical range
// [x * n/8, (x+1) * n/8), so neighbouring tiles share that XCD's L2.
__device__ __forceinline__ int64_t xcd_remap(int64_t bid, int64_t nwg) {
    const int64_t per = nwg >> 3;
    return (bid & 7) * per + (bid >> 3);
}

// M0 is reserved to the compiler; the DMA asm below sets it on purpose
#pragma clang diagnostic ignored "-Winline-asm"

// 16 bytes per lane from global memory (base + 32-bit per-lane offset) into
// LDS at wave_base + 16 * lane: global_load_lds_dwordx4 with M0 holding the
// wave's LDS base.  It is issued from inline asm on purpose: the compiler's
// wait-count tracking of LDS DMA cannot tell the stages of this pipeline
// apart and would drain every DMA in flight before each fragment read.  The
// instruction has no destination register; completion is awaited with the
// explicit vmcnt waits of the pipelines that use it, and no other code in
// those kernels uses M0.
// The base address and the LDS base are wave-uniform; readfirstlane states
// that to the compiler where it cannot prove it.
__device__ __forceinline__ void dma16(const uint8_t* gbase, uint32_t voff, uint32_t lds_wave_base) {
    const uint64_t g = reinterpret_cast<uint64_t>(gbase);
    const uint64_t gu = (static_cast<uint64_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(g >> 32))) << 32) |
                        static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(g)));
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_wave_base);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(m0), "v"(voff), "s"(reinterpret_cast<const uint8_t*>(gu))
                 : "memory", "m0");
}

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;

// s_waitcnt with vmcnt(n) and the other counters left alone
constexpr int vmcnt_imm(int n) { return 0x3F70 | (n & 15) | (((n >> 4) & 3) << 14); }
template <int N>
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(vmcnt_imm(N)); }

}  // namespace moe
