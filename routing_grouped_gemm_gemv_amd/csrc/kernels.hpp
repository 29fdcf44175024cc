// Host-side launchers of the MoE kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// ---- routing -----------------------------------------------------------------
// logits64 [T, E] float64 = x [T, D] . router [E, D]^T
hipError_t launch_router_logits(const void* x, const void* router, int64_t T, int D, int E,
                                int dtype, double* logits64, hipStream_t stream);
// scores, selection bias, top-k, weights; optional float32 logits export
hipError_t launch_topk(const double* logits64, int64_t T, int E, int K, int score, int renorm,
                       float route_scale, int n_group, int topk_group, const float* bias, const uint8_t* mask,
                       float* logits_out, int32_t* ids, float* w, hipStream_t stream,
                       const int32_t* given);
// compute units of the current device
int compute_units();
// whether launch_route runs the single fused kernel (bf16 operands, E <= 512,
// no group-limited select)
bool route_fused(int E, int dtype, int n_group);
// decode-sized batches in moe_forward: logits, then top-k and the dispatch
// permutation in one kernel (given: replayed ids or null); the same picks and
// rows as launch_route (or launch_route_replay) followed by launch_permute
bool route_permute_fused(int64_t T);
hipError_t launch_route_permute(const void* x, const void* router, int64_t T, int D, int E, int K, int dtype,
                                int score, int renorm, float route_scale, int n_group, int topk_group,
                                const float* bias, const int32_t* given, const uint8_t* mask, double* logits64,
                                float* logits_out, int32_t* ids, float* w, int32_t* counts, int32_t* offsets,
                                int32_t* perm_token, int32_t* inv_pos, hipStream_t stream);
// logits + top-k: one fused kernel where route_fused(), else the two kernels
// above through logits64 [T, E]; both give the same bits
hipError_t launch_route(const void* x, const void* router, int64_t T, int D, int E, int K, int dtype,
                        int score, int renorm, float route_scale, int n_group, int topk_group, const float* bias,
                        const uint8_t* mask, double* logits64, float* logits_out, int32_t* ids, float* w,
                        hipStream_t stream);
// routing replay: logits through logits64, then the given ids with weights
// from their scores (tokens with invalid given ids are treated as masked);
// n_group is the layer's, which selects the same top-k code as its forward
hipError_t launch_route_replay(const void* x, const void* router, int64_t T, int D, int E, int K, int dtype,
                               int score, int renorm, float route_scale, int n_group, const int32_t* given,
                               const uint8_t* mask, double* logits64, float* logits_out, int32_t* ids, float* w,
                               hipStream_t stream);

// ---- dispatch ----------------------------------------------------------------
struct PermutePlan {
    int pairs_per_block;  // multiple of 256
    int blocks;
    int id_bits;          // bits that distinguish expert ids
};
PermutePlan permute_plan(int64_t P, int E);
size_t permute_ws_bytes(int64_t P, int E);  // block histogram + block bases
hipError_t launch_permute(const int32_t* ids, int64_t T, int K, int E, int32_t* ws_i32,
                          int32_t* counts, int32_t* offsets, int32_t* perm_token, int32_t* inv_pos,
                          hipStream_t stream);

// ---- experts -----------------------------------------------------------------
size_t experts_ws_bytes(int64_t rows_max, int G, int D, int I, int dtype);
// x_rows: rows of x (the gathered rows index it); rows_max: rows of the output
hipError_t launch_experts(const void* x, int64_t x_rows, const int32_t* perm_token, const int32_t* offsets,
                          int G, int64_t rows_max, int D, int I, int dtype, const void* gate_up,
                          const void* down, void* y, void* ws, hipStream_t stream);
// few rows per group (decode-sized batches): one wave per 16-row block and
// 16-column weight slice, the same bits as launch_experts; bf16 only, the
// same workspace
bool experts_use_skinny(int64_t rows_max, int G, int dtype);
// one token whose K picks (and shared expert) fit one workgroup of the fused
// down + combine kernel
bool decode_combine_fits(int64_t T, int K, bool shared);
hipError_t launch_experts_decode_combine(const void* x, const int32_t* perm_token, const int32_t* offsets, int G,
                                         int K, int D, int I, const void* gate_up, const void* down, void* y,
                                         void* ws, int Is, const void* gate_up_s, const void* down_s, void* y_s,
                                         void* act_s, const int32_t* ids, const int32_t* inv_pos, const float* w,
                                         int out_f32, void* out, hipStream_t stream);
hipError_t launch_experts_skinny(const void* x, const int32_t* perm_token, const int32_t* offsets, int G,
                                 int64_t rows_max, int D, int I, const void* gate_up, const void* down, void* y,
                                 void* ws, hipStream_t stream);
// the routed experts (as launch_experts_skinny) and a shared expert of rows_s
// identity rows in the same two launches; act_s: its activations
// [rows_s][Is] bf16
hipError_t launch_experts_skinny_pair(const void* x, const int32_t* perm_token, const int32_t* offsets, int G,
                                      int64_t rows_max, int D, int I, const void* gate_up, const void* down, void* y,
                                      void* ws, int64_t rows_s, int Is, const void* gate_up_s, const void* down_s,
                                      void* y_s, void* act_s, hipStream_t stream);

// ---- combine -----------------------------------------------------------------
// mode 0: float32 fold; mode 1: float64 sum rounded once
hipError_t launch_combine(const void* y, const int32_t* inv_pos, const float* w, const void* shared,
                          int64_t T, int D, int K, int dtype, int out_dtype, int mode, void* out,
                          hipStream_t stream);


// ---- backward ------------------------------------------------------------------
struct BwdArgs {
    int64_t T;
    int D, E, K, I, Is, score, renorm;
    float route_scale;
    const void *x, *router, *gate_up, *down, *gate_up_shared, *down_shared;  // bf16
    const void *dout, *y;                                                    // bf16 [T, D], [P, D]
    const int32_t *topk_ids, *offsets, *perm_token, *inv_pos;
    const float* topk_w;
    const uint8_t* mask;
    float *dx, *d_router, *d_gate_up, *d_down, *d_gate_up_shared, *d_down_shared;
    void* ws;
};
size_t backward_ws_bytes(int64_t T, int D, int E, int K, int I, int Is);
// whether every buffer the backward's GEMMs stage spans less than 4 GiB
bool backward_fits_dma(int64_t T, int D, int K, int I, int Is);
hipError_t launch_backward(const BwdArgs& a, hipStream_t stream);
// T == 0: zeroes the weight gradients (dx has no elements)
hipError_t launch_backward_empty(const BwdArgs& a, hipStream_t stream);

}  // namespace moe
