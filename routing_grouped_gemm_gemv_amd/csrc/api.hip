// C ABI of the MoE layer forward: argument validation, workspace layout and
// the order of launches.  Every check happens before the first launch, so a
// rejected call leaves the outputs untouched (fail closed, as the RL-Kernel
// roadmap's issue buckets require of unsupported configurations).
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <initializer_list>
#include <mutex>
#include <string>

#include "../../include/moe.h"
#include "kernels.hpp"

namespace {

thread_local std::string g_last_error;

moe_status fail(moe_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

moe_status ok() {
    g_last_error.clear();
    return MOE_OK;
}

size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

constexpr int64_t kMaxPairs = (static_cast<int64_t>(1) << 31) - 1;

// size of the fixed scratch of moe_forward_noalloc (MOE_NOALLOC_SCRATCH_BYTES)
constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;

// 0 and 1 both mean: no group-limited select
int n_group(const moe_shape* s) { return s->n_group > 1 ? s->n_group : 1; }

moe_status check_shape(const moe_shape* s) {
    if (s == nullptr) return fail(MOE_ERR_INVALID, "shape is NULL");
    if (s->T < 0) return fail(MOE_ERR_INVALID, "T = %lld is negative", static_cast<long long>(s->T));
    if (s->D <= 0 || s->E <= 0 || s->K <= 0 || s->I <= 0 || s->Is < 0)
        return fail(MOE_ERR_INVALID, "D, E, K, I must be positive and Is non-negative (D=%d E=%d K=%d I=%d Is=%d)",
                    s->D, s->E, s->K, s->I, s->Is);
    if (s->score != MOE_SOFTMAX && s->score != MOE_SIGMOID && s->score != MOE_SQRTSOFTPLUS)
        return fail(MOE_ERR_INVALID, "unknown score function %d", s->score);
    if (s->n_group < 0 || s->topk_group < 0)
        return fail(MOE_ERR_INVALID, "n_group = %d and topk_group = %d must be non-negative", s->n_group, s->topk_group);
    if (s->n_group > 1) {
        if (s->E % s->n_group != 0 || s->E / s->n_group < 2)
            return fail(MOE_ERR_INVALID, "E = %d must split into n_group = %d groups of at least 2 experts", s->E,
                        s->n_group);
        if (s->topk_group < 1 || s->topk_group > s->n_group)
            return fail(MOE_ERR_INVALID, "topk_group = %d must lie in [1, n_group = %d]", s->topk_group, s->n_group);
        if (s->K > s->topk_group * (s->E / s->n_group))
            return fail(MOE_ERR_INVALID, "K = %d exceeds the %d experts of the kept groups", s->K,
                        s->topk_group * (s->E / s->n_group));
        if (s->n_group > 64) return fail(MOE_ERR_UNSUPPORTED, "n_group = %d exceeds 64", s->n_group);
    }
    if (s->dtype != MOE_BF16 && s->dtype != MOE_F32) return fail(MOE_ERR_INVALID, "unknown operand dtype %d", s->dtype);
    if (s->renorm != 0 && s->renorm != 1) return fail(MOE_ERR_INVALID, "renorm must be 0 or 1, got %d", s->renorm);
    if (s->combine != MOE_COMBINE_F32_FOLD && s->combine != MOE_COMBINE_F64)
        return fail(MOE_ERR_INVALID, "unknown combine mode %d", s->combine);
    if (!isfinite(s->route_scale) || !(s->route_scale > 0.0f))
        return fail(MOE_ERR_INVALID, "route_scale must be finite and positive");
    if (s->K > s->E) return fail(MOE_ERR_INVALID, "K = %d exceeds E = %d", s->K, s->E);
    if (s->E > 1024) return fail(MOE_ERR_UNSUPPORTED, "E = %d exceeds 1024", s->E);
    if (s->K > 16) return fail(MOE_ERR_UNSUPPORTED, "K = %d exceeds 16", s->K);
    if (s->D % 64 != 0) return fail(MOE_ERR_UNSUPPORTED, "D = %d is not a multiple of 64", s->D);
    if (s->I % 64 != 0) return fail(MOE_ERR_UNSUPPORTED, "I = %d is not a multiple of 64", s->I);
    if (s->Is % 64 != 0) return fail(MOE_ERR_UNSUPPORTED, "Is = %d is not a multiple of 64", s->Is);
    if (s->T > kMaxPairs / s->K) return fail(MOE_ERR_UNSUPPORTED, "T*K exceeds 2^31 - 1");
    return MOE_OK;
}

// gfx950 only; the answer is cached per device
moe_status check_device() {
    static std::mutex mu;
    static int arch_ok[64];  // 0 unknown, 1 ok, 2 unsupported
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(err));
    if (dev < 0 || dev >= 64) return fail(MOE_ERR_UNSUPPORTED, "device index %d out of range", dev);
    std::lock_guard<std::mutex> lock(mu);
    if (arch_ok[dev] == 0) {
        hipDeviceProp_t prop;
        err = hipGetDeviceProperties(&prop, dev);
        if (err != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(err));
        arch_ok[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        if (arch_ok[dev] == 2) return fail(MOE_ERR_UNSUPPORTED, "device %d is %s, not gfx950", dev, prop.gcnArchName);
    }
    if (arch_ok[dev] == 2) return fail(MOE_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
    return MOE_OK;
}

moe_status hip_status(hipError_t err, const char* what) {
    if (err != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
    return MOE_OK;
}

size_t elem_bytes(int dtype) { return dtype == MOE_BF16 ? 2 : 4; }

// Whether every non-NULL pointer is a multiple of `align` bytes.  The kernels
// move activations, weights, outputs, gradients and workspace in 16-byte
// vectors and index arrays and per-token floats as 4-byte words.
bool aligned(size_t align, std::initializer_list<const void*> ptrs) {
    for (const void* p : ptrs)
        if (p != nullptr && reinterpret_cast<uintptr_t>(p) % align != 0) return false;
    return true;
}

size_t route_ws(const moe_shape* s) { return align256(sizeof(double) * static_cast<size_t>(s->T) * s->E); }
size_t permute_ws(const moe_shape* s) { return align256(moe::permute_ws_bytes(s->T * s->K, s->E)); }
size_t experts_ws(const moe_shape* s) { return align256(moe::experts_ws_bytes(s->T * s->K, s->E, s->D, s->I, s->dtype)); }

// Workspace of moe_forward, in order: logits64, ids, weights, counts, offsets,
// perm_token, inv_pos, permute scratch, expert scratch, y, shared_out.
struct ForwardLayout {
    size_t logits64, ids, w, counts, offsets, perm, inv, perm_ws, exp_ws, y, shared, shared_act, total;
};

// whether moe_forward runs the shared expert in the routed experts' launches
bool shared_with_routed(const moe_shape* s) {
    return s->Is > 0 && moe::experts_use_skinny(s->T * s->K, s->E, s->dtype) &&
           moe::experts_use_skinny(s->T, 1, s->dtype);
}

ForwardLayout forward_layout(const moe_shape* s) {
    ForwardLayout L;
    const size_t T = static_cast<size_t>(s->T);
    const size_t P = T * s->K;
    const size_t eb = elem_bytes(s->dtype);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += align256(bytes);
        return at;
    };
    L.logits64 = take(sizeof(double) * T * s->E);
    L.ids = take(sizeof(int32_t) * P);
    L.w = take(sizeof(float) * P);
    L.counts = take(sizeof(int32_t) * s->E);
    L.offsets = take(sizeof(int32_t) * (s->E + 1));
    L.perm = take(sizeof(int32_t) * P);
    L.inv = take(sizeof(int32_t) * P);
    L.perm_ws = take(moe::permute_ws_bytes(static_cast<int64_t>(P), s->E));
    const size_t ex_routed = moe::experts_ws_bytes(static_cast<int64_t>(P), s->E, s->D, s->I, s->dtype);
    const size_t ex_shared = s->Is > 0 ? moe::experts_ws_bytes(s->T, 1, s->D, s->Is, s->dtype) : 0;
    L.exp_ws = take(ex_routed > ex_shared ? ex_routed : ex_shared);
    L.y = take(eb * P * s->D);
    L.shared = take(s->Is > 0 ? eb * T * s->D : 0);
    // both expert MLPs on the skinny path run in shared launches: the shared
    // expert's activations then need a place of their own
    L.shared_act = take(shared_with_routed(s) ? sizeof(uint16_t) * T * s->Is : 0);
    L.total = off;
    return L;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status status) {
    switch (status) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_INVALID: return "MOE_ERR_INVALID";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
        case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
        case MOE_ERR_HIP: return "MOE_ERR_HIP";
    }
    return "unknown moe_status";
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

moe_status moe_workspace_size(const moe_shape* shape, size_t* bytes) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    if (bytes == nullptr) return fail(MOE_ERR_INVALID, "bytes is NULL");
    *bytes = forward_layout(shape).total;
    return ok();
}

moe_status moe_route(const moe_shape* shape, const void* x, const void* router, const float* sel_bias,
                     const uint8_t* mask, float* logits, int32_t* topk_ids, float* topk_w, void* ws,
                     size_t ws_bytes, hipStream_t stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    if (!aligned(16, {x, router, ws}) || !aligned(4, {sel_bias, logits, topk_ids, topk_w}))
        return fail(MOE_ERR_INVALID, "moe_route: x, router and ws must be 16-byte aligned, the other arrays 4-byte");
    if (shape->T == 0) return ok();
    if (!x || !router || !topk_ids || !topk_w) return fail(MOE_ERR_INVALID, "moe_route: x, router, topk_ids and topk_w are required");
    if (!ws || ws_bytes < route_ws(shape))
        return fail(MOE_ERR_WORKSPACE, "moe_route needs %zu workspace bytes, got %zu", route_ws(shape), ws ? ws_bytes : 0);
    if ((st = check_device()) != MOE_OK) return st;
    double* l64 = static_cast<double*>(ws);
    if ((st = hip_status(moe::launch_route(x, router, shape->T, shape->D, shape->E, shape->K, shape->dtype,
                                           shape->score, shape->renorm, shape->route_scale, n_group(shape),
                                           shape->topk_group, sel_bias, mask, l64, logits, topk_ids, topk_w, stream),
                         "routing launch")) != MOE_OK)
        return st;
    return ok();
}

moe_status moe_route_replay(const moe_shape* shape, const void* x, const void* router, const int32_t* replay_ids,
                            const uint8_t* mask, float* logits, int32_t* topk_ids, float* topk_w, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    if (!aligned(16, {x, router, ws}) || !aligned(4, {replay_ids, logits, topk_ids, topk_w}))
        return fail(MOE_ERR_INVALID, "moe_route_replay: x, router and ws must be 16-byte aligned, the other arrays 4-byte");
    if (shape->T == 0) return ok();
    if (!x || !router || !replay_ids || !topk_ids || !topk_w)
        return fail(MOE_ERR_INVALID, "moe_route_replay: x, router, replay_ids, topk_ids and topk_w are required");
    if (!ws || ws_bytes < route_ws(shape))
        return fail(MOE_ERR_WORKSPACE, "moe_route_replay needs %zu workspace bytes, got %zu", route_ws(shape),
                    ws ? ws_bytes : 0);
    if ((st = check_device()) != MOE_OK) return st;
    double* l64 = static_cast<double*>(ws);
    if ((st = hip_status(moe::launch_route_replay(x, router, shape->T, shape->D, shape->E, shape->K, shape->dtype,
                                                  shape->score, shape->renorm, shape->route_scale, n_group(shape),
                                                  replay_ids, mask,
                                                  l64, logits, topk_ids, topk_w, stream),
                         "routing replay launch")) != MOE_OK)
        return st;
    return ok();
}

moe_status moe_permute(const moe_shape* shape, const int32_t* topk_ids, int32_t* counts, int32_t* offsets,
                       int32_t* perm_token, int32_t* inv_pos, void* ws, size_t ws_bytes, hipStream_t stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    if (!aligned(16, {ws}) || !aligned(4, {topk_ids, counts, offsets, perm_token, inv_pos}))
        return fail(MOE_ERR_INVALID, "moe_permute: ws must be 16-byte aligned, the int32 arrays 4-byte");
    if (shape->T == 0) return ok();
    if (!topk_ids || !counts || !offsets || !perm_token || !inv_pos)
        return fail(MOE_ERR_INVALID, "moe_permute: topk_ids, counts, offsets, perm_token and inv_pos are required");
    if (!ws || ws_bytes < permute_ws(shape))
        return fail(MOE_ERR_WORKSPACE, "moe_permute needs %zu workspace bytes, got %zu", permute_ws(shape), ws ? ws_bytes : 0);
    if ((st = check_device()) != MOE_OK) return st;
    if ((st = hip_status(moe::launch_permute(topk_ids, shape->T, shape->K, shape->E, static_cast<int32_t*>(ws), counts,
                                             offsets, perm_token, inv_pos, stream),
                         "permute launch")) != MOE_OK)
        return st;
    return ok();
}

// The routed-expert MLP: the skinny kernels when groups hold few rows on
// average (decode-sized batches), the tiled persistent kernels otherwise.
// Both compute every element by the same MFMA chain and rounding, so the
// choice never changes a result.
static hipError_t run_experts(const void* x, int64_t x_rows, const int32_t* perm, const int32_t* offsets, int G,
                              int64_t rows, int D, int I, int dtype, const void* gate_up, const void* down, void* y,
                              void* ws, hipStream_t stream) {
    if (moe::experts_use_skinny(rows, G, dtype))
        return moe::launch_experts_skinny(x, perm, offsets, G, rows, D, I, gate_up, down, y, ws, stream);
    return moe::launch_experts(x, x_rows, perm, offsets, G, rows, D, I, dtype, gate_up, down, y, ws, stream);
}

moe_status moe_experts(const moe_shape* shape, const void* x, const int32_t* perm_token, const int32_t* offsets,
                       const void* gate_up, const void* down, void* y, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    if (!aligned(16, {x, gate_up, down, y, ws}) || !aligned(4, {perm_token, offsets}))
        return fail(MOE_ERR_INVALID, "moe_experts: x, gate_up, down, y and ws must be 16-byte aligned, the int32 arrays 4-byte");
    if (shape->T == 0) return ok();
    if (!x || !gate_up || !down || !y) return fail(MOE_ERR_INVALID, "moe_experts: x, gate_up, down and y are required");
    if (offsets == nullptr && shape->E != 1)
        return fail(MOE_ERR_INVALID, "moe_experts: offsets may be NULL only for a single group (E == 1)");
    if (!ws || ws_bytes < experts_ws(shape))
        return fail(MOE_ERR_WORKSPACE, "moe_experts needs %zu workspace bytes, got %zu", experts_ws(shape), ws ? ws_bytes : 0);
    if ((st = check_device()) != MOE_OK) return st;
    const int64_t rows = shape->T * shape->K;
    const int64_t x_rows = perm_token != nullptr ? shape->T : rows;
    if ((st = hip_status(run_experts(x, x_rows, perm_token, offsets, shape->E, rows, shape->D, shape->I,
                                             shape->dtype, gate_up, down, y, ws, stream),
                         "experts launch")) != MOE_OK)
        return st;
    return ok();
}

moe_status moe_combine(const moe_shape* shape, const void* y, const int32_t* inv_pos, const float* topk_w,
                       const void* shared_out, int32_t out_dtype, void* out, hipStream_t stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    if (!aligned(16, {y, shared_out, out}) || !aligned(4, {inv_pos, topk_w}))
        return fail(MOE_ERR_INVALID, "moe_combine: y, shared_out and out must be 16-byte aligned, inv_pos and topk_w 4-byte");
    if (out_dtype != MOE_BF16 && out_dtype != MOE_F32) return fail(MOE_ERR_INVALID, "unknown out_dtype %d", out_dtype);
    if (shape->T == 0) return ok();
    if (!y || !inv_pos || !topk_w || !out) return fail(MOE_ERR_INVALID, "moe_combine: y, inv_pos, topk_w and out are required");
    if ((st = check_device()) != MOE_OK) return st;
    if ((st = hip_status(moe::launch_combine(y, inv_pos, topk_w, shared_out, shape->T, shape->D, shape->K, shape->dtype,
                                             out_dtype, shape->combine, out, stream),
                         "combine launch")) != MOE_OK)
        return st;
    return ok();
}

// The argument checks of the forward entry points, before any device call.
static moe_status check_forward_args(const moe_shape* shape, const moe_weights* weights, const void* x,
                                     const float* sel_bias, const int32_t* replay_ids, int32_t out_dtype,
                                     const void* out, const moe_trace* trace, const void* ws) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    if (!weights) return fail(MOE_ERR_INVALID, "moe_forward: weights are required");
    if (!weights->router || !weights->gate_up || !weights->down)
        return fail(MOE_ERR_INVALID, "moe_forward: router, gate_up and down weights are required");
    if (shape->Is > 0 && (!weights->gate_up_shared || !weights->down_shared))
        return fail(MOE_ERR_INVALID, "moe_forward: Is > 0 needs gate_up_shared and down_shared");
    if (out_dtype != MOE_BF16 && out_dtype != MOE_F32) return fail(MOE_ERR_INVALID, "unknown out_dtype %d", out_dtype);
    {
        moe_trace t{};
        if (trace) t = *trace;
        if (!aligned(16, {x, out, ws, weights->router, weights->gate_up, weights->down, weights->gate_up_shared,
                          weights->down_shared, t.y, t.shared_out}) ||
            !aligned(4, {sel_bias, replay_ids, t.logits, t.topk_ids, t.topk_w, t.counts, t.offsets, t.perm_token,
                         t.inv_pos}))
            return fail(MOE_ERR_INVALID,
                        "moe_forward: x, out, ws, the weights and the trace's y and shared_out must be 16-byte "
                        "aligned, the other arrays 4-byte");
    }
    if (shape->T > 0 && (!x || !out)) return fail(MOE_ERR_INVALID, "moe_forward: x and out are required");
    return MOE_OK;
}

static moe_status forward_impl(const moe_shape* shape, const moe_weights* weights, const void* x,
                               const float* sel_bias, const int32_t* replay_ids, const uint8_t* mask,
                               int32_t out_dtype, void* out, const moe_trace* trace, void* ws, size_t ws_bytes,
                               hipStream_t stream) {
    moe_status st = check_forward_args(shape, weights, x, sel_bias, replay_ids, out_dtype, out, trace, ws);
    if (st != MOE_OK) return st;
    if (shape->T == 0) return ok();
    const ForwardLayout L = forward_layout(shape);
    if (!ws || ws_bytes < L.total)
        return fail(MOE_ERR_WORKSPACE, "moe_forward needs %zu workspace bytes, got %zu", L.total, ws ? ws_bytes : 0);
    if ((st = check_device()) != MOE_OK) return st;

    uint8_t* base = static_cast<uint8_t*>(ws);
    moe_trace tr{};
    if (trace) tr = *trace;
    double* l64 = reinterpret_cast<double*>(base + L.logits64);
    int32_t* ids = tr.topk_ids ? tr.topk_ids : reinterpret_cast<int32_t*>(base + L.ids);
    float* tw = tr.topk_w ? tr.topk_w : reinterpret_cast<float*>(base + L.w);
    int32_t* counts = tr.counts ? tr.counts : reinterpret_cast<int32_t*>(base + L.counts);
    int32_t* offsets = tr.offsets ? tr.offsets : reinterpret_cast<int32_t*>(base + L.offsets);
    int32_t* perm = tr.perm_token ? tr.perm_token : reinterpret_cast<int32_t*>(base + L.perm);
    int32_t* inv = tr.inv_pos ? tr.inv_pos : reinterpret_cast<int32_t*>(base + L.inv);
    void* y = tr.y ? tr.y : static_cast<void*>(base + L.y);
    void* sh = shape->Is > 0 ? (tr.shared_out ? tr.shared_out : static_cast<void*>(base + L.shared)) : nullptr;
    void* exw = base + L.exp_ws;
    const int64_t T = shape->T;

    if (moe::route_permute_fused(T)) {
        // decode-sized batch: top-k and the permutation in one launch (a
        // replay takes the given ids and no selection bias; the layer's
        // n_group still selects the top-k code of its forward)
        const bool rp = replay_ids != nullptr;
        if ((st = hip_status(moe::launch_route_permute(
                                 x, weights->router, T, shape->D, shape->E, shape->K, shape->dtype, shape->score,
                                 shape->renorm, shape->route_scale, n_group(shape), shape->topk_group,
                                 rp ? nullptr : sel_bias, replay_ids, mask, l64, tr.logits, ids, tw, counts, offsets,
                                 perm, inv, stream),
                             "routing launch")) != MOE_OK)
            return st;
    } else {
        if (replay_ids != nullptr) {
            if ((st = hip_status(moe::launch_route_replay(x, weights->router, T, shape->D, shape->E, shape->K,
                                                          shape->dtype, shape->score, shape->renorm, shape->route_scale,
                                                          n_group(shape), replay_ids, mask, l64, tr.logits, ids, tw, stream),
                                 "routing replay launch")) != MOE_OK)
                return st;
        } else if ((st = hip_status(moe::launch_route(x, weights->router, T, shape->D, shape->E, shape->K, shape->dtype,
                                                      shape->score, shape->renorm, shape->route_scale, n_group(shape),
                                                      shape->topk_group, sel_bias, mask, l64, tr.logits, ids, tw, stream),
                                    "routing launch")) != MOE_OK) {
            return st;
        }
        if ((st = hip_status(moe::launch_permute(ids, T, shape->K, shape->E, reinterpret_cast<int32_t*>(base + L.perm_ws),
                                                 counts, offsets, perm, inv, stream),
                             "permute launch")) != MOE_OK)
            return st;
    }
    if (T == 1 && shape->dtype == 0 && shape->combine == MOE_COMBINE_F32_FOLD &&
        moe::decode_combine_fits(T, shape->K, shape->Is > 0) && moe::experts_use_skinny(shape->K, shape->E, 0) &&
        (shape->Is == 0 || shared_with_routed(shape))) {
        // one token: the experts' down projections and the combine in one launch
        // (the same bits as the launches below)
        if ((st = hip_status(moe::launch_experts_decode_combine(
                                 x, perm, offsets, shape->E, shape->K, shape->D, shape->I, weights->gate_up,
                                 weights->down, y, exw, shape->Is, weights->gate_up_shared, weights->down_shared, sh,
                                 base + L.shared_act, ids, inv, tw, out_dtype == MOE_F32 ? 1 : 0, out, stream),
                             "experts + combine launch")) != MOE_OK)
            return st;
        return ok();
    }
    if (shared_with_routed(shape)) {
        if ((st = hip_status(moe::launch_experts_skinny_pair(
                                 x, perm, offsets, shape->E, T * shape->K, shape->D, shape->I, weights->gate_up,
                                 weights->down, y, exw, T, shape->Is, weights->gate_up_shared, weights->down_shared,
                                 sh, base + L.shared_act, stream),
                             "experts launch")) != MOE_OK)
            return st;
    } else if ((st = hip_status(run_experts(x, T, perm, offsets, shape->E, T * shape->K, shape->D, shape->I,
                                            shape->dtype, weights->gate_up, weights->down, y, exw, stream),
                                "routed experts launch")) != MOE_OK) {
        return st;
    }
    if (sh != nullptr && !shared_with_routed(shape)) {
        if ((st = hip_status(run_experts(x, T, nullptr, nullptr, 1, T, shape->D, shape->Is, shape->dtype,
                                                 weights->gate_up_shared, weights->down_shared, sh, exw, stream),
                             "shared expert launch")) != MOE_OK)
            return st;
    }
    if ((st = hip_status(moe::launch_combine(y, inv, tw, sh, T, shape->D, shape->K, shape->dtype, out_dtype, shape->combine,
                                             out, stream),
                         "combine launch")) != MOE_OK)
        return st;
    return ok();
}

moe_status moe_forward(const moe_shape* shape, const moe_weights* weights, const void* x, const float* sel_bias,
                       const uint8_t* mask, int32_t out_dtype, void* out, const moe_trace* trace, void* ws,
                       size_t ws_bytes, hipStream_t stream) {
    return forward_impl(shape, weights, x, sel_bias, nullptr, mask, out_dtype, out, trace, ws, ws_bytes, stream);
}

// Scratch of moe_forward_noalloc: one fixed array per device, part of the
// library's device code, so that the call needs no allocation.  Host code
// never uses the array's name as an address (on the host it is a stand-in):
// the device address comes from hipGetSymbolAddress, once per device, with
// that device current.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

static moe_status scratch_address(void** out) {
    static std::mutex mu;
    static void* ptrs[64];
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(err));
    if (dev < 0 || dev >= 64) return fail(MOE_ERR_UNSUPPORTED, "device index %d out of range", dev);
    std::lock_guard<std::mutex> lock(mu);
    if (ptrs[dev] == nullptr) {
        void* p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(err));
        if (p == nullptr) return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        ptrs[dev] = p;
    }
    *out = ptrs[dev];
    return MOE_OK;
}

moe_status moe_forward_noalloc(const moe_shape* shape, const moe_weights* weights, const void* x,
                               const float* sel_bias, const uint8_t* mask, int32_t out_dtype, void* out,
                               const moe_trace* trace, hipStream_t stream) {
    moe_status st = check_forward_args(shape, weights, x, sel_bias, nullptr, out_dtype, out, trace, nullptr);
    if (st != MOE_OK) return st;
    const size_t need = forward_layout(shape).total;
    if (need > kScratchBytes)
        return fail(MOE_ERR_UNSUPPORTED,
                    "moe_forward_noalloc: this shape needs %zu bytes of scratch, above the fixed %zu; "
                    "call moe_forward with a workspace instead",
                    need, kScratchBytes);
    if (shape->T == 0) return ok();
    if ((st = check_device()) != MOE_OK) return st;
    void* ws = nullptr;
    if ((st = scratch_address(&ws)) != MOE_OK) return st;
    return forward_impl(shape, weights, x, sel_bias, nullptr, mask, out_dtype, out, trace, ws, kScratchBytes, stream);
}

moe_status moe_forward_replay(const moe_shape* shape, const moe_weights* weights, const void* x,
                              const int32_t* replay_ids, const uint8_t* mask, int32_t out_dtype, void* out,
                              const moe_trace* trace, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (replay_ids == nullptr && shape != nullptr && shape->T > 0)
        return fail(MOE_ERR_INVALID, "moe_forward_replay: replay_ids is required");
    return forward_impl(shape, weights, x, nullptr, replay_ids, mask, out_dtype, out, trace, ws, ws_bytes, stream);
}

moe_status moe_backward_workspace_size(const moe_shape* shape, size_t* bytes) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    if (bytes == nullptr) return fail(MOE_ERR_INVALID, "bytes is NULL");
    *bytes = moe::backward_ws_bytes(shape->T, shape->D, shape->E, shape->K, shape->I, shape->Is);
    return ok();
}

moe_status moe_backward(const moe_shape* shape, const moe_weights* weights, const void* x, const uint8_t* mask,
                        const moe_trace* fwd, const void* dout, const moe_grads* grads, void* ws, size_t ws_bytes,
                        hipStream_t stream) {
    moe_status st = check_shape(shape);
    if (st != MOE_OK) return st;
    if (shape->dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "moe_backward: bf16 operands only");
    if (!moe::backward_fits_dma(shape->T, shape->D, shape->K, shape->I, shape->Is))
        return fail(MOE_ERR_UNSUPPORTED, "moe_backward: T*K*max(D, 2I) bf16 values must stay below 4 GiB");
    if (!weights || !weights->router || !weights->gate_up || !weights->down)
        return fail(MOE_ERR_INVALID, "moe_backward: router, gate_up and down weights are required");
    if (shape->Is > 0 && (!weights->gate_up_shared || !weights->down_shared))
        return fail(MOE_ERR_INVALID, "moe_backward: Is > 0 needs gate_up_shared and down_shared");
    if (!grads || !grads->d_router || !grads->d_gate_up || !grads->d_down)
        return fail(MOE_ERR_INVALID, "moe_backward: d_router, d_gate_up and d_down are required");
    if (shape->Is > 0 && (!grads->d_gate_up_shared || !grads->d_down_shared))
        return fail(MOE_ERR_INVALID, "moe_backward: Is > 0 needs d_gate_up_shared and d_down_shared");
    moe_trace t{};
    if (fwd) t = *fwd;
    if (!aligned(16, {x, dout, ws, weights->router, weights->gate_up, weights->down, weights->gate_up_shared,
                      weights->down_shared, t.y, grads->dx, grads->d_router, grads->d_gate_up, grads->d_down,
                      grads->d_gate_up_shared, grads->d_down_shared}) ||
        !aligned(4, {t.topk_ids, t.topk_w, t.offsets, t.perm_token, t.inv_pos}))
        return fail(MOE_ERR_INVALID,
                    "moe_backward: x, dout, ws, the weights, the trace's y and the gradients must be 16-byte "
                    "aligned, the trace's index and weight arrays 4-byte");
    if (shape->T > 0) {
        if (!x || !dout || !grads->dx) return fail(MOE_ERR_INVALID, "moe_backward: x, dout and dx are required");
        if (!fwd || !t.topk_ids || !t.topk_w || !t.offsets || !t.perm_token || !t.inv_pos || !t.y)
            return fail(MOE_ERR_INVALID,
                        "moe_backward: the forward trace needs topk_ids, topk_w, offsets, perm_token, inv_pos and y");
        const size_t need = moe::backward_ws_bytes(shape->T, shape->D, shape->E, shape->K, shape->I, shape->Is);
        if (!ws || ws_bytes < need)
            return fail(MOE_ERR_WORKSPACE, "moe_backward needs %zu workspace bytes, got %zu", need, ws ? ws_bytes : 0);
    }
    if ((st = check_device()) != MOE_OK) return st;
    moe::BwdArgs a{};
    a.T = shape->T;
    a.D = shape->D;
    a.E = shape->E;
    a.K = shape->K;
    a.I = shape->I;
    a.Is = shape->Is;
    a.score = shape->score;
    a.renorm = shape->renorm;
    a.route_scale = shape->route_scale;
    a.x = x;
    a.router = weights->router;
    a.gate_up = weights->gate_up;
    a.down = weights->down;
    a.gate_up_shared = weights->gate_up_shared;
    a.down_shared = weights->down_shared;
    a.dout = dout;
    a.y = t.y;
    a.topk_ids = t.topk_ids;
    a.offsets = t.offsets;
    a.perm_token = t.perm_token;
    a.inv_pos = t.inv_pos;
    a.topk_w = t.topk_w;
    a.mask = mask;
    a.dx = grads->dx;
    a.d_router = grads->d_router;
    a.d_gate_up = grads->d_gate_up;
    a.d_down = grads->d_down;
    a.d_gate_up_shared = grads->d_gate_up_shared;
    a.d_down_shared = grads->d_down_shared;
    a.ws = ws;
    if (shape->T == 0) {
        if ((st = hip_status(moe::launch_backward_empty(a, stream), "backward launch")) != MOE_OK) return st;
        return ok();
    }
    if ((st = hip_status(moe::launch_backward(a, stream), "backward launch")) != MOE_OK) return st;
    return ok();
}

}  // extern "C"
