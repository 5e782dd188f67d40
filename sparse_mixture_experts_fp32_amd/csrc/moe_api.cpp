// C ABI of the routed MoE FFN forward pass: argument checks, workspace layout
// and kernel launches on the caller's stream. No allocation, no host sync.
#include "moe.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "launch.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int ok() {
    g_last_error.clear();
    return MOE_OK;
}

int hip_status(hipError_t err, const char* where) {
    if (err == hipSuccess) return ok();
    return fail(MOE_ERR_HIP, "%s: %s", where, hipGetErrorString(err));
}

constexpr size_t kWsAlign = 256;

size_t align_up(size_t v) { return (v + kWsAlign - 1) / kWsAlign * kWsAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_shape(const moe_shape_t* s) {
    if (s == nullptr) return fail(MOE_ERR_INVALID_ARG, "shape is NULL");
    if (s->T < 0) return fail(MOE_ERR_INVALID_ARG, "T = %lld < 0", static_cast<long long>(s->T));
    if (s->E < 1 || s->E > 1024) return fail(MOE_ERR_INVALID_ARG, "E = %d outside [1, 1024]", s->E);
    if (s->k < 1 || s->k > s->E || s->k > 64)
        return fail(MOE_ERR_INVALID_ARG, "k = %d outside [1, min(E, 64)] (E = %d)", s->k, s->E);
    if (s->d < 128 || s->d % 128 != 0 || s->d > (1 << 20))
        return fail(MOE_ERR_INVALID_ARG, "d = %d is not a positive multiple of 128 (<= 2^20)", s->d);
    if (s->h < 128 || s->h % 128 != 0 || s->h > (1 << 20))
        return fail(MOE_ERR_INVALID_ARG, "h = %d is not a positive multiple of 128 (<= 2^20)", s->h);
    if (s->T * static_cast<int64_t>(s->k) >= (int64_t(1) << 31))
        return fail(MOE_ERR_UNSUPPORTED, "T * k = %lld >= 2^31", static_cast<long long>(s->T * s->k));
    if ((s->T + 3) / 4 >= (int64_t(1) << 31) || (s->T + 63) / 64 > 65535)
        return fail(MOE_ERR_UNSUPPORTED, "T = %lld too large for one launch", static_cast<long long>(s->T));
    return MOE_OK;
}

#define MOE_CHECK_PTR(p)                                                               \
    do {                                                                               \
        if ((p) == nullptr) return fail(MOE_ERR_INVALID_ARG, "%s is NULL", #p);        \
        if (!aligned16(p)) return fail(MOE_ERR_INVALID_ARG, "%s is not 16-byte aligned", #p); \
    } while (0)

int check_ws(void* ws, size_t ws_bytes, size_t need) {
    if (need == 0) return MOE_OK;
    if (ws == nullptr) return fail(MOE_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
    if ((reinterpret_cast<uintptr_t>(ws) & (kWsAlign - 1)) != 0)
        return fail(MOE_ERR_WORKSPACE, "workspace is not %zu-byte aligned", kWsAlign);
    if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, need);
    return MOE_OK;
}

size_t permute_ws(const moe_shape_t* s) {
    const int64_t n = s->T * s->k;
    if (n == 0) return 0;
    return align_up(sizeof(int32_t) * static_cast<size_t>(s->E) * moe::permute_nchunks(n));
}

size_t route_ws(const moe_shape_t* s) {
    if (s->T == 0) return 0;
    return align_up(moe::router_parts_bytes(s->d, s->E));
}

// The grouped GEMM's workspace: the m-tile list, then each expert's first m-tile index.
size_t ffn_tiles_bytes(const moe_shape_t* s) {
    return align_up(sizeof(int4) * static_cast<size_t>(moe::ffn_max_tiles(s->T * s->k, s->E)));
}

size_t ffn_ws(const moe_shape_t* s) {
    const int64_t n = s->T * s->k;
    if (n == 0) return 0;
    return ffn_tiles_bytes(s) + align_up(sizeof(int32_t) * (static_cast<size_t>(s->E) + 1));
}

size_t aux_ws(const moe_shape_t* s) {
    if (s->T == 0) return 0;
    return align_up(moe::aux_ws_bytes(s->T, s->E));
}

// Quantile Balancing selects k + 1 experts per token with one wavefront.
int check_qb_shape(const moe_shape_t* s) {
    int st = check_shape(s);
    if (st != MOE_OK) return st;
    if (s->k >= s->E || s->k > 63)
        return fail(MOE_ERR_INVALID_ARG, "Quantile Balancing needs k < E and k <= 63 (k = %d, E = %d)", s->k, s->E);
    return MOE_OK;
}

int check_bins(float lo, float width, int32_t n_bins) {
    if (!std::isfinite(lo)) return fail(MOE_ERR_INVALID_ARG, "lo is not finite");
    if (!std::isfinite(width) || !(width > 0.f)) return fail(MOE_ERR_INVALID_ARG, "width must be finite and > 0");
    if (n_bins < 1 || n_bins > moe::qb_max_bins())
        return fail(MOE_ERR_INVALID_ARG, "n_bins = %d outside [1, %d]", n_bins, moe::qb_max_bins());
    return MOE_OK;
}

struct FfnWs {
    int4* tiles;
    int32_t* tile_start;
};

FfnWs ffn_carve(const moe_shape_t* s, void* ws) {
    char* b = static_cast<char*>(ws);
    return FfnWs{reinterpret_cast<int4*>(b), reinterpret_cast<int32_t*>(b + ffn_tiles_bytes(s))};
}

// Byte offsets of every slot of moe_forward's workspace; after the public slots
// come the permute scratch, the tile list and the router's weight parts, then
// the total.
constexpr int kFwdPermuteWs = MOE_FWD_NUM_SLOTS, kFwdFfnWs = MOE_FWD_NUM_SLOTS + 1,
              kFwdRouteWs = MOE_FWD_NUM_SLOTS + 2, kFwdTotal = MOE_FWD_NUM_SLOTS + 3;

void forward_layout(const moe_shape_t* s, size_t off[kFwdTotal + 1]) {
    const size_t T = static_cast<size_t>(s->T), E = s->E, k = s->k, d = s->d, h = s->h;
    const size_t sizes[kFwdTotal] = {
        4 * T * E, 4 * T * k, 4 * T * k, 4 * (E + 1), 4 * T * k, 4 * T * k,
        2 * T * k * h, 4 * T * k * d, permute_ws(s), ffn_ws(s), route_ws(s)};
    size_t at = 0;
    for (int i = 0; i < kFwdTotal; ++i) {
        off[i] = at;
        at += align_up(sizes[i]);
    }
    off[kFwdTotal] = at;
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_str(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported size";
        case MOE_ERR_WORKSPACE: return "workspace too small";
        case MOE_ERR_HIP: return "HIP error";
        default: return "unknown status";
    }
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

size_t moe_workspace_bytes(const moe_shape_t* shape, int call) {
    if (check_shape(shape) != MOE_OK) return 0;
    switch (call) {
        case MOE_CALL_PERMUTE: ok(); return permute_ws(shape);
        case MOE_CALL_EXPERT_FFN: ok(); return ffn_ws(shape);
        case MOE_CALL_ROUTE: ok(); return route_ws(shape);
        case MOE_CALL_AUX_LOSS: ok(); return aux_ws(shape);
        case MOE_CALL_FORWARD: {
            size_t off[kFwdTotal + 1];
            forward_layout(shape, off);
            ok();
            return off[kFwdTotal];
        }
        default: fail(MOE_ERR_INVALID_ARG, "unknown call %d", call); return 0;
    }
}

int moe_forward_ws_offset(const moe_shape_t* shape, int slot, size_t* offset) {
    int st = check_shape(shape);
    if (st != MOE_OK) return st;
    if (slot < 0 || slot >= MOE_FWD_NUM_SLOTS) return fail(MOE_ERR_INVALID_ARG, "unknown slot %d", slot);
    if (offset == nullptr) return fail(MOE_ERR_INVALID_ARG, "offset is NULL");
    size_t off[kFwdTotal + 1];
    forward_layout(shape, off);
    *offset = off[slot];
    return ok();
}

int moe_route(const moe_shape_t* shape, const uint16_t* x, const float* w_router, const float* router_bias,
              float* logits, int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes, void* stream) {
    int st = check_shape(shape);
    if (st != MOE_OK) return st;
    if (shape->T == 0) return ok();
    MOE_CHECK_PTR(x);
    MOE_CHECK_PTR(w_router);
    if (router_bias != nullptr && !aligned16(router_bias))
        return fail(MOE_ERR_INVALID_ARG, "router_bias is not 16-byte aligned");
    MOE_CHECK_PTR(logits);
    MOE_CHECK_PTR(topk_idx);
    MOE_CHECK_PTR(topk_w);
    st = check_ws(ws, ws_bytes, route_ws(shape));
    if (st != MOE_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t err = moe::launch_router_gemm(x, w_router, router_bias, logits, shape->T, shape->d, shape->E,
                                             static_cast<uint16_t*>(ws), s);
    if (err != hipSuccess) return hip_status(err, "router_gemm launch");
    err = moe::launch_topk_softmax(logits, shape->T, shape->E, shape->k, topk_idx, topk_w, s);
    return hip_status(err, "topk_softmax launch");
}

int moe_topk_softmax(const moe_shape_t* shape, const float* logits, int32_t* topk_idx, float* topk_w,
                     void* stream) {
    int st = check_shape(shape);
    if (st != MOE_OK) return st;
    if (shape->T == 0) return ok();
    MOE_CHECK_PTR(logits);
    MOE_CHECK_PTR(topk_idx);
    MOE_CHECK_PTR(topk_w);
    hipError_t err = moe::launch_topk_softmax(logits, shape->T, shape->E, shape->k, topk_idx, topk_w,
                                              static_cast<hipStream_t>(stream));
    return hip_status(err, "topk_softmax launch");
}

int moe_permute(const moe_shape_t* shape, const uint16_t* x, const int32_t* topk_idx, int32_t* expert_offsets,
                int32_t* row_of, int32_t* row_src, uint16_t* x_perm, void* ws, size_t ws_bytes, void* stream) {
    int st = check_shape(shape);
    if (st != MOE_OK) return st;
    MOE_CHECK_PTR(expert_offsets);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (shape->T == 0) {  // still a valid empty grouping: all offsets are 0
        hipError_t err = moe::launch_zero_i32(expert_offsets, shape->E + 1, s);
        return hip_status(err, "expert_offsets clear");
    }
    MOE_CHECK_PTR(topk_idx);
    MOE_CHECK_PTR(row_of);
    MOE_CHECK_PTR(row_src);
    if (x_perm != nullptr) {  // x is only read by the gather
        MOE_CHECK_PTR(x);
        if (!aligned16(x_perm)) return fail(MOE_ERR_INVALID_ARG, "x_perm is not 16-byte aligned");
    }
    st = check_ws(ws, ws_bytes, permute_ws(shape));
    if (st != MOE_OK) return st;
    hipError_t err = moe::launch_permute(x, topk_idx, shape->T, shape->d, shape->E, shape->k, expert_offsets,
                                         row_of, row_src, x_perm, static_cast<int32_t*>(ws), s);
    return hip_status(err, "permute launch");
}

int moe_expert_ffn(const moe_shape_t* shape, const uint16_t* a, const int32_t* a_rows,
                   const int32_t* expert_offsets, const uint16_t* w_gate, const uint16_t* w_up,
                   const uint16_t* w_down, uint16_t* h_act, float* y_rows, void* ws, size_t ws_bytes, void* stream) {
    int st = check_shape(shape);
    if (st != MOE_OK) return st;
    if (shape->T == 0) return ok();
    MOE_CHECK_PTR(a);
    if (a_rows != nullptr && !aligned16(a_rows)) return fail(MOE_ERR_INVALID_ARG, "a_rows is not 16-byte aligned");
    MOE_CHECK_PTR(expert_offsets);
    MOE_CHECK_PTR(w_gate);
    MOE_CHECK_PTR(w_up);
    MOE_CHECK_PTR(w_down);
    MOE_CHECK_PTR(h_act);
    MOE_CHECK_PTR(y_rows);
    st = check_ws(ws, ws_bytes, ffn_ws(shape));
    if (st != MOE_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t n = shape->T * shape->k;
    const FfnWs fw = ffn_carve(shape, ws);
    hipError_t err = moe::launch_build_tiles(expert_offsets, n, shape->E, fw.tiles, fw.tile_start, s);
    if (err != hipSuccess) return hip_status(err, "build_tiles launch");
    err = moe::launch_gate_up(a, a_rows, shape->T, fw.tiles, fw.tile_start, n, shape->d, shape->E, shape->h,
                              w_gate, w_up, h_act, s);
    if (err != hipSuccess) return hip_status(err, "gate_up launch");
    err = moe::launch_down(h_act, fw.tiles, fw.tile_start, n, shape->d, shape->E, shape->h, w_down, y_rows, s);
    return hip_status(err, "down launch");
}

int moe_expert_gate_up(const moe_shape_t* shape, const uint16_t* a, const int32_t* a_rows,
                       const int32_t* expert_offsets, const uint16_t* w_gate, const uint16_t* w_up, uint16_t* h_act,
                       void* ws, size_t ws_bytes, void* stream) {
    int st = check_shape(shape);
    if (st != MOE_OK) return st;
    if (shape->T == 0) return ok();
    MOE_CHECK_PTR(a);
    if (a_rows != nullptr && !aligned16(a_rows)) return fail(MOE_ERR_INVALID_ARG, "a_rows is not 16-byte aligned");
    MOE_CHECK_PTR(expert_offsets);
    MOE_CHECK_PTR(w_gate);
    MOE_CHECK_PTR(w_up);
    MOE_CHECK_PTR(h_act);
    st = check_ws(ws, ws_bytes, ffn_ws(shape));
    if (st != MOE_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t n = shape->T * shape->k;
    const FfnWs fw = ffn_carve(shape, ws);
    hipError_t err = moe::launch_build_tiles(expert_offsets, n, shape->E, fw.tiles, fw.tile_start, s);
    if (err != hipSuccess) return hip_status(err, "build_tiles launch");
    err = moe::launch_gate_up(a, a_rows, shape->T, fw.tiles, fw.tile_start, n, shape->d, shape->E, shape->h,
                              w_gate, w_up, h_act, s);
    return hip_status(err, "gate_up launch");
}

int moe_expert_down(const moe_shape_t* shape, const uint16_t* h_act, const int32_t* expert_offsets,
                    const uint16_t* w_down, float* y_rows, void* ws, size_t ws_bytes, void* stream) {
    int st = check_shape(shape);
    if (st != MOE_OK) return st;
    if (shape->T == 0) return ok();
    MOE_CHECK_PTR(h_act);
    MOE_CHECK_PTR(expert_offsets);
    MOE_CHECK_PTR(w_down);
    MOE_CHECK_PTR(y_rows);
    st = check_ws(ws, ws_bytes, ffn_ws(shape));
    if (st != MOE_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t n = shape->T * shape->k;
    const FfnWs fw = ffn_carve(shape, ws);
    hipError_t err = moe::launch_build_tiles(expert_offsets, n, shape->E, fw.tiles, fw.tile_start, s);
    if (err != hipSuccess) return hip_status(err, "build_tiles launch");
    err = moe::launch_down(h_act, fw.tiles, fw.tile_start, n, shape->d, shape->E, shape->h, w_down, y_rows, s);
    return hip_status(err, "down launch");
}

int moe_combine(const moe_shape_t* shape, const float* y_rows, const int32_t* row_of, const float* topk_w,
                float* out, void* stream) {
    int st = check_shape(shape);
    if (st != MOE_OK) return st;
    if (shape->T == 0) return ok();
    MOE_CHECK_PTR(y_rows);
    MOE_CHECK_PTR(row_of);
    MOE_CHECK_PTR(topk_w);
    MOE_CHECK_PTR(out);
    hipError_t err = moe::launch_combine(y_rows, row_of, topk_w, shape->T, shape->d, shape->k,
                                         shape->T * shape->k, out, static_cast<hipStream_t>(stream));
    return hip_status(err, "combine launch");
}

int moe_aux_loss(const moe_shape_t* shape, const float* logits, float* prob_mean, float* aux_loss, void* ws,
                 size_t ws_bytes, void* stream) {
    int st = check_shape(shape);
    if (st != MOE_OK) return st;
    if (shape->T == 0) return ok();
    MOE_CHECK_PTR(logits);
    MOE_CHECK_PTR(prob_mean);
    MOE_CHECK_PTR(aux_loss);
    st = check_ws(ws, ws_bytes, aux_ws(shape));
    if (st != MOE_OK) return st;
    hipError_t err = moe::launch_aux_loss(logits, shape->T, shape->E, prob_mean, aux_loss, ws,
                                          static_cast<hipStream_t>(stream));
    return hip_status(err, "aux_loss launch");
}

int moe_qb_route(const moe_shape_t* shape, const float* logits, const float* qb_bias, int32_t* topk_idx,
                 float* topk_w, float* alpha, void* stream) {
    int st = check_qb_shape(shape);
    if (st != MOE_OK) return st;
    if (shape->T == 0) return ok();
    MOE_CHECK_PTR(logits);
    MOE_CHECK_PTR(qb_bias);
    MOE_CHECK_PTR(topk_idx);
    MOE_CHECK_PTR(topk_w);
    MOE_CHECK_PTR(alpha);
    hipError_t err = moe::launch_qb_select(logits, qb_bias, shape->T, shape->E, shape->k, topk_idx, topk_w, alpha,
                                           static_cast<hipStream_t>(stream));
    return hip_status(err, "qb_select launch");
}

int moe_qb_histogram(const moe_shape_t* shape, const float* logits, const float* alpha, float lo, float width,
                     int32_t n_bins, int32_t* hist, void* stream) {
    int st = check_qb_shape(shape);
    if (st != MOE_OK) return st;
    st = check_bins(lo, width, n_bins);
    if (st != MOE_OK) return st;
    MOE_CHECK_PTR(hist);
    if (shape->T > 0) {
        MOE_CHECK_PTR(logits);
        MOE_CHECK_PTR(alpha);
    }
    hipError_t err = moe::launch_qb_histogram(logits, alpha, shape->T, shape->E, lo, width, n_bins, hist,
                                              static_cast<hipStream_t>(stream));
    return hip_status(err, "qb_histogram launch");
}

int moe_qb_update(const moe_shape_t* shape, const int32_t* hist, float lo, float width, int32_t n_bins,
                  const float* bias_in, float* bias_out, void* stream) {
    int st = check_qb_shape(shape);
    if (st != MOE_OK) return st;
    st = check_bins(lo, width, n_bins);
    if (st != MOE_OK) return st;
    MOE_CHECK_PTR(hist);
    MOE_CHECK_PTR(bias_in);
    MOE_CHECK_PTR(bias_out);
    hipError_t err = moe::launch_qb_update(hist, shape->E, shape->k, n_bins, lo, width, bias_in, bias_out,
                                           static_cast<hipStream_t>(stream));
    return hip_status(err, "qb_update launch");
}

int moe_forward(const moe_shape_t* shape, const uint16_t* x, const float* w_router, const float* router_bias,
                const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down, float* out, void* ws,
                size_t ws_bytes, void* stream) {
    int st = check_shape(shape);
    if (st != MOE_OK) return st;
    if (shape->T == 0) return ok();
    MOE_CHECK_PTR(x);
    MOE_CHECK_PTR(w_router);
    if (router_bias != nullptr && !aligned16(router_bias))
        return fail(MOE_ERR_INVALID_ARG, "router_bias is not 16-byte aligned");
    MOE_CHECK_PTR(w_gate);
    MOE_CHECK_PTR(w_up);
    MOE_CHECK_PTR(w_down);
    MOE_CHECK_PTR(out);
    size_t off[kFwdTotal + 1];
    forward_layout(shape, off);
    st = check_ws(ws, ws_bytes, off[kFwdTotal]);
    if (st != MOE_OK) return st;
    char* base = static_cast<char*>(ws);
    auto at = [&](int slot) { return static_cast<void*>(base + off[slot]); };
    float* logits = static_cast<float*>(at(MOE_FWD_LOGITS));
    int32_t* idx = static_cast<int32_t*>(at(MOE_FWD_TOPK_IDX));
    float* w = static_cast<float*>(at(MOE_FWD_TOPK_W));
    int32_t* offsets = static_cast<int32_t*>(at(MOE_FWD_EXPERT_OFFSETS));
    int32_t* row_of = static_cast<int32_t*>(at(MOE_FWD_ROW_OF));
    int32_t* row_src = static_cast<int32_t*>(at(MOE_FWD_ROW_SRC));
    uint16_t* h_act = static_cast<uint16_t*>(at(MOE_FWD_H));
    float* y_rows = static_cast<float*>(at(MOE_FWD_Y));
    int32_t* count_ws = static_cast<int32_t*>(at(kFwdPermuteWs));
    const FfnWs fw = ffn_carve(shape, at(kFwdFfnWs));
    uint16_t* router_parts = static_cast<uint16_t*>(at(kFwdRouteWs));
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t T = shape->T, n = shape->T * shape->k;
    const int d = shape->d, E = shape->E, k = shape->k, h = shape->h;

    hipError_t err = moe::launch_router_gemm(x, w_router, router_bias, logits, T, d, E, router_parts, s);
    if (err != hipSuccess) return hip_status(err, "router_gemm launch");
    err = moe::launch_topk_softmax(logits, T, E, k, idx, w, s);
    if (err != hipSuccess) return hip_status(err, "topk_softmax launch");
    // the dispatch gather is fused into the gate/up pass: it reads x through row_src
    err = moe::launch_permute(x, idx, T, d, E, k, offsets, row_of, row_src, nullptr, count_ws, s);
    if (err != hipSuccess) return hip_status(err, "permute launch");
    err = moe::launch_build_tiles(offsets, n, E, fw.tiles, fw.tile_start, s);
    if (err != hipSuccess) return hip_status(err, "build_tiles launch");
    err = moe::launch_gate_up(x, row_src, T, fw.tiles, fw.tile_start, n, d, E, h, w_gate, w_up, h_act, s);
    if (err != hipSuccess) return hip_status(err, "gate_up launch");
    err = moe::launch_down(h_act, fw.tiles, fw.tile_start, n, d, E, h, w_down, y_rows, s);
    if (err != hipSuccess) return hip_status(err, "down launch");
    err = moe::launch_combine(y_rows, row_of, w, T, d, k, n, out, s);
    return hip_status(err, "combine launch");
}

}  // extern "C"
