// C ABI of the routed MoE FFN forward pass: argument checks, workspace layout
// and kernel launches on the caller's stream. No allocation, no host sync.
#include "moe.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
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
    return align_up(moe::router_ws_bytes(s->T, s->d, s->E));
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

// Grouped-GEMM workspace for n_rows rows over E groups: m-tile list, then first m-tile per group.
size_t ffn_ws_rows(int64_t n_rows, int E) {
    if (n_rows == 0) return 0;
    return align_up(sizeof(int4) * static_cast<size_t>(moe::ffn_max_tiles(n_rows, E))) +
           align_up(sizeof(int32_t) * (static_cast<size_t>(E) + 1));
}

struct FfnWs {
    int4* tiles;
    int32_t* tile_start;
};

FfnWs ffn_carve(const moe_shape_t* s, void* ws) {
    char* b = static_cast<char*>(ws);
    return FfnWs{reinterpret_cast<int4*>(b), reinterpret_cast<int32_t*>(b + ffn_tiles_bytes(s))};
}

FfnWs ffn_carve_rows(int64_t n_rows, int E, void* ws) {
    char* b = static_cast<char*>(ws);
    const size_t tiles = align_up(sizeof(int4) * static_cast<size_t>(moe::ffn_max_tiles(n_rows, E)));
    return FfnWs{reinterpret_cast<int4*>(b), reinterpret_cast<int32_t*>(b + tiles)};
}

// ------------------------------------------------------------ LatentMoE

int check_latent_shape(const moe_latent_shape_t* s) {
    if (s == nullptr) return fail(MOE_ERR_INVALID_ARG, "shape is NULL");
    // the routed path is a plain routed layer of width l
    const moe_shape_t r{s->T, s->l, s->E, s->k, s->h};
    int st = check_shape(&r);
    if (st != MOE_OK) return st;
    if (s->d < 128 || s->d % 128 != 0 || s->d > (1 << 20))
        return fail(MOE_ERR_INVALID_ARG, "d = %d is not a positive multiple of 128 (<= 2^20)", s->d);
    if (s->l > moe::combine_rmsnorm_max_width())
        return fail(MOE_ERR_UNSUPPORTED, "l = %d > %d", s->l, moe::combine_rmsnorm_max_width());
    if (s->n_shared < 0 || s->n_shared > 8)
        return fail(MOE_ERR_INVALID_ARG, "n_shared = %d outside [0, 8]", s->n_shared);
    if (s->n_shared > 0 && (s->h_shared < 128 || s->h_shared % 128 != 0 || s->h_shared > (1 << 20)))
        return fail(MOE_ERR_INVALID_ARG, "h_shared = %d is not a positive multiple of 128 (<= 2^20)", s->h_shared);
    if (s->T * static_cast<int64_t>(s->n_shared) >= (int64_t(1) << 31))
        return fail(MOE_ERR_UNSUPPORTED, "n_shared * T >= 2^31");
    return MOE_OK;
}

// slots: the public intermediates, then the permute scratch, the routed / dense /
// shared tile lists, the row maps and the router's weight parts
constexpr int kLatPermuteWs = MOE_LAT_NUM_SLOTS, kLatFfnWs = MOE_LAT_NUM_SLOTS + 1,
              kLatDenseWs = MOE_LAT_NUM_SLOTS + 2, kLatSharedWs = MOE_LAT_NUM_SLOTS + 3,
              kLatMaps = MOE_LAT_NUM_SLOTS + 4, kLatRouteWs = MOE_LAT_NUM_SLOTS + 5,
              kLatTotal = MOE_LAT_NUM_SLOTS + 6;

int latent_groups(const moe_latent_shape_t* s) { return s->n_shared > 0 ? s->n_shared : 1; }

// row maps: dense offsets [2], shared offsets [S + 1], shared rows [S * T]
size_t maps_shared_off(const moe_latent_shape_t*) { return align_up(2 * sizeof(int32_t)); }
size_t maps_shared_rows(const moe_latent_shape_t* s) {
    return maps_shared_off(s) + align_up(sizeof(int32_t) * (static_cast<size_t>(s->n_shared) + 1));
}

void latent_layout(const moe_latent_shape_t* s, size_t off[kLatTotal + 1]) {
    const size_t T = static_cast<size_t>(s->T), E = s->E, k = s->k, d = s->d, l = s->l, h = s->h;
    const size_t S = static_cast<size_t>(s->n_shared), hs = s->n_shared > 0 ? s->h_shared : 0;
    const moe_shape_t r{s->T, s->l, s->E, s->k, s->h};
    const moe_shape_t g{s->T, s->d, s->E, s->k, s->h};  // the router reads x (width d)
    const size_t sizes[kLatTotal] = {
        4 * T * E, 4 * T * k, 4 * T * k, 4 * (E + 1), 4 * T * k, 4 * T * k, 2 * T * l, 2 * T * k * h,
        4 * T * k * l, 2 * T * l, 2 * S * T * hs, 4 * S * T * d,
        permute_ws(&r), ffn_ws(&r), ffn_ws_rows(s->T, 1), ffn_ws_rows(s->T * s->n_shared, latent_groups(s)),
        maps_shared_rows(s) + 4 * S * T, route_ws(&g)};
    size_t at = 0;
    for (int i = 0; i < kLatTotal; ++i) {
        off[i] = at;
        at += align_up(sizes[i]);
    }
    off[kLatTotal] = at;
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

int check_mx_shape(const moe_shape_t* s) {
    int st = check_shape(s);
    if (st != MOE_OK) return st;
    if (s->d % 512 != 0 || s->h % 512 != 0)
        return fail(MOE_ERR_UNSUPPORTED, "the MX path needs d and h to be multiples of 512 (d = %d, h = %d)", s->d,
                    s->h);
    const int64_t n = s->T * static_cast<int64_t>(s->k);
    if (n * std::max(s->d, s->h) >= (int64_t(1) << 32))
        return fail(MOE_ERR_UNSUPPORTED, "the MX path addresses its E4M3 rows with 32-bit offsets: T * k * max(d, h) = %lld "
                    ">= 2^32", static_cast<long long>(n * std::max(s->d, s->h)));
    return MOE_OK;
}

// MX forward slots, then the permute scratch, the tile list and the router parts.
constexpr int kMxPermuteWs = MOE_MX_NUM_SLOTS, kMxFfnWs = MOE_MX_NUM_SLOTS + 1, kMxRouteWs = MOE_MX_NUM_SLOTS + 2,
              kMxTotal = MOE_MX_NUM_SLOTS + 3;

void mx_layout(const moe_shape_t* s, size_t off[kMxTotal + 1]) {
    const size_t T = static_cast<size_t>(s->T), E = s->E, k = s->k, d = s->d, h = s->h;
    const size_t sizes[kMxTotal] = {4 * T * E, 4 * T * k, 4 * T * k, 4 * (E + 1), 4 * T * k, 4 * T * k,
                                    T * d, T * d / 32, 4 * T * k * h, T * k * h, T * k * h / 32, 4 * T * k * d,
                                    permute_ws(s), ffn_ws(s), route_ws(s)};
    size_t at = 0;
    for (int i = 0; i < kMxTotal; ++i) {
        off[i] = at;
        at += align_up(sizes[i]);
    }
    off[kMxTotal] = at;
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
        case MOE_CALL_MX_FORWARD: {
            if (check_mx_shape(shape) != MOE_OK) return 0;
            size_t off[kMxTotal + 1];
            mx_layout(shape, off);
            ok();
            return off[kMxTotal];
        }
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

// ------------------------------------------------ moe_permute without a workspace
// The permute's only scratch is the (expert, chunk) count matrix: E <= 1024 experts
// times at most 32 chunks of int32, 128 KiB. moe_permute_noalloc keeps it in this
// array, one copy per GPU for the life of the process. Host code never passes the
// array's name to a kernel (on the host it only stands for the symbol): its device
// address is looked up once per device with that device current and kept here.
static __device__ __align__(256) int32_t scratch[MOE_NOALLOC_SCRATCH_BYTES / sizeof(int32_t)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device.
int scratch_on_current_device(int32_t** out) {
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return hip_status(err, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device %d beyond the %d this build tracks", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return hip_status(err, "hipGetSymbolAddress(scratch)");
        if (p == nullptr) return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) gave NULL");
        g_scratch_ptr[dev] = static_cast<int32_t*>(p);
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}
}  // namespace

int moe_permute_noalloc(const moe_shape_t* shape, const uint16_t* x, const int32_t* topk_idx,
                        int32_t* expert_offsets, int32_t* row_of, int32_t* row_src, uint16_t* x_perm, void* stream) {
    int st = check_shape(shape);
    if (st != MOE_OK) return st;
    MOE_CHECK_PTR(expert_offsets);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (shape->T == 0) {
        hipError_t err = moe::launch_zero_i32(expert_offsets, shape->E + 1, s);
        return hip_status(err, "expert_offsets clear");
    }
    MOE_CHECK_PTR(topk_idx);
    MOE_CHECK_PTR(row_of);
    MOE_CHECK_PTR(row_src);
    if (x_perm != nullptr) {
        MOE_CHECK_PTR(x);
        if (!aligned16(x_perm)) return fail(MOE_ERR_INVALID_ARG, "x_perm is not 16-byte aligned");
    }
    const size_t need = permute_ws(shape);
    if (need > MOE_NOALLOC_SCRATCH_BYTES)
        return fail(MOE_ERR_UNSUPPORTED, "permute scratch of %zu bytes exceeds the fixed %d bytes", need,
                    MOE_NOALLOC_SCRATCH_BYTES);
    int32_t* counts = nullptr;
    st = scratch_on_current_device(&counts);
    if (st != MOE_OK) return st;
    // every count the scan and rank kernels read is written by this call's count kernel first,
    // so what an earlier call left in the array does not matter
    hipError_t err = moe::launch_permute(x, topk_idx, shape->T, shape->d, shape->E, shape->k, expert_offsets,
                                         row_of, row_src, x_perm, counts, s);
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

int moe_pack_weights(int64_t groups, int32_t N, int32_t K, const uint16_t* w, uint16_t* w_packed, void* stream) {
    if (groups < 0 || N < 0 || N % 16 != 0 || K < 32 || K % 32 != 0 || K > (1 << 20))
        return fail(MOE_ERR_INVALID_ARG, "bad weight shape (groups %lld, N %d, K %d; N a multiple of 16, K of 32)",
                    static_cast<long long>(groups), N, K);
    if (groups == 0 || N == 0) return ok();
    MOE_CHECK_PTR(w);
    MOE_CHECK_PTR(w_packed);
    const uintptr_t bytes = static_cast<uintptr_t>(groups) * static_cast<uintptr_t>(N) * static_cast<uintptr_t>(K) * 2u;
    const uintptr_t a = reinterpret_cast<uintptr_t>(w), b = reinterpret_cast<uintptr_t>(w_packed);
    if (a < b + bytes && b < a + bytes)
        return fail(MOE_ERR_INVALID_ARG, "w_packed overlaps w (no packing in place)");
    hipError_t err = moe::launch_pack_weights(w, groups * N, K, w_packed, static_cast<hipStream_t>(stream));
    return hip_status(err, "pack_weights launch");
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


size_t moe_latent_workspace_bytes(const moe_latent_shape_t* shape) {
    if (check_latent_shape(shape) != MOE_OK) return 0;
    size_t off[kLatTotal + 1];
    latent_layout(shape, off);
    ok();
    return off[kLatTotal];
}

int moe_latent_ws_offset(const moe_latent_shape_t* shape, int slot, size_t* offset) {
    int st = check_latent_shape(shape);
    if (st != MOE_OK) return st;
    if (slot < 0 || slot >= MOE_LAT_NUM_SLOTS) return fail(MOE_ERR_INVALID_ARG, "unknown slot %d", slot);
    if (offset == nullptr) return fail(MOE_ERR_INVALID_ARG, "offset is NULL");
    size_t off[kLatTotal + 1];
    latent_layout(shape, off);
    *offset = off[slot];
    return ok();
}

int moe_combine_rmsnorm(const moe_shape_t* shape, const float* y_rows, const int32_t* row_of, const float* topk_w,
                        const float* gain, float eps, float* u_out, uint16_t* r_out, void* stream) {
    int st = check_shape(shape);
    if (st != MOE_OK) return st;
    if (shape->d > moe::combine_rmsnorm_max_width())
        return fail(MOE_ERR_UNSUPPORTED, "row width %d > %d", shape->d, moe::combine_rmsnorm_max_width());
    if (!std::isfinite(eps) || eps < 0.f) return fail(MOE_ERR_INVALID_ARG, "eps must be finite and >= 0");
    if (shape->T == 0) return ok();
    MOE_CHECK_PTR(y_rows);
    MOE_CHECK_PTR(row_of);
    MOE_CHECK_PTR(topk_w);
    MOE_CHECK_PTR(gain);
    if (u_out != nullptr && !aligned16(u_out)) return fail(MOE_ERR_INVALID_ARG, "u_out is not 16-byte aligned");
    MOE_CHECK_PTR(r_out);
    hipError_t err = moe::launch_combine_rmsnorm(y_rows, row_of, topk_w, shape->T, shape->d, shape->k,
                                                 shape->T * shape->k, gain, eps, u_out, r_out,
                                                 static_cast<hipStream_t>(stream));
    return hip_status(err, "combine_rmsnorm launch");
}

int moe_latent_forward(const moe_latent_shape_t* shape, const uint16_t* x, const float* w_router,
                       const float* router_bias, const uint16_t* w_proj_down, const uint16_t* w_gate,
                       const uint16_t* w_up, const uint16_t* w_down, const float* rms_gain, float rms_eps,
                       const uint16_t* w_proj_up, const uint16_t* shared_gate, const uint16_t* shared_up,
                       const uint16_t* shared_down, float* out, void* ws, size_t ws_bytes, void* stream) {
    int st = check_latent_shape(shape);
    if (st != MOE_OK) return st;
    if (!std::isfinite(rms_eps) || rms_eps < 0.f) return fail(MOE_ERR_INVALID_ARG, "rms_eps must be finite and >= 0");
    if (shape->T == 0) return ok();
    MOE_CHECK_PTR(x);
    MOE_CHECK_PTR(w_router);
    if (router_bias != nullptr && !aligned16(router_bias))
        return fail(MOE_ERR_INVALID_ARG, "router_bias is not 16-byte aligned");
    MOE_CHECK_PTR(w_proj_down);
    MOE_CHECK_PTR(w_gate);
    MOE_CHECK_PTR(w_up);
    MOE_CHECK_PTR(w_down);
    MOE_CHECK_PTR(rms_gain);
    MOE_CHECK_PTR(w_proj_up);
    if (shape->n_shared > 0) {
        MOE_CHECK_PTR(shared_gate);
        MOE_CHECK_PTR(shared_up);
        MOE_CHECK_PTR(shared_down);
    }
    MOE_CHECK_PTR(out);
    size_t off[kLatTotal + 1];
    latent_layout(shape, off);
    st = check_ws(ws, ws_bytes, off[kLatTotal]);
    if (st != MOE_OK) return st;
    char* base = static_cast<char*>(ws);
    auto at = [&](int slot) { return static_cast<void*>(base + off[slot]); };
    float* logits = static_cast<float*>(at(MOE_LAT_LOGITS));
    int32_t* idx = static_cast<int32_t*>(at(MOE_LAT_TOPK_IDX));
    float* w = static_cast<float*>(at(MOE_LAT_TOPK_W));
    int32_t* offsets = static_cast<int32_t*>(at(MOE_LAT_EXPERT_OFFSETS));
    int32_t* row_of = static_cast<int32_t*>(at(MOE_LAT_ROW_OF));
    int32_t* row_src = static_cast<int32_t*>(at(MOE_LAT_ROW_SRC));
    uint16_t* z = static_cast<uint16_t*>(at(MOE_LAT_Z));
    uint16_t* h_act = static_cast<uint16_t*>(at(MOE_LAT_H));
    float* y_rows = static_cast<float*>(at(MOE_LAT_Y));
    uint16_t* r = static_cast<uint16_t*>(at(MOE_LAT_R));
    uint16_t* sh_h = static_cast<uint16_t*>(at(MOE_LAT_SHARED_H));
    float* sh_y = static_cast<float*>(at(MOE_LAT_SHARED_Y));
    int32_t* count_ws = static_cast<int32_t*>(at(kLatPermuteWs));
    char* maps = static_cast<char*>(at(kLatMaps));
    int32_t* dense_off = reinterpret_cast<int32_t*>(maps);
    int32_t* shared_off = reinterpret_cast<int32_t*>(maps + maps_shared_off(shape));
    int32_t* shared_rows = reinterpret_cast<int32_t*>(maps + maps_shared_rows(shape));
    uint16_t* router_parts = static_cast<uint16_t*>(at(kLatRouteWs));
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t T = shape->T, n = shape->T * shape->k;
    const int d = shape->d, l = shape->l, E = shape->E, k = shape->k, h = shape->h;
    const int S = shape->n_shared, hs = shape->h_shared;
    const moe_shape_t rs{T, l, E, k, h};
    const FfnWs fw = ffn_carve(&rs, at(kLatFfnWs));
    const FfnWs dw = ffn_carve_rows(T, 1, at(kLatDenseWs));
    const FfnWs sw = ffn_carve_rows(T * S, latent_groups(shape), at(kLatSharedWs));

#define MOE_TRY(call, what)                              \
    do {                                                 \
        hipError_t e_ = (call);                          \
        if (e_ != hipSuccess) return hip_status(e_, what); \
    } while (0)
    MOE_TRY(moe::launch_latent_maps(T, S, dense_off, shared_off, shared_rows, s), "latent_maps launch");
    // router on x, then the grouping by expert
    MOE_TRY(moe::launch_router_gemm(x, w_router, router_bias, logits, T, d, E, router_parts, s), "router_gemm launch");
    MOE_TRY(moe::launch_topk_softmax(logits, T, E, k, idx, w, s), "topk_softmax launch");
    MOE_TRY(moe::launch_permute(nullptr, idx, T, l, E, k, offsets, row_of, row_src, nullptr, count_ws, s),
            "permute launch");
    // z = x W_down_proj^T (bf16)
    MOE_TRY(moe::launch_build_tiles(dense_off, T, 1, dw.tiles, dw.tile_start, s), "build_tiles launch");
    MOE_TRY(moe::launch_dense(x, nullptr, T, dw.tiles, dw.tile_start, T, 1, w_proj_down, l, d, z, true, s),
            "down projection launch");
    // routed experts on z (rows gathered through row_src), then u and RMSNorm(u)
    MOE_TRY(moe::launch_build_tiles(offsets, n, E, fw.tiles, fw.tile_start, s), "build_tiles launch");
    MOE_TRY(moe::launch_gate_up(z, row_src, T, fw.tiles, fw.tile_start, n, l, E, h, w_gate, w_up, h_act, s),
            "gate_up launch");
    MOE_TRY(moe::launch_down(h_act, fw.tiles, fw.tile_start, n, l, E, h, w_down, y_rows, s), "down launch");
    MOE_TRY(moe::launch_combine_rmsnorm(y_rows, row_of, w, T, l, k, n, rms_gain, rms_eps, nullptr, r, s),
            "combine_rmsnorm launch");
    // out = RMSNorm(u) W_up_proj^T (float32) ...
    MOE_TRY(moe::launch_dense(r, nullptr, T, dw.tiles, dw.tile_start, T, 1, w_proj_up, d, l, out, false, s),
            "up projection launch");
    if (S > 0) {  // ... + the shared experts on x
        MOE_TRY(moe::launch_build_tiles(shared_off, T * S, S, sw.tiles, sw.tile_start, s), "build_tiles launch");
        MOE_TRY(moe::launch_gate_up(x, shared_rows, T, sw.tiles, sw.tile_start, T * S, d, S, hs, shared_gate,
                                    shared_up, sh_h, s), "shared gate_up launch");
        MOE_TRY(moe::launch_down(sh_h, sw.tiles, sw.tile_start, T * S, d, S, hs, shared_down, sh_y, s),
                "shared down launch");
        MOE_TRY(moe::launch_add_shared(out, sh_y, T, d, S, s), "add_shared launch");
    }
#undef MOE_TRY
    return ok();
}


int moe_mx_quantize_weights(int64_t groups, int32_t N, int32_t K, const uint16_t* w, uint8_t* q, uint8_t* scales,
                            void* stream) {
    if (groups < 0 || N < 0 || N % 16 != 0 || K < 512 || K % 512 != 0 || K > (1 << 20))
        return fail(MOE_ERR_INVALID_ARG, "bad weight shape (groups %lld, N %d, K %d; N a multiple of 16, K of 512)",
                    static_cast<long long>(groups), N, K);
    if (groups * N * static_cast<int64_t>(K / 32) >= (int64_t(1) << 40))
        return fail(MOE_ERR_UNSUPPORTED, "weights too large");
    if (groups == 0 || N == 0) return ok();
    MOE_CHECK_PTR(w);
    MOE_CHECK_PTR(q);
    MOE_CHECK_PTR(scales);
    hipError_t err = moe::launch_mx_quantize(w, false, groups * N, K, true, q, scales,
                                             static_cast<hipStream_t>(stream));
    return hip_status(err, "mx_quantize launch");
}

int moe_mx_quantize_rows(int64_t rows, int32_t K, const void* in, int32_t in_is_f32, uint8_t* q, uint8_t* scales,
                         void* stream) {
    if (rows < 0 || K < 32 || K % 32 != 0 || K > (1 << 20))
        return fail(MOE_ERR_INVALID_ARG, "bad row shape (rows %lld, K %d; K a multiple of 32)",
                    static_cast<long long>(rows), K);
    if (rows == 0) return ok();
    MOE_CHECK_PTR(in);
    MOE_CHECK_PTR(q);
    if (scales == nullptr) return fail(MOE_ERR_INVALID_ARG, "scales is NULL");
    hipError_t err = moe::launch_mx_quantize(in, in_is_f32 != 0, rows, K, false, q, scales,
                                             static_cast<hipStream_t>(stream));
    return hip_status(err, "mx_quantize launch");
}

int moe_mx_expert_ffn(const moe_shape_t* shape, const uint8_t* a_q, const uint8_t* a_s, const int32_t* a_rows,
                      const int32_t* expert_offsets, const uint8_t* wg_q, const uint8_t* wg_s, const uint8_t* wu_q,
                      const uint8_t* wu_s, const uint8_t* wd_q, const uint8_t* wd_s, float* h_act, uint8_t* h_q,
                      uint8_t* h_s, float* y_rows, void* ws, size_t ws_bytes, void* stream) {
    int st = check_mx_shape(shape);
    if (st != MOE_OK) return st;
    if (shape->T == 0) return ok();
    MOE_CHECK_PTR(a_q);
    MOE_CHECK_PTR(a_s);
    if (a_rows != nullptr && !aligned16(a_rows)) return fail(MOE_ERR_INVALID_ARG, "a_rows is not 16-byte aligned");
    MOE_CHECK_PTR(expert_offsets);
    MOE_CHECK_PTR(wg_q);
    MOE_CHECK_PTR(wg_s);
    MOE_CHECK_PTR(wu_q);
    MOE_CHECK_PTR(wu_s);
    MOE_CHECK_PTR(wd_q);
    MOE_CHECK_PTR(wd_s);
    MOE_CHECK_PTR(h_act);
    MOE_CHECK_PTR(h_q);
    MOE_CHECK_PTR(h_s);
    MOE_CHECK_PTR(y_rows);
    st = check_ws(ws, ws_bytes, ffn_ws(shape));
    if (st != MOE_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t n = shape->T * shape->k;
    const int d = shape->d, E = shape->E, h = shape->h;
    const FfnWs fw = ffn_carve(shape, ws);
    hipError_t err = moe::launch_build_tiles_rows(expert_offsets, n, E, moe::mx_tile_rows(), fw.tiles, fw.tile_start, s);
    if (err != hipSuccess) return hip_status(err, "build_tiles launch");
    err = moe::launch_mx_ffn_pass(true, a_q, a_s, a_rows, a_rows ? shape->T : n, fw.tiles, fw.tile_start, n, E,
                                  wg_q, wg_s, wu_q, wu_s, h, d, h_act, s);
    if (err != hipSuccess) return hip_status(err, "mx gate_up launch");
    err = moe::launch_mx_quantize(h_act, true, n, h, false, h_q, h_s, s);
    if (err != hipSuccess) return hip_status(err, "mx_quantize launch");
    err = moe::launch_mx_ffn_pass(false, h_q, h_s, nullptr, n, fw.tiles, fw.tile_start, n, E, wd_q, wd_s, nullptr,
                                  nullptr, d, h, y_rows, s);
    return hip_status(err, "mx down launch");
}

int moe_mx_expert_gate_up(const moe_shape_t* shape, const uint8_t* a_q, const uint8_t* a_s, const int32_t* a_rows,
                          const int32_t* expert_offsets, const uint8_t* wg_q, const uint8_t* wg_s,
                          const uint8_t* wu_q, const uint8_t* wu_s, float* h_act, void* ws, size_t ws_bytes,
                          void* stream) {
    int st = check_mx_shape(shape);
    if (st != MOE_OK) return st;
    if (shape->T == 0) return ok();
    MOE_CHECK_PTR(a_q);
    MOE_CHECK_PTR(a_s);
    if (a_rows != nullptr && !aligned16(a_rows)) return fail(MOE_ERR_INVALID_ARG, "a_rows is not 16-byte aligned");
    MOE_CHECK_PTR(expert_offsets);
    MOE_CHECK_PTR(wg_q);
    MOE_CHECK_PTR(wg_s);
    MOE_CHECK_PTR(wu_q);
    MOE_CHECK_PTR(wu_s);
    MOE_CHECK_PTR(h_act);
    st = check_ws(ws, ws_bytes, ffn_ws(shape));
    if (st != MOE_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t n = shape->T * shape->k;
    const FfnWs fw = ffn_carve(shape, ws);
    hipError_t err = moe::launch_build_tiles_rows(expert_offsets, n, shape->E, moe::mx_tile_rows(), fw.tiles, fw.tile_start, s);
    if (err != hipSuccess) return hip_status(err, "build_tiles launch");
    err = moe::launch_mx_ffn_pass(true, a_q, a_s, a_rows, a_rows ? shape->T : n, fw.tiles, fw.tile_start, n,
                                  shape->E, wg_q, wg_s, wu_q, wu_s, shape->h, shape->d, h_act, s);
    return hip_status(err, "mx gate_up launch");
}

int moe_mx_expert_down(const moe_shape_t* shape, const uint8_t* h_q, const uint8_t* h_s,
                       const int32_t* expert_offsets, const uint8_t* wd_q, const uint8_t* wd_s, float* y_rows,
                       void* ws, size_t ws_bytes, void* stream) {
    int st = check_mx_shape(shape);
    if (st != MOE_OK) return st;
    if (shape->T == 0) return ok();
    MOE_CHECK_PTR(h_q);
    MOE_CHECK_PTR(h_s);
    MOE_CHECK_PTR(expert_offsets);
    MOE_CHECK_PTR(wd_q);
    MOE_CHECK_PTR(wd_s);
    MOE_CHECK_PTR(y_rows);
    st = check_ws(ws, ws_bytes, ffn_ws(shape));
    if (st != MOE_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t n = shape->T * shape->k;
    const FfnWs fw = ffn_carve(shape, ws);
    hipError_t err = moe::launch_build_tiles_rows(expert_offsets, n, shape->E, moe::mx_tile_rows(), fw.tiles, fw.tile_start, s);
    if (err != hipSuccess) return hip_status(err, "build_tiles launch");
    err = moe::launch_mx_ffn_pass(false, h_q, h_s, nullptr, n, fw.tiles, fw.tile_start, n, shape->E, wd_q, wd_s,
                                  nullptr, nullptr, shape->d, shape->h, y_rows, s);
    return hip_status(err, "mx down launch");
}

int moe_mx_forward_ws_offset(const moe_shape_t* shape, int slot, size_t* offset) {
    int st = check_mx_shape(shape);
    if (st != MOE_OK) return st;
    if (slot < 0 || slot >= MOE_MX_NUM_SLOTS) return fail(MOE_ERR_INVALID_ARG, "unknown slot %d", slot);
    if (offset == nullptr) return fail(MOE_ERR_INVALID_ARG, "offset is NULL");
    size_t off[kMxTotal + 1];
    mx_layout(shape, off);
    *offset = off[slot];
    return ok();
}

int moe_mx_forward(const moe_shape_t* shape, const uint16_t* x, const float* w_router, const float* router_bias,
                   const uint8_t* wg_q, const uint8_t* wg_s, const uint8_t* wu_q, const uint8_t* wu_s,
                   const uint8_t* wd_q, const uint8_t* wd_s, float* out, void* ws, size_t ws_bytes, void* stream) {
    int st = check_mx_shape(shape);
    if (st != MOE_OK) return st;
    if (shape->T == 0) return ok();
    MOE_CHECK_PTR(x);
    MOE_CHECK_PTR(w_router);
    if (router_bias != nullptr && !aligned16(router_bias))
        return fail(MOE_ERR_INVALID_ARG, "router_bias is not 16-byte aligned");
    MOE_CHECK_PTR(wg_q);
    MOE_CHECK_PTR(wg_s);
    MOE_CHECK_PTR(wu_q);
    MOE_CHECK_PTR(wu_s);
    MOE_CHECK_PTR(wd_q);
    MOE_CHECK_PTR(wd_s);
    MOE_CHECK_PTR(out);
    size_t off[kMxTotal + 1];
    mx_layout(shape, off);
    st = check_ws(ws, ws_bytes, off[kMxTotal]);
    if (st != MOE_OK) return st;
    char* base = static_cast<char*>(ws);
    auto at = [&](int slot) { return static_cast<void*>(base + off[slot]); };
    float* logits = static_cast<float*>(at(MOE_MX_LOGITS));
    int32_t* idx = static_cast<int32_t*>(at(MOE_MX_TOPK_IDX));
    float* w = static_cast<float*>(at(MOE_MX_TOPK_W));
    int32_t* offsets = static_cast<int32_t*>(at(MOE_MX_EXPERT_OFFSETS));
    int32_t* row_of = static_cast<int32_t*>(at(MOE_MX_ROW_OF));
    int32_t* row_src = static_cast<int32_t*>(at(MOE_MX_ROW_SRC));
    uint8_t* x_q = static_cast<uint8_t*>(at(MOE_MX_X_Q));
    uint8_t* x_s = static_cast<uint8_t*>(at(MOE_MX_X_S));
    float* h_act = static_cast<float*>(at(MOE_MX_H));
    uint8_t* h_q = static_cast<uint8_t*>(at(MOE_MX_H_Q));
    uint8_t* h_s = static_cast<uint8_t*>(at(MOE_MX_H_S));
    float* y_rows = static_cast<float*>(at(MOE_MX_Y));
    int32_t* count_ws = static_cast<int32_t*>(at(kMxPermuteWs));
    const FfnWs fw = ffn_carve(shape, at(kMxFfnWs));
    uint16_t* router_parts = static_cast<uint16_t*>(at(kMxRouteWs));
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t T = shape->T, n = shape->T * shape->k;
    const int d = shape->d, E = shape->E, k = shape->k, h = shape->h;

    hipError_t err = moe::launch_router_gemm(x, w_router, router_bias, logits, T, d, E, router_parts, s);
    if (err != hipSuccess) return hip_status(err, "router_gemm launch");
    err = moe::launch_topk_softmax(logits, T, E, k, idx, w, s);
    if (err != hipSuccess) return hip_status(err, "topk_softmax launch");
    err = moe::launch_permute(x, idx, T, d, E, k, offsets, row_of, row_src, nullptr, count_ws, s);
    if (err != hipSuccess) return hip_status(err, "permute launch");
    err = moe::launch_mx_quantize(x, false, T, d, false, x_q, x_s, s);
    if (err != hipSuccess) return hip_status(err, "mx_quantize launch");
    err = moe::launch_build_tiles_rows(offsets, n, E, moe::mx_tile_rows(), fw.tiles, fw.tile_start, s);
    if (err != hipSuccess) return hip_status(err, "build_tiles launch");
    err = moe::launch_mx_ffn_pass(true, x_q, x_s, row_src, T, fw.tiles, fw.tile_start, n, E, wg_q, wg_s, wu_q, wu_s,
                                  h, d, h_act, s);
    if (err != hipSuccess) return hip_status(err, "mx gate_up launch");
    err = moe::launch_mx_quantize(h_act, true, n, h, false, h_q, h_s, s);
    if (err != hipSuccess) return hip_status(err, "mx_quantize launch");
    err = moe::launch_mx_ffn_pass(false, h_q, h_s, nullptr, n, fw.tiles, fw.tile_start, n, E, wd_q, wd_s, nullptr,
                                  nullptr, d, h, y_rows, s);
    if (err != hipSuccess) return hip_status(err, "mx down launch");
    err = moe::launch_combine(y_rows, row_of, w, T, d, k, n, out, s);
    return hip_status(err, "combine launch");
}

}  // extern "C"
