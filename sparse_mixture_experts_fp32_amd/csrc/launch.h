// Host-side launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

size_t router_ws_bytes(int64_t T, int d, int E);  // workspace of launch_router_gemm (weight parts, partial sums)
hipError_t launch_router_gemm(const uint16_t* x, const float* w, const float* bias, float* logits, int64_t T, int d,
                              int E, void* ws, hipStream_t stream);
hipError_t launch_topk_softmax(const float* logits, int64_t T, int E, int k, int32_t* topk_idx,
                               float* topk_w, hipStream_t stream);

hipError_t launch_zero_i32(int32_t* p, int n, hipStream_t stream);  // fill kernel, safe under graph capture
int permute_chunk(int64_t n_assign);
int permute_nchunks(int64_t n_assign);
hipError_t launch_permute(const uint16_t* x, const int32_t* topk_idx, int64_t T, int d, int E, int k,
                          int32_t* expert_offsets, int32_t* row_of, int32_t* row_src, uint16_t* x_perm,
                          int32_t* count_ws, hipStream_t stream);

int ffn_tile_rows();
int ffn_max_tiles(int64_t n_rows, int E);
hipError_t launch_build_tiles(const int32_t* expert_offsets, int64_t n_rows, int E, int4* tiles,
                              int32_t* tile_start, hipStream_t stream);
// the same with m-tiles of up to bm rows (bm >= 128, a multiple of 16)
hipError_t launch_build_tiles_rows(const int32_t* expert_offsets, int64_t n_rows, int E, int bm, int4* tiles,
                                   int32_t* tile_start, hipStream_t stream);
// The expert GEMM passes on the LDS-ring kernel (ffn_ring.hip); expert weights in the packed
// layout of moe_pack_weights. a_rows == nullptr: GEMM row r is a[r] (a = x_perm); else it is
// a[a_rows[r]] (a = x with a_nrows rows).
hipError_t launch_gate_up(const uint16_t* a, const int32_t* a_rows, int64_t a_nrows, const int4* tiles,
                          const int32_t* tile_start, int64_t n_rows, int d, int E, int h, const uint16_t* w_gate,
                          const uint16_t* w_up, uint16_t* h_act, hipStream_t stream);
hipError_t launch_down(const uint16_t* h_act, const int4* tiles, const int32_t* tile_start, int64_t n_rows, int d,
                       int E, int h, const uint16_t* w_down, float* y_rows, hipStream_t stream);
// plain products c = a w^T per group (bf16 or float32 out)
hipError_t launch_dense(const uint16_t* a, const int32_t* a_rows, int64_t a_nrows, const int4* tiles,
                        const int32_t* tile_start, int64_t n_rows, int E, const uint16_t* w, int N, int K, void* c,
                        bool bf16_out, hipStream_t stream);
// row-major bf16 [rows, K] (rows % 16 == 0, K % 32 == 0) -> packed 16 x 32 fragment-order tiles
hipError_t launch_pack_weights(const uint16_t* w, int64_t rows, int K, uint16_t* out, hipStream_t stream);

hipError_t launch_combine(const float* y_rows, const int32_t* row_of, const float* topk_w, int64_t T,
                          int d, int k, int64_t n_rows, float* out, hipStream_t stream);

hipError_t launch_qb_select(const float* logits, const float* bias, int64_t T, int E, int k, int32_t* topk_idx,
                            float* topk_w, float* alpha, hipStream_t stream);
int qb_max_bins();
hipError_t launch_qb_histogram(const float* logits, const float* alpha, int64_t T, int E, float lo, float width,
                               int n_bins, int32_t* hist, hipStream_t stream);
hipError_t launch_qb_update(const int32_t* hist, int E, int k, int n_bins, float lo, float width,
                            const float* bias_in, float* bias_out, hipStream_t stream);
size_t aux_ws_bytes(int64_t T, int E);
hipError_t launch_aux_loss(const float* logits, int64_t T, int E, float* prob_mean, float* aux_loss, void* ws,
                           hipStream_t stream);

int combine_rmsnorm_max_width();
hipError_t launch_combine_rmsnorm(const float* y_rows, const int32_t* row_of, const float* topk_w, int64_t T, int l,
                                  int k, int64_t n_rows, const float* gain, float eps, float* u_out,
                                  uint16_t* r_out, hipStream_t stream);
hipError_t launch_latent_maps(int64_t T, int S, int32_t* dense_off, int32_t* shared_off, int32_t* shared_rows,
                              hipStream_t stream);
hipError_t launch_add_shared(float* out, const float* ys, int64_t T, int d, int S, hipStream_t stream);

int mx_tile_rows();
hipError_t launch_mx_quantize(const void* in, bool in_f32, int64_t rows, int K, bool fp4, uint8_t* q,
                              uint8_t* scales, hipStream_t stream);
hipError_t launch_mx_ffn_pass(bool gated, const uint8_t* a, const uint8_t* a_scales, const int32_t* a_rows,
                              int64_t a_nrows, const int4* tiles, const int32_t* tile_start, int64_t n_rows, int E,
                              const uint8_t* w0q, const uint8_t* w0s, const uint8_t* w1q, const uint8_t* w1s, int N,
                              int K, float* c, hipStream_t stream);

}  // namespace moe
