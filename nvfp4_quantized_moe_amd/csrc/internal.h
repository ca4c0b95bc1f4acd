// Internal launchers shared between the entry points and the layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

// Launch sizes that depend only on the device (CU count times resident
// workgroups per CU) are queried once per device and kept in a table of
// atomics, one slot per device: concurrent first calls compute the same value,
// and a value is read or written whole. 0 = not yet known.
constexpr int kMaxDevices = 64;
inline int nvfp4_current_device() {
  int dev = 0;
  return (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxDevices) ? dev : -1;
}

// Quantizer workspace: per-workgroup amax partials, uint32 [B][1024].
size_t nvfp4_quant_ws_layout(int64_t B);
// rows_dev (optional, device): the number of valid rows is min(M, rows_dev[0]).
// clear (optional, device): n_clear <= 256 words zeroed before the quantize kernel
// runs (by the amax pass, or by a fill when amax_in is given).
int nvfp4_launch_quantize(const void* x_bf16, int64_t B, int64_t M, int64_t K, const float* amax_in,
                          const int32_t* rows_dev, uint8_t* q, uint8_t* sf, float* gs_out, void* ws,
                          uint32_t* clear, int n_clear, hipStream_t stream);

// Quantize with fixed global scales gs_in[b] (device): one launch, no amax pass.
int nvfp4_launch_quantize_static(const void* x_bf16, int64_t B, int64_t M, int64_t K, const float* gs_in,
                                 const int32_t* rows_dev, uint8_t* q, uint8_t* sf, hipStream_t stream);

// Route workspace: per-chunk counts and bases, int32 [nchunks][num_local] each.
constexpr int kRouteChunk = 1024;
size_t nvfp4_route_ws(int32_t T, int32_t k, int32_t num_local);
int nvfp4_launch_route(const int32_t* topk_ids, const float* topk_w, int32_t T, int32_t k, int32_t expert_start,
                       int32_t num_local, int32_t tile_m, int32_t* counts, int32_t* offsets, int32_t* slot_token,
                       int32_t* slot_expert, float* slot_weight, int32_t* token_slot, int32_t* tile_table,
                       void* ws, hipStream_t stream);

int nvfp4_launch_grouped_gemm(const uint8_t* a_q, const uint8_t* a_sf, const int32_t* a_row_index,
                              const float* a_gs, const uint8_t* b_packed, const float* b_gs,
                              const int32_t* offsets, const int32_t* tile_table, int32_t num_local,
                              int32_t rows_cap, int32_t N, int32_t K, int32_t tile_m, int32_t epilogue, void* d,
                              float* amax_out, hipStream_t stream);

// L1 with the SiLU*up epilogue writing h as NVFP4 (fixed global scale out_gs[0]).
int nvfp4_launch_grouped_gemm_nvfp4(const uint8_t* a_q, const uint8_t* a_sf, const int32_t* a_row_index,
                                    const float* a_gs, const uint8_t* b_packed, const float* b_gs, int32_t dual_gs,
                                    const int32_t* offsets, const int32_t* tile_table, int32_t num_local,
                                    int32_t rows_cap, int32_t N, int32_t K, int32_t tile_m, const float* out_gs,
                                    uint8_t* d_q, uint8_t* d_sf, hipStream_t stream);

int nvfp4_launch_scatter(const void* y_bf16, const int32_t* token_slot, const float* topk_w, int32_t T, int32_t k,
                         int32_t H, void* out_bf16, hipStream_t stream);
int nvfp4_launch_fill_u32(uint32_t* p, int n, uint32_t v, hipStream_t stream);

// Prefill-sized batches: quantize x from its amax partials (in ws) and run
// the route's scan and scatter from the per-chunk histograms (in route_ws,
// from nvfp4_launch_amax_count) in one launch. NVFP4_ERR_ARG when more than
// kFusedRouteMaxCounts histogram entries (nchunks x num_local): then use
// nvfp4_launch_quantize_from_partials and nvfp4_launch_route_from_counts.
constexpr int64_t kFusedRouteMaxCounts = 1 << 16;
int nvfp4_launch_quantize_route(const void* x_bf16, int64_t M, int64_t K, const void* ws, int n_partial,
                                uint8_t* q, uint8_t* sf, float* gs_out, const int32_t* topk_ids,
                                const float* topk_w, int32_t T, int32_t k, int32_t expert_start, int32_t num_local,
                                int32_t tile_m, const void* route_ws, int32_t* counts, int32_t* offsets,
                                int32_t* slot_token, int32_t* slot_expert, float* slot_weight, int32_t* token_slot,
                                int32_t* tile_table, hipStream_t stream);

// Static layer, prefill-sized batches: quantize x with gs_in[0] and count the
// route's per-chunk histograms (into route_ws) in one launch.
int nvfp4_launch_quantize_static_count(const void* x_bf16, int64_t M, int64_t K, const float* gs_in, uint8_t* q,
                                       uint8_t* sf, const int32_t* topk_ids, int32_t T, int32_t k,
                                       int32_t expert_start, int32_t num_local, void* route_ws, hipStream_t stream);

// Decode-sized batches (T*k <= 1024): one launch for the amax partials of x
// (nvfp4_amax_route_grid(T*H) of them, in partial) and the whole route.
int nvfp4_amax_route_grid(int64_t per);
constexpr int kAmaxRouteMaxGrid = 1024;  // most partials nvfp4_amax_route_grid returns
int nvfp4_launch_amax_route(const void* x_bf16, int64_t per, int64_t K, uint32_t* partial, uint32_t* clear,
                            int n_clear, const int32_t* topk_ids, const float* topk_w, int32_t T, int32_t k,
                            int32_t expert_start, int32_t num_local, int32_t tile_m, int32_t* counts,
                            int32_t* offsets, int32_t* slot_token, int32_t* slot_expert, float* slot_weight,
                            int32_t* token_slot, int32_t* tile_table, hipStream_t stream);
// Larger batches: one launch for the amax partials of x (nvfp4_amax_grid(T*H)
// of them, in partial) and the route's per-chunk histograms (in route_ws);
// nvfp4_launch_route_from_counts then finishes the route.
int nvfp4_amax_grid(int64_t per);
int nvfp4_launch_amax_count(const void* x_bf16, int64_t per, int64_t K, uint32_t* partial, uint32_t* clear,
                            int n_clear, const int32_t* topk_ids, int32_t T, int32_t k, int32_t expert_start,
                            int32_t num_local, void* route_ws, hipStream_t stream);
int nvfp4_launch_route_from_counts(const int32_t* topk_ids, const float* topk_w, int32_t T, int32_t k,
                                   int32_t expert_start, int32_t num_local, int32_t tile_m, int32_t* counts,
                                   int32_t* offsets, int32_t* slot_token, int32_t* slot_expert, float* slot_weight,
                                   int32_t* token_slot, int32_t* tile_table, void* route_ws, hipStream_t stream);
int nvfp4_launch_quantize_from_partials(const void* x_bf16, int64_t M, int64_t K, const void* ws, int n_partial,
                                        uint8_t* q, uint8_t* sf, float* gs_out, hipStream_t stream);
