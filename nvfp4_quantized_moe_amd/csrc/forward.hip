// The whole expert-FFN layer on one rank's share of experts, workspace
// layout, and the small host entry points.
//
// tests history, moe_pipeline commit: quantize -> L1 (gate+up) -> SiLU*up ->
//   re-quantize -> L2 (down) -> weighted scatter.
// nvfp4_mega_moe.py history, alpha commit: L1 uses the activation
//   quantizer's gs, L2 the gs returned by re-quantizing h.
// nvfp4_cutedsl.py history, graph-compatibility commits: no host
//   synchronisation, buffers sized for the worst case, device-side offsets,
//   no early return when there are zero slots.
// nvfp4_mega_moe.py history, expert-parallel note: the layer writes a local
//   partial output; the caller reduces across ranks.
#include "common.h"
#include "internal.h"

using namespace nvfp4;

extern "C" const char* nvfp4_status_string(int status) {
  switch (status) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_NULL: return "a required pointer is NULL";
    case NVFP4_ERR_SHAPE: return "invalid size or shape";
    case NVFP4_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
    case NVFP4_ERR_WORKSPACE: return "workspace too small";
    case NVFP4_ERR_HIP: return "kernel launch failed";
    case NVFP4_ERR_ARG: return "unknown option value";
    default: return "unknown status";
  }
}

extern "C" int nvfp4moe_version(void) { return 300; }

extern "C" int32_t nvfp4_moe_tile_m(int32_t T, int32_t k, int32_t num_local) {
  // prefill-shaped (96-row tiles) when the slot capacity averages >= 64 rows
  // per local expert, else decode-shaped (32-row tiles)
  return ((int64_t)T * k >= (int64_t)64 * num_local) ? 96 : 32;
}

extern "C" size_t nvfp4_moe_ws_layout(int32_t T, int32_t k, int32_t hidden, int32_t inter, int32_t num_local,
                                      int32_t tile_m, size_t* off) {
  size_t o[NVFP4_WS_NREGIONS];
  const size_t cap = (size_t)T * k;
  size_t p = 0;
  auto put = [&](int r, size_t bytes) {
    o[r] = p;
    p += nvfp4_align256(bytes);
  };
  put(NVFP4_WS_X_Q, (size_t)T * hidden / 2);
  put(NVFP4_WS_X_SF, (size_t)T * hidden / 16);
  put(NVFP4_WS_SCALARS, 16);
  put(NVFP4_WS_COUNTS, (size_t)num_local * 4);
  put(NVFP4_WS_OFFSETS, (size_t)(num_local + 1) * 4);
  put(NVFP4_WS_SLOT_TOKEN, cap * 4);
  put(NVFP4_WS_SLOT_EXPERT, cap * 4);
  put(NVFP4_WS_SLOT_WEIGHT, cap * 4);
  put(NVFP4_WS_TOKEN_SLOT, cap * 4);
  put(NVFP4_WS_TILES, (size_t)nvfp4_tile_table_len((int64_t)cap, num_local, tile_m) * 4);
  put(NVFP4_WS_ROUTE_SCRATCH, nvfp4_route_ws(T, k, num_local));
  put(NVFP4_WS_H, cap * inter * 2);
  put(NVFP4_WS_H_Q, cap * inter / 2);
  put(NVFP4_WS_H_SF, cap * inter / 16);
  put(NVFP4_WS_Y, cap * hidden * 2);
  // amax partials: of the quantizer's amax pass, or of the fused amax + route launch
  const size_t qs = nvfp4_quant_ws_layout(1);
  put(NVFP4_WS_QUANT_SCRATCH, qs > (size_t)kAmaxRouteMaxGrid * 4 ? qs : (size_t)kAmaxRouteMaxGrid * 4);
  o[NVFP4_WS_END] = p;
  if (off)
    for (int r = 0; r < NVFP4_WS_NREGIONS; ++r) off[r] = o[r];
  return p;
}

extern "C" size_t nvfp4_moe_ws_bytes(int32_t T, int32_t k, int32_t hidden, int32_t inter, int32_t num_local) {
  if (T < 0 || k < 1 || hidden < 1 || inter < 1 || num_local < 1) return 0;
  return nvfp4_moe_ws_layout(T, k, hidden, inter, num_local, nvfp4_moe_tile_m(T, k, num_local), nullptr);
}

// Argument checks shared by both layer entry points (all before any launch).
static int check_forward_args(const nvfp4_moe_weights* w, const void* x_bf16, int32_t T, const int32_t* topk_ids,
                              const float* topk_w, int32_t k, void* out_bf16, void* ws, size_t ws_bytes) {
  if (!w) return NVFP4_ERR_NULL;
  const int32_t L = w->num_local, H = w->hidden, I = w->inter;
  if (T < 0 || k < 1 || k > 64 || L < 1 || L > 4096 || H <= 0 || I <= 0) return NVFP4_ERR_SHAPE;
  if (H % 128 != 0 || I % 128 != 0) return NVFP4_ERR_SHAPE;
  if ((int64_t)T * k >= (1ll << 30)) return NVFP4_ERR_SHAPE;
  // the GEMMs address one expert's packed weights, the activation rows and one output row tile with 32-bit offsets
  if ((int64_t)2 * I * H / 32 * 18 >= (1ll << 31) || (int64_t)T * (H / 2) >= (1ll << 31) ||
      (int64_t)T * k * (I / 2) >= (1ll << 31) || (int64_t)2 * I * 256 >= (1ll << 31) ||
      (int64_t)H * 256 >= (1ll << 31))
    return NVFP4_ERR_SHAPE;
  if (w->w1_dual_gs != 0 && w->w1_dual_gs != 1) return NVFP4_ERR_ARG;
  if (!w->w1 || !w->w1_gs || !w->w2 || !w->w2_gs || !ws) return NVFP4_ERR_NULL;
  if (T > 0 && (!x_bf16 || !topk_ids || !topk_w || !out_bf16)) return NVFP4_ERR_NULL;
  if (!nvfp4_aligned16(w->w1) || !nvfp4_aligned16(w->w2) || !nvfp4_aligned16(ws)) return NVFP4_ERR_ALIGN;
  if (T > 0 && (!nvfp4_aligned16(x_bf16) || !nvfp4_aligned16(out_bf16))) return NVFP4_ERR_ALIGN;
  if (ws_bytes < nvfp4_moe_ws_bytes(T, k, H, I, L)) return NVFP4_ERR_WORKSPACE;
  return NVFP4_OK;
}

// The dynamic layer; with ev != NULL, event ev[i + 1] (when not NULL) is
// recorded on the stream after the launches of stage i (NVFP4_STAGE_*), and
// ev[0] before the first launch.
static int moe_forward(const nvfp4_moe_weights* w, const void* x_bf16, int32_t T, const int32_t* topk_ids,
                       const float* topk_w, int32_t k, int32_t expert_start, void* out_bf16, void* ws,
                       size_t ws_bytes, hipStream_t stream, hipEvent_t* ev) {
  int st = check_forward_args(w, x_bf16, T, topk_ids, topk_w, k, out_bf16, ws, ws_bytes);
  if (st) return st;
  auto mark = [&](int i) -> int {
    if (ev && ev[i] && hipEventRecord(ev[i], stream) != hipSuccess) return NVFP4_ERR_HIP;
    return NVFP4_OK;
  };
  const int32_t L = w->num_local, H = w->hidden, I = w->inter;
  const int32_t tile_m = nvfp4_moe_tile_m(T, k, L);
  size_t o[NVFP4_WS_NREGIONS];
  nvfp4_moe_ws_layout(T, k, H, I, L, tile_m, o);
  char* base = reinterpret_cast<char*>(ws);
  auto R = [&](int r) { return base + o[r]; };
  uint8_t* x_q = reinterpret_cast<uint8_t*>(R(NVFP4_WS_X_Q));
  uint8_t* x_sf = reinterpret_cast<uint8_t*>(R(NVFP4_WS_X_SF));
  float* scalars = reinterpret_cast<float*>(R(NVFP4_WS_SCALARS));
  int32_t* counts = reinterpret_cast<int32_t*>(R(NVFP4_WS_COUNTS));
  int32_t* offsets = reinterpret_cast<int32_t*>(R(NVFP4_WS_OFFSETS));
  int32_t* slot_token = reinterpret_cast<int32_t*>(R(NVFP4_WS_SLOT_TOKEN));
  int32_t* slot_expert = reinterpret_cast<int32_t*>(R(NVFP4_WS_SLOT_EXPERT));
  float* slot_weight = reinterpret_cast<float*>(R(NVFP4_WS_SLOT_WEIGHT));
  int32_t* token_slot = reinterpret_cast<int32_t*>(R(NVFP4_WS_TOKEN_SLOT));
  int32_t* tiles = reinterpret_cast<int32_t*>(R(NVFP4_WS_TILES));
  void* route_ws = R(NVFP4_WS_ROUTE_SCRATCH);
  uint16_t* h = reinterpret_cast<uint16_t*>(R(NVFP4_WS_H));
  uint8_t* h_q = reinterpret_cast<uint8_t*>(R(NVFP4_WS_H_Q));
  uint8_t* h_sf = reinterpret_cast<uint8_t*>(R(NVFP4_WS_H_SF));
  uint16_t* y = reinterpret_cast<uint16_t*>(R(NVFP4_WS_Y));
  void* qws = R(NVFP4_WS_QUANT_SCRATCH);
  const int32_t cap = T * k;

  if ((st = mark(0))) return st;
  if (cap <= 1024) {
    // decode-sized batches: a1 (amax partials of x, which also zero the scalars
    // gs_x, amax_h, gs_h, reserved) and a3 (route) share one launch; then a2
    const int gx = nvfp4_amax_route_grid((int64_t)T * H);
    if ((st = nvfp4_launch_amax_route(x_bf16, (int64_t)T * H, H, reinterpret_cast<uint32_t*>(qws),
                                      reinterpret_cast<uint32_t*>(scalars), 4, topk_ids, topk_w, T, k,
                                      expert_start, L, tile_m, counts, offsets, slot_token, slot_expert,
                                      slot_weight, token_slot, tiles, stream)))
      return st;
    if ((st = mark(1 + NVFP4_STAGE_AMAX_ROUTE))) return st;
    if ((st = nvfp4_launch_quantize_from_partials(x_bf16, T, H, qws, gx, x_q, x_sf, &scalars[0], stream)))
      return st;
    if ((st = mark(1 + NVFP4_STAGE_QUANT_X)) || (st = mark(1 + NVFP4_STAGE_ROUTE))) return st;
  } else {
    // a1 (amax partials of x, which also zero the scalars gs_x, amax_h, gs_h,
    // reserved) and a3's per-chunk histograms share one launch; then a2, then
    // the rest of a3
    if ((st = nvfp4_launch_amax_count(x_bf16, (int64_t)T * H, H, reinterpret_cast<uint32_t*>(qws),
                                      reinterpret_cast<uint32_t*>(scalars), 4, topk_ids, T, k, expert_start, L,
                                      route_ws, stream)))
      return st;
    if ((st = mark(1 + NVFP4_STAGE_AMAX_ROUTE))) return st;
    // a2 with the rest of a3 (scan and scatter) in its launch, or, past the
    // fused route's size limit, a2 and then a3's two launches
    const int gx = nvfp4_amax_grid((int64_t)T * H);
    st = nvfp4_launch_quantize_route(x_bf16, T, H, qws, gx, x_q, x_sf, &scalars[0], topk_ids, topk_w, T, k,
                                     expert_start, L, tile_m, route_ws, counts, offsets, slot_token, slot_expert,
                                     slot_weight, token_slot, tiles, stream);
    if (st == NVFP4_ERR_ARG) {
      if ((st = nvfp4_launch_quantize_from_partials(x_bf16, T, H, qws, gx, x_q, x_sf, &scalars[0], stream)))
        return st;
      if ((st = mark(1 + NVFP4_STAGE_QUANT_X))) return st;
      if ((st = nvfp4_launch_route_from_counts(topk_ids, topk_w, T, k, expert_start, L, tile_m, counts, offsets,
                                               slot_token, slot_expert, slot_weight, token_slot, tiles, route_ws,
                                               stream)))
        return st;
    } else if (st) {
      return st;
    } else if ((st = mark(1 + NVFP4_STAGE_QUANT_X))) {
      return st;
    }
    if ((st = mark(1 + NVFP4_STAGE_ROUTE))) return st;
  }
  if (cap > 0) {
    // a4/a5: L1 with the fused SiLU*up epilogue and amax of h
    if ((st = nvfp4_launch_grouped_gemm(x_q, x_sf, slot_token, &scalars[0], w->w1, w->w1_gs, offsets,
                                        tiles, L, cap, 2 * I, H, tile_m,
                                        w->w1_dual_gs ? NVFP4_EPI_SILU_MUL_DUAL : NVFP4_EPI_SILU_MUL, h,
                                        &scalars[1], stream)))
      return st;
  }
  if ((st = mark(1 + NVFP4_STAGE_L1))) return st;
  // a6: re-quantize the S valid rows of h with gs_h = amax_h / 2688
  if ((st = nvfp4_launch_quantize(h, 1, cap, I, &scalars[1], &offsets[L], h_q, h_sf, &scalars[2], qws, nullptr,
                                  0, stream)))
    return st;
  if ((st = mark(1 + NVFP4_STAGE_QUANT_H))) return st;
  if (cap > 0) {
    // a7: L2 in slot order
    if ((st = nvfp4_launch_grouped_gemm(h_q, h_sf, nullptr, &scalars[2], w->w2, w->w2_gs, offsets,
                                        tiles, L, cap, H, I, tile_m, NVFP4_EPI_BF16, y, nullptr, stream)))
      return st;
  }
  if ((st = mark(1 + NVFP4_STAGE_L2))) return st;
  // a8: weighted scatter back to token rows
  if ((st = nvfp4_launch_scatter(y, token_slot, topk_w, T, k, H, out_bf16, stream))) return st;
  return mark(1 + NVFP4_STAGE_SCATTER);
}

extern "C" int nvfp4_moe_forward(const nvfp4_moe_weights* w, const void* x_bf16, int32_t T, const int32_t* topk_ids,
                                 const float* topk_w, int32_t k, int32_t expert_start, void* out_bf16, void* ws,
                                 size_t ws_bytes, void* stream) {
  return moe_forward(w, x_bf16, T, topk_ids, topk_w, k, expert_start, out_bf16, ws, ws_bytes, (hipStream_t)stream,
                     nullptr);
}

extern "C" int nvfp4_moe_forward_stage_events(const nvfp4_moe_weights* w, const void* x_bf16, int32_t T,
                                              const int32_t* topk_ids, const float* topk_w, int32_t k,
                                              int32_t expert_start, void* out_bf16, void* ws, size_t ws_bytes,
                                              void* const* events, void* stream) {
  if (!events) return NVFP4_ERR_NULL;
  hipEvent_t ev[NVFP4_NSTAGES + 1];
  for (int i = 0; i <= NVFP4_NSTAGES; ++i) ev[i] = reinterpret_cast<hipEvent_t>(events[i]);
  return moe_forward(w, x_bf16, T, topk_ids, topk_w, k, expert_start, out_bf16, ws, ws_bytes, (hipStream_t)stream,
                     ev);
}

// The layer with fixed global scales gs_in = (gs_x, gs_h), measured once
// beforehand (nvfp4_cutedsl.py history, static-scale commit: warmup measures
// the L1 input's and the L1 output's gs; inference quantizes with them and
// no max reduction). For prefill-shaped batches four launches on top of the
// route: quantize x, L1 whose epilogue writes h as NVFP4 (no BF16 h, no
// separate re-quantization), L2, scatter; decode-shaped batches keep BF16 h
// and quantize it with gs_h in a launch of its own.
extern "C" int nvfp4_moe_forward_static(const nvfp4_moe_weights* w, const void* x_bf16, int32_t T,
                                        const int32_t* topk_ids, const float* topk_w, int32_t k,
                                        int32_t expert_start, const float* gs_in, void* out_bf16, void* ws,
                                        size_t ws_bytes, void* stream_) {
  int st = check_forward_args(w, x_bf16, T, topk_ids, topk_w, k, out_bf16, ws, ws_bytes);
  if (st) return st;
  if (!gs_in) return NVFP4_ERR_NULL;
  const int32_t L = w->num_local, H = w->hidden, I = w->inter;
  hipStream_t stream = (hipStream_t)stream_;
  const int32_t tile_m = nvfp4_moe_tile_m(T, k, L);
  size_t o[NVFP4_WS_NREGIONS];
  nvfp4_moe_ws_layout(T, k, H, I, L, tile_m, o);
  char* base = reinterpret_cast<char*>(ws);
  auto R = [&](int r) { return base + o[r]; };
  uint8_t* x_q = reinterpret_cast<uint8_t*>(R(NVFP4_WS_X_Q));
  uint8_t* x_sf = reinterpret_cast<uint8_t*>(R(NVFP4_WS_X_SF));
  int32_t* counts = reinterpret_cast<int32_t*>(R(NVFP4_WS_COUNTS));
  int32_t* offsets = reinterpret_cast<int32_t*>(R(NVFP4_WS_OFFSETS));
  int32_t* slot_token = reinterpret_cast<int32_t*>(R(NVFP4_WS_SLOT_TOKEN));
  int32_t* slot_expert = reinterpret_cast<int32_t*>(R(NVFP4_WS_SLOT_EXPERT));
  float* slot_weight = reinterpret_cast<float*>(R(NVFP4_WS_SLOT_WEIGHT));
  int32_t* token_slot = reinterpret_cast<int32_t*>(R(NVFP4_WS_TOKEN_SLOT));
  int32_t* tiles = reinterpret_cast<int32_t*>(R(NVFP4_WS_TILES));
  void* route_ws = R(NVFP4_WS_ROUTE_SCRATCH);
  uint16_t* h = reinterpret_cast<uint16_t*>(R(NVFP4_WS_H));
  float* scalars = reinterpret_cast<float*>(R(NVFP4_WS_SCALARS));
  uint8_t* h_q = reinterpret_cast<uint8_t*>(R(NVFP4_WS_H_Q));
  uint8_t* h_sf = reinterpret_cast<uint8_t*>(R(NVFP4_WS_H_SF));
  uint16_t* y = reinterpret_cast<uint16_t*>(R(NVFP4_WS_Y));
  const int32_t cap = T * k;

  if (cap > 1024) {
    // a2 with gs_x (one pass over x) and a3's per-chunk histograms in one
    // launch, then the rest of a3
    if ((st = nvfp4_launch_quantize_static_count(x_bf16, T, H, &gs_in[0], x_q, x_sf, topk_ids, T, k, expert_start, L,
                                                 route_ws, stream)))
      return st;
    if ((st = nvfp4_launch_route_from_counts(topk_ids, topk_w, T, k, expert_start, L, tile_m, counts, offsets,
                                             slot_token, slot_expert, slot_weight, token_slot, tiles, route_ws,
                                             stream)))
      return st;
  } else {
    // a2 with gs_x: one pass over x; a3: route
    if (T > 0 && (st = nvfp4_launch_quantize_static(x_bf16, 1, T, H, &gs_in[0], nullptr, x_q, x_sf, stream)))
      return st;
    if ((st = nvfp4_launch_route(topk_ids, topk_w, T, k, expert_start, L, tile_m, counts, offsets, slot_token,
                                 slot_expert, slot_weight, token_slot, tiles, route_ws, stream)))
      return st;
  }
  if (cap > 0) {
    if (tile_m >= 64) {
      // a4/a5/a6: L1, SiLU*up and NVFP4 h with gs_h in one kernel
      if ((st = nvfp4_launch_grouped_gemm_nvfp4(x_q, x_sf, slot_token, &gs_in[0], w->w1, w->w1_gs, w->w1_dual_gs,
                                                offsets, tiles, L, cap, 2 * I, H, tile_m, &gs_in[1], h_q, h_sf,
                                                stream)))
        return st;
    } else {
      // decode-shaped batches: h is small, and the NVFP4 epilogue's registers
      // (the next item's stages stay in flight across it) would cost the
      // weight-streaming GEMM a quarter of its resident workgroups; BF16 h,
      // then one fixed-scale quantization of its valid rows (the amax the
      // BF16 epilogue raises goes to the unused scalars region)
      if ((st = nvfp4_launch_grouped_gemm(x_q, x_sf, slot_token, &gs_in[0], w->w1, w->w1_gs, offsets, tiles, L,
                                          cap, 2 * I, H, tile_m,
                                          w->w1_dual_gs ? NVFP4_EPI_SILU_MUL_DUAL : NVFP4_EPI_SILU_MUL, h,
                                          &scalars[1], stream)))
        return st;
      if ((st = nvfp4_launch_quantize_static(h, 1, cap, I, &gs_in[1], &offsets[L], h_q, h_sf, stream))) return st;
    }
    // a7: L2 in slot order, alpha = gs_h * w2_gs[e]
    if ((st = nvfp4_launch_grouped_gemm(h_q, h_sf, nullptr, &gs_in[1], w->w2, w->w2_gs, offsets, tiles, L, cap, H,
                                        I, tile_m, NVFP4_EPI_BF16, y, nullptr, stream)))
      return st;
  }
  // a8: weighted scatter back to token rows
  return nvfp4_launch_scatter(y, token_slot, topk_w, T, k, H, out_bf16, stream);
}
