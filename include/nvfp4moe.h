/*
 * nvfp4moe — NVFP4 mixture-of-experts expert FFN on AMD Instinct MI355X (gfx950).
 *
 * C ABI of libnvfp4moe.so. The layer runs in six steps (tests history of the
 * nvfp4-megamoe-kernel project, moe_pipeline commit): quantize the BF16
 * activation to NVFP4; L1 grouped GEMM (gate+up); SiLU(gate)*up, re-quantized;
 * L2 grouped GEMM (down_proj); weighted scatter back to token rows.
 *
 * NVFP4 storage used throughout:
 *   - values: E2M1 nibbles, bit 3 = sign, bits 2:0 index {0,0.5,1,1.5,2,3,4,6};
 *     two per byte along K, element 2j in the low nibble of byte j;
 *     a [rows, K] tensor is stored as uint8 [rows, K/2], row-major;
 *   - block scales: one E4M3 (float8_e4m3fn) bit pattern per 16 consecutive
 *     K elements, uint8 [rows, K/16], row-major, never negative, at most 448;
 *   - global scale: float32 gs = amax / 2688 (= 6 * 448) per tensor;
 *     value = E2M1(nibble) * E4M3(scale) * gs.
 * BF16 tensors are passed as raw 16-bit patterns (void*).
 *
 * Conventions for every entry point:
 *   - Pointers are device pointers unless marked (host). The caller owns all
 *     memory; the library never allocates or frees memory, holds no data from
 *     one call to the next, and reads no environment variables. Its only
 *     process-wide state is launch sizes that depend on the device alone (CU
 *     count times resident workgroups per CU), queried on the first call on
 *     each device and kept per device, and the device array (with its address
 *     per device) that nvfp4_quantize_noalloc uses in place of a workspace.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream) and never synchronize with the host.
 *   - Every entry point that launches work returns an int: NVFP4_OK (0) or
 *     one of the nvfp4_status codes below (declared int so that the ABI does
 *     not depend on the size of an enum).
 *   - Arguments are validated on the host before anything is launched; a
 *     rejected call returns a nonzero status and launches nothing. A launch
 *     failure returns NVFP4_ERR_HIP (the error is taken with hipGetLastError,
 *     without synchronizing).
 *   - Data-dependent conditions are not errors: expert ids outside this
 *     rank's range are dropped, and zero local slots give a zero output.
 *   - Device pointers must be 16-byte aligned; floating-point inputs finite.
 *   - Calls that share no output buffers may run concurrently.
 */
#ifndef NVFP4MOE_H
#define NVFP4MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NVFP4_OK = 0,
  NVFP4_ERR_NULL = 1,       /* a required pointer is NULL */
  NVFP4_ERR_SHAPE = 2,      /* a size is negative, zero where it must not be, or not a multiple it must be */
  NVFP4_ERR_ALIGN = 3,      /* a device pointer is not 16-byte aligned */
  NVFP4_ERR_WORKSPACE = 4,  /* workspace smaller than the matching *_ws_bytes() */
  NVFP4_ERR_HIP = 5,        /* a kernel launch failed */
  NVFP4_ERR_ARG = 6         /* an enum or option value is unknown */
} nvfp4_status;

/* Static description of a status code (host). */
const char* nvfp4_status_string(int status);

/* Library version as major*10000 + minor*100 + patch (host). */
int nvfp4moe_version(void);

/* ---------------------------------------------------------------- quantize
 * Activation/weight quantizer (nvfp4_mega_moe.py history: overflow-fix commit,
 * alpha commit and three-quantizer-bugs commit; tests history: packing along K).
 *
 * x_bf16 holds B independent tensors, each [M, K] BF16 row-major
 * (B*M*K elements). Tensor b gets its own global scale:
 *   amax_b = max |x_b|   (or amax_in[b] when amax_in != NULL)
 *   gs_b   = RN_f32(amax_b / 2688)                         -> gs_out[b]
 * and for every row and 16-element block with bmax = max |x| in the block:
 *   sf     = nearest E4M3 to bmax / (6 gs_b), ties to even, saturating at 448
 *   nibble = sign bit of x | nearest E2M1 magnitude index of |x| / (E4M3(sf) gs_b),
 *            ties to the even index, saturating at 6; magnitude 0 where sf == 0
 * Both roundings are decided exactly (as on the real quotient). amax == 0 gives
 * gs = 0, sf = 0 and magnitude 0.
 *   q  : uint8 [B, M, K/2]    sf : uint8 [B, M, K/16]    gs_out : float [B]
 *   amax_in : float [B] or NULL (device; the h path passes the L1 epilogue's amax)
 *   ws : scratch of at least nvfp4_quantize_ws_bytes(B, M, K) bytes: the
 *        per-workgroup amax partials, a fixed number per tensor, so the size
 *        depends on B alone (M and K are accepted for a stable signature)
 * Requires B >= 1, M >= 0, K > 0, K % 32 == 0.
 */
size_t nvfp4_quantize_ws_bytes(int64_t B, int64_t M, int64_t K);
int nvfp4_quantize(const void* x_bf16, int64_t B, int64_t M, int64_t K, const float* amax_in,
                   uint8_t* q, uint8_t* sf, float* gs_out, void* ws, size_t ws_bytes, void* stream);

/* nvfp4_quantize for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments, results, kernels and launches without the workspace.
 * The amax partials live in a device array of the library, 256 KB on each
 * device it runs on (allocated when the library's code is loaded there, kept
 * until the process ends); its address is taken on the first call on a device.
 * The call allocates and frees nothing. Calls on one device share that array,
 * so calls that overlap on one device (concurrent streams, threads) race;
 * with amax_in != NULL the array is not used. Requires B <= 128 (more tensors
 * return NVFP4_ERR_WORKSPACE) and otherwise what nvfp4_quantize requires.
 */
int nvfp4_quantize_noalloc(const void* x_bf16, int64_t B, int64_t M, int64_t K, const float* amax_in,
                           uint8_t* q, uint8_t* sf, float* gs_out, void* stream);

/* Quantize with fixed global scales (nvfp4_cutedsl.py history, page 2,
 * static-scale commit: a warmup pass measures gs once; afterwards activations
 * are quantized with that gs and no max reduction). As nvfp4_quantize with
 * gs_b = gs_in[b] (device float [B], finite and >= 0; 0 gives all zeros), no
 * amax pass and no workspace. Where |x| exceeds 2688 * gs_b the block scale
 * saturates at 448 and magnitudes at 6. One launch.
 * Requires 1 <= B <= 65535, M >= 0, K > 0, K % 32 == 0.
 */
int nvfp4_quantize_static(const void* x_bf16, int64_t B, int64_t M, int64_t K, const float* gs_in,
                          uint8_t* q, uint8_t* sf, void* stream);

/* ------------------------------------------------------------------- route
 * Slot routing for one rank's share of experts (nvfp4_mega_moe.py history:
 * local-expert-id commit; src history: one 1-D slot order for both GEMMs;
 * nvfp4_cutedsl.py history: bincount/cumsum int32 offsets and sort by expert).
 *
 * topk_ids int32 [T, k] are global expert ids; local = id - expert_start is
 * kept when 0 <= local < num_local and dropped otherwise. S = number of kept
 * (t, j) pairs. Slots are ordered by (local expert, t*k + j):
 *   counts      int32 [num_local]     kept pairs per local expert
 *   offsets     int32 [num_local + 1] exclusive prefix sum; offsets[num_local] = S
 *   slot_token  int32 [T*k]  token of slot s, -1 for s >= S
 *   slot_expert int32 [T*k]  local expert of slot s, -1 for s >= S
 *   slot_weight float [T*k]  topk_w of slot s, 0 for s >= S
 *   token_slot  int32 [T*k]  slot of pair t*k + j, -1 when dropped
 *   tile_table  int32 [nvfp4_tile_table_len(T*k, num_local, tile_m)]
 *               [0] = n tiles; then n pairs (expert, first slot): expert e
 *               contributes ceil(counts[e] / tile_m) tiles starting at
 *               offsets[e], offsets[e] + tile_m, ... in expert order.
 * ws: at least moe_route_ws_bytes(T, k, num_local) bytes.
 * Requires T >= 0, 1 <= k <= 64, 1 <= num_local <= 4096, tile_m a multiple of 16 in [16, 256],
 * T*k < 2^30.
 */
size_t moe_route_ws_bytes(int32_t T, int32_t k, int32_t num_local);
int64_t nvfp4_tile_table_len(int64_t slot_capacity, int32_t num_local, int32_t tile_m);
int moe_route_slots(const int32_t* topk_ids, const float* topk_w, int32_t T, int32_t k,
                    int32_t expert_start, int32_t num_local, int32_t tile_m,
                    int32_t* counts, int32_t* offsets, int32_t* slot_token, int32_t* slot_expert,
                    float* slot_weight, int32_t* token_slot, int32_t* tile_table,
                    void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------- weight packing
 * Offline weight preparation, step three (after quantize and fold): the
 * grouped GEMM reads weights in a packed order that matches its MFMA operand
 * fragments, so that every load instruction of a wave reads one contiguous
 * 1 KB (or 256 B) block. Packing is a byte permutation of (q, sf); nothing is
 * rounded. (Layout of this library's own design; the NVFP4 values and scales
 * are those of nvfp4_quantize.)
 *
 * Input: B matrices, q uint8 [B, N, K/2] and sf uint8 [B, N, K/16], row-major.
 * Output: packed uint8 [B][N/32][K/128][2304], one 2304-byte chunk per
 * (matrix b, 32-row subtile t, 128-element K stage c):
 *   chunk[h*1024 + 16*l + i] = q [b, 32t + l%32, 64c + 32*(l/32) + 16h + i]
 *                                           h in {0,1}, l in [0,64), i in [0,16)
 *   chunk[2048 + 4*l + i]    = sf[b, 32t + l%32, 8c + 4*(l/32) + i]        i in [0,4)
 * Size: nvfp4_packed_bytes(B, N, K) = B * N * K * 9/16 bytes (same as q + sf).
 * Requires B >= 0, N % 32 == 0, K % 128 == 0; nvfp4_packed_bytes returns -1 otherwise.
 */
int64_t nvfp4_packed_bytes(int64_t B, int64_t N, int64_t K);
int nvfp4_pack_weights(const uint8_t* q, const uint8_t* sf, int64_t B, int64_t N, int64_t K,
                       uint8_t* packed, void* stream);

/* ------------------------------------------------------------ grouped GEMM
 * NVFP4 x NVFP4 grouped GEMM over slot rows (nvfp4_mega_moe.py history: alpha
 * commit; src history: 1-D slot ids, gather only for L1; tests history:
 * [expert0 | expert1 | ...] row layout for the 2-D x 3-D grouped GEMM).
 *
 * For every tile (e, r0) of tile_table and every slot row s in
 * [r0, min(r0 + tile_m, offsets[e+1])):
 *   a = a_row_index ? a_row_index[s] : s          (L1 gathers token rows)
 *   G[s, n] = alpha_e * sum_k A_hat[a, k] * W_hat_e[n, k],  alpha_e = RN_f32(a_gs[0] * b_gs[e])
 * with A_hat, W_hat the exact dequantized values without global scale and the
 * sum in float32.
 *   a_q uint8 [*, K/2], a_sf uint8 [*, K/16] (row-major NVFP4);
 *   b_packed: the L expert matrices W_e [N, K] packed by nvfp4_pack_weights (B = L);
 *   a_gs float [1]; b_gs float [L]; offsets int32 [L+1]; tile_table as from moe_route_slots
 *   with the same tile_m; rows_cap = capacity of the row arrays (tile_table holds at
 *   most nvfp4_tile_table_len(rows_cap, L, tile_m) entries).
 * epilogue NVFP4_EPI_BF16:        d = BF16 [rows_cap, N], d[s, n] = RN_bf16(G[s, n]).
 * epilogue NVFP4_EPI_SILU_MUL:    N = 2*I (gate rows [0, I), up rows [I, 2I) of W_e;
 *   nvfp4_cutedsl.py history, intermediate-split commit), d = BF16 [rows_cap, I],
 *   g = RN_bf16(G[s, n]), u = RN_bf16(G[s, I + n]), d[s, n] = RN_bf16(silu(g) * u)
 *   with silu(g) = g / (1 + exp(-g)) in float32; amax_out[0] is raised (atomic max)
 *   to max |d| over the rows written, so the caller sets it to 0 first.
 * epilogue NVFP4_EPI_SILU_MUL_DUAL: as NVFP4_EPI_SILU_MUL for an L1 weight whose gate and
 *   up halves keep their own global scales (no nvfp4_fold_scales): b_gs is float [L, 2]
 *   = (gs_gate, gs_up) and the gate columns take alpha = RN_f32(a_gs[0] * b_gs[e][0]), the up
 *   columns RN_f32(a_gs[0] * b_gs[e][1]) (the alpha commit's global-scale treatment applied to
 *   each half, instead of the finalize_weights fold).
 * Activation row indices must satisfy (row + 1) * K/2 < 2^31, as must rows_cap * K/2,
 * N * K * 9/16 and 256 * N (32-bit buffer offsets); NVFP4_ERR_SHAPE otherwise.
 * Only rows of listed tiles are written. Requires K % 128 == 0, N % 64 == 0
 * (N % 128 == 0 for NVFP4_EPI_SILU_MUL), 1 <= L, tile_m 32 (decode-shaped
 * batches), 64, 96 (prefill-shaped) or 128 (large groups).
 */
enum { NVFP4_EPI_BF16 = 0, NVFP4_EPI_SILU_MUL = 1, NVFP4_EPI_SILU_MUL_DUAL = 2 };
int nvfp4_grouped_gemm(const uint8_t* a_q, const uint8_t* a_sf, const int32_t* a_row_index,
                       const float* a_gs, const uint8_t* b_packed, const float* b_gs,
                       const int32_t* offsets, const int32_t* tile_table, int32_t num_local,
                       int32_t rows_cap, int32_t N, int32_t K, int32_t tile_m, int32_t epilogue,
                       void* d, float* amax_out, void* stream);

/* L1 with h written as NVFP4: the NVFP4_EPI_SILU_MUL (dual_gs = 0) or
 * NVFP4_EPI_SILU_MUL_DUAL (dual_gs = 1) GEMM, whose BF16 h[s, n] is quantized
 * in the epilogue with the fixed global scale out_gs[0] (device float [1]) by
 * exactly the rules of nvfp4_quantize_static: d_q uint8 [rows_cap, N/4],
 * d_sf uint8 [rows_cap, N/32] (h = [rows_cap, N/2] row-major, 16-column
 * blocks). This fuses the re-quantization of h into L1 once gs_h is fixed
 * (nvfp4_cutedsl.py history, static-scale commit); no BF16 h and no amax are
 * written. Same shapes, tile heights and limits as nvfp4_grouped_gemm with
 * N % 128 == 0; d_q 16-byte aligned.
 */
int nvfp4_grouped_gemm_silu_nvfp4(const uint8_t* a_q, const uint8_t* a_sf, const int32_t* a_row_index,
                                  const float* a_gs, const uint8_t* b_packed, const float* b_gs, int32_t dual_gs,
                                  const int32_t* offsets, const int32_t* tile_table, int32_t num_local,
                                  int32_t rows_cap, int32_t N, int32_t K, int32_t tile_m, const float* out_gs,
                                  uint8_t* d_q, uint8_t* d_sf, void* stream);

/* ------------------------------------------------------- weighted scatter
 * out[t, :] = RN_bf16( sum over j = 0..k-1 with token_slot[t*k+j] >= 0 of
 *                      topk_w[t, j] * y[token_slot[t*k+j], :] ), float32, increasing j;
 * 0 for tokens with no local pair (nvfp4_cutedsl.py history: scatter with routing
 * weights; made order-fixed). y BF16 [*, H]; out BF16 [T, H]; H % 8 == 0.
 */
int moe_weighted_scatter(const void* y_bf16, const int32_t* token_slot, const float* topk_w,
                         int32_t T, int32_t k, int32_t H, void* out_bf16, void* stream);

/* ---------------------------------------------------------- scale folding
 * Offline weight preparation (nvfp4_cutedsl.py history, finalize_weights commit):
 * gate and up carry their own global scales; both are brought to
 * gs1[e] = max(gs_gate[e], gs_up[e]) by rewriting the block scales of the half
 * with the smaller scale: ratio = RN_f32(gs_p / gs1), sf' = E4M3 nearest-even,
 * saturating, of RN_f32(E4M3(sf) * ratio). Equal scales leave sf unchanged.
 *   w1_sf uint8 [L, 2I, K/16] in place; gs_gate, gs_up float [L]; gs1 float [L] out.
 */
int nvfp4_fold_scales(uint8_t* w1_sf, const float* gs_gate, const float* gs_up, float* gs1,
                      int32_t num_local, int32_t inter, int32_t K, void* stream);

/* ------------------------------------------------------------ whole layer
 * One rank's share of the MoE expert FFN (nvfp4_mega_moe.py history:
 * expert-parallel note — the layer writes a local partial output and the
 * caller reduces across ranks). Steps, all on `stream`, no host sync:
 *   quantize x (own gs) -> route -> L1 grouped GEMM with the SiLU*up epilogue
 *   (alpha = gs_x * w1_gs[e]) -> re-quantize h (gs_h from the epilogue's amax)
 *   -> L2 grouped GEMM (alpha = gs_h * w2_gs[e]) -> weighted scatter.
 * Weights (host struct of device pointers), L = num_local, each packed by
 * nvfp4_pack_weights from its row-major NVFP4 form:
 *   w1: W1 [L, 2I, H] packed (B = L, N = 2I, K = H), w1_gs [L]
 *       gate rows [0,I), up rows [I,2I), gate/up scales folded to one gs (nvfp4_fold_scales);
 *       or, with w1_dual_gs = 1, unfolded scales and w1_gs [L, 2] = (gs_gate, gs_up)
 *   w2: W2 [L, H, I] packed (B = L, N = H, K = I),   w2_gs [L]
 * x_bf16 [T, H]; topk_ids int32 [T, k] global ids; topk_w float [T, k];
 * out_bf16 [T, H] (tokens with no local expert get zeros).
 * ws: at least nvfp4_moe_ws_bytes(...) bytes; its regions (nvfp4_moe_ws_layout)
 * hold the intermediates after the call. Requires H % 128 == 0, I % 128 == 0,
 * T*k < 2^30, and T*H/2, T*k*I/2, 2I*H*9/16, 512*I and 256*H below 2^31.
 */
typedef struct {
  int32_t num_local, hidden, inter;
  const uint8_t* w1;
  const float* w1_gs;
  const uint8_t* w2;
  const float* w2_gs;
  int32_t w1_dual_gs;  /* 0: w1_gs [L] (folded); 1: w1_gs [L, 2] (gate, up) */
} nvfp4_moe_weights;

enum {
  NVFP4_WS_X_Q = 0, NVFP4_WS_X_SF, NVFP4_WS_SCALARS, NVFP4_WS_COUNTS, NVFP4_WS_OFFSETS,
  NVFP4_WS_SLOT_TOKEN, NVFP4_WS_SLOT_EXPERT, NVFP4_WS_SLOT_WEIGHT, NVFP4_WS_TOKEN_SLOT,
  NVFP4_WS_TILES, NVFP4_WS_ROUTE_SCRATCH, NVFP4_WS_H, NVFP4_WS_H_Q, NVFP4_WS_H_SF, NVFP4_WS_Y,
  NVFP4_WS_QUANT_SCRATCH, NVFP4_WS_END, NVFP4_WS_NREGIONS
};
/* Scalars region (float[4]): [0] gs_x, [1] amax_h, [2] gs_h, [3] reserved. */

/* Byte offset of every workspace region (host array of NVFP4_WS_NREGIONS entries;
 * entry NVFP4_WS_END is the total size). Returns the total size. */
size_t nvfp4_moe_ws_layout(int32_t T, int32_t k, int32_t hidden, int32_t inter, int32_t num_local,
                           int32_t tile_m, size_t* offsets_out);
size_t nvfp4_moe_ws_bytes(int32_t T, int32_t k, int32_t hidden, int32_t inter, int32_t num_local);
/* GEMM row-tile height the layer uses for a given batch: 32 when decode-shaped, 96 when
 * prefill-shaped (slot capacity T*k of at least 64 rows per local expert). */
int32_t nvfp4_moe_tile_m(int32_t T, int32_t k, int32_t num_local);
int nvfp4_moe_forward(const nvfp4_moe_weights* w, const void* x_bf16, int32_t T,
                      const int32_t* topk_ids, const float* topk_w, int32_t k, int32_t expert_start,
                      void* out_bf16, void* ws, size_t ws_bytes, void* stream);

/* nvfp4_moe_forward with per-stage timing: the same launches, with HIP events
 * recorded on `stream` between them, so that the caller can time each step of
 * the real layer. events: host array of NVFP4_NSTAGES + 1 hipEvent_t the caller
 * created (timing enabled); events[0] is recorded before the first launch and
 * events[i + 1] after the launches of stage i:
 *   NVFP4_STAGE_AMAX_ROUTE  a1, amax of x, sharing its launch with a3: the whole
 *                           route when T*k <= 1024, else the per-chunk histograms
 *   NVFP4_STAGE_QUANT_X     a2, block quantization of x; when T*k > 1024 its launch
 *                           also runs the rest of a3 (scan, slot scatter, tile table)
 *   NVFP4_STAGE_ROUTE       no launch of its own (events back to back), except for
 *                           very large routes (more than 65536 histogram entries:
 *                           ceil(T*k / 1024) x num_local), which take separate scan
 *                           and scatter launches here
 *   NVFP4_STAGE_L1          a4 + a5, L1 grouped GEMM with the SiLU*up epilogue
 *   NVFP4_STAGE_QUANT_H     a6, re-quantization of h
 *   NVFP4_STAGE_L2          a7, L2 grouped GEMM
 *   NVFP4_STAGE_SCATTER     a8, weighted scatter
 * A NULL entry skips that record; a NULL events array returns NVFP4_ERR_NULL,
 * a failed event record NVFP4_ERR_HIP. Arguments and results as
 * nvfp4_moe_forward.
 */
enum {
  NVFP4_STAGE_AMAX_ROUTE = 0, NVFP4_STAGE_QUANT_X, NVFP4_STAGE_ROUTE, NVFP4_STAGE_L1, NVFP4_STAGE_QUANT_H,
  NVFP4_STAGE_L2, NVFP4_STAGE_SCATTER, NVFP4_NSTAGES
};
int nvfp4_moe_forward_stage_events(const nvfp4_moe_weights* w, const void* x_bf16, int32_t T,
                                   const int32_t* topk_ids, const float* topk_w, int32_t k, int32_t expert_start,
                                   void* out_bf16, void* ws, size_t ws_bytes, void* const* events, void* stream);

/* The layer with fixed global scales (nvfp4_cutedsl.py history, page 2,
 * static-scale commit: warmup measures gs for the L1 input and for the L1
 * output; inference quantizes with them, no max reduction, no host sync).
 * gs_in: device float [2] = (gs_x, gs_h), e.g. the scalars [0] and [2] that
 * nvfp4_moe_forward leaves in its workspace for a calibration batch. Steps:
 * nvfp4_quantize_static of x with gs_x -> route -> L1 whose epilogue writes h
 * as NVFP4 with gs_h (nvfp4_grouped_gemm_silu_nvfp4) -> L2 (alpha = gs_h *
 * w2_gs[e]) -> weighted scatter. Decode-shaped batches (nvfp4_moe_tile_m ==
 * 32) write BF16 h and quantize it with gs_h in a launch of its own instead.
 * With the gs values nvfp4_moe_forward measured for the same inputs, the
 * output equals nvfp4_moe_forward's bit for bit. Same arguments, workspace
 * and limits as nvfp4_moe_forward; the SCALARS region is left unspecified.
 */
int nvfp4_moe_forward_static(const nvfp4_moe_weights* w, const void* x_bf16, int32_t T,
                             const int32_t* topk_ids, const float* topk_w, int32_t k, int32_t expert_start,
                             const float* gs_in, void* out_bf16, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* NVFP4MOE_H */
