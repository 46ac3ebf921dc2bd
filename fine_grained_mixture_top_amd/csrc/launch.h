// Internal launchers shared by the translation units of the MoE library.
// Every launcher only enqueues work on `st` and returns the runtime status of
// the launch; all shapes were validated by the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

enum Dtype { DT_F32 = 0, DT_BF16 = 1 };

// Sizes every grouped GEMM launcher needs: element type, layer sizes, row
// capacity of the per-row buffers, and whether to keep to the 128-row tile
// kernels.
struct GemmDims {
  int dtype;
  int T, d, E, n;
  size_t cap;
  bool small_tiles;
};

// Column tile of the dH GEMM, which decides how many fp32 score-gradient
// partials each row gets (n / dh_block(g)).
int dh_block(const GemmDims& g);
inline int dh_partials(const GemmDims& g) { return g.n / dh_block(g); }

// ---- grouped GEMMs (gemm_kernels.hip) ----
hipError_t launch_router_logits(int dtype, const void* x, const void* w_r, const float* bias,
                                float* logits, int T, int d, int E, hipStream_t st);
hipError_t launch_up_swiglu(const GemmDims& g, const void* x, const void* w1, const int32_t* row_token,
                            const int32_t* offsets, void* H, void* A, hipStream_t st);
hipError_t launch_down(const GemmDims& g, const void* A, const void* w2, const int32_t* offsets, void* Y,
                       hipStream_t st);
hipError_t launch_dh(const GemmDims& g, const void* d_o, const void* w2, const void* H,
                     const int32_t* row_token, const float* row_gate, const int32_t* offsets, void* dH,
                     void* As, float* dS_part, hipStream_t st);
// dXt = dH W1^T plus, per row r, the router term dz[r] * w_rT[e_r] ([E][d],
// the transposed router weights)
hipError_t launch_dxt(const GemmDims& g, const void* dH, const void* w1, const int32_t* offsets, void* dXt,
                      const float* dz, const void* w_rT, hipStream_t st);
// dW1 / dW2: `ws` (wgt_ws_bytes(g) bytes, 256-byte aligned; may be null when
// that is 0) holds the tile plan and the fp32 partial sums of experts whose
// reduction is split.
hipError_t launch_dw1(const GemmDims& g, const void* x, const void* dH, const int32_t* row_token,
                      const int32_t* offsets, void* dW1, void* ws, hipStream_t st);
hipError_t launch_dw2(const GemmDims& g, const void* As, const void* d_o, const int32_t* row_token,
                      const int32_t* offsets, void* dW2, void* ws, hipStream_t st);
size_t wgt_ws_bytes(const GemmDims& g);
// dW1 / dW2 also take row_token = null: x (dO) is then already gathered per
// row ([cap][d]).

// C[r] = A[r] W[e_r] over the routed rows (no gather); W[e] is [K][N] when
// w_kn, else [N][K]; A [cap][K], C [cap][N] (dtype).  Unfused layer.
hipError_t launch_rows_gemm(const GemmDims& g, const void* A, int K, const void* W, int N, bool w_kn,
                            const int32_t* offsets, void* C, hipStream_t st);

// ---- MXFP8 forward (mx_kernels.hip) ----
// Shapes the MX GEMMs take: bf16 layer, d and n multiples of 256, at most 2048.
bool mx_shape_ok(const GemmDims& g);
// rows [rows][K] bf16 -> E4M3 codes [rows][K] and E8M0 scales [rows][K/32];
// nrows (device) bounds the rows when set.
hipError_t launch_mx_quant_rows(const void* src, int K, long long rows, const int32_t* nrows, uint8_t* q,
                                uint8_t* s, hipStream_t st, int bN = 0);
// the MXFP8 activation-gradient GEMM also takes 2n (<= 2048) as a reduction
bool mx_bwd_shape_ok(const GemmDims& g);
// score-gradient partials per row that launch_dh_mx writes (its column tile
// is fixed, whatever dh_block(g) picks for the bf16 dH kernel)
int dh_mx_partials(const GemmDims& g);
// dXt = dH W1^T on MXFP8 operands: dH codes [cap][2n] and scales [cap][2n/32],
// W1 codes [E][d][2n] (rows along 2n) and scales [E][2n/128][d][4]; the
// router term as launch_dxt
hipError_t launch_dxt_mx(const GemmDims& g, const uint8_t* dhq, const uint8_t* dhs, const uint8_t* w1q,
                         const uint8_t* w1s, const int32_t* offsets, void* dXt, const float* dz, const void* w_rT,
                         hipStream_t st);
// dA' = dO W2^T on MXFP8 operands with the dH epilogue (as launch_dh): dO
// codes [T][d] and scales [T][d/32] gathered per row, W2 codes [E][n][d]
// (rows along d) and scales [E][d/128][n][4]; dS partials: n / 256 per row
hipError_t launch_dh_mx(const GemmDims& g, const uint8_t* doq, const uint8_t* dos, const uint8_t* w2q,
                        const uint8_t* w2s, const int32_t* row_token, const float* row_gate, const int32_t* offsets,
                        const void* H, void* dH, void* As, float* dS_part, hipStream_t st);
// MXFP8 weight gradients.  Each expert's segment of routed rows, padded
// with zero rows to a multiple of 128 (one GEMM stage), is quantized along
// its rows.  padoff [E+1]: prefix of the padded lengths; stage_e: the expert
// of each 128-row stage (mx_seg_rows_bound(g) / 128 entries at most).
long long mx_seg_rows_bound(const GemmDims& g);
bool mx_wgrad_shape_ok(const GemmDims& g);
hipError_t launch_mx_pad_offsets(const int32_t* offsets, int E, int32_t* padoff, int32_t* stage_e, hipStream_t st);
// src rows [*][C] bf16 (gathered through idx when set) -> codes, per expert
// [C][Kp_e] at byte C * padoff[e], and stage-blocked scales (dword
// (padoff[e]/128 + s) * C + c: column c's four block scales of stage s)
hipError_t launch_mx_quant_seg(const void* src, int C, const int32_t* idx, const int32_t* offsets,
                               const int32_t* padoff, const int32_t* stage_e, const GemmDims& g, uint8_t* q,
                               uint32_t* sblk, hipStream_t st);
// dW[e] (Ma x Nb, bf16) = A_e B_e^T from segment-quantized operands A (Ma
// columns) and B (Nb columns)
hipError_t launch_wgrad_mx(const GemmDims& g, int Ma, int Nb, const int32_t* padoff, const uint8_t* qa,
                           const uint32_t* sa, const uint8_t* qb, const uint32_t* sb, void* dW, hipStream_t st);
// W [E][K][N] bf16 -> codes [E][N][K] and scales [E][K/128][N] (4 bytes each)
hipError_t launch_mx_quant_w(const void* W, int E, int K, int N, uint8_t* q, uint8_t* sblk, hipStream_t st);
hipError_t launch_up_mx(const GemmDims& g, const uint8_t* xq, const uint8_t* xs, const uint8_t* w1q,
                        const uint8_t* w1s, const int32_t* row_token, const int32_t* offsets, void* H, void* A,
                        hipStream_t st);
hipError_t launch_down_mx(const GemmDims& g, const uint8_t* aq, const uint8_t* as, const uint8_t* w2q,
                          const uint8_t* w2s, const int32_t* offsets, void* Y, hipStream_t st);

// ---- unfused layer (unfused_kernels.hip); rows 0 .. *nrows-1 of cap ----
hipError_t launch_gather_rows(int dtype, const void* src, int width, const int32_t* idx, const int32_t* nrows,
                              size_t cap, void* dst, hipStream_t st);
hipError_t launch_swiglu_fwd(int dtype, const void* H, int n, const int32_t* nrows, size_t cap, void* A,
                             hipStream_t st);
hipError_t launch_row_dot(int dtype, const void* a, const void* b, int width, const int32_t* nrows, size_t cap,
                          float* out, hipStream_t st);
hipError_t launch_swiglu_bwd(int dtype, const void* dAp, const void* H, const void* A, const float* gate, int n,
                             const int32_t* nrows, size_t cap, void* dH, void* As, hipStream_t st);
// dW_r = x^T dz_dense, reduction split in dwr_splits() chunks whose fp32
// partials ([splits][d][E]) go to `partials` and are then summed in order.
int dwr_splits(int T, int d, int E);
hipError_t launch_dwr(int dtype, const void* x, const void* dz_dense, int T, int d, int E,
                      void* dWr, float* partials, hipStream_t st);

// ---- routing (route_kernels.hip) ----
struct RouteBufs {
  float* logits;
  int32_t* topk_idx;
  float* topk_gate;
  int32_t* counts;
  int32_t* counts_raw;
  int32_t* offsets;
  int32_t* tile_offsets;
  int32_t* row_token;
  int32_t* row_expert;
  float* row_gate;
  int32_t* tok_ptr;
  int32_t* tok_row;
};
// Membership rows are padded to mask_pitch(T) tokens (16-byte aligned).
int mask_pitch(int T);
struct RouteScratch {
  uint8_t* mask;       // [E][pitch] membership bytes
  float* scoresT;      // [E][pitch] scores, expert-major (token rounding only)
  int32_t* rowmap;     // [E][pitch] row of (e, t)
  int32_t* tblk;       // rows per 64-token block, then their scan (token rounding only)
  float* tstat;        // [2][T] set-softmax max and sum per token (token rounding only)
  int32_t* chunk_cnt;  // [E][route_chunks(T)] member counts per chunk of 4096 tokens
};
// chunks of 4096 tokens of the membership rows
int route_chunks(int T);
hipError_t launch_route_select(const RouteBufs& rb, const RouteScratch& sc, int T, int E, int K,
                               int tile, int round_mode, uint64_t round_seed, hipStream_t st);

// ---- aggregation and router backward (aggregate_kernels.hip) ----
hipError_t launch_aggregate_o(int dtype, const void* Y, const float* row_gate,
                              const int32_t* tok_ptr, const int32_t* tok_row, int T, int d,
                              void* O, hipStream_t st);
hipError_t launch_bias_grad(const float* dz_row, const int32_t* offsets, int E, float* db,
                            hipStream_t st);
hipError_t launch_transpose(int dtype, const void* src, int rows, int cols, void* dst,
                            hipStream_t st);
// router backward per token (see aggregate_kernels.hip)
struct RouterDzArgs {
  const float* dS_part;    // [cap][nparts] dH-epilogue partials of dS
  int nparts;
  const float* row_gate;   // [cap]
  const int32_t* row_expert;
  const int32_t* tok_ptr;  // [T+1]
  const int32_t* tok_row;  // [cap]
  int T, E;
  float* dS_row;           // [cap] out
  float* dz_row;           // [cap] out
  void* dz_dense;          // [T][E] out (dtype)
};
hipError_t launch_router_dz(int dtype, const RouterDzArgs& a, hipStream_t st);
// dX[t] = sum over token t's rows of dXt[r] (rows with their router term)
hipError_t launch_aggregate_dx(int dtype, const void* dXt, const int32_t* tok_ptr, const int32_t* tok_row, int T,
                               int d, void* dX, hipStream_t st);
}  // namespace moe
