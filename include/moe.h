/*
 * moe.h -- C ABI of the fine-grained MoE layer for MI355X (gfx950).
 *
 * One MoE layer on one GPU: top-K token-choice routing (optionally with token
 * rounding), the gather-fused grouped GEMMs of the forward (up-projection with
 * SwiGLU, down-projection), the weighted expert aggregation, and the
 * memory-efficient backward that keeps only the up-projection output H
 * between forward and backward and recomputes the router gradient from dO and
 * the recomputed activations instead of from a cached down-projection output.
 *
 * Sources (web pages about SonicMoE, cited by title and section):
 *   [A] "DeepSeek做大→Mega MoE，Tri Dao团队加快→SonicMoE" (article on the
 *       authors' Blackwell blog): "MoE 与它的隐患" (standard MoE workflow
 *       figures, routing metadata), "核心创新：一次算法级的重新设计" (reordered
 *       contraction, gather fusion, SwiGLU epilogue, dH kernel), "实验结果"
 *       (problem dimensions T, d, n, E, K).
 *   [B] "SonicMoE：突破细粒度MoE硬件效率瓶颈，实现高稀疏性下的极致训练加速":
 *       algorithm paragraph (router gradient without cached activations),
 *       scheduling paragraph (token rounding to tile multiples), kernel-list
 *       paragraph (up-proj A, down-proj Y, aggregation O; dH, up-proj
 *       gradient, dX, dW1, dW2; host launches kernels by GEMM configuration).
 *
 * Conventions shared by every entry point
 *   - All tensors are dense row-major.  x [T,d], w_r [d,E], w1 [E,d,2n]
 *     (columns 0..n-1 of each expert feed SiLU, columns n..2n-1 are the
 *     "up" half), w2 [E,n,d], o / d_o / dx [T,d], dw_r [d,E], dw1 / dw2 as
 *     w1 / w2.  Element type: desc->dtype (fp32 or bf16) for all of these.
 *     Router scores, gates, per-row score gradients and bias are fp32.
 *   - Every pointer except the host-side moe_desc is a device pointer owned
 *     by the caller.  The library never allocates or frees memory; scratch
 *     space comes from the caller's workspace (moe_workspace_bytes), except
 *     for moe_route_noalloc, which uses one static device array per GPU.
 *   - Calls are stream-ordered and asynchronous on the hipStream_t passed in
 *     (NULL = the default stream); buffers must stay valid until the stream
 *     work completes.  No call synchronises the host.
 *   - Arguments are validated on the host before anything is launched: an
 *     error return means nothing was enqueued.  A launch failure reported by
 *     the runtime returns MOE_EHIP (work enqueued before it may have run).
 *   - Results are bit-identical from run to run (no floating-point atomics).
 *   - Gradients are written, never accumulated.  Every expert's dw1 / dw2
 *     slice is written, zeros for an expert that received no rows.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define MOE_OK          0
#define MOE_EINVAL     -1  /* null pointer, K < 1, K > E, T < 1, bad flag/mode */
#define MOE_ESHAPE     -2  /* dims the kernels do not support (see moe_desc) */
#define MOE_EDTYPE     -3  /* unknown dtype */
#define MOE_EWORKSPACE -4  /* workspace smaller than moe_workspace_bytes */
#define MOE_EHIP       -5  /* the HIP runtime reported an error */
#define MOE_ENOSCRATCH -6  /* moe_route_noalloc: the call needs more scratch
                              than the library's static MOE_SCRATCH_BYTES */

/* element types */
#define MOE_F32  0
#define MOE_BF16 1

/* token rounding modes ([B] scheduling paragraph) */
#define MOE_ROUND_OFF        0
#define MOE_ROUND_NEAREST    1  /* up when count mod tile >= tile/2 */
#define MOE_ROUND_STOCHASTIC 2  /* up with probability (count mod tile)/tile */

/* desc->flags */
#define MOE_FLAG_SCORES_GIVEN 1u  /* moe_route reads routing->logits as the
                                     router scores instead of computing them */
#define MOE_FLAG_GEMM_128     2u  /* run every grouped GEMM with the 128-row
                                     tile kernels (by default bf16 layers whose
                                     sizes are multiples of 256 use 256 x 256
                                     tiles); results agree to rounding, the
                                     workspace size may differ */
#define MOE_FLAG_MXFP8_WGRAD  4u  /* moe_bwd_mxfp8 also runs the two weight-
                                     gradient GEMMs on MXFP8 operands (see
                                     moe_bwd_mxfp8); ignored by the other calls */

/* kernel ids reported in moe_profile.kernel (one per launch, in order) */
#define MOE_K_ROUTER_LOGITS 0   /* z = x w_r + b                                  */
#define MOE_K_ROUTE_SELECT  1   /* top-K, token rounding, segments, token CSR      */
#define MOE_K_UP            2   /* K1: gathered x w1 with the SwiGLU epilogue -> H, A */
#define MOE_K_DOWN          3   /* K2: A w2 -> Y                                   */
#define MOE_K_AGG_O         4   /* K3: O = sum of gate * Y                         */
#define MOE_K_DH            5   /* K4: dO w2^T with the dH epilogue -> dH, A_s, dS */
#define MOE_K_ROUTER_GRAD   6   /* dS partials -> dS, dz per row and dense dz      */
#define MOE_K_DWR           7   /* dw_r = x^T dz                                   */
#define MOE_K_WR_T          8   /* w_r transposed for the dXt router term          */
#define MOE_K_DXT           9   /* K5: dH w1^T + dz w_r^T per row -> dXt           */
#define MOE_K_AGG_DX       10   /* K6: dX = sum of a token's dXt rows              */
#define MOE_K_DW1          11   /* K7: dw1 = x_g^T dH                              */
#define MOE_K_DW2          12   /* K8: dw2 = A_s^T dO_g                            */
#define MOE_K_DB           13   /* db = per-expert sum of dz                       */
/* launched by the unfused layer only (moe_fwd_unfused / moe_bwd_unfused) */
#define MOE_K_GATHER       14   /* rows of x (fwd) or d_o (bwd) gathered per row   */
#define MOE_K_SWIGLU       15   /* A = SwiGLU(H), element-wise                     */
#define MOE_K_ROW_DOT      16   /* dS = <dO_g, Y> per row                          */
#define MOE_K_DA           17   /* dA' = dO_g w2^T                                 */
#define MOE_K_SWIGLU_BWD   18   /* dH, A_s from dA', H, A and the gates            */
/* launched by the MXFP8 forward only (moe_fwd_mxfp8) */
#define MOE_K_MX_QUANT_ROWS 19  /* x or A rows -> E4M3 codes + E8M0 scales         */
#define MOE_K_MX_QUANT_W   20   /* w1 or w2 -> transposed codes + scales           */
#define MOE_K_UP_MX        21   /* K1 on MXFP8 operands (SwiGLU epilogue) -> H, A  */
#define MOE_K_DOWN_MX      22   /* K2 on MXFP8 operands -> Y                       */
#define MOE_K_DXT_MX       23   /* K5 on MXFP8 operands -> dXt (moe_bwd_mxfp8)     */
#define MOE_K_DH_MX        24   /* K4 on MXFP8 operands -> dH, A_s, dS             */
/* launched by moe_bwd_mxfp8 with MOE_FLAG_MXFP8_WGRAD */
#define MOE_K_MX_PAD_OFFSETS 25 /* padded segment offsets and stage -> expert map  */
#define MOE_K_MX_QUANT_SEG 26   /* an expert segment's rows quantized along the rows */
#define MOE_K_DW1_MX       27   /* K7 on MXFP8 operands                            */
#define MOE_K_DW2_MX       28   /* K8 on MXFP8 operands                            */
#define MOE_K_COUNT        29

/* workspace phases */
#define MOE_WS_ROUTE 0
#define MOE_WS_FWD   1
#define MOE_WS_BWD   2
#define MOE_WS_BWD_UNFUSED 3  /* moe_bwd_unfused */
#define MOE_WS_FWD_MXFP8   4  /* moe_fwd_mxfp8 (0 when the shape is unsupported) */
#define MOE_WS_BWD_MXFP8   5  /* moe_bwd_mxfp8 (0 when the shape is unsupported) */

/* internal workspace items exposed for inspection (moe_workspace_offset) */
#define MOE_ITEM_Y        0  /* fwd: down-proj output Y [cap, d] (dtype)          */
#define MOE_ITEM_A        1  /* fwd: SwiGLU output A [cap, n] (dtype)             */
#define MOE_ITEM_DH       2  /* bwd: dH [cap, 2n] (dtype)                         */
#define MOE_ITEM_AS       3  /* bwd: gate-scaled A [cap, n] (dtype)               */
#define MOE_ITEM_DXT      4  /* bwd: per-row input gradient with its router term,
                                dXt_r + dz_r w_r[:, e_r]^T [cap, d] (dtype)    */
#define MOE_ITEM_DS       5  /* bwd: per-row score gradient dS [cap] (fp32)       */
#define MOE_ITEM_DZ       6  /* bwd: per-row router-logit gradient dz [cap] (fp32) */
/* MXFP8 forward workspace (E4M3 codes and E8M0 scale codes are uint8) */
#define MOE_ITEM_MX_XQ    7  /* x codes [T, d]                                    */
#define MOE_ITEM_MX_XS    8  /* x scales [T, d/32]                                */
#define MOE_ITEM_MX_W1Q   9  /* w1 codes, transposed: [E, 2n, d]                  */
#define MOE_ITEM_MX_W1S  10  /* w1 scales [E, d/128, 2n, 4]: byte b of a column's
                                word = block 4g + b along d                       */
#define MOE_ITEM_MX_W2Q  11  /* w2 codes, transposed: [E, d, n]                   */
#define MOE_ITEM_MX_W2S  12  /* w2 scales [E, n/128, d, 4]                        */
#define MOE_ITEM_MX_A    13  /* SwiGLU output A [cap, n] (bf16)                   */
#define MOE_ITEM_MX_AQ   14  /* A codes [cap, n]                                  */
#define MOE_ITEM_MX_AS   15  /* A scales [cap, n/32]                              */
#define MOE_ITEM_MX_Y    16  /* down-proj output Y [cap, d] (bf16)                */
/* MXFP8 backward workspace (its other items sit where MOE_WS_BWD has them) */
#define MOE_ITEM_MX_DHQ  17  /* dH codes [cap, 2n]                                */
#define MOE_ITEM_MX_DHS  18  /* dH scales [cap, 2n/32]                            */
#define MOE_ITEM_MX_W1RQ 19  /* w1 codes along 2n: [E, d, 2n]                     */
#define MOE_ITEM_MX_W1RS 20  /* w1 scales [E, 2n/128, d, 4]                       */
#define MOE_ITEM_MX_DOQ  21  /* d_o codes [T, d]                                  */
#define MOE_ITEM_MX_DOS  22  /* d_o scales [T, d/32]                              */
#define MOE_ITEM_MX_W2RQ 23  /* w2 codes along d: [E, n, d]                       */
#define MOE_ITEM_MX_W2RS 24  /* w2 scales [E, d/128, n, 4]                        */
/* MXFP8 weight gradients (MOE_WS_BWD_MXFP8 with MOE_FLAG_MXFP8_WGRAD).  Each
 * expert's segment of c_e routed rows is padded with zero rows to
 * Kp_e = c_e rounded up to 128 and quantized along its rows; padoff [E+1]
 * int32 holds the prefix of Kp_e.  A segment operand of C columns is, per
 * expert, codes [C][Kp_e] at byte C * padoff[e] and scales as dwords: dword
 * (padoff[e]/128 + s) * C + c = column c's four block scales (bytes b = 0..3:
 * segment rows 128 s + 32 b .. +31) */
#define MOE_ITEM_MX_WG_PADOFF 25  /* padoff [E+1] int32                             */
#define MOE_ITEM_MX_WG_XQ  26  /* x rows gathered per segment, C = d: codes        */
#define MOE_ITEM_MX_WG_XS  27  /*   and scales                                    */
#define MOE_ITEM_MX_WG_HQ  28  /* dH rows (bf16 as the dH kernel wrote them), C = 2n */
#define MOE_ITEM_MX_WG_HS  29
#define MOE_ITEM_MX_WG_AQ  30  /* A_s rows (bf16), C = n                            */
#define MOE_ITEM_MX_WG_AS  31
#define MOE_ITEM_MX_WG_OQ  32  /* d_o rows gathered per segment, C = d              */
#define MOE_ITEM_MX_WG_OS  33

/*
 * Layer description (host struct).
 *   T, d, E, n, K: tokens, hidden size, experts, expert intermediate size,
 *     experts per token ([A] "实验结果" uses these names).
 *   Supported by the kernels: T >= 1, 1 <= K <= E, E % 8 == 0, E <= 1024,
 *     d % 128 == 0, n % 64 == 0, tile 128 or 256 (else MOE_ESHAPE).
 *   dtype: MOE_F32 or MOE_BF16.
 *   round_mode / tile / round_seed: token rounding ([B] scheduling
 *     paragraph): counts become multiples of `tile`, the row tile of the
 *     grouped GEMMs they feed (256 for bf16 layers whose d and n are
 *     multiples of 256, 128 otherwise and with MOE_FLAG_GEMM_128); any
 *     supported value is correct, the matching one removes the most padding.
 *     round_seed drives MOE_ROUND_STOCHASTIC only.
 *   flags: MOE_FLAG_* bits.
 *   profile: NULL, or where to record per-kernel launch timing.
 */
/*
 * Optional launch timing (for measurement only).  When moe_desc.profile is
 * non-NULL, each entry point records start[count] / stop[count] (hipEvent_t
 * handles created by the caller) on its stream around every kernel it
 * launches, stores the kernel's MOE_K_* id in kernel[count] and increments
 * count; entries beyond capacity are not recorded.  The caller reads the
 * elapsed times after the stream has completed.
 */
typedef struct moe_profile {
    int32_t  capacity;
    int32_t  count;
    void**   start;    /* [capacity] hipEvent_t */
    void**   stop;     /* [capacity] hipEvent_t */
    int32_t* kernel;   /* [capacity] host array */
} moe_profile;

typedef struct moe_desc {
    int32_t  T, d, E, n, K;
    int32_t  dtype;
    int32_t  round_mode;
    int32_t  tile;
    uint64_t round_seed;
    uint32_t flags;
    uint32_t reserved;      /* must be 0 */
    moe_profile* profile;   /* NULL, or launch timing (see moe_profile) */
} moe_desc;

/*
 * Routing metadata, written by moe_route and read by moe_fwd / moe_bwd.
 * All device pointers, caller-allocated; cap = moe_row_capacity(desc).
 * This compact form replaces the pages' binary T x E routing mask ([A]
 * "MoE 与它的隐患").  Rows are grouped by expert ("expert-sorted"), and inside
 * an expert in ascending token id.
 *   logits      [T*E] fp32  router scores z = x w_r + bias (an input when
 *                           MOE_FLAG_SCORES_GIVEN is set)
 *   topk_idx    [T*K] int32 per token, the K experts of largest score in
 *                           descending order; equal scores: smaller id first
 *   topk_gate   [T*K] fp32  softmax of the K selected scores, same order
 *   counts      [E]   int32 rows per expert after token rounding
 *   counts_raw  [E]   int32 rows per expert of plain top-K
 *   offsets     [E+1] int32 exclusive prefix sum of counts; offsets[E] = P
 *   tile_offsets[E+1] int32 exclusive prefix sum of ceil(counts/tile)
 *   row_token   [cap] int32 token of each row
 *   row_expert  [cap] int32 expert of each row
 *   row_gate    [cap] fp32  gate of each row: softmax of the token's scores
 *                           over its final expert set
 *   tok_ptr     [T+1] int32 CSR over tokens: rows of token t are
 *   tok_row     [cap] int32 tok_row[tok_ptr[t] .. tok_ptr[t+1]), ascending
 */
typedef struct moe_routing {
    float*   logits;
    int32_t* topk_idx;
    float*   topk_gate;
    int32_t* counts;
    int32_t* counts_raw;
    int32_t* offsets;
    int32_t* tile_offsets;
    int32_t* row_token;
    int32_t* row_expert;
    float*   row_gate;
    int32_t* tok_ptr;
    int32_t* tok_row;
} moe_routing;

/* Upper bound on routed rows P: T*K without rounding, T*K + E*tile/2
 * (nearest) or T*K + E*(tile-1) (stochastic), never above T*E.  The
 * rounding terms follow from [B] scheduling paragraph: each expert's count
 * moves to a multiple of the tile by at most one tile (here by at most
 * tile/2 when rounding to nearest and by at most tile-1 when rounding up at
 * random), and never beyond the T tokens there are.
 * Returns 0 for an invalid descriptor.  Host only. */
size_t moe_row_capacity(const moe_desc* desc);

/* Bytes of device workspace the phase `which` (MOE_WS_*) needs; 0 for an
 * invalid descriptor.  Host only.  The workspace must be 256-byte aligned. */
size_t moe_workspace_bytes(const moe_desc* desc, int which);

/* Byte offset of an internal item (MOE_ITEM_*) inside the workspace of its
 * phase, or (size_t)-1 when the item does not exist.  Host only.  The item
 * holds the value computed by the most recent call of that phase. */
size_t moe_workspace_offset(const moe_desc* desc, int item);

/*
 * Routing ([A] "MoE 与它的隐患": routing metadata; [B] scheduling paragraph).
 *   x [T,d], w_r [d,E] (dtype), bias [E] fp32 or NULL; ignored when
 *   MOE_FLAG_SCORES_GIVEN is set (then routing->logits is read).
 *   Computes the scores, the top-K selection, token rounding when
 *   desc->round_mode != 0, and every other field of *routing.
 *   ws: MOE_WS_ROUTE workspace (ws_bytes >= moe_workspace_bytes).
 *   Integer outputs are exact: the same scores always give the same rows.
 */
int moe_route(const moe_desc* desc, const void* x, const void* w_r, const float* bias,
              const moe_routing* routing, void* ws, size_t ws_bytes, void* stream);

/*
 * Forward ([B] kernel-list paragraph: up-proj A, down-proj Y, aggregation O;
 * [A] second point: gather fusion and SwiGLU in the GEMM epilogue).
 *   x [T,d], w1 [E,d,2n], w2 [E,n,d] (dtype); routing from moe_route.
 *   o [T,d] (dtype): O_t = sum over token t's rows of gate * Y.
 *   h_cache [cap,2n] (dtype): H = x[row_token] w1[e] per row, the only
 *     activation kept for the backward.
 *   ws: MOE_WS_FWD workspace (holds A and Y while the call runs).
 */
int moe_fwd(const moe_desc* desc, const void* x, const void* w1, const void* w2,
            const moe_routing* routing, void* o, void* h_cache, void* ws, size_t ws_bytes,
            void* stream);

/*
 * Backward of L = <d_o, O> ([A] first point: reordered contraction, no Y
 * cached, no extra GEMM; [B] algorithm and kernel-list paragraphs).
 *   Reads x, w_r, w1, w2, routing, h_cache (from moe_fwd), d_o [T,d].
 *   Writes dx [T,d], dw_r [d,E], dw1 [E,d,2n], dw2 [E,n,d] (dtype), and when
 *   non-NULL ds [cap] fp32 (per-row score gradient <dO_t, Y_r>) and
 *   db [E] fp32 (bias gradient; the bias itself is not a trained input).
 *   ws: MOE_WS_BWD workspace.
 */
int moe_bwd(const moe_desc* desc, const void* x, const void* w_r, const void* w1,
            const void* w2, const moe_routing* routing, const void* h_cache, const void* d_o,
            void* dx, void* dw_r, void* dw1, void* dw2, float* ds, float* db, void* ws,
            size_t ws_bytes, void* stream);

/*
 * The unfused layer: the standard MoE workflow that SonicMoE is set against
 * ([A] "MoE 与它的隐患": forward and backward workflow figures; [B] algorithm
 * paragraph), for comparison with moe_fwd / moe_bwd.  Same inputs, outputs,
 * conventions and results (to rounding) as the fused calls; what differs is
 * the work: x and d_o are gathered into per-row buffers by kernels of their
 * own, SwiGLU and its backward run as element-wise kernels between the GEMMs,
 * the per-row activations X_g, H, A and Y are kept from forward to backward,
 * and the score gradient is the row dot product dS_r = <dO_t, Y_r>.
 *
 * moe_unfused_cache_bytes: bytes of that activation cache: the blocks
 *   X_g [cap,d], H [cap,2n], A [cap,n] and Y [cap,d] (dtype, rows in routed
 *   order), in that order, each starting at a 256-byte boundary; 0 for an
 *   invalid descriptor.  Host only.
 * moe_fwd_unfused: as moe_fwd, with `cache` (256-byte aligned, at least
 *   moe_unfused_cache_bytes) in place of h_cache and the forward workspace.
 * moe_bwd_unfused: as moe_bwd, reading `cache` as the forward left it;
 *   ws: MOE_WS_BWD_UNFUSED workspace.
 */
size_t moe_unfused_cache_bytes(const moe_desc* desc);

int moe_fwd_unfused(const moe_desc* desc, const void* x, const void* w1, const void* w2,
                    const moe_routing* routing, void* o, void* cache, size_t cache_bytes, void* stream);

int moe_bwd_unfused(const moe_desc* desc, const void* x, const void* w_r, const void* w1,
                    const void* w2, const moe_routing* routing, const void* cache, const void* d_o,
                    void* dx, void* dw_r, void* dw1, void* dw2, float* ds, float* db, void* ws,
                    size_t ws_bytes, void* stream);

/*
 * Forward with MXFP8 grouped GEMMs (the pages' next precision step, [A]
 * closing "未来展望" paragraph; format: OCP Microscaling (MX) specification
 * v1.0, E4M3 elements, one E8M0 power-of-two scale per 32 values along each
 * GEMM's reduction).  Same arguments and outputs as moe_fwd for a bf16 layer:
 * x, w1 and w2 are quantized inside the call (x and w1 along d, w2 along n;
 * each element rounded to nearest, ties to even, after division by its
 * block scale 2^(floor(log2 amax) - 8); beyond 448 it saturates), the
 * up-projection and down-projection run on the MX-scaled matrix cores with
 * fp32 accumulation, A is quantized along n from its bf16 value, and o and
 * h_cache are written in bf16 as by moe_fwd, so moe_bwd can follow.
 *   Shapes: dtype MOE_BF16 (else MOE_EDTYPE); d and n multiples of 256 and
 *   at most 2048 (else MOE_ESHAPE).
 *   ws: MOE_WS_FWD_MXFP8 workspace.
 */
int moe_fwd_mxfp8(const moe_desc* desc, const void* x, const void* w1, const void* w2,
                  const moe_routing* routing, void* o, void* h_cache, void* ws, size_t ws_bytes,
                  void* stream);

/*
 * Backward with the two activation-gradient GEMMs on MXFP8 operands (E4M3,
 * one E8M0 scale per 32 values, as in moe_fwd_mxfp8): dA' = d_o w2^T with
 * d_o and each expert's w2 quantized along d, feeding the dH epilogue; and
 * dXt = dH w1^T with dH (as that epilogue wrote it, bf16) and each expert's
 * w1 quantized along 2n.  The aggregation and the router backward are
 * moe_bwd's.  The weight-gradient GEMMs are moe_bwd's too, unless
 * desc->flags has MOE_FLAG_MXFP8_WGRAD: then they also take MXFP8 operands,
 * quantized along their reduction, each expert's rows (32-row blocks that
 * start at the expert's first row, the last one zero-padded): dW1[e] =
 * X_g^T dH from the gathered x rows and dH, dW2[e] = A_s^T dO_g from A_s
 * (both as the dH kernel wrote them, bf16) and the gathered d_o rows.  Same
 * arguments and outputs as moe_bwd.
 *   Shapes: those of moe_fwd_mxfp8 with n at most 1024, and with
 *   MOE_FLAG_MXFP8_WGRAD also (cap + 127 E) * max(d, 2n) below 2^31, the
 *   padded segment operands' byte range (else MOE_ESHAPE); dtype MOE_BF16
 *   (else MOE_EDTYPE).
 *   ws: MOE_WS_BWD_MXFP8 workspace (larger with MOE_FLAG_MXFP8_WGRAD).
 */
int moe_bwd_mxfp8(const moe_desc* desc, const void* x, const void* w_r, const void* w1,
                  const void* w2, const moe_routing* routing, const void* h_cache, const void* d_o,
                  void* dx, void* dw_r, void* dw1, void* dw2, float* ds, float* db, void* ws,
                  size_t ws_bytes, void* stream);

/*
 * Routing without a caller workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Same arguments, results and errors as moe_route
 * minus ws / ws_bytes: the routing scratch (membership bytes, row map, and
 * with token rounding the transposed scores and per-token counters) lives in
 * one static device array of MOE_SCRATCH_BYTES per GPU, which each GPU the
 * library runs on holds until the process ends.  The call allocates nothing.
 *   Limit: moe_workspace_bytes(desc, MOE_WS_ROUTE) <= MOE_SCRATCH_BYTES
 *   (about 5 bytes per token and expert without token rounding, 9 with it:
 *   e.g. T = 32768 with E = 256 and rounding off, or E = 128 with rounding),
 *   else MOE_ENOSCRATCH before anything is enqueued.
 *   The first call on a device resolves that device's copy of the array
 *   (make it outside graph capture).  Every call on one GPU uses the same
 *   array: calls that overlap on one GPU (other streams, other threads) race
 *   and must be ordered by the caller.  What the scratch must start with is
 *   cleared inside the call, by kernels (no runtime memset), so the call can
 *   be captured and replayed.
 */
#define MOE_SCRATCH_BYTES ((size_t)64 << 20)
int moe_route_noalloc(const moe_desc* desc, const void* x, const void* w_r, const float* bias,
                      const moe_routing* routing, void* stream);

/* Static text for a status code.  Host only. */
const char* moe_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
