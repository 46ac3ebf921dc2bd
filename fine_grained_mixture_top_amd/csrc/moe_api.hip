// C ABI of the MoE layer (declared in include/moe.h): argument validation,
// workspace layout and the launch sequence of each phase.  Everything here
// runs on the host; it only enqueues kernels on the caller's stream.
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/moe.h"
#include "launch.h"

// Routing scratch of moe_route_noalloc: one copy per GPU, alive until the
// process ends.  Host code never passes this name to a kernel (on the host it
// is only a stand-in for the symbol); it uses the device address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[MOE_SCRATCH_BYTES];

namespace {

using namespace moe;

constexpr size_t ALIGN = 256;
size_t up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

size_t elem_size(int dtype) { return dtype == MOE_BF16 ? 2 : 4; }

int validate_desc(const moe_desc* d) {
  if (!d) return MOE_EINVAL;
  if (d->reserved != 0) return MOE_EINVAL;
  if ((d->flags & ~(MOE_FLAG_SCORES_GIVEN | MOE_FLAG_GEMM_128 | MOE_FLAG_MXFP8_WGRAD)) != 0) return MOE_EINVAL;
  if (d->T < 1 || d->d < 1 || d->E < 1 || d->n < 1 || d->K < 1 || d->K > d->E) return MOE_EINVAL;
  if (d->round_mode < MOE_ROUND_OFF || d->round_mode > MOE_ROUND_STOCHASTIC) return MOE_EINVAL;
  if (d->dtype != MOE_F32 && d->dtype != MOE_BF16) return MOE_EDTYPE;
  if (d->tile != 128 && d->tile != 256) return MOE_ESHAPE;
  if (d->E % 8 != 0 || d->E > 1024) return MOE_ESHAPE;
  if (d->d % 128 != 0 || d->n % 64 != 0) return MOE_ESHAPE;
  if ((int64_t)d->T * d->E > INT32_MAX - 1) return MOE_ESHAPE;  // rows are int32
  return MOE_OK;
}

size_t capacity(const moe_desc* d) {
  size_t base = (size_t)d->T * d->K;
  size_t extra = 0;
  if (d->round_mode == MOE_ROUND_NEAREST) extra = (size_t)d->E * (d->tile / 2);
  if (d->round_mode == MOE_ROUND_STOCHASTIC) extra = (size_t)d->E * (d->tile - 1);
  size_t cap = base + extra;
  size_t all = (size_t)d->T * d->E;
  return cap < all ? cap : all;
}

// Workspace items, in order, for each phase.
struct Layout {
  size_t off[32];
  size_t total;
};

Layout route_layout(const moe_desc* d) {
  Layout L{};
  size_t o = 0;
  const size_t TEp = (size_t)mask_pitch(d->T) * d->E;
  const size_t tr = d->round_mode ? 1 : 0;
  L.off[0] = o; o = up(o + TEp);                                  // mask
  L.off[1] = o; o = up(o + tr * TEp * 4);                         // scoresT
  L.off[2] = o; o = up(o + TEp * 4);                              // rowmap
  L.off[3] = o; o = up(o + tr * 2 * ((size_t)(d->T + 63) / 64 + 4) * 4);  // 64-token block sums, offsets
  L.off[4] = o; o = up(o + tr * (size_t)d->T * 8);                // tstat
  L.off[5] = o; o = up(o + (size_t)d->E * route_chunks(d->T) * 4); // chunk counts
  L.total = o;
  return L;
}

GemmDims gemm_dims(const moe_desc* d) {
  return GemmDims{d->dtype, d->T, d->d, d->E, d->n, capacity(d), (d->flags & MOE_FLAG_GEMM_128) != 0};
}

Layout fwd_layout(const moe_desc* d) {
  Layout L{};
  const size_t cap = capacity(d), es = elem_size(d->dtype);
  size_t o = 0;
  L.off[0] = o; o = up(o + cap * d->n * es);   // A
  L.off[1] = o; o = up(o + cap * d->d * es);   // Y
  L.total = o;
  return L;
}

Layout bwd_layout(const moe_desc* d) {
  Layout L{};
  const size_t cap = capacity(d), es = elem_size(d->dtype);
  const size_t np = (size_t)dh_partials(gemm_dims(d));
  size_t o = 0;
  L.off[0] = o; o = up(o + cap * 2 * d->n * es);          // dH
  L.off[1] = o; o = up(o + cap * d->n * es);              // A_s
  L.off[2] = o; o = up(o + cap * np * 4);                 // dS partials
  L.off[3] = o; o = up(o + cap * 4);                      // dS per row
  L.off[4] = o; o = up(o + cap * 4);                      // dz per row
  L.off[5] = o; o = up(o + (size_t)d->T * d->E * es);     // dz dense [T][E]
  L.off[6] = o; o = up(o + (size_t)d->E * d->d * es);     // W_r^T [E][d]
  L.off[7] = o; o = up(o + cap * d->d * es);              // dXt
  L.off[8] = o; o = up(o + (size_t)dwr_splits(d->T, d->d, d->E) * d->d * d->E * 4);  // dW_r partials
  L.off[9] = o; o = up(o + wgt_ws_bytes(gemm_dims(d)));                               // dW1 / dW2 plan + partials
  L.total = o;
  return L;
}

// Unfused layer: the activation cache kept from forward to backward holds the
// gathered inputs X_g, H, A and Y of every routed row.
Layout unfused_cache_layout(const moe_desc* d) {
  Layout L{};
  const size_t cap = capacity(d), es = elem_size(d->dtype);
  size_t o = 0;
  L.off[0] = o; o = up(o + cap * d->d * es);       // X_g
  L.off[1] = o; o = up(o + cap * 2 * d->n * es);   // H
  L.off[2] = o; o = up(o + cap * d->n * es);       // A
  L.off[3] = o; o = up(o + cap * d->d * es);       // Y
  L.total = o;
  return L;
}

Layout unfused_bwd_layout(const moe_desc* d) {
  Layout L{};
  const size_t cap = capacity(d), es = elem_size(d->dtype);
  size_t o = 0;
  L.off[0] = o; o = up(o + cap * d->d * es);              // dO_g
  L.off[1] = o; o = up(o + cap * d->n * es);              // dA' = dO_g W2^T
  L.off[2] = o; o = up(o + cap * 2 * d->n * es);          // dH
  L.off[3] = o; o = up(o + cap * d->n * es);              // A_s
  L.off[4] = o; o = up(o + cap * 4 * 3);                  // dS = <dO_g, Y>, dS per row, dz per row
  L.off[5] = o; o = up(o + (size_t)d->T * d->E * es);     // dz dense [T][E]
  L.off[6] = o; o = up(o + (size_t)d->E * d->d * es);     // W_r^T [E][d]
  L.off[7] = o; o = up(o + cap * d->d * es);              // dXt
  L.off[8] = o; o = up(o + (size_t)dwr_splits(d->T, d->d, d->E) * d->d * d->E * 4);  // dW_r partials
  L.off[9] = o; o = up(o + wgt_ws_bytes(gemm_dims(d)));                               // dW1 / dW2 plan + partials
  L.total = o;
  return L;
}

// MXFP8 forward workspace: quantized operands, A (bf16 and quantized), Y.
Layout mx_fwd_layout(const moe_desc* d) {
  Layout L{};
  const size_t cap = capacity(d), T = d->T, D = d->d, n = d->n, E = d->E;
  size_t o = 0;
  L.off[0] = o; o = up(o + T * D);                       // x codes [T][d]
  L.off[1] = o; o = up(o + T * (D / 32));                // x scales [T][d/32]
  L.off[2] = o; o = up(o + E * 2 * n * D);               // W1^T codes [E][2n][d]
  L.off[3] = o; o = up(o + E * (D / 128) * 2 * n * 4);   // W1 scales [E][d/128][2n][4]
  L.off[4] = o; o = up(o + E * D * n);                   // W2^T codes [E][d][n]
  L.off[5] = o; o = up(o + E * (n / 128) * D * 4);       // W2 scales [E][n/128][d][4]
  L.off[6] = o; o = up(o + cap * n * 2);                 // A (bf16)
  L.off[7] = o; o = up(o + cap * n);                     // A codes [cap][n]
  L.off[8] = o; o = up(o + cap * (n / 32));              // A scales [cap][n/32]
  L.off[9] = o; o = up(o + cap * D * 2);                 // Y (bf16)
  L.total = o;
  return L;
}

// MXFP8 backward workspace: the bf16 backward's items, then the quantized
// operands of the two activation-gradient GEMMs.
Layout mx_bwd_layout(const moe_desc* d) {
  Layout L = bwd_layout(d);
  const size_t cap = capacity(d), D = d->d, n = d->n, E = d->E;
  size_t o = L.total;
  L.off[10] = o; o = up(o + cap * 2 * n);                 // dH codes [cap][2n]
  L.off[11] = o; o = up(o + cap * (2 * n / 32));          // dH scales [cap][2n/32]
  L.off[12] = o; o = up(o + E * D * 2 * n);               // W1 codes, rows along 2n [E][d][2n]
  L.off[13] = o; o = up(o + E * (2 * n / 128) * D * 4);   // W1 scales [E][2n/128][d][4]
  L.off[14] = o; o = up(o + (size_t)d->T * D);            // dO codes [T][d]
  L.off[15] = o; o = up(o + (size_t)d->T * (D / 32));     // dO scales [T][d/32]
  L.off[16] = o; o = up(o + E * n * D);                   // W2 codes, rows along d [E][n][d]
  L.off[17] = o; o = up(o + E * (D / 128) * n * 4);       // W2 scales [E][d/128][n][4]
  if (d->flags & MOE_FLAG_MXFP8_WGRAD) {
    // weight-gradient operands quantized along each expert's padded rows
    const size_t rows = (size_t)mx_seg_rows_bound(gemm_dims(d));
    L.off[18] = o; o = up(o + (E + 1) * 4);                 // padoff [E+1]
    L.off[19] = o; o = up(o + rows / 128 * 4);              // expert of each 128-row stage
    const size_t cols[4] = {D, 2 * n, n, D};                // x_g, dH, A_s, dO_g
    for (int i = 0; i < 4; ++i) {
      L.off[20 + 2 * i] = o; o = up(o + cols[i] * rows);    // codes
      L.off[21 + 2 * i] = o; o = up(o + cols[i] * rows / 32);  // scales
    }
  }
  L.total = o;
  return L;
}

// shapes moe_bwd_mxfp8 takes (with the weight-gradient GEMMs too when flagged)
bool mx_bwd_ok(const moe_desc* d) {
  const GemmDims g = gemm_dims(d);
  if (!mx_bwd_shape_ok(g)) return false;
  return !(d->flags & MOE_FLAG_MXFP8_WGRAD) || mx_wgrad_shape_ok(g);
}

int check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return MOE_OK;
  if (!ws) return MOE_EINVAL;
  if (((uintptr_t)ws & (ALIGN - 1)) != 0) return MOE_EINVAL;
  if (ws_bytes < need) return MOE_EWORKSPACE;
  return MOE_OK;
}

bool routing_ok(const moe_routing* r) {
  return r && r->logits && r->topk_idx && r->topk_gate && r->counts && r->counts_raw && r->offsets &&
         r->tile_offsets && r->row_token && r->row_expert && r->row_gate && r->tok_ptr && r->tok_row;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

// Event pair around one launch when the caller asked for timing.
struct Timed {
  moe_profile* p;
  hipStream_t st;
  int slot;
  Timed(const moe_desc* d, hipStream_t s, int kernel) : p(d->profile), st(s), slot(-1) {
    if (p && p->count < p->capacity && p->start && p->stop) {
      slot = p->count++;
      if (p->kernel) p->kernel[slot] = kernel;
      (void)hipEventRecord((hipEvent_t)p->start[slot], st);
    }
  }
  ~Timed() {
    if (slot >= 0) (void)hipEventRecord((hipEvent_t)p->stop[slot], st);
  }
};

#define MOE_TRY(kid, expr)                    \
  do {                                        \
    Timed _t(desc, st, (kid));                \
    hipError_t _e = (expr);                   \
    if (_e != hipSuccess) return MOE_EHIP;    \
  } while (0)

}  // namespace

extern "C" {

size_t moe_row_capacity(const moe_desc* desc) {
  if (validate_desc(desc) != MOE_OK) return 0;
  return capacity(desc);
}

size_t moe_workspace_bytes(const moe_desc* desc, int which) {
  if (validate_desc(desc) != MOE_OK) return 0;
  switch (which) {
    case MOE_WS_ROUTE: return route_layout(desc).total;
    case MOE_WS_FWD: return fwd_layout(desc).total;
    case MOE_WS_BWD: return bwd_layout(desc).total;
    case MOE_WS_BWD_UNFUSED: return unfused_bwd_layout(desc).total;
    case MOE_WS_FWD_MXFP8: return mx_shape_ok(gemm_dims(desc)) ? mx_fwd_layout(desc).total : 0;
    case MOE_WS_BWD_MXFP8: return mx_bwd_ok(desc) ? mx_bwd_layout(desc).total : 0;
    default: return 0;
  }
}

size_t moe_workspace_offset(const moe_desc* desc, int item) {
  if (validate_desc(desc) != MOE_OK) return (size_t)-1;
  switch (item) {
    case MOE_ITEM_A: return fwd_layout(desc).off[0];
    case MOE_ITEM_Y: return fwd_layout(desc).off[1];
    case MOE_ITEM_DH: return bwd_layout(desc).off[0];
    case MOE_ITEM_AS: return bwd_layout(desc).off[1];
    case MOE_ITEM_DS: return bwd_layout(desc).off[3];
    case MOE_ITEM_DZ: return bwd_layout(desc).off[4];
    case MOE_ITEM_DXT: return bwd_layout(desc).off[7];
    default: break;
  }
  if (item >= MOE_ITEM_MX_XQ && item <= MOE_ITEM_MX_Y) {
    if (!mx_shape_ok(gemm_dims(desc))) return (size_t)-1;
    return mx_fwd_layout(desc).off[item - MOE_ITEM_MX_XQ];
  }
  if (item >= MOE_ITEM_MX_DHQ && item <= MOE_ITEM_MX_W2RS) {
    if (!mx_bwd_ok(desc)) return (size_t)-1;
    return mx_bwd_layout(desc).off[10 + item - MOE_ITEM_MX_DHQ];
  }
  if (item >= MOE_ITEM_MX_WG_PADOFF && item <= MOE_ITEM_MX_WG_OS) {
    if (!mx_bwd_ok(desc) || !(desc->flags & MOE_FLAG_MXFP8_WGRAD)) return (size_t)-1;
    const Layout L = mx_bwd_layout(desc);
    return item == MOE_ITEM_MX_WG_PADOFF ? L.off[18] : L.off[20 + item - MOE_ITEM_MX_WG_XQ];
  }
  return (size_t)-1;
}

}  // extern "C"

namespace {

// Device address of this GPU's copy of `scratch`, resolved once per device
// (with that device current) and kept; null if the runtime fails.
constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
void* scratch_dev[MAX_DEVICES] = {};

void* scratch_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    scratch_dev[dev] = p;
  }
  return scratch_dev[dev];
}

int route_checks(const moe_desc* desc, const void* x, const void* w_r, const moe_routing* routing) {
  int s = validate_desc(desc);
  if (s != MOE_OK) return s;
  const bool given = (desc->flags & MOE_FLAG_SCORES_GIVEN) != 0;
  if (!routing_ok(routing)) return MOE_EINVAL;
  if (!given && (!x || !w_r)) return MOE_EINVAL;
  return MOE_OK;
}

// The routing launch sequence on a validated descriptor; `ws` holds
// route_layout(desc).total bytes.
int route_impl(const moe_desc* desc, const void* x, const void* w_r, const float* bias,
               const moe_routing* routing, char* ws, void* stream) {
  const bool given = (desc->flags & MOE_FLAG_SCORES_GIVEN) != 0;
  const Layout L = route_layout(desc);
  hipStream_t st = (hipStream_t)stream;
  char* w = ws;
  if (!given)
    MOE_TRY(MOE_K_ROUTER_LOGITS,
            launch_router_logits(desc->dtype, x, w_r, bias, routing->logits, desc->T, desc->d, desc->E, st));
  RouteBufs rb{routing->logits,     routing->topk_idx,  routing->topk_gate, routing->counts,
               routing->counts_raw, routing->offsets,   routing->tile_offsets, routing->row_token,
               routing->row_expert, routing->row_gate,  routing->tok_ptr,   routing->tok_row};
  const bool tr = desc->round_mode != 0;
  RouteScratch sc{(uint8_t*)(w + L.off[0]), tr ? (float*)(w + L.off[1]) : nullptr, (int32_t*)(w + L.off[2]),
                  tr ? (int32_t*)(w + L.off[3]) : nullptr, tr ? (float*)(w + L.off[4]) : nullptr,
                  (int32_t*)(w + L.off[5])};
  MOE_TRY(MOE_K_ROUTE_SELECT, launch_route_select(rb, sc, desc->T, desc->E, desc->K, desc->tile,
                                                  desc->round_mode, desc->round_seed, st));
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_route(const moe_desc* desc, const void* x, const void* w_r, const float* bias,
              const moe_routing* routing, void* ws, size_t ws_bytes, void* stream) {
  int s = route_checks(desc, x, w_r, routing);
  if (s != MOE_OK) return s;
  if ((s = check_ws(ws, ws_bytes, route_layout(desc).total)) != MOE_OK) return s;
  return route_impl(desc, x, w_r, bias, routing, (char*)ws, stream);
}

int moe_route_noalloc(const moe_desc* desc, const void* x, const void* w_r, const float* bias,
                      const moe_routing* routing, void* stream) {
  int s = route_checks(desc, x, w_r, routing);
  if (s != MOE_OK) return s;
  if (route_layout(desc).total > MOE_SCRATCH_BYTES) return MOE_ENOSCRATCH;
  void* ws = scratch_for_current_device();
  if (!ws) return MOE_EHIP;
  return route_impl(desc, x, w_r, bias, routing, (char*)ws, stream);
}

int moe_fwd(const moe_desc* desc, const void* x, const void* w1, const void* w2,
            const moe_routing* routing, void* o, void* h_cache, void* ws, size_t ws_bytes, void* stream) {
  int s = validate_desc(desc);
  if (s != MOE_OK) return s;
  if (!x || !w1 || !w2 || !o || !h_cache || !routing_ok(routing)) return MOE_EINVAL;
  const Layout L = fwd_layout(desc);
  if ((s = check_ws(ws, ws_bytes, L.total)) != MOE_OK) return s;

  hipStream_t st = (hipStream_t)stream;
  char* w = (char*)ws;
  void* A = w + L.off[0];
  void* Y = w + L.off[1];
  const size_t cap = capacity(desc);
  const moe_desc& D = *desc;
  const GemmDims g = gemm_dims(desc);
  MOE_TRY(MOE_K_UP, launch_up_swiglu(g, x, w1, routing->row_token, routing->offsets, h_cache, A, st));
  MOE_TRY(MOE_K_DOWN, launch_down(g, A, w2, routing->offsets, Y, st));
  MOE_TRY(MOE_K_AGG_O, launch_aggregate_o(D.dtype, Y, routing->row_gate, routing->tok_ptr, routing->tok_row, D.T, D.d, o,
                             st));
  return MOE_OK;
}

}  // extern "C"

namespace {
// The backward's launch sequence; mx: the two activation-gradient GEMMs on
// MXFP8 operands (workspace laid out by mx_bwd_layout).
int bwd_impl(const moe_desc* desc, const void* x, const void* w_r, const void* w1, const void* w2,
             const moe_routing* routing, const void* h_cache, const void* d_o, void* dx, void* dw_r, void* dw1,
             void* dw2, float* ds, float* db, void* ws, size_t ws_bytes, void* stream, bool mx) {
  int s = validate_desc(desc);
  if (s != MOE_OK) return s;
  if (mx) {
    if (desc->dtype != MOE_BF16) return MOE_EDTYPE;
    if (!mx_bwd_ok(desc)) return MOE_ESHAPE;
  }
  if (!x || !w_r || !w1 || !w2 || !h_cache || !d_o || !dx || !dw_r || !dw1 || !dw2 || !routing_ok(routing))
    return MOE_EINVAL;
  const Layout L = mx ? mx_bwd_layout(desc) : bwd_layout(desc);
  if ((s = check_ws(ws, ws_bytes, L.total)) != MOE_OK) return s;

  hipStream_t st = (hipStream_t)stream;
  char* w = (char*)ws;
  const moe_desc& D = *desc;
  const size_t cap = capacity(desc);
  void* dH = w + L.off[0];
  void* As = w + L.off[1];
  float* dS_part = (float*)(w + L.off[2]);
  float* dS_row = ds ? ds : (float*)(w + L.off[3]);
  float* dz_row = (float*)(w + L.off[4]);
  void* dz_dense = w + L.off[5];
  void* w_rT = w + L.off[6];
  void* dXt = w + L.off[7];
  const moe_routing& R = *routing;

  // dH kernel: dA' = dO W2^T with the recompute-A epilogue (dH, A_s, dS parts)
  const GemmDims g = gemm_dims(desc);
  if (mx) {
    // dO and W2 quantized along d (W2 by the rows of each expert's [n][d])
    uint8_t *doq = (uint8_t*)(w + L.off[14]), *dos = (uint8_t*)(w + L.off[15]);
    uint8_t *w2q = (uint8_t*)(w + L.off[16]), *w2s = (uint8_t*)(w + L.off[17]);
    MOE_TRY(MOE_K_MX_QUANT_ROWS, launch_mx_quant_rows(d_o, D.d, D.T, nullptr, doq, dos, st));
    MOE_TRY(MOE_K_MX_QUANT_W, launch_mx_quant_rows(w2, D.d, (long long)D.E * D.n, nullptr, w2q, w2s, st, D.n));
    MOE_TRY(MOE_K_DH_MX, launch_dh_mx(g, doq, dos, w2q, w2s, R.row_token, R.row_gate, R.offsets, h_cache, dH, As,
                                      dS_part, st));
  } else {
    MOE_TRY(MOE_K_DH, launch_dh(g, d_o, w2, h_cache, R.row_token, R.row_gate, R.offsets, dH, As, dS_part, st));
  }
  // router backward (dS -> dz per row and dense), then the activation
  // gradient: dXt = dH W1^T with each row's router term dz_r W_r^T[e_r] added
  // in the GEMM's epilogue, dX = the sum of a token's dXt rows; then
  // dW_r = X^T dz
  MOE_TRY(MOE_K_WR_T, launch_transpose(D.dtype, w_r, D.d, D.E, w_rT, st));
  {
    // the dS partial count is that of the dH kernel actually launched
    const int nparts = mx ? dh_mx_partials(g) : dh_partials(g);
    const RouterDzArgs ra{dS_part, nparts, R.row_gate, R.row_expert, R.tok_ptr, R.tok_row, D.T, D.E,
                          dS_row,  dz_row, dz_dense};
    MOE_TRY(MOE_K_ROUTER_GRAD, launch_router_dz(D.dtype, ra, st));
  }
  if (mx) {
    // dH and W1 quantized along 2n (dH from the bf16 values just written)
    uint8_t *dhq = (uint8_t*)(w + L.off[10]), *dhs = (uint8_t*)(w + L.off[11]);
    uint8_t *w1q = (uint8_t*)(w + L.off[12]), *w1s = (uint8_t*)(w + L.off[13]);
    MOE_TRY(MOE_K_MX_QUANT_ROWS, launch_mx_quant_rows(dH, 2 * D.n, (long long)cap, R.offsets + D.E, dhq, dhs, st));
    MOE_TRY(MOE_K_MX_QUANT_W, launch_mx_quant_rows(w1, 2 * D.n, (long long)D.E * D.d, nullptr, w1q, w1s, st, D.d));
    MOE_TRY(MOE_K_DXT_MX, launch_dxt_mx(g, dhq, dhs, w1q, w1s, R.offsets, dXt, dz_row, w_rT, st));
  } else {
    MOE_TRY(MOE_K_DXT, launch_dxt(g, dH, w1, R.offsets, dXt, dz_row, w_rT, st));
  }
  MOE_TRY(MOE_K_AGG_DX, launch_aggregate_dx(D.dtype, dXt, R.tok_ptr, R.tok_row, D.T, D.d, dx, st));
  MOE_TRY(MOE_K_DWR, launch_dwr(D.dtype, x, dz_dense, D.T, D.d, D.E, dw_r, (float*)(w + L.off[8]), st));
  // weight gradients
  if (mx && (D.flags & MOE_FLAG_MXFP8_WGRAD)) {
    // operands quantized along each expert's rows: x_g and dH for dW1, A_s and
    // dO_g for dW2
    int32_t* padoff = (int32_t*)(w + L.off[18]);
    int32_t* stage_e = (int32_t*)(w + L.off[19]);
    uint8_t* q[4];
    uint32_t* sc[4];
    for (int i = 0; i < 4; ++i) {
      q[i] = (uint8_t*)(w + L.off[20 + 2 * i]);
      sc[i] = (uint32_t*)(w + L.off[21 + 2 * i]);
    }
    MOE_TRY(MOE_K_MX_PAD_OFFSETS, launch_mx_pad_offsets(R.offsets, D.E, padoff, stage_e, st));
    MOE_TRY(MOE_K_MX_QUANT_SEG, launch_mx_quant_seg(x, D.d, R.row_token, R.offsets, padoff, stage_e, g, q[0], sc[0], st));
    MOE_TRY(MOE_K_MX_QUANT_SEG, launch_mx_quant_seg(dH, 2 * D.n, nullptr, R.offsets, padoff, stage_e, g, q[1], sc[1], st));
    MOE_TRY(MOE_K_DW1_MX, launch_wgrad_mx(g, D.d, 2 * D.n, padoff, q[0], sc[0], q[1], sc[1], dw1, st));
    MOE_TRY(MOE_K_MX_QUANT_SEG, launch_mx_quant_seg(As, D.n, nullptr, R.offsets, padoff, stage_e, g, q[2], sc[2], st));
    MOE_TRY(MOE_K_MX_QUANT_SEG, launch_mx_quant_seg(d_o, D.d, R.row_token, R.offsets, padoff, stage_e, g, q[3], sc[3], st));
    MOE_TRY(MOE_K_DW2_MX, launch_wgrad_mx(g, D.n, D.d, padoff, q[2], sc[2], q[3], sc[3], dw2, st));
  } else {
    void* wws = wgt_ws_bytes(g) ? (void*)(w + L.off[9]) : nullptr;
    MOE_TRY(MOE_K_DW1, launch_dw1(g, x, dH, R.row_token, R.offsets, dw1, wws, st));
    MOE_TRY(MOE_K_DW2, launch_dw2(g, As, d_o, R.row_token, R.offsets, dw2, wws, st));
  }
  if (db) MOE_TRY(MOE_K_DB, launch_bias_grad(dz_row, R.offsets, D.E, db, st));
  return MOE_OK;
}
}  // namespace

extern "C" {

int moe_bwd(const moe_desc* desc, const void* x, const void* w_r, const void* w1, const void* w2,
            const moe_routing* routing, const void* h_cache, const void* d_o, void* dx, void* dw_r,
            void* dw1, void* dw2, float* ds, float* db, void* ws, size_t ws_bytes, void* stream) {
  return bwd_impl(desc, x, w_r, w1, w2, routing, h_cache, d_o, dx, dw_r, dw1, dw2, ds, db, ws, ws_bytes, stream,
                  false);
}

int moe_bwd_mxfp8(const moe_desc* desc, const void* x, const void* w_r, const void* w1, const void* w2,
                  const moe_routing* routing, const void* h_cache, const void* d_o, void* dx, void* dw_r,
                  void* dw1, void* dw2, float* ds, float* db, void* ws, size_t ws_bytes, void* stream) {
  return bwd_impl(desc, x, w_r, w1, w2, routing, h_cache, d_o, dx, dw_r, dw1, dw2, ds, db, ws, ws_bytes, stream,
                  true);
}

int moe_fwd_mxfp8(const moe_desc* desc, const void* x, const void* w1, const void* w2,
                  const moe_routing* routing, void* o, void* h_cache, void* ws, size_t ws_bytes, void* stream) {
  int s = validate_desc(desc);
  if (s != MOE_OK) return s;
  if (desc->dtype != MOE_BF16) return MOE_EDTYPE;
  const GemmDims g = gemm_dims(desc);
  if (!mx_shape_ok(g)) return MOE_ESHAPE;
  if (!x || !w1 || !w2 || !o || !h_cache || !routing_ok(routing)) return MOE_EINVAL;
  const Layout L = mx_fwd_layout(desc);
  if ((s = check_ws(ws, ws_bytes, L.total)) != MOE_OK) return s;

  hipStream_t st = (hipStream_t)stream;
  uint8_t* w = (uint8_t*)ws;
  const moe_desc& D = *desc;
  const moe_routing& R = *routing;
  const size_t cap = capacity(desc);
  uint8_t *xq = w + L.off[0], *xs = w + L.off[1], *w1q = w + L.off[2], *w1s = w + L.off[3];
  uint8_t *w2q = w + L.off[4], *w2s = w + L.off[5], *aq = w + L.off[7], *as = w + L.off[8];
  void* A = w + L.off[6];
  void* Y = w + L.off[9];
  // operands quantized along each GEMM's reduction: x and W1 along d, W2 along n
  MOE_TRY(MOE_K_MX_QUANT_ROWS, launch_mx_quant_rows(x, D.d, D.T, nullptr, xq, xs, st));
  MOE_TRY(MOE_K_MX_QUANT_W, launch_mx_quant_w(w1, D.E, D.d, 2 * D.n, w1q, w1s, st));
  MOE_TRY(MOE_K_MX_QUANT_W, launch_mx_quant_w(w2, D.E, D.n, D.d, w2q, w2s, st));
  MOE_TRY(MOE_K_UP_MX, launch_up_mx(g, xq, xs, w1q, w1s, R.row_token, R.offsets, h_cache, A, st));
  // A along n, from the bf16 values the up-projection stored
  MOE_TRY(MOE_K_MX_QUANT_ROWS, launch_mx_quant_rows(A, D.n, (long long)cap, R.offsets + D.E, aq, as, st));
  MOE_TRY(MOE_K_DOWN_MX, launch_down_mx(g, aq, as, w2q, w2s, R.offsets, Y, st));
  MOE_TRY(MOE_K_AGG_O, launch_aggregate_o(D.dtype, Y, R.row_gate, R.tok_ptr, R.tok_row, D.T, D.d, o, st));
  return MOE_OK;
}

size_t moe_unfused_cache_bytes(const moe_desc* desc) {
  if (validate_desc(desc) != MOE_OK) return 0;
  return unfused_cache_layout(desc).total;
}

int moe_fwd_unfused(const moe_desc* desc, const void* x, const void* w1, const void* w2,
                    const moe_routing* routing, void* o, void* cache, size_t cache_bytes, void* stream) {
  int s = validate_desc(desc);
  if (s != MOE_OK) return s;
  if (!x || !w1 || !w2 || !o || !routing_ok(routing)) return MOE_EINVAL;
  const Layout C = unfused_cache_layout(desc);
  if ((s = check_ws(cache, cache_bytes, C.total)) != MOE_OK) return s;

  hipStream_t st = (hipStream_t)stream;
  char* c = (char*)cache;
  void* Xg = c + C.off[0];
  void* H = c + C.off[1];
  void* A = c + C.off[2];
  void* Y = c + C.off[3];
  const size_t cap = capacity(desc);
  const moe_desc& D = *desc;
  const GemmDims g = gemm_dims(desc);
  const moe_routing& R = *routing;
  const int32_t* P = R.offsets + D.E;
  MOE_TRY(MOE_K_GATHER, launch_gather_rows(D.dtype, x, D.d, R.row_token, P, cap, Xg, st));
  MOE_TRY(MOE_K_UP, launch_rows_gemm(g, Xg, D.d, w1, 2 * D.n, true, R.offsets, H, st));
  MOE_TRY(MOE_K_SWIGLU, launch_swiglu_fwd(D.dtype, H, D.n, P, cap, A, st));
  MOE_TRY(MOE_K_DOWN, launch_down(g, A, w2, R.offsets, Y, st));
  MOE_TRY(MOE_K_AGG_O, launch_aggregate_o(D.dtype, Y, R.row_gate, R.tok_ptr, R.tok_row, D.T, D.d, o, st));
  return MOE_OK;
}

int moe_bwd_unfused(const moe_desc* desc, const void* x, const void* w_r, const void* w1, const void* w2,
                    const moe_routing* routing, const void* cache, const void* d_o, void* dx, void* dw_r,
                    void* dw1, void* dw2, float* ds, float* db, void* ws, size_t ws_bytes, void* stream) {
  int s = validate_desc(desc);
  if (s != MOE_OK) return s;
  if (!x || !w_r || !w1 || !w2 || !cache || !d_o || !dx || !dw_r || !dw1 || !dw2 || !routing_ok(routing))
    return MOE_EINVAL;
  if (((uintptr_t)cache & (ALIGN - 1)) != 0) return MOE_EINVAL;
  const Layout L = unfused_bwd_layout(desc);
  if ((s = check_ws(ws, ws_bytes, L.total)) != MOE_OK) return s;

  hipStream_t st = (hipStream_t)stream;
  const Layout C = unfused_cache_layout(desc);
  const char* c = (const char*)cache;
  const void* Xg = c + C.off[0];
  const void* H = c + C.off[1];
  const void* A = c + C.off[2];
  const void* Y = c + C.off[3];
  char* w = (char*)ws;
  const moe_desc& D = *desc;
  const size_t cap = capacity(desc);
  void* dOg = w + L.off[0];
  void* dAp = w + L.off[1];
  void* dH = w + L.off[2];
  void* As = w + L.off[3];
  float* dS_dot = (float*)(w + L.off[4]);
  float* dS_row = ds ? ds : dS_dot + cap;
  float* dz_row = dS_dot + 2 * cap;
  void* dz_dense = w + L.off[5];
  void* w_rT = w + L.off[6];
  void* dXt = w + L.off[7];
  const moe_routing& R = *routing;
  const int32_t* P = R.offsets + D.E;
  const GemmDims g = gemm_dims(desc);

  // dO gathered per row; dS = <dO_g, Y> from the cached Y
  MOE_TRY(MOE_K_GATHER, launch_gather_rows(D.dtype, d_o, D.d, R.row_token, P, cap, dOg, st));
  MOE_TRY(MOE_K_ROW_DOT, launch_row_dot(D.dtype, dOg, Y, D.d, P, cap, dS_dot, st));
  // dA' = dO_g W2^T, then the SwiGLU backward as a kernel of its own
  MOE_TRY(MOE_K_DA, launch_rows_gemm(g, dOg, D.d, w2, D.n, false, R.offsets, dAp, st));
  MOE_TRY(MOE_K_SWIGLU_BWD, launch_swiglu_bwd(D.dtype, dAp, H, A, R.row_gate, D.n, P, cap, dH, As, st));
  // input and router gradients as in the fused layer, from the one dS part
  MOE_TRY(MOE_K_WR_T, launch_transpose(D.dtype, w_r, D.d, D.E, w_rT, st));
  const RouterDzArgs ra{dS_dot, 1, R.row_gate, R.row_expert, R.tok_ptr, R.tok_row, D.T, D.E,
                        dS_row, dz_row, dz_dense};
  MOE_TRY(MOE_K_ROUTER_GRAD, launch_router_dz(D.dtype, ra, st));
  MOE_TRY(MOE_K_DXT, launch_dxt(g, dH, w1, R.offsets, dXt, dz_row, w_rT, st));
  MOE_TRY(MOE_K_AGG_DX, launch_aggregate_dx(D.dtype, dXt, R.tok_ptr, R.tok_row, D.T, D.d, dx, st));
  MOE_TRY(MOE_K_DWR, launch_dwr(D.dtype, x, dz_dense, D.T, D.d, D.E, dw_r, (float*)(w + L.off[8]), st));
  // weight gradients from the cached, already gathered rows
  void* wws = wgt_ws_bytes(g) ? (void*)(w + L.off[9]) : nullptr;
  MOE_TRY(MOE_K_DW1, launch_dw1(g, Xg, dH, nullptr, R.offsets, dw1, wws, st));
  MOE_TRY(MOE_K_DW2, launch_dw2(g, As, dOg, nullptr, R.offsets, dw2, wws, st));
  if (db) MOE_TRY(MOE_K_DB, launch_bias_grad(dz_row, R.offsets, D.E, db, st));
  return MOE_OK;
}

const char* moe_strerror(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_ESHAPE: return "unsupported shape";
    case MOE_EDTYPE: return "unsupported dtype";
    case MOE_EWORKSPACE: return "workspace too small";
    case MOE_EHIP: return "HIP runtime error";
    case MOE_ENOSCRATCH: return "routing needs more than the library's static scratch (MOE_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

}  // extern "C"
