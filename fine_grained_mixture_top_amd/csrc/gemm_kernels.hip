// Instantiations of the grouped GEMM for the MoE layer's eight GEMMs and the
// host-side choice of tile configuration per GEMM ([B] kernel-list paragraph:
// the host launches each kernel with its chosen GEMM configuration).
#include <algorithm>
#include <type_traits>

#include "epilogues.h"
#include "grouped_gemm4.h"
#include "grouped_gemm5.h"
#include "launch.h"

namespace moe {

namespace {

int num_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 256;
  return cus;
}

template <typename K>
int occupancy(K kernel) {
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, kernel, 256, 0) != hipSuccess || blocks < 1)
    blocks = 1;
  return blocks;
}

// Persistent launch: one workgroup per resident slot, never more than tiles.
template <typename T, int BM, int BN, bool WGT, int BL, bool PAIRED, class Epi, int PF = 1>
hipError_t run_gemm(const GemmShape& s, const Operand& A, const Operand& B,
                    const typename Epi::Params& ep, long long max_tiles, hipStream_t st) {
  auto kern = grouped_gemm_kernel<T, BM, BN, WGT, BL, PAIRED, Epi, PF>;
  static const int occ = occupancy(kern);  // per instantiation, fixed for the process
  long long slots = (long long)num_cus() * occ;
  long long grid = std::min(max_tiles, slots);
  if (grid < 1) grid = 1;
  if (grid >= 8) grid = (grid + 7) / 8 * 8;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), 0, st, s, A, B, ep);
  return hipGetLastError();
}

// 256 x 256 tile kernel: one 512-thread workgroup per CU (LDS-bound).
template <bool WGT, bool BMN, bool PAIRED, class Epi, int GATH = 0>
hipError_t run_gemm4(const GemmShape& s, const Operand& A, const Operand& B, size_t a_bytes, size_t b_bytes,
                     const typename Epi::Params& ep, long long max_tiles, hipStream_t st) {
  auto kern = g4::grouped_gemm4_kernel<WGT, BMN, PAIRED, Epi, GATH>;
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, g4::SMEM);
  if (attr != hipSuccess) return attr;
  long long grid = std::min<long long>(max_tiles, num_cus());
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(g4::NTH), g4::SMEM, st, s, A, B, (uint32_t)a_bytes,
                     (uint32_t)b_bytes, ep);
  return hipGetLastError();
}

// Row-mode 256 x 256 tile kernel with k = 64 per stage (one workgroup per CU).
template <bool BMN, bool PAIRED, class Epi, bool TCHA = false>
hipError_t run_gemm5(const GemmShape& s, const Operand& A, const Operand& B, size_t a_bytes, size_t b_bytes,
                     const typename Epi::Params& ep, long long max_tiles, hipStream_t st) {
  auto kern = g5::grouped_gemm5_kernel<BMN, PAIRED, Epi, TCHA>;
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, g5::SMEM);
  if (attr != hipSuccess) return attr;
  long long grid = std::min<long long>(max_tiles, num_cus());
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(g5::NTH), g5::SMEM, st, s, A, B, (uint32_t)a_bytes,
                     (uint32_t)b_bytes, ep);
  return hipGetLastError();
}

// Row-mode GEMMs of the 256 x 256 tile family: k = 64 stages for
// reductions of at least 512 (measured faster there: up, dH, dXt), k = 32
// stages for short ones (the down-projection at n = 256, where the deeper
// pipeline of the k = 32 kernel wins).
template <bool BMN, bool PAIRED, class Epi>
hipError_t run_row256(const GemmShape& s, const Operand& A, const Operand& B, size_t a_bytes, size_t b_bytes,
                      const typename Epi::Params& ep, long long max_tiles, hipStream_t st) {
  // k = 64 stages from K = 512 up; K = 256 with k-contiguous weights too
  // (dXt at n = 128: 0.509 -> 0.494 ms at T = 16384, d = 2048, E = 256; the
  // down-projection at K = 256 is 2% faster on the k = 32 kernel, at K = 128
  // 4% slower: 0.333 against 0.348 ms at the same shape).  Weights
  // stored [k][n] with both K and N from 1024 up go to the k = 32 kernel,
  // whose three stages in flight measured faster there: up 2.19 -> 2.14 ms,
  // down 1.17 -> 1.12 at d = 2048, E = 64, n = 1024; up 8.83 -> 8.58, down
  // 4.50 -> 4.37 at d = 7168, E = 256, n = 2048 (up at N = 512 and 256 and
  // the k-contiguous weights of dH and dXt are faster on the k = 64 one).
  const bool long_mn = BMN && s.N >= 1024 && s.K >= 1024;
  if (!long_mn && s.K % g5::BK == 0 && (s.K >= (BMN ? 512 : 256) || (BMN && s.K == 128))) {
    // k-contiguous weights and A rows read without an index, shared by at
    // least four column tiles: the A-row touch variant
    if constexpr (!BMN)
      if (A.idx == nullptr && s.N / g5::BN >= 4)
        return run_gemm5<BMN, PAIRED, Epi, true>(s, A, B, a_bytes, b_bytes, ep, max_tiles, st);
    return run_gemm5<BMN, PAIRED, Epi>(s, A, B, a_bytes, b_bytes, ep, max_tiles, st);
  }
  return run_gemm4<false, BMN, PAIRED, Epi>(s, A, B, a_bytes, b_bytes, ep, max_tiles, st);
}

// Buffer-addressed operands use 32-bit byte offsets with the top half of the
// range kept as the out-of-bounds marker.
bool fits_g4(size_t bytes) { return bytes < (size_t)g4::OOB; }

long long row_tiles_bound(size_t cap, int E, int BM) { return (long long)(cap + BM - 1) / BM + E; }

// ---------------------------------------------------------------------------
// configurations: bf16 uses 128 x 128 tiles (two workgroups per CU), 128 x 64
// where a dimension is only a multiple of 64; the fp32 path (small checks)
// uses 128 x 64 tiles.
// ---------------------------------------------------------------------------

template <typename T> struct Cfg;
template <> struct Cfg<bf16_t> {
  static constexpr int BIG = 128, SMALL = 128;   // column tile of down / dXt
  __host__ static int bm_rows() { return 256; }
};
template <> struct Cfg<float> {
  static constexpr int BIG = 64, SMALL = 64;
  __host__ static int bm_rows() { return 128; }
};

// rows tile of the ROW-mode GEMMs
constexpr int ROWS_TILE = 128;
template <typename T> constexpr int ROWS = ROWS_TILE;

template <typename T, int BM, int BN>
hipError_t router_logits_t(const void* x, const void* w_r, const float* bias, float* logits, int T_, int d, int E,
                           hipStream_t st) {
  using Epi = EpiStore<T, float, BM, BN>;
  GemmShape s{nullptr, 1, T_, (E + BN - 1) / BN * BN, d, E, 1};
  Operand A{x, nullptr, 0, d};
  Operand B{w_r, nullptr, 0, E};
  typename Epi::Params ep{logits, E, bias};
  long long tiles = (long long)((T_ + BM - 1) / BM) * ((E + BN - 1) / BN);
  return run_gemm<T, BM, BN, false, B_KN, false, Epi>(s, A, B, ep, tiles, st);
}
template <typename T>
hipError_t router_logits(const void* x, const void* w_r, const float* bias, float* logits, int T_,
                         int d, int E, hipStream_t st) {
  if constexpr (std::is_same<T, bf16_t>::value) {
    // this GEMM is bound by its loads (N = E is small, every tile re-reads
    // W_r): 128-row tiles halve the W_r re-reads per token and win where
    // they still give two tiles per CU (T = 32768, d = 2048, E = 256:
    // 0.078 -> 0.059 ms); with fewer, 64-row tiles keep two per CU (T =
    // 32768, d = 1536, E = 128: 0.035 ms against 0.036 for 128 rows)
    const long long tiles128 = (long long)((T_ + 127) / 128) * ((E + 127) / 128);
    if (tiles128 >= 2LL * num_cus()) return router_logits_t<T, 128, 128>(x, w_r, bias, logits, T_, d, E, st);
    return router_logits_t<T, 64, 128>(x, w_r, bias, logits, T_, d, E, st);
  }
  return router_logits_t<T, ROWS<T>, 64>(x, w_r, bias, logits, T_, d, E, st);
}

template <typename T, int BN>
hipError_t up_swiglu_t(const GemmDims& g, const void* x, const void* w1, const int32_t* row_token,
                       const int32_t* offsets, void* H, void* A, hipStream_t st) {
  constexpr int BM = ROWS<T>;
  const int n = g.n, d = g.d, E = g.E;
  using Epi = EpiSwiGLU<T, BM, BN>;
  GemmShape s{offsets, E, 0, 2 * n, d, 2 * n, 1};
  Operand a{x, row_token, 0, d};
  Operand b{w1, nullptr, (long long)d * 2 * n, 2 * n};
  typename Epi::Params ep{reinterpret_cast<T*>(H), reinterpret_cast<T*>(A), n};
  // two k steps of loads in flight: the gathered token rows come from L2 / MALL
  return run_gemm<T, BM, BN, false, B_KN, true, Epi, 2>(s, a, b, ep,
                                                         row_tiles_bound(g.cap, E, BM) * (2 * n / BN), st);
}
hipError_t up_swiglu_g4(const GemmDims& g, const void* x, const void* w1, const int32_t* row_token,
                        const int32_t* offsets, void* H, void* A, hipStream_t st) {
  const int n = g.n, d = g.d, E = g.E;
  using Epi = g4::G4SwiGLU;
  GemmShape s{offsets, E, 0, 2 * n, d, 2 * n, 1};
  Operand a{x, row_token, 0, d};
  Operand b{w1, nullptr, (long long)d * 2 * n, 2 * n};
  typename Epi::Params ep{reinterpret_cast<bf16_t*>(H), reinterpret_cast<bf16_t*>(A), n};
  return run_row256<true, true, Epi>(s, a, b, (size_t)g.T * d * 2, (size_t)d * 2 * n * 2, ep,
                                     row_tiles_bound(g.cap, E, g4::BM) * (2 * n / g4::BN), st);
}
bool up_g4(const GemmDims& g) {
  return g.dtype == DT_BF16 && !g.small_tiles && (2 * g.n) % 256 == 0 && g.d % 32 == 0 &&
         fits_g4((size_t)g.T * g.d * 2) && fits_g4((size_t)g.d * 2 * g.n * 2);
}
template <typename T>
hipError_t up_swiglu(const GemmDims& g, const void* x, const void* w1, const int32_t* row_token,
                     const int32_t* offsets, void* H, void* A, hipStream_t st) {
  if constexpr (std::is_same<T, bf16_t>::value) {
    if (up_g4(g)) return up_swiglu_g4(g, x, w1, row_token, offsets, H, A, st);
    return up_swiglu_t<T, 128>(g, x, w1, row_token, offsets, H, A, st);
  } else {
    return up_swiglu_t<T, 64>(g, x, w1, row_token, offsets, H, A, st);
  }
}

template <typename T, int BN>
hipError_t down_t(const GemmDims& g, const void* A, const void* w2, const int32_t* offsets, void* Y,
                  hipStream_t st) {
  constexpr int BM = ROWS<T>;
  const int n = g.n, d = g.d, E = g.E;
  using Epi = EpiStore<T, T, BM, BN>;
  GemmShape s{offsets, E, 0, d, n, d, 1};
  Operand a{A, nullptr, 0, n};
  Operand b{w2, nullptr, (long long)n * d, d};
  typename Epi::Params ep{reinterpret_cast<T*>(Y), d, nullptr};
  return run_gemm<T, BM, BN, false, B_KN, false, Epi>(s, a, b, ep, row_tiles_bound(g.cap, E, BM) * (d / BN), st);
}
bool down_g4(const GemmDims& g) {
  return g.dtype == DT_BF16 && !g.small_tiles && g.d % 256 == 0 && g.n % 32 == 0 &&
         fits_g4(g.cap * g.n * 2) && fits_g4((size_t)g.n * g.d * 2);
}
template <typename T>
hipError_t down(const GemmDims& g, const void* A, const void* w2, const int32_t* offsets, void* Y, hipStream_t st) {
  if constexpr (std::is_same<T, bf16_t>::value) {
    if (down_g4(g)) {
      const int n = g.n, d = g.d, E = g.E;
      using Epi = g4::G4Store;
      GemmShape s{offsets, E, 0, d, n, d, 1};
      Operand a{A, nullptr, 0, n};
      Operand b{w2, nullptr, (long long)n * d, d};
      typename Epi::Params ep{reinterpret_cast<bf16_t*>(Y), d};
      return run_row256<true, false, Epi>(s, a, b, g.cap * n * 2, (size_t)n * d * 2, ep,
                                          row_tiles_bound(g.cap, E, g4::BM) * (d / g4::BN), st);
    }
  }
  if (g.d % Cfg<T>::BIG == 0) return down_t<T, Cfg<T>::BIG>(g, A, w2, offsets, Y, st);
  return down_t<T, Cfg<T>::SMALL>(g, A, w2, offsets, Y, st);
}

// dH: the column tile decides the number of score-gradient partials per row
bool dh_g4(const GemmDims& g) {
  return g.dtype == DT_BF16 && !g.small_tiles && g.n % 256 == 0 && g.d % 32 == 0 &&
         fits_g4((size_t)g.T * g.d * 2) && fits_g4((size_t)g.n * g.d * 2);
}
int dh_bn(const GemmDims& g) {
  if (g.dtype != DT_BF16) return 32;
  if (dh_g4(g)) return g4::BN;
  return g.n % 128 == 0 ? 128 : 64;
}

template <typename T, int BN>
hipError_t dh_t(const GemmDims& g, const void* d_o, const void* w2, const void* H, const int32_t* row_token,
                const float* row_gate, const int32_t* offsets, void* dH, void* As, float* dS_part, hipStream_t st) {
  constexpr int BM = ROWS<T>;
  const int n = g.n, d = g.d, E = g.E;
  using Epi = EpiDH<T, BM, BN>;
  GemmShape s{offsets, E, 0, n, d, n, 1};
  Operand a{d_o, row_token, 0, d};
  Operand b{w2, nullptr, (long long)n * d, d};  // W2[e] is [n][d]: row j holds k = 0..d-1
  typename Epi::Params ep{reinterpret_cast<const T*>(H), row_gate, reinterpret_cast<T*>(dH),
                          reinterpret_cast<T*>(As), dS_part, n, n / BN};
  return run_gemm<T, BM, BN, false, B_NK, false, Epi>(s, a, b, ep, row_tiles_bound(g.cap, E, BM) * (n / BN), st);
}
template <typename T>
hipError_t dh(const GemmDims& g, const void* d_o, const void* w2, const void* H, const int32_t* row_token,
              const float* row_gate, const int32_t* offsets, void* dH, void* As, float* dS_part, hipStream_t st) {
  if constexpr (std::is_same<T, bf16_t>::value) {
    const int bn = dh_bn(g);
    if (bn == g4::BN) {
      const int n = g.n, d = g.d, E = g.E;
      using Epi = EpiDH<bf16_t, g4::EROWS, g4::BN, g4::NTH>;
      GemmShape s{offsets, E, 0, n, d, n, 1};
      Operand a{d_o, row_token, 0, d};
      Operand b{w2, nullptr, (long long)n * d, d};
      typename Epi::Params ep{reinterpret_cast<const bf16_t*>(H), row_gate, reinterpret_cast<bf16_t*>(dH),
                              reinterpret_cast<bf16_t*>(As), dS_part, n, n / g4::BN};
      const long long tiles = row_tiles_bound(g.cap, E, g4::BM) * (n / g4::BN);
      if (d % g5::BK == 0 && d >= 512)  // k = 64 stages, H loads of the epilogue one pass ahead
        return run_gemm5<false, false, g5::G5DH>(s, a, b, (size_t)g.T * d * 2, (size_t)n * d * 2, ep, tiles, st);
      return run_gemm4<false, false, false, Epi>(s, a, b, (size_t)g.T * d * 2, (size_t)n * d * 2, ep, tiles, st);
    }
    if (bn == 128) return dh_t<T, 128>(g, d_o, w2, H, row_token, row_gate, offsets, dH, As, dS_part, st);
    return dh_t<T, 64>(g, d_o, w2, H, row_token, row_gate, offsets, dH, As, dS_part, st);
  } else {
    return dh_t<T, 32>(g, d_o, w2, H, row_token, row_gate, offsets, dH, As, dS_part, st);
  }
}

template <typename T, int BN>
hipError_t dxt_t(const GemmDims& g, const void* dH, const void* w1, const int32_t* offsets, void* dXt,
                 const float* dz, const void* w_rT, hipStream_t st) {
  constexpr int BM = ROWS<T>;
  const int n = g.n, d = g.d, E = g.E;
  using Epi = EpiStore<T, T, BM, BN>;
  GemmShape s{offsets, E, 0, d, 2 * n, d, 1};
  Operand a{dH, nullptr, 0, 2 * n};
  Operand b{w1, nullptr, (long long)d * 2 * n, 2 * n};  // W1[e] is [d][2n]: row i holds k = 0..2n-1
  typename Epi::Params ep{reinterpret_cast<T*>(dXt), d, nullptr, dz, reinterpret_cast<const T*>(w_rT)};
  return run_gemm<T, BM, BN, false, B_NK, false, Epi>(s, a, b, ep, row_tiles_bound(g.cap, E, BM) * (d / BN), st);
}
bool dxt_g4(const GemmDims& g) {
  return g.dtype == DT_BF16 && !g.small_tiles && g.d % 256 == 0 && (2 * g.n) % 32 == 0 &&
         fits_g4(g.cap * 2 * g.n * 2) && fits_g4((size_t)g.d * 2 * g.n * 2);
}
template <typename T>
hipError_t dxt(const GemmDims& g, const void* dH, const void* w1, const int32_t* offsets, void* dXt,
               const float* dz, const void* w_rT, hipStream_t st) {
  if constexpr (std::is_same<T, bf16_t>::value) {
    if (dxt_g4(g)) {
      const int n = g.n, d = g.d, E = g.E;
      using Epi = g4::G4StoreRouter;
      GemmShape s{offsets, E, 0, d, 2 * n, d, 1};
      Operand a{dH, nullptr, 0, 2 * n};
      Operand b{w1, nullptr, (long long)d * 2 * n, 2 * n};
      typename Epi::Params ep{reinterpret_cast<bf16_t*>(dXt), d, dz, reinterpret_cast<const bf16_t*>(w_rT),
                              (uint32_t)(g.cap * 4), (uint32_t)((size_t)E * d * 2)};
      return run_row256<false, false, Epi>(s, a, b, g.cap * 2 * n * 2, (size_t)d * 2 * n * 2, ep,
                                           row_tiles_bound(g.cap, E, g4::BM) * (d / g4::BN), st);
    }
  }
  if (g.d % Cfg<T>::BIG == 0) return dxt_t<T, Cfg<T>::BIG>(g, dH, w1, offsets, dXt, dz, w_rT, st);
  return dxt_t<T, Cfg<T>::SMALL>(g, dH, w1, offsets, dXt, dz, w_rT, st);
}

// ---------------------------------------------------------------------------
// Weight gradients.  An expert's weight-gradient tiles each reduce over all of
// the expert's rows, so under skewed routing a few tiles are far longer than
// the rest.  Before the GEMM, k_wgt_plan (one workgroup) builds its tile plan:
//  * an expert with more than `split` rows has its reduction cut into equal
//    chunks of at most `split` rows; each chunk's tiles write fp32 partial
//    sums to their own slot, and k_wgt_reduce adds them in chunk order (a
//    fixed order: results do not depend on timing);
//  * units (MU m tiles x all n tiles of one chunk) are sorted by rows, largest
//    first; the GEMM deals their tiles to its workgroups round by round in
//    alternating direction, so every workgroup gets a similar share of large
//    and small tiles, and the tiles of one unit run side by side on one XCD
//    (they share the chunk's rows in that XCD's L2).
// ---------------------------------------------------------------------------

struct WgtPolicy {
  int MT, NT, MU;
  int split;          // rows above which an expert is split (also the chunk bound); 0 = never
  size_t max_slots;   // partial slots needed at most
  size_t max_units;   // plan units at most
};

WgtPolicy wgt_policy(const GemmDims& g, int M, int N) {
  WgtPolicy p{};
  p.MT = M / g4::BM;
  p.NT = N / g4::BN;
  p.MU = 1;
  for (int mu = p.MT; mu >= 1; --mu)
    if (p.MT % mu == 0 && mu * p.NT <= 64) { p.MU = mu; break; }
  // half the rows a workgroup would reduce with the work spread evenly over
  // 256 workgroups (one per CU), never below 2048; a fixed count keeps the
  // workspace size a function of the shapes alone
  const long long tiles = (long long)p.MT * p.NT;
  long long sp = (long long)g.cap * tiles / (2LL * 256);
  sp = std::max<long long>(2048, (sp + 255) / 256 * 256);
  p.split = (sp >= (long long)g.cap || sp > (1LL << 30)) ? 0 : (int)sp;
  // every split expert has more than `split` rows and at most ceil(c/split) chunks
  const size_t whole = p.split ? g.cap / (size_t)p.split : 0;
  p.max_slots = p.split ? whole + std::min<size_t>((size_t)g.E, whole) : 0;
  p.max_units = ((size_t)g.E + p.max_slots) * (size_t)(p.MT / p.MU);
  return p;
}

// Plan buffer: [0] units, [16] split experts, then the split list (int4
// {e, first slot, chunks, 0} per split expert) and the sorted units.
struct WgtPlanLayout {
  size_t split_off, units_off, plan_bytes, partial_off, total;
};
WgtPlanLayout wgt_layout(const GemmDims& g, const WgtPolicy& p, int M, int N) {
  WgtPlanLayout L{};
  L.split_off = 256;
  L.units_off = L.split_off + ((size_t)g.E * 16 + 255) / 256 * 256;
  L.plan_bytes = L.units_off + p.max_units * sizeof(PlanUnit);
  L.partial_off = (L.plan_bytes + 255) / 256 * 256;
  L.total = L.partial_off + p.max_slots * (size_t)M * N * 4;
  return L;
}

__device__ __forceinline__ int plan_scan1024(int v, int* lds, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) lds[wave] = incl;
  __syncthreads();
  int base = 0, tot = 0;
  for (int x = 0; x < 16; ++x) {
    const int sv = lds[x];
    if (x < wave) base += sv;
    tot += sv;
  }
  __syncthreads();
  *total = tot;
  return base + incl - v;
}

// One 1024-thread workgroup (E <= 1024).
__global__ void __launch_bounds__(1024)
k_wgt_plan(const int32_t* __restrict__ offsets, int E, int MT, int MU, int split, int* __restrict__ plan,
           int4* __restrict__ split_list, PlanUnit* __restrict__ units) {
  __shared__ int gp[MAX_E + 1];     // chunk groups of experts before e
  __shared__ int base_rows[MAX_E];  // rows per chunk (split experts)
  __shared__ int slot0[MAX_E];      // first partial slot, -1 if not split
  __shared__ int hist[1024];
  __shared__ int sc[16];
  const int tid = threadIdx.x;
  const int e = tid;
  int q = 0, brows = 0, cnt = 0;
  if (e < E) {
    cnt = offsets[e + 1] - offsets[e];
    q = 1;
    if (split > 0 && cnt > split) {
      const int q0 = (cnt + split - 1) / split;
      brows = ((cnt + q0 - 1) / q0 + 31) / 32 * 32;
      q = (cnt + brows - 1) / brows;  // chunks that hold rows
    }
  }
  int ngroups, nsplit, nslots;
  const int g0 = plan_scan1024(q, sc, &ngroups);
  const int isz = q > 1 ? 1 : 0;
  const int si = plan_scan1024(isz, sc, &nsplit);
  const int s0 = plan_scan1024(q > 1 ? q : 0, sc, &nslots);
  if (e < E) {
    gp[e] = g0;
    base_rows[e] = brows;
    slot0[e] = q > 1 ? s0 : -1;
    if (q > 1) split_list[si] = make_int4(e, s0, q, 0);
  }
  if (tid == 0) {
    gp[E] = ngroups;
    plan[16] = nsplit;
  }
  hist[tid] = 0;
  __syncthreads();
  const int UPG = MT / MU;
  const int U = ngroups * UPG;
  // group g -> (expert, chunk, rows); sort key: k steps of 32 rows, descending
  auto group_of = [&](int g, int& ge, int& ch, int& r0, int& rn) {
    int lo = 0, hi = E - 1;  // largest e with gp[e] <= g
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (gp[mid] <= g) lo = mid; else hi = mid - 1;
    }
    ge = lo;
    ch = g - gp[lo];
    const int c = offsets[lo + 1] - offsets[lo];
    if (slot0[lo] < 0) {
      r0 = offsets[lo];
      rn = c;
    } else {
      r0 = offsets[lo] + ch * base_rows[lo];
      rn = min(base_rows[lo], c - ch * base_rows[lo]);
    }
  };
  for (int g = tid; g < ngroups; g += 1024) {
    int ge, ch, r0, rn;
    group_of(g, ge, ch, r0, rn);
    atomicAdd(&hist[1023 - min(1023, rn >> 5)], 1);
  }
  __syncthreads();
  int tot;
  const int start = plan_scan1024(hist[tid], sc, &tot);
  __syncthreads();
  hist[tid] = start;  // next free position of bucket tid
  __syncthreads();
  for (int g = tid; g < ngroups; g += 1024) {
    int ge, ch, r0, rn;
    group_of(g, ge, ch, r0, rn);
    // position among the sorted groups (groups of equal key in arrival
    // order: the order only decides which workgroup runs a tile, never its
    // result); a group's units stay together
    const int i = atomicAdd(&hist[1023 - min(1023, rn >> 5)], 1);
    PlanUnit pu;
    pu.e = ge;
    pu.seg0 = r0;
    pu.segn = rn;
    pu.slot = slot0[ge] < 0 ? -1 : slot0[ge] + ch;
    pu.pad[0] = pu.pad[1] = pu.pad[2] = 0;
    for (int m = 0; m < UPG; ++m) {
      pu.mt0 = m * MU;
      units[(size_t)i * UPG + m] = pu;
    }
  }
  if (tid == 0) plan[0] = U;
}

// out[e] = sum over chunks c of P[first slot of e + c] for every split
// expert (M x N elements each, bf16 out), in chunk order.  Workgroups stride
// over (split expert, 2048-element block) items.
__global__ void __launch_bounds__(256)
k_wgt_reduce(const int* __restrict__ plan, const int4* __restrict__ split_list, int M, int N,
             const float* __restrict__ P, bf16_t* __restrict__ out) {
  const int nsplit = plan[16];
  const long long mn = (long long)M * N;
  const long long per = mn / 2048;  // M and N are multiples of 256
  const long long items = (long long)nsplit * per;
  for (long long u = blockIdx.x; u < items; u += gridDim.x) {
    const int4 sl = split_list[u / per];
    const long long off = (u % per) * 2048 + threadIdx.x * 8;
    const float* src = P + (long long)sl.y * mn + off;
    float4 a0 = *reinterpret_cast<const float4*>(src), a1 = *reinterpret_cast<const float4*>(src + 4);
    for (int c = 1; c < sl.z; ++c) {
      const float4 b0 = *reinterpret_cast<const float4*>(src + c * mn);
      const float4 b1 = *reinterpret_cast<const float4*>(src + c * mn + 4);
      a0.x += b0.x; a0.y += b0.y; a0.z += b0.z; a0.w += b0.w;
      a1.x += b1.x; a1.y += b1.y; a1.z += b1.z; a1.w += b1.w;
    }
    uint4 v;
    v.x = f2bf2(a0.x, a0.y);
    v.y = f2bf2(a0.z, a0.w);
    v.z = f2bf2(a1.x, a1.y);
    v.w = f2bf2(a1.z, a1.w);
    *reinterpret_cast<uint4*>(out + (long long)sl.x * mn + off) = v;
  }
}

// Weight-gradient GEMM on the 256-tile kernel (C = M x N per expert, bf16):
// plan, GEMM, then the sum of split experts' partials.
hipError_t wgt_g4(const GemmDims& g, const int32_t* offsets, int M, int N, const Operand& a, const Operand& b,
                  size_t a_bytes, size_t b_bytes, void* C, void* ws, hipStream_t st) {
  const WgtPolicy pol = wgt_policy(g, M, N);
  const WgtPlanLayout L = wgt_layout(g, pol, M, N);
  char* w = static_cast<char*>(ws);
  int* plan = reinterpret_cast<int*>(w);
  int4* split_list = reinterpret_cast<int4*>(w + L.split_off);
  PlanUnit* units = reinterpret_cast<PlanUnit*>(w + L.units_off);
  float* partial = reinterpret_cast<float*>(w + L.partial_off);
  hipLaunchKernelGGL(k_wgt_plan, dim3(1), dim3(1024), 0, st, offsets, g.E, pol.MT, pol.MU, pol.split, plan,
                     split_list, units);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  GemmShape s{offsets, g.E, M, N, 0, N, 1};
  s.plan = WgtPlan{plan, units, pol.MU};
  using Epi = g4::G4StoreW;
  typename Epi::Params ep{reinterpret_cast<bf16_t*>(C), N, partial};
  // which operand's rows are gathered (dW1: x, dW2: dO; neither when the
  // rows come pre-gathered) is a template parameter of the kernel
  const int gath = (a.idx ? 1 : 0) | (b.idx ? 2 : 0);
  auto run = [&](auto G) {
    constexpr int GA = decltype(G)::value;
    return run_gemm4<true, true, false, Epi, GA>(s, a, b, a_bytes, b_bytes, ep, num_cus(), st);
  };
  switch (gath) {
    case 1: err = run(std::integral_constant<int, 1>()); break;
    case 2: err = run(std::integral_constant<int, 2>()); break;
    case 3: err = run(std::integral_constant<int, 3>()); break;
    default: err = run(std::integral_constant<int, 0>()); break;
  }
  if (err != hipSuccess || pol.split == 0) return err;
  hipLaunchKernelGGL(k_wgt_reduce, dim3((unsigned)(2 * num_cus())), dim3(256), 0, st, plan, split_list, M, N,
                     partial, reinterpret_cast<bf16_t*>(C));
  return hipGetLastError();
}

template <typename T, int BMW, int BN>
hipError_t dw1_t(const GemmDims& g, const void* x, const void* dH, const int32_t* row_token,
                 const int32_t* offsets, void* dW1, hipStream_t st) {
  const int n = g.n, d = g.d, E = g.E;
  using Epi = EpiStore<T, T, BMW, BN>;
  GemmShape s{offsets, E, d, 2 * n, 0, 2 * n, 1};
  Operand a{x, row_token, 0, d};
  Operand b{dH, nullptr, 0, 2 * n};
  typename Epi::Params ep{reinterpret_cast<T*>(dW1), 2 * n, nullptr};
  return run_gemm<T, BMW, BN, true, B_KN, false, Epi>(s, a, b, ep, (long long)E * (d / BMW) * (2 * n / BN), st);
}
bool dw1_g4(const GemmDims& g) {
  return g.dtype == DT_BF16 && !g.small_tiles && g.d % 256 == 0 && (2 * g.n) % 256 == 0 &&
         fits_g4(std::max<size_t>(g.T, g.cap) * g.d * 2) && fits_g4(g.cap * 2 * g.n * 2);
}
template <typename T>
hipError_t dw1(const GemmDims& g, const void* x, const void* dH, const int32_t* row_token, const int32_t* offsets,
               void* dW1, void* ws, hipStream_t st) {
  if constexpr (std::is_same<T, bf16_t>::value) {
    if (dw1_g4(g)) {
      const int n = g.n, d = g.d;
      Operand a{x, row_token, 0, d};
      Operand b{dH, nullptr, 0, 2 * n};
      const size_t xrows = row_token ? (size_t)g.T : g.cap;  // null: x already gathered per row
      return wgt_g4(g, offsets, d, 2 * n, a, b, xrows * d * 2, g.cap * 2 * n * 2, dW1, ws, st);
    }
    return dw1_t<T, 128, 128>(g, x, dH, row_token, offsets, dW1, st);
  } else {
    return dw1_t<T, 128, 64>(g, x, dH, row_token, offsets, dW1, st);
  }
}

template <typename T, int BMW, int BN>
hipError_t dw2_t(const GemmDims& g, const void* As, const void* d_o, const int32_t* row_token,
                 const int32_t* offsets, void* dW2, hipStream_t st) {
  const int n = g.n, d = g.d, E = g.E;
  using Epi = EpiStore<T, T, BMW, BN>;
  GemmShape s{offsets, E, n, d, 0, d, 1};
  Operand a{As, nullptr, 0, n};
  Operand b{d_o, row_token, 0, d};
  typename Epi::Params ep{reinterpret_cast<T*>(dW2), d, nullptr};
  return run_gemm<T, BMW, BN, true, B_KN, false, Epi>(s, a, b, ep, (long long)E * (n / BMW) * (d / BN), st);
}
bool dw2_g4(const GemmDims& g) {
  return g.dtype == DT_BF16 && !g.small_tiles && g.n % 256 == 0 && g.d % 256 == 0 &&
         fits_g4(g.cap * g.n * 2) && fits_g4(std::max<size_t>(g.T, g.cap) * g.d * 2);
}
template <typename T>
hipError_t dw2(const GemmDims& g, const void* As, const void* d_o, const int32_t* row_token, const int32_t* offsets,
               void* dW2, void* ws, hipStream_t st) {
  if constexpr (std::is_same<T, bf16_t>::value) {
    if (dw2_g4(g)) {
      const int n = g.n, d = g.d;
      Operand a{As, nullptr, 0, n};
      Operand b{d_o, row_token, 0, d};
      const size_t orows = row_token ? (size_t)g.T : g.cap;  // null: dO already gathered per row
      return wgt_g4(g, offsets, n, d, a, b, g.cap * n * 2, orows * d * 2, dW2, ws, st);
    }
    if (g.n % 128 == 0) return dw2_t<T, 128, 128>(g, As, d_o, row_token, offsets, dW2, st);
    return dw2_t<T, 64, 128>(g, As, d_o, row_token, offsets, dW2, st);
  } else {
    if (g.n % 128 == 0) return dw2_t<T, 128, 64>(g, As, d_o, row_token, offsets, dW2, st);
    return dw2_t<T, 64, 64>(g, As, d_o, row_token, offsets, dW2, st);
  }
}

// C[r] = A[r] W[e_r] for every routed row r (segment rows, no gather): W[e]
// is [K][N] (w_kn) or [N][K].  Used by the unfused layer.
template <typename T, int BL, int BN>
hipError_t rows_gemm_t(const GemmDims& g, const void* A, int K, const void* W, int N, const int32_t* offsets,
                       void* C, hipStream_t st) {
  constexpr int BM = ROWS<T>;
  using Epi = EpiStore<T, T, BM, BN>;
  GemmShape s{offsets, g.E, 0, (N + BN - 1) / BN * BN, K, N, 1};
  Operand a{A, nullptr, 0, K};
  Operand b{W, nullptr, (long long)K * N, BL == B_KN ? N : K};
  typename Epi::Params ep{reinterpret_cast<T*>(C), N, nullptr};
  return run_gemm<T, BM, BN, false, BL, false, Epi>(s, a, b, ep, row_tiles_bound(g.cap, g.E, BM) * ((N + BN - 1) / BN),
                                                    st);
}
template <typename T>
hipError_t rows_gemm(const GemmDims& g, const void* A, int K, const void* W, int N, bool w_kn,
                     const int32_t* offsets, void* C, hipStream_t st) {
  if constexpr (std::is_same<T, bf16_t>::value) {
    if (!g.small_tiles && N % 256 == 0 && K % 32 == 0 && fits_g4(g.cap * (size_t)K * 2) &&
        fits_g4((size_t)K * N * 2)) {
      using Epi = g4::G4Store;
      GemmShape s{offsets, g.E, 0, N, K, N, 1};
      Operand a{A, nullptr, 0, K};
      Operand b{W, nullptr, (long long)K * N, w_kn ? N : K};
      typename Epi::Params ep{reinterpret_cast<bf16_t*>(C), N};
      const long long tiles = row_tiles_bound(g.cap, g.E, g4::BM) * (N / g4::BN);
      if (w_kn) return run_row256<true, false, Epi>(s, a, b, g.cap * (size_t)K * 2, (size_t)K * N * 2, ep, tiles, st);
      return run_row256<false, false, Epi>(s, a, b, g.cap * (size_t)K * 2, (size_t)K * N * 2, ep, tiles, st);
    }
  }
  constexpr int BN = Cfg<T>::BIG;
  if (w_kn) return rows_gemm_t<T, B_KN, BN>(g, A, K, W, N, offsets, C, st);
  return rows_gemm_t<T, B_NK, BN>(g, A, K, W, N, offsets, C, st);
}

// Router weight gradient dW_r = X^T dz: one dense reduction over all T
// tokens with only (d/BM) x (E/BN) output tiles, so the reduction is split
// into chunks whose fp32 partials are summed in a fixed order afterwards.
template <typename TO>
__global__ void k_sum_partials(const float* __restrict__ part, int splits, long long count,
                               TO* __restrict__ out) {
  const long long i = ((long long)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i >= count) return;
  float4 acc = *reinterpret_cast<const float4*>(part + i);
  for (int s = 1; s < splits; ++s) {
    const float4 v = *reinterpret_cast<const float4*>(part + (long long)s * count + i);
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  out[i] = Elem<TO>::from_f(acc.x);
  out[i + 1] = Elem<TO>::from_f(acc.y);
  out[i + 2] = Elem<TO>::from_f(acc.z);
  out[i + 3] = Elem<TO>::from_f(acc.w);
}

template <typename T, int BN>
hipError_t dwr_t(const void* x, const void* dz, int T_, int d, int E, float* part, int splits, hipStream_t st) {
  constexpr int BM = 128;
  using Epi = EpiStore<T, float, BM, BN>;
  const int NT = (E + BN - 1) / BN;
  GemmShape s{nullptr, 1, d, NT * BN, T_, E, splits};
  Operand a{x, nullptr, 0, d};
  Operand b{dz, nullptr, 0, E};
  typename Epi::Params ep{part, E, nullptr};
  return run_gemm<T, BM, BN, true, B_KN, false, Epi>(s, a, b, ep, (long long)splits * (d / BM) * NT, st);
}

// x^T dz: each column tile of dz re-reads all of x, so bf16 takes 128
// columns of E per tile where E allows (x read E / 128 times, not E / 64)
template <typename T>
hipError_t dwr(const void* x, const void* dz, int T_, int d, int E, void* dWr, float* part, hipStream_t st) {
  const int splits = dwr_splits(T_, d, E);
  hipError_t err;
  if (std::is_same<T, bf16_t>::value && E % 128 == 0) err = dwr_t<T, 128>(x, dz, T_, d, E, part, splits, st);
  else err = dwr_t<T, 64>(x, dz, T_, d, E, part, splits, st);
  if (err != hipSuccess) return err;
  const long long count = (long long)d * E;  // multiple of 4: d % 128 == 0
  hipLaunchKernelGGL(k_sum_partials<T>, dim3((unsigned)((count / 4 + 255) / 256)), dim3(256), 0, st, part,
                     splits, count, reinterpret_cast<T*>(dWr));
  return hipGetLastError();
}

}  // namespace

int dh_block(const GemmDims& g) { return dh_bn(g); }

int dwr_splits(int T, int d, int E) {
  const int bn = E % 128 == 0 ? 128 : 64;  // the column tile of the bf16 launch
  const int tiles = (d / 128) * ((E + bn - 1) / bn);
  // at least one tile per CU; up to two while chunks keep 1024 rows or more
  // (shorter chunks mostly add fp32 partial traffic and per-tile overhead:
  // measured at d = 1536, E = 128, T = 32768: 22 splits 0.055 ms, 43 splits
  // 0.062 ms; d = 2048, E = 256: T = 32768 at 8 splits 0.100 ms and 16
  // splits 0.069 ms, T = 16384 at 8 splits 0.056 ms and 16 splits 0.045 ms)
  int s = std::max((256 + tiles - 1) / tiles, std::min((512 + tiles - 1) / tiles, T / 1024));
  const int kmax = (T + 255) / 256;            // at least 4 k steps of 64 per chunk
  if (s > kmax) s = kmax;
  if (s > 64) s = 64;
  return s < 1 ? 1 : s;
}

#define MOE_DISPATCH(dtype, fn, ...) \
  ((dtype) == DT_BF16 ? fn<bf16_t>(__VA_ARGS__) : fn<float>(__VA_ARGS__))

hipError_t launch_router_logits(int dtype, const void* x, const void* w_r, const float* bias,
                                float* logits, int T, int d, int E, hipStream_t st) {
  return MOE_DISPATCH(dtype, router_logits, x, w_r, bias, logits, T, d, E, st);
}
#define MOE_GDISPATCH(g, fn, ...) \
  ((g).dtype == DT_BF16 ? fn<bf16_t>(g, __VA_ARGS__) : fn<float>(g, __VA_ARGS__))

hipError_t launch_up_swiglu(const GemmDims& g, const void* x, const void* w1, const int32_t* row_token,
                            const int32_t* offsets, void* H, void* A, hipStream_t st) {
  return MOE_GDISPATCH(g, up_swiglu, x, w1, row_token, offsets, H, A, st);
}
hipError_t launch_down(const GemmDims& g, const void* A, const void* w2, const int32_t* offsets, void* Y,
                       hipStream_t st) {
  return MOE_GDISPATCH(g, down, A, w2, offsets, Y, st);
}
hipError_t launch_dh(const GemmDims& g, const void* d_o, const void* w2, const void* H,
                     const int32_t* row_token, const float* row_gate, const int32_t* offsets, void* dH,
                     void* As, float* dS_part, hipStream_t st) {
  return MOE_GDISPATCH(g, dh, d_o, w2, H, row_token, row_gate, offsets, dH, As, dS_part, st);
}
hipError_t launch_dxt(const GemmDims& g, const void* dH, const void* w1, const int32_t* offsets, void* dXt,
                      const float* dz, const void* w_rT, hipStream_t st) {
  return MOE_GDISPATCH(g, dxt, dH, w1, offsets, dXt, dz, w_rT, st);
}
hipError_t launch_dw1(const GemmDims& g, const void* x, const void* dH, const int32_t* row_token,
                      const int32_t* offsets, void* dW1, void* ws, hipStream_t st) {
  return MOE_GDISPATCH(g, dw1, x, dH, row_token, offsets, dW1, ws, st);
}
hipError_t launch_dw2(const GemmDims& g, const void* As, const void* d_o, const int32_t* row_token,
                      const int32_t* offsets, void* dW2, void* ws, hipStream_t st) {
  return MOE_GDISPATCH(g, dw2, As, d_o, row_token, offsets, dW2, ws, st);
}
size_t wgt_ws_bytes(const GemmDims& g) {
  size_t b = 0;
  if (dw1_g4(g)) b = std::max(b, wgt_layout(g, wgt_policy(g, g.d, 2 * g.n), g.d, 2 * g.n).total);
  if (dw2_g4(g)) b = std::max(b, wgt_layout(g, wgt_policy(g, g.n, g.d), g.n, g.d).total);
  return b;
}
hipError_t launch_rows_gemm(const GemmDims& g, const void* A, int K, const void* W, int N, bool w_kn,
                            const int32_t* offsets, void* C, hipStream_t st) {
  return MOE_GDISPATCH(g, rows_gemm, A, K, W, N, w_kn, offsets, C, st);
}
hipError_t launch_dwr(int dtype, const void* x, const void* dz_dense, int T, int d, int E, void* dWr,
                      float* partials, hipStream_t st) {
  return MOE_DISPATCH(dtype, dwr, x, dz_dense, T, d, E, dWr, partials, st);
}

}  // namespace moe
