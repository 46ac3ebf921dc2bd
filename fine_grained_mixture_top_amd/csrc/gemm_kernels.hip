// Instantiations of the grouped GEMM for the MoE layer's eight GEMMs and the
// host-side choice of tile configuration per GEMM ([B] kernel-list paragraph:
// the host launches each kernel with its chosen GEMM configuration).
#include <algorithm>
#include <type_traits>

#include "epilogues.h"
#include "grouped_gemm4.h"
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
template <bool WGT, bool BMN, bool PAIRED, class Epi>
hipError_t run_gemm4(const GemmShape& s, const Operand& A, const Operand& B, size_t a_bytes, size_t b_bytes,
                     const typename Epi::Params& ep, long long max_tiles, hipStream_t st) {
  auto kern = g4::grouped_gemm4_kernel<WGT, BMN, PAIRED, Epi>;
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, g4::SMEM);
  if (attr != hipSuccess) return attr;
  long long grid = std::min<long long>(max_tiles, num_cus());
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(g4::NTH), g4::SMEM, st, s, A, B, (uint32_t)a_bytes,
                     (uint32_t)b_bytes, ep);
  return hipGetLastError();
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

template <typename T>
hipError_t router_logits(const void* x, const void* w_r, const float* bias, float* logits, int T_,
                         int d, int E, hipStream_t st) {
  constexpr int BM = ROWS<T>, BN = std::is_same<T, bf16_t>::value ? 128 : 64;
  using Epi = EpiStore<T, float, BM, BN>;
  GemmShape s{nullptr, 1, T_, (E + BN - 1) / BN * BN, d, E, 1};
  Operand A{x, nullptr, 0, d};
  Operand B{w_r, nullptr, 0, E};
  typename Epi::Params ep{logits, E, bias};
  long long tiles = (long long)((T_ + BM - 1) / BM) * ((E + BN - 1) / BN);
  return run_gemm<T, BM, BN, false, B_KN, false, Epi>(s, A, B, ep, tiles, st);
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
  return run_gemm4<false, true, true, Epi>(s, a, b, (size_t)g.T * d * 2, (size_t)d * 2 * n * 2, ep,
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
      return run_gemm4<false, true, false, Epi>(s, a, b, g.cap * n * 2, (size_t)n * d * 2, ep,
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
      return run_gemm4<false, false, false, Epi>(s, a, b, (size_t)g.T * d * 2, (size_t)n * d * 2, ep,
                                                 row_tiles_bound(g.cap, E, g4::BM) * (n / g4::BN), st);
    }
    if (bn == 128) return dh_t<T, 128>(g, d_o, w2, H, row_token, row_gate, offsets, dH, As, dS_part, st);
    return dh_t<T, 64>(g, d_o, w2, H, row_token, row_gate, offsets, dH, As, dS_part, st);
  } else {
    return dh_t<T, 32>(g, d_o, w2, H, row_token, row_gate, offsets, dH, As, dS_part, st);
  }
}

template <typename T, int BN>
hipError_t dxt_t(const GemmDims& g, const void* dH, const void* w1, const int32_t* offsets, void* dXt,
                 hipStream_t st) {
  constexpr int BM = ROWS<T>;
  const int n = g.n, d = g.d, E = g.E;
  using Epi = EpiStore<T, T, BM, BN>;
  GemmShape s{offsets, E, 0, d, 2 * n, d, 1};
  Operand a{dH, nullptr, 0, 2 * n};
  Operand b{w1, nullptr, (long long)d * 2 * n, 2 * n};  // W1[e] is [d][2n]: row i holds k = 0..2n-1
  typename Epi::Params ep{reinterpret_cast<T*>(dXt), d, nullptr};
  return run_gemm<T, BM, BN, false, B_NK, false, Epi>(s, a, b, ep, row_tiles_bound(g.cap, E, BM) * (d / BN), st);
}
bool dxt_g4(const GemmDims& g) {
  return g.dtype == DT_BF16 && !g.small_tiles && g.d % 256 == 0 && (2 * g.n) % 32 == 0 &&
         fits_g4(g.cap * 2 * g.n * 2) && fits_g4((size_t)g.d * 2 * g.n * 2);
}
template <typename T>
hipError_t dxt(const GemmDims& g, const void* dH, const void* w1, const int32_t* offsets, void* dXt,
               hipStream_t st) {
  if constexpr (std::is_same<T, bf16_t>::value) {
    if (dxt_g4(g)) {
      const int n = g.n, d = g.d, E = g.E;
      using Epi = g4::G4Store;
      GemmShape s{offsets, E, 0, d, 2 * n, d, 1};
      Operand a{dH, nullptr, 0, 2 * n};
      Operand b{w1, nullptr, (long long)d * 2 * n, 2 * n};
      typename Epi::Params ep{reinterpret_cast<bf16_t*>(dXt), d};
      return run_gemm4<false, false, false, Epi>(s, a, b, g.cap * 2 * n * 2, (size_t)d * 2 * n * 2, ep,
                                                 row_tiles_bound(g.cap, E, g4::BM) * (d / g4::BN), st);
    }
  }
  if (g.d % Cfg<T>::BIG == 0) return dxt_t<T, Cfg<T>::BIG>(g, dH, w1, offsets, dXt, st);
  return dxt_t<T, Cfg<T>::SMALL>(g, dH, w1, offsets, dXt, st);
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
         fits_g4((size_t)g.T * g.d * 2) && fits_g4(g.cap * 2 * g.n * 2);
}
template <typename T>
hipError_t dw1(const GemmDims& g, const void* x, const void* dH, const int32_t* row_token, const int32_t* offsets,
               void* dW1, hipStream_t st) {
  if constexpr (std::is_same<T, bf16_t>::value) {
    if (dw1_g4(g)) {
      const int n = g.n, d = g.d, E = g.E;
      using Epi = g4::G4Store;
      GemmShape s{offsets, E, d, 2 * n, 0, 2 * n, 1};
      Operand a{x, row_token, 0, d};
      Operand b{dH, nullptr, 0, 2 * n};
      typename Epi::Params ep{reinterpret_cast<bf16_t*>(dW1), 2 * n};
      return run_gemm4<true, true, false, Epi>(s, a, b, (size_t)g.T * d * 2, g.cap * 2 * n * 2, ep,
                                               (long long)E * (d / g4::BM) * (2 * n / g4::BN), st);
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
         fits_g4(g.cap * g.n * 2) && fits_g4((size_t)g.T * g.d * 2);
}
template <typename T>
hipError_t dw2(const GemmDims& g, const void* As, const void* d_o, const int32_t* row_token, const int32_t* offsets,
               void* dW2, hipStream_t st) {
  if constexpr (std::is_same<T, bf16_t>::value) {
    if (dw2_g4(g)) {
      const int n = g.n, d = g.d, E = g.E;
      using Epi = g4::G4Store;
      GemmShape s{offsets, E, n, d, 0, d, 1};
      Operand a{As, nullptr, 0, n};
      Operand b{d_o, row_token, 0, d};
      typename Epi::Params ep{reinterpret_cast<bf16_t*>(dW2), d};
      return run_gemm4<true, true, false, Epi>(s, a, b, g.cap * n * 2, (size_t)g.T * d * 2, ep,
                                               (long long)E * (n / g4::BM) * (d / g4::BN), st);
    }
    if (g.n % 128 == 0) return dw2_t<T, 128, 128>(g, As, d_o, row_token, offsets, dW2, st);
    return dw2_t<T, 64, 128>(g, As, d_o, row_token, offsets, dW2, st);
  } else {
    if (g.n % 128 == 0) return dw2_t<T, 128, 64>(g, As, d_o, row_token, offsets, dW2, st);
    return dw2_t<T, 64, 64>(g, As, d_o, row_token, offsets, dW2, st);
  }
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

template <typename T>
hipError_t dwr(const void* x, const void* dz, int T_, int d, int E, void* dWr, float* part, hipStream_t st) {
  constexpr int BM = 128, BN = 64;
  using Epi = EpiStore<T, float, BM, BN>;
  const int NT = (E + BN - 1) / BN;
  const int splits = dwr_splits(T_, d, E);
  GemmShape s{nullptr, 1, d, NT * BN, T_, E, splits};
  Operand a{x, nullptr, 0, d};
  Operand b{dz, nullptr, 0, E};
  typename Epi::Params ep{part, E, nullptr};
  hipError_t err = run_gemm<T, BM, BN, true, B_KN, false, Epi>(s, a, b, ep,
                                                               (long long)splits * (d / BM) * NT, st);
  if (err != hipSuccess) return err;
  const long long count = (long long)d * E;  // multiple of 4: d % 128 == 0
  hipLaunchKernelGGL(k_sum_partials<T>, dim3((unsigned)((count / 4 + 255) / 256)), dim3(256), 0, st, part,
                     splits, count, reinterpret_cast<T*>(dWr));
  return hipGetLastError();
}

}  // namespace

int dh_block(const GemmDims& g) { return dh_bn(g); }

int dwr_splits(int T, int d, int E) {
  const int tiles = (d / 128) * ((E + 63) / 64);
  int s = (512 + tiles - 1) / tiles;           // about two resident tiles per CU
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
                      hipStream_t st) {
  return MOE_GDISPATCH(g, dxt, dH, w1, offsets, dXt, st);
}
hipError_t launch_dw1(const GemmDims& g, const void* x, const void* dH, const int32_t* row_token,
                      const int32_t* offsets, void* dW1, hipStream_t st) {
  return MOE_GDISPATCH(g, dw1, x, dH, row_token, offsets, dW1, st);
}
hipError_t launch_dw2(const GemmDims& g, const void* As, const void* d_o, const int32_t* row_token,
                      const int32_t* offsets, void* dW2, hipStream_t st) {
  return MOE_GDISPATCH(g, dw2, As, d_o, row_token, offsets, dW2, st);
}
hipError_t launch_dwr(int dtype, const void* x, const void* dz_dense, int T, int d, int E, void* dWr,
                      float* partials, hipStream_t st) {
  return MOE_DISPATCH(dtype, dwr, x, dz_dense, T, d, E, dWr, partials, st);
}

}  // namespace moe
