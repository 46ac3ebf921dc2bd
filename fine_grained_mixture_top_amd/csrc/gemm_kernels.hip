// Instantiations of the grouped GEMM for the MoE layer's eight GEMMs and the
// host-side choice of tile configuration per GEMM ([B] kernel-list paragraph:
// the host launches each kernel with its chosen GEMM configuration).
#include <algorithm>

#include "epilogues.h"
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
template <typename T, int BM, int BN, bool WGT, int BL, bool PAIRED, class Epi>
hipError_t run_gemm(const GemmShape& s, const Operand& A, const Operand& B,
                    const typename Epi::Params& ep, long long max_tiles, hipStream_t st) {
  auto kern = grouped_gemm_kernel<T, BM, BN, WGT, BL, PAIRED, Epi>;
  static const int occ = occupancy(kern);  // per instantiation, fixed for the process
  long long slots = (long long)num_cus() * occ;
  long long grid = std::min(max_tiles, slots);
  if (grid < 1) grid = 1;
  if (grid >= 8) grid = (grid + 7) / 8 * 8;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), 0, st, s, A, B, ep);
  return hipGetLastError();
}

long long row_tiles_bound(size_t cap, int E, int BM) { return (long long)(cap + BM - 1) / BM + E; }

// ---------------------------------------------------------------------------
// per-dtype configurations
// ---------------------------------------------------------------------------

template <typename T> struct Cfg;
template <> struct Cfg<bf16_t> {
  static constexpr int UP_BN = 128, DOWN_BN = 128, DH_BN = 64, DXT_BN = 128;
  static constexpr int DW1_BN = 128, DW2_BN = 128, R_BN = 64, DWR_BN = 64;
};
template <> struct Cfg<float> {
  static constexpr int UP_BN = 64, DOWN_BN = 64, DH_BN = 32, DXT_BN = 64;
  static constexpr int DW1_BN = 64, DW2_BN = 64, R_BN = 64, DWR_BN = 64;
};

constexpr int BM = 128;  // routed-row tile; equals the token-rounding tile

template <typename T>
hipError_t router_logits(const void* x, const void* w_r, const float* bias, float* logits, int T_,
                         int d, int E, hipStream_t st) {
  constexpr int BN = Cfg<T>::R_BN;
  using Epi = EpiStore<T, float, BM, BN>;
  GemmShape s{nullptr, nullptr, 1, T_, (E + BN - 1) / BN * BN, d, E};
  Operand A{x, nullptr, 0, d};
  Operand B{w_r, nullptr, 0, E};
  typename Epi::Params ep{logits, E, bias};
  long long tiles = (long long)((T_ + BM - 1) / BM) * ((E + BN - 1) / BN);
  return run_gemm<T, BM, BN, false, B_KN, false, Epi>(s, A, B, ep, tiles, st);
}

template <typename T>
hipError_t up_swiglu(const void* x, const void* w1, const int32_t* row_token, const int32_t* offsets,
                     const int32_t* tile_offsets, int E, int d, int n, size_t cap, void* H, void* A,
                     hipStream_t st) {
  constexpr int BN = Cfg<T>::UP_BN;
  using Epi = EpiSwiGLU<T, BM, BN>;
  GemmShape s{offsets, tile_offsets, E, 0, 2 * n, d, 2 * n};
  Operand a{x, row_token, 0, d};
  Operand b{w1, nullptr, (long long)d * 2 * n, 2 * n};
  typename Epi::Params ep{reinterpret_cast<T*>(H), reinterpret_cast<T*>(A), n};
  return run_gemm<T, BM, BN, false, B_KN, true, Epi>(s, a, b, ep,
                                                      row_tiles_bound(cap, E, BM) * (2 * n / BN), st);
}

template <typename T>
hipError_t down(const void* A, const void* w2, const int32_t* offsets, const int32_t* tile_offsets,
                int E, int d, int n, size_t cap, void* Y, hipStream_t st) {
  constexpr int BN = Cfg<T>::DOWN_BN;
  using Epi = EpiStore<T, T, BM, BN>;
  GemmShape s{offsets, tile_offsets, E, 0, d, n, d};
  Operand a{A, nullptr, 0, n};
  Operand b{w2, nullptr, (long long)n * d, d};
  typename Epi::Params ep{reinterpret_cast<T*>(Y), d, nullptr};
  return run_gemm<T, BM, BN, false, B_KN, false, Epi>(s, a, b, ep,
                                                       row_tiles_bound(cap, E, BM) * (d / BN), st);
}

template <typename T>
hipError_t dh(const void* d_o, const void* w2, const void* H, const int32_t* row_token,
              const float* row_gate, const int32_t* offsets, const int32_t* tile_offsets, int E, int d,
              int n, size_t cap, void* dH, void* As, float* dS_part, hipStream_t st) {
  constexpr int BN = Cfg<T>::DH_BN;
  using Epi = EpiDH<T, BM, BN>;
  GemmShape s{offsets, tile_offsets, E, 0, n, d, n};
  Operand a{d_o, row_token, 0, d};
  Operand b{w2, nullptr, (long long)n * d, d};  // W2[e] is [n][d]: row j holds k = 0..d-1
  typename Epi::Params ep{reinterpret_cast<const T*>(H), row_gate, reinterpret_cast<T*>(dH),
                          reinterpret_cast<T*>(As), dS_part, n, n / BN};
  return run_gemm<T, BM, BN, false, B_NK, false, Epi>(s, a, b, ep,
                                                       row_tiles_bound(cap, E, BM) * (n / BN), st);
}

template <typename T>
hipError_t dxt(const void* dH, const void* w1, const int32_t* offsets, const int32_t* tile_offsets,
               int E, int d, int n, size_t cap, void* dXt, hipStream_t st) {
  constexpr int BN = Cfg<T>::DXT_BN;
  using Epi = EpiStore<T, T, BM, BN>;
  GemmShape s{offsets, tile_offsets, E, 0, d, 2 * n, d};
  Operand a{dH, nullptr, 0, 2 * n};
  Operand b{w1, nullptr, (long long)d * 2 * n, 2 * n};  // W1[e] is [d][2n]: row i holds k = 0..2n-1
  typename Epi::Params ep{reinterpret_cast<T*>(dXt), d, nullptr};
  return run_gemm<T, BM, BN, false, B_NK, false, Epi>(s, a, b, ep,
                                                       row_tiles_bound(cap, E, BM) * (d / BN), st);
}

template <typename T>
hipError_t dw1(const void* x, const void* dH, const int32_t* row_token, const int32_t* offsets, int E,
               int d, int n, void* dW1, hipStream_t st) {
  constexpr int BN = Cfg<T>::DW1_BN;
  using Epi = EpiStore<T, T, BM, BN>;
  GemmShape s{offsets, nullptr, E, d, 2 * n, 0, 2 * n};
  Operand a{x, row_token, 0, d};
  Operand b{dH, nullptr, 0, 2 * n};
  typename Epi::Params ep{reinterpret_cast<T*>(dW1), 2 * n, nullptr};
  return run_gemm<T, BM, BN, true, B_KN, false, Epi>(s, a, b, ep,
                                                      (long long)E * (d / BM) * (2 * n / BN), st);
}

template <typename T, int BMW>
hipError_t dw2_impl(const void* As, const void* d_o, const int32_t* row_token, const int32_t* offsets,
                    int E, int d, int n, void* dW2, hipStream_t st) {
  constexpr int BN = Cfg<T>::DW2_BN;
  using Epi = EpiStore<T, T, BMW, BN>;
  GemmShape s{offsets, nullptr, E, n, d, 0, d};
  Operand a{As, nullptr, 0, n};
  Operand b{d_o, row_token, 0, d};
  typename Epi::Params ep{reinterpret_cast<T*>(dW2), d, nullptr};
  return run_gemm<T, BMW, BN, true, B_KN, false, Epi>(s, a, b, ep,
                                                       (long long)E * (n / BMW) * (d / BN), st);
}

template <typename T>
hipError_t dw2(const void* As, const void* d_o, const int32_t* row_token, const int32_t* offsets, int E,
               int d, int n, void* dW2, hipStream_t st) {
  if (n % 128 == 0) return dw2_impl<T, 128>(As, d_o, row_token, offsets, E, d, n, dW2, st);
  return dw2_impl<T, 64>(As, d_o, row_token, offsets, E, d, n, dW2, st);
}

template <typename T>
hipError_t dwr(const void* x, const void* dz, int T_, int d, int E, void* dWr, hipStream_t st) {
  constexpr int BN = Cfg<T>::DWR_BN;
  using Epi = EpiStore<T, T, BM, BN>;
  GemmShape s{nullptr, nullptr, 1, d, (E + BN - 1) / BN * BN, T_, E};
  Operand a{x, nullptr, 0, d};
  Operand b{dz, nullptr, 0, E};
  typename Epi::Params ep{reinterpret_cast<T*>(dWr), E, nullptr};
  return run_gemm<T, BM, BN, true, B_KN, false, Epi>(s, a, b, ep,
                                                      (long long)(d / BM) * ((E + BN - 1) / BN), st);
}

}  // namespace

int dh_block(int dtype) { return dtype == DT_BF16 ? Cfg<bf16_t>::DH_BN : Cfg<float>::DH_BN; }

#define MOE_DISPATCH(dtype, fn, ...) \
  ((dtype) == DT_BF16 ? fn<bf16_t>(__VA_ARGS__) : fn<float>(__VA_ARGS__))

hipError_t launch_router_logits(int dtype, const void* x, const void* w_r, const float* bias,
                                float* logits, int T, int d, int E, hipStream_t st) {
  return MOE_DISPATCH(dtype, router_logits, x, w_r, bias, logits, T, d, E, st);
}
hipError_t launch_up_swiglu(int dtype, const void* x, const void* w1, const int32_t* row_token,
                            const int32_t* offsets, const int32_t* tile_offsets, int E, int d, int n,
                            size_t cap, void* H, void* A, hipStream_t st) {
  return MOE_DISPATCH(dtype, up_swiglu, x, w1, row_token, offsets, tile_offsets, E, d, n, cap, H, A, st);
}
hipError_t launch_down(int dtype, const void* A, const void* w2, const int32_t* offsets,
                       const int32_t* tile_offsets, int E, int d, int n, size_t cap, void* Y,
                       hipStream_t st) {
  return MOE_DISPATCH(dtype, down, A, w2, offsets, tile_offsets, E, d, n, cap, Y, st);
}
hipError_t launch_dh(int dtype, const void* d_o, const void* w2, const void* H,
                     const int32_t* row_token, const float* row_gate, const int32_t* offsets,
                     const int32_t* tile_offsets, int E, int d, int n, size_t cap, void* dH, void* As,
                     float* dS_part, hipStream_t st) {
  return MOE_DISPATCH(dtype, dh, d_o, w2, H, row_token, row_gate, offsets, tile_offsets, E, d, n, cap,
                      dH, As, dS_part, st);
}
hipError_t launch_dxt(int dtype, const void* dH, const void* w1, const int32_t* offsets,
                      const int32_t* tile_offsets, int E, int d, int n, size_t cap, void* dXt,
                      hipStream_t st) {
  return MOE_DISPATCH(dtype, dxt, dH, w1, offsets, tile_offsets, E, d, n, cap, dXt, st);
}
hipError_t launch_dw1(int dtype, const void* x, const void* dH, const int32_t* row_token,
                      const int32_t* offsets, int E, int d, int n, void* dW1, hipStream_t st) {
  return MOE_DISPATCH(dtype, dw1, x, dH, row_token, offsets, E, d, n, dW1, st);
}
hipError_t launch_dw2(int dtype, const void* As, const void* d_o, const int32_t* row_token,
                      const int32_t* offsets, int E, int d, int n, void* dW2, hipStream_t st) {
  return MOE_DISPATCH(dtype, dw2, As, d_o, row_token, offsets, E, d, n, dW2, st);
}
hipError_t launch_dwr(int dtype, const void* x, const void* dz_dense, int T, int d, int E, void* dWr,
                      hipStream_t st) {
  return MOE_DISPATCH(dtype, dwr, x, dz_dense, T, d, E, dWr, st);
}

}  // namespace moe
