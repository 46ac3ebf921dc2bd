// MXFP8 grouped GEMMs: quantization of the GEMM operands to the OCP MX
// format (E4M3 elements, one E8M0 scale per 32 consecutive values along the
// reduction) and the two forward GEMMs and two activation-gradient GEMMs on
// the MX-scaled MFMA (grouped_gemm_mx.h).  The pages name MXFP8 as the method's next precision
// step ([A] closing "未来展望" paragraph); the format is the OCP MX
// specification's (section 5: blocks and scales; section 6.3: the shared
// exponent floor(log2(amax)) - emax of the element type, 8 for E4M3).
//
// Rounding: elements round to nearest, ties to even, after an exact
// power-of-two division by the block scale; magnitudes beyond 448 saturate
// to 448 (the block's largest value lands in [256, 512) before rounding, so
// only the top of that range saturates).  An all-zero block gets scale code
// 0 and zero elements.
#include <algorithm>

#include "grouped_gemm_mx.h"
#include "launch.h"

namespace moe {

namespace {

// E8M0 scale code of a block whose largest magnitude is amax (> 0)
__device__ __forceinline__ int scale_code(float amax) {
  const int c = (int)(__float_as_uint(amax) >> 23) - 8;  // floor(log2 amax) - 8 + 127
  return c < 0 ? 0 : (c > 254 ? 254 : c);
}

// E4M3 codes of four values already clamped to [-448, 448], packed into a
// word (value i in byte i), by the hardware conversion: nearest code, ties to
// even, subnormal codes below 2^-6, the sign kept on zero.  The MXFP8 parity
// tests run every finite bf16 pattern below 2^61 through it against the
// oracle's encoder.
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

__device__ __forceinline__ float clamp448(float x) { return __builtin_amdgcn_fmed3f(x, -448.f, 448.f); }

// quantize 32 values (fp32 holding bf16 values) to codes packed 4 per word;
// returns the scale code
__device__ __forceinline__ int quant32(const float (&v)[32], uint32_t (&q)[8]) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  if (amax == 0.f) {
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = 0u;
    return 0;
  }
  const int sc = scale_code(amax);
  const float inv = __uint_as_float((uint32_t)(254 - sc) << 23);  // 2^(127 - sc)
#pragma unroll
  for (int i = 0; i < 8; ++i)
    q[i] = e4m3_pack4(clamp448(v[4 * i] * inv), clamp448(v[4 * i + 1] * inv), clamp448(v[4 * i + 2] * inv),
                      clamp448(v[4 * i + 3] * inv));
  return sc;
}

// rows [rows][K] bf16 -> codes [rows][K], scales [rows][K/32]; one thread per
// block of 32.  rows = *nrows when nrows is set (launched over the capacity).
// bN > 0: the rows are E stacked [bN][K] weight matrices whose scales go to
// the stage-blocked layout [E][K/128][bN] (4 bytes each) instead.
__global__ void __launch_bounds__(256)
k_mx_quant_rows(const bf16_t* __restrict__ src, int K, long long rows, const int32_t* __restrict__ nrows,
                uint8_t* __restrict__ q, uint8_t* __restrict__ s, int bN) {
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  const int nb = K / 32;
  const long long row = t / nb;
  const int kb = (int)(t % nb);
  const long long nr = nrows ? (long long)*nrows : rows;
  if (row >= nr) return;
  const uint4* p = reinterpret_cast<const uint4*>(src + row * K + kb * 32);
  float v[32];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint4 u = p[c];
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[8 * c + 2 * i] = __uint_as_float(w[i] << 16);
      v[8 * c + 2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  uint32_t qw[8];
  const int sc = quant32(v, qw);
  uint4* o = reinterpret_cast<uint4*>(q + row * K + kb * 32);
  o[0] = make_uint4(qw[0], qw[1], qw[2], qw[3]);
  o[1] = make_uint4(qw[4], qw[5], qw[6], qw[7]);
  if (bN > 0) {
    const long long e = row / bN, col = row % bN;
    s[((e * (K / 128) + kb / 4) * bN + col) * 4 + (kb & 3)] = (uint8_t)sc;
  } else {
    s[row * nb + kb] = (uint8_t)sc;
  }
}

// weights W [E][K][N] bf16 -> transposed codes [E][N][K] and stage-blocked
// scales [E][K/128][N] (dword per column and 128-k group, byte b = k-block b
// of the group).  One workgroup per (expert, 128-k group, 64 columns): the
// 128 x 64 tile is read in whole rows, each thread quantizes one
// (column, 32-k block) from LDS, and the codes leave as 128-byte rows of the
// transposed matrix.
__global__ void __launch_bounds__(256)
k_mx_quant_w(const bf16_t* __restrict__ W, int K, int N, uint8_t* __restrict__ q, uint32_t* __restrict__ sblk) {
  __shared__ bf16_t tin[128][64 + 2];
  __shared__ uint32_t tout[64][32 + 1];  // codes of 64 columns x 128 k, 4 per word
  const int tid = threadIdx.x;
  const int cg = blockIdx.x, kg = blockIdx.y, e = blockIdx.z;
  const int c0 = cg * 64, k0 = kg * 128;
  const bf16_t* src = W + ((long long)e * K + k0) * N + c0;
#pragma unroll
  for (int it = 0; it < 8; ++it) {  // 128 rows x 64 columns, 4 columns (8 bytes) per thread
    const int v = it * 256 + tid, r = v >> 4, c4 = (v & 15) * 4;
    const uint2 x = *reinterpret_cast<const uint2*>(src + (long long)r * N + c4);
    tin[r][c4] = (bf16_t)(x.x & 0xffffu);
    tin[r][c4 + 1] = (bf16_t)(x.x >> 16);
    tin[r][c4 + 2] = (bf16_t)(x.y & 0xffffu);
    tin[r][c4 + 3] = (bf16_t)(x.y >> 16);
  }
  __syncthreads();
  const int col = tid & 63, b = tid >> 6;  // 32-k block b of the group
  float v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = __uint_as_float((uint32_t)tin[32 * b + i][col] << 16);
  uint32_t qw[8];
  const int sc = quant32(v, qw);
#pragma unroll
  for (int i = 0; i < 8; ++i) tout[col][8 * b + i] = qw[i];
  // the group's four block scales of this column, one byte each
  __shared__ uint32_t ts[4][64];
  ts[b][col] = (uint32_t)sc;
  __syncthreads();
  if (tid < 64) sblk[((long long)e * (K / 128) + kg) * N + c0 + tid] =
      ts[0][tid] | (ts[1][tid] << 8) | (ts[2][tid] << 16) | (ts[3][tid] << 24);
#pragma unroll
  for (int it = 0; it < 2; ++it) {  // 64 rows of 128 bytes, 16 bytes per thread
    const int v2 = it * 256 + tid, r = v2 >> 3, ch = v2 & 7;
    *reinterpret_cast<uint4*>(q + ((long long)e * N + c0 + r) * K + k0 + ch * 16) =
        make_uint4(tout[r][4 * ch], tout[r][4 * ch + 1], tout[r][4 * ch + 2], tout[r][4 * ch + 3]);
  }
}

// Weight-gradient operands: each expert's segment of routed rows is
// quantized along its rows (the weight-gradient GEMMs' reduction), the
// segment padded with zero rows to a multiple of 128 (one GEMM stage).
// padoff[e] = sum over experts before e of the padded lengths; stage_e[g] =
// the expert of global stage g (g < padoff[E] / 128).  One workgroup.
__global__ void __launch_bounds__(1024)
k_mx_pad_offsets(const int32_t* __restrict__ offsets, int E, int32_t* __restrict__ padoff,
                 int32_t* __restrict__ stage_e) {
  __shared__ int32_t ps[1025];
  __shared__ int32_t wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int len = tid < E ? (offsets[tid + 1] - offsets[tid] + 127) / 128 * 128 : 0;
  int incl = len;
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int base = 0;
  for (int x = 0; x < w; ++x) base += wsum[x];
  if (tid < E) ps[tid] = base + incl - len;
  if (tid == E - 1) ps[E] = base + incl;
  __syncthreads();
  for (int e = tid; e <= E; e += 1024) padoff[e] = ps[e];
  // stage map: expert e owns stages ps[e]/128 .. ps[e+1]/128 - 1; stage g's
  // expert is the last e with ps[e] <= 128 g (binary search; ps ascending,
  // empty experts share their start with the next one)
  const int stages = ps[E] / 128;
  for (int g = tid; g < stages; g += 1024) {
    int lo = 0, hi = E;  // ps[lo] <= 128 g < ps[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (ps[mid] <= 128 * g) lo = mid;
      else hi = mid;
    }
    stage_e[g] = lo;
  }
}

// src rows [*][C] bf16 (row r of expert e's segment is src[idx[seg0 + r]],
// or src[seg0 + r] without idx) -> per expert, codes [C][Kp_e] at byte
// C * padoff[e] (Kp_e = padded segment length) and stage-blocked scales: the
// dword (padoff[e] / 128 + s) * C + c holds column c's four block scales of
// stage s (byte b = rows 128 s + 32 b .. +31).  One workgroup per (64
// columns, global stage): the 128 x 64 tile is read in whole rows, 16 bytes
// per thread (zeros past the segment), each thread quantizes one (column,
// 32-row block) from LDS, and the codes leave as 128-byte rows.  Workgroups past the last stage
// return.
__global__ void __launch_bounds__(256)
k_mx_quant_seg(const bf16_t* __restrict__ src, int C, const int32_t* __restrict__ idx,
               const int32_t* __restrict__ offsets, const int32_t* __restrict__ padoff,
               const int32_t* __restrict__ stage_e, int E, uint8_t* __restrict__ q, uint32_t* __restrict__ sblk) {
  __shared__ __attribute__((aligned(16))) bf16_t tin[128][64 + 8];  // rows of 144 bytes: 16-byte stores
  __shared__ uint32_t tout[64][32 + 1];
  __shared__ uint32_t ts[4][64];
  const int tid = threadIdx.x;
  const int c0 = blockIdx.x * 64, g = blockIdx.y;
  if (g >= padoff[E] / 128) return;  // uniform over the workgroup
  const int e = stage_e[g];
  const int seg0 = offsets[e], segn = offsets[e + 1] - seg0;
  const int pe = padoff[e], kp = padoff[e + 1] - pe;
  const int s = g - pe / 128;  // stage of the segment
#pragma unroll
  for (int it = 0; it < 4; ++it) {  // 128 rows x 64 columns, 8 columns (16 bytes) per thread
    const int v = it * 256 + tid, r = v >> 3, c8 = (v & 7) * 8;
    const int sr = 128 * s + r;
    uint4 x = make_uint4(0u, 0u, 0u, 0u);
    if (sr < segn) {
      const long long row = idx ? (long long)idx[seg0 + sr] : (long long)(seg0 + sr);
      x = *reinterpret_cast<const uint4*>(src + row * C + c0 + c8);
    }
    *reinterpret_cast<uint4*>(&tin[r][c8]) = x;
  }
  __syncthreads();
  const int col = tid & 63, b = tid >> 6;  // 32-row block b of the stage
  float v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = __uint_as_float((uint32_t)tin[32 * b + i][col] << 16);
  uint32_t qw[8];
  const int sc = quant32(v, qw);
#pragma unroll
  for (int i = 0; i < 8; ++i) tout[col][8 * b + i] = qw[i];
  ts[b][col] = (uint32_t)sc;
  __syncthreads();
  if (tid < 64)
    sblk[(long long)(pe / 128 + s) * C + c0 + tid] = ts[0][tid] | (ts[1][tid] << 8) | (ts[2][tid] << 16) | (ts[3][tid] << 24);
  uint8_t* qe = q + (long long)C * pe;
#pragma unroll
  for (int it = 0; it < 2; ++it) {  // 64 rows of 128 bytes, 16 bytes per thread
    const int v2 = it * 256 + tid, r = v2 >> 3, ch = v2 & 7;
    *reinterpret_cast<uint4*>(qe + (long long)(c0 + r) * kp + 128 * s + ch * 16) =
        make_uint4(tout[r][4 * ch], tout[r][4 * ch + 1], tout[r][4 * ch + 2], tout[r][4 * ch + 3]);
  }
}

int cu_count() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 256;
  return cus;
}

template <bool PAIRED, class Epi>
hipError_t run_gemm_mx(const GemmShape& s, const Operand& A, const Operand& B, const uint8_t* ascale,
                       const uint32_t* bscale, size_t a_bytes, size_t b_bytes, size_t as_bytes, size_t bs_bytes,
                       const typename Epi::Params& ep, long long max_tiles, hipStream_t st) {
  auto kern = gmx::grouped_gemm_mx_kernel<PAIRED, Epi>;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, gmx::SMEM);
  if (attr != hipSuccess) return attr;
  long long grid = std::min<long long>(max_tiles, cu_count());
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(gmx::NTH), gmx::SMEM, st, s, A, B, ascale, bscale,
                     (uint32_t)a_bytes, (uint32_t)b_bytes, (uint32_t)as_bytes, (uint32_t)bs_bytes, ep);
  return hipGetLastError();
}

long long tiles_bound(size_t cap, int E) { return (long long)(cap + gmx::BM - 1) / gmx::BM + E; }

}  // namespace

int dh_mx_partials(const GemmDims& g) { return g.n / gmx::BN; }

bool mx_bwd_shape_ok(const GemmDims& g) {
  return mx_shape_ok(g) && 2 * g.n / 32 <= gmx::MAX_PA && g.cap * (size_t)2 * g.n < (size_t)g4::OOB;
}

bool mx_shape_ok(const GemmDims& g) {
  return g.dtype == DT_BF16 && g.d % 256 == 0 && g.n % 256 == 0 && g.d / 32 <= gmx::MAX_PA &&
         g.n / 32 <= gmx::MAX_PA && (size_t)g.T * g.d < (size_t)g4::OOB && g.cap * (size_t)g.d < (size_t)g4::OOB;
}

hipError_t launch_mx_quant_rows(const void* src, int K, long long rows, const int32_t* nrows, uint8_t* q,
                                uint8_t* s, hipStream_t st, int bN) {
  const long long threads = rows * (K / 32);
  if (threads <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_mx_quant_rows, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st,
                     (const bf16_t*)src, K, rows, nrows, q, s, bN);
  return hipGetLastError();
}

hipError_t launch_mx_quant_w(const void* W, int E, int K, int N, uint8_t* q, uint8_t* sblk, hipStream_t st) {
  // K a multiple of 128, N a multiple of 64 (the MX shapes)
  hipLaunchKernelGGL(k_mx_quant_w, dim3((unsigned)(N / 64), (unsigned)(K / 128), (unsigned)E), dim3(256), 0, st,
                     (const bf16_t*)W, K, N, q, reinterpret_cast<uint32_t*>(sblk));
  return hipGetLastError();
}

hipError_t launch_up_mx(const GemmDims& g, const uint8_t* xq, const uint8_t* xs, const uint8_t* w1q,
                        const uint8_t* w1s, const int32_t* row_token, const int32_t* offsets, void* H, void* A,
                        hipStream_t st) {
  const int n = g.n, d = g.d, E = g.E;
  using Epi = g4::G4SwiGLU;
  GemmShape s{offsets, E, 0, 2 * n, d, 2 * n, 1};
  Operand a{xq, row_token, 0, d};
  Operand b{w1q, nullptr, (long long)2 * n * d, d};
  typename Epi::Params ep{reinterpret_cast<bf16_t*>(H), reinterpret_cast<bf16_t*>(A), n};
  return run_gemm_mx<true, Epi>(s, a, b, xs, reinterpret_cast<const uint32_t*>(w1s), (size_t)g.T * d,
                                (size_t)2 * n * d, (size_t)g.T * (d / 32), (size_t)(d / 128) * 2 * n * 4, ep,
                                tiles_bound(g.cap, E) * (2 * n / gmx::BN), st);
}

hipError_t launch_dxt_mx(const GemmDims& g, const uint8_t* dhq, const uint8_t* dhs, const uint8_t* w1q,
                         const uint8_t* w1s, const int32_t* offsets, void* dXt, const float* dz, const void* w_rT,
                         hipStream_t st) {
  const int n = g.n, d = g.d, E = g.E;
  using Epi = g4::G4StoreRouter;
  GemmShape s{offsets, E, 0, d, 2 * n, d, 1};
  Operand a{dhq, nullptr, 0, 2 * n};
  Operand b{w1q, nullptr, (long long)d * 2 * n, 2 * n};
  typename Epi::Params ep{reinterpret_cast<bf16_t*>(dXt), d, dz, reinterpret_cast<const bf16_t*>(w_rT),
                          (uint32_t)(g.cap * 4), (uint32_t)((size_t)E * d * 2)};
  return run_gemm_mx<false, Epi>(s, a, b, dhs, reinterpret_cast<const uint32_t*>(w1s), g.cap * 2 * n,
                                 (size_t)d * 2 * n, g.cap * (2 * n / 32), (size_t)(2 * n / 128) * d * 4, ep,
                                 tiles_bound(g.cap, E) * (d / gmx::BN), st);
}

hipError_t launch_dh_mx(const GemmDims& g, const uint8_t* doq, const uint8_t* dos, const uint8_t* w2q,
                        const uint8_t* w2s, const int32_t* row_token, const float* row_gate, const int32_t* offsets,
                        const void* H, void* dH, void* As, float* dS_part, hipStream_t st) {
  const int n = g.n, d = g.d, E = g.E;
  using Epi = g5::G5DH;
  GemmShape s{offsets, E, 0, n, d, n, 1};
  Operand a{doq, row_token, 0, d};
  Operand b{w2q, nullptr, (long long)n * d, d};
  typename Epi::Params ep{reinterpret_cast<const bf16_t*>(H), row_gate, reinterpret_cast<bf16_t*>(dH),
                          reinterpret_cast<bf16_t*>(As), dS_part, n, n / gmx::BN};
  return run_gemm_mx<false, Epi>(s, a, b, dos, reinterpret_cast<const uint32_t*>(w2s), (size_t)g.T * d,
                                 (size_t)n * d, (size_t)g.T * (d / 32), (size_t)(d / 128) * n * 4, ep,
                                 tiles_bound(g.cap, E) * (n / gmx::BN), st);
}

hipError_t launch_mx_pad_offsets(const int32_t* offsets, int E, int32_t* padoff, int32_t* stage_e, hipStream_t st) {
  hipLaunchKernelGGL(k_mx_pad_offsets, dim3(1), dim3(1024), 0, st, offsets, E, padoff, stage_e);
  return hipGetLastError();
}

long long mx_seg_rows_bound(const GemmDims& g) { return (long long)g.cap + 127LL * g.E; }

hipError_t launch_mx_quant_seg(const void* src, int C, const int32_t* idx, const int32_t* offsets,
                               const int32_t* padoff, const int32_t* stage_e, const GemmDims& g, uint8_t* q,
                               uint32_t* sblk, hipStream_t st) {
  const long long stages = (mx_seg_rows_bound(g) + 127) / 128;
  hipLaunchKernelGGL(k_mx_quant_seg, dim3((unsigned)(C / 64), (unsigned)stages), dim3(256), 0, st,
                     (const bf16_t*)src, C, idx, offsets, padoff, stage_e, g.E, q, sblk);
  return hipGetLastError();
}

bool mx_wgrad_shape_ok(const GemmDims& g) {
  const size_t rows = (size_t)mx_seg_rows_bound(g);
  const size_t widest = (size_t)std::max(std::max(g.d, 2 * g.n), g.n);
  return g.dtype == DT_BF16 && g.d % 256 == 0 && g.n % 256 == 0 && g.E <= MAX_E && widest * rows < (size_t)g4::OOB;
}

hipError_t launch_wgrad_mx(const GemmDims& g, int Ma, int Nb, const int32_t* padoff, const uint8_t* qa,
                           const uint32_t* sa, const uint8_t* qb, const uint32_t* sb, void* dW, hipStream_t st) {
  using Epi = g4::G4Store;
  auto kern = gmx::grouped_gemm_mxw_kernel<Epi>;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, gmx::WSMEM);
  if (attr != hipSuccess) return attr;
  const size_t rows = (size_t)mx_seg_rows_bound(g);
  const long long tiles = (long long)g.E * (Ma / gmx::BM) * (Nb / gmx::BN);
  long long grid = std::min<long long>(tiles, cu_count());
  if (grid < 1) grid = 1;
  typename Epi::Params ep{reinterpret_cast<bf16_t*>(dW), Nb};
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(gmx::NTH), gmx::WSMEM, st, g.E, Ma, Nb, padoff, qa, sa, qb,
                     sb, (uint32_t)(rows * Ma), (uint32_t)(rows * Nb), (uint32_t)(rows / 128 * Ma * 4),
                     (uint32_t)(rows / 128 * Nb * 4), ep);
  return hipGetLastError();
}

hipError_t launch_down_mx(const GemmDims& g, const uint8_t* aq, const uint8_t* as, const uint8_t* w2q,
                          const uint8_t* w2s, const int32_t* offsets, void* Y, hipStream_t st) {
  const int n = g.n, d = g.d, E = g.E;
  using Epi = g4::G4Store;
  GemmShape s{offsets, E, 0, d, n, d, 1};
  Operand a{aq, nullptr, 0, n};
  Operand b{w2q, nullptr, (long long)d * n, n};
  typename Epi::Params ep{reinterpret_cast<bf16_t*>(Y), d};
  return run_gemm_mx<false, Epi>(s, a, b, as, reinterpret_cast<const uint32_t*>(w2s), g.cap * n, (size_t)d * n,
                                 g.cap * (n / 32), (size_t)(n / 128) * d * 4, ep,
                                 tiles_bound(g.cap, E) * (d / gmx::BN), st);
}

}  // namespace moe
