// The unfused layer: the standard MoE workflow the pages set SonicMoE
// against ([A] "MoE 与它的隐患", figure captions of the forward and backward
// workflow; [B] algorithm paragraph), built from this library's kernels as an
// ablation.  Each step that SonicMoE fuses runs here as a kernel of its own:
// the token rows are gathered into a buffer before the up-projection, SwiGLU
// and its backward are element-wise kernels between GEMMs, the routed-row
// activations X_g, H, A and Y are cached from forward to backward, and the
// score gradient is the row dot product dS_r = <dO_g[r], Y[r]>.
//
// Every kernel covers rows 0 .. P-1 with P = offsets[E] read on the device,
// launched over the row capacity.
#include "device_common.h"
#include "launch.h"

namespace moe {

namespace {

// dst[r] = src[idx[r]] (16-byte chunks; one wave per row)
template <typename T>
__global__ void __launch_bounds__(256)
k_gather_rows(const T* __restrict__ src, int width, const int32_t* __restrict__ idx,
              const int32_t* __restrict__ nrows, T* __restrict__ dst) {
  constexpr int V = 16 / sizeof(T);
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (r >= *nrows) return;
  const uint4* s = reinterpret_cast<const uint4*>(src + (size_t)idx[r] * width);
  uint4* o = reinterpret_cast<uint4*>(dst + (size_t)r * width);
  for (int c = lane; c < width / V; c += 64) o[c] = s[c];
}

template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

template <typename T>
__device__ __forceinline__ void store8(T* p, const float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = (uint32_t)f2bf(v[2 * i]) | ((uint32_t)f2bf(v[2 * i + 1]) << 16);
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
}

// A[r][j] = silu(H[r][j]) * H[r][n + j]  (8 columns per thread)
template <typename T>
__global__ void __launch_bounds__(256)
k_swiglu_fwd(const T* __restrict__ H, int n, const int32_t* __restrict__ nrows, T* __restrict__ A) {
  const long long v = (long long)blockIdx.x * 256 + threadIdx.x;
  const int per = n / 8;
  const long long r = v / per;
  const int j = (int)(v % per) * 8;
  if (r >= *nrows) return;
  float g[8], u[8], a[8];
  load8(H + r * 2 * n + j, g);
  load8(H + r * 2 * n + n + j, u);
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = g[i] * sigmoidf_(g[i]) * u[i];
  store8(A + r * n + j, a);
}

// dS[r] = <a[r], b[r]> over `width` columns (fp32 sum; one wave per row)
template <typename T>
__global__ void __launch_bounds__(256)
k_row_dot(const T* __restrict__ a, const T* __restrict__ b, int width, const int32_t* __restrict__ nrows,
          float* __restrict__ out) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (r >= *nrows) return;
  float s = 0.f;
  for (int c = lane * 8; c < width; c += 64 * 8) {
    float x[8], y[8];
    load8(a + (size_t)r * width + c, x);
    load8(b + (size_t)r * width + c, y);
#pragma unroll
    for (int i = 0; i < 8; ++i) s = fmaf(x[i], y[i], s);
  }
  s = wave_sum(s);
  if (lane == 0) out[r] = s;
}

// SwiGLU backward from dA' = dO_g W2^T (stored), the cached H and A:
//   dA = gate dA';  dG = dA U s (1 + G (1 - s));  dU = dA silu(G);  A_s = gate A
template <typename T>
__global__ void __launch_bounds__(256)
k_swiglu_bwd(const T* __restrict__ dAp, const T* __restrict__ H, const T* __restrict__ A,
             const float* __restrict__ gate, int n, const int32_t* __restrict__ nrows, T* __restrict__ dH,
             T* __restrict__ As) {
  const long long v = (long long)blockIdx.x * 256 + threadIdx.x;
  const int per = n / 8;
  const long long r = v / per;
  const int j = (int)(v % per) * 8;
  if (r >= *nrows) return;
  float dap[8], g[8], u[8], a[8], dg[8], du[8], as[8];
  load8(dAp + r * n + j, dap);
  load8(H + r * 2 * n + j, g);
  load8(H + r * 2 * n + n + j, u);
  load8(A + r * n + j, a);
  const float gt = gate[r];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float sg = sigmoidf_(g[i]);
    const float da = gt * dap[i];
    dg[i] = da * u[i] * sg * (1.f + g[i] * (1.f - sg));
    du[i] = da * g[i] * sg;
    as[i] = gt * a[i];
  }
  store8(dH + r * 2 * n + j, dg);
  store8(dH + r * 2 * n + n + j, du);
  store8(As + r * n + j, as);
}

unsigned blocks_rows(size_t cap) { return (unsigned)((cap + 3) / 4); }
unsigned blocks_elems(size_t cap, int n) { return (unsigned)((cap * (size_t)(n / 8) + 255) / 256); }

}  // namespace

hipError_t launch_gather_rows(int dtype, const void* src, int width, const int32_t* idx, const int32_t* nrows,
                              size_t cap, void* dst, hipStream_t st) {
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(k_gather_rows<bf16_t>, dim3(blocks_rows(cap)), dim3(256), 0, st, (const bf16_t*)src, width,
                       idx, nrows, (bf16_t*)dst);
  else
    hipLaunchKernelGGL(k_gather_rows<float>, dim3(blocks_rows(cap)), dim3(256), 0, st, (const float*)src, width,
                       idx, nrows, (float*)dst);
  return hipGetLastError();
}

hipError_t launch_swiglu_fwd(int dtype, const void* H, int n, const int32_t* nrows, size_t cap, void* A,
                             hipStream_t st) {
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(k_swiglu_fwd<bf16_t>, dim3(blocks_elems(cap, n)), dim3(256), 0, st, (const bf16_t*)H, n,
                       nrows, (bf16_t*)A);
  else
    hipLaunchKernelGGL(k_swiglu_fwd<float>, dim3(blocks_elems(cap, n)), dim3(256), 0, st, (const float*)H, n,
                       nrows, (float*)A);
  return hipGetLastError();
}

hipError_t launch_row_dot(int dtype, const void* a, const void* b, int width, const int32_t* nrows, size_t cap,
                          float* out, hipStream_t st) {
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(k_row_dot<bf16_t>, dim3(blocks_rows(cap)), dim3(256), 0, st, (const bf16_t*)a,
                       (const bf16_t*)b, width, nrows, out);
  else
    hipLaunchKernelGGL(k_row_dot<float>, dim3(blocks_rows(cap)), dim3(256), 0, st, (const float*)a,
                       (const float*)b, width, nrows, out);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(int dtype, const void* dAp, const void* H, const void* A, const float* gate, int n,
                             const int32_t* nrows, size_t cap, void* dH, void* As, hipStream_t st) {
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(k_swiglu_bwd<bf16_t>, dim3(blocks_elems(cap, n)), dim3(256), 0, st, (const bf16_t*)dAp,
                       (const bf16_t*)H, (const bf16_t*)A, gate, n, nrows, (bf16_t*)dH, (bf16_t*)As);
  else
    hipLaunchKernelGGL(k_swiglu_bwd<float>, dim3(blocks_elems(cap, n)), dim3(256), 0, st, (const float*)dAp,
                       (const float*)H, (const float*)A, gate, n, nrows, (float*)dH, (float*)As);
  return hipGetLastError();
}

}  // namespace moe
