// Expert aggregation (O and dX) and the small router-backward kernels.
//
// Aggregation ([B] kernel-list paragraph: the expert-aggregation kernel; it
// is the only non-GEMM kernel of the layer) is a gather-sum over each
// token's rows: bandwidth-bound, so it is one wave per token, 16-byte loads,
// several rows in flight per lane, fp32 accumulation in a fixed (ascending
// row) order, no atomics.
//
// Router backward ([B] algorithm paragraph: the router gradient comes from
// the reordered contraction, no cached Y): dS per row is the sum of the dH
// kernel's per-column-tile partials; dz = gate * (dS - sum over the token's
// set of gate * dS) is the softmax-over-set backward.  It runs per token
// between the dH and dXt GEMMs (k_router_dz), so the dXt GEMM's epilogue
// adds each row's router term dz_r W_r^T[e_r] to its output row, and dX is
// then a plain gather-sum of those rows: the router-weight rows are read once
// per output tile instead of once per routed row.
#include "device_common.h"
#include "launch.h"

namespace moe {

namespace {

template <typename T>
__device__ __forceinline__ void load_vec(const T* p, float (&v)[16 / sizeof(T)]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  if constexpr (sizeof(T) == 2) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    v[0] = __uint_as_float(u.x); v[1] = __uint_as_float(u.y);
    v[2] = __uint_as_float(u.z); v[3] = __uint_as_float(u.w);
  }
}

template <typename T>
__device__ __forceinline__ void store_vec(T* p, const float (&v)[16 / sizeof(T)]) {
  uint4 u;
  if constexpr (sizeof(T) == 2) {
    uint32_t w[4];
#pragma unroll
    // (one conversion per value here: the paired form made the compiler keep
    // the dX kernel's whole accumulator set live twice)
    for (int i = 0; i < 4; ++i) w[i] = (uint32_t)f2bf(v[2 * i]) | ((uint32_t)f2bf(v[2 * i + 1]) << 16);
    u = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    u = make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3]));
  }
  *reinterpret_cast<uint4*>(p) = u;
}

constexpr int UNR = 4;  // rows in flight per lane
// Column chunks per lane per pass (CPL) are a template parameter: the
// launcher picks the smallest CPL (at most 4) that covers a row's 16-byte
// chunks in as few passes as CPL = 4 would, so no chunk slot idles (d = 1536
// bf16: 192 chunks = 64 lanes x 3) and fewer registers stay live.

// Streaming 16-byte load (read once: keep it out of the caches' way).
typedef uint32_t u32x4_v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream(const void* p) {
  const u32x4_v v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_v*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

template <typename T>
__device__ __forceinline__ void unpack(const uint4 u, float (&v)[16 / sizeof(T)]) {
  if constexpr (sizeof(T) == 2) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    v[0] = __uint_as_float(u.x); v[1] = __uint_as_float(u.y);
    v[2] = __uint_as_float(u.z); v[3] = __uint_as_float(u.w);
  }
}

// O[t] = sum over token t's rows (ascending) of gate_r * Y[r] (gate 1 when
// row_gate is null: the dX aggregation).  One wave per token; each lane owns
// up to CPL 16-byte column chunks per pass and keeps UNR rows x CPL chunks of
// loads in flight.
template <typename T, int CPL>
__global__ void __launch_bounds__(256)
k_aggregate_o(const T* __restrict__ Y, const float* __restrict__ row_gate,
              const int32_t* __restrict__ tok_ptr, const int32_t* __restrict__ tok_row, int Tn, int d,
              T* __restrict__ O) {
  constexpr int V = 16 / sizeof(T);
  const int lane = threadIdx.x & 63;
  const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (t >= Tn) return;
  const int j0 = tok_ptr[t], j1 = tok_ptr[t + 1];
  const int nch = d / V;
  for (int cb = 0; cb < nch; cb += 64 * CPL) {
    float acc[CPL][V];
#pragma unroll
    for (int c = 0; c < CPL; ++c)
#pragma unroll
      for (int i = 0; i < V; ++i) acc[c][i] = 0.f;
    for (int j = j0; j < j1; j += UNR) {
      uint4 raw[UNR][CPL];
      float g[UNR];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const bool ok = j + u < j1;
        const int r = ok ? tok_row[j + u] : 0;
        g[u] = ok ? (row_gate ? row_gate[r] : 1.f) : 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const int ch = cb + lane + 64 * c;
          raw[u][c] = (ok && ch < nch) ? ld_stream(Y + (size_t)r * d + ch * V) : make_uint4(0, 0, 0, 0);
        }
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u)
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          float v[V];
          unpack<T>(raw[u][c], v);
#pragma unroll
          for (int i = 0; i < V; ++i) acc[c][i] = fmaf(g[u], v[i], acc[c][i]);
        }
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int ch = cb + lane + 64 * c;
      if (ch < nch) store_vec<T>(O + (size_t)t * d + ch * V, acc[c]);
    }
  }
}

// Router backward per token: dS_r = sum of the row's dH-epilogue partials
// (fixed order), dz_r = g_r (dS_r - sum_j g_j dS_j) over the token's set;
// dS_r and dz_r are written per row and dz as the token's dense row (zeros
// outside its set) for the router weight gradient.  Sixteen lanes per token
// (four tokens per wave, sixteen per workgroup): lane s takes the token's
// rows s, s + 16, ..., the set sum is a fixed butterfly over the sixteen
// lanes, and the dense rows are assembled in LDS (E floats per token) and
// leave as one contiguous block per wave.  The kernel is a chain of dependent
// loads (token CSR -> row -> partials, gate, expert); packing four tokens per
// wave puts the whole batch in flight at once.
template <typename T>
__global__ void __launch_bounds__(256)
k_router_dz(const float* __restrict__ dS_part, int nparts, const float* __restrict__ row_gate,
            const int32_t* __restrict__ row_expert, const int32_t* __restrict__ tok_ptr,
            const int32_t* __restrict__ tok_row, int Tn, int E, float* __restrict__ dS_row,
            float* __restrict__ dz_row, T* __restrict__ dz_dense) {
  extern __shared__ float dzs[];  // [16][E]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = wave * 4 + (lane >> 4), sub = lane & 15;
  const int tw = blockIdx.x * 16 + wave * 4;  // the wave's first token
  const int t = tw + (lane >> 4);
  const bool live = t < Tn;
  float* dense = dzs + slot * E;
  for (int e = sub; e < E; e += 16) dense[e] = 0.f;
  int j0 = 0, j1 = 0;
  if (live) {
    j0 = tok_ptr[t];
    j1 = tok_ptr[t + 1];
  }
  // rows sub, sub + 16, ... of the token: the first kept in registers
  const bool mine = j0 + sub < j1;
  const int r0 = mine ? tok_row[j0 + sub] : 0;
  float s0 = 0.f, g0 = 0.f;
  if (mine) {
    for (int q = 0; q < nparts; ++q) s0 += dS_part[(size_t)r0 * nparts + q];
    g0 = row_gate[r0];
  }
  float part = g0 * s0;
  for (int j = j0 + sub + 16; j < j1; j += 16) {
    const int r = tok_row[j];
    float sv = 0.f;
    for (int q = 0; q < nparts; ++q) sv += dS_part[(size_t)r * nparts + q];
    part += row_gate[r] * sv;
  }
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) part += __shfl_xor(part, m, 16);
  const float tot = part;
  if (mine) {
    const float dz = g0 * (s0 - tot);
    dS_row[r0] = s0;
    dz_row[r0] = dz;
    dense[row_expert[r0]] = dz;
  }
  for (int j = j0 + sub + 16; j < j1; j += 16) {
    const int r = tok_row[j];
    float sv = 0.f;
    for (int q = 0; q < nparts; ++q) sv += dS_part[(size_t)r * nparts + q];
    const float dz = row_gate[r] * (sv - tot);
    dS_row[r] = sv;
    dz_row[r] = dz;
    dense[row_expert[r]] = dz;
  }
  // the wave's four dense rows are one contiguous block of dz_dense (LDS
  // accesses of one wave complete in order, so no barrier is needed)
  const int nt = min(4, Tn - tw);
  const float* wdense = dzs + wave * 4 * E;
  for (int i = lane; i < nt * E; i += 64) dz_dense[(size_t)tw * E + i] = Elem<T>::from_f(wdense[i]);
}

// db[e] = sum of dz over expert e's rows (fixed per-thread split and tree).
__global__ void __launch_bounds__(1024)
k_bias_grad(const float* __restrict__ dz_row, const int32_t* __restrict__ offsets, float* __restrict__ db) {
  __shared__ float red[16];
  const int e = blockIdx.x;
  const int r0 = offsets[e], r1 = offsets[e + 1];
  // four independent partial sums per thread keep four loads in flight
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
  int r = r0 + threadIdx.x;
  for (; r + 3 * 1024 < r1; r += 4 * 1024) {
    s0 += dz_row[r];
    s1 += dz_row[r + 1024];
    s2 += dz_row[r + 2 * 1024];
    s3 += dz_row[r + 3 * 1024];
  }
  for (; r < r1; r += 1024) s0 += dz_row[r];
  float s = wave_sum((s0 + s1) + (s2 + s3));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
    for (int w = 0; w < 16; ++w) t += red[w];
    db[e] = t;
  }
}

// dst[c][r] = src[r][c]
template <typename T>
__global__ void k_transpose(const T* __restrict__ src, int rows, int cols, T* __restrict__ dst) {
  __shared__ T tile[32][33];
  const int r0 = blockIdx.y * 32, c0 = blockIdx.x * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int i = ty; i < 32; i += 8) {
    const int r = r0 + i, c = c0 + tx;
    if (r < rows && c < cols) tile[i][tx] = src[(size_t)r * cols + c];
  }
  __syncthreads();
  for (int i = ty; i < 32; i += 8) {
    const int c = c0 + i, r = r0 + tx;
    if (r < rows && c < cols) dst[(size_t)c * rows + r] = tile[tx][i];
  }
}

}  // namespace

// chunks per lane: fewest passes of 64 x 4 chunks, then the smallest CPL
// that keeps that number of passes
int agg_cpl(int nch) {
  const int passes = (nch + 255) / 256;
  const int per = (nch + 64 * passes - 1) / (64 * passes);
  return per < 1 ? 1 : (per > 4 ? 4 : per);
}

template <typename TE, int CPL>
void agg_o_launch(const void* Y, const float* row_gate, const int32_t* tok_ptr, const int32_t* tok_row, int T,
                  int d, void* O, hipStream_t st) {
  hipLaunchKernelGGL((k_aggregate_o<TE, CPL>), dim3((T + 3) / 4), dim3(256), 0, st, (const TE*)Y, row_gate, tok_ptr,
                     tok_row, T, d, (TE*)O);
}
template <typename TE>
void agg_o_t(const void* Y, const float* row_gate, const int32_t* tok_ptr, const int32_t* tok_row, int T, int d,
             void* O, hipStream_t st) {
  switch (agg_cpl(d / (16 / (int)sizeof(TE)))) {
    case 1: agg_o_launch<TE, 1>(Y, row_gate, tok_ptr, tok_row, T, d, O, st); break;
    case 2: agg_o_launch<TE, 2>(Y, row_gate, tok_ptr, tok_row, T, d, O, st); break;
    case 3: agg_o_launch<TE, 3>(Y, row_gate, tok_ptr, tok_row, T, d, O, st); break;
    default: agg_o_launch<TE, 4>(Y, row_gate, tok_ptr, tok_row, T, d, O, st); break;
  }
}

hipError_t launch_aggregate_o(int dtype, const void* Y, const float* row_gate, const int32_t* tok_ptr,
                              const int32_t* tok_row, int T, int d, void* O, hipStream_t st) {
  if (dtype == DT_BF16) agg_o_t<bf16_t>(Y, row_gate, tok_ptr, tok_row, T, d, O, st);
  else agg_o_t<float>(Y, row_gate, tok_ptr, tok_row, T, d, O, st);
  return hipGetLastError();
}

hipError_t launch_aggregate_dx(int dtype, const void* dXt, const int32_t* tok_ptr, const int32_t* tok_row, int T,
                               int d, void* dX, hipStream_t st) {
  return launch_aggregate_o(dtype, dXt, nullptr, tok_ptr, tok_row, T, d, dX, st);
}

hipError_t launch_router_dz(int dtype, const RouterDzArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)((a.T + 15) / 16)), block(256);
  const size_t lds = (size_t)16 * a.E * sizeof(float);  // 64 KB at E = 1024
  static const hipError_t attr = [] {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_router_dz<bf16_t>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 16 * 1024 * 4);
    if (e == hipSuccess)
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_router_dz<float>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, 16 * 1024 * 4);
    return e;
  }();
  if (attr != hipSuccess) return attr;
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(k_router_dz<bf16_t>, grid, block, lds, st, a.dS_part, a.nparts, a.row_gate, a.row_expert,
                       a.tok_ptr, a.tok_row, a.T, a.E, a.dS_row, a.dz_row, (bf16_t*)a.dz_dense);
  else
    hipLaunchKernelGGL(k_router_dz<float>, grid, block, lds, st, a.dS_part, a.nparts, a.row_gate, a.row_expert,
                       a.tok_ptr, a.tok_row, a.T, a.E, a.dS_row, a.dz_row, (float*)a.dz_dense);
  return hipGetLastError();
}


hipError_t launch_bias_grad(const float* dz_row, const int32_t* offsets, int E, float* db, hipStream_t st) {
  hipLaunchKernelGGL(k_bias_grad, dim3(E), dim3(1024), 0, st, dz_row, offsets, db);
  return hipGetLastError();
}

hipError_t launch_transpose(int dtype, const void* src, int rows, int cols, void* dst, hipStream_t st) {
  dim3 grid((cols + 31) / 32, (rows + 31) / 32), block(256);
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(k_transpose<bf16_t>, grid, block, 0, st, (const bf16_t*)src, rows, cols, (bf16_t*)dst);
  else
    hipLaunchKernelGGL(k_transpose<float>, grid, block, 0, st, (const float*)src, rows, cols, (float*)dst);
  return hipGetLastError();
}

}  // namespace moe
