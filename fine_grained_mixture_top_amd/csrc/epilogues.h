// Epilogues of the grouped GEMM: what each MoE kernel does with its
// accumulator tile while it is still in registers ([A] "核心创新" second
// point: SwiGLU fused into the up-projection epilogue; the dH kernel's
// epilogue recomputes the activation and forms the score gradient).
#pragma once

#include "grouped_gemm.h"

namespace moe {

// Copy rows of a staged tile (row pitch LD elements) to global memory in
// 16-byte pieces.  dst(r) -> destination of row r (null = skip); only the
// first `cols` columns exist.
template <typename TO, class F>
__device__ __forceinline__ void store_rows(const TO* s, int LD, int rows, int cols, int tid, F dst) {
  constexpr int V = 16 / (int)sizeof(TO);
  const int cpr = cols / V;
  for (int v = tid; v < rows * cpr; v += 256) {
    int r = v / cpr, ch = v - r * cpr;
    TO* d = dst(r);
    if (d) *reinterpret_cast<uint4*>(d + ch * V) = *reinterpret_cast<const uint4*>(s + r * LD + ch * V);
  }
}

// C[row, n0 + col] = acc (+ bias[col]), converted to TO.
// ROW mode: row = routed row; WGT mode: row = e*M + m (rows of all experts'
// [M][N] slices are contiguous).
template <typename T, typename TO, int BM, int BN>
struct EpiStore {
  struct Params {
    TO* C;
    long long ldc;
    const float* bias;  // per column, may be null
  };
  static constexpr int V = 16 / (int)sizeof(TO);
  static constexpr int LD = BN + V;
  static constexpr int SMEM = BM * LD * (int)sizeof(TO);
  using G = TileGeom<T, BM, BN>;

  __device__ static void run(const Params& p, const GemmShape& s, const TileCtx& c,
                             f32x4_v (&acc)[G::FM][G::FN], char* smem) {
    TO* Cs = reinterpret_cast<TO*>(smem);
    const int cols = min(BN, s.n_valid - c.n0);
#pragma unroll
    for (int fn = 0; fn < G::FN; ++fn) {
      const int col = frag_col<T, BM, BN>(c, fn);
      const float b = (p.bias && col < cols) ? p.bias[c.n0 + col] : 0.f;
#pragma unroll
      for (int fm = 0; fm < G::FM; ++fm)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          Cs[frag_row<T, BM, BN>(c, fm, j) * LD + col] = Elem<TO>::from_f(acc[fm][fn][j] + b);
    }
    __syncthreads();
    store_rows<TO>(Cs, LD, BM, cols, c.tid, [&](int r) -> TO* {
      return r < c.m_valid ? p.C + (c.out_row0 + r) * p.ldc + c.n0 : nullptr;
    });
  }
};

// Up-projection epilogue (K1): the tile holds matching gate / up columns
// (ColPaired).  H is rounded to the storage type first and A = silu(G)*U is
// formed from the rounded values, so the backward's recomputation of A from
// the cached H reproduces it exactly.
template <typename T, int BM, int BN>
struct EpiSwiGLU {
  struct Params {
    T* H;     // [rows, 2n]
    T* A;     // [rows, n]
    int n;
  };
  static constexpr int V = 16 / (int)sizeof(T);
  static constexpr int LDH = BN + V, LDA = BN / 2 + V;
  static constexpr int SMEM = BM * (LDH + LDA) * (int)sizeof(T);
  using G = TileGeom<T, BM, BN>;
  static_assert(G::FN % 2 == 0, "paired tile needs an even fragment count");

  __device__ static void run(const Params& p, const GemmShape&, const TileCtx& c,
                             f32x4_v (&acc)[G::FM][G::FN], char* smem) {
    T* Hs = reinterpret_cast<T*>(smem);
    T* As = Hs + BM * LDH;
#pragma unroll
    for (int q = 0; q < G::FN / 2; ++q) {
      const int jj = (c.wn * (G::FN / 2) + q) * 16 + (c.lane & 15);
#pragma unroll
      for (int fm = 0; fm < G::FM; ++fm)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = frag_row<T, BM, BN>(c, fm, j);
          const float g = through<T>(acc[fm][2 * q][j]);
          const float u = through<T>(acc[fm][2 * q + 1][j]);
          const float a = g * sigmoidf_(g) * u;
          Hs[r * LDH + jj] = Elem<T>::from_f(g);
          Hs[r * LDH + BN / 2 + jj] = Elem<T>::from_f(u);
          As[r * LDA + jj] = Elem<T>::from_f(a);
        }
    }
    __syncthreads();
    const int j0 = c.nt * (BN / 2);
    const long long ldh = 2LL * p.n;
    store_rows<T>(Hs, LDH, BM, BN / 2, c.tid, [&](int r) -> T* {
      return r < c.m_valid ? p.H + (c.out_row0 + r) * ldh + j0 : nullptr;
    });
    store_rows<T>(Hs + BN / 2, LDH, BM, BN / 2, c.tid, [&](int r) -> T* {
      return r < c.m_valid ? p.H + (c.out_row0 + r) * ldh + p.n + j0 : nullptr;
    });
    store_rows<T>(As, LDA, BM, BN / 2, c.tid, [&](int r) -> T* {
      return r < c.m_valid ? p.A + (c.out_row0 + r) * (long long)p.n + j0 : nullptr;
    });
  }
};

// dH epilogue (K4).  acc = dA' = dO[tok] W2^T for columns j of this tile.
// From the cached H it recomputes A = silu(G)*U, then
//   dS partial = sum_j dA'_j A_j          (the reordered router contraction)
//   dA = gate * dA',  dG = dA*U*s*(1+G*(1-s)),  dU = dA*silu(G)
//   A_s = gate * A                        (operand of the dW2 GEMM)
template <typename T, int BM, int BN>
struct EpiDH {
  struct Params {
    const T* H;           // [rows, 2n]
    const float* gate;    // [rows]
    T* dH;                // [rows, 2n]
    T* As;                // [rows, n]
    float* dS_part;       // [rows, NT]
    int n;
    int NT;
  };
  static constexpr int V = 16 / (int)sizeof(T);
  static constexpr int LDD = 2 * BN + V, LDS_ = BN + V;
  static constexpr int SMEM = BM * (LDD + LDS_) * (int)sizeof(T) + 2 * BM * 4;
  using G = TileGeom<T, BM, BN>;

  __device__ static void run(const Params& p, const GemmShape&, const TileCtx& c,
                             f32x4_v (&acc)[G::FM][G::FN], char* smem) {
    T* dHs = reinterpret_cast<T*>(smem);
    T* Ass = dHs + BM * LDD;
    float* red = reinterpret_cast<float*>(Ass + BM * LDS_);
    const long long ldh = 2LL * p.n;
    float psum[G::FM][4];
#pragma unroll
    for (int fm = 0; fm < G::FM; ++fm)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = frag_row<T, BM, BN>(c, fm, j);
        const long long grow = c.out_row0 + (r < c.m_valid ? r : c.m_valid - 1);
        const float gt = p.gate[grow];
        const T* hrow = p.H + grow * ldh + c.n0;
        float ps = 0.f;
#pragma unroll
        for (int fn = 0; fn < G::FN; ++fn) {
          const int col = frag_col<T, BM, BN>(c, fn);
          const float g = Elem<T>::to_f(hrow[col]);
          const float u = Elem<T>::to_f(hrow[p.n + col]);
          const float sg = sigmoidf_(g);
          const float sl = g * sg;
          const float a = sl * u;
          const float dap = acc[fm][fn][j];
          ps += dap * a;
          const float da = gt * dap;
          dHs[r * LDD + col] = Elem<T>::from_f(da * u * sg * (1.f + g * (1.f - sg)));
          dHs[r * LDD + BN + col] = Elem<T>::from_f(da * sl);
          Ass[r * LDS_ + col] = Elem<T>::from_f(gt * a);
        }
        psum[fm][j] = ps;
      }
    // row sums over this wave's columns, then over the two column waves
#pragma unroll
    for (int fm = 0; fm < G::FM; ++fm)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float v = sum16(psum[fm][j]);
        if ((c.lane & 15) == 0) red[c.wn * BM + frag_row<T, BM, BN>(c, fm, j)] = v;
      }
    __syncthreads();
    for (int r = c.tid; r < c.m_valid; r += 256)
      p.dS_part[(c.out_row0 + r) * p.NT + c.nt] = red[r] + red[BM + r];
    store_rows<T>(dHs, LDD, BM, BN, c.tid, [&](int r) -> T* {
      return r < c.m_valid ? p.dH + (c.out_row0 + r) * ldh + c.n0 : nullptr;
    });
    store_rows<T>(dHs + BN, LDD, BM, BN, c.tid, [&](int r) -> T* {
      return r < c.m_valid ? p.dH + (c.out_row0 + r) * ldh + p.n + c.n0 : nullptr;
    });
    store_rows<T>(Ass, LDS_, BM, BN, c.tid, [&](int r) -> T* {
      return r < c.m_valid ? p.As + (c.out_row0 + r) * (long long)p.n + c.n0 : nullptr;
    });
  }
};

}  // namespace moe
