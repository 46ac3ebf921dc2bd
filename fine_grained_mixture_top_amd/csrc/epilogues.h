// Epilogues of the grouped GEMM: what each MoE kernel does with its
// accumulator tile ([A] "核心创新" second point: SwiGLU fused into the
// up-projection epilogue; the dH kernel's epilogue recomputes the activation
// and forms the score gradient).
//
// The main loop parks the fp32 tile in LDS ([BM][BN + 4], see stage_acc);
// every epilogue then walks it in 8-column chunks of whole rows, NTH threads
// at a time, so its global reads and writes are coalesced 16-byte accesses
// and the element-wise math keeps few values live.
#pragma once

#include "grouped_gemm.h"

namespace moe {

// C[row, n0 + col] = acc (+ bias[col]), converted to TO.
// ROW mode: row = routed row; WGT mode: row = slice*M + m (rows of all
// slices' [M][N] blocks are contiguous).
template <typename T, typename TO, int BM, int BN, int NTH = 256>
struct EpiStore {
  struct Params {
    TO* C;
    long long ldc;
    const float* bias;  // per column, may be null
    // router term of the input-gradient rows, may be null: C[row, col] +=
    // dz[row] * v[e, col] (v: the transposed router weights, [E][ldc])
    const float* dz;
    const TO* v;
  };
  static constexpr int SMEM = 0;

  __device__ __forceinline__ static void run(const Params& p, const GemmShape& s, const TileCtx& c,
                                             const float* Cs, char*) {
    constexpr int LDC = BN + 4, CPR = BN / 8;
    const int cols = min(BN, s.n_valid - c.n0);
    for (int v = c.tid; v < BM * CPR; v += NTH) {
      const int r = v / CPR, ch = v % CPR;
      if (r < c.m_valid && ch * 8 < cols) {
        float x[8];
        ld8(Cs + r * LDC + ch * 8, x);
        if (p.bias) {
#pragma unroll
          for (int i = 0; i < 8; ++i) x[i] += p.bias[c.n0 + ch * 8 + i];
        }
        if (p.dz) {
          const float z = p.dz[c.out_row0 + r];
          const TO* vr = p.v + (long long)c.e * p.ldc + c.n0 + ch * 8;
#pragma unroll
          for (int i = 0; i < 8; ++i) x[i] = fmaf(z, Elem<TO>::to_f(vr[i]), x[i]);
        }
        st8<TO>(p.C + (c.out_row0 + r) * p.ldc + c.n0 + ch * 8, x);
      }
    }
  }
};

// Up-projection epilogue (K1).  The staged tile holds BN/2 gate columns then
// the matching BN/2 "up" columns (global columns j0.. and n + j0..).  H is
// rounded to the storage type first and A = silu(G)*U is formed from the
// rounded values, so the backward's recomputation of A from the cached H
// reproduces it exactly.
template <typename T, int BM, int BN, int NTH = 256>
struct EpiSwiGLU {
  struct Params {
    T* H;     // [rows, 2n]
    T* A;     // [rows, n]
    int n;
  };
  static constexpr int SMEM = 0;

  __device__ __forceinline__ static void run(const Params& p, const GemmShape&, const TileCtx& c,
                                             const float* Cs, char*) {
    constexpr int LDC = BN + 4, CPR = BN / 16;
    const int j0 = c.nt * (BN / 2);
    const long long ldh = 2LL * p.n;
    for (int v = c.tid; v < BM * CPR; v += NTH) {
      const int r = v / CPR, jj = (v % CPR) * 8;
      if (r < c.m_valid) {
        float g[8], u[8], a[8];
        ld8(Cs + r * LDC + jj, g);
        ld8(Cs + r * LDC + BN / 2 + jj, u);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          g[i] = through<T>(g[i]);
          u[i] = through<T>(u[i]);
          a[i] = g[i] * sigmoidf_(g[i]) * u[i];
        }
        const long long row = c.out_row0 + r;
        st8<T>(p.H + row * ldh + j0 + jj, g);
        st8<T>(p.H + row * ldh + p.n + j0 + jj, u);
        st8<T>(p.A + row * (long long)p.n + j0 + jj, a);
      }
    }
  }
};

// dH epilogue (K4).  The staged tile is dA' = dO[tok] W2^T for columns
// j = n0 .. n0+BN-1.  From the cached H it recomputes A = silu(G)*U, then
//   dS partial = sum_j dA'_j A_j          (the reordered router contraction)
//   dA = gate * dA',  dG = dA*U*s*(1+G*(1-s)),  dU = dA*silu(G)
//   A_s = gate * A                        (operand of the dW2 GEMM)
// The BN/8 chunks of a row sit on consecutive lanes, which sum the row's
// partial with shuffles.
template <typename T, int BM, int BN, int NTH = 256>
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
  static constexpr int SMEM = 0;
  static_assert((BN / 8) <= 64 && (64 % (BN / 8)) == 0, "row chunks must tile a wave");

  __device__ __forceinline__ static void run(const Params& p, const GemmShape&, const TileCtx& c,
                                             const float* Cs, char*) {
    constexpr int LDC = BN + 4, CPR = BN / 8;
    const long long ldh = 2LL * p.n;
    for (int v = c.tid; v < BM * CPR; v += NTH) {
      const int r = v / CPR, ch = v % CPR;
      const bool valid = r < c.m_valid;
      const long long grow = c.out_row0 + (valid ? r : c.m_valid - 1);
      const int col = c.n0 + ch * 8;
      float dap[8], g[8], u[8];
      ld8(Cs + r * LDC + ch * 8, dap);
      ld8g<T>(p.H + grow * ldh + col, g);
      ld8g<T>(p.H + grow * ldh + p.n + col, u);
      const float gt = p.gate[grow];
      float dg[8], du[8], as[8];
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float sg = sigmoidf_(g[i]);
        const float sl = g[i] * sg;
        const float a = sl * u[i];
        ps += dap[i] * a;
        const float da = gt * dap[i];
        dg[i] = da * u[i] * sg * (1.f + g[i] * (1.f - sg));
        du[i] = da * sl;
        as[i] = gt * a;
      }
      if (valid) {
        st8<T>(p.dH + grow * ldh + col, dg);
        st8<T>(p.dH + grow * ldh + p.n + col, du);
        st8<T>(p.As + grow * (long long)p.n + col, as);
      }
#pragma unroll
      for (int o = 1; o < CPR; o <<= 1) ps += __shfl_xor(ps, o, 64);
      if (valid && ch == 0) p.dS_part[grow * p.NT + c.nt] = ps;
    }
  }
};

}  // namespace moe
