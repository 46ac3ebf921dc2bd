// Grouped GEMM over ragged expert segments for gfx950: one main loop (MFMA,
// LDS-staged tiles, gathered rows) and a per-kernel epilogue functor.
//
// The pages describe every MoE GEMM as a shared main loop plus a customised
// epilogue, with gathered token rows loaded inside the GEMM instead of by a
// separate gather kernel ([A] "核心创新" second point, and the "软件抽象层 QuACK"
// section).  This is the gfx950 form of that idea:
//
//  * 256 threads = 4 waves of 64 in a 2 x 2 grid; each wave owns a
//    (BM/2) x (BN/2) sub-tile of 16 x 16 MFMA fragments.
//  * bf16: v_mfma_f32_16x16x32_bf16 (8 bf16 of A and of B per lane);
//    fp32:  v_mfma_f32_16x16x4_f32, eight of them per 32-wide k step.
//    A and B feed each MFMA through the same (lane, element) -> k mapping, so
//    every k of the step is summed exactly once.  The accumulator of a 16 x 16
//    fragment holds column lane%16, rows 4*(lane/16)+j, j = 0..3.
//  * LDS holds both operands k-contiguous: As[BM][BK+VEC], Bs[BN][BK+VEC]
//    (16 bytes of padding per row).  Operands that are contiguous along M or
//    N in memory (weights in the forward, gathered rows in the weight
//    gradients) are transposed in registers, in VEC x VEC blocks, on their way
//    into LDS.
//  * Global loads of the next k step are issued into registers before the
//    MFMAs of the current step run.
//  * Persistent: the grid is sized to the machine, each workgroup walks the
//    tile list with stride gridDim.x, from an XCD-aware starting id so that
//    neighbouring tiles (same expert, same rows) share an XCD's L2.
//
// Two modes:
//  ROW mode (K1, K2, K4, K5 and the router GEMM): C rows are the routed rows of
//    an expert segment, A rows are gathered (A.idx[row]) or direct; B is the
//    expert's weight, stored [N][K] (k-contiguous) or [K][N].
//    Tiles: (expert, m tile, n tile) from tile_offsets (prefix of m tiles).
//  WGT mode (K7, K8, router weight gradient): C = sum over an expert's rows r
//    of A[r]^T B[r]; both operands are [rows][M] / [rows][N] with rows
//    gathered or direct; the reduction runs over the ragged segment.
#pragma once

#include "device_common.h"

namespace moe {

struct Operand {
  const void* ptr;     // base pointer
  const int32_t* idx;  // optional gather: segment row -> source row
  long long estride;   // elements between experts (weights); 0 otherwise
  int ld;              // elements between rows
};

struct GemmShape {
  const int32_t* offsets;       // [E+1] row segments; null = one segment
  const int32_t* tile_offsets;  // [E+1] m-tile prefix (ROW mode); null = dense
  int E;                        // experts (1 when dense)
  int M, N, K;                  // ROW: M = rows if dense; WGT: K = rows if dense
  int n_valid;                  // existing columns (<= N rounded up to BN)
};

struct TileCtx {
  int e, mt, nt;
  int seg0, segn;   // segment of the tile's expert
  int m_valid;      // valid rows of this tile (ROW mode)
  long long out_row0;  // ROW: first routed row of the tile; WGT: e*M + mt*BM
  int n0;           // first column of the tile
  int tid, lane, wm, wn;
};

// column remap used by the SwiGLU up-projection: tile column c lives in
// fragment f = c/16; even fragments are gate columns, odd ones the matching
// "up" columns, so each wave holds gate and up values of the same j in the
// same lane.  Global column = (f&1)*half + j0 + (f>>1)*16 + c%16.
struct ColPaired {
  __device__ static int map(int c, int n0_pairs, int half) {
    int f = c >> 4;
    return (f & 1) * half + n0_pairs + (f >> 1) * 16 + (c & 15);
  }
};

template <typename T, int BM, int BN>
struct TileGeom {
  static constexpr int VEC = Elem<T>::VEC;
  static constexpr int BK = Elem<T>::BK;
  static constexpr int LDK = BK + VEC;     // LDS row pitch (elements)
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int FM = WM / 16, FN = WN / 16;
  static constexpr int MAIN_LDS = (BM + BN) * LDK * (int)sizeof(T);
  static_assert(FM >= 1 && FN >= 1, "tile too small");
};

// ---------------------------------------------------------------------------
// loaders
// ---------------------------------------------------------------------------

// R rows of BK contiguous k values; row pointers are fixed per tile.
template <typename T, int R>
struct KMajorLoad {
  static constexpr int VEC = Elem<T>::VEC, BK = Elem<T>::BK, LDK = BK + VEC;
  static constexpr int CPR = BK / VEC;
  static constexpr int NV = R * CPR;
  static constexpr int PER = (NV + 255) / 256;
  const T* ptr[PER];
  uint4 reg[PER];

  // rowptr(r) returns the source row pointer of tile row r (always valid).
  template <class F>
  __device__ void setup(int tid, F rowptr) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      int v = tid + p * 256;
      int r = v / CPR, c = v % CPR;
      ptr[p] = (v < NV) ? rowptr(r < R ? r : 0) + c * VEC : nullptr;
    }
  }
  __device__ void load(int k0) {
#pragma unroll
    for (int p = 0; p < PER; ++p)
      if (ptr[p]) reg[p] = *reinterpret_cast<const uint4*>(ptr[p] + k0);
  }
  __device__ void store(T* lds, int tid) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      int v = tid + p * 256;
      if (v < NV) {
        int r = v / CPR, c = v % CPR;
        *reinterpret_cast<uint4*>(lds + r * LDK + c * VEC) = reg[p];
      }
    }
  }
};

// Transpose a VEC x VEC block held as VEC row vectors (rows = k, columns =
// m/n) into VEC column vectors (one per m/n, holding VEC consecutive k).
__device__ __forceinline__ void transpose_block(const uint4 (&in)[8], uint4 (&out)[8]) {
  const uint32_t* r = reinterpret_cast<const uint32_t*>(in);
  uint32_t* o = reinterpret_cast<uint32_t*>(out);
#pragma unroll
  for (int i = 0; i < 8; ++i) {        // output column (16-bit element i)
#pragma unroll
    for (int m = 0; m < 4; ++m) {      // output dword = k pair (2m, 2m+1)
      uint32_t lo = r[(2 * m) * 4 + (i >> 1)];
      uint32_t hi = r[(2 * m + 1) * 4 + (i >> 1)];
      o[i * 4 + m] = (i & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
    }
  }
}
__device__ __forceinline__ void transpose_block(const uint4 (&in)[4], uint4 (&out)[4]) {
  const uint32_t* r = reinterpret_cast<const uint32_t*>(in);
  uint32_t* o = reinterpret_cast<uint32_t*>(out);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) o[i * 4 + j] = r[j * 4 + i];
}

// BK k-rows x R columns, contiguous along the columns in memory; written to
// LDS transposed ([R][LDK], k contiguous).  Work unit: a VEC x VEC block.
template <typename T, int R>
struct MNMajorLoad {
  static constexpr int VEC = Elem<T>::VEC, BK = Elem<T>::BK, LDK = BK + VEC;
  static constexpr int KB = BK / VEC, CB = R / VEC;
  static constexpr int NB = KB * CB;
  static constexpr int PER = (NB + 255) / 256;
  int col[PER];      // source column offset of the block, -1 = invalid/idle
  uint4 reg[PER][VEC];

  // colmap(c) -> source column of tile column c, or -1 when it does not exist
  template <class F>
  __device__ void setup(int vt, F colmap) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      int b = vt + p * 256;
      col[p] = (b < NB) ? colmap((b % CB) * VEC) : -1;
    }
  }
  // rowptr(k) -> pointer to k-row k of the source, or null when k is invalid
  template <class F>
  __device__ void load(int vt, int k0, F rowptr) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      int b = vt + p * 256;
      int kb = b / CB;
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        const T* rp = (col[p] >= 0) ? rowptr(k0 + kb * VEC + j) : nullptr;
        reg[p][j] = rp ? *reinterpret_cast<const uint4*>(rp + col[p]) : make_uint4(0, 0, 0, 0);
      }
    }
  }
  __device__ void store(T* lds, int vt) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      int b = vt + p * 256;
      if (b < NB) {
        int kb = b / CB, cb = b % CB;
        uint4 out[VEC];
        transpose_block(reg[p], out);
#pragma unroll
        for (int i = 0; i < VEC; ++i)
          *reinterpret_cast<uint4*>(lds + (cb * VEC + i) * LDK + kb * VEC) = out[i];
      }
    }
  }
};

// ---------------------------------------------------------------------------
// MFMA step over one LDS-resident k tile
// ---------------------------------------------------------------------------

template <typename T, int BM, int BN>
struct Mma;

template <int BM, int BN>
struct Mma<bf16_t, BM, BN> {
  using G = TileGeom<bf16_t, BM, BN>;
  __device__ static void step(const bf16_t* As, const bf16_t* Bs, f32x4_v (&acc)[G::FM][G::FN],
                              int lane, int wm, int wn) {
    const int r16 = lane & 15, kq = (lane >> 4) * 8;
#pragma unroll
    for (int ks = 0; ks < G::BK; ks += 32) {
      bf16x8_v a[G::FM], b[G::FN];
#pragma unroll
      for (int fm = 0; fm < G::FM; ++fm)
        a[fm] = __builtin_bit_cast(bf16x8_v, *reinterpret_cast<const uint4*>(
                                                 As + (wm * G::WM + fm * 16 + r16) * G::LDK + ks + kq));
#pragma unroll
      for (int fn = 0; fn < G::FN; ++fn)
        b[fn] = __builtin_bit_cast(bf16x8_v, *reinterpret_cast<const uint4*>(
                                                 Bs + (wn * G::WN + fn * 16 + r16) * G::LDK + ks + kq));
#pragma unroll
      for (int fm = 0; fm < G::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < G::FN; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[fm], b[fn], acc[fm][fn], 0, 0, 0);
    }
  }
};

template <int BM, int BN>
struct Mma<float, BM, BN> {
  using G = TileGeom<float, BM, BN>;
  __device__ static void step(const float* As, const float* Bs, f32x4_v (&acc)[G::FM][G::FN],
                              int lane, int wm, int wn) {
    const int r16 = lane & 15, kq = (lane >> 4) * 8;
    float a[G::FM][8], b[G::FN][8];
#pragma unroll
    for (int fm = 0; fm < G::FM; ++fm) {
      const float* p = As + (wm * G::WM + fm * 16 + r16) * G::LDK + kq;
      *reinterpret_cast<float4*>(&a[fm][0]) = *reinterpret_cast<const float4*>(p);
      *reinterpret_cast<float4*>(&a[fm][4]) = *reinterpret_cast<const float4*>(p + 4);
    }
#pragma unroll
    for (int fn = 0; fn < G::FN; ++fn) {
      const float* p = Bs + (wn * G::WN + fn * 16 + r16) * G::LDK + kq;
      *reinterpret_cast<float4*>(&b[fn][0]) = *reinterpret_cast<const float4*>(p);
      *reinterpret_cast<float4*>(&b[fn][4]) = *reinterpret_cast<const float4*>(p + 4);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int fm = 0; fm < G::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < G::FN; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[fm][j], b[fn][j], acc[fm][fn], 0, 0, 0);
  }
};

// ---------------------------------------------------------------------------
// epilogue helpers: stage fragment values in LDS, then write whole rows
// ---------------------------------------------------------------------------

// Row/col of element j of fragment (fm, fn) inside the tile.
template <typename T, int BM, int BN>
__device__ __forceinline__ int frag_row(const TileCtx& c, int fm, int j) {
  return c.wm * TileGeom<T, BM, BN>::WM + fm * 16 + (c.lane >> 4) * 4 + j;
}
template <typename T, int BM, int BN>
__device__ __forceinline__ int frag_col(const TileCtx& c, int fn) {
  return c.wn * TileGeom<T, BM, BN>::WN + fn * 16 + (c.lane & 15);
}

// Copy a staged [rows][COLS + pad] tile of TO to global memory, 16 bytes at a
// time; dst(r) gives the destination of row r's first element (or null).
template <typename TO, int ROWS, int COLS, class F>
__device__ __forceinline__ void store_staged(const TO* s, int tid, F dst) {
  constexpr int V = 16 / (int)sizeof(TO);
  constexpr int LD = COLS + V;
  constexpr int CPR = COLS / V;
  for (int v = tid; v < ROWS * CPR; v += 256) {
    int r = v / CPR, c = v % CPR;
    TO* d = dst(r);
    if (d) *reinterpret_cast<uint4*>(d + c * V) = *reinterpret_cast<const uint4*>(s + r * LD + c * V);
  }
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------

// B operand layouts for ROW mode
enum BLayout { B_NK = 0, B_KN = 1 };  // [N][K] (k-contiguous) or [K][N]

template <typename T, int BM, int BN, bool WGT, int BL, bool PAIRED, class Epi>
__global__ void __launch_bounds__(256)
grouped_gemm_kernel(GemmShape s, Operand A, Operand B, typename Epi::Params ep) {
  using G = TileGeom<T, BM, BN>;
  constexpr int SMEM = (G::MAIN_LDS > Epi::SMEM) ? G::MAIN_LDS : Epi::SMEM;
  __shared__ __attribute__((aligned(16))) char smem[SMEM];
  T* As = reinterpret_cast<T*>(smem);
  T* Bs = As + BM * G::LDK;

  TileCtx c;
  c.tid = threadIdx.x;
  c.lane = c.tid & 63;
  const int wave = c.tid >> 6;
  c.wm = wave >> 1;
  c.wn = wave & 1;

  const int NT = (s.N + BN - 1) / BN;
  int total;
  if (!WGT) {
    const int mtiles = s.tile_offsets ? s.tile_offsets[s.E] : (s.M + BM - 1) / BM;
    total = mtiles * NT;
  } else {
    total = s.E * (s.M / BM) * NT;
  }

  for (int t = xcd_virtual_id(blockIdx.x, gridDim.x); t < total; t += gridDim.x) {
    // ---- decode the tile ----
    if (!WGT) {
      const int mg = t / NT;
      c.nt = t % NT;
      if (s.tile_offsets) {
        c.e = upper_index(s.tile_offsets, s.E + 1, mg);
        c.mt = mg - s.tile_offsets[c.e];
        c.seg0 = s.offsets[c.e];
        c.segn = s.offsets[c.e + 1] - c.seg0;
      } else {
        c.e = 0; c.mt = mg; c.seg0 = 0; c.segn = s.M;
      }
      c.m_valid = min(BM, c.segn - c.mt * BM);
      c.out_row0 = (long long)c.seg0 + (long long)c.mt * BM;
    } else {
      const int MT = s.M / BM;
      c.e = t / (MT * NT);
      const int rem = t % (MT * NT);
      c.mt = rem / NT;
      c.nt = rem % NT;
      c.seg0 = s.offsets ? s.offsets[c.e] : 0;
      c.segn = s.offsets ? s.offsets[c.e + 1] - c.seg0 : s.K;
      c.m_valid = BM;
      c.out_row0 = (long long)c.e * s.M + (long long)c.mt * BM;
    }
    c.n0 = c.nt * BN;

    f32x4_v acc[G::FM][G::FN];
#pragma unroll
    for (int i = 0; i < G::FM; ++i)
#pragma unroll
      for (int j = 0; j < G::FN; ++j) acc[i][j] = f32x4_v{0.f, 0.f, 0.f, 0.f};

    if (!WGT) {
      // ---------------- ROW mode ----------------
      const T* abase = reinterpret_cast<const T*>(A.ptr);
      const T* bbase = reinterpret_cast<const T*>(B.ptr) + (long long)c.e * B.estride;
      KMajorLoad<T, BM> la;
      la.setup(c.tid, [&](int r) {
        int m = c.mt * BM + r;
        int row = c.seg0 + (m < c.segn ? m : c.segn - 1);  // rows past the end repeat the last one
        long long src = A.idx ? A.idx[row] : row;
        return abase + src * A.ld;
      });
      const int nk = s.K / G::BK;
      const int half = s.N / 2, n0p = c.nt * (BN / 2);
      if (BL == B_NK) {
        KMajorLoad<T, BN> lb;
        lb.setup(c.tid, [&](int r) {
          int col = c.n0 + r;
          if (col >= s.n_valid) col = s.n_valid - 1;
          return bbase + (long long)col * B.ld;
        });
        la.load(0);
        lb.load(0);
        for (int kt = 0; kt < nk; ++kt) {
          __syncthreads();
          la.store(As, c.tid);
          lb.store(Bs, c.tid);
          __syncthreads();
          if (kt + 1 < nk) { la.load((kt + 1) * G::BK); lb.load((kt + 1) * G::BK); }
          Mma<T, BM, BN>::step(As, Bs, acc, c.lane, c.wm, c.wn);
        }
      } else {
        MNMajorLoad<T, BN> lb;
        const int vt = (c.tid + 128) & 255;  // B blocks start where A's extra work ends
        lb.setup(vt, [&](int cc) {
          int col = PAIRED ? ColPaired::map(cc, n0p, half) : c.n0 + cc;
          return (PAIRED || col < s.n_valid) ? col : -1;
        });
        auto brow = [&](int k) -> const T* { return bbase + (long long)k * B.ld; };
        la.load(0);
        lb.load(vt, 0, brow);
        for (int kt = 0; kt < nk; ++kt) {
          __syncthreads();
          la.store(As, c.tid);
          lb.store(Bs, vt);
          __syncthreads();
          if (kt + 1 < nk) { la.load((kt + 1) * G::BK); lb.load(vt, (kt + 1) * G::BK, brow); }
          Mma<T, BM, BN>::step(As, Bs, acc, c.lane, c.wm, c.wn);
        }
      }
    } else {
      // ---------------- WGT mode ----------------
      const T* abase = reinterpret_cast<const T*>(A.ptr);
      const T* bbase = reinterpret_cast<const T*>(B.ptr);
      MNMajorLoad<T, BM> la;
      MNMajorLoad<T, BN> lb;
      const int vta = c.tid, vtb = (c.tid + 128) & 255;
      const int m0 = c.mt * BM;
      la.setup(vta, [&](int cc) { return m0 + cc; });
      lb.setup(vtb, [&](int cc) { int col = c.n0 + cc; return col < s.n_valid ? col : -1; });
      auto arow = [&](int k) -> const T* {
        if (k >= c.segn) return nullptr;
        long long src = A.idx ? A.idx[c.seg0 + k] : (long long)(c.seg0 + k);
        return abase + src * A.ld;
      };
      auto brow = [&](int k) -> const T* {
        if (k >= c.segn) return nullptr;
        long long src = B.idx ? B.idx[c.seg0 + k] : (long long)(c.seg0 + k);
        return bbase + src * B.ld;
      };
      const int nk = (c.segn + G::BK - 1) / G::BK;
      if (nk > 0) {
        la.load(vta, 0, arow);
        lb.load(vtb, 0, brow);
      }
      for (int kt = 0; kt < nk; ++kt) {
        __syncthreads();
        la.store(As, vta);
        lb.store(Bs, vtb);
        __syncthreads();
        if (kt + 1 < nk) { la.load(vta, (kt + 1) * G::BK, arow); lb.load(vtb, (kt + 1) * G::BK, brow); }
        Mma<T, BM, BN>::step(As, Bs, acc, c.lane, c.wm, c.wn);
      }
    }

    __syncthreads();  // LDS is reused by the epilogue
    Epi::run(ep, s, c, acc, smem);
    __syncthreads();  // and by the next tile's main loop
  }
}

}  // namespace moe
