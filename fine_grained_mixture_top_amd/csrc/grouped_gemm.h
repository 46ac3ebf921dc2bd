// Grouped GEMM over ragged expert segments for gfx950: one main loop (MFMA,
// LDS-staged tiles, gathered rows) and a per-kernel epilogue functor.
//
// The pages describe every MoE GEMM as a shared main loop plus a customised
// epilogue, with gathered token rows loaded inside the GEMM instead of by a
// separate gather kernel ([A] "核心创新" second point, and the "软件抽象层 QuACK"
// section).  This is the gfx950 form of that idea:
//
//  * 256 threads = 4 waves of 64 in a 2 x 2 grid; each wave owns a
//    (BM/2) x (BN/2) sub-tile of 16 x 16 MFMA fragments.  Tiles are sized so
//    that two workgroups fit on a CU (the second one hides the first one's
//    memory latency).
//  * bf16: v_mfma_f32_16x16x32_bf16 (8 bf16 of A and of B per lane);
//    fp32:  v_mfma_f32_16x16x4_f32, eight of them per 32-wide k step.
//    A and B feed each MFMA through the same (lane, element) -> k mapping, so
//    every k of the step is summed exactly once.  The accumulator of a 16 x 16
//    fragment holds column lane%16, rows 4*(lane/16)+j, j = 0..3.
//  * Operand tiles reach LDS as plain 16-byte copies of global rows, in the
//    layout they have in memory:
//      k-contiguous operands (token rows, weights read along k) as
//        [rows][BK + VEC]; fragments are one ds_read_b128 per lane;
//      m/n-contiguous operands (weights read across k in the forward, the
//        gathered rows of the weight gradients) as [BK][cols + 16]; fragments
//        come from two ds_read_b64_tr_b16 per lane, the LDS transpose read
//        (lane i of each 16-lane group receives column i of a 4 x 16 block).
//    The fp32 path has no 32-bit transpose read and transposes m/n-contiguous
//    operands in registers instead.
//  * Two LDS stages: the next k step is written while the MFMAs of the current
//    one run, one barrier per k step; global loads of step k+2 are in flight
//    meanwhile.
//  * Epilogues first park the fp32 accumulator tile in LDS, then every thread
//    processes 8-column chunks of whole rows, so the element-wise math has
//    few live registers and every global access is a coalesced 16-byte one.
//  * Persistent: the grid is sized to the machine, each workgroup walks the
//    tile list with stride gridDim.x, from an XCD-aware starting id so that
//    neighbouring tiles (same expert, same rows) share an XCD's L2.
//
// Two modes:
//  ROW mode (K1, K2, K4, K5 and the router GEMM): C rows are the routed rows of
//    an expert segment, A rows are gathered (A.idx[row]) or direct; B is the
//    expert's weight, stored [N][K] (k-contiguous) or [K][N].  Tiles are
//    (expert, m tile, n tile); each workgroup builds the prefix of m tiles per
//    expert from the segment offsets in LDS.
//  WGT mode (K7, K8, router weight gradient): C = sum over an expert's rows r
//    of A[r]^T B[r]; both operands are [rows][M] / [rows][N] with rows
//    gathered or direct; the reduction runs over the ragged segment
//    (optionally split into chunks written as separate fp32 slices).
#pragma once

#include <type_traits>
#include <utility>

#include "device_common.h"

namespace moe {

struct Operand {
  const void* ptr;     // base pointer
  const int32_t* idx;  // optional gather: segment row -> source row
  long long estride;   // elements between experts (weights); 0 otherwise
  int ld;              // elements between rows
};

// Tile plan of a weight-gradient GEMM on the 256-tile kernel.  A unit is MU
// consecutive m tiles times all n tiles of one (expert, row chunk) pair;
// units are sorted by rows, largest first, and their tiles are dealt to the
// workgroups round by round, reversing direction every round.
struct PlanUnit {
  int e;      // expert
  int seg0;   // first routed row of the chunk
  int segn;   // rows of the chunk
  int slot;   // fp32 partial slot of the chunk, -1 when the expert is not split
  int mt0;    // first m tile of the unit
  int pad[3];
};
struct WgtPlan {
  const int* nunits;      // [1] units in the plan
  const PlanUnit* units;  // [nunits], sorted
  int MU;
};

struct GemmShape {
  const int32_t* offsets;  // [E+1] row segments; null = one segment
  int E;                   // experts (1 when dense)
  int M, N, K;             // ROW: M = rows if dense; WGT: K = rows if dense
  int n_valid;             // existing columns (<= N rounded up to BN)
  int ksplit;              // WGT: chunks each expert's reduction is split into
                           //   (output slice (e*ksplit + s) holds chunk s); 1 = none
  WgtPlan plan{};          // WGT, 256-tile kernel: the tile plan
};

struct TileCtx {
  int e, mt, nt;
  int seg0, segn;      // segment of the tile's expert
  int m_valid;         // valid rows of this tile (ROW mode)
  long long out_row0;  // ROW: first routed row of the tile; WGT: slice*M + mt*BM
  int slot;            // WGT with kchunk: partial slot of the tile's chunk, -1 = stored whole
  int n0;              // first column of the tile
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

// LDS layout of one operand tile of R rows (m or n) by BK k.
template <typename T, int R, bool MN>
struct OpTile {
  static constexpr int VEC = Elem<T>::VEC, BK = Elem<T>::BK;
  static constexpr bool NAT = MN && sizeof(T) == 2;  // natural [BK][R] layout + transpose reads
  static constexpr int LD = NAT ? R + 16 : BK + VEC;  // row pitch (elements)
  static constexpr int SIZE = NAT ? BK * LD : R * LD;  // elements
};

template <typename T, int BM, int BN, bool AMN, bool BMN>
struct TileGeom {
  static constexpr int VEC = Elem<T>::VEC;
  static constexpr int BK = Elem<T>::BK;
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int FM = WM / 16, FN = WN / 16;
  using TA = OpTile<T, BM, AMN>;
  using TB = OpTile<T, BN, BMN>;
  static constexpr int STAGE = TA::SIZE + TB::SIZE;  // elements per LDS stage
  static constexpr int MAIN_LDS = 2 * STAGE * (int)sizeof(T);
  static constexpr int LDC = BN + 4;                  // fp32 staging pitch
  static constexpr int STAGE_C = BM * LDC * 4;        // bytes of the fp32 tile
  static_assert(FM >= 1 && FN >= 1, "tile too small");
};

// ---------------------------------------------------------------------------
// loaders (global -> registers -> LDS)
// ---------------------------------------------------------------------------

// R rows of BK contiguous k values; row pointers are fixed per tile.
// Thread v takes 16-byte chunk v % CPR of row v / CPR (one row per 8 lanes).
template <typename T, int R, int D>
struct KMajorLoad {
  static constexpr int VEC = Elem<T>::VEC, BK = Elem<T>::BK, LD = OpTile<T, R, false>::LD;
  static constexpr int CPR = BK / VEC;
  static constexpr int NV = R * CPR;
  static constexpr int PER = (NV + 255) / 256;
  const T* ptr[PER];
  uint4 reg[D][PER];  // D k steps in flight

  // rowptr(r) returns the source row pointer of tile row r (always valid).
  template <class F>
  __device__ __forceinline__ void setup(int tid, F rowptr) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int v = tid + p * 256;
      const int r = v / CPR, c = v % CPR;
      ptr[p] = (v < NV) ? rowptr(r < R ? r : 0) + c * VEC : nullptr;
    }
  }
  static constexpr bool FULL = NV % 256 == 0;  // every thread has PER chunks
  template <int S>
  __device__ __forceinline__ void load(int k0) {
#pragma unroll
    for (int p = 0; p < PER; ++p)
      if (FULL || ptr[p]) reg[S][p] = *reinterpret_cast<const uint4*>(ptr[p] + k0);
  }
  template <int S>
  __device__ __forceinline__ void store(T* lds, int tid) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int v = tid + p * 256;
      if (FULL || v < NV) {
        const int r = v / CPR, c = v % CPR;
        *reinterpret_cast<uint4*>(lds + r * LD + c * VEC) = reg[S][p];
      }
    }
  }
};

// BK k-rows of R contiguous columns, copied as they are into a natural
// [BK][R + 16] LDS tile (bf16).  Thread v takes 16-byte chunk v % CPR of
// k-row v / CPR.  colmap(c) gives the source column of tile column c (-1 =
// absent).  The k-rows are rows seg0 .. seg0+segn-1 of the source, gathered
// through idx when it is set; the gather indices of a stage are fetched one
// stage ahead (stages are loaded in order), so a data load never waits for
// its own index load.
template <typename T, int R, int D>
struct NatLoad {
  static constexpr int VEC = Elem<T>::VEC, BK = Elem<T>::BK, LD = OpTile<T, R, true>::LD;
  static constexpr int CPR = R / VEC;
  static constexpr int NV = BK * CPR;
  static constexpr int PER = (NV + 255) / 256;
  int col[PER];
  int nidx[PER];      // source rows of the next stage (-1 = past the segment)
  uint4 reg[D][PER];
  const T* base;
  const int32_t* idx;
  int ld, seg0, segn;

  __device__ __forceinline__ int src_row(int k) const {
    if (k >= segn) return -1;
    return idx ? idx[seg0 + k] : seg0 + k;
  }
  template <class F>
  __device__ __forceinline__ void setup(int tid, F colmap, const T* base_, const int32_t* idx_, int ld_,
                                        int seg0_, int segn_) {
    base = base_; idx = idx_; ld = ld_; seg0 = seg0_; segn = segn_;
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int v = tid + p * 256;
      col[p] = (v < NV) ? colmap((v % CPR) * VEC) : -1;
      nidx[p] = (v < NV) ? src_row(v / CPR) : -1;  // stage 0
    }
  }
  template <int S>
  __device__ __forceinline__ void load(int tid, int k0) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int v = tid + p * 256;
      const int row = (col[p] >= 0) ? nidx[p] : -1;
      reg[S][p] = row >= 0 ? *reinterpret_cast<const uint4*>(base + (long long)row * ld + col[p])
                           : make_uint4(0, 0, 0, 0);
      if (v < NV) nidx[p] = src_row(k0 + BK + v / CPR);  // next stage
    }
  }
  template <int S>
  __device__ __forceinline__ void store(T* lds, int tid) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int v = tid + p * 256;
      if (NV % 256 == 0 || v < NV) *reinterpret_cast<uint4*>(lds + (v / CPR) * LD + (v % CPR) * VEC) = reg[S][p];
    }
  }
};

// fp32 m/n-contiguous operands: 4 x 4 blocks transposed in registers into the
// k-contiguous layout.  Block b covers k block b % KB and column block b / KB.
__device__ __forceinline__ void transpose4(const uint4 (&in)[4], uint4 (&out)[4]) {
  const uint32_t* r = reinterpret_cast<const uint32_t*>(in);
  uint32_t* o = reinterpret_cast<uint32_t*>(out);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) o[i * 4 + j] = r[j * 4 + i];
}

template <int R, int D>
struct TransLoadF32 {
  static constexpr int VEC = 4, BK = Elem<float>::BK, LD = OpTile<float, R, true>::LD;
  static constexpr int KB = BK / VEC, CB = R / VEC;
  static constexpr int NB = KB * CB;
  static constexpr int PER = (NB + 255) / 256;
  int col[PER];
  uint4 reg[D][PER][VEC];
  const float* base;
  const int32_t* idx;
  int ld, seg0, segn;

  template <class F>
  __device__ __forceinline__ void setup(int tid, F colmap, const float* base_, const int32_t* idx_, int ld_,
                                        int seg0_, int segn_) {
    base = base_; idx = idx_; ld = ld_; seg0 = seg0_; segn = segn_;
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int b = tid + p * 256;
      col[p] = (b < NB) ? colmap((b / KB) * VEC) : -1;
    }
  }
  template <int S>
  __device__ __forceinline__ void load(int tid, int k0) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int b = tid + p * 256;
      const int kb = b % KB;
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        const int k = k0 + kb * VEC + j;
        const int row = (col[p] >= 0 && k < segn) ? (idx ? idx[seg0 + k] : seg0 + k) : -1;
        reg[S][p][j] = row >= 0 ? *reinterpret_cast<const uint4*>(base + (long long)row * ld + col[p])
                                : make_uint4(0, 0, 0, 0);
      }
    }
  }
  template <int S>
  __device__ __forceinline__ void store(float* lds, int tid) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int b = tid + p * 256;
      if (b < NB) {
        const int kb = b % KB, cb = b / KB;
        uint4 out[VEC];
        transpose4(reg[S][p], out);
#pragma unroll
        for (int i = 0; i < VEC; ++i)
          *reinterpret_cast<uint4*>(lds + (cb * VEC + i) * LD + kb * VEC) = out[i];
      }
    }
  }
};

// Loader for an m/n-contiguous operand of element type T.
template <typename T, int R, int D> struct MNLoadSel { using type = NatLoad<T, R, D>; };
template <int R, int D> struct MNLoadSel<float, R, D> { using type = TransLoadF32<R, D>; };
template <typename T, int R, int D> using MNLoad = typename MNLoadSel<T, R, D>::type;

// ---------------------------------------------------------------------------
// MFMA over one LDS-resident k tile
// ---------------------------------------------------------------------------

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// 8 consecutive k (ks + 8*(lane/16) .. +7) of tile row / column rc0 + lane%16.
template <typename T, int R, bool MN>
__device__ __forceinline__ bf16x8_v frag(const T* tile, int rc0, int ks, int lane) {
  using L = OpTile<T, R, MN>;
  const int q = lane & 15, g = lane >> 4;
  if constexpr (L::NAT) {
    // lane q of the group addresses k-row (q/4) of a 4-row block and column
    // chunk (q%4)*4; the transpose read hands it column q of that block
    const T* p0 = tile + (ks + 8 * g + (q >> 2)) * L::LD + rc0 + (q & 3) * 4;
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p0));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p0 + 4 * L::LD));
    const v8i16 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8_v, v);
  } else {
    return __builtin_bit_cast(bf16x8_v, *reinterpret_cast<const uint4*>(tile + (rc0 + q) * L::LD + ks + 8 * g));
  }
}

template <typename T, int BM, int BN, bool AMN, bool BMN>
struct Mma;

template <int BM, int BN, bool AMN, bool BMN>
struct Mma<bf16_t, BM, BN, AMN, BMN> {
  using G = TileGeom<bf16_t, BM, BN, AMN, BMN>;
  static constexpr int KS = G::BK / 32;  // MFMA k steps per LDS stage
  __device__ __forceinline__ static void fetch(const bf16_t* As, const bf16_t* Bs, bf16x8_v (&a)[G::FM],
                                               bf16x8_v (&b)[G::FN], int ks, int lane, int wm, int wn) {
#pragma unroll
    for (int fm = 0; fm < G::FM; ++fm) a[fm] = frag<bf16_t, BM, AMN>(As, wm * G::WM + fm * 16, ks, lane);
#pragma unroll
    for (int fn = 0; fn < G::FN; ++fn) b[fn] = frag<bf16_t, BN, BMN>(Bs, wn * G::WN + fn * 16, ks, lane);
  }
  // The fragments of k step ks+1 are read from LDS while the MFMAs of step ks run.
  __device__ __forceinline__ static void step(const bf16_t* As, const bf16_t* Bs, f32x4_v (&acc)[G::FM][G::FN],
                                              int lane, int wm, int wn) {
    bf16x8_v a[2][G::FM], b[2][G::FN];
    fetch(As, Bs, a[0], b[0], 0, lane, wm, wn);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (s + 1 < KS) fetch(As, Bs, a[(s + 1) & 1], b[(s + 1) & 1], (s + 1) * 32, lane, wm, wn);
#pragma unroll
      for (int fm = 0; fm < G::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < G::FN; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s & 1][fm], b[s & 1][fn], acc[fm][fn], 0, 0, 0);
    }
  }
};

template <int BM, int BN, bool AMN, bool BMN>
struct Mma<float, BM, BN, AMN, BMN> {
  using G = TileGeom<float, BM, BN, AMN, BMN>;
  __device__ __forceinline__ static void step(const float* As, const float* Bs, f32x4_v (&acc)[G::FM][G::FN],
                                              int lane, int wm, int wn) {
    constexpr int LDA = G::TA::LD, LDB = G::TB::LD;
    const int r16 = lane & 15, kq = (lane >> 4) * 8;
    float a[G::FM][8], b[G::FN][8];
#pragma unroll
    for (int fm = 0; fm < G::FM; ++fm) {
      const float* p = As + (wm * G::WM + fm * 16 + r16) * LDA + kq;
      *reinterpret_cast<float4*>(&a[fm][0]) = *reinterpret_cast<const float4*>(p);
      *reinterpret_cast<float4*>(&a[fm][4]) = *reinterpret_cast<const float4*>(p + 4);
    }
#pragma unroll
    for (int fn = 0; fn < G::FN; ++fn) {
      const float* p = Bs + (wn * G::WN + fn * 16 + r16) * LDB + kq;
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
// the k loop
// ---------------------------------------------------------------------------

template <int V> struct Slot { static constexpr int value = V; };

// LDS holds two stages (A tile then B tile, STAGE elements each); D register
// slots hold the global loads of the next D k steps.  Stage k lives in slot
// k % D.  The caller has already issued the loads of stage 0 into slot 0
// (for the next tile, before the current tile's epilogue, so that their
// latency hides behind it).  Top of step k: LDS[k&1] = stage k, slot
// (k+1)%D = stage k+1.  Step k: write stage k+1 to LDS[(k+1)&1], refill its
// slot with stage k+1+D, run the MFMAs of stage k, barrier.  The loop is
// unrolled D times so slot indices are compile-time constants.
template <int D, typename T, int BM, int BN, bool AMN, bool BMN, class Load, class Store>
__device__ __forceinline__ void pipeline(int nk, f32x4_v (&acc)[BM / 32][BN / 32], T* lds, const TileCtx& c,
                                         Load load, Store store) {
  using G = TileGeom<T, BM, BN, AMN, BMN>;
  auto a_of = [&](int st) { return lds + st * G::STAGE; };
  auto b_of = [&](int st) { return lds + st * G::STAGE + G::TA::SIZE; };
  if (nk <= 0) return;
  store(Slot<0>(), a_of(0), b_of(0));
  [&]<int... I>(std::integer_sequence<int, I...>) {
    ((1 + I < nk ? (load(Slot<(1 + I) % D>(), 1 + I), 0) : 0), ...);
  }(std::make_integer_sequence<int, D>{});
  __syncthreads();
  for (int k0 = 0; k0 < nk; k0 += D) {
    [&]<int... J>(std::integer_sequence<int, J...>) {
      (([&] {
         const int k = k0 + J;
         if (k < nk) {
           constexpr int nxt = (J + 1) % D;  // slot of stage k+1 (k0 is a multiple of D)
           if (k + 1 < nk) store(Slot<nxt>(), a_of((k + 1) & 1), b_of((k + 1) & 1));
           if (k + 1 + D < nk) load(Slot<nxt>(), k + 1 + D);
           Mma<T, BM, BN, AMN, BMN>::step(a_of(k & 1), b_of(k & 1), acc, c.lane, c.wm, c.wn);
           __syncthreads();
         }
       }()), ...);
    }(std::make_integer_sequence<int, D>{});
  }
}

// ---------------------------------------------------------------------------
// epilogue staging: the fp32 accumulator tile in LDS, [BM][BN + 4]
// ---------------------------------------------------------------------------

// PAIRED tiles are written un-interleaved: gate columns first (BN/2), then up.
template <int BM, int BN, bool PAIRED>
__device__ __forceinline__ void stage_acc(float* Cs, const f32x4_v (&acc)[BM / 32][BN / 32], const TileCtx& c) {
  constexpr int FM = BM / 32, FN = BN / 32, LDC = BN + 4;
#pragma unroll
  for (int fn = 0; fn < FN; ++fn) {
    const int f = c.wn * FN + fn;  // fragment column index in the tile
    int col;
    if (PAIRED) col = (f & 1) * (BN / 2) + (f >> 1) * 16 + (c.lane & 15);
    else col = f * 16 + (c.lane & 15);
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int j = 0; j < 4; ++j) Cs[(c.wm * (BM / 2) + fm * 16 + (c.lane >> 4) * 4 + j) * LDC + col] = acc[fm][fn][j];
  }
}

// 8 consecutive floats of the staged tile (a typed LDS access: lds_sync()).
__device__ __forceinline__ void ld8(const float* p, float (&v)[8]) {
  const f32x4_v a = lds_ld_f4(p), b = lds_ld_f4(p + 4);
  v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3]; v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
}

// 8 values of type TO to global memory (16 bytes for bf16, 32 for fp32).
template <typename TO>
__device__ __forceinline__ void st8(TO* p, const float (&v)[8]) {
  if constexpr (sizeof(TO) == 2) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = (uint32_t)f2bf(v[2 * i]) | ((uint32_t)f2bf(v[2 * i + 1]) << 16);
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
}

// 8 values of type T from global memory as floats.
template <typename T>
__device__ __forceinline__ void ld8g(const T* p, float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    ld8(reinterpret_cast<const float*>(p), v);
  }
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------

enum BLayout { B_NK = 0, B_KN = 1 };  // ROW-mode weight: [N][K] (k-contiguous) or [K][N]

constexpr int MAX_E = 1024;

template <typename T, int BM, int BN, bool WGT, int BL, bool PAIRED, class Epi, int PF = 1>
__global__ void __launch_bounds__(256, 2)
grouped_gemm_kernel(GemmShape s, Operand A, Operand B, typename Epi::Params ep) {
  constexpr bool AMN = WGT;
  constexpr bool BMN = WGT || BL == B_KN;
  using G = TileGeom<T, BM, BN, AMN, BMN>;
  constexpr int NEED = G::STAGE_C + Epi::SMEM;
  constexpr int SMEM = (G::MAIN_LDS > NEED) ? G::MAIN_LDS : NEED;
  __shared__ __attribute__((aligned(16))) char smem[SMEM];
  __shared__ int tprefix[WGT ? 1 : MAX_E + 1];

  TileCtx c;
  c.tid = threadIdx.x;
  c.lane = c.tid & 63;
  const int wave = c.tid >> 6;
  c.wm = wave >> 1;
  c.wn = wave & 1;

  const int NT = (s.N + BN - 1) / BN;
  int total;
  if (!WGT) {
    if (s.offsets) {
      // prefix of m tiles per expert, with this kernel's BM
      __shared__ int wsum[4];
      int carry = 0;
      for (int e0 = 0; e0 < s.E; e0 += 256) {
        const int e = e0 + c.tid;
        const int tiles = e < s.E ? (s.offsets[e + 1] - s.offsets[e] + BM - 1) / BM : 0;
        int incl = tiles;
        for (int o = 1; o < 64; o <<= 1) {
          const int y = __shfl_up(incl, o, 64);
          if (c.lane >= o) incl += y;
        }
        if (c.lane == 63) wsum[wave] = incl;
        __syncthreads();
        int base = carry, tot = 0;
        for (int w = 0; w < 4; ++w) {
          if (w < wave) base += wsum[w];
          tot += wsum[w];
        }
        if (e < s.E) tprefix[e] = base + incl - tiles;
        carry += tot;
        __syncthreads();
      }
      if (c.tid == 0) tprefix[s.E] = carry;
      __syncthreads();
      total = tprefix[s.E] * NT;
    } else {
      total = ((s.M + BM - 1) / BM) * NT;
    }
  } else {
    total = s.E * s.ksplit * (s.M / BM) * NT;
  }

  T* lds = reinterpret_cast<T*>(smem);
  float* Cs = reinterpret_cast<float*>(smem);

  // tile t -> expert, m tile, n tile and the rows it covers
  auto decode = [&](int t, TileCtx& d) {
    if (!WGT) {
      const int mg = t / NT;
      d.nt = t % NT;
      if (s.offsets) {
        d.e = upper_index(tprefix, s.E + 1, mg);
        d.mt = mg - tprefix[d.e];
        d.seg0 = s.offsets[d.e];
        d.segn = s.offsets[d.e + 1] - d.seg0;
      } else {
        d.e = 0; d.mt = mg; d.seg0 = 0; d.segn = s.M;
      }
      d.m_valid = min(BM, d.segn - d.mt * BM);
      d.out_row0 = (long long)d.seg0 + (long long)d.mt * BM;
    } else {
      const int MT = s.M / BM;
      const int es = t / (MT * NT);  // (expert, split)
      d.e = es / s.ksplit;
      const int sp = es % s.ksplit;
      const int rem = t % (MT * NT);
      d.mt = rem / NT;
      d.nt = rem % NT;
      d.seg0 = s.offsets ? s.offsets[d.e] : 0;
      d.segn = s.offsets ? s.offsets[d.e + 1] - d.seg0 : s.K;
      if (s.ksplit > 1) {  // chunk sp of the segment, a whole number of k steps
        const int steps = (d.segn + G::BK - 1) / G::BK;
        const int per = (steps + s.ksplit - 1) / s.ksplit * G::BK;
        const int lo = min(d.segn, sp * per);
        d.seg0 += lo;
        d.segn = min(d.segn, lo + per) - lo;
      }
      d.m_valid = BM;
      d.out_row0 = (long long)es * s.M + (long long)d.mt * BM;
    }
    d.n0 = d.nt * BN;
  };

  // loaders live across tiles: the next tile's first k step is fetched
  // before the current tile's epilogue
  using LA = typename std::conditional<WGT, MNLoad<T, BM, PF>, KMajorLoad<T, BM, PF>>::type;
  using LB = typename std::conditional<(!WGT && BL == B_NK), KMajorLoad<T, BN, PF>, MNLoad<T, BN, PF>>::type;
  LA la;
  LB lb;
  const T* abase = reinterpret_cast<const T*>(A.ptr);
  auto setup = [&](const TileCtx& d) {
    if constexpr (!WGT) {
      la.setup(d.tid, [&](int r) {
        const int m = d.mt * BM + r;
        const int row = d.seg0 + (m < d.segn ? m : d.segn - 1);  // rows past the end repeat the last one
        const long long src = A.idx ? A.idx[row] : row;
        return abase + src * A.ld;
      });
      const T* bbase = reinterpret_cast<const T*>(B.ptr) + (long long)d.e * B.estride;
      if constexpr (BL == B_NK) {
        lb.setup(d.tid, [&](int r) {
          int col = d.n0 + r;
          if (col >= s.n_valid) col = s.n_valid - 1;
          return bbase + (long long)col * B.ld;
        });
      } else {
        const int half = s.N / 2, n0p = d.nt * (BN / 2);
        lb.setup(d.tid, [&](int cc) {
          const int col = PAIRED ? ColPaired::map(cc, n0p, half) : d.n0 + cc;
          return (PAIRED || col < s.n_valid) ? col : -1;
        }, bbase, nullptr, B.ld, 0, s.K);
      }
    } else {
      const T* bbase = reinterpret_cast<const T*>(B.ptr);
      const int m0 = d.mt * BM;
      la.setup(d.tid, [&](int cc) { return m0 + cc; }, abase, A.idx, A.ld, d.seg0, d.segn);
      lb.setup(d.tid, [&](int cc) { const int col = d.n0 + cc; return col < s.n_valid ? col : -1; }, bbase, B.idx,
               B.ld, d.seg0, d.segn);
    }
  };
  auto load = [&](auto S, int k) {
    constexpr int SV = decltype(S)::value;
    if constexpr (!WGT && BL == B_NK) {
      la.template load<SV>(k * G::BK);
      lb.template load<SV>(k * G::BK);
    } else if constexpr (!WGT) {
      la.template load<SV>(k * G::BK);
      lb.template load<SV>(c.tid, k * G::BK);
    } else {
      la.template load<SV>(c.tid, k * G::BK);
      lb.template load<SV>(c.tid, k * G::BK);
    }
  };
  auto store = [&](auto S, T* a, T* b) {
    constexpr int SV = decltype(S)::value;
    la.template store<SV>(a, c.tid);
    lb.template store<SV>(b, c.tid);
  };
  auto ksteps = [&](const TileCtx& d) { return WGT ? (d.segn + G::BK - 1) / G::BK : s.K / G::BK; };

  int t = xcd_virtual_id(blockIdx.x, gridDim.x);
  if (t < total) {
    decode(t, c);
    setup(c);
    if (ksteps(c) > 0) load(Slot<0>(), 0);
  }
  while (t < total) {
    f32x4_v acc[G::FM][G::FN];
#pragma unroll
    for (int i = 0; i < G::FM; ++i)
#pragma unroll
      for (int j = 0; j < G::FN; ++j) acc[i][j] = f32x4_v{0.f, 0.f, 0.f, 0.f};
    pipeline<PF, T, BM, BN, AMN, BMN>(ksteps(c), acc, lds, c, load, store);

    // park the fp32 tile in LDS, fetch the next tile's first k step, then
    // run the functor's pass over the parked tile
    stage_acc<BM, BN, PAIRED>(Cs, acc, c);
    const int tn = t + gridDim.x;
    TileCtx cn = c;
    if (tn < total) {
      decode(tn, cn);
      setup(cn);
      if (ksteps(cn) > 0) load(Slot<0>(), 0);
    }
    __syncthreads();
    Epi::run(ep, s, c, Cs, smem + G::STAGE_C);
    __syncthreads();  // LDS is reused by the next tile's main loop
    c = cn;
    t = tn;
  }
}

}  // namespace moe
