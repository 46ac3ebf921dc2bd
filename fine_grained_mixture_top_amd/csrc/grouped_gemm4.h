// Large-tile grouped GEMM for bf16 on gfx950 (the MoE layer's six grouped
// GEMMs when their dimensions are multiples of 256).  Same contract as the
// kernel in grouped_gemm.h (ROW and WGT modes, gathered rows, the epilogue
// functors of epilogues.h), different machinery:
//
//  * 256 x 256 output tile, 512 threads = 8 waves in a 2 (m) x 4 (n) grid;
//    each wave owns 128 x 64 outputs as 4 x 2 blocks of
//    v_mfma_f32_32x32x16_bf16.  The MFMA's first operand is the N-side
//    fragment and its second the M-side one, so accumulator element e of a
//    block holds (m = lane % 32, n = 8*(e/4) + 4*(lane/32) + e%4): four
//    consecutive columns of one row per lane.
//  * Operand tiles go from memory straight into LDS with buffer loads that
//    write LDS (16 bytes per lane, 1 KB per instruction, no registers);
//    rows outside a segment are addressed past the buffer's record count and
//    read as zeros.  Four LDS stages of k = 32 (32 KB each): three are in
//    flight while the MFMAs of the fourth run, which covers HBM latency
//    without spending registers.
//  * Layouts (16-byte chunks XOR-swizzled so that fragment reads hit
//    distinct banks):
//      k-contiguous operands: [256 rows][32 k], 64-byte rows, chunk c of row
//        r in slot c ^ ((r >> 2) & 3); a fragment is one ds_read_b128;
//      m/n-contiguous operands: [32 k-rows][256 cols], 512-byte rows, chunk
//        c of k-row kr in slot c ^ (4 * (kr & 3)); a fragment is two
//        ds_read_b64_tr_b16 (the LDS transpose read).
//  * Epilogue: the tile is parked in LDS as fp32 in eight passes of 32 rows
//    (the four waves holding those rows write, then all 512 threads run the
//    functor on them), so the functors of the 128-row kernel apply
//    unchanged.  The staging area lies over the last stage only: before the
//    epilogue of a tile, the first three stages of the workgroup's next tile
//    are already being loaded, so that tile's start does not wait for memory.
#pragma once

#include <type_traits>

#include "epilogues.h"

namespace moe {
namespace g4 {

constexpr int BM = 256, BN = 256, BK = 32, NS = 4, NTH = 512;
constexpr int OPB = 256 * BK * 2;            // bytes of one operand tile per stage
constexpr int STAGE = 2 * OPB;               // 32 KB
constexpr int EROWS = 32;                    // epilogue rows per pass
constexpr int LDC = BN + 4;                  // fp32 staging pitch (floats)
constexpr int CS_OFF = (NS - 1) * STAGE;     // staging area: over the last stage
constexpr int STAGE_C = EROWS * LDC * 4;     // 33280 bytes
constexpr int WAVE_LDS = 7168;              // private epilogue area per wave
constexpr int WE_OFF = (NS - 1) * STAGE;     // wave areas: over the last stage and above
constexpr int SMEM_PASS = NS * STAGE > CS_OFF + STAGE_C ? NS * STAGE : CS_OFF + STAGE_C;
constexpr int SMEM_WAVE = NS * STAGE > WE_OFF + 8 * WAVE_LDS ? NS * STAGE : WE_OFF + 8 * WAVE_LDS;
constexpr int SMEM = SMEM_PASS > SMEM_WAVE ? SMEM_PASS : SMEM_WAVE;
constexpr uint32_t OOB = 0x80000000u;        // byte offset past every record count
constexpr int LPS = 4;                       // 16-byte loads per thread per stage

typedef __attribute__((address_space(3))) void lds_void_t;
typedef float f32x16_v __attribute__((ext_vector_type(16)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, voff, 0, 0, 0);
}

__device__ __forceinline__ int swz_kc(int r) { return (r >> 2) & 3; }
__device__ __forceinline__ int swz_mn(int kr) { return 4 * (kr & 3); }

// s_waitcnt with vmcnt(n) only (expcnt and lgkmcnt at their maximum).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// ---------------------------------------------------------------------------
// operand loaders: each wave issues two 1 KB instructions per operand per stage
// ---------------------------------------------------------------------------

// k-contiguous rows.  Instruction i of wave w covers tile rows
// (2w + i) * 16 .. +15; lane l takes row rb + l/4, slot l%4.
struct KCLoad {
  uint32_t off[2];  // byte offset of this lane's chunk at k = 0 (OOB when absent)
  template <class F>
  __device__ __forceinline__ void setup(int w, int lane, F rowoff) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = (2 * w + i) * 16 + (lane >> 2);
      const uint32_t ro = rowoff(r);
      off[i] = ro == OOB ? OOB : ro + (uint32_t)(((lane & 3) ^ swz_kc(r)) * 16);
    }
  }
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, char* op, int w, int k0) const {
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16(rs, op + (2 * w + i) * 1024, off[i] + (uint32_t)k0 * 2u);
  }
};

// m/n-contiguous rows (k-rows of 256 columns).  Instruction i of wave w
// covers k-rows (2w + i) * 2 and +1 (lanes 0..31 and 32..63), slot l % 32.
// The column part of the offset is fixed per tile; the row part is either
// (k0 + kr) * ld (weights) or idx[seg0 + k0 + kr] * ld (segment rows).
// Gathered segment rows take their indices from registers for a tile's
// first NS - 1 stages (loaded with the tile's setup) and from an LDS ring
// after that: while stage k's data loads are issued, one wave loads stage
// k + 1's 32 indices into the ring with a buffer -> LDS load, which the
// kernel's wait for stage k - 1 covers.  (An index loaded into a register
// one stage ahead makes the wave wait for it, and so for every load issued
// before it, as soon as the offset is formed.)
constexpr int IRING = 64;  // ints per ring slot: one 64-lane buffer -> LDS load of 4 bytes
// G: the rows are gathered through an index (fixed per launch)
template <bool G>
struct MNLoad4 {
  uint32_t coff[2];   // column byte offset of this lane's chunk (OOB if absent)
  int kr[2];          // k-row of each instruction within the stage
  // segment rows
  const int32_t* idx;
  int seg0, segn;
  uint32_t ldb;       // row pitch in bytes
  uint32_t rcur[2];   // row byte offsets of the stage being issued (OOB past the segment)
  int ip0[2], ip1[2], ip2[2];     // gathered: source rows of stages 0 .. NS-2 (-1 past the segment)
  __amdgpu_buffer_rsrc_t ridx;    // gathered: the segment's indices (records up to its end)

  template <class F>
  __device__ __forceinline__ void setup_cols(int w, int lane, F colmap) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      kr[i] = (2 * w + i) * 2 + (lane >> 5);
      const int chunk = (lane & 31) ^ swz_mn(kr[i]);
      const int col = colmap(chunk * 8);
      coff[i] = col < 0 ? OOB : (uint32_t)col * 2u;
    }
  }
  __device__ __forceinline__ void setup_rows(const int32_t* idx_, int seg0_, int segn_, uint32_t ldb_) {
    idx = idx_; seg0 = seg0_; segn = segn_; ldb = ldb_;
    if constexpr (G) {
      ridx = make_rsrc(idx_, (uint32_t)(seg0_ + segn_) * 4u);
      static_assert(NS == 4, "three register stages");
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        ip0[i] = kr[i] < segn ? idx[seg0 + kr[i]] : -1;
        ip1[i] = BK + kr[i] < segn ? idx[seg0 + BK + kr[i]] : -1;
        ip2[i] = 2 * BK + kr[i] < segn ? idx[seg0 + 2 * BK + kr[i]] : -1;
      }
    }
  }
  // weights: k-row kr of stage k0 sits at (k0 + kr) * ldb
  __device__ __forceinline__ void issue_w(__amdgpu_buffer_rsrc_t rs, char* op, int w, int k0) const {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t o = coff[i] == OOB ? OOB : coff[i] + (uint32_t)(k0 + kr[i]) * ldb;
      dma16(rs, op + (2 * w + i) * 1024, o);
    }
  }
  // segment rows of stage k < NS - 1 (a tile's first stages): gathered ones
  // from the registers
  __device__ __forceinline__ void rows_pre(int k) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int kk = k * BK + kr[i];
      int src;
      if constexpr (G) src = k == 0 ? ip0[i] : (k == 1 ? ip1[i] : ip2[i]);
      else src = kk < segn ? seg0 + kk : -1;
      rcur[i] = src < 0 ? OOB : (uint32_t)src * ldb;
    }
  }
  // segment rows of stage k >= NS - 1: gathered ones from the ring
  __device__ __forceinline__ void rows_ring(int k, const int* ring) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int kk = k * BK + kr[i];
      int src;
      if constexpr (G) src = kk < segn ? ring[(k % NS) * IRING + kr[i]] : -1;
      else src = kk < segn ? seg0 + kk : -1;
      rcur[i] = src < 0 ? OOB : (uint32_t)src * ldb;
    }
  }
  // gathered: indices of stage k into its ring slot (lanes 0..31: k-rows
  // 0..31; the other lanes and rows past the segment read nothing and write 0)
  __device__ __forceinline__ void idx_dma(char* ring, int k, int lane) const {
    const int kk = k * BK + (lane & 31);
    const uint32_t o = (lane < 32 && kk < segn) ? (uint32_t)(seg0 + kk) * 4u : OOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ridx, (lds_void_t*)(ring + (k % NS) * IRING * 4), 4, o, 0, 0, 0);
  }
  __device__ __forceinline__ void dma(__amdgpu_buffer_rsrc_t rs, char* op, int w) const {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t o = (coff[i] == OOB || rcur[i] == OOB) ? OOB : rcur[i] + coff[i];
      dma16(rs, op + (2 * w + i) * 1024, o);
    }
  }
};

// ---------------------------------------------------------------------------
// fragments (32 rows / columns by 8 consecutive k per lane)
// ---------------------------------------------------------------------------

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef short v8i16_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

// k-contiguous tile: row rb + lane%32, k = 16s + 8*(lane/32) .. +7
__device__ __forceinline__ bf16x8_v frag_kc(const char* op, int rb, int s, int lane) {
  const int r = rb + (lane & 31);
  const int c = 2 * s + (lane >> 5);
  return *reinterpret_cast<const bf16x8_v*>(op + r * 64 + ((c ^ swz_kc(r)) * 16));
}

// LDS transpose read.  Through a restrict-qualified pointer the read carries
// alias-scope information; without any, the compiler makes it wait for every
// buffer -> LDS load in flight (vmcnt(0)), the stages being loaded behind it
// included (see lds_sync() in device_common.h).
__device__ __forceinline__ v4i16_t ds_tr16(const lds_v4i16_t* __restrict__ p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<lds_v4i16_t*>(p));
}

// m/n-contiguous tile: column cb + lane%32, k = 16s + 8*(lane/32) .. +7.
// Lane q of each 16-lane group addresses k-row (q/4) of a 4 x 16 block and
// column chunk (q%4)*4; the transpose read hands it column q of the block.
__device__ __forceinline__ bf16x8_v frag_mn(const char* op, int cb, int s, int lane) {
  const int q = lane & 15, g = lane >> 4;
  const int col = cb + 16 * (g & 1) + (q & 3) * 4;
  const int k0 = 16 * s + 8 * (g >> 1) + (q >> 2);
  auto addr = [&](int kr) { return op + kr * 512 + ((((col >> 3) ^ swz_mn(kr)) * 16) + (col & 7) * 2); };
  const v4i16_t lo = ds_tr16((const lds_v4i16_t*)addr(k0));
  const v4i16_t hi = ds_tr16((const lds_v4i16_t*)addr(k0 + 4));
  return __builtin_bit_cast(bf16x8_v, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <bool MN>
__device__ __forceinline__ bf16x8_v frag(const char* op, int base, int s, int lane) {
  if constexpr (MN) return frag_mn(op, base, s, lane);
  else return frag_kc(op, base, s, lane);
}

template <bool AMN, bool BMN>
struct Frags {
  bf16x8_v m[4], n[2];
  __device__ __forceinline__ void read(const char* st, int s, int lane, int wm, int wn) {
#pragma unroll
    for (int j = 0; j < 4; ++j) m[j] = frag<AMN>(st, wm * 128 + 32 * j, s, lane);
#pragma unroll
    for (int i = 0; i < 2; ++i) n[i] = frag<BMN>(st + OPB, wn * 64 + 32 * i, s, lane);
  }
};

template <bool AMN, bool BMN>
__device__ __forceinline__ void mma(f32x16_v (&acc)[2][4], const Frags<AMN, BMN>& f) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.n[i], f.m[j], acc[i][j], 0, 0, 0);
}

// ---------------------------------------------------------------------------
// wave-local epilogues: each wave converts its own 128 x 64 block, 32 rows at a
// time, stages it as bf16 in a private LDS area and stores whole row segments;
// no workgroup barrier.  (Epilogues that need whole rows, such as the dH one,
// use the workgroup-wide passes instead.)
// ---------------------------------------------------------------------------

template <class E, class = void> struct is_wave_epi : std::false_type {};
template <class E> struct is_wave_epi<E, std::void_t<decltype(E::WAVE)>> : std::bool_constant<E::WAVE> {};

// A wave epilogue may stage per-tile operands in LDS: PRE_BYTES per tile, in
// two slots that alternate between consecutive tiles of a workgroup.
// pre_issue (all waves) issues buffer -> LDS loads into the tile's slot just
// before the tile's first stage, so the kernel's wait for that stage covers
// them, and the data are in LDS long before the epilogue reads them; run
// then takes the slot as a fifth argument.
template <class E, class = void> struct pre_bytes : std::integral_constant<int, 0> {};
template <class E>
struct pre_bytes<E, std::void_t<decltype(E::PRE_BYTES)>> : std::integral_constant<int, E::PRE_BYTES> {};

// 16-byte store of an output that is read again only by a later kernel:
// non-temporal, so it does not push operand lines out of the L2
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void st_out(void* p, uint4 x) {
  const u32x4_t v = {x.x, x.y, x.z, x.w};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
}

__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d) {
  return make_uint2(f2bf2(a, b), f2bf2(c, d));
}

// C[row, n0 + col] = acc as bf16.
struct G4Store {
  static constexpr bool WAVE = true;
  struct Params {
    bf16_t* C;
    long long ldc;
  };
  __device__ __forceinline__ static void run(const Params& p, const TileCtx& c, const f32x16_v (&acc)[2][4],
                                             char* area) {
    constexpr int LD = 72;  // [32][64 + 8] bf16
    bf16_t* L = reinterpret_cast<bf16_t*>(area);
    const int cl = c.lane & 31, hl = c.lane >> 5;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rb = c.wm * 128 + 32 * j;  // tile row of the block's first row
      if (rb >= c.m_valid) break;          // uniform over the wave
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int eg = 0; eg < 4; ++eg)
          lds_st8(L + cl * LD + 32 * i + 8 * eg + 4 * hl,
                  pack4(acc[i][j][4 * eg], acc[i][j][4 * eg + 1], acc[i][j][4 * eg + 2], acc[i][j][4 * eg + 3]));
      // rows r = lane / 8 + 8 q, chunks ch = lane % 8; a block with every
      // row valid (all but an expert's last) reads its four chunks first, so
      // its stores wait for LDS once
      bf16_t* out = p.C + (c.out_row0 + rb) * p.ldc + c.n0 + c.wn * 64 + (c.lane & 7) * 8;
      if (rb + 32 <= c.m_valid) {
        uint4 x[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) x[q] = lds_ld16(L + ((c.lane >> 3) + 8 * q) * LD + (c.lane & 7) * 8);
#pragma unroll
        for (int q = 0; q < 4; ++q) st_out(out + ((c.lane >> 3) + 8 * q) * p.ldc, x[q]);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = (c.lane >> 3) + 8 * q;
          const uint4 x = lds_ld16(L + r * LD + (c.lane & 7) * 8);
          if (rb + r < c.m_valid) st_out(out + r * p.ldc, x);
        }
      }
    }
  }
};

// Input-gradient rows with the router term: C[row, col] = acc + dz[row] *
// v[e, col] as bf16, dz the row's score gradient (fp32, one per routed row)
// and v the expert's row of the transposed router weights ([E][ldc] bf16).
// The tile's 256 dz values and 256 v columns are staged in LDS with the
// tile's first loads (rows past the buffer read as zero), and the rank-1
// term starts the accumulators: one 32 x 32 x 16 bf16 MFMA per block, k = 0
// and 1 carrying v against dz split into bf16 hi + lo parts (dz to about
// 2^-17 relative), the other k zero.  In the MFMA pipe it costs 8 of the
// tile's hundreds of MFMAs, where a per-element multiply-add in the epilogue
// would stall the wave after its last MFMA.
struct G4StoreRouter {
  static constexpr bool WAVE = true;
  static constexpr bool INIT = true;
  static constexpr int PRE_BYTES = 256 * 4 + 256 * 2;
  struct Params {
    bf16_t* C;
    long long ldc;
    const float* dz;
    const bf16_t* v;
    uint32_t dz_bytes, v_bytes;
  };
  __device__ __forceinline__ static void pre_issue(const Params& p, const TileCtx& c, char* slot, int w, int lane) {
    if (w < 4) {
      const __amdgpu_buffer_rsrc_t r = make_rsrc(p.dz, p.dz_bytes);
      const uint32_t o = ((uint32_t)c.out_row0 + (uint32_t)(64 * w + lane)) * 4u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(slot + 256 * w), 4, o, 0, 0, 0);
    } else if (w < 6) {
      const __amdgpu_buffer_rsrc_t r = make_rsrc(p.v, p.v_bytes);
      const uint32_t o = ((uint32_t)c.e * (uint32_t)p.ldc + (uint32_t)c.n0) * 2u + (uint32_t)(256 * (w - 4) + 4 * lane);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(slot + 1024 + 256 * (w - 4)), 4, o, 0, 0, 0);
    }
  }
  // accumulators = dz (x) v over the wave's 128 x 64 block; the slot's data
  // must be visible (after the kernel's wait for the tile's first stage)
  __device__ __forceinline__ static void init(const Params&, const TileCtx& c, f32x16_v (&acc)[2][4],
                                              const char* slot) {
    const int l32 = c.lane & 31;
    const bool k01 = c.lane < 32;  // lanes holding k = 0..7
    const float* zs = reinterpret_cast<const float*>(slot);
    const bf16_t* vs = reinterpret_cast<const bf16_t*>(slot + 1024);
    bf16x8_v nf[2], mf[4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint16_t v = k01 ? vs[c.wn * 64 + 32 * i + l32] : (uint16_t)0;
      v8i16_t x = {(short)v, (short)v, 0, 0, 0, 0, 0, 0};
      nf[i] = __builtin_bit_cast(bf16x8_v, x);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float z = k01 ? zs[c.wm * 128 + 32 * j + l32] : 0.f;
      const uint16_t hi = f2bf(z);
      const uint16_t lo = f2bf(z - __uint_as_float((uint32_t)hi << 16));
      v8i16_t x = {(short)hi, (short)lo, 0, 0, 0, 0, 0, 0};
      mf[j] = __builtin_bit_cast(bf16x8_v, x);
    }
    f32x16_v zero;
#pragma unroll
    for (int e = 0; e < 16; ++e) zero[e] = 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(nf[i], mf[j], zero, 0, 0, 0);
  }
  __device__ __forceinline__ static void run(const Params& p, const TileCtx& c, const f32x16_v (&acc)[2][4],
                                             char* area, const char*) {
    G4Store::run(G4Store::Params{p.C, p.ldc}, c, acc, area);
  }
};

// Epilogues whose init hook starts the accumulators (else they start at zero)
template <class E, class = void> struct has_init : std::false_type {};
template <class E> struct has_init<E, std::void_t<decltype(E::INIT)>> : std::bool_constant<E::INIT> {};

// Weight-gradient store: tiles of an expert stored whole go to C as bf16
// (G4Store); tiles of one chunk of a split expert write their fp32 partial
// sums to slot c.slot of P ([slots][M][ldc]), summed later in chunk order.
struct G4StoreW {
  static constexpr bool WAVE = true;
  struct Params {
    bf16_t* C;
    long long ldc;
    float* P;
  };
  __device__ __forceinline__ static void run(const Params& p, const TileCtx& c, const f32x16_v (&acc)[2][4],
                                             char* area) {
    if (c.slot < 0) {
      G4Store::run(G4Store::Params{p.C, p.ldc}, c, acc, area);
      return;
    }
    const int cl = c.lane & 31, hl = c.lane >> 5;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float* row = p.P + (c.out_row0 + c.wm * 128 + 32 * j + cl) * p.ldc + c.n0 + c.wn * 64 + 4 * hl;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int eg = 0; eg < 4; ++eg)
          *reinterpret_cast<float4*>(row + 32 * i + 8 * eg) =
              make_float4(acc[i][j][4 * eg], acc[i][j][4 * eg + 1], acc[i][j][4 * eg + 2], acc[i][j][4 * eg + 3]);
    }
  }
};

// Up-projection: the B tile's columns are arranged so that wave wn holds the
// gate columns j0 + 32 wn .. +31 in its first 32 columns and the matching up
// columns in its last 32 (j0 = 128 * nt), so gate and up of one element sit in
// the same lane.  H is rounded to bf16 first and A = silu(G) * U is formed
// from the rounded values (the backward recomputes A from the cached H).
struct G4SwiGLU {
  static constexpr bool WAVE = true;
  struct Params {
    bf16_t* H;  // [rows, 2n]
    bf16_t* A;  // [rows, n]
    int n;
  };
  // tile column of the B tile (chunk-aligned) -> global column of W1
  __device__ __forceinline__ static int col(int cc, int nt, int n) {
    const int wv = cc >> 6, cw = cc & 63;
    const int j = nt * 128 + wv * 32 + (cw & 31);
    return cw < 32 ? j : n + j;
  }
  __device__ __forceinline__ static void run(const Params& p, const TileCtx& c, const f32x16_v (&acc)[2][4],
                                             char* area) {
    constexpr int LH = 72, LA = 40;  // H block [32][32 gate + 32 up + 8], A block [32][32 + 8]
    bf16_t* Lh = reinterpret_cast<bf16_t*>(area);
    bf16_t* La = Lh + 32 * LH;
    const int cl = c.lane & 31, hl = c.lane >> 5;
    const int j0 = c.nt * 128 + c.wn * 32;
    const long long ldh = 2LL * p.n;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rb = c.wm * 128 + 32 * j;
      if (rb >= c.m_valid) break;
#pragma unroll
      for (int eg = 0; eg < 4; ++eg) {
        // H rounded to bf16 once (packed pairs); A from the rounded values
        const uint2 hg = pack4(acc[0][j][4 * eg], acc[0][j][4 * eg + 1], acc[0][j][4 * eg + 2], acc[0][j][4 * eg + 3]);
        const uint2 hu = pack4(acc[1][j][4 * eg], acc[1][j][4 * eg + 1], acc[1][j][4 * eg + 2], acc[1][j][4 * eg + 3]);
        const float g[4] = {__uint_as_float(hg.x << 16), __uint_as_float(hg.x & 0xffff0000u),
                            __uint_as_float(hg.y << 16), __uint_as_float(hg.y & 0xffff0000u)};
        const float u[4] = {__uint_as_float(hu.x << 16), __uint_as_float(hu.x & 0xffff0000u),
                            __uint_as_float(hu.y << 16), __uint_as_float(hu.y & 0xffff0000u)};
        float a[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) a[e] = g[e] * sigmoidf_(g[e]) * u[e];
        const int cc = 8 * eg + 4 * hl;
        lds_st8(Lh + cl * LH + cc, hg);
        lds_st8(Lh + cl * LH + 32 + cc, hu);
        lds_st8(La + cl * LA + cc, pack4(a[0], a[1], a[2], a[3]));
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {  // H: 32 rows x (4 gate + 4 up) chunks
        const int v = c.lane + 64 * q, r = v >> 3, ch = v & 7;
        const uint4 x = lds_ld16(Lh + r * LH + ch * 8);
        const int gc = ch < 4 ? j0 + ch * 8 : p.n + j0 + (ch - 4) * 8;
        if (rb + r < c.m_valid) st_out(p.H + (c.out_row0 + rb + r) * ldh + gc, x);
      }
#pragma unroll
      for (int q = 0; q < 2; ++q) {  // A: 32 rows x 4 chunks
        const int v = c.lane + 64 * q, r = v >> 2, ch = v & 3;
        const uint4 x = lds_ld16(La + r * LA + ch * 8);
        if (rb + r < c.m_valid)
          *reinterpret_cast<uint4*>(p.A + (c.out_row0 + rb + r) * (long long)p.n + j0 + ch * 8) = x;  // read next by K2
      }
    }
  }
};

#define G4_SCHED(mask, n) __builtin_amdgcn_sched_group_barrier(mask, n, 0)

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------

// WGT: weight-gradient mode (both operands m/n-contiguous segment rows);
// otherwise ROW mode with A k-contiguous and B [N][K] (BMN = false) or [K][N]
// (BMN = true).  PAIRED: B columns arranged for G4SwiGLU (gate and up of the
// same j in the same wave).
// GATH (weight gradients): bit 0 = A rows gathered through A.idx, bit 1 =
// B rows through B.idx (A.idx / B.idx non-null exactly then)
template <bool WGT, bool BMN, bool PAIRED, class Epi, int GATH = 0>
__global__ void __launch_bounds__(NTH, 1)
grouped_gemm4_kernel(GemmShape s, Operand A, Operand B, uint32_t a_bytes, uint32_t b_bytes,
                     typename Epi::Params ep) {
  constexpr bool AMN = WGT;
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  // ROW: tprefix[e] = row tiles of experts before e; workgroup v takes tiles
  // v, v + G, v + 2G, ...  WGT: tiles of the plan's sorted units; in round r
  // workgroup v takes tile r*G + v (r even) or r*G + G-1-v (r odd), which
  // spreads the large units' tiles evenly over the workgroups.  v is the
  // XCD-grouped id, so consecutive tiles share an XCD's L2 either way.
  __shared__ int tprefix[WGT ? 1 : MAX_E + 1];
  // row mode: the workgroup's next tile, looked up by wave 0 at the start
  // of the current tile (its expert and row tile written to nxe, the
  // expert's two row offsets loaded into nxt[0..1] by a buffer -> LDS load,
  // the other lanes writing 0) and read by every wave once the tile is done,
  // so that moving to the next tile waits for no LDS search and no global
  // load.  Two slots by tile parity: no barrier separates the reads of one
  // slot from wave 0's next write to the other.  (The barriers are
  // lds_sync(): a __syncthreads() would make every wave wait for that load,
  // and so for every stage in flight.)
  __shared__ int nxe[2][2];
  __shared__ __attribute__((aligned(256))) int nxt[2][WGT ? 1 : 64];
  // weight gradients: index rings of the gathered A / B rows (see MNLoad4)
  constexpr bool GA = WGT && (GATH & 1), GB = WGT && (GATH & 2);
  __shared__ __attribute__((aligned(256))) int iring[2][GA || GB ? NS * IRING : 1];
  constexpr int PREB = pre_bytes<Epi>::value;
  __shared__ __attribute__((aligned(256))) char pre_lds[PREB > 0 ? 2 * PREB : 16];  // wave epilogues' tile operands

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w >> 2, wn = w & 3;

  const int NT = s.N / BN;
  const int UT = WGT ? s.plan.MU * NT : 1;  // tiles per plan unit
  int total;
  if constexpr (!WGT) {
    __shared__ int wsum[8];
    int carry = 0;
    for (int e0 = 0; e0 < s.E; e0 += NTH) {
      const int e = e0 + tid;
      const int tiles = e < s.E ? (s.offsets[e + 1] - s.offsets[e] + BM - 1) / BM : 0;
      int incl = tiles;
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
      }
      if (lane == 63) wsum[w] = incl;
      __syncthreads();
      int base = carry, tot = 0;
      for (int x = 0; x < NTH / 64; ++x) {
        if (x < w) base += wsum[x];
        tot += wsum[x];
      }
      if (e < s.E) tprefix[e] = base + incl - tiles;
      carry += tot;
      __syncthreads();
    }
    if (tid == 0) tprefix[s.E] = carry;
    __syncthreads();
    total = tprefix[s.E] * NT;
  } else {
    total = __builtin_amdgcn_readfirstlane(s.plan.nunits[0]) * UT;
  }
  const int G = gridDim.x;
  // the tile loop's barriers: lds_sync() in row mode (see nxe / nxt above);
  // __syncthreads() for the weight gradients, measured 2-4% faster there
  auto tile_sync = [&]() {
    if constexpr (WGT) __syncthreads();
    else lds_sync();
  };
  const int vid = xcd_virtual_id(blockIdx.x, G);
  // tile of round r, -1 past the end
  auto tile_of = [&](int r) -> int {
    int t;
    if constexpr (WGT) t = r * G + ((r & 1) ? G - 1 - vid : vid);
    else t = r * G + vid;
    return t < total ? t : -1;
  };

  float* Cs = reinterpret_cast<float*>(smem + CS_OFF);
  const char* abase = reinterpret_cast<const char*>(A.ptr);
  const char* bbase = reinterpret_cast<const char*>(B.ptr);

  // tile t -> expert, m tile, n tile, rows
  // wave 0 (row mode): look up tile t, the workgroup's tile of round q,
  // into slot q & 1 of nxe / nxt (see above)
  auto lookup_next = [&](int t, int q) {
    if (w != 0 || t < 0) return;
    const int mg = t / NT;
    const int e = upper_index(tprefix, s.E + 1, mg);
    if (lane == 0) {
      nxe[q & 1][0] = e;
      nxe[q & 1][1] = mg - tprefix[e];
    }
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(s.offsets, (uint32_t)(s.E + 1) * 4u);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ro, (lds_void_t*)nxt[q & 1], 4,
                                             lane < 2 ? (uint32_t)(e + lane) * 4u : OOB, 0, 0, 0);
  };
  // pre (row mode): from slot q & 1 of nxe / nxt, the tile of round q
  auto decode = [&](int t, TileCtx& c, bool pre = false, int q = 0) {
    c.tid = tid; c.lane = lane; c.wm = wm; c.wn = wn;
    if constexpr (!WGT) {
      const int mg = t / NT;
      c.nt = t % NT;
      if (pre) {
        c.e = nxe[q & 1][0];
        c.mt = nxe[q & 1][1];
        c.seg0 = nxt[q & 1][0];
        c.segn = nxt[q & 1][1] - c.seg0;
      } else {
        c.e = upper_index(tprefix, s.E + 1, mg);
        c.mt = mg - tprefix[c.e];
        c.seg0 = s.offsets[c.e];
        c.segn = s.offsets[c.e + 1] - c.seg0;
      }
      c.m_valid = min(BM, c.segn - c.mt * BM);
      c.out_row0 = (long long)c.seg0 + (long long)c.mt * BM;
      c.slot = -1;
    } else {
      const int4* u = reinterpret_cast<const int4*>(s.plan.units + t / UT);
      const int4 u0 = u[0], u1 = u[1];
      const int ti = t % UT;
      c.e = u0.x;
      c.seg0 = u0.y;
      c.segn = u0.z;
      c.slot = u0.w;
      c.mt = u1.x + ti / NT;
      c.nt = ti % NT;
      c.m_valid = BM;
      c.out_row0 = (long long)(c.slot >= 0 ? c.slot : c.e) * s.M + (long long)c.mt * BM;
    }
    c.n0 = c.nt * BN;
  };
  auto ksteps = [&](const TileCtx& c) { return WGT ? (c.segn + BK - 1) / BK : s.K / BK; };

  // operand loaders (state of the tile whose loads are being issued)
  __amdgpu_buffer_rsrc_t ra, rb;
  KCLoad la_kc, lb_kc;
  MNLoad4<GA> la_mn;
  MNLoad4<GB> lb_mn;
  // (A row touch for the weight gradients, wave 7 reading 4 bytes of some
  // of a later stage's lines of the operand a plan unit's tiles share, was
  // measured faster while the compiler drained every stage in flight; with
  // the pipeline intact it cost 2-5% (dW1 0.398 -> 0.413 ms, dW2 0.217 ->
  // 0.225 at T = 32768, d = 1536, E = 128, n = 256) and is gone.)
  auto setup = [&](const TileCtx& c) {
    if constexpr (!WGT) {
      ra = make_rsrc(abase, a_bytes);
      la_kc.setup(w, lane, [&](int r) -> uint32_t {
        const int m = c.mt * BM + r;
        const int row = c.seg0 + (m < c.segn ? m : c.segn - 1);  // rows past the end repeat the last one
        const uint32_t src = A.idx ? (uint32_t)A.idx[row] : (uint32_t)row;
        return src * (uint32_t)A.ld * 2u;
      });
      const char* be = bbase + (long long)c.e * B.estride * 2;
      rb = make_rsrc(be, b_bytes);
      if constexpr (!BMN) {
        lb_kc.setup(w, lane, [&](int r) -> uint32_t { return (uint32_t)(c.n0 + r) * (uint32_t)B.ld * 2u; });
      } else {
        lb_mn.setup_cols(w, lane, [&](int cc) {
          if constexpr (PAIRED) return G4SwiGLU::col(cc, c.nt, s.N / 2);
          return c.n0 + cc;
        });
        lb_mn.ldb = (uint32_t)B.ld * 2u;
      }
    } else {
      ra = make_rsrc(abase, a_bytes);
      rb = make_rsrc(bbase, b_bytes);
      const int m0 = c.mt * BM;
      la_mn.setup_cols(w, lane, [&](int cc) { return m0 + cc; });
      lb_mn.setup_cols(w, lane, [&](int cc) { return c.n0 + cc; });
      la_mn.setup_rows(A.idx, c.seg0, c.segn, (uint32_t)A.ld * 2u);
      lb_mn.setup_rows(B.idx, c.seg0, c.segn, (uint32_t)B.ld * 2u);
    }
  };
  // PRE: one of a tile's first NS - 1 stages (issued by prime)
  auto issue = [&](int k, auto PRE) {
    char* st = smem + (k % NS) * STAGE;
    const int k0 = k * BK;
    if constexpr (!WGT) {
      la_kc.issue(ra, st, w, k0);
      if constexpr (!BMN) lb_kc.issue(rb, st + OPB, w, k0);
      else lb_mn.issue_w(rb, st + OPB, w, k0);
    } else {
      // stage k's rows (from the ring from stage NS - 1 on, read before the
      // ring's next load is issued), then wave 6 loads the indices of stage
      // k + 1 of each gathered operand into the ring ahead of its data loads
      // of stage k
      if constexpr (decltype(PRE)::value) {
        la_mn.rows_pre(k);
        lb_mn.rows_pre(k);
      } else {
        la_mn.rows_ring(k, iring[0]);
        lb_mn.rows_ring(k, iring[1]);
      }
      if ((GA || GB) && w == 6 && k + 1 >= NS - 1 && (k + 1) * BK < la_mn.segn) {
        if constexpr (GA) la_mn.idx_dma(reinterpret_cast<char*>(iring[0]), k + 1, lane);
        if constexpr (GB) lb_mn.idx_dma(reinterpret_cast<char*>(iring[1]), k + 1, lane);
      }
      la_mn.dma(ra, st, w);
      lb_mn.dma(rb, st + OPB, w);
    }
  };
  // first stages of a tile (stages 0 .. NS-2, fewer for short reductions)
  auto prime = [&](const TileCtx& c) {
    const int nk = ksteps(c);
    for (int k = 0; k < NS - 1 && k < nk; ++k) issue(k, std::true_type());
  };

  int r = 0;
  int t = tile_of(0);
  TileCtx c;
  if (t >= 0) {
    decode(t, c);
    setup(c);
    if constexpr (PREB > 0) Epi::pre_issue(ep, c, pre_lds, w, lane);
    prime(c);
  }
  while (t >= 0) {
    const int nk = ksteps(c);
    f32x16_v acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    if constexpr (!WGT) lookup_next(tile_of(r + 1), r + 1);
    if (nk > 0) {
      // stage 0 complete: at least LPS data loads were issued after it by
      // every later stage of this tile and, for tiles after the first, the
      // previous epilogue's stores came after those (they only add to it)
      static_assert(NS == 4, "the waits below assume three stages in flight");
      if (nk >= 3) wait_vm<2 * LPS>();
      else if (nk == 2) wait_vm<LPS>();
      else wait_vm<0>();
      tile_sync();
      if constexpr (has_init<Epi>::value) Epi::init(ep, c, acc, pre_lds + (r & 1) * PREB);
      Frags<AMN, BMN> f0, f1;
      f0.read(smem, 0, lane, wm, wn);
      // one k step: MFMAs of sub-step 0 while sub-step 1's fragments load,
      // barrier (stage k+1 landed, stage k-1's buffer free), next stage's
      // loads, MFMAs of sub-step 1 while the next stage's first fragments load
      auto body = [&](int k, auto MAIN) {
        const char* cur = smem + (k % NS) * STAGE;
        f1.read(cur, 1, lane, wm, wn);
        mma(acc, f0);
#pragma unroll
        for (int i = 0; i < 6; ++i) { G4_SCHED(0x008, 1); G4_SCHED(0x100, 1); }
        G4_SCHED(0x008, 2);
        if constexpr (decltype(MAIN)::value) {
          // stage k+1 complete: at least the LPS data loads of stage k+2
          // were issued after its last load (other loads only add to that)
          wait_vm<LPS>();
        } else {
          wait_vm<0>();
        }
        tile_sync();
        if constexpr (decltype(MAIN)::value) issue(k + NS - 1, std::false_type());
        if (k + 1 < nk) f0.read(smem + ((k + 1) % NS) * STAGE, 0, lane, wm, wn);
        mma(acc, f1);
        if constexpr (decltype(MAIN)::value) {
#pragma unroll
          for (int i = 0; i < 4; ++i) { G4_SCHED(0x008, 1); G4_SCHED(0x020, 1); G4_SCHED(0x100, 1); }
          G4_SCHED(0x100, 2);
          G4_SCHED(0x008, 4);
        }
      };
      int k = 0;
      for (; k + NS - 1 < nk; ++k) body(k, std::true_type());
      for (; k < nk; ++k) body(k, std::false_type());
    }
    tile_sync();  // every wave is done reading the stages

    // ---- next tile's first stages, then this tile's epilogue ----
    const int tn = tile_of(r + 1);
    TileCtx cn = c;
    if (tn >= 0) {
      decode(tn, cn, !WGT, r + 1);
      setup(cn);
      if constexpr (PREB > 0) Epi::pre_issue(ep, cn, pre_lds + ((r + 1) & 1) * PREB, w, lane);
      prime(cn);
    }
    // The epilogue starts once those stages have landed.  Run against the
    // stage loads, its LDS traffic and stores cost the down-projection 1-3%
    // and the weight gradients about 3% (measured at T = 32768, d = 1536,
    // E = 128, n = 256 and T = 16384, d = 2048, E = 256, n = 128).
    wait_vm<0>();
    if constexpr (PREB > 0) {
      Epi::run(ep, c, acc, smem + WE_OFF + w * WAVE_LDS, pre_lds + (r & 1) * PREB);
    } else if constexpr (is_wave_epi<Epi>::value) {
      Epi::run(ep, c, acc, smem + WE_OFF + w * WAVE_LDS);
    } else {
    // eight passes of 32 rows: pass p holds block j = p % 4 of the waves of
    // m half p / 4
#pragma unroll 1
    for (int p = 0; p < BM / EROWS; ++p) {
      TileCtx cp = c;
      cp.out_row0 = c.out_row0 + p * EROWS;
      cp.m_valid = min(EROWS, c.m_valid - p * EROWS);
      if (cp.m_valid <= 0) break;  // uniform over the workgroup
      if (wm == (p >> 2)) {
        const int jp = p & 3;
        const int cl = lane & 31, hl = lane >> 5;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (j != jp) continue;
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int eg = 0; eg < 4; ++eg) {
              lds_st_f4(Cs + cl * LDC + wn * 64 + 32 * i + 8 * eg + 4 * hl, acc[i][j][4 * eg],
                        acc[i][j][4 * eg + 1], acc[i][j][4 * eg + 2], acc[i][j][4 * eg + 3]);
            }
        }
      }
      tile_sync();
      Epi::run(ep, s, cp, Cs, nullptr);
      tile_sync();
    }
    }
    c = cn;
    t = tn;
    ++r;
  }
}

}  // namespace g4
}  // namespace moe
