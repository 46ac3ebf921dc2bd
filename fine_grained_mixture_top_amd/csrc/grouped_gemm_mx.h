// Row-mode grouped GEMM with MXFP8 operands on gfx950: the up-projection
// (SwiGLU epilogue), the down-projection, and the two activation-gradient
// GEMMs (dH with its pass epilogue, dXt) with both operands in the OCP MX
// format -- E4M3 elements, one E8M0 power-of-two scale per 32 consecutive k
// -- multiplied by v_mfma_scale_f32_32x32x64_f8f6f4, which applies the block
// scales inside the matrix core and accumulates in fp32.
//
// Tile, wave and scheduling layout as the bf16 row-mode kernels
// (grouped_gemm5.h): 256 x 256 tiles, 8 waves in 2 (m) x 4 (n), 128 x 64
// outputs per wave, the N-side operand first in the MFMA (so each lane's
// accumulators are four consecutive columns of one row and the bf16 kernels'
// wave-local epilogues apply unchanged), persistent XCD-grouped walk over the
// expert-major tile list, the next tile's first stage loaded before the
// epilogue.  What is specific to MXFP8:
//  * Both operands are k-contiguous bytes: A = routed rows [rows][K]
//    (gathered through idx or direct), B = an expert's transposed weights
//    [N][K].  A stage is k = 128, one 128-byte line per row and operand
//    (32 KB each), loaded straight into LDS; two stages.
//  * LDS rows are 128 bytes with 16-byte chunk c of row r in slot c ^ (r & 7):
//    the fragment reads (16 bytes per lane, 8 consecutive rows per LDS cycle
//    group) hit 8 distinct slots.
//  * Fragments: for the 64-k step s of a stage, lane l of a 32-row block
//    holds row l % 32, bytes k = 64s + 16h .. +15 and 64s + 32 + 16h .. +15
//    (h = l / 32); the block scale of (row, 32-k block b of the step) is
//    taken from lane row + 32 b.  Both operands use this placement, so the
//    contraction pairs equal k and each 32-k block meets its own scale.
//  * Scales: A's (per routed row, K/32 bytes) for the whole tile are loaded
//    into LDS with the tile's first stage; B's are stored blocked per stage,
//    [E][K/128][N] dwords (the four block scales of one column and stage),
//    and loaded with each stage.
#pragma once

#include "grouped_gemm4.h"
#include "grouped_gemm5.h"

namespace moe {
namespace gmx {

using g4::f32x16_v;
using g4::make_rsrc;
using g4::OOB;
using g4::wait_vm;

typedef int i32x8_v __attribute__((ext_vector_type(8)));

constexpr int BM = 256, BN = 256, BK = 128, NS = 2, NTH = 512;
constexpr int OPB = 256 * BK;             // bytes of one operand tile per stage (32 KB)
constexpr int BSC = 256 * 4;              // B scales of a stage: one dword per column
constexpr int STAGE = 2 * OPB + BSC;      // 65 KB
constexpr int LPS = 8;                    // 16-byte data loads per thread per stage
constexpr int MAX_PA = 64;                // A scale bytes per row: K <= 2048
constexpr int ASC_OFF = NS * STAGE;       // A scales of the tile: [256 rows][K/32]
constexpr int SMEM = ASC_OFF + 256 * MAX_PA;
constexpr int WE_OFF = STAGE;             // wave-local epilogue areas: over stage 1
constexpr int CS_OFF = STAGE;             // fp32 staging of the pass epilogue: over stage 1
static_assert(CS_OFF + g4::STAGE_C <= 2 * STAGE, "pass staging fits over stage 1");
static_assert(WE_OFF + 8 * g4::WAVE_LDS <= 2 * STAGE, "wave areas fit over stage 1");
static_assert(STAGE % 1024 == 0, "stage alignment");

// buffer -> LDS loads; soff (wave-uniform) is added to the per-lane voff
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t voff, uint32_t soff = 0) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (g4::lds_void_t*)lds, 4, voff, soff, 0, 0);
}
__device__ __forceinline__ void dma16s(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (g4::lds_void_t*)lds, 16, voff, soff, 0, 0);
}

__device__ __forceinline__ int swz(int r) { return r & 7; }

// k-contiguous byte rows, 128 bytes per row and stage.  Instruction i (0..3)
// of wave w covers tile rows (4w + i) * 8 .. +7; lane l takes row rb + l/8
// and LDS slot l % 8, which holds chunk (l % 8) ^ swz(row) of that row.
struct KCLoad {
  uint32_t off[4];
  template <class F>
  __device__ __forceinline__ void setup(int w, int lane, F rowoff) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (4 * w + i) * 8 + (lane >> 3);
      off[i] = rowoff(r) + (uint32_t)(((lane & 7) ^ swz(r)) * 16);
    }
  }
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, char* op, int w, int k0) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16s(rs, op + (4 * w + i) * 1024, off[i], (uint32_t)k0);
  }
};

// 16 bytes of row rb + lane % 32 at chunk c of the current stage
__device__ __forceinline__ uint4 chunk(const char* op, int r, int c) {
  return lds_ld16(op + r * BK + ((c ^ swz(r)) & 7) * 16);
}

// operand fragment of 32 rows for the 64-k step s of a stage
__device__ __forceinline__ i32x8_v frag(const char* op, int rb, int s, int lane) {
  const int r = rb + (lane & 31), h = lane >> 5;
  const uint4 lo = chunk(op, r, 4 * s + h), hi = chunk(op, r, 4 * s + 2 + h);
  i32x8_v v;
  v[0] = (int)lo.x; v[1] = (int)lo.y; v[2] = (int)lo.z; v[3] = (int)lo.w;
  v[4] = (int)hi.x; v[5] = (int)hi.y; v[6] = (int)hi.z; v[7] = (int)hi.w;
  return v;
}

// one 64-k step s of a stage: B fragments of the wave's two column blocks,
// then per row block its A fragment and two MFMAs.  asc / bsc: the stage's
// scale dwords (4 blocks of 32 k) of this lane's rows / columns.
__device__ __forceinline__ void step(f32x16_v (&acc)[2][4], const char* st, int s, int lane, int wm, int wn,
                                     const uint32_t (&asc)[4], const uint32_t (&bsc)[2]) {
  const int sh = 8 * (2 * s + (lane >> 5));
  i32x8_v n[2];
  int sn[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    n[i] = frag(st + OPB, wn * 64 + 32 * i, s, lane);
    sn[i] = (int)__builtin_amdgcn_ubfe(bsc[i], sh, 8);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const i32x8_v m = frag(st, wm * 128 + 32 * j, s, lane);
    const int sm = (int)__builtin_amdgcn_ubfe(asc[j], sh, 8);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(n[i], m, acc[i][j], 0, 0, 0, sn[i], 0, sm);
  }
}

// A: routed rows of fp8 codes (A.idx gathers them), A.ld = K bytes per row;
// ascale: their E8M0 scales, K/32 bytes per row, same row numbering.
// B: the expert's transposed fp8 weights [N][K] (B.estride bytes per expert);
// bscale: [E][K/128][N] dwords.  PAIRED arranges B's columns for G4SwiGLU.
template <bool PAIRED, class Epi>
__global__ void __launch_bounds__(NTH, 1)
grouped_gemm_mx_kernel(GemmShape s, Operand A, Operand B, const uint8_t* __restrict__ ascale,
                       const uint32_t* __restrict__ bscale, uint32_t a_bytes, uint32_t b_bytes,
                       uint32_t as_bytes, uint32_t bs_bytes, typename Epi::Params ep) {
  static_assert(g4::is_wave_epi<Epi>::value || g5::has_prefetch<Epi>::value,
                "wave-local epilogues or the pass epilogue with prefetched operands");
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  __shared__ int tprefix[MAX_E + 1];
  constexpr int PREB = g4::pre_bytes<Epi>::value;
  __shared__ __attribute__((aligned(256))) char pre_lds[PREB > 0 ? 2 * PREB : 16];  // wave epilogues' tile operands
  // the experts' row offsets, and the gathered A rows' indices of the
  // workgroup's next tile (loaded into LDS while the current tile computes,
  // so that moving to the next tile waits for no global load)
  __shared__ int soff[MAX_E + 1];
  __shared__ int nidx[BM];
  // (not with the dH epilogue, whose registers are all in use: there the
  // extra live values of the prefetch spill)
  constexpr bool NPRE = !g5::has_prefetch<Epi>::value;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w >> 2, wn = w & 3;
  const int NT = s.N / BN;
  const int PA = s.K / 32;  // A scale bytes per row
  {
    __shared__ int wsum[8];
    int carry = 0;
    for (int e0 = 0; e0 < s.E; e0 += NTH) {
      const int e = e0 + tid;
      const int o0 = e < s.E ? s.offsets[e] : 0;
      const int tiles = e < s.E ? (s.offsets[e + 1] - o0 + BM - 1) / BM : 0;
      if (NPRE && e < s.E) soff[e] = o0;
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
    if (tid == 0) {
      tprefix[s.E] = carry;
      if (NPRE) soff[s.E] = s.offsets[s.E];
    }
    __syncthreads();
  }
  const int total = tprefix[s.E] * NT;
  const int G = gridDim.x;
  const int vid = xcd_virtual_id(blockIdx.x, G);
  auto tile_of = [&](int r) -> int {
    const int t = r * G + vid;
    return t < total ? t : -1;
  };
  const int nk = s.K / BK;
  const char* abase = reinterpret_cast<const char*>(A.ptr);
  const char* bbase = reinterpret_cast<const char*>(B.ptr);

  auto decode = [&](int t, TileCtx& c) {
    c.tid = tid; c.lane = lane; c.wm = wm; c.wn = wn;
    const int mg = t / NT;
    c.nt = t % NT;
    c.e = upper_index(tprefix, s.E + 1, mg);
    c.mt = mg - tprefix[c.e];
    if constexpr (NPRE) {
      c.seg0 = soff[c.e];
      c.segn = soff[c.e + 1] - c.seg0;
    } else {
      c.seg0 = s.offsets[c.e];
      c.segn = s.offsets[c.e + 1] - c.seg0;
    }
    c.m_valid = min(BM, c.segn - c.mt * BM);
    c.out_row0 = (long long)c.seg0 + (long long)c.mt * BM;
    c.slot = -1;
    c.n0 = c.nt * BN;
  };

  __amdgpu_buffer_rsrc_t ra, rb, ras, rbs;
  KCLoad la, lb;
  uint32_t bso = 0;          // B-scale dword offset of this lane's column (waves 0..3)
  // source row of tile row r; pre: the gathered rows' indices are in nidx
  auto src_row = [&](const TileCtx& c, int r, auto PRE) -> uint32_t {
    const int m = c.mt * BM + r;
    const int row = c.seg0 + (m < c.segn ? m : c.segn - 1);  // rows past the end repeat the last one
    if constexpr (decltype(PRE)::value) return A.idx ? (uint32_t)nidx[r] : (uint32_t)row;
    else return A.idx ? (uint32_t)A.idx[row] : (uint32_t)row;
  };
  auto colmap = [&](const TileCtx& c, int cc) -> int {
    if constexpr (PAIRED) return g4::G4SwiGLU::col(cc, c.nt, s.N / 2);
    return c.n0 + cc;
  };
  auto setup = [&](const TileCtx& c, auto pre) {
    ra = make_rsrc(abase, a_bytes);
    la.setup(w, lane, [&](int r) -> uint32_t { return src_row(c, r, pre) * (uint32_t)A.ld; });
    rb = make_rsrc(bbase + (long long)c.e * B.estride, b_bytes);
    lb.setup(w, lane, [&](int r) -> uint32_t { return (uint32_t)colmap(c, r) * (uint32_t)B.ld; });
    ras = make_rsrc(ascale, as_bytes);
    rbs = make_rsrc(bscale + (long long)c.e * nk * s.N, bs_bytes);
    bso = w < 4 ? (uint32_t)colmap(c, 64 * w + lane) * 4u : 0u;
  };
  // the tile's A scales: PA instructions of 64 dwords, wave w taking
  // w, w + 8, ...; dword q of the block is byte 4 (q % (PA/4)) of row q / (PA/4)
  auto issue_ascale = [&](const TileCtx& c, auto pre) {
    const int dpr = PA / 4;
#pragma unroll 1
    for (int i = w; i < PA; i += 8) {
      const int q = i * 64 + lane;
      dma4(ras, smem + ASC_OFF + i * 256, src_row(c, q / dpr, pre) * (uint32_t)PA + (uint32_t)(q % dpr) * 4u);
    }
  };
  auto issue = [&](int k) {
    char* st = smem + (k & 1) * STAGE;
    const int k0 = k * BK;
    la.issue(ra, st, w, k0);
    lb.issue(rb, st + OPB, w, k0);
    if (w < 4) dma4(rbs, st + 2 * OPB + w * 256, bso, (uint32_t)(k * s.N) * 4u);
  };
  // scale dwords of stage k for this lane's 4 row blocks and 2 column blocks
  auto read_scales = [&](int k, uint32_t (&asc)[4], uint32_t (&bsc)[2]) {
    const char* st = smem + (k & 1) * STAGE;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      asc[j] = *reinterpret_cast<const uint32_t*>(smem + ASC_OFF + (wm * 128 + 32 * j + (lane & 31)) * PA + 4 * k);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      bsc[i] = *reinterpret_cast<const uint32_t*>(st + 2 * OPB + (wn * 64 + 32 * i + (lane & 31)) * 4);
  };

  int r = 0;
  int t = tile_of(0);
  TileCtx c;
  if (t >= 0) {
    decode(t, c);
    setup(c, std::false_type());
    if constexpr (PREB > 0) Epi::pre_issue(ep, c, pre_lds, w, lane);
    issue_ascale(c, std::false_type());
    issue(0);
  }
  while (t >= 0) {
    f32x16_v acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    // stage 1 overwrites the previous tile's epilogue areas
    lds_sync();
    if (nk > 1) issue(1);
    // wave 0: the gathered rows' indices of the next tile into nidx (its
    // loads after stage 1's; its waits for stages 0 and 1 cover them: every
    // wave reads nidx after the tile's last barrier)
    if (NPRE && A.idx && w == 0) {
      const int tn = tile_of(r + 1);
      if (tn >= 0) {
        TileCtx q;
        decode(tn, q);
        const __amdgpu_buffer_rsrc_t ri = make_rsrc(A.idx, (uint32_t)soff[s.E] * 4u);
#pragma unroll
        for (int i = 0; i < BM / 64; ++i) {
          const int m = q.mt * BM + 64 * i + lane;
          const int row = q.seg0 + (m < q.segn ? m : q.segn - 1);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(ri, (g4::lds_void_t*)(nidx + 64 * i), 4, (uint32_t)row * 4u, 0, 0,
                                                   0);
        }
      }
    }
    // the A scales and stage 0 are complete once only stage 1's loads remain
    if (nk > 1) {
      if (w < 4) wait_vm<LPS + 1>();
      else wait_vm<LPS>();
    } else {
      wait_vm<0>();
    }
    lds_sync();
    if constexpr (g4::has_init<Epi>::value) Epi::init(ep, c, acc, pre_lds + (r & 1) * PREB);
    uint32_t asc[4], bsc[2];
    read_scales(0, asc, bsc);
    // one 64-k step per iteration, two per stage; after a stage's second
    // step: stage k+1 complete, the barrier frees stage k for stage k+2, and
    // stage k+1's scales are read before the next loads are issued
#pragma unroll 1
    for (int it = 0; it < 2 * nk; ++it) {
      const int k = it >> 1, sidx = it & 1;
      step(acc, smem + (k & 1) * STAGE, sidx, lane, wm, wn, asc, bsc);
      if (sidx == 1 && k + 1 < nk) {
        wait_vm<0>();
        lds_sync();
        read_scales(k + 1, asc, bsc);
        if (k + 2 < nk) issue(k + 2);
      }
    }
    lds_sync();  // every wave is done reading the stages and the A scales

    const int tn = tile_of(r + 1);
    TileCtx cn = c;
    if (tn >= 0) {
      decode(tn, cn);
      setup(cn, std::bool_constant<NPRE>());
      if constexpr (PREB > 0) Epi::pre_issue(ep, cn, pre_lds + ((r + 1) & 1) * PREB, w, lane);
      issue_ascale(cn, std::bool_constant<NPRE>());
      issue(0);
    }
    if constexpr (PREB > 0) {
      Epi::run(ep, c, acc, smem + WE_OFF + w * g4::WAVE_LDS, pre_lds + (r & 1) * PREB);
    } else if constexpr (g4::is_wave_epi<Epi>::value) {
      Epi::run(ep, c, acc, smem + WE_OFF + w * g4::WAVE_LDS);
    } else {
      // eight passes of 32 rows (pass p holds block j = p % 4 of the waves of
      // m half p / 4), each pass's global operands loaded one pass ahead
      float* Cs = reinterpret_cast<float*>(smem + CS_OFF);
      typename Epi::Pre pcur, pnxt;
      Epi::load(ep, c, 0, pcur);
#pragma unroll 1
      for (int p = 0; p < BM / g4::EROWS; ++p) {
        if (c.m_valid - p * g4::EROWS <= 0) break;  // uniform over the workgroup
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
                lds_st_f4(Cs + cl * g4::LDC + wn * 64 + 32 * i + 8 * eg + 4 * hl, acc[i][j][4 * eg],
                          acc[i][j][4 * eg + 1], acc[i][j][4 * eg + 2], acc[i][j][4 * eg + 3]);
              }
          }
        }
        lds_sync();
        if (p + 1 < BM / g4::EROWS) Epi::load(ep, c, p + 1, pnxt);
        Epi::run(ep, c, p, Cs, pcur);
        pcur = pnxt;
        lds_sync();
      }
    }
    c = cn;
    t = tn;
    ++r;
  }
}

// Weight-gradient GEMM on MXFP8 operands: for each expert e,
// C[e] (Ma x Nb) = A_e B_e^T, A_e = [Ma][Kp_e] and B_e = [Nb][Kp_e] codes
// whose reduction runs along the expert's rows (padded to Kp_e, a multiple of
// 128, by k_mx_quant_seg), at byte Ma * padoff[e] (Nb * padoff[e]) of qa
// (qb); both operands' scales stage-blocked: dword (padoff[e] / 128 + k) *
// Ma + m of sa holds row m's four block scales of stage k (likewise sb).
// Tiles (e, m tile, n tile) in that order, each reducing over all of its
// expert's stages (none for an expert without rows: its tiles store zeros).
// Loads per wave and stage: 4 + 4 code instructions and one scale dword
// (waves 0..3 the B scales of the tile's 256 columns, 4..7 the A scales of
// its 256 rows).  Same fragments, MFMA step and wave-local epilogue as the
// row-mode kernel.
constexpr int WSC_OFF = 2 * OPB;               // B scales of a stage, then A scales
constexpr int WSTAGE = 2 * OPB + 2 * BSC;      // 66 KB
constexpr int WSMEM = NS * WSTAGE;
constexpr int WLPS = 9;                        // loads per wave per stage
static_assert(WSTAGE + 8 * g4::WAVE_LDS <= WSMEM, "wave areas fit over stage 1");
static_assert(WSTAGE % 1024 == 0, "stage alignment");

template <class Epi>
__global__ void __launch_bounds__(NTH, 1)
grouped_gemm_mxw_kernel(int E, int Ma, int Nb, const int32_t* __restrict__ padoff, const uint8_t* __restrict__ qa,
                        const uint32_t* __restrict__ sa, const uint8_t* __restrict__ qb,
                        const uint32_t* __restrict__ sb, uint32_t qa_bytes, uint32_t qb_bytes, uint32_t sa_bytes,
                        uint32_t sb_bytes, typename Epi::Params ep) {
  static_assert(g4::is_wave_epi<Epi>::value, "wave-local epilogues");
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  __shared__ int poff[MAX_E + 1];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w >> 2, wn = w & 3;
  for (int e = tid; e <= E; e += NTH) poff[e] = padoff[e];
  __syncthreads();
  const int MT = Ma / BM, NT = Nb / BN;
  const int total = E * MT * NT;
  const int G = gridDim.x;
  const int vid = xcd_virtual_id(blockIdx.x, G);
  auto tile_of = [&](int r) -> int {
    const int t = r * G + vid;
    return t < total ? t : -1;
  };
  int kp = 0, sbase = 0;  // the tile's padded rows and first stage
  auto decode = [&](int t, TileCtx& c) {
    c.tid = tid; c.lane = lane; c.wm = wm; c.wn = wn;
    c.e = t / (MT * NT);
    c.mt = (t / NT) % MT;
    c.nt = t % NT;
    c.seg0 = poff[c.e];
    c.segn = poff[c.e + 1] - c.seg0;
    c.m_valid = BM;
    c.out_row0 = (long long)c.e * Ma + (long long)c.mt * BM;
    c.slot = -1;
    c.n0 = c.nt * BN;
  };
  __amdgpu_buffer_rsrc_t ra = make_rsrc(qa, qa_bytes), rb = make_rsrc(qb, qb_bytes);
  __amdgpu_buffer_rsrc_t rsa = make_rsrc(sa, sa_bytes), rsb = make_rsrc(sb, sb_bytes);
  KCLoad la, lb;
  uint32_t so = 0;  // scale dword offset of this lane's row (waves 4..7) or column (waves 0..3) at stage 0
  auto setup = [&](const TileCtx& c) {
    kp = c.segn;
    sbase = c.seg0 / BK;
    const uint32_t abase = (uint32_t)Ma * (uint32_t)c.seg0, bbase = (uint32_t)Nb * (uint32_t)c.seg0;
    la.setup(w, lane, [&](int r) -> uint32_t { return abase + (uint32_t)(c.mt * BM + r) * (uint32_t)kp; });
    lb.setup(w, lane, [&](int r) -> uint32_t { return bbase + (uint32_t)(c.n0 + r) * (uint32_t)kp; });
    so = w < 4 ? ((uint32_t)sbase * (uint32_t)Nb + (uint32_t)(c.n0 + 64 * w + lane)) * 4u
               : ((uint32_t)sbase * (uint32_t)Ma + (uint32_t)(c.mt * BM + 64 * (w - 4) + lane)) * 4u;
  };
  auto issue = [&](int k) {
    char* st = smem + (k & 1) * WSTAGE;
    const int k0 = k * BK;
    la.issue(ra, st, w, k0);
    lb.issue(rb, st + OPB, w, k0);
    if (w < 4) dma4(rsb, st + WSC_OFF + w * 256, so, (uint32_t)(k * Nb) * 4u);
    else dma4(rsa, st + WSC_OFF + BSC + (w - 4) * 256, so, (uint32_t)(k * Ma) * 4u);
  };
  auto read_scales = [&](int k, uint32_t (&asc)[4], uint32_t (&bsc)[2]) {
    const char* st = smem + (k & 1) * WSTAGE;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      asc[j] = *reinterpret_cast<const uint32_t*>(st + WSC_OFF + BSC + (wm * 128 + 32 * j + (lane & 31)) * 4);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      bsc[i] = *reinterpret_cast<const uint32_t*>(st + WSC_OFF + (wn * 64 + 32 * i + (lane & 31)) * 4);
  };

  int r = 0;
  int t = tile_of(0);
  TileCtx c;
  if (t >= 0) {
    decode(t, c);
    setup(c);
    if (kp > 0) issue(0);
  }
  while (t >= 0) {
    const int nk = kp / BK;
    f32x16_v acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    // stage 1 overwrites the previous tile's epilogue areas
    lds_sync();
    if (nk > 0) {
      if (nk > 1) issue(1);
      if (nk > 1) wait_vm<WLPS>();
      else wait_vm<0>();
      lds_sync();
      uint32_t asc[4], bsc[2];
      read_scales(0, asc, bsc);
#pragma unroll 1
      for (int it = 0; it < 2 * nk; ++it) {
        const int k = it >> 1, sidx = it & 1;
        step(acc, smem + (k & 1) * WSTAGE, sidx, lane, wm, wn, asc, bsc);
        if (sidx == 1 && k + 1 < nk) {
          wait_vm<0>();
          lds_sync();
          read_scales(k + 1, asc, bsc);
          if (k + 2 < nk) issue(k + 2);
        }
      }
    }
    lds_sync();  // every wave is done reading the stages

    const int tn = tile_of(r + 1);
    TileCtx cn = c;
    if (tn >= 0) {
      decode(tn, cn);
      setup(cn);
      if (kp > 0) issue(0);
    }
    Epi::run(ep, c, acc, smem + WSTAGE + w * g4::WAVE_LDS);
    c = cn;
    t = tn;
    ++r;
  }
}

}  // namespace gmx
}  // namespace moe
