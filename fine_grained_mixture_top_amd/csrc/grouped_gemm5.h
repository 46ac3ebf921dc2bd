// Row-mode grouped GEMM for bf16 on gfx950 with k = 64 per stage: the
// up-projection, down-projection, dH and dXt GEMMs (every row of A is one
// routed row, gathered or contiguous; B is an expert's weight matrix).
//
// Same tile and wave layout as the 256 x 256 kernel of grouped_gemm4.h
// (8 waves in 2 (m) x 4 (n), 128 x 64 outputs each, v_mfma_f32_32x32x16_bf16,
// N-side fragment as the MFMA's first operand) and the same epilogues.  What
// differs is the k depth of a stage:
//  * A CU's loads are limited by the number of cache lines it can request per
//    clock, not by bytes: a load instruction that touches 64 bytes of each of
//    16 rows costs as much as one that touches 128 bytes of each of 8 rows.
//    With k = 64 per stage every row segment of a k-contiguous operand tile
//    is 128 bytes (a whole line), half the lines per byte of k = 32.
//  * Two stages of 64 KB (A 256 x 64 and B 64 x 256 or 256 x 64): one is
//    computed while the other loads, with one workgroup barrier per stage.
//  * Layouts: k-contiguous operands [256 rows][64 k] with 128-byte rows,
//    16-byte chunk c of row r in slot c ^ ((r >> 1) & 7), which keeps the
//    fragment reads (32 rows x 2 chunks per wave) conflict-free; weight tiles
//    stored [k][n] are [64 k-rows][256 cols] with the 512-byte-row layout and
//    transpose reads of the 256 x 256 kernel.
//  * The epilogue areas lie over stage 1: the next tile's stage 0 is loaded
//    before the epilogue, its stage 1 once every wave has finished it.
//  * A-row touches (host-selected TCHA variant): the tiles that share a row
//    block run side by side on one XCD, so wave 7 reads 4 bytes of a share
//    of the block's A lines two stages ahead, and its waits count them.
#pragma once

#include "grouped_gemm4.h"

namespace moe {
namespace g5 {

using g4::dma16;
using g4::f32x16_v;
using g4::make_rsrc;
using g4::OOB;
using g4::wait_vm;

constexpr int BM = 256, BN = 256, BK = 64, NS = 2, NTH = 512;
constexpr int OPB = 256 * BK * 2;  // bytes of one operand tile per stage (32 KB)
constexpr int STAGE = 2 * OPB;     // 64 KB
constexpr int LPS = 8;             // 16-byte loads per thread per stage (4 per operand)
constexpr int EROWS = g4::EROWS;
constexpr int LDC = g4::LDC;
constexpr int CS_OFF = STAGE;      // fp32 staging of the pass epilogue: over stage 1
constexpr int WE_OFF = STAGE;      // wave-local epilogue areas: over stage 1
constexpr int SMEM = NS * STAGE;
static_assert(CS_OFF + g4::STAGE_C <= SMEM, "pass staging fits over stage 1");
static_assert(WE_OFF + 8 * g4::WAVE_LDS <= SMEM, "wave areas fit over stage 1");

__device__ __forceinline__ int swz_kc(int r) { return (r >> 1) & 7; }

// k-contiguous rows, 128 bytes per row and stage.  Instruction i (0..3) of
// wave w covers tile rows (4w + i) * 8 .. +7; lane l takes row rb + l/8 and
// LDS slot l%8, which holds chunk (l%8) ^ swz(row) of that row.
struct KCLoad5 {
  uint32_t off[4];  // byte offset of this lane's chunk at k = 0
  template <class F>
  __device__ __forceinline__ void setup(int w, int lane, F rowoff) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (4 * w + i) * 8 + (lane >> 3);
      const uint32_t ro = rowoff(r);
      off[i] = ro == OOB ? OOB : ro + (uint32_t)(((lane & 7) ^ swz_kc(r)) * 16);
    }
  }
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, char* op, int w, int k0) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(rs, op + (4 * w + i) * 1024, off[i] + (uint32_t)k0 * 2u);
  }
};

// Weights stored [k][n]: k-rows of 256 columns.  Instruction i of wave w
// covers k-rows (4w + i) * 2 and +1 (lanes 0..31 and 32..63), slot l % 32.
struct MNLoad5 {
  uint32_t coff[4];  // column byte offset of this lane's chunk (OOB if absent)
  int kr[4];         // k-row of each instruction within the stage
  uint32_t ldb;      // row pitch in bytes
  template <class F>
  __device__ __forceinline__ void setup_cols(int w, int lane, F colmap) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kr[i] = (4 * w + i) * 2 + (lane >> 5);
      const int chunk = (lane & 31) ^ g4::swz_mn(kr[i]);
      const int col = colmap(chunk * 8);
      coff[i] = col < 0 ? OOB : (uint32_t)col * 2u;
    }
  }
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, char* op, int w, int k0) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t o = coff[i] == OOB ? OOB : coff[i] + (uint32_t)(k0 + kr[i]) * ldb;
      dma16(rs, op + (4 * w + i) * 1024, o);
    }
  }
};

// k-contiguous tile: row rb + lane%32, k = 16s + 8*(lane/32) .. +7 (s = 0..3)
__device__ __forceinline__ bf16x8_v frag_kc(const char* op, int rb, int s, int lane) {
  const int r = rb + (lane & 31);
  const int c = 2 * s + (lane >> 5);
  return *reinterpret_cast<const bf16x8_v*>(op + r * 128 + ((c ^ swz_kc(r)) & 7) * 16);
}

template <bool BMN>
struct Frags {
  bf16x8_v m[4], n[2];
  __device__ __forceinline__ void read(const char* st, int s, int lane, int wm, int wn) {
#pragma unroll
    for (int j = 0; j < 4; ++j) m[j] = frag_kc(st, wm * 128 + 32 * j, s, lane);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if constexpr (BMN) n[i] = g4::frag_mn(st + OPB, wn * 64 + 32 * i, s, lane);
      else n[i] = frag_kc(st + OPB, wn * 64 + 32 * i, s, lane);
    }
  }
};

template <bool BMN>
__device__ __forceinline__ void mma(f32x16_v (&acc)[2][4], const Frags<BMN>& f) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.n[i], f.m[j], acc[i][j], 0, 0, 0);
}

// dH epilogue with its cached-H loads issued one pass ahead.  Same
// arithmetic as EpiDH (recompute A from H, dS partial, dSwiGLU, A_s = gate A)
// on the 256-column tile; each pass covers 32 rows, and every thread owns
// chunk tid % 32 of rows tid / 32 and tid / 32 + 16.  The H values, gates of
// pass p + 1 are loaded before pass p is computed, so their latency is not
// paid once per pass.
struct G5DH {
  using Params = typename EpiDH<bf16_t, EROWS, BN, NTH>::Params;
  static constexpr bool PREFETCH = true;
  struct Pre {
    uint4 g[2], u[2];
    float gate[2];
  };
  __device__ __forceinline__ static long long row_of(const TileCtx& c, int pass, int it) {
    const int r = pass * EROWS + (c.tid >> 5) + 16 * it;
    return c.out_row0 + (r < c.m_valid ? r : c.m_valid - 1);
  }
  __device__ __forceinline__ static void load(const Params& p, const TileCtx& c, int pass, Pre& x) {
    const long long ldh = 2LL * p.n;
    const int col = c.n0 + (c.tid & 31) * 8;
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const long long grow = row_of(c, pass, it);
      x.g[it] = *reinterpret_cast<const uint4*>(p.H + grow * ldh + col);
      x.u[it] = *reinterpret_cast<const uint4*>(p.H + grow * ldh + p.n + col);
      x.gate[it] = p.gate[grow];
    }
  }
  __device__ __forceinline__ static void unpack8(const uint4 w, float (&v)[8]) {
    const uint32_t q[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(q[i] << 16);
      v[2 * i + 1] = __uint_as_float(q[i] & 0xffff0000u);
    }
  }
  __device__ __forceinline__ static void run(const Params& p, const TileCtx& c, int pass, const float* Cs,
                                             const Pre& x) {
    const long long ldh = 2LL * p.n;
    const int ch = c.tid & 31;
    const int col = c.n0 + ch * 8;
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int r = (c.tid >> 5) + 16 * it;
      const bool valid = pass * EROWS + r < c.m_valid;
      const long long grow = row_of(c, pass, it);
      float dap[8], g[8], u[8];
      ld8(Cs + r * LDC + ch * 8, dap);
      unpack8(x.g[it], g);
      unpack8(x.u[it], u);
      const float gt = x.gate[it];
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
        st8<bf16_t>(p.dH + grow * ldh + col, dg);
        st8<bf16_t>(p.dH + grow * ldh + p.n + col, du);
        st8<bf16_t>(p.As + grow * (long long)p.n + col, as);
      }
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) ps += __shfl_xor(ps, o, 64);
      if (valid && ch == 0) p.dS_part[grow * p.NT + c.nt] = ps;
    }
  }
};

template <class E, class = void> struct has_prefetch : std::false_type {};
template <class E> struct has_prefetch<E, std::void_t<decltype(E::PREFETCH)>> : std::bool_constant<E::PREFETCH> {};

// A: routed rows (A.idx gathers them), k-contiguous, K = s.K.  B: the
// expert's weights, [N][K] (BMN = false) or [K][N] (BMN = true; PAIRED
// arranges the columns for G4SwiGLU).  Workgroup v takes tiles v, v + G, ...
// of the expert-major tile list (v the XCD-grouped id).
template <bool BMN, bool PAIRED, class Epi, bool TCHA = false>
__global__ void __launch_bounds__(NTH, 1)
grouped_gemm5_kernel(GemmShape s, Operand A, Operand B, uint32_t a_bytes, uint32_t b_bytes,
                     typename Epi::Params ep) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  __shared__ int tprefix[MAX_E + 1];
  // the experts' row offsets, and the gathered A rows' indices of the
  // workgroup's next tile (loaded into LDS while the current tile computes,
  // so that moving to the next tile waits for no global load)
  __shared__ int soff[MAX_E + 1];
  __shared__ int nidx[BM];
  __shared__ __attribute__((aligned(256))) char touch_sink[256];  // written by the A-row touches, never read
  constexpr int PREB = g4::pre_bytes<Epi>::value;
  __shared__ __attribute__((aligned(256))) char pre_lds[PREB > 0 ? 2 * PREB : 16];  // wave epilogues' tile operands

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w >> 2, wn = w & 3;
  const int NT = s.N / BN;
  {
    __shared__ int wsum[8];
    int carry = 0;
    for (int e0 = 0; e0 < s.E; e0 += NTH) {
      const int e = e0 + tid;
      const int o0 = e < s.E ? s.offsets[e] : 0;
      const int tiles = e < s.E ? (s.offsets[e + 1] - o0 + BM - 1) / BM : 0;
      if (e < s.E) soff[e] = o0;
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
      soff[s.E] = s.offsets[s.E];
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
  float* Cs = reinterpret_cast<float*>(smem + CS_OFF);

  auto decode = [&](int t, TileCtx& c) {
    c.tid = tid; c.lane = lane; c.wm = wm; c.wn = wn;
    const int mg = t / NT;
    c.nt = t % NT;
    c.e = upper_index(tprefix, s.E + 1, mg);
    c.mt = mg - tprefix[c.e];
    c.seg0 = soff[c.e];
    c.segn = soff[c.e + 1] - c.seg0;
    c.m_valid = min(BM, c.segn - c.mt * BM);
    c.out_row0 = (long long)c.seg0 + (long long)c.mt * BM;
    c.slot = -1;
    c.n0 = c.nt * BN;
  };

  __amdgpu_buffer_rsrc_t ra, rb;
  KCLoad5 la, lb_kc;
  MNLoad5 lb_mn;
  // A-row touch (TCHA, chosen by the host for k-contiguous weights when A's
  // rows are read without an index and NT >= 4, i.e. dXt): the NT tiles of
  // one row block share its A rows and run side by side on one XCD; when
  // wave 7 issues stage k, tile nt also reads 4 bytes of a 1/S share of the
  // 256 A lines of stage k + 2 into a scratch LDS area (S = NT clamped to
  // 4..8, the share chosen by nt mod S), so that the row block's tiles bring
  // different lines into L2 a stage ahead of their loads.  Past the last
  // stage the touch reads nothing (out-of-range offset) but is still issued,
  // so that wave 7's load counts stay fixed.  dXt 0.527 -> 0.501 ms at
  // d = 1536, n = 256 and 2.01 -> 1.95 ms at d = 2048, n = 1024.  (A B-line
  // touch of the [k][n] weights of the up-projection helped while the
  // compiler drained every stage in flight; with the pipeline intact it cost
  // about 1.5% and is gone.)
  constexpr bool TOUCH = TCHA;
  static_assert(!(TCHA && BMN), "A-row touches read k-contiguous A rows beside k-contiguous weights");
  const int tshare = NT < 4 ? 4 : (NT > 8 ? 8 : NT);  // S
  uint32_t tch_col = OOB;  // byte offset of this lane's A line at k = 0
  auto setup_touch = [&](const TileCtx& c) {
    if constexpr (!TOUCH) return;
    const int per = (256 + tshare - 1) / tshare;  // 32..64 lines per tile and stage
    const int q = (c.nt % tshare) * per + lane;
    const int m = c.mt * BM + q;
    tch_col = (lane < per && q < 256 && m < c.segn) ? (uint32_t)(c.seg0 + m) * (uint32_t)A.ld * 2u : OOB;
  };
  auto touch = [&](int k) {
    const int kt = k + 2;
    uint32_t o = OOB;
    if (kt < nk && tch_col != OOB) o = tch_col + (uint32_t)(kt * BK) * 2u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (g4::lds_void_t*)touch_sink, 4, o, 0, 0, 0);
  };
  auto setup = [&](const TileCtx& c, bool pre) {
    ra = make_rsrc(abase, a_bytes);
    la.setup(w, lane, [&](int r) -> uint32_t {
      const int m = c.mt * BM + r;
      const int row = c.seg0 + (m < c.segn ? m : c.segn - 1);  // rows past the end repeat the last one
      const uint32_t src = A.idx ? (uint32_t)(pre ? nidx[r] : A.idx[row]) : (uint32_t)row;
      return src * (uint32_t)A.ld * 2u;
    });
    rb = make_rsrc(bbase + (long long)c.e * B.estride * 2, b_bytes);
    if constexpr (!BMN) {
      lb_kc.setup(w, lane, [&](int r) -> uint32_t { return (uint32_t)(c.n0 + r) * (uint32_t)B.ld * 2u; });
    } else {
      lb_mn.setup_cols(w, lane, [&](int cc) {
        if constexpr (PAIRED) return g4::G4SwiGLU::col(cc, c.nt, s.N / 2);
        return c.n0 + cc;
      });
      lb_mn.ldb = (uint32_t)B.ld * 2u;
    }
    if (TOUCH && w == 7) setup_touch(c);
  };
  auto issue = [&](int k) {
    char* st = smem + (k & 1) * STAGE;
    const int k0 = k * BK;
    la.issue(ra, st, w, k0);
    if constexpr (!BMN) lb_kc.issue(rb, st + OPB, w, k0);
    else lb_mn.issue(rb, st + OPB, w, k0);
    if (TOUCH && w == 7) touch(k);
  };

  int r = 0;
  int t = tile_of(0);
  TileCtx c;
  if (t >= 0) {
    decode(t, c);
    setup(c, false);
    if constexpr (PREB > 0) Epi::pre_issue(ep, c, pre_lds, w, lane);
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

    // stage 1 overwrites the previous tile's epilogue areas: every wave must
    // be done with them.  After the dH epilogue (workgroup passes with
    // prefetched loads) the tile starts once its stores and stage 0 are
    // done: measured 1-2% faster there, while the wave epilogues gain from
    // loading stage 1 during stage 0 (dXt 5-6% faster than with that drain).
    if constexpr (has_prefetch<Epi>::value) wait_vm<0>();
    lds_sync();
    if (nk > 1) issue(1);
    // wave 0: the gathered rows' indices of the next tile into nidx (its
    // loads after stage 1's; its waits for stages 0 and 1 cover them: every
    // wave reads nidx after the tile's last barrier)
    if (A.idx && w == 0) {
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
    // stage 0 complete: only stage 1's loads came after it (and, for tiles
    // after the first, the previous epilogue's stores before those)
    // (wave 7: also the touches issued with stages 0 and 1)
    if (TOUCH && w == 7) {
      if (nk > 1) wait_vm<LPS + 2>();
      else wait_vm<1>();
    } else {
      if (nk > 1) wait_vm<LPS>();
      else wait_vm<0>();
    }
    lds_sync();
    if constexpr (g4::has_init<Epi>::value) Epi::init(ep, c, acc, pre_lds + (r & 1) * PREB);
    Frags<BMN> f0, f1;
    f0.read(smem, 0, lane, wm, wn);
    for (int k = 0; k < nk; ++k) {
      const char* cur = smem + (k & 1) * STAGE;
      f1.read(cur, 1, lane, wm, wn);
      mma(acc, f0);
      f0.read(cur, 2, lane, wm, wn);
      mma(acc, f1);
      f1.read(cur, 3, lane, wm, wn);
      mma(acc, f0);
      if (k + 1 < nk) {
        // stage k+1 complete (nothing was issued after it); the barrier also
        // frees stage k's buffer for stage k+2
        // (wave 7: its touch issued with stage k+1 may still be out)
        if (TOUCH && w == 7) wait_vm<1>();
        else wait_vm<0>();
        lds_sync();
        if (k + 2 < nk) issue(k + 2);
        f0.read(smem + ((k + 1) & 1) * STAGE, 0, lane, wm, wn);
      }
      mma(acc, f1);
    }
    lds_sync();  // every wave is done reading the stages

    // ---- next tile's stage 0, then this tile's epilogue ----
    const int tn = tile_of(r + 1);
    TileCtx cn = c;
    if (tn >= 0) {
      decode(tn, cn);
      setup(cn, true);
      if constexpr (PREB > 0) Epi::pre_issue(ep, cn, pre_lds + ((r + 1) & 1) * PREB, w, lane);
      issue(0);
    }
    if constexpr (PREB > 0) {
      Epi::run(ep, c, acc, smem + WE_OFF + w * g4::WAVE_LDS, pre_lds + (r & 1) * PREB);
    } else if constexpr (g4::is_wave_epi<Epi>::value) {
      Epi::run(ep, c, acc, smem + WE_OFF + w * g4::WAVE_LDS);
    } else if constexpr (has_prefetch<Epi>::value) {
      // eight passes of 32 rows, each pass's global operands loaded one ahead
      typename Epi::Pre cur, nxt;
      Epi::load(ep, c, 0, cur);
#pragma unroll 1
      for (int p = 0; p < BM / EROWS; ++p) {
        if (c.m_valid - p * EROWS <= 0) break;  // uniform over the workgroup
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
        lds_sync();
        if (p + 1 < BM / EROWS) Epi::load(ep, c, p + 1, nxt);
        Epi::run(ep, c, p, Cs, cur);
        cur = nxt;
        lds_sync();
      }
    } else {
      // eight passes of 32 rows: pass p holds block j = p % 4 of the waves
      // of m half p / 4
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
        lds_sync();
        Epi::run(ep, s, cp, Cs, nullptr);
        lds_sync();
      }
    }
    c = cn;
    t = tn;
    ++r;
  }
}

}  // namespace g5
}  // namespace moe
