// Routing: top-K selection, optional token rounding, expert-sorted segments
// and the per-token CSR.  All integer results are exact and independent of
// thread timing: counts and ranks come from ordered scans, never from the
// order in which atomics land.
//
// The pages keep the routing metadata as a binary token x expert mask
// ([A] "MoE 与它的隐患", figure captions).  Here the mask is a byte array
// laid out expert-major ([E][T]) so that each expert's token scan is one
// coalesced sweep; the GEMMs consume the compact segment form built from it.
// Token rounding follows [B] (scheduling paragraph): counts become multiples
// of the GEMM tile, at most one tile away from the plain count.
#include <algorithm>

#include "device_common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr uint64_t GOLDEN = 0x9E3779B97F4A7C15ull;

// SplitMix64 output function (Steele, Lea & Flood 2014).
__device__ __forceinline__ uint64_t splitmix64(uint64_t x) {
  uint64_t z = x + GOLDEN;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Order-preserving map of a float score to uint32 (larger score, larger
// key); -0 and +0 map to the same key, as they compare equal.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive scan of one int per thread over a 256-thread block, in thread
// order; returns the prefix and writes the block total to *total.
__device__ __forceinline__ int block_scan256(int v, int* lds /* >= 4 ints */, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) lds[wave] = incl;
  __syncthreads();
  int base = 0, tot = 0;
  for (int w = 0; w < 4; ++w) {
    int s = lds[w];
    if (w < wave) base += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + incl - v;
}

// Same for 1024 threads.
__device__ __forceinline__ int block_scan1024(int v, int* lds /* >= 16 ints */, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) lds[wave] = incl;
  __syncthreads();
  int base = 0, tot = 0;
  for (int w = 0; w < 16; ++w) {
    int s = lds[w];
    if (w < wave) base += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + incl - v;
}

// Inverse of score_key (-0 comes back as +0).
__device__ __forceinline__ float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// 64-bit max over the 16 lanes of a DPP row: rotations by 8, 4, 2, 1.
__device__ __forceinline__ uint64_t row_max16(uint64_t b) {
#define MOE_ROR_MAX(o)                                                                                  \
  {                                                                                                     \
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, 0x120 + (o), 0xF, 0xF, false); \
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), 0x120 + (o), 0xF, 0xF, false); \
    const uint64_t ob = ((uint64_t)hi << 32) | lo;                                                      \
    b = ob > b ? ob : b;                                                                                \
  }
  MOE_ROR_MAX(8) MOE_ROR_MAX(4) MOE_ROR_MAX(2) MOE_ROR_MAX(1)
#undef MOE_ROR_MAX
  return b;
}

// G lanes per token (16 or 32), MAXV >= E / G scores per lane: K rounds of
// an arg-max over the token's scores.  Each score is held as one 64-bit key,
// (order-preserving score bits, ~expert id), so the larger key is the larger
// score and, among equal scores, the smaller expert; a round is a max over
// the lane's keys, a max over the group (DPP rotations inside a 16-lane row,
// one lane exchange between rows for G = 32), and clearing the winner's key.
// Slot k's score is kept by lane k % G of the group.  Writes the slot-ordered
// experts, their softmax gates and the membership bytes; with tok_ptr also
// tok_ptr[t] = t*K (every token keeps exactly K rows when there is no token
// rounding).  (T = 32768, E = 128, K = 8: 23 -> 16 us against a compare-and-
// branch version with the same lane layout.)
template <int G, int MAXV>
__global__ void __launch_bounds__(256)
k_topk(const float* __restrict__ scores, int T, int E, int K, int mpitch, int32_t* __restrict__ topk_idx,
       float* __restrict__ topk_gate, uint8_t* __restrict__ mask, int32_t* __restrict__ tok_ptr) {
  static_assert(G == 16 || G == 32, "DPP rows of 16 lanes");
  const int lane = threadIdx.x & (G - 1);
  const int t = (blockIdx.x * 256 + threadIdx.x) / G;
  const bool live = t < T;  // groups never straddle a wave, so exchanges stay inside live groups
  const float* z = scores + (size_t)(live ? t : 0) * E;
  uint64_t key[MAXV];
  float zs[MAXV];
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int e = lane + G * i;
    const bool ok = live && e < E;
    key[i] = ok ? ((uint64_t)score_key(z[e]) << 32) | (0xffffffffu - (uint32_t)e) : 0ull;  // 0: no score
    zs[i] = 0.f;
  }
  for (int k = 0; k < K; ++k) {
    uint64_t b = key[0];
#pragma unroll
    for (int i = 1; i < MAXV; ++i) b = key[i] > b ? key[i] : b;
    if constexpr (G == 32) {
      const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)b, 16, 64);
      const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(b >> 32), 16, 64);
      const uint64_t ob = ((uint64_t)hi << 32) | lo;
      b = ob > b ? ob : b;
    }
    b = row_max16(b);
#pragma unroll
    for (int i = 0; i < MAXV; ++i) key[i] = key[i] == b ? 0ull : key[i];  // keys are distinct
    const int be = (int)(0xffffffffu - (uint32_t)b);
    const float bv = key_score((uint32_t)(b >> 32));
    if ((k & (G - 1)) == lane) {
#pragma unroll
      for (int i = 0; i < MAXV; ++i)
        if (i == k / G) zs[i] = bv;
    }
    if (lane == 0 && live) {
      topk_idx[(size_t)t * K + k] = be;
      mask[(size_t)be * mpitch + t] = 1;
    }
  }
  const float m = __shfl(zs[0], (threadIdx.x & 63) & ~(G - 1), 64);  // slot 0: largest score
  float part = 0.f;
#pragma unroll
  for (int i = 0; i < MAXV; ++i)
    if (lane + G * i < K) part += __expf(zs[i] - m);
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) part += __shfl_xor(part, o, 64);
  if (!live) return;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int k = lane + G * i;
    if (k < K) topk_gate[(size_t)t * K + k] = __expf(zs[i] - m) / part;
  }
  if (tok_ptr && lane == 0) {
    tok_ptr[t] = t * K;
    if (t == T - 1) tok_ptr[T] = T * K;
  }
}

// Membership counts per (expert, chunk of CHUNK tokens): chunk_cnt[e][c]
// (one 256-thread workgroup per chunk, 16 tokens per thread; mask rows are
// 16-byte aligned and zero past T).  The per-expert counts are their sums
// (k_scan_experts), and the chunk counts let k_compact split a heavy
// expert's tokens over many workgroups.
constexpr int CHUNK = 256 * 16;
__global__ void __launch_bounds__(256)
k_chunk_count(const uint8_t* __restrict__ mask, int mpitch, int nch, int32_t* __restrict__ chunk_cnt) {
  __shared__ int lds[8];
  const int c = blockIdx.x, e = blockIdx.y;
  const int t0 = c * CHUNK + threadIdx.x * 16;
  int v = 0;
  if (t0 < mpitch) {
    const uint4 u = *reinterpret_cast<const uint4*>(mask + (size_t)e * mpitch + t0);
    // each byte is 0 or 1: the byte sum of a word is its popcount
    v = __popc(u.x) + __popc(u.y) + __popc(u.z) + __popc(u.w);
  }
  int total;
  block_scan256(v, lds, &total);
  if (threadIdx.x == 0) chunk_cnt[(size_t)e * nch + c] = total;
}

__device__ __forceinline__ int expert_total(const int32_t* __restrict__ chunk_cnt, int nch, int e) {
  int c = 0;
  for (int i = 0; i < nch; ++i) c += chunk_cnt[(size_t)e * nch + i];
  return c;
}

// scores [T][E] -> scoresT [E][pitch]
__global__ void k_transpose_scores(const float* __restrict__ in, int T, int E, int pitch,
                                   float* __restrict__ out) {
  __shared__ float tile[32][33];
  const int t0 = blockIdx.x * 32, e0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 256 threads: ty 0..7
  for (int r = ty; r < 32; r += 8) {
    int t = t0 + r, e = e0 + tx;
    if (t < T && e < E) tile[r][tx] = in[(size_t)t * E + e];
  }
  __syncthreads();
  for (int r = ty; r < 32; r += 8) {
    int e = e0 + r, t = t0 + tx;
    if (t < T && e < E) out[(size_t)e * pitch + t] = tile[tx][r];
  }
}

// Token rounding works on 16-token groups: one 16-byte load of membership
// bytes and four 16-byte loads of expert-major scores per thread.
constexpr int TR_THREADS = 1024;
constexpr int TR_GROUP = 16;

// Candidate bits of one 16-token group (bit i: token t0 + i is a candidate,
// i.e. inside [0, T) with membership byte == want) and their score keys.
struct TrGroup {
  uint4 mbytes;
  uint32_t cand;
  uint32_t key[TR_GROUP];
};

__device__ __forceinline__ void tr_load(const uint8_t* m, const float* z, int t0, int T, uint32_t want,
                                        TrGroup& g) {
  g.mbytes = *reinterpret_cast<const uint4*>(m + t0);
  const uint32_t w[4] = {g.mbytes.x, g.mbytes.y, g.mbytes.z, g.mbytes.w};
  g.cand = 0;
#pragma unroll
  for (int i = 0; i < TR_GROUP; ++i)
    if (t0 + i < T && ((w[i >> 2] >> (8 * (i & 3))) & 0xffu) == want) g.cand |= 1u << i;
  if (g.cand) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 v = *reinterpret_cast<const float4*>(z + t0 + 4 * q);
      g.key[4 * q + 0] = score_key(v.x);
      g.key[4 * q + 1] = score_key(v.y);
      g.key[4 * q + 2] = score_key(v.z);
      g.key[4 * q + 3] = score_key(v.w);
    }
  }
}

// Token rounding of one expert per workgroup.  c = plain count; r = rounded
// count.  r < c: keep the r best-ranked routed tokens; r > c: add the r - c
// best-ranked tokens not routed to this expert.  Rank: score descending, then
// token id ascending.  The threshold key is found by an MSB-first radix select
// over the order-preserving score keys (digits of 12, 10 and 10 bits, counted
// in an LDS histogram); candidates with exactly the threshold key are then
// taken in ascending token order.  Counts are exact, so the result does not
// depend on the order in which the histogram atomics land.
// LDSK (mask rows of at most TR_LDS_TOKENS tokens): the candidates' keys are
// read from HBM once into LDS (0 marks a non-candidate; a candidate's key is
// at least 1) and the radix passes and the final selection sweep LDS; else
// every pass re-reads the expert's scores and membership bytes.
constexpr int TR_LDS_TOKENS = 32768;
template <bool LDSK>
__global__ void __launch_bounds__(TR_THREADS)
k_token_round(const float* __restrict__ scoresT, uint8_t* __restrict__ mask, int mpitch,
              int32_t* __restrict__ chunk_cnt, int nch, int32_t* __restrict__ counts_raw, int T, int M,
              int mode, uint64_t seed) {
  static_assert(TR_THREADS * TR_GROUP == 4 * CHUNK && TR_THREADS / 64 == 16, "a sweep is four chunks");
  extern __shared__ __attribute__((aligned(16))) uint32_t kl[];  // LDSK: [mpitch] candidate keys
  __shared__ int hist[4096];
  __shared__ int sh[20];
  const int e = blockIdx.x;
  const int c = expert_total(chunk_cnt, nch, e);
  if (threadIdx.x == 0) counts_raw[e] = c;
  const int rem = c % M;
  if (rem == 0) return;
  int r;
  {
    const int down = c - rem;
    bool up;
    if (mode == 1) {
      up = rem >= M / 2;
    } else {
      int bits = 31 - __clz(M);  // M is a power of two
      uint64_t u = splitmix64(seed ^ ((uint64_t)e * GOLDEN)) >> (64 - bits);
      up = (uint64_t)rem > u;
    }
    r = up ? down + M : down;
    if (r > T) r = down;
  }
  const bool drop = r < c;
  const uint32_t want = drop ? 1u : 0u;  // candidates: routed (drop) or not (add)
  const int k_sel = drop ? r : r - c;    // candidates to select
  uint8_t* m = mask + (size_t)e * mpitch;
  const float* z = scoresT + (size_t)e * mpitch;
  const int tid = threadIdx.x;
  constexpr int SWEEP = TR_THREADS * TR_GROUP;

  if constexpr (LDSK) {
    for (int base = 0; base < mpitch; base += SWEEP) {
      const int t0 = base + tid * TR_GROUP;
      if (t0 >= mpitch) continue;
      TrGroup g;
      tr_load(m, z, t0, T, want, g);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = ((g.cand >> (4 * q + i)) & 1u) ? max(g.key[4 * q + i], 1u) : 0u;
        *reinterpret_cast<uint4*>(kl + t0 + 4 * q) = make_uint4(v[0], v[1], v[2], v[3]);
      }
    }
    __syncthreads();
  }

  uint32_t prefix = 0, pmask = 0;
  int kk = k_sel;
  if (k_sel > 0) {
    for (int pass = 0; pass < 3; ++pass) {
      const int width = pass == 0 ? 12 : 10;
      const int shift = pass == 0 ? 20 : (pass == 1 ? 10 : 0);
      const int nb = 1 << width;
      for (int i = tid; i < nb; i += TR_THREADS) hist[i] = 0;
      __syncthreads();
      if constexpr (LDSK) {
        for (int t = tid; t < mpitch; t += TR_THREADS) {
          const uint32_t k = kl[t];
          if (k && (k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & (nb - 1)], 1);
        }
      } else {
        for (int base = 0; base < mpitch; base += SWEEP) {
          const int t0 = base + tid * TR_GROUP;
          if (t0 >= mpitch) continue;
          TrGroup g;
          tr_load(m, z, t0, T, want, g);
#pragma unroll
          for (int i = 0; i < TR_GROUP; ++i)
            if (((g.cand >> i) & 1u) && (g.key[i] & pmask) == prefix)
              atomicAdd(&hist[(g.key[i] >> shift) & (nb - 1)], 1);
        }
      }
      __syncthreads();
      // Bins in descending order: thread tid owns bins nb-1-per*tid down to
      // nb-per*(tid+1); a scan in thread order counts the candidates above.
      const int per = nb / TR_THREADS;
      int cnt[4] = {0, 0, 0, 0};
      int s = 0;
      for (int j = 0; j < per; ++j) {
        cnt[j] = hist[nb - 1 - per * tid - j];
        s += cnt[j];
      }
      int tot;
      int above = block_scan1024(s, sh, &tot);
      if (above < kk && above + s >= kk) {
        for (int j = 0; j < per; ++j) {
          if (above + cnt[j] >= kk) {
            sh[16] = nb - 1 - per * tid - j;
            sh[17] = kk - above;
            break;
          }
          above += cnt[j];
        }
      }
      __syncthreads();
      prefix |= (uint32_t)sh[16] << shift;
      pmask |= (uint32_t)(nb - 1) << shift;
      kk = sh[17];
      __syncthreads();
    }
  }
  // prefix = threshold key; kk = how many threshold-key candidates to take
  int carry = 0;
  for (int base = 0; base < mpitch; base += SWEEP) {
    const int t0 = base + tid * TR_GROUP;
    TrGroup g;
    g.cand = 0;
    uint32_t gt = 0, eq = 0;
    if (t0 < mpitch) {
      if constexpr (LDSK) {
        g.mbytes = *reinterpret_cast<const uint4*>(m + t0);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint4 v = *reinterpret_cast<const uint4*>(kl + t0 + 4 * q);
          g.key[4 * q] = v.x; g.key[4 * q + 1] = v.y; g.key[4 * q + 2] = v.z; g.key[4 * q + 3] = v.w;
        }
#pragma unroll
        for (int i = 0; i < TR_GROUP; ++i)
          if (g.key[i]) g.cand |= 1u << i;
      } else {
        tr_load(m, z, t0, T, want, g);
      }
      if (k_sel > 0) {
#pragma unroll
        for (int i = 0; i < TR_GROUP; ++i)
          if ((g.cand >> i) & 1u) {
            if (g.key[i] > prefix) gt |= 1u << i;
            if (g.key[i] == prefix) eq |= 1u << i;
          }
      }
    }
    int tot;
    int run = carry + block_scan1024(__popc(eq), sh, &tot);
    uint32_t sel = gt;
#pragma unroll
    for (int i = 0; i < TR_GROUP; ++i)
      if ((eq >> i) & 1u) {
        if (run < kk) sel |= 1u << i;
        ++run;
      }
    // drop: unselected candidates leave; add: selected candidates join
    const uint32_t flip = drop ? (g.cand & ~sel) : (g.cand & sel);
    if (flip) {
      uint32_t w[4] = {g.mbytes.x, g.mbytes.y, g.mbytes.z, g.mbytes.w};
#pragma unroll
      for (int i = 0; i < TR_GROUP; ++i)
        if ((flip >> i) & 1u) w[i >> 2] ^= 1u << (8 * (i & 3));
      *reinterpret_cast<uint4*>(m + t0) = make_uint4(w[0], w[1], w[2], w[3]);
      g.mbytes = make_uint4(w[0], w[1], w[2], w[3]);
    }
    carry += tot;
    // the expert's new chunk counts: a sweep is four chunks of 256 threads
    int c = t0 < mpitch ? __popc(g.mbytes.x) + __popc(g.mbytes.y) + __popc(g.mbytes.z) + __popc(g.mbytes.w) : 0;
    for (int o = 32; o >= 1; o >>= 1) c += __shfl_xor(c, o, 64);
    if ((tid & 63) == 0) sh[tid >> 6] = c;  // sh[0..15]: free between the scans
    __syncthreads();
    if (tid < SWEEP / CHUNK) {
      const int ch = base / CHUNK + tid;
      if (ch < nch) chunk_cnt[(size_t)e * nch + ch] = sh[4 * tid] + sh[4 * tid + 1] + sh[4 * tid + 2] + sh[4 * tid + 3];
    }
    __syncthreads();
  }
}

// counts (and counts2 when set) = per-expert sums of the chunk counts;
// offsets / tile_offsets: exclusive scans of counts and ceil(counts / tile).
__global__ void __launch_bounds__(1024)
k_scan_experts(const int32_t* __restrict__ chunk_cnt, int nch, int E, int tile, int32_t* __restrict__ counts,
               int32_t* __restrict__ counts2, int32_t* __restrict__ offsets, int32_t* __restrict__ tile_offsets) {
  __shared__ int lds[16];
  const int e = threadIdx.x;
  const int c = e < E ? expert_total(chunk_cnt, nch, e) : 0;
  if (e < E) {
    counts[e] = c;
    if (counts2) counts2[e] = c;
  }
  int tot1, tot2;
  const int o = block_scan1024(c, lds, &tot1);
  const int to = block_scan1024((c + tile - 1) / tile, lds, &tot2);
  if (e < E) {
    offsets[e] = o;
    tile_offsets[e] = to;
  }
  if (e == 0) {
    offsets[E] = tot1;
    tile_offsets[E] = tot2;
  }
}

// Rows of expert e: its member tokens in ascending order, at offsets[e].
// One 256-thread workgroup per (chunk, expert), 16 consecutive tokens (one
// 16-byte mask load) per thread; the chunk's first row is offsets[e] plus the
// counts of the expert's earlier chunks, so a heavy expert's tokens spread
// over as many workgroups as it has chunks.  rowmap[e][t] = row of (e, t).
__global__ void __launch_bounds__(256)
k_compact(const uint8_t* __restrict__ mask, int mpitch, const int32_t* __restrict__ chunk_cnt, int nch,
          const int32_t* __restrict__ offsets, int32_t* __restrict__ row_token, int32_t* __restrict__ row_expert,
          int32_t* __restrict__ rowmap) {
  __shared__ int sh[8];
  const int c = blockIdx.x, e = blockIdx.y;
  int base = offsets[e];
  for (int i = 0; i < c; ++i) base += chunk_cnt[(size_t)e * nch + i];
  const int t0 = c * CHUNK + threadIdx.x * 16;
  uint4 u = make_uint4(0, 0, 0, 0);
  if (t0 < mpitch) u = *reinterpret_cast<const uint4*>(mask + (size_t)e * mpitch + t0);
  const int cnt = __popc(u.x) + __popc(u.y) + __popc(u.z) + __popc(u.w);
  int tot;
  int row = base + block_scan256(cnt, sh, &tot);
  if (cnt == 0) return;
  int32_t* rm = rowmap + (size_t)e * mpitch;
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if ((w[i >> 2] >> (8 * (i & 3))) & 0xffu) {
      const int t = t0 + i;
      row_token[row] = t;
      row_expert[row] = e;
      rm[t] = row;
      ++row;
    }
  }
}

// Plain top-K: each token's rows are its K slots sorted by expert id; the
// row gate is the slot's top-K gate.  For K <= 16 one thread per (token,
// slot): the slot lands at its rank among the token's slots (the number of
// slots with a smaller expert id; ids are distinct).  (One thread per token
// left only two waves per CU for this latency-bound lookup: 12 us at
// T = 32768, K = 8.)
__global__ void __launch_bounds__(256)
k_tok_fill_slots(const int32_t* __restrict__ topk_idx, const float* __restrict__ topk_gate,
                 const int32_t* __restrict__ rowmap, int mpitch, int T, int K,
                 int32_t* __restrict__ tok_row, float* __restrict__ row_gate) {
  const long long q = (long long)blockIdx.x * 256 + threadIdx.x;
  if (q >= (long long)T * K) return;
  const int t = (int)(q / K), j = (int)(q % K);
  const int32_t* idx = topk_idx + (size_t)t * K;
  const int e = idx[j];
  int pos = 0;
#pragma unroll
  for (int k = 0; k < 16; ++k)
    if (k < K) pos += idx[k] < e ? 1 : 0;
  const int row = rowmap[(size_t)e * mpitch + t];
  tok_row[(size_t)t * K + pos] = row;
  row_gate[row] = topk_gate[q];
}

// Same for K > 16: one thread per token, a selection pass per position.
__global__ void __launch_bounds__(256)
k_tok_fill_topk(const int32_t* __restrict__ topk_idx, const float* __restrict__ topk_gate,
                const int32_t* __restrict__ rowmap, int mpitch, int T, int K,
                int32_t* __restrict__ tok_row, float* __restrict__ row_gate) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  const int32_t* idx = topk_idx + (size_t)t * K;
  const float* g = topk_gate + (size_t)t * K;
  int32_t* out = tok_row + (size_t)t * K;
  int prev = -1;
  for (int j = 0; j < K; ++j) {
    int best = 0x7fffffff, bk = 0;
    for (int k = 0; k < K; ++k) {
      const int e = idx[k];
      if (e > prev && e < best) { best = e; bk = k; }
    }
    const int row = rowmap[(size_t)best * mpitch + t];
    out[j] = row;
    row_gate[row] = g[bk];
    prev = best;
  }
}

// Per-token passes over the final membership (token rounding only).  A
// workgroup takes 64 tokens (one per lane) with TOK_SLICES waves; wave s
// takes the contiguous expert range [s*ceil(E/S), (s+1)*ceil(E/S)), so the
// waves' results in wave order follow ascending expert id.  Sixteen waves
// per 64 tokens keep each lane's chain of membership loads short (E / 16
// experts) and the chip full (T = 32768: 8192 waves).
constexpr int TOK_SLICES = 16;
struct TokSlice {
  int lo, hi;
};
__device__ __forceinline__ TokSlice tok_slice(int E, int s) {
  const int q = (E + TOK_SLICES - 1) / TOK_SLICES;
  const int lo = min(E, s * q);
  return TokSlice{lo, min(E, lo + q)};
}

// tstat[t], tstat[T + t] = max and sum of exp(score - max) over token t's
// final expert set (the set softmax); blksum[b] = rows of the workgroup's 64
// tokens.
__global__ void __launch_bounds__(64 * TOK_SLICES)
k_tok_stats(const uint8_t* __restrict__ mask, int mpitch, const float* __restrict__ scoresT, int T, int E,
            float* __restrict__ tstat, int32_t* __restrict__ blksum) {
  __shared__ float smx[TOK_SLICES][64], ssum[TOK_SLICES][64];
  __shared__ int scnt[TOK_SLICES][64];
  const int lane = threadIdx.x & 63, s = threadIdx.x >> 6;
  const int t = blockIdx.x * 64 + lane;
  const TokSlice sl = tok_slice(E, s);
  int cnt = 0;
  float mx = -INFINITY, sum = 0.f;
  if (t < T) {
#pragma unroll 8
    for (int e = sl.lo; e < sl.hi; ++e) {
      if (mask[(size_t)e * mpitch + t]) {
        const float z = scoresT[(size_t)e * mpitch + t];
        ++cnt;
        if (z > mx) {
          sum = sum * __expf(mx - z) + 1.f;
          mx = z;
        } else {
          sum += __expf(z - mx);
        }
      }
    }
  }
  smx[s][lane] = mx;
  ssum[s][lane] = sum;
  scnt[s][lane] = cnt;
  __syncthreads();
  if (s != 0) return;
  float M = smx[0][lane];
  int C = scnt[0][lane];
  for (int j = 1; j < TOK_SLICES; ++j) {
    M = fmaxf(M, smx[j][lane]);
    C += scnt[j][lane];
  }
  // rows of the workgroup's 64 tokens, for the scan of block sums
  int bsum = C;
  for (int o = 32; o >= 1; o >>= 1) bsum += __shfl_xor(bsum, o, 64);
  if (lane == 0) blksum[blockIdx.x] = bsum;
  if (t >= T) return;
  float S = 0.f;
  for (int j = 0; j < TOK_SLICES; ++j)
    if (scnt[j][lane]) S += ssum[j][lane] * __expf(smx[j][lane] - M);
  tstat[t] = M;
  tstat[(size_t)T + t] = S;
}

// out[0..n] = exclusive scan of cnt[0..n-1] (out[n] = the total): one
// 1024-thread block, each sweep taking 16384 consecutive counts, 16 per
// thread, read and written as four 16-byte words (both arrays are 16-byte
// aligned; a partial last group of a sweep goes element by element).  With
// token rounding it scans the rows of the 64-token blocks.
__global__ void __launch_bounds__(1024)
k_tok_scan(const int32_t* __restrict__ cnt, int T, int32_t* __restrict__ out) {
  __shared__ int lds[16];
  constexpr int PER = 16;
  int carry = 0;
  for (int base = 0; base < T; base += 1024 * PER) {
    const int t0 = base + threadIdx.x * PER;
    const bool whole = t0 + PER <= T;
    int v[PER];
    if (whole) {
#pragma unroll
      for (int q = 0; q < PER / 4; ++q) {
        const int4 u = *reinterpret_cast<const int4*>(cnt + t0 + 4 * q);
        v[4 * q] = u.x; v[4 * q + 1] = u.y; v[4 * q + 2] = u.z; v[4 * q + 3] = u.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < PER; ++j) v[j] = t0 + j < T ? cnt[t0 + j] : 0;
    }
    int sum = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) sum += v[j];
    int tot;
    int run = carry + block_scan1024(sum, lds, &tot);
    int o[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      o[j] = run;
      run += v[j];
    }
    if (whole) {
#pragma unroll
      for (int q = 0; q < PER / 4; ++q)
        *reinterpret_cast<int4*>(out + t0 + 4 * q) = make_int4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
    } else {
#pragma unroll
      for (int j = 0; j < PER; ++j)
        if (t0 + j < T) out[t0 + j] = o[j];
    }
    carry += tot;
  }
  if (threadIdx.x == 0) out[T] = carry;
}

// Token rounding: per token, its rows in ascending expert order and each
// row's gate, the softmax of the token's scores over its final set; and
// tok_ptr, from the scanned block sums (blkoff) and an in-wave scan.
__global__ void __launch_bounds__(64 * TOK_SLICES)
k_tok_fill(const uint8_t* __restrict__ mask, int mpitch, const int32_t* __restrict__ rowmap,
           const float* __restrict__ scoresT, const float* __restrict__ tstat,
           const int32_t* __restrict__ blkoff, int T, int E, int32_t* __restrict__ tok_ptr,
           int32_t* __restrict__ tok_row, float* __restrict__ row_gate) {
  __shared__ int scnt[TOK_SLICES][64];
  const int lane = threadIdx.x & 63, s = threadIdx.x >> 6;
  const int t = blockIdx.x * 64 + lane;
  const TokSlice sl = tok_slice(E, s);
  int cnt = 0;
  if (t < T) {
#pragma unroll 8
    for (int e = sl.lo; e < sl.hi; ++e) cnt += mask[(size_t)e * mpitch + t];
  }
  scnt[s][lane] = cnt;
  __syncthreads();
  // the token's first row: its block's offset plus the rows of the block's
  // earlier tokens (an exclusive scan over the wave's lanes, one per token)
  int before = 0, C = 0;
  for (int q = 0; q < TOK_SLICES; ++q) {
    const int v = scnt[q][lane];
    C += v;
    if (q < s) before += v;
  }
  int incl = C;
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  const int first = blkoff[blockIdx.x] + incl - C;
  if (s == 0 && t < T) tok_ptr[t] = first;
  if (s == 0 && t == T - 1) tok_ptr[T] = first + C;
  if (t >= T || cnt == 0) return;
  int j = first + before;
  const float mx = tstat[t], inv = 1.f / tstat[(size_t)T + t];
  for (int e = sl.lo; e < sl.hi; ++e) {
    if (mask[(size_t)e * mpitch + t]) {
      const int row = rowmap[(size_t)e * mpitch + t];
      tok_row[j++] = row;
      row_gate[row] = __expf(scoresT[(size_t)e * mpitch + t] - mx) * inv;
    }
  }
}

}  // namespace

// Clears n16 16-byte words.  The membership bytes are cleared by a kernel
// rather than a runtime memset, so that the routing launch sequence can be
// captured into a HIP graph and replayed.
static __global__ void k_zero16(uint4* __restrict__ p, long long n16) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

int mask_pitch(int T) { return (T + 15) / 16 * 16; }
int route_chunks(int T) { return (mask_pitch(T) + CHUNK - 1) / CHUNK; }

hipError_t launch_route_select(const RouteBufs& rb, const RouteScratch& sc, int T, int E, int K,
                               int tile, int round_mode, uint64_t round_seed, hipStream_t st) {
  hipError_t err;
  const int mp = mask_pitch(T);
  {
    const long long n16 = (long long)E * mp / 16;  // mp is a multiple of 16
    const long long blocks = std::min<long long>((n16 + 255) / 256, 4096);
    hipLaunchKernelGGL(k_zero16, dim3((unsigned)blocks), dim3(256), 0, st, reinterpret_cast<uint4*>(sc.mask), n16);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  int32_t* fixed_ptr = round_mode == 0 ? rb.tok_ptr : nullptr;
  auto topk = [&](auto kern, int G) {
    const long long threads = (long long)T * G;
    hipLaunchKernelGGL(kern, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, rb.logits, T, E, K, mp,
                       rb.topk_idx, rb.topk_gate, sc.mask, fixed_ptr);
  };
  if (E <= 128) topk(k_topk<16, 8>, 16);
  else if (E <= 256) topk(k_topk<16, 16>, 16);
  else if (E <= 512) topk(k_topk<32, 16>, 32);
  else topk(k_topk<32, 32>, 32);
  const int nch = route_chunks(T);
  const dim3 cgrid((unsigned)nch, (unsigned)E);
  // membership counts per chunk (with rounding, the rounding kernel rewrites
  // those of the experts it changes)
  hipLaunchKernelGGL(k_chunk_count, cgrid, dim3(256), 0, st, sc.mask, mp, nch, sc.chunk_cnt);
  if (round_mode != 0) {
    hipLaunchKernelGGL(k_transpose_scores, dim3((T + 31) / 32, (E + 31) / 32), dim3(256), 0, st,
                       rb.logits, T, E, mp, sc.scoresT);
    if (mp <= TR_LDS_TOKENS) {
      static const hipError_t attr =
          hipFuncSetAttribute(reinterpret_cast<const void*>(k_token_round<true>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, TR_LDS_TOKENS * 4);
      if (attr != hipSuccess) return attr;
      hipLaunchKernelGGL(k_token_round<true>, dim3(E), dim3(TR_THREADS), (size_t)mp * 4, st, sc.scoresT, sc.mask, mp,
                         sc.chunk_cnt, nch, rb.counts_raw, T, tile, round_mode, round_seed);
    } else {
      hipLaunchKernelGGL(k_token_round<false>, dim3(E), dim3(TR_THREADS), 0, st, sc.scoresT, sc.mask, mp,
                         sc.chunk_cnt, nch, rb.counts_raw, T, tile, round_mode, round_seed);
    }
  }
  hipLaunchKernelGGL(k_scan_experts, dim3(1), dim3(1024), 0, st, sc.chunk_cnt, nch, E, tile, rb.counts,
                     round_mode == 0 ? rb.counts_raw : (int32_t*)nullptr, rb.offsets, rb.tile_offsets);
  hipLaunchKernelGGL(k_compact, cgrid, dim3(256), 0, st, sc.mask, mp, sc.chunk_cnt, nch, rb.offsets, rb.row_token,
                     rb.row_expert, sc.rowmap);
  if (round_mode == 0) {
    if (K <= 16)
      hipLaunchKernelGGL(k_tok_fill_slots, dim3((unsigned)(((long long)T * K + 255) / 256)), dim3(256), 0, st,
                         rb.topk_idx, rb.topk_gate, sc.rowmap, mp, T, K, rb.tok_row, rb.row_gate);
    else
      hipLaunchKernelGGL(k_tok_fill_topk, dim3((T + 255) / 256), dim3(256), 0, st, rb.topk_idx, rb.topk_gate,
                         sc.rowmap, mp, T, K, rb.tok_row, rb.row_gate);
  } else {
    const unsigned blocks = (unsigned)((T + 63) / 64);
    int32_t* blksum = sc.tblk;                           // [blocks], then the scanned offsets [blocks + 1]
    int32_t* blkoff = blksum + ((blocks + 3) / 4) * 4;
    hipLaunchKernelGGL(k_tok_stats, dim3(blocks), dim3(64 * TOK_SLICES), 0, st, sc.mask, mp, sc.scoresT, T, E,
                       sc.tstat, blksum);
    hipLaunchKernelGGL(k_tok_scan, dim3(1), dim3(1024), 0, st, blksum, (int)blocks, blkoff);
    hipLaunchKernelGGL(k_tok_fill, dim3(blocks), dim3(64 * TOK_SLICES), 0, st, sc.mask, mp, sc.rowmap,
                       sc.scoresT, sc.tstat, blkoff, T, E, rb.tok_ptr, rb.tok_row, rb.row_gate);
  }
  return hipGetLastError();
}

}  // namespace moe
