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

// a beats b: larger score, equal scores -> smaller expert id.
__device__ __forceinline__ bool beats(float av, int ae, float bv, int be) {
  return av > bv || (av == bv && ae < be);
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

// G lanes per token (G = 16 or 64): K rounds of an arg-max over the token's
// scores held E/G per lane.  Writes the slot-ordered experts, their softmax
// gates and the membership bytes; with fixed_ptr also tok_ptr[t] = t*K (every
// token keeps exactly K rows when there is no token rounding).  Slot k's score
// is kept by lane k % G of the group.
template <int G>
__global__ void __launch_bounds__(256)
k_topk(const float* __restrict__ scores, int T, int E, int K, int mpitch, int32_t* __restrict__ topk_idx,
       float* __restrict__ topk_gate, uint8_t* __restrict__ mask, int32_t* __restrict__ tok_ptr) {
  constexpr int MAXV = 16;  // E <= 16 * G
  const int lane = threadIdx.x & (G - 1);
  const int t = (blockIdx.x * 256 + threadIdx.x) / G;
  const bool live = t < T;  // groups never straddle a wave, so shuffles stay inside live groups
  const float* z = scores + (size_t)(live ? t : 0) * E;
  float v[MAXV], zs[MAXV];
  uint32_t taken = 0;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int e = lane + G * i;
    const bool ok = live && e < E;
    v[i] = ok ? z[e] : 0.f;
    zs[i] = 0.f;
    if (!ok) taken |= 1u << i;
  }
  for (int k = 0; k < K; ++k) {
    float bv = 0.f;
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
      if (!(taken & (1u << i))) {
        const int e = lane + G * i;
        if (be == 0x7fffffff || beats(v[i], e, bv, be)) { bv = v[i]; be = e; }
      }
    }
#pragma unroll
    for (int o = G / 2; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oe = __shfl_xor(be, o, 64);
      if (oe != 0x7fffffff && (be == 0x7fffffff || beats(ov, oe, bv, be))) { bv = ov; be = oe; }
    }
    if (live && (be & (G - 1)) == lane) taken |= 1u << (be / G);
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

// counts[e] = number of member tokens of expert e (one workgroup per expert;
// mask rows are 16-byte aligned and zero past T).
__global__ void __launch_bounds__(256)
k_expert_count(const uint8_t* __restrict__ mask, int mpitch, int32_t* __restrict__ counts,
               int32_t* __restrict__ counts2) {
  __shared__ int lds[8];
  const int e = blockIdx.x;
  const uint4* m = reinterpret_cast<const uint4*>(mask + (size_t)e * mpitch);
  int c = 0;
  for (int i = threadIdx.x; i < mpitch / 16; i += 256) {
    const uint4 u = m[i];
    // each byte is 0 or 1: the byte sum of a word is its popcount
    c += __popc(u.x) + __popc(u.y) + __popc(u.z) + __popc(u.w);
  }
  int total;
  block_scan256(c, lds, &total);
  if (threadIdx.x == 0) {
    counts[e] = total;
    if (counts2) counts2[e] = total;
  }
}

// scores [T][E] -> scoresT [E][T]
__global__ void k_transpose_scores(const float* __restrict__ in, int T, int E, float* __restrict__ out) {
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
    if (t < T && e < E) out[(size_t)e * T + t] = tile[tx][r];
  }
}

// Token rounding of one expert per workgroup.  c = plain count; r = rounded
// count.  r < c: keep the r best-ranked routed tokens; r > c: add the r - c
// best-ranked tokens not routed to this expert.  Rank: score descending, then
// token id ascending.  The threshold score is found by an MSB-first radix
// select over the order-preserving score keys; equal-key candidates are then
// taken in ascending token order.
__global__ void __launch_bounds__(256)
k_token_round(const float* __restrict__ scoresT, uint8_t* __restrict__ mask, int mpitch,
              const int32_t* __restrict__ counts_raw, int T, int M, int mode, uint64_t seed) {
  __shared__ int hist[256];
  __shared__ int sh[8];
  const int e = blockIdx.x;
  const int c = counts_raw[e];
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
  const uint8_t want = drop ? 1 : 0;         // candidates: routed (drop) or not (add)
  const int k_sel = drop ? r : r - c;        // candidates to select
  uint8_t* m = mask + (size_t)e * mpitch;
  const float* z = scoresT + (size_t)e * T;

  uint32_t prefix = 0, pmask = 0;
  int kk = k_sel;
  if (k_sel > 0) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = threadIdx.x; i < 256; i += 256) hist[i] = 0;
      __syncthreads();
      for (int t = threadIdx.x; t < T; t += 256) {
        if (m[t] == want) {
          uint32_t key = score_key(z[t]);
          if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255], 1);
        }
      }
      __syncthreads();
      if (threadIdx.x == 0) {
        int above = 0, dsel = 0;
        for (int dgt = 255; dgt >= 0; --dgt) {
          if (above + hist[dgt] >= kk) { dsel = dgt; break; }
          above += hist[dgt];
        }
        sh[0] = dsel;
        sh[1] = kk - above;
      }
      __syncthreads();
      prefix |= (uint32_t)sh[0] << shift;
      pmask |= 0xffu << shift;
      kk = sh[1];
      __syncthreads();
    }
  }
  // prefix = threshold key; kk = how many equal-key candidates to take
  int carry = 0;
  for (int base = 0; base < T; base += 256) {
    const int t = base + threadIdx.x;
    bool cand = false, gt = false, eq = false;
    if (t < T) {
      cand = m[t] == want;
      if (cand && k_sel > 0) {
        uint32_t key = score_key(z[t]);
        gt = key > prefix;
        eq = key == prefix;
      }
    }
    int tot;
    const int rank = block_scan256(eq ? 1 : 0, sh, &tot);
    const bool sel = gt || (eq && carry + rank < kk);
    if (t < T && cand) {
      if (drop && !sel) m[t] = 0;
      if (!drop && sel) m[t] = 1;
    }
    carry += tot;
  }
}

// offsets / tile_offsets: exclusive scans of counts and ceil(counts / tile).
__global__ void __launch_bounds__(1024)
k_scan_experts(const int32_t* __restrict__ counts, int E, int tile, int32_t* __restrict__ offsets,
               int32_t* __restrict__ tile_offsets) {
  __shared__ int lds[16];
  const int e = threadIdx.x;
  const int c = e < E ? counts[e] : 0;
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
// Each thread takes 16 consecutive tokens (one 16-byte mask load) per sweep.
// rowmap[e][t] = row of (e, t); tokcnt (token rounding only) counts rows per
// token.
__global__ void __launch_bounds__(256)
k_compact(const uint8_t* __restrict__ mask, int mpitch, const int32_t* __restrict__ offsets, int T,
          int32_t* __restrict__ row_token, int32_t* __restrict__ row_expert,
          int32_t* __restrict__ rowmap, int32_t* __restrict__ tokcnt) {
  __shared__ int sh[8];
  const int e = blockIdx.x;
  const uint8_t* m = mask + (size_t)e * mpitch;
  int32_t* rm = rowmap + (size_t)e * mpitch;
  int carry = offsets[e];
  for (int base = 0; base < mpitch; base += 256 * 16) {
    const int t0 = base + threadIdx.x * 16;
    uint4 u = make_uint4(0, 0, 0, 0);
    if (t0 < mpitch) u = *reinterpret_cast<const uint4*>(m + t0);
    const int cnt = __popc(u.x) + __popc(u.y) + __popc(u.z) + __popc(u.w);
    int tot;
    int row = carry + block_scan256(cnt, sh, &tot);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if ((w[i >> 2] >> (8 * (i & 3))) & 0xffu) {
        const int t = t0 + i;
        row_token[row] = t;
        row_expert[row] = e;
        rm[t] = row;
        if (tokcnt) atomicAdd(&tokcnt[t], 1);
        ++row;
      }
    }
    carry += tot;
  }
}

// Plain top-K: each token's rows are its K slots sorted by expert id; the
// row gate is the slot's top-K gate.
__global__ void __launch_bounds__(256)
k_tok_fill_topk(const int32_t* __restrict__ topk_idx, const float* __restrict__ topk_gate,
                const int32_t* __restrict__ rowmap, int mpitch, int T, int K,
                int32_t* __restrict__ tok_row, float* __restrict__ row_gate) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  const int32_t* idx = topk_idx + (size_t)t * K;
  const float* g = topk_gate + (size_t)t * K;
  int32_t* out = tok_row + (size_t)t * K;
  // selection sort by expert id; K is small (<= E) and ids are distinct
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

// tok_ptr = exclusive scan of per-token row counts (one 1024-thread block,
// each thread a contiguous run of tokens).
__global__ void __launch_bounds__(1024)
k_tok_scan(const int32_t* __restrict__ tokcnt, int T, int32_t* __restrict__ tok_ptr) {
  __shared__ int lds[16];
  const int per = (T + 1023) / 1024;
  const int t0 = threadIdx.x * per;
  int s = 0;
  for (int i = 0; i < per; ++i)
    if (t0 + i < T) s += tokcnt[t0 + i];
  int tot;
  int run = block_scan1024(s, lds, &tot);
  for (int i = 0; i < per; ++i)
    if (t0 + i < T) {
      tok_ptr[t0 + i] = run;
      run += tokcnt[t0 + i];
    }
  if (threadIdx.x == 0) tok_ptr[T] = tot;
}

// Token rounding: per token, its rows in ascending expert order and each
// row's gate, the softmax of the token's scores over its final set.
__global__ void __launch_bounds__(256)
k_tok_fill(const uint8_t* __restrict__ mask, int mpitch, const int32_t* __restrict__ rowmap,
           const float* __restrict__ scores, const int32_t* __restrict__ tok_ptr, int T, int E,
           int32_t* __restrict__ tok_row, float* __restrict__ row_gate) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  const float* z = scores + (size_t)t * E;
  float mx = -INFINITY;
  for (int e = 0; e < E; ++e)
    if (mask[(size_t)e * mpitch + t]) mx = fmaxf(mx, z[e]);
  float sum = 0.f;
  for (int e = 0; e < E; ++e)
    if (mask[(size_t)e * mpitch + t]) sum += __expf(z[e] - mx);
  int j = tok_ptr[t];
  for (int e = 0; e < E; ++e)
    if (mask[(size_t)e * mpitch + t]) {
      const int row = rowmap[(size_t)e * mpitch + t];
      tok_row[j++] = row;
      row_gate[row] = __expf(z[e] - mx) / sum;
    }
}

}  // namespace

int mask_pitch(int T) { return (T + 15) / 16 * 16; }

hipError_t launch_route_select(const RouteBufs& rb, const RouteScratch& sc, int T, int E, int K,
                               int tile, int round_mode, uint64_t round_seed, hipStream_t st) {
  hipError_t err;
  const int mp = mask_pitch(T);
  if ((err = hipMemsetAsync(sc.mask, 0, (size_t)E * mp, st)) != hipSuccess) return err;
  int32_t* fixed_ptr = round_mode == 0 ? rb.tok_ptr : nullptr;
  if (E <= 256) {
    const long long threads = (long long)T * 16;
    hipLaunchKernelGGL(k_topk<16>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, rb.logits, T, E,
                       K, mp, rb.topk_idx, rb.topk_gate, sc.mask, fixed_ptr);
  } else {
    const long long threads = (long long)T * 64;
    hipLaunchKernelGGL(k_topk<64>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, rb.logits, T, E,
                       K, mp, rb.topk_idx, rb.topk_gate, sc.mask, fixed_ptr);
  }
  if (round_mode == 0) {
    hipLaunchKernelGGL(k_expert_count, dim3(E), dim3(256), 0, st, sc.mask, mp, rb.counts_raw, rb.counts);
  } else {
    hipLaunchKernelGGL(k_expert_count, dim3(E), dim3(256), 0, st, sc.mask, mp, rb.counts_raw,
                       (int32_t*)nullptr);
    hipLaunchKernelGGL(k_transpose_scores, dim3((T + 31) / 32, (E + 31) / 32), dim3(256), 0, st,
                       rb.logits, T, E, sc.scoresT);
    hipLaunchKernelGGL(k_token_round, dim3(E), dim3(256), 0, st, sc.scoresT, sc.mask, mp, rb.counts_raw,
                       T, tile, round_mode, round_seed);
    hipLaunchKernelGGL(k_expert_count, dim3(E), dim3(256), 0, st, sc.mask, mp, rb.counts,
                       (int32_t*)nullptr);
  }
  hipLaunchKernelGGL(k_scan_experts, dim3(1), dim3(1024), 0, st, rb.counts, E, tile, rb.offsets,
                     rb.tile_offsets);
  if (round_mode == 0) {
    hipLaunchKernelGGL(k_compact, dim3(E), dim3(256), 0, st, sc.mask, mp, rb.offsets, T, rb.row_token,
                       rb.row_expert, sc.rowmap, (int32_t*)nullptr);
    hipLaunchKernelGGL(k_tok_fill_topk, dim3((T + 255) / 256), dim3(256), 0, st, rb.topk_idx, rb.topk_gate,
                       sc.rowmap, mp, T, K, rb.tok_row, rb.row_gate);
  } else {
    if ((err = hipMemsetAsync(sc.tokcnt, 0, (size_t)T * sizeof(int32_t), st)) != hipSuccess) return err;
    hipLaunchKernelGGL(k_compact, dim3(E), dim3(256), 0, st, sc.mask, mp, rb.offsets, T, rb.row_token,
                       rb.row_expert, sc.rowmap, sc.tokcnt);
    hipLaunchKernelGGL(k_tok_scan, dim3(1), dim3(1024), 0, st, sc.tokcnt, T, rb.tok_ptr);
    hipLaunchKernelGGL(k_tok_fill, dim3((T + 255) / 256), dim3(256), 0, st, sc.mask, mp, sc.rowmap, rb.logits,
                       rb.tok_ptr, T, E, rb.tok_row, rb.row_gate);
  }
  return hipGetLastError();
}

}  // namespace moe
