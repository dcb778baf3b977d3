// Sampler run by one wavefront: turns one request's logits (in LDS) into a
// code.  Mizuoto "Fish Speech" engine page, "as upstream": a draw is
// argmax(probs / -log u) and top-k is fixed at 30; the order of the steps,
// tie rules and float formats are the reading documented with the oracle:
//   greedy when T <= 0 (or NaN): argmax, lowest index on ties;
//   candidates: the n = clamp(top_k, 1, min(V, 64)) largest logits ordered by
//   (value desc, index asc); z = l / T; e_j = f32(exp(f64(z_j - z_0)));
//   S = sequential f32 sum in rank order; p_j = e_j / S; running f32 sums
//   c_j; keep ranks 0..m with m the first j where c_j >= top_p (else n-1);
//   u_j = (floor(splitmix64(bits(u) << 32 | j) / 2^40) + 0.5) * 2^-24 (f64),
//   E_j = f32(-log(u_j)); code = kept candidate with the largest f32
//   p_j / E_j, lowest rank on ties.
#pragma once
#include "device_common.h"

namespace s2f {

// (v, i) sorts before (w, k) when v is larger, or equal with a lower index.
__device__ __forceinline__ bool key_before(float v, int i, float w, int k) {
  return v > w || (v == w && i < k);
}

// Bitonic sort of one (value, index) pair per lane into rank order
// (lane 0 = first).
__device__ __forceinline__ void wave_sort_desc(float& v, int& i) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      float ov = __shfl_xor(v, j, 64);
      int oi = __shfl_xor(i, j, 64);
      bool up = (lane & k) == 0;          // this k-block is sorted "first to last"
      bool lower = (lane & j) == 0;       // this lane holds the lower position of the pair
      bool mine_first = key_before(v, i, ov, oi);
      bool keep_mine = (lower == up) ? mine_first : !mine_first;
      if (!keep_mine) { v = ov; i = oi; }
    }
  }
}

// Wave-wide argmax by (value desc, index asc); returns the winner in all lanes.
__device__ __forceinline__ void wave_best(float& v, int& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float ov = __shfl_xor(v, o, 64);
    int oi = __shfl_xor(i, o, 64);
    if (key_before(ov, oi, v, i)) { v = ov; i = oi; }
  }
}

// Exclusive prefix sum across the wave.
__device__ __forceinline__ int wave_excl_scan(int x) {
  const int lane = threadIdx.x & 63;
  int incl = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  return incl - x;
}

// L: logits in LDS [V].  cval/cidx: LDS scratch [64]; mark: LDS scratch
// [ceil(V/32)] words (used only when more than 64 values tie around the
// top-k threshold).  Must be called by all 64 lanes of one wave.
__device__ int sample_wave(const float* L, int V, float T, float top_p, int top_k, float u,
                           float* cval, int* cidx, u32* mark) {
  const int lane = threadIdx.x & 63;
  constexpr int BIG = 0x7FFFFFFF;
  if (!(T > 0.0f)) {
    float bv = -INFINITY; int bi = BIG;
    for (int i = lane; i < V; i += 64) {
      float x = L[i];
      if (key_before(x, i, bv, bi)) { bv = x; bi = i; }
    }
    wave_best(bv, bi);
    return bi < V ? bi : 0;
  }
  const int n = max(1, min(top_k, min(V, TOPK_MAX)));
  // 1. each lane's best element; the n-th best lane maximum bounds the top-n from below
  float mv = -INFINITY; int mi = BIG;
  for (int i = lane; i < V; i += 64) {
    float x = L[i];
    if (key_before(x, i, mv, mi)) { mv = x; mi = i; }
  }
  float sv = mv; int si = mi;
  wave_sort_desc(sv, si);
  const float t = __shfl(sv, n - 1, 64);
  // 2. candidates: every value >= t (a superset of the top n).  While more
  //    than 64 values pass, raise t by bisection between t and the maximum,
  //    keeping at least n values at or above it.
  float t_lo = t;
  int total = 0;
  {
    int cnt = 0;
    for (int i = lane; i < V; i += 64) cnt += (L[i] >= t_lo) ? 1 : 0;
    total = wave_sum_i(cnt);
    float t_hi = __shfl(sv, 0, 64);          // the maximum
    for (int round = 0; round < 32 && total > 64; ++round) {
      const float mid = t_lo + 0.5f * (t_hi - t_lo);
      if (!(mid > t_lo) || !(mid < t_hi)) break;   // no representable value in between
      int c2 = 0;
      for (int i = lane; i < V; i += 64) c2 += (L[i] >= mid) ? 1 : 0;
      const int tot2 = wave_sum_i(c2);
      if (tot2 >= n) { t_lo = mid; total = tot2; }
      else t_hi = mid;
    }
  }
  int cnt = 0;
  for (int i = lane; i < V; i += 64) cnt += (L[i] >= t_lo) ? 1 : 0;
  float cv; int ci;
  if (total <= 64) {
    int off = wave_excl_scan(cnt);
    for (int i = lane; i < V; i += 64) {
      float x = L[i];
      if (x >= t_lo) { cval[off] = x; cidx[off] = i; ++off; }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    cv = lane < total ? cval[lane] : -INFINITY;
    ci = lane < total ? cidx[lane] : BIG;
    wave_sort_desc(cv, ci);
  } else {
    // many ties around the threshold: n rounds of exact selection
    const int words = (V + 31) >> 5;
    for (int w = lane; w < words; w += 64) mark[w] = 0u;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    cv = -INFINITY; ci = BIG;
    for (int r = 0; r < n; ++r) {
      float bv = -INFINITY; int bi = BIG;
      for (int i = lane; i < V; i += 64) {
        if ((mark[i >> 5] >> (i & 31)) & 1u) continue;
        float x = L[i];
        if (key_before(x, i, bv, bi)) { bv = x; bi = i; }
      }
      wave_best(bv, bi);
      if (lane == r) { cv = bv; ci = bi; }
      if (lane == 0 && bi < V) mark[bi >> 5] |= 1u << (bi & 31);
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    }
  }
  // 3. lane j < n holds the rank-j candidate
  const bool act = lane < n;
  const float z = act ? cv / T : 0.0f;
  const float z0 = __shfl(z, 0, 64);
  const float d = z - z0;
  const float e = act ? (float)exp((double)d) : 0.0f;
  float S = 0.0f;
  for (int j = 0; j < n; ++j) S += __shfl(e, j, 64);
  const float p = act ? e / S : 0.0f;
  float c = 0.0f, my_c = 0.0f;
  for (int j = 0; j < n; ++j) {
    c += __shfl(p, j, 64);
    if (lane == j) my_c = c;
  }
  const u64 ge = __ballot(act && my_c >= top_p);
  const int m = ge ? (__ffsll((long long)ge) - 1) : (n - 1);
  // 4. exponential race over the kept ranks 0..m
  const u64 h = splitmix64(((u64)__float_as_uint(u) << 32) + (u64)lane);
  const double uj = ((double)(h >> 40) + 0.5) * (1.0 / 16777216.0);
  const float E = (float)(-log(uj));
  float key = (lane <= m) ? p / E : -INFINITY;
  int kl = lane;
  wave_best(key, kl);
  return __shfl(ci, kl, 64);
}

}  // namespace s2f
