// Sampler: turns one request's logits into a code.  Mizuoto "Fish Speech"
// engine page, section "What matches upstream": a draw is argmax(probs /
// -log u) and top-k is fixed at 30; the order of the steps, tie rules and
// float formats are the reading documented with the oracle:
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

// One compare-exchange step of the bitonic network: partner lane ^ J,
// this lane's k-block sorted first to last when (lane & K) == 0.
template <int K, int J>
__device__ __forceinline__ void bitonic_step(float& v, int& i, int lane) {
  const float ov = xor_lane_f<J>(v, lane);
  const int oi = xor_lane<J>(i, lane);
  const bool up = (lane & K) == 0;
  const bool lower = (lane & J) == 0;     // this lane holds the lower position of the pair
  const bool mine_first = key_before(v, i, ov, oi);
  const bool keep_mine = (lower == up) ? mine_first : !mine_first;
  v = keep_mine ? v : ov;
  i = keep_mine ? i : oi;
}

template <int K, int J>
__device__ __forceinline__ void bitonic_merge(float& v, int& i, int lane) {
  bitonic_step<K, J>(v, i, lane);
  if constexpr (J > 1) bitonic_merge<K, J / 2>(v, i, lane);
}

template <int K>
__device__ __forceinline__ void bitonic_sort(float& v, int& i, int lane) {
  if constexpr (K > 2) bitonic_sort<K / 2>(v, i, lane);
  bitonic_merge<K, K / 2>(v, i, lane);
}

// Bitonic sort of one (value, index) pair per lane into rank order
// (lane 0 = first).
__device__ __forceinline__ void wave_sort_desc(float& v, int& i, int lane) { bitonic_sort<64>(v, i, lane); }

template <int O>
__device__ __forceinline__ void best_step(float& v, int& i, int lane) {
  const float ov = xor_lane_f<O>(v, lane);
  const int oi = xor_lane<O>(i, lane);
  if (key_before(ov, oi, v, i)) { v = ov; i = oi; }
  if constexpr (O > 1) best_step<O / 2>(v, i, lane);
}

// Wave-wide argmax by (value desc, index asc); returns the winner in all lanes.
__device__ __forceinline__ void wave_best(float& v, int& i) {
  int lane;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
  best_step<32>(v, i, lane);
}

// ----------------------------------------------------------------- block
// The whole block (NTHREADS threads) samples one request.  Thread t holds
// logits t, t + NTHREADS, ... in registers (VPT of them, V <= VPT * NTHREADS).
constexpr int SAMP_TAU = 16;       // thresholds per search round: lo + (hi - lo) j / 16
constexpr int SAMP_ROUNDS = 8;     // search rounds before the exact fallback

// LDS scratch: cval/cidx [TOPK_MAX] candidates, red [2][NWAVE][SAMP_TAU]
// words for the cross-wave counts (two buffers, so one barrier per round).
struct SampScratch {
  float* cval;
  int* cidx;
  int* red;
};


// Threshold j of a search round over [lo, lo + d]; one explicit fma so that
// the counting pass and the decision after it agree on every bit.
__device__ __forceinline__ float samp_tau(float lo, float d, int j) {
  return __builtin_fmaf(d, (float)j * (1.0f / SAMP_TAU), lo);
}

// Block-wide best (value desc, index asc); every thread gets the winner.
// buf: NWAVE floats + NWAVE ints of LDS, not touched again before the next
// barrier by any thread.
__device__ __forceinline__ void block_best(float& v, int& i, int* buf, int tid) {
  const int w = tid >> 6, lane = tid & 63;
  wave_best(v, i);
  float* bf = reinterpret_cast<float*>(buf);
  if (lane == 0) { bf[w] = v; buf[NWAVE + w] = i; }
  __syncthreads();
  v = bf[0]; i = buf[NWAVE];
#pragma unroll
  for (int k = 1; k < NWAVE; ++k) {
    const float ov = bf[k];
    const int oi = buf[NWAVE + k];
    if (key_before(ov, oi, v, i)) { v = ov; i = oi; }
  }
}

// The request's V logits as plain floats in device memory (finite values).
struct PlainLogits {
  const float* L;
  template <int VPT>
  __device__ __forceinline__ void load(float (&x)[VPT], int tid, int V) const {
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int i = tid + j * NTHREADS;
      x[j] = (i < V) ? L[i] : -INFINITY;
    }
  }
};

// Returns the sampled code in every lane of wave 0 (other waves: undefined).
// src: the request's V logits (finite values); src.load gives thread t its
// logits t, t + NTHREADS, ... (-inf past V).
template <int VPT, typename Src>
__device__ __forceinline__ int sample_block(const Src& src, int V, float T, float top_p, int top_k, float u,
                                            const SampScratch& sc) {
  // The thread index goes through an opaque move so that nothing derived
  // from it (sort masks, hash offsets) is hoisted out of the caller's loops,
  // where it would stay live in registers across every other phase.
  int tid;
  asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"((int)threadIdx.x));
  const int lane = tid & 63, w = tid >> 6;
  constexpr int BIG = 0x7FFFFFFF;
  float x[VPT];
  src.load(x, tid, V);
  // The race's exponential of rank `lane` depends only on the uniform: for
  // plain logits it is computed while they are in flight.
  const u64 h = splitmix64(((u64)__float_as_uint(u) << 32) + (u64)lane);
  const double uj = ((double)(h >> 40) + 0.5) * (1.0 / 16777216.0);
  const float E = (float)(-log(uj));
  int buf = 0;
  if (!(T > 0.0f)) {                                   // greedy: argmax, lowest index on ties
    float bv = -INFINITY; int bi = BIG;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int i = tid + j * NTHREADS;
      if (i < V && key_before(x[j], i, bv, bi)) { bv = x[j]; bi = i; }
    }
    block_best(bv, bi, sc.red, tid);
    return bi < V ? bi : 0;
  }
  const int n = max(1, min(top_k, min(V, TOPK_MAX)));

  // 1. range of the logits
  float mx = -INFINITY, mn = INFINITY;
#pragma unroll
  for (int j = 0; j < VPT; ++j)
    if (tid + j * NTHREADS < V) { mx = fmaxf(mx, x[j]); mn = fminf(mn, x[j]); }
  mx = wave_max(mx);
  mn = wave_min(mn);
  {
    float* bf = reinterpret_cast<float*>(sc.red);
    if (lane == 0) { bf[w] = mx; bf[NWAVE + w] = mn; }
    __syncthreads();
    mx = bf[0]; mn = bf[NWAVE];
#pragma unroll
    for (int k = 1; k < NWAVE; ++k) { mx = fmaxf(mx, bf[k]); mn = fminf(mn, bf[NWAVE + k]); }
    buf = 1;
  }

  // 2. threshold search.  Invariant: cnt = #{x >= lo} >= n.  Each round counts
  //    the values at or above 15 evenly spaced thresholds in [lo, hi] and
  //    keeps the highest one that still passes n values, until at most
  //    TOPK_MAX values pass: those are a superset of the top n.
  float lo = mn, hi = mx;
  int cnt = V;
  const bool finite = __builtin_isfinite(lo) && __builtin_isfinite(hi);
  // Per-wave counts of the values >= lo, when the round that set lo left
  // them in a buffer no later round has overwritten (rounds alternate two
  // buffers): the compaction below then needs no counting pass of its own.
  const int* lo_counts = nullptr;
  int lo_j = 0, lo_round = -2, last_round = -1;
  for (int r = 0; r < SAMP_ROUNDS && finite && cnt > TOPK_MAX; ++r) {
    last_round = r;
    const float d = hi - lo;
    int* rb = sc.red + buf * (NWAVE * SAMP_TAU);
#pragma unroll
    for (int jt = 1; jt < SAMP_TAU; ++jt) {
      const float tau = samp_tau(lo, d, jt);
      int cj = 0;
#pragma unroll
      for (int j = 0; j < VPT; ++j) cj += __popcll(__ballot(x[j] >= tau));
      if (lane == 0) rb[w * SAMP_TAU + jt] = cj;      // wave-uniform count
    }
    __syncthreads();
    buf ^= 1;
    int tot = 0;
    if (lane < SAMP_TAU) {
#pragma unroll
      for (int k = 0; k < NWAVE; ++k) tot += rb[k * SAMP_TAU + lane];
    }
    const u64 ge = __ballot(lane >= 1 && lane < SAMP_TAU && tot >= n);
    const int jb = ge ? 63 - __clzll((long long)ge) : 0;   // counts fall with j: ge is 1..jb
    const float nlo = jb ? samp_tau(lo, d, jb) : lo;
    const float nhi = (jb + 1 < SAMP_TAU) ? samp_tau(lo, d, jb + 1) : hi;
    const int ncnt = jb ? __builtin_amdgcn_readlane(tot, jb) : cnt;
    if (!(nlo > lo) && !(nhi < hi)) break;                 // the interval no longer shrinks
    if (jb) { lo_counts = rb; lo_j = jb; lo_round = r; }
    lo = nlo; hi = nhi; cnt = ncnt;
  }
  if (last_round - lo_round > 1) lo_counts = nullptr;

  float cv = -INFINITY; int ci = BIG;                   // wave 0: lane j = rank j
  if (cnt <= TOPK_MAX) {
    // 3a. compact the cnt values >= lo into LDS, then sort them in wave 0
    int off = 0;
    if (lo_counts) {
      for (int k = 0; k < w; ++k) off += lo_counts[k * SAMP_TAU + lo_j];
    } else {
      int* rb = sc.red + buf * (NWAVE * SAMP_TAU);
      int wc = 0;
#pragma unroll
      for (int j = 0; j < VPT; ++j) wc += __popcll(__ballot(x[j] >= lo));
      if (lane == 0) rb[w] = wc;
      __syncthreads();
      for (int k = 0; k < w; ++k) off += rb[k];
    }
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const u64 b = __ballot(x[j] >= lo);
      if (x[j] >= lo) {
        const int pos = off + (int)__builtin_amdgcn_mbcnt_hi((u32)(b >> 32), __builtin_amdgcn_mbcnt_lo((u32)b, 0u));
        sc.cval[pos] = x[j];
        sc.cidx[pos] = tid + j * NTHREADS;
      }
      off += __popcll(b);
    }
    __syncthreads();
    if (w == 0) {
      cv = lane < cnt ? sc.cval[lane] : -INFINITY;
      ci = lane < cnt ? sc.cidx[lane] : BIG;
      wave_sort_desc(cv, ci, lane);
    }
  } else {
    // 3b. many ties around the threshold: n rounds of exact block-wide selection
    u32 taken = 0u;
    for (int r = 0; r < n; ++r) {
      float bv = -INFINITY; int bi = BIG;
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        const int i = tid + j * NTHREADS;
        if (i < V && !((taken >> j) & 1u) && key_before(x[j], i, bv, bi)) { bv = x[j]; bi = i; }
      }
      block_best(bv, bi, sc.red + buf * (NWAVE * SAMP_TAU), tid);
      buf ^= 1;
      if (w == 0 && lane == r) { cv = bv; ci = bi; }
#pragma unroll
      for (int j = 0; j < VPT; ++j)
        if (tid + j * NTHREADS == bi) taken |= 1u << j;
    }
  }
  if (w != 0) return 0;

  // 4. lane j < n holds the rank-j candidate: tempered softmax over them
  const bool act = lane < n;
  const float z = act ? cv / T : 0.0f;
  const float z0 = readlane_f(z, 0);
  const float dz = z - z0;
  const float e = act ? (float)exp((double)dz) : 0.0f;
  // Sequential f32 sums in rank order, unrolled over all 64 lanes: e and p
  // are exactly 0 past rank n-1, and adding +0 to a non-negative sum leaves
  // it bit-identical, so the chains equal the n-term ones.
  float S = 0.0f;
#pragma unroll
  for (int j = 0; j < TOPK_MAX; ++j) S += readlane_f(e, j);
  const float p = act ? e / S : 0.0f;
  float c = 0.0f, my_c = 0.0f;
#pragma unroll
  for (int j = 0; j < TOPK_MAX; ++j) {
    c += readlane_f(p, j);
    my_c = (lane == j) ? c : my_c;
  }
  const u64 ge = __ballot(act && my_c >= top_p);
  const int m = ge ? (__ffsll((long long)ge) - 1) : (n - 1);
  // 5. exponential race over the kept ranks 0..m (E computed at the start)
  float key = (lane <= m) ? p / E : -INFINITY;
  int kl = lane;
  wave_best(key, kl);
  return __builtin_amdgcn_readlane(ci, kl);
}

// Sampler entry for any V <= 2 * 8 * NTHREADS.
template <typename Src>
__device__ __forceinline__ int sample_from(const Src& src, int V, float T, float top_p, int top_k, float u,
                                           const SampScratch& sc) {
  if (V <= 8 * NTHREADS) return sample_block<8>(src, V, T, top_p, top_k, u, sc);
  return sample_block<16>(src, V, T, top_p, top_k, u, sc);
}
__device__ __forceinline__ int sample_request(const float* L, int V, float T, float top_p, int top_k, float u,
                                              const SampScratch& sc) {
  return sample_from(PlainLogits{L}, V, T, top_p, top_k, u, sc);
}

}  // namespace s2f
