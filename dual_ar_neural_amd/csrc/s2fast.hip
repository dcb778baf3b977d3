// s2fast: persistent per-frame Fast-AR decoder for gfx950 (MI355X).
//
// One cooperative launch decodes one frame of one request: 256 blocks (one
// per CU) walk the nine decode steps together.  Every weight matrix is split
// by rows across the blocks and streamed once per step with non-temporal
// 16-byte loads; the blocks meet at device-wide flag barriers between the
// phases whose inputs depend on every block's outputs.
//
// Per decode step k (window [hidden, emb(c_0), ..., emb(c_{k-1})], positions
// restart at 0; "Fast-AR codebook decoding and the generation main loop",
// sections 2-4) and per layer:
//   A  RMSNorm(x) -> fused wqkv rows                                  | sync
//   B  per KV group: q/k RMSNorm + pair RoPE + causal attention (mask
//      offset 0) -> wo restricted to the group's columns; the 8 group
//      partial sums meet in an int64 fixed-point accumulator          | sync
//   C  x_mid = x + attn; RMSNorm -> w1, w3 rows -> silu(a1) * a3      | sync
//   D  w2 rows; x = x_mid + ffn                                        | sync
// then fast_norm -> untied fast_output rows -> logits | sync, and the sampler
// (every block draws the same code from the same logits).
//
// The method recomputes the whole window at every call (no KV cache).  The
// window's rows 0..k-1 are computed from the same inputs at every call, so
// their keys/values are identical; this kernel keeps them per frame and only
// pushes the new row(s) through the layers (rows 0 and 1 at step 1, row k
// after), which computes the same logits.
#include "device_common.h"
#include "sampler.h"
#include "../../include/s2fast.h"

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

using namespace s2f;

namespace {

struct LayerPtr {
  const void *attn_norm, *wqkv, *q_norm, *k_norm, *wo, *ffn_norm, *w1, *w3, *w2;
};

struct FrameArgs {
  // shape
  int in_dim, dim, n_layer, n_head, n_kv, hd, ffn, V, ncb, ctx_len;
  float eps;
  int has_proj, has_qkn;
  int qkv_dim, attn_dim, gheads, gw;
  int kmax;   // LDS activation row stride (floats)
  int rmax;   // rows-per-block bound for the reduction buffer
  // weights
  const void* proj;
  const void* emb;
  const void* fnorm;
  const void* outw;
  LayerPtr L[S2FAST_MAX_LAYERS];
  const float* rope;  // [2][ctx_len][hd/2]: cos then sin
  // the request this launch decodes
  const float* hidden;     // [in_dim]
  const int* sem_code;     // [1]
  const float* uniforms;   // [ncb-1]
  const float* temp;       // [1]
  const float* top_p;      // [1]
  const int* top_k;        // [1]
  const int* forced;       // [ncb] teacher-forced codes, or nullptr
  int* codes_out;          // [ncb] or nullptr
  float* logits_out;       // [ncb-1][V] or nullptr
  // scratch (device; cross-block traffic only through sc1 accesses)
  float* xin0;             // [dim] fast_project_in(hidden)
  float* x;                // [MMAX][dim] residual stream of the new rows
  float* qkv;              // [MMAX][qkv_dim]
  long long* acc;          // [MMAX][dim] fixed-point attention output (0 at entry and exit)
  float* g;                // [MMAX][ffn]
  float* kv;               // [n_layer][ctx][n_kv][2][hd] this frame's keys/values
  float* logits;           // [V]
  u32* flags;              // [P][64] per-block barrier epochs
  u32 epoch0;              // epoch reached before this launch
  u32* err;                // watchdog word
};

// ---------------------------------------------------------------- LDS map
struct Lds {
  float* act;    // [MMAX][kmax]; also the sampler's logits
  float* red;    // [rmax][NWAVE][MMAX]
  float* small;  // [64]: rms scratch, epilogue temporaries
  float* q;      // [MMAX][gheads][hd]
  float* kc;     // [ctx][hd]
  float* vc;     // [ctx][hd]
  float* sc;     // [MMAX][gheads][ctx] attention probabilities
  float* a1;     // [rmax][MMAX] w1 outputs before SwiGLU
  float* cval;   // [64]
  int* cidx;     // [64]
  u32* mark;     // [256]
  int* codes;    // [16]
  int* flag;     // [4]
};

__host__ __device__ inline size_t lds_floats(int kmax, int rmax, int gheads, int hd, int ctx, int V) {
  size_t act = (size_t)MMAX * kmax;
  if ((size_t)V > act) act = V;
  return act + (size_t)rmax * NWAVE * MMAX + 64 + (size_t)MMAX * gheads * hd + 2 * (size_t)ctx * hd +
         (size_t)MMAX * gheads * ctx + (size_t)rmax * MMAX + 64 + 64 + 256 + 16 + 4;
}

__device__ inline Lds carve(float* base, const FrameArgs& a) {
  Lds s;
  size_t act = (size_t)MMAX * a.kmax;
  if ((size_t)a.V > act) act = a.V;
  float* p = base;
  s.act = p; p += act;
  s.red = p; p += (size_t)a.rmax * NWAVE * MMAX;
  s.small = p; p += 64;
  s.q = p; p += (size_t)MMAX * a.gheads * a.hd;
  s.kc = p; p += (size_t)a.ctx_len * a.hd;
  s.vc = p; p += (size_t)a.ctx_len * a.hd;
  s.sc = p; p += (size_t)MMAX * a.gheads * a.ctx_len;
  s.a1 = p; p += (size_t)a.rmax * MMAX;
  s.cval = p; p += 64;
  s.cidx = reinterpret_cast<int*>(p); p += 64;
  s.mark = reinterpret_cast<u32*>(p); p += 256;
  s.codes = reinterpret_cast<int*>(p); p += 16;
  s.flag = reinterpret_cast<int*>(p);
  return s;
}

// rows [r0, r1) of an n-row matrix owned by part `j` of `parts`
__device__ __forceinline__ void split_rows(int n, int j, int parts, int& r0, int& r1) {
  r0 = (int)(((long long)n * j) / parts);
  r1 = (int)(((long long)n * (j + 1)) / parts);
}

// --------------------------------------------------------------- grid sync
// Device-wide barrier.  Every thread first waits for its own stores (vmcnt),
// the block meets at s_barrier, then wave 0 publishes the block's epoch and
// polls every block's flag with coherent loads.  Returns false (after
// raising the watchdog word) if a flag does not arrive within SPIN_LIMIT
// polls; the caller then leaves the kernel.
__device__ bool grid_sync(const FrameArgs& a, u32& epoch, const Lds& s) {
  wait_vmem();
  __syncthreads();
  ++epoch;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int P = gridDim.x;
    if (lane == 0) st_coh(a.flags + 64 * blockIdx.x, epoch);
    u32 spins = 0;
    bool ok = true;
    while (true) {
      bool done = true;
      for (int b = lane; b < P; b += 64) done = done && (ld_coh(a.flags + 64 * b) >= epoch);
      if (__ballot(done) == ~0ull) break;
      if (++spins > SPIN_LIMIT) { ok = false; break; }
    }
    if (lane == 0) {
      if (!ok) atomicOr(a.err, 1u);
      s.flag[0] = ok ? 0 : 1;
    }
  }
  __syncthreads();
  return s.flag[0] == 0;
}

// --------------------------------------------------------------- GEMV
// Rows [row0, row0+nrows) of W (row stride ldw elements), columns
// [col0, col0+K), against M activation rows in LDS (row stride act_ld).
// Each wave takes a contiguous range of 64-segment chunks (16 bytes per
// lane) of the block's rows and leaves per-(row, wave, m) partial sums in
// red, which the caller zeroes beforehand and reduces in wave order.
template <typename WT>
__device__ __forceinline__ void gemv(const WT* __restrict__ W, long long ldw, int col0, int K, int row0,
                                     int nrows, const float* act, int act_ld, int M, float* red) {
  constexpr int EPL = WTraits<WT>::EPL;
  constexpr int U = 4;
  const int S = K / EPL;
  const int C = (S + 63) >> 6;
  const int T = nrows * C;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t0 = (int)(((long long)T * wave) / NWAVE);
  const int t1 = (int)(((long long)T * (wave + 1)) / NWAVE);
  if (t0 >= t1) return;
  float acc[MMAX];
#pragma unroll
  for (int m = 0; m < MMAX; ++m) acc[m] = 0.0f;
  int cur = t0 / C;
  auto flush = [&](int r) {
#pragma unroll
    for (int m = 0; m < MMAX; ++m) {
      if (m < M) {
        float v = wave_sum(acc[m]);
        if (lane == 0) red[((size_t)r * NWAVE + wave) * MMAX + m] = v;
      }
      acc[m] = 0.0f;
    }
  };
  for (int t = t0; t < t1; t += U) {
    uint4 q[U];
    int seg[U], rr[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int tt = t + u;
      rr[u] = tt / C;
      seg[u] = (tt - rr[u] * C) * 64 + lane;
      ok[u] = (tt < t1) && (seg[u] < S);
      if (ok[u]) q[u] = ld_stream(W + (long long)(row0 + rr[u]) * ldw + col0 + (long long)seg[u] * EPL);
      else q[u] = make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (t + u < t1) {
        if (rr[u] != cur) { flush(cur); cur = rr[u]; }
        if (ok[u]) {
          float w[EPL];
          WTraits<WT>::unpack(q[u], w);
#pragma unroll
          for (int m = 0; m < MMAX; ++m) {
            if (m < M) {
              const float* ap = act + (size_t)m * act_ld + (size_t)seg[u] * EPL;
#pragma unroll
              for (int e = 0; e < EPL; ++e) acc[m] = fmaf(w[e], ap[e], acc[m]);
            }
          }
        }
      }
    }
  }
  flush(cur);
}

__device__ __forceinline__ void zero_lds(float* p, int n) {
  for (int i = threadIdx.x; i < n; i += NTHREADS) p[i] = 0.0f;
}

// sum of the per-wave partials of row r, activation row m
__device__ __forceinline__ float red_sum(const float* red, int r, int m) {
  float v = 0.0f;
#pragma unroll
  for (int w = 0; w < NWAVE; ++w) v += red[((size_t)r * NWAVE + w) * MMAX + m];
  return v;
}

// RMSNorm of M rows of length K held in LDS, in place: x / sqrt(mean(x^2) + eps) * w
// ("Model loading and GGUF", section 2.2: eps 1e-6; Mizuoto page: float32).
template <typename WT>
__device__ void rms_norm_rows(float* act, int act_ld, int M, int K, const WT* w, float eps, float* small) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int m = 0; m < M; ++m) {
    float ss = 0.0f;
    for (int k = threadIdx.x; k < K; k += NTHREADS) {
      float v = act[(size_t)m * act_ld + k];
      ss = fmaf(v, v, ss);
    }
    ss = wave_sum(ss);
    if (lane == 0) small[m * NWAVE + wave] = ss;
  }
  __syncthreads();
  if (threadIdx.x < M) {
    float t = 0.0f;
    for (int w2 = 0; w2 < NWAVE; ++w2) t += small[threadIdx.x * NWAVE + w2];
    small[32 + threadIdx.x] = sqrtf(t / (float)K + eps);
  }
  __syncthreads();
  for (int m = 0; m < M; ++m) {
    const float den = small[32 + m];
    for (int k = threadIdx.x; k < K; k += NTHREADS)
      act[(size_t)m * act_ld + k] = act[(size_t)m * act_ld + k] / den * WTraits<WT>::one(w, k);
  }
  __syncthreads();
}

// Layer input of new row m at window position pos, element k: position 0 is
// the hidden state (through fast_project_in when present), position j >= 1
// is fast_embeddings[c_{j-1}] ("Fast-AR codebook decoding ...", section 2).
template <typename WT>
__device__ __forceinline__ float layer0_input(const FrameArgs& a, const Lds& s, int pos, int k) {
  if (pos == 0) return a.has_proj ? ld_coh(a.xin0 + k) : a.hidden[k];
  const WT* e = reinterpret_cast<const WT*>(a.emb) + (size_t)s.codes[pos - 1] * a.dim;
  return WTraits<WT>::one(e, k);
}

__device__ __forceinline__ int row_pos(int step, int m) { return step == 1 ? m : step; }

// one 128-wide (or narrower) head vector per wave: RMSNorm with weight w, then
// pair RoPE at position pos; in place in LDS.
template <typename WT>
__device__ __forceinline__ void head_norm_rope(float* v, int hd, const WT* w, bool do_norm, float eps,
                                               const float* rope, int ctx, int pos) {
  const int lane = threadIdx.x & 63;
  // lane owns the pair (2*lane, 2*lane+1) when 2*lane < hd
  const bool own = 2 * lane < hd;
  float x0 = own ? v[2 * lane] : 0.0f;
  float x1 = own ? v[2 * lane + 1] : 0.0f;
  if (do_norm) {
    float ss = wave_sum(fmaf(x0, x0, x1 * x1));
    const float den = sqrtf(ss / (float)hd + eps);
    if (own) {
      x0 = x0 / den * WTraits<WT>::one(w, 2 * lane);
      x1 = x1 / den * WTraits<WT>::one(w, 2 * lane + 1);
    }
  }
  if (own) {
    const float c = rope[(size_t)pos * (hd / 2) + lane];
    const float sn = rope[(size_t)ctx * (hd / 2) + (size_t)pos * (hd / 2) + lane];
    v[2 * lane] = x0 * c - x1 * sn;
    v[2 * lane + 1] = x0 * sn + x1 * c;
  }
}

// --------------------------------------------------------------- phases
template <typename WT>
__device__ void phase_qkv(const FrameArgs& a, const Lds& s, int l, int step, int M) {
  const int D = a.dim;
  for (int m = 0; m < M; ++m) {
    const int pos = row_pos(step, m);
    for (int k = threadIdx.x; k < D; k += NTHREADS)
      s.act[(size_t)m * a.kmax + k] = (l == 0) ? layer0_input<WT>(a, s, pos, k) : ld_coh(a.x + (size_t)m * D + k);
  }
  int r0, r1;
  split_rows(a.qkv_dim, blockIdx.x, gridDim.x, r0, r1);
  zero_lds(s.red, (r1 - r0) * NWAVE * MMAX);
  __syncthreads();
  rms_norm_rows<WT>(s.act, a.kmax, M, D, reinterpret_cast<const WT*>(a.L[l].attn_norm), a.eps, s.small);
  gemv<WT>(reinterpret_cast<const WT*>(a.L[l].wqkv), D, 0, D, r0, r1 - r0, s.act, a.kmax, M, s.red);
  __syncthreads();
  for (int i = threadIdx.x; i < (r1 - r0) * M; i += NTHREADS) {
    const int r = i / M, m = i % M;
    st_coh(a.qkv + (size_t)m * a.qkv_dim + r0 + r, red_sum(s.red, r, m));
  }
}

template <typename WT>
__device__ void phase_attn_wo(const FrameArgs& a, const Lds& s, int l, int step, int M) {
  const int P = gridDim.x;
  const int g = blockIdx.x % a.n_kv;              // KV group of this block
  const int rg = blockIdx.x / a.n_kv;             // rank inside the group
  const int Pg = (P - g + a.n_kv - 1) / a.n_kv;   // blocks in the group
  int r0, r1;
  split_rows(a.dim, rg, Pg, r0, r1);
  const int hd = a.hd, H = a.n_head, G = a.n_kv, gh = a.gheads;
  const int first_new = (step == 1) ? 0 : step;   // positions < first_new come from this frame's cache
  const int last_pos = (step == 1) ? 1 : step;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const WT* qn = reinterpret_cast<const WT*>(a.L[l].q_norm);
  const WT* kn = reinterpret_cast<const WT*>(a.L[l].k_norm);
  float* kvl = a.kv + (size_t)l * a.ctx_len * G * 2 * hd;   // [ctx][G][2][hd]
  const bool need_attn = (r1 > r0) || rg == 0;
  if (need_attn) {
    // cached keys/values of positions < first_new
    for (int i = threadIdx.x; i < first_new * hd; i += NTHREADS) {
      const int j = i / hd, d = i % hd;
      s.kc[(size_t)j * hd + d] = ld_coh(kvl + (((size_t)j * G + g) * 2 + 0) * hd + d);
      s.vc[(size_t)j * hd + d] = ld_coh(kvl + (((size_t)j * G + g) * 2 + 1) * hd + d);
    }
    // new rows: raw q (the group's heads), k, v
    for (int m = 0; m < M; ++m) {
      const int pos = row_pos(step, m);
      const float* src = a.qkv + (size_t)m * a.qkv_dim;
      for (int i = threadIdx.x; i < gh * hd; i += NTHREADS)
        s.q[(size_t)m * gh * hd + i] = ld_coh(src + (size_t)g * gh * hd + i);
      for (int d = threadIdx.x; d < hd; d += NTHREADS) {
        s.kc[(size_t)pos * hd + d] = ld_coh(src + (size_t)H * hd + (size_t)g * hd + d);
        s.vc[(size_t)pos * hd + d] = ld_coh(src + (size_t)(H + G) * hd + (size_t)g * hd + d);
      }
    }
    __syncthreads();
    // q/k RMSNorm + RoPE: one wave per head vector
    const int nvec = M * gh + M;
    for (int v = wave; v < nvec; v += NWAVE) {
      if (v < M * gh) {
        const int m = v / gh;
        head_norm_rope<WT>(s.q + (size_t)v * hd, hd, qn, a.has_qkn, a.eps, a.rope, a.ctx_len, row_pos(step, m));
      } else {
        const int m = v - M * gh;
        const int pos = row_pos(step, m);
        head_norm_rope<WT>(s.kc + (size_t)pos * hd, hd, kn, a.has_qkn, a.eps, a.rope, a.ctx_len, pos);
      }
    }
    __syncthreads();
    // keep this step's keys/values for later steps of the frame
    if (rg == 0) {
      for (int m = 0; m < M; ++m) {
        const int pos = row_pos(step, m);
        for (int d = threadIdx.x; d < hd; d += NTHREADS) {
          st_coh(kvl + (((size_t)pos * G + g) * 2 + 0) * hd + d, s.kc[(size_t)pos * hd + d]);
          st_coh(kvl + (((size_t)pos * G + g) * 2 + 1) * hd + d, s.vc[(size_t)pos * hd + d]);
        }
      }
    }
    // scaled dot-product attention, causal with offset 0: row at position p
    // sees positions 0..p.  One wave per (row, head).
    const float scale = 1.0f / sqrtf((float)hd);
    for (int pr = wave; pr < M * gh; pr += NWAVE) {
      const int m = pr / gh, hh = pr % gh;
      const int pos = row_pos(step, m);
      const float* qv = s.q + (size_t)pr * hd;
      float* sc = s.sc + (size_t)pr * a.ctx_len;
      const float q0 = lane < hd ? qv[lane] : 0.0f;
      const float q1 = lane + 64 < hd ? qv[lane + 64] : 0.0f;
      float mx = -INFINITY;
      for (int j = 0; j <= pos; ++j) {
        const float k0 = lane < hd ? s.kc[(size_t)j * hd + lane] : 0.0f;
        const float k1 = lane + 64 < hd ? s.kc[(size_t)j * hd + lane + 64] : 0.0f;
        const float dot = wave_sum(fmaf(q0, k0, q1 * k1)) * scale;
        if (lane == 0) sc[j] = dot;
        mx = fmaxf(mx, dot);
      }
      __builtin_amdgcn_wave_barrier();
      float den = 0.0f;
      for (int j = 0; j <= pos; ++j) den += expf(sc[j] - mx);
      float o0 = 0.0f, o1 = 0.0f;
      for (int j = 0; j <= pos; ++j) {
        const float pj = expf(sc[j] - mx) / den;
        if (lane < hd) o0 = fmaf(pj, s.vc[(size_t)j * hd + lane], o0);
        if (lane + 64 < hd) o1 = fmaf(pj, s.vc[(size_t)j * hd + lane + 64], o1);
      }
      float* o = s.act + (size_t)m * a.kmax + (size_t)hh * hd;
      if (lane < hd) o[lane] = o0;
      if (lane + 64 < hd) o[lane + 64] = o1;
    }
    (void)last_pos;
  }
  zero_lds(s.red, (r1 - r0) * NWAVE * MMAX);
  __syncthreads();
  // wo restricted to this group's columns [g*gw, (g+1)*gw)
  gemv<WT>(reinterpret_cast<const WT*>(a.L[l].wo), a.attn_dim, g * a.gw, a.gw, r0, r1 - r0, s.act, a.kmax, M, s.red);
  __syncthreads();
  for (int i = threadIdx.x; i < (r1 - r0) * M; i += NTHREADS) {
    const int r = i / M, m = i % M;
    atomic_add_coh(a.acc + (size_t)m * a.dim + r0 + r, to_fx(red_sum(s.red, r, m)));
  }
}

template <typename WT>
__device__ __forceinline__ float x_mid_of(const FrameArgs& a, const Lds& s, int l, int step, int m, int k) {
  const float xin = (l == 0) ? layer0_input<WT>(a, s, row_pos(step, m), k) : ld_coh(a.x + (size_t)m * a.dim + k);
  return xin + from_fx(ld_coh(a.acc + (size_t)m * a.dim + k));
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

template <typename WT>
__device__ void phase_ffn_up(const FrameArgs& a, const Lds& s, int l, int step, int M) {
  const int D = a.dim;
  for (int m = 0; m < M; ++m)
    for (int k = threadIdx.x; k < D; k += NTHREADS) s.act[(size_t)m * a.kmax + k] = x_mid_of<WT>(a, s, l, step, m, k);
  int r0, r1;
  split_rows(a.ffn, blockIdx.x, gridDim.x, r0, r1);
  const int nr = r1 - r0;
  zero_lds(s.red, nr * NWAVE * MMAX);
  __syncthreads();
  rms_norm_rows<WT>(s.act, a.kmax, M, D, reinterpret_cast<const WT*>(a.L[l].ffn_norm), a.eps, s.small);
  gemv<WT>(reinterpret_cast<const WT*>(a.L[l].w1), D, 0, D, r0, nr, s.act, a.kmax, M, s.red);
  __syncthreads();
  for (int i = threadIdx.x; i < nr * M; i += NTHREADS) s.a1[i] = red_sum(s.red, i / M, i % M);
  __syncthreads();
  zero_lds(s.red, nr * NWAVE * MMAX);
  __syncthreads();
  gemv<WT>(reinterpret_cast<const WT*>(a.L[l].w3), D, 0, D, r0, nr, s.act, a.kmax, M, s.red);
  __syncthreads();
  for (int i = threadIdx.x; i < nr * M; i += NTHREADS) {
    const int r = i / M, m = i % M;
    st_coh(a.g + (size_t)m * a.ffn + r0 + r, silu(s.a1[i]) * red_sum(s.red, r, m));
  }
}

template <typename WT>
__device__ void phase_ffn_down(const FrameArgs& a, const Lds& s, int l, int step, int M) {
  for (int m = 0; m < M; ++m)
    for (int k = threadIdx.x; k < a.ffn; k += NTHREADS) s.act[(size_t)m * a.kmax + k] = ld_coh(a.g + (size_t)m * a.ffn + k);
  int r0, r1;
  split_rows(a.dim, blockIdx.x, gridDim.x, r0, r1);
  zero_lds(s.red, (r1 - r0) * NWAVE * MMAX);
  __syncthreads();
  gemv<WT>(reinterpret_cast<const WT*>(a.L[l].w2), a.ffn, 0, a.ffn, r0, r1 - r0, s.act, a.kmax, M, s.red);
  __syncthreads();
  for (int i = threadIdx.x; i < (r1 - r0) * M; i += NTHREADS) {
    const int r = i / M, m = i % M;
    const int k = r0 + r;
    const float xm = x_mid_of<WT>(a, s, l, step, m, k);
    st_coh(a.x + (size_t)m * a.dim + k, xm + red_sum(s.red, r, m));
    st_coh(a.acc + (size_t)m * a.dim + k, 0ll);
  }
}

template <typename WT>
__device__ void phase_head(const FrameArgs& a, const Lds& s, int step, int M) {
  const int D = a.dim;
  for (int k = threadIdx.x; k < D; k += NTHREADS) s.act[k] = ld_coh(a.x + (size_t)(M - 1) * D + k);
  int r0, r1;
  split_rows(a.V, blockIdx.x, gridDim.x, r0, r1);
  zero_lds(s.red, (r1 - r0) * NWAVE * MMAX);
  __syncthreads();
  rms_norm_rows<WT>(s.act, a.kmax, 1, D, reinterpret_cast<const WT*>(a.fnorm), a.eps, s.small);
  gemv<WT>(reinterpret_cast<const WT*>(a.outw), D, 0, D, r0, r1 - r0, s.act, a.kmax, 1, s.red);
  __syncthreads();
  for (int r = threadIdx.x; r < r1 - r0; r += NTHREADS) {
    const float v = red_sum(s.red, r, 0);
    st_coh(a.logits + r0 + r, v);
    if (a.logits_out) a.logits_out[(size_t)(step - 1) * a.V + r0 + r] = v;
  }
}

template <typename WT>
__device__ void phase_project_in(const FrameArgs& a, const Lds& s) {
  for (int k = threadIdx.x; k < a.in_dim; k += NTHREADS) s.act[k] = a.hidden[k];
  int r0, r1;
  split_rows(a.dim, blockIdx.x, gridDim.x, r0, r1);
  zero_lds(s.red, (r1 - r0) * NWAVE * MMAX);
  __syncthreads();
  gemv<WT>(reinterpret_cast<const WT*>(a.proj), a.in_dim, 0, a.in_dim, r0, r1 - r0, s.act, a.kmax, 1, s.red);
  __syncthreads();
  for (int r = threadIdx.x; r < r1 - r0; r += NTHREADS) st_coh(a.xin0 + r0 + r, red_sum(s.red, r, 0));
}

template <typename WT>
__global__ void __launch_bounds__(NTHREADS) frame_kernel(FrameArgs a) {
  extern __shared__ float lds_base[];
  const Lds s = carve(lds_base, a);
  u32 epoch = a.epoch0;
  const int V = a.V;
  if (threadIdx.x == 0) {
    const int c0 = a.forced ? a.forced[0] : a.sem_code[0];
    s.codes[0] = min(max(c0, 0), V - 1);     // clamp both ways (main loop, section 5.2)
    if (a.forced)
      for (int j = 1; j < a.ncb; ++j) s.codes[j] = min(max(a.forced[j], 0), V - 1);
  }
  __syncthreads();
  if (a.has_proj) {
    phase_project_in<WT>(a, s);
    if (!grid_sync(a, epoch, s)) return;
  }
  for (int step = 1; step < a.ncb; ++step) {
    const int M = (step == 1) ? 2 : 1;
    for (int l = 0; l < a.n_layer; ++l) {
      phase_qkv<WT>(a, s, l, step, M);
      if (!grid_sync(a, epoch, s)) return;
      phase_attn_wo<WT>(a, s, l, step, M);
      if (!grid_sync(a, epoch, s)) return;
      phase_ffn_up<WT>(a, s, l, step, M);
      if (!grid_sync(a, epoch, s)) return;
      phase_ffn_down<WT>(a, s, l, step, M);
      if (!grid_sync(a, epoch, s)) return;
    }
    phase_head<WT>(a, s, step, M);
    if (a.forced) continue;            // teacher forcing: the next prefix is known
    if (!grid_sync(a, epoch, s)) return;
    for (int v = threadIdx.x; v < V; v += NTHREADS) s.act[v] = ld_coh(a.logits + v);
    __syncthreads();
    if (threadIdx.x < 64) {
      const int code = sample_wave(s.act, V, a.temp[0], a.top_p[0], a.top_k[0], a.uniforms[step - 1],
                                   s.cval, s.cidx, s.mark);
      if (threadIdx.x == 0) s.codes[step] = min(max(code, 0), V - 1);
    }
    __syncthreads();
  }
  if (blockIdx.x == 0 && a.codes_out && threadIdx.x < a.ncb) a.codes_out[threadIdx.x] = s.codes[threadIdx.x];
}

__global__ void __launch_bounds__(64) sample_kernel(int V, const float* logits, const float* temp, const float* top_p,
                                                    const int* top_k, const float* u, int* codes) {
  extern __shared__ float lds_base[];
  float* L = lds_base;
  float* cval = L + V;
  int* cidx = reinterpret_cast<int*>(cval + 64);
  u32* mark = reinterpret_cast<u32*>(cidx + 64);
  const int b = blockIdx.x;
  for (int i = threadIdx.x; i < V; i += 64) L[i] = logits[(size_t)b * V + i];
  __syncthreads();
  const int c = sample_wave(L, V, temp[b], top_p[b], top_k[b], u[b], cval, cidx, mark);
  if (threadIdx.x == 0) codes[b] = c;
}

}  // namespace

// =================================================================== host

struct s2fast_ctx {
  s2fast_config cfg;
  s2fast_weights w;
  int device = 0;
  int ncu = 0;
  size_t lds_bytes = 0;
  int kmax = 0, rmax = 0;
  float* rope = nullptr;
  float* xin0 = nullptr;
  float* x = nullptr;
  float* qkv = nullptr;
  long long* acc = nullptr;
  float* g = nullptr;
  float* kv = nullptr;
  float* logits = nullptr;
  u32* flags = nullptr;
  u32* err = nullptr;
  u32 epoch = 0;
};

namespace {

bool is_gfx950(int dev) {
  hipDeviceProp_t p;
  if (hipGetDeviceProperties(&p, dev) != hipSuccess) return false;
  return std::strncmp(p.gcnArchName, "gfx950", 6) == 0;
}

// bf16 rounding straight from double: 8 significant bits, ties to even
double bf16_round(double v) {
  int e = 0;
  const double m = std::frexp(v, &e);
  return std::ldexp(std::nearbyint(std::ldexp(m, 8)), e - 8);
}

void rope_table_host(int hd, int ctx, float base, float* c, float* s) {
  for (int p = 0; p < ctx; ++p)
    for (int i = 0; i < hd / 2; ++i) {
      const double th = (double)p * std::pow((double)base, -2.0 * i / (double)hd);
      c[p * (hd / 2) + i] = (float)bf16_round(std::cos(th));
      s[p * (hd / 2) + i] = (float)bf16_round(std::sin(th));
    }
}

int syncs_for(const s2fast_config& c, bool forced) {
  const int per_step = 4 * c.n_layer + (forced ? 0 : 1);
  return (c.has_project_in ? 1 : 0) + (c.num_codebooks - 1) * per_step;
}

void free_ctx(s2fast_ctx* c) {
  if (!c) return;
  void* ptrs[] = {c->rope, c->xin0, c->x, c->qkv, c->acc, c->g, c->kv, c->logits, c->flags, c->err};
  for (void* p : ptrs)
    if (p) (void)hipFree(p);
  delete c;
}

template <typename T>
hipError_t dalloc(T** p, size_t n) {
  return hipMalloc(reinterpret_cast<void**>(p), n * sizeof(T) > 0 ? n * sizeof(T) : 16);
}

int launch_frame(s2fast_ctx* c, const FrameArgs& fa_in, hipStream_t stream) {
  FrameArgs fa = fa_in;
  const u32 n = (u32)syncs_for(c->cfg, fa.forced != nullptr);
  if (c->epoch > 0xF0000000u) {
    if (hipMemsetAsync(c->flags, 0, (size_t)c->ncu * 64 * sizeof(u32), stream) != hipSuccess) return S2FAST_ERR_HIP;
    c->epoch = 0;
  }
  fa.epoch0 = c->epoch;
  void* args[] = {&fa};
  const void* fn = c->cfg.weight_dtype == S2FAST_BF16 ? reinterpret_cast<const void*>(&frame_kernel<uint16_t>)
                                                       : reinterpret_cast<const void*>(&frame_kernel<float>);
  hipError_t e = hipLaunchCooperativeKernel(fn, dim3(c->ncu), dim3(NTHREADS), args, c->lds_bytes, stream);
  if (e != hipSuccess) return S2FAST_ERR_HIP;
  c->epoch += n;
  return S2FAST_OK;
}

void fill_shape(const s2fast_ctx* c, FrameArgs& fa) {
  const s2fast_config& k = c->cfg;
  std::memset(&fa, 0, sizeof(fa));
  fa.in_dim = k.in_dim; fa.dim = k.dim; fa.n_layer = k.n_layer; fa.n_head = k.n_head; fa.n_kv = k.n_head_kv;
  fa.hd = k.head_dim; fa.ffn = k.ffn_dim; fa.V = k.codebook_size; fa.ncb = k.num_codebooks; fa.ctx_len = k.context;
  fa.eps = k.norm_eps; fa.has_proj = k.has_project_in; fa.has_qkn = k.has_qk_norm;
  fa.qkv_dim = (k.n_head + 2 * k.n_head_kv) * k.head_dim;
  fa.attn_dim = k.n_head * k.head_dim;
  fa.gheads = k.n_head / k.n_head_kv;
  fa.gw = fa.gheads * k.head_dim;
  fa.kmax = c->kmax; fa.rmax = c->rmax;
  fa.proj = c->w.project_in; fa.emb = c->w.embeddings; fa.fnorm = c->w.norm; fa.outw = c->w.output;
  for (int l = 0; l < k.n_layer; ++l) {
    const s2fast_layer_weights& L = c->w.layers[l];
    fa.L[l] = LayerPtr{L.attention_norm, L.wqkv, L.q_norm, L.k_norm, L.wo, L.ffn_norm, L.w1, L.w3, L.w2};
  }
  fa.rope = c->rope;
  fa.xin0 = c->xin0; fa.x = c->x; fa.qkv = c->qkv; fa.acc = c->acc; fa.g = c->g; fa.kv = c->kv;
  fa.logits = c->logits; fa.flags = c->flags; fa.err = c->err;
}

}  // namespace

extern "C" {

const char* s2fast_strerror(int code) {
  switch (code) {
    case S2FAST_OK: return "ok";
    case S2FAST_ERR_ARG: return "invalid argument or unsupported shape";
    case S2FAST_ERR_NO_FAST_DECODER: return "model has no fast decoder (a required Fast-AR weight is missing)";
    case S2FAST_ERR_HIDDEN_DIM: return "hidden state width does not match the model";
    case S2FAST_ERR_PREFIX_LEN: return "prefix must hold fewer codes than there are codebooks";
    case S2FAST_ERR_BATCH: return "batch size outside [1, max_batch]";
    case S2FAST_ERR_HIP: return "HIP runtime error";
    case S2FAST_ERR_NOMEM: return "out of memory";
    case S2FAST_ERR_DEVICE: return "unsupported device (needs gfx950 with co-resident cooperative blocks)";
    default: return "unknown error";
  }
}

int s2fast_create(const s2fast_config* cfg, const s2fast_weights* w, s2fast_ctx** out) {
  if (!cfg || !w || !out) return S2FAST_ERR_ARG;
  *out = nullptr;
  const s2fast_config& k = *cfg;
  const int epl = k.weight_dtype == S2FAST_BF16 ? 8 : 4;
  if (k.weight_dtype != S2FAST_BF16 && k.weight_dtype != S2FAST_F32) return S2FAST_ERR_ARG;
  if (k.n_layer < 1 || k.n_layer > S2FAST_MAX_LAYERS) return S2FAST_ERR_ARG;
  if (k.n_head < 1 || k.n_head_kv < 1 || k.n_head % k.n_head_kv != 0 || k.n_head_kv > 64) return S2FAST_ERR_ARG;
  if (k.head_dim < 2 || k.head_dim > 128 || (k.head_dim & 1)) return S2FAST_ERR_ARG;
  if (k.dim < epl || k.in_dim < epl || k.ffn_dim < epl || k.dim > 16384 || k.in_dim > 16384 || k.ffn_dim > 16384)
    return S2FAST_ERR_ARG;
  if (k.dim % epl || k.in_dim % epl || k.ffn_dim % epl) return S2FAST_ERR_ARG;
  if (((k.n_head / k.n_head_kv) * k.head_dim) % epl) return S2FAST_ERR_ARG;
  if (k.codebook_size < 2 || k.codebook_size > 8192) return S2FAST_ERR_ARG;
  if (k.num_codebooks < 2 || k.num_codebooks > 16 || k.context < k.num_codebooks || k.context > 16) return S2FAST_ERR_ARG;
  if (!k.has_project_in && k.in_dim != k.dim) return S2FAST_ERR_ARG;
  if (!(k.norm_eps >= 0.0f) || !(k.rope_base > 0.0f)) return S2FAST_ERR_ARG;
  if (k.max_batch < 1 || k.max_batch > 4096) return S2FAST_ERR_ARG;
  // the fast decoder's tensors ("Model loading and GGUF", section 3)
  if (!w->embeddings || !w->norm || !w->output) return S2FAST_ERR_NO_FAST_DECODER;
  if (k.has_project_in && !w->project_in) return S2FAST_ERR_NO_FAST_DECODER;
  for (int l = 0; l < k.n_layer; ++l) {
    const s2fast_layer_weights& L = w->layers[l];
    if (!L.attention_norm || !L.wqkv || !L.wo || !L.ffn_norm || !L.w1 || !L.w3 || !L.w2)
      return S2FAST_ERR_NO_FAST_DECODER;
    if (k.has_qk_norm && (!L.q_norm || !L.k_norm)) return S2FAST_ERR_NO_FAST_DECODER;
  }

  // 16-byte weight loads need 16-byte aligned tensors
  auto misaligned = [](const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u); };
  if (misaligned(w->project_in) || misaligned(w->embeddings) || misaligned(w->norm) || misaligned(w->output))
    return S2FAST_ERR_ARG;
  for (int l = 0; l < k.n_layer; ++l) {
    const s2fast_layer_weights& L = w->layers[l];
    for (const void* p : {L.attention_norm, L.wqkv, L.q_norm, L.k_norm, L.wo, L.ffn_norm, L.w1, L.w3, L.w2})
      if (misaligned(p)) return S2FAST_ERR_ARG;
  }

  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return S2FAST_ERR_HIP;
  if (!is_gfx950(dev)) return S2FAST_ERR_DEVICE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return S2FAST_ERR_HIP;
  if (!prop.cooperativeLaunch) return S2FAST_ERR_DEVICE;

  s2fast_ctx* c = new (std::nothrow) s2fast_ctx();
  if (!c) return S2FAST_ERR_NOMEM;
  c->cfg = k;
  c->w = *w;
  c->device = dev;
  c->ncu = prop.multiProcessorCount;
  if (c->ncu < k.n_head_kv || c->ncu > 1024) { free_ctx(c); return S2FAST_ERR_DEVICE; }
  const int qkv_dim = (k.n_head + 2 * k.n_head_kv) * k.head_dim;
  const int gheads = k.n_head / k.n_head_kv;
  c->kmax = std::max(std::max(k.dim, k.in_dim), std::max(k.ffn_dim, gheads * k.head_dim));
  c->kmax = (c->kmax + 3) & ~3;
  // rows per block: largest split over the phases (+1 for uneven splits)
  const int P = c->ncu;
  const int per_group = (P + k.n_head_kv - 1) / k.n_head_kv;
  const int groups_min = P / k.n_head_kv;
  int rmax = 0;
  for (int n : {qkv_dim, k.ffn_dim, k.dim, k.codebook_size}) rmax = std::max(rmax, (n + P - 1) / P);
  rmax = std::max(rmax, (k.dim + groups_min - 1) / std::max(groups_min, 1));
  (void)per_group;
  c->rmax = rmax + 1;
  size_t lds = lds_floats(c->kmax, c->rmax, gheads, k.head_dim, k.context, k.codebook_size) * sizeof(float);
  // more than half of the CU's 160 KB: exactly one block per CU
  const size_t one_per_cu = 84 * 1024;
  if (lds < one_per_cu) lds = one_per_cu;
  if (lds > (size_t)prop.sharedMemPerBlock) { free_ctx(c); return S2FAST_ERR_ARG; }
  c->lds_bytes = lds;
  const void* fn = k.weight_dtype == S2FAST_BF16 ? reinterpret_cast<const void*>(&frame_kernel<uint16_t>)
                                                 : reinterpret_cast<const void*>(&frame_kernel<float>);
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess) {
    free_ctx(c); return S2FAST_ERR_HIP;
  }
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, NTHREADS, lds) != hipSuccess) { free_ctx(c); return S2FAST_ERR_HIP; }
  if (nb < 1) { free_ctx(c); return S2FAST_ERR_DEVICE; }

  const int half = k.head_dim / 2;
  std::vector<float> rope((size_t)2 * k.context * half);
  rope_table_host(k.head_dim, k.context, k.rope_base, rope.data(), rope.data() + (size_t)k.context * half);
  bool ok = dalloc(&c->rope, rope.size()) == hipSuccess && dalloc(&c->xin0, (size_t)k.dim) == hipSuccess &&
            dalloc(&c->x, (size_t)MMAX * k.dim) == hipSuccess && dalloc(&c->qkv, (size_t)MMAX * qkv_dim) == hipSuccess &&
            dalloc(&c->acc, (size_t)MMAX * k.dim) == hipSuccess && dalloc(&c->g, (size_t)MMAX * k.ffn_dim) == hipSuccess &&
            dalloc(&c->kv, (size_t)k.n_layer * k.context * k.n_head_kv * 2 * k.head_dim) == hipSuccess &&
            dalloc(&c->logits, (size_t)k.codebook_size) == hipSuccess && dalloc(&c->flags, (size_t)P * 64) == hipSuccess &&
            dalloc(&c->err, 64) == hipSuccess;
  if (!ok) { free_ctx(c); return S2FAST_ERR_NOMEM; }
  ok = hipMemcpy(c->rope, rope.data(), rope.size() * sizeof(float), hipMemcpyHostToDevice) == hipSuccess &&
       hipMemset(c->acc, 0, (size_t)MMAX * k.dim * sizeof(long long)) == hipSuccess &&
       hipMemset(c->flags, 0, (size_t)P * 64 * sizeof(u32)) == hipSuccess &&
       hipMemset(c->err, 0, 64 * sizeof(u32)) == hipSuccess && hipDeviceSynchronize() == hipSuccess;
  if (!ok) { free_ctx(c); return S2FAST_ERR_HIP; }
  *out = c;
  return S2FAST_OK;
}

void s2fast_destroy(s2fast_ctx* ctx) {
  if (!ctx) return;
  (void)hipDeviceSynchronize();
  free_ctx(ctx);
}

int s2fast_syncs_per_frame(const s2fast_ctx* ctx, int32_t B) {
  if (!ctx || B < 1) return -1;
  return B * syncs_for(ctx->cfg, false);
}

int s2fast_decode_frame(s2fast_ctx* ctx, int32_t B, const float* hidden, const int32_t* sem_code,
                        const float* uniforms, const float* temperature, const float* top_p,
                        const int32_t* top_k, int32_t* codes, void* stream) {
  if (!ctx) return S2FAST_ERR_ARG;
  if (B < 1 || B > ctx->cfg.max_batch) return S2FAST_ERR_BATCH;
  if (!hidden || !sem_code || !uniforms || !temperature || !top_p || !top_k || !codes) return S2FAST_ERR_ARG;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const s2fast_config& k = ctx->cfg;
  FrameArgs fa;
  fill_shape(ctx, fa);
  int rc = S2FAST_OK;
  for (int b = 0; b < B && rc == S2FAST_OK; ++b) {
    fa.hidden = hidden + (size_t)b * k.in_dim;
    fa.sem_code = sem_code + b;
    fa.uniforms = uniforms + (size_t)b * (k.num_codebooks - 1);
    fa.temp = temperature + b;
    fa.top_p = top_p + b;
    fa.top_k = top_k + b;
    fa.forced = nullptr;
    fa.codes_out = codes + (size_t)b * k.num_codebooks;
    fa.logits_out = nullptr;
    rc = launch_frame(ctx, fa, st);
  }
  if (rc != S2FAST_OK) {
    // a failed frame leaves codebooks 1.. at 0 ("Fast-AR codebook decoding ...", section 5.2)
    (void)hipMemset2DAsync(codes + 1, (size_t)k.num_codebooks * sizeof(int32_t), 0,
                           (size_t)(k.num_codebooks - 1) * sizeof(int32_t), (size_t)B, st);
  }
  return rc;
}

int s2fast_forward_logits(s2fast_ctx* ctx, int32_t B, const float* hidden, const int32_t* codes, float* logits,
                          void* stream) {
  if (!ctx) return S2FAST_ERR_ARG;
  if (B < 1 || B > ctx->cfg.max_batch) return S2FAST_ERR_BATCH;
  if (!hidden || !codes || !logits) return S2FAST_ERR_ARG;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const s2fast_config& k = ctx->cfg;
  FrameArgs fa;
  fill_shape(ctx, fa);
  for (int b = 0; b < B; ++b) {
    fa.hidden = hidden + (size_t)b * k.in_dim;
    fa.sem_code = codes + (size_t)b * k.num_codebooks;
    fa.forced = codes + (size_t)b * k.num_codebooks;
    fa.codes_out = nullptr;
    fa.logits_out = logits + (size_t)b * (k.num_codebooks - 1) * k.codebook_size;
    const int rc = launch_frame(ctx, fa, st);
    if (rc != S2FAST_OK) return rc;
  }
  return S2FAST_OK;
}

int s2fast_test_rope_table(int32_t head_dim, int32_t context, float rope_base, float* cos_out, float* sin_out) {
  if (!cos_out || !sin_out || head_dim < 2 || (head_dim & 1) || context < 1 || !(rope_base > 0.0f))
    return S2FAST_ERR_ARG;
  rope_table_host(head_dim, context, rope_base, cos_out, sin_out);
  return S2FAST_OK;
}

int s2fast_test_sample(int32_t B, int32_t V, const float* logits, const float* temperature, const float* top_p,
                       const int32_t* top_k, const float* u, int32_t* codes, void* stream) {
  if (B < 1 || V < 1 || V > 8192 || !logits || !temperature || !top_p || !top_k || !u || !codes) return S2FAST_ERR_ARG;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return S2FAST_ERR_HIP;
  if (!is_gfx950(dev)) return S2FAST_ERR_DEVICE;
  const size_t lds = ((size_t)V + 64 + 64 + 256) * sizeof(float);
  hipLaunchKernelGGL(sample_kernel, dim3(B), dim3(64), lds, reinterpret_cast<hipStream_t>(stream), V, logits,
                     temperature, top_p, top_k, u, codes);
  return hipGetLastError() == hipSuccess ? S2FAST_OK : S2FAST_ERR_HIP;
}

}  // extern "C"
