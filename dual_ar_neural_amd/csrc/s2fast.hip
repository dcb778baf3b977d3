// s2fast: persistent per-frame Fast-AR decoder for gfx950 (MI355X).
//
// One cooperative launch decodes one frame of one request: 256 blocks (one
// per CU) walk the nine decode steps together.  Every weight matrix is split
// by rows across the blocks and streamed once per step with non-temporal
// 16-byte loads.  Every phase's input depends on every block's outputs of
// the phase before.  Where those outputs are plain values, each block writes
// them as tagged values (the launch's tag beside each float) and the next
// phase's loads wait on the tags ("tag"); the attention phase's int64
// accumulator sums and its keys/values are read after a device-wide flag
// barrier ("sync").
//
// Per decode step k (window [hidden, emb(c_0), ..., emb(c_{k-1})], positions
// restart at 0; "Fast-AR codebook decoding and the generation main loop",
// sections 2-4) and per layer:
//   A  RMSNorm(x) -> fused wqkv rows                                  | tag
//   B  per KV group: q/k RMSNorm + pair RoPE + causal attention (mask
//      offset 0) -> wo restricted to the group's columns; the 8 group
//      partial sums meet in an int64 fixed-point accumulator          | sync
//   C  x_mid = x + attn; RMSNorm -> w1, w3 rows -> silu(a1) * a3      | tag
//   D  w2 rows; x = x_mid + ffn                                        | tag
// then fast_norm -> untied fast_output rows -> logits | tag, and the sampler
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
#include <mutex>
#include <new>
#include <vector>

using namespace s2f;

namespace {

struct LayerPtr {
  const void *attn_norm, *wqkv, *q_norm, *k_norm, *wo, *ffn_norm, *w1, *w3, *w2;
  // per-row float32 scales of int8 matrices (nullptr: the matrices carry their values)
  const float *s_qkv, *s_wo, *s_w1, *s_w3, *s_w2;
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
  const float* proj_scale;   // row scales of int8 fast_project_in / fast_output, or nullptr
  const float* out_scale;
  LayerPtr L[S2FAST_MAX_LAYERS];
  const float* rope;  // [2][ctx_len][hd/2]: cos then sin
  // Layer-0 q/k/v of every embedding row, [V][qkv_dim]:
  // wqkv . (attention_norm * e_c) / rms(e_c).  A new row at position >= 2
  // is fast_embeddings[c] of a code this block already knows, so its
  // layer-0 projection is a row of this table (built once per context).
  const float* qkv0;
  // the request this launch decodes
  const float* hidden;     // [in_dim]
  const int* sem_code;     // [1]
  const float* uniforms;   // [ncb-1]
  const float* temp;       // [1]
  const float* top_p;      // [1]
  const int* top_k;        // [1]
  const int* forced;       // teacher-forced codes (forced_ld of them), or nullptr
  int* codes_out;          // [ncb] or nullptr
  float* logits_out;       // [lo_rows][V] or nullptr
  int nsteps;              // decode steps this launch runs (ncb-1 for a whole frame)
  int forced_ld;           // codes per request in `forced`
  int lo_first, lo_rows;   // logits_out row of step s >= lo_first is s - lo_first
  // Per-frame arena.  Every (step, layer) output has its own 256-byte
  // aligned region, written once per frame.  The outputs of the wqkv, w1/w3,
  // w2 and head phases are tagged values (the launch's tag beside each
  // float): their readers wait on the tags with coherent loads and need no
  // grid sync, and every read of them is such a load.  The attention
  // accumulators (device atomics), the keys/values and fast_project_in's
  // output are read only after the grid sync that follows their writes, so
  // those readers may use ordinary L2-cacheable loads: no stale copy of
  // such a region can exist in any L2 (the kernel starts with an acquire
  // that invalidates lines cached by earlier frames).
  float* xin0;             // [dim] fast_project_in(hidden)
  u64* x;                  // [slot][MMAX][dim] residual stream after each layer (tagged)
  u64* qkv;                // [slot][MMAX][qkv_dim] (tagged)
  long long* acc;          // [slot][MMAX][dim] fixed-point attention output (zero between frames)
  u64* g;                  // [slot][MMAX][ffn] (tagged)
  float* kv;               // [n_layer][ctx][kv_pos] this frame's keys/values ([n_kv][2][hd] per position)
  int kv_pos;              // floats per position: n_kv * 2 * hd rounded up to a 128-byte line, so
                           // positions written at different steps never share a cache line
  u64* logits;             // [step][V] (tagged)
  long long x_slot, qkv_slot, acc_slot, g_slot, logits_slot;  // region strides (elements)
  u32* flags;              // [P][64] per-block barrier epochs
  u32 epoch0;              // epoch reached before this launch; epoch0 + 1 tags its outputs
  u32* err;                // watchdog words (see Watch)
  Watch watch;
  u32* tlog;               // optional [P][TLOG_MAX][TLOG_W] wall-clock marks
  u32 tlog_epoch;          // scratch for the marks: epoch at the phase start
};
constexpr int TLOG_MAX = 256;
constexpr int TLOG_W = 8;   // per sync point: phase done, released, then in-phase marks 2..7
constexpr int GEMV_RING = 4;   // weight chunks in flight per wave


// ---------------------------------------------------------------- LDS map
struct Lds {
  float* act;    // [MMAX][kmax] GEMV activations (see phys())
  float* red;    // [rmax][MMAX][NWAVE] per-wave GEMV partials
  float* small;  // [64]: rms scratch, epilogue temporaries
  float* q;      // [MMAX][gheads][hd]
  float* kc;     // [ctx][hd]
  float* vc;     // [ctx][hd]
  float* cval;   // [64] sampler candidates
  int* cidx;     // [64]
  u32* mark;     // [256] sampler cross-wave scratch
  int* codes;    // [16]
  int* flag;     // [8]: [0] grid sync result, [1] timeline record, [2..3] launch exit, [4] a tag wait gave up
  float* fnw;    // [dim] fast_norm weight (loaded once per frame)
  float* qkn;    // [n_layer][2][hd] q_norm and k_norm weights (loaded once per frame)
  float* rope;   // [2][ctx][hd/2] cos and sin (loaded once per frame)
  float* rsc;    // [rmax] the phase's row scales (int8 matrices; 1 otherwise)
};

__host__ __device__ inline size_t lds_floats(int kmax, int rmax, int gheads, int hd, int ctx, int V, int dim,
                                             int n_layer) {
  const size_t act = ((size_t)MMAX * kmax + 3) & ~(size_t)3;   // keeps the regions after it 16-byte aligned
  return act + (size_t)rmax * NWAVE * MMAX + 64 + (size_t)MMAX * gheads * hd + 2 * (size_t)ctx * hd +
         2 * TOPK_MAX + 256 + 16 + 8 + (size_t)dim + (size_t)n_layer * 2 * hd +
         (size_t)ctx * hd + (size_t)rmax;
}

__device__ inline Lds carve(float* base, const FrameArgs& a) {
  Lds s;
  const size_t act = ((size_t)MMAX * a.kmax + 3) & ~(size_t)3;
  float* p = base;
  s.act = p; p += act;
  s.red = p; p += (size_t)a.rmax * NWAVE * MMAX;
  s.small = p; p += 64;
  s.q = p; p += (size_t)MMAX * a.gheads * a.hd;
  s.kc = p; p += (size_t)a.ctx_len * a.hd;
  s.vc = p; p += (size_t)a.ctx_len * a.hd;
  s.cval = p; p += TOPK_MAX;
  s.cidx = reinterpret_cast<int*>(p); p += TOPK_MAX;
  s.mark = reinterpret_cast<u32*>(p); p += 256;
  s.codes = reinterpret_cast<int*>(p); p += 16;
  s.flag = reinterpret_cast<int*>(p); p += 8;
  s.fnw = p; p += a.dim;
  s.qkn = p; p += (size_t)a.n_layer * 2 * a.hd;
  s.rope = p; p += (size_t)a.ctx_len * a.hd;
  s.rsc = p;
  return s;
}

// window position of new row m at decode step `step`: rows 0 and 1 at step 1, row `step` after
__device__ __forceinline__ int row_pos(int step, int m) { return step == 1 ? m : step; }

// per-(step, layer) regions of the frame arena
__device__ __forceinline__ size_t slot_of(const FrameArgs& a, int step, int l) { return (size_t)(step - 1) * a.n_layer + l; }
__device__ __forceinline__ u64* xb(const FrameArgs& a, int step, int l) { return a.x + slot_of(a, step, l) * a.x_slot; }
__device__ __forceinline__ u64* qkvb(const FrameArgs& a, int step, int l) { return a.qkv + slot_of(a, step, l) * a.qkv_slot; }
__device__ __forceinline__ u64* gb(const FrameArgs& a, int step, int l) { return a.g + slot_of(a, step, l) * a.g_slot; }
__device__ __forceinline__ long long* accb(const FrameArgs& a, int step, int l) { return a.acc + slot_of(a, step, l) * a.acc_slot; }
__device__ __forceinline__ u64* logitsb(const FrameArgs& a, int step) { return a.logits + (size_t)(step - 1) * a.logits_slot; }
// tag of this launch's tagged outputs (never 0, the arena's cleared state)
__device__ __forceinline__ u32 out_tag(const FrameArgs& a) { return a.epoch0 + 1u; }

// plain (L2-cacheable) loads of arena data
__device__ __forceinline__ u64 ld64(const void* p) { return *reinterpret_cast<const u64*>(p); }

// The thread index through an opaque move: values derived from it are then
// computed where they are used instead of being hoisted out of the frame's
// phase loop, where they would stay live (and spill) across every phase.
__device__ __forceinline__ int tidx() {
  int t;
  asm volatile("v_mov_b32 %0, %1" : "=v"(t) : "v"((int)threadIdx.x));
  return t;
}

// Number of `width`-item steps of a staging batch at `base` over n items, through
// an opaque scalar move.  The consuming half of a batch bounds its loop with
// this value instead of repeating the loading half's test: the compiler can
// then not treat the two halves as control-equivalent and hoist conversions
// of loaded values (each with a wait on its load) above the weight prologue
// issued between them.
__device__ __forceinline__ int steps_opaque(int n, int base, int width = NTHREADS) {
  const int k = (n - base + width - 1) / width;
  int r;
  asm volatile("s_mov_b32 %0, %1" : "=s"(r) : "s"(k));
  return r;
}

// rows [r0, r1) of an n-row matrix owned by part `j` of `parts`
// (n * parts stays far below 2^32 for every matrix here)
__device__ __forceinline__ void split_rows(int n, int j, int parts, int& r0, int& r1) {
  r0 = (int)(((unsigned)n * (unsigned)j) / (unsigned)parts);
  r1 = (int)(((unsigned)n * (unsigned)(j + 1)) / (unsigned)parts);
}

// --------------------------------------------------------------- grid sync
// Device-wide barrier.  Every thread first waits for its own stores
// (vmcnt(0); no weight loads are in flight here), the block meets at
// s_barrier, then wave 0 publishes the block's epoch and polls every block's
// flag with coherent loads.  Returns false (after raising the watchdog word)
// if a flag does not arrive within SPIN_LIMIT polls; the caller then leaves
// the kernel.  With LOG, instrumented runs record the arrival and release
// times under the sync's index (callers that number their records
// otherwise pass false).
template <typename Args, bool LOG = true>
__device__ __forceinline__ bool grid_sync(const Args& a, u32& epoch, int* lds_flag) {
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this thread's output stores are done
  __syncthreads();
  const u32 idx = epoch - a.epoch0;
  if (LOG && a.tlog && tidx() == 0 && idx < TLOG_MAX)
    a.tlog[((size_t)blockIdx.x * TLOG_MAX + idx) * TLOG_W] = (u32)wall_clock64();
  ++epoch;
  if (tidx() < 64) {
    const int lane = tidx();
    const int P = gridDim.x;
    if (lane == 0) st_coh(a.flags + 64 * blockIdx.x, epoch);
    // the epoch to wait for; the test hook waits for one no block publishes
    const u32 want = a.watch.give_up ? epoch + 0x40000000u : epoch;
    const u32 limit = a.watch.give_up ? 1u : SPIN_LIMIT;
    u32 spins = 0;
    bool ok = true;
    while (true) {
      // the first four flags of a lane are loaded unconditionally, so all four
      // are in flight together (guarded or short-circuit loads would cost one
      // memory round trip each); blocks beyond 256 are polled after them
      u32 f[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) f[q] = ld_coh(a.flags + 64 * min(lane + 64 * q, P - 1));
      bool done = (f[0] >= want) & (f[1] >= want) & (f[2] >= want) & (f[3] >= want);
      for (int b = lane + 256; b < P; b += 64) done &= ld_coh(a.flags + 64 * b) >= want;
      if (__ballot(done) == ~0ull) break;
      if (++spins > limit) { ok = false; break; }
    }
    if (lane == 0) {
      if (!ok) atomicOr(a.err + W_ERR, 1u);
      lds_flag[0] = ok ? 0 : 1;
      if (LOG && a.tlog && idx < TLOG_MAX) a.tlog[((size_t)blockIdx.x * TLOG_MAX + idx) * TLOG_W + 1] = (u32)wall_clock64();
    }
  }
  __syncthreads();
  return lds_flag[0] == 0;
}


// End of a launch.  Every block counts itself out; the last one out finds
// whether any barrier wait of the launch gave up (the watchdog word).  If so
// it runs `recover` with all of its threads (restore the state the next
// launch relies on, and write the outputs the failure convention asks for),
// raises the context's sticky status, which s2fast_status reports, and
// clears the watchdog word.  It also resets the exit count for the next
// launch.  Every block reaches this point: each barrier wait is bounded.
template <typename Args, typename Recover>
__device__ __forceinline__ void launch_exit(const Args& a, int* lds_flag, const Recover& recover) {
  wait_vmem();
  __syncthreads();
  if (tidx() == 0) {
    const u32 n = __hip_atomic_fetch_add(a.err + W_EXITS, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    lds_flag[2] = (n + 1 == gridDim.x) ? 1 : 0;
    lds_flag[3] = lds_flag[2] ? (int)ld_coh(a.err + W_ERR) : 0;
  }
  __syncthreads();
  if (!lds_flag[2]) return;
  if (lds_flag[3]) {
    recover();
    wait_vmem();
    __syncthreads();
    if (tidx() == 0) {
      atomicOr(a.err + W_STATUS, 1u);
      st_coh(a.err + W_ERR, 0u);
    }
  }
  if (tidx() == 0) st_coh(a.err + W_EXITS, 0u);
}

// Zero n 8-byte words with every thread of the block (recovery only).
__device__ __forceinline__ void zero_words64(long long* p, size_t n) {
  for (size_t i = tidx(); i < n; i += NTHREADS) st_coh(p + i, 0ll);
}
__device__ __forceinline__ void zero_words32(int* p, size_t n) {
  for (size_t i = tidx(); i < n; i += NTHREADS) st_coh(p + i, 0);
}

// in-phase timeline mark (instrumented runs only): word w of the current
// phase's record, by thread 0
template <typename Args>
__device__ __forceinline__ void mark(const Args& a, u32 phase, int w) {
  if (a.tlog && tidx() == 0 && phase < TLOG_MAX)
    a.tlog[((size_t)blockIdx.x * TLOG_MAX + phase) * TLOG_W + w] = (u32)wall_clock64();
}

// --------------------------------------------------------------- staging
// Cross-block inputs (arena regions) are read with plain 8-byte loads.  Every
// helper issues a batch of independent loads per thread before using any of
// them, so a phase pays about one memory round trip for its activations.
// Position of natural element k of a GEMV activation row of width K in LDS.
// For bf16 weights a lane consumes 8 columns (16 bytes of weights) per load;
// its 8 activation floats are kept as two 16-byte halves in two separate
// half-rows, so each half is one conflict-free ds_read_b128 across the wave
// (lane-consecutive 16-byte addresses); int8 weights (16 columns a load) use
// four quarter-rows the same way.  f32 weights consume 4 columns, which is
// already one lane-consecutive 16-byte read: identity.
template <typename WT>
__device__ __forceinline__ int phys(int k, int K) {
  // G = EPL / 4 groups of four columns per lane load; group g of segment sg
  // sits at sg * 4 in the g-th of G equal parts of the row
  constexpr int EPL = WTraits<WT>::EPL, G = EPL / 4;
  if (G == 1) return k;
  return ((k / EPL) << 2) + (k & 3) + ((k >> 2) % G) * (K / G);
}

typedef float v4f __attribute__((ext_vector_type(4)));         // native vectors stay in registers
typedef long long v2ll __attribute__((ext_vector_type(2)));

// Activation staging.  A batch covers NS steps of NTHREADS 16-byte quads
// (four consecutive floats); step j of thread t takes quad base + j*NTHREADS
// + t.  All loads of a batch are issued before any is used and none is
// guarded: a step past the end re-reads the thread's first quad of the
// batch (the cache lines its first load fetched), so every address stays in
// bounds.  The first batch takes a hook that runs right after its loads are
// issued; the phase issues its weight prologue there, so the activation
// loads it waits on are not queued behind a chip-wide burst of weight loads.
// The consuming half of a batch is bounded by the opaque step count.
struct NoHook {
  __device__ __forceinline__ void operator()() const {}
};

__device__ __forceinline__ int quad_of(int base, int j, int nq) {
  const int q = base + j * NTHREADS + tidx();
  return q < nq ? q : min(base + tidx(), nq - 1);
}

// Four consecutive weights w[4c..4c+3] in their storage format: 8 bytes for
// bf16, 16 for f32.
template <typename WT> struct WQuad;
template <> struct WQuad<uint16_t> {
  using type = u64;
  __device__ static __forceinline__ type load(const uint16_t* w, int c) {
    return *gbl(reinterpret_cast<const u64*>(w + 4 * c));
  }
  __device__ static __forceinline__ float get(type b, int e) { return __uint_as_float((u32)(b >> (16 * e)) << 16); }
};
template <> struct WQuad<float> {
  using type = v4f;
  __device__ static __forceinline__ type load(const float* w, int c) {
    return *gbl(reinterpret_cast<const v4f*>(w + 4 * c));
  }
  __device__ static __forceinline__ float get(type b, int e) { return b[e]; }
};

// n floats (n a multiple of 4, src 16-byte aligned) of arena data into LDS;
// PERM places them for a GEMV over K = n columns (four consecutive columns
// stay consecutive in that layout).
template <typename WT, bool PERM, int NS, typename Hook>
__device__ __forceinline__ void stage_arena(float* dst, const float* src, int n, const Hook& hook) {
  const int nq = n >> 2;
  auto batch = [&](int base, const auto& after) __attribute__((always_inline)) {
    v4f v[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) v[j] = *reinterpret_cast<const v4f*>(src + 4 * quad_of(base, j, nq));
    after();
    const int nj = steps_opaque(nq, base);
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      if (j >= nj) break;
      const int q = base + j * NTHREADS + tidx();
      if (q < nq) *reinterpret_cast<v4f*>(dst + (PERM ? phys<WT>(4 * q, n) : 4 * q)) = v[j];
    }
  };
  batch(0, hook);
  for (int base = NTHREADS * NS; base < nq; base += NTHREADS * NS) batch(base, NoHook{});
}

// Wait until the tagged words t[0..N) all carry `tag`.  The caller has
// issued their first loads (ordinary ones, from addr(i)) before using any of
// them; the words still stale are loaded again with coherent loads, all
// together, until every one is current.
// After SPIN_LIMIT rounds the watchdog word and the block's failure flag
// are raised and the stale values stand: the block leaves the kernel at the
// end of the phase.  The watchdog test hook (Watch) makes every tagged wait
// give up at once.
struct TagWait {
  u32* err;      // the launch's watchdog words
  int* fail;     // the block's failure flag (LDS)
  u32 tag;       // the tag this launch writes
  u32 give_up;   // test hook
};

template <int N, typename Addr>
__device__ __forceinline__ void tag_wait(const TagWait& w, u64 (&t)[N], const Addr& addr) {
  const u32 tag = w.tag;
  if (w.give_up) {
    atomicOr(w.err + W_ERR, 1u);
    *w.fail = 1;
    return;
  }
  bool stale = false;
#pragma unroll
  for (int i = 0; i < N; ++i) stale |= !tag_is(t[i], tag);
  u32 spins = 0;
  while (stale) {
#pragma unroll
    for (int i = 0; i < N; ++i)
      if (!tag_is(t[i], tag)) t[i] = ld_coh64(addr(i));
    stale = false;
#pragma unroll
    for (int i = 0; i < N; ++i) stale |= !tag_is(t[i], tag);
    if (stale && ++spins > SPIN_LIMIT) {
      atomicOr(w.err + W_ERR, 1u);
      *w.fail = 1;
      break;
    }
  }
}

// the frame kernel's tagged waits: failure flag flag[4]
__device__ __forceinline__ TagWait frame_tw(const FrameArgs& a, const Lds& s) {
  return TagWait{a.err, s.flag + 4, out_tag(a), a.watch.give_up};
}

// A step's logits as this launch's tagged values, for the sampler: the
// loads wait on their tags.
struct TaggedLogits {
  TagWait w;
  const u64* L;
  template <int VPT>
  __device__ __forceinline__ void load(float (&x)[VPT], int tid, int V) const {
    u64 t[VPT];
#pragma unroll
    for (int j = 0; j < VPT; ++j) t[j] = ld_tagged(L + min(tid + j * NTHREADS, V - 1));
    tag_wait(w, t, [&](int j) __attribute__((always_inline)) { return L + min(tid + j * NTHREADS, V - 1); });
#pragma unroll
    for (int j = 0; j < VPT; ++j) x[j] = (tid + j * NTHREADS < V) ? tag_val(t[j]) : -INFINITY;
  }
};

// n tagged floats (n a multiple of 4) of this launch into LDS in the GEMV
// layout over K = n columns, as stage_arena, each load waiting on its tag.
template <typename WT, int NS, typename Hook>
__device__ __forceinline__ void stage_tagged(const TagWait& w, float* dst, const u64* src, int n, const Hook& hook) {
  const int nq = n >> 2;
  auto batch = [&](int base, const auto& after) __attribute__((always_inline)) {
    u64 t[4 * NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const u64* p = src + 4 * quad_of(base, j, nq);
      ld_tagged2(p, t[4 * j], t[4 * j + 1]);
      ld_tagged2(p + 2, t[4 * j + 2], t[4 * j + 3]);
    }
    after();
    tag_wait(w, t, [&](int i) __attribute__((always_inline)) {
      return src + 4 * quad_of(base, i >> 2, nq) + (i & 3);
    });
    const int nj = steps_opaque(nq, base);
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      if (j >= nj) break;
      const int q = base + j * NTHREADS + tidx();
      if (q < nq) {
        v4f o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = tag_val(t[4 * j + e]);
        *reinterpret_cast<v4f*>(dst + phys<WT>(4 * q, n)) = o;
      }
    }
  };
  batch(0, hook);
  for (int base = NTHREADS * NS; base < nq; base += NTHREADS * NS) batch(base, NoHook{});
}

// Per-wave partial sums of squares of rows 0 and 1 into small[m * NWAVE + wave].
__device__ __forceinline__ void store_ss(float* small, int M, float ss0, float ss1) {
  const int wave = tidx() >> 6, lane = tidx() & 63;
  const float t0 = wave_sum(ss0);
  const float t1 = wave_sum(ss1);
  if (lane == 0) {
    small[wave] = t0;
    if (M > 1) small[NWAVE + wave] = t1;
  }
}

// sqrt(mean(x_m^2) + eps) of row m over K columns from the per-wave partials
__device__ __forceinline__ float norm_den(const float* small, int m, int K, float eps) {
  float t = 0.0f;
#pragma unroll
  for (int w = 0; w < NWAVE; ++w) t += small[m * NWAVE + w];
  return sqrtf(t / (float)K + eps);
}

// Layer input x of the M new rows into LDS act rows (GEMV layout over dim
// columns), already multiplied by this phase's RMSNorm weight; with ADD_ACC
// the fixed-point attention accumulator is added first (x_mid = x + attention
// output).  The RMS itself divides the GEMV outputs (norm_den): the row
// sums of squares are left as per-wave partials in small[m * NWAVE + wave].
// TAGGED: layers >= 1, whose input is the previous layer's tagged output.
template <typename WT, bool ADD_ACC, bool TAGGED, typename Hook>
__device__ __forceinline__ void stage_rows(const FrameArgs& a, const Lds& s, int l, int step, int M,
                                           const typename VecOf<WT>::type* normw, const Hook& hook) {
  using VT = typename VecOf<WT>::type;
  constexpr int NS = TAGGED ? 2 : 3;
  const int hq = a.dim >> 2;
  const int nq = M * hq;
  // float32 source rows: the previous layer's output, or at layer 0 the
  // hidden state (through fast_project_in when present) at window position 0;
  // layer 0 at positions j >= 1 takes fast_embeddings[c_{j-1}]
  // ("Fast-AR codebook decoding ...", section 2)
  const u64* tsrc = TAGGED ? xb(a, step, l - 1) : nullptr;
  const float* fsrc = a.has_proj ? a.xin0 : a.hidden;
  float ss0 = 0.0f, ss1 = 0.0f;
  auto batch = [&](int base, const auto& after) __attribute__((always_inline)) {
    u64 t[TAGGED ? 4 * NS : 1];
    v4f xv[NS];
    v2ll a0[NS], a1[NS];
    typename WQuad<VT>::type wv[NS], ev[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int q = quad_of(base, j, nq);
      const int m = q >= hq ? 1 : 0, c = q - m * hq;   // M <= 2
      wv[j] = WQuad<VT>::load(normw, c);   // the RMSNorm weight, same round trip
      if constexpr (TAGGED) {
        const u64* p = tsrc + (size_t)m * a.dim + 4 * c;
        ld_tagged2(p, t[4 * j], t[4 * j + 1]);
        ld_tagged2(p + 2, t[4 * j + 2], t[4 * j + 3]);
      } else {
        xv[j] = *reinterpret_cast<const v4f*>(fsrc + 4 * c);
        // position >= 1: the embedding row of the previous code (otherwise
        // row 0, loaded and not used, so that the load needs no branch)
        const int pos = row_pos(step, m);
        const int code = pos > 0 ? s.codes[max(pos - 1, 0)] : 0;
        ev[j] = WQuad<VT>::load(reinterpret_cast<const VT*>(a.emb) + (size_t)code * a.dim, c);
      }
      if (ADD_ACC) {
        const long long* ac = accb(a, step, l) + (size_t)m * a.dim + 4 * c;
        a0[j] = *reinterpret_cast<const v2ll*>(ac);
        a1[j] = *reinterpret_cast<const v2ll*>(ac + 2);
      }
    }
    after();
    if constexpr (TAGGED)
      tag_wait(frame_tw(a, s), t, [&](int i) __attribute__((always_inline)) {
        const int q = quad_of(base, i >> 2, nq);
        const int m = q >= hq ? 1 : 0, c = q - m * hq;
        return tsrc + (size_t)m * a.dim + 4 * c + (i & 3);
      });
    const int nj = steps_opaque(nq, base);
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      if (j >= nj) break;
      const int qu = base + j * NTHREADS + tidx();
      const int q = min(qu, nq - 1);
      const int m = q >= hq ? 1 : 0, c = q - m * hq;
      float v[4];
      if constexpr (TAGGED) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = tag_val(t[4 * j + e]);
      } else {
        const bool emb = row_pos(step, m) > 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = emb ? WQuad<VT>::get(ev[j], e) : xv[j][e];
      }
      if (ADD_ACC) {
        v[0] += from_fx(a0[j][0]); v[1] += from_fx(a0[j][1]);
        v[2] += from_fx(a1[j][0]); v[3] += from_fx(a1[j][1]);
      }
      if (qu < nq) {
        float t2 = (m == 0) ? ss0 : ss1;
#pragma unroll
        for (int e = 0; e < 4; ++e) t2 = fmaf(v[e], v[e], t2);
        if (m == 0) ss0 = t2; else ss1 = t2;
        v4f o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = v[e] * WQuad<VT>::get(wv[j], e);
        *reinterpret_cast<v4f*>(s.act + (size_t)m * a.kmax + phys<WT>(4 * c, a.dim)) = o;
      }
    }
  };
  batch(0, hook);
  for (int base = NTHREADS * NS; base < nq; base += NTHREADS * NS) batch(base, NoHook{});
  store_ss(s.small, M, ss0, ss1);
}

template <typename WT, bool ADD_ACC, typename Hook>
__device__ __forceinline__ void stage_layer_input(const FrameArgs& a, const Lds& s, int l, int step, int M,
                                                  const typename VecOf<WT>::type* normw, const Hook& hook) {
  if (l > 0) stage_rows<WT, ADD_ACC, true>(a, s, l, step, M, normw, hook);
  else stage_rows<WT, ADD_ACC, false>(a, s, l, step, M, normw, hook);
}

// --------------------------------------------------------------- GEMV
// A "chunk" is 64 consecutive 16-byte segments of one weight row (one load
// per lane, 1 KB per wave).  A block's GEMV covers virtual rows [0, nrows)
// of up to two matrices with the same column range (rows < nr_a from
// matrix a, the rest from matrix b: w1 and w3 of the SwiGLU run as one
// GEMV).  Each wave takes a contiguous range of the block's chunks and
// leaves per-(row, wave, m) partial sums in red, which the caller zeroes
// beforehand and reduces in wave order.
//
// Weight loads go into a ring of RING register slots: each step issues the
// load RING-1 chunks ahead and consumes the oldest, so RING-1 chunks stay in
// flight while one is multiplied.  The loads are ordinary non-temporal loads
// the compiler sees, so it places the vmcnt waits itself (in-order retirement
// lets it wait for exactly the slot being consumed).  Every issue step loads
// one 16-byte value per lane, a valid dummy address past the wave's range.
//
// The first RING-1 loads of a phase (its "prologue") are issued when the
// phase starts, before its activation staging and normalisation, which they
// overlap.  A phase's slots never outlive the phase: nothing in flight is
// carried across the grid barrier or the phase loop.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int RING = GEMV_RING;

__device__ __forceinline__ void load16_nt(u32x4& d, const void* p) {
  d = __builtin_nontemporal_load(gbl(reinterpret_cast<const u32x4*>(p)));
}

struct Plan {
  const char* base_a;   // block's first row in matrix a (bytes)
  const char* base_b;   // block's first row in matrix b
  const char* dummy;    // always-valid address for loads past the range
  long long row_bytes;
  int nr_a, nrows, K, S, C, t0, t1;
  int it, ir, ic;       // issue cursor
  const char* irow;
  int r0, r1, g;        // the block's output rows [r0, r1) (and KV group for wo)
};

template <typename WT>
__device__ __forceinline__ Plan make_plan(const WT* Wa, const WT* Wb, long long ldw, int col0, int K, int row0,
                                          int nr_a, int nrows) {
  constexpr int EPL = WTraits<WT>::EPL;
  Plan p;
  p.row_bytes = ldw * (long long)sizeof(WT);
  p.base_a = reinterpret_cast<const char*>(Wa + (long long)row0 * ldw + col0);
  p.base_b = Wb ? reinterpret_cast<const char*>(Wb + (long long)row0 * ldw + col0) : p.base_a;
  p.dummy = reinterpret_cast<const char*>(Wa);
  p.nr_a = nr_a;
  p.nrows = nrows;
  p.K = K;
  p.S = K / EPL;
  p.C = (p.S + 63) >> 6;
  const int T = nrows * p.C;
  const int wave = __builtin_amdgcn_readfirstlane(tidx() >> 6);   // the plan is wave-uniform
  p.t0 = (int)(((long long)T * wave) / NWAVE);
  p.t1 = (int)(((long long)T * (wave + 1)) / NWAVE);
  p.it = p.t0;
  p.ir = p.C ? p.t0 / p.C : 0;
  p.ic = p.t0 - p.ir * p.C;
  p.irow = (p.ir < nr_a) ? p.base_a + (long long)p.ir * p.row_bytes : p.base_b + (long long)(p.ir - nr_a) * p.row_bytes;
  return p;
}

__device__ __forceinline__ void plan_issue(Plan& p, u32x4& d) {
  const int lane = tidx() & 63;
  const char* addr = p.dummy;
  if (p.it < p.t1) {
    const int seg = p.ic * 64 + lane;
    addr = (seg < p.S) ? p.irow + (long long)seg * 16 : p.irow;
    ++p.it;
    if (++p.ic == p.C) {
      p.ic = 0;
      ++p.ir;
      p.irow = (p.ir < p.nr_a) ? p.base_a + (long long)p.ir * p.row_bytes
                               : p.base_b + (long long)(p.ir - p.nr_a) * p.row_bytes;
    }
  }
  load16_nt(d, addr);
}

// The scheduling fences keep the prologue's loads together where the phase
// places them: the scheduler would otherwise interleave the consumers of the
// staging loads issued just before, each with a wait on those loads, between
// the weight loads.
template <int R>
__device__ __forceinline__ void gemv_prologue(Plan& p, u32x4 (&slot)[R]) {
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < R - 1; ++j) plan_issue(p, slot[j]);
  __builtin_amdgcn_sched_barrier(0);
}

// Body: consume the wave's chunks against MM activation rows in LDS (GEMV
// layout, row stride act_ld).  The chunk cursor is wave-uniform, so every
// branch here is a scalar branch; the per-lane tail of a row (segments past
// K) is handled by zeroing the lane's weights, not by a branch.
template <typename WT, int MM, int R>
__device__ __forceinline__ void gemv_rows(Plan& p, u32x4 (&slot)[R], const float* act, int act_ld, float* red) {
  constexpr int EPL = WTraits<WT>::EPL;
  const int wave = __builtin_amdgcn_readfirstlane(tidx() >> 6), lane = tidx() & 63;
  const int t0 = p.t0, t1 = p.t1;
  if (t0 >= t1) return;
  const int C = p.C, S = p.S;
  int cr = t0 / C, cc = t0 - cr * C;
  float acc[MM];
#pragma unroll
  for (int m = 0; m < MM; ++m) acc[m] = 0.0f;
  auto flush = [&](int r) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < MM; ++m) {
      const float v = wave_sum(acc[m]);
      if (lane == 0) red[((size_t)r * MMAX + m) * NWAVE + wave] = v;
      acc[m] = 0.0f;
    }
  };
  constexpr int G = EPL / 4;   // four-column groups a load covers (phys places group g in part g of G)
  const int Kg = p.K / G;
  auto consume = [&](const u32x4& q) __attribute__((always_inline)) {
    const int seg = cc * 64 + lane;
    const bool live = seg < S;
    const int sg = live ? seg : 0;
    float w[EPL];
    WTraits<WT>::unpack(make_uint4(q.x, q.y, q.z, q.w), w);
#pragma unroll
    for (int e = 0; e < EPL; ++e) w[e] = live ? w[e] : 0.0f;
#pragma unroll
    for (int m = 0; m < MM; ++m) {
      const float* row = act + (size_t)m * act_ld;
      float s0 = acc[m];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float4 x = *reinterpret_cast<const float4*>(row + (size_t)g * Kg + (size_t)sg * 4);
        s0 = fmaf(w[4 * g + 0], x.x, s0); s0 = fmaf(w[4 * g + 1], x.y, s0);
        s0 = fmaf(w[4 * g + 2], x.z, s0); s0 = fmaf(w[4 * g + 3], x.w, s0);
      }
      acc[m] = s0;
    }
    if (++cc == C) { cc = 0; flush(cr); ++cr; }
  };
  for (int t = t0; t < t1; t += R) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      plan_issue(p, slot[(r + R - 1) % R]);
      if (t + r < t1) consume(slot[r]);
    }
  }
  if (cc != 0) flush(cr);   // the wave's range ended inside a row
}

template <typename WT, int R>
__device__ __forceinline__ void gemv_body(Plan& p, u32x4 (&slot)[R], const float* act, int act_ld, int M,
                                          float* red) {
  if (M == 1) gemv_rows<WT, 1>(p, slot, act, act_ld, red);
  else gemv_rows<WT, 2>(p, slot, act, act_ld, red);
}

__device__ __forceinline__ void zero_lds(float* p, int n) {
  for (int i = tidx(); i < n; i += NTHREADS) p[i] = 0.0f;
}

// sum of the per-wave partials of row r, activation row m
static_assert(NWAVE == 8, "red_sum reads the wave partials as two float4");
__device__ __forceinline__ float red_sum(const float* red, int r, int m) {
  // the NWAVE partials of (r, m) are contiguous: two 16-byte LDS reads
  const float4* q = reinterpret_cast<const float4*>(red + ((size_t)r * MMAX + m) * NWAVE);
  const float4 a = q[0], b = q[1];
  return ((((((a.x + a.y) + a.z) + a.w) + b.x) + b.y) + b.z) + b.w;
}

// RMSNorm of M rows of K values held in LDS in GEMV layout, in place:
// x / sqrt(mean(x^2) + eps) * w ("Model loading and GGUF", section 2.2:
// eps 1e-6; Mizuoto page: computed in float32).

// Layer-0 input of new row m at window position pos, one element (used for
// the few rows a block owns in the w2 phase).
template <typename WT>
__device__ __forceinline__ float layer0_input(const FrameArgs& a, const Lds& s, int pos, int k) {
  using VT = typename VecOf<WT>::type;
  if (pos == 0) return a.has_proj ? a.xin0[k] : a.hidden[k];
  const VT* e = reinterpret_cast<const VT*>(a.emb) + (size_t)s.codes[pos - 1] * a.dim;
  return WTraits<VT>::one(e, k);
}

// One head vector per wave: RMSNorm with weight w (optional), then pair RoPE
// at position pos; in place in LDS.
__device__ __forceinline__ void head_norm_rope(float* v, int hd, const float* w, bool do_norm, float eps,
                                               const float* rope, int ctx, int pos) {
  const int lane = tidx() & 63;
  const bool own = 2 * lane < hd;   // lane owns the pair (2*lane, 2*lane+1)
  const int pl = own ? lane : 0;    // loads stay unconditional (see the attention scores)
  float x0 = v[2 * pl], x1 = v[2 * pl + 1];
  const float w0 = w[2 * pl], w1 = w[2 * pl + 1];
  const float c = rope[(size_t)pos * (hd / 2) + pl];
  const float sn = rope[(size_t)ctx * (hd / 2) + (size_t)pos * (hd / 2) + pl];
  if (!own) { x0 = 0.0f; x1 = 0.0f; }
  if (do_norm) {
    float ss = wave_sum(fmaf(x0, x0, x1 * x1));
    const float den = sqrtf(ss / (float)hd + eps);
    x0 = x0 / den * w0;
    x1 = x1 / den * w1;
  }
  if (own) {
    v[2 * lane] = x0 * c - x1 * sn;
    v[2 * lane + 1] = x0 * sn + x1 * c;
  }
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// x_mid of one element (the rows a block owns in the w2 phase)
template <typename WT>
__device__ __forceinline__ float x_mid_of(const FrameArgs& a, const Lds& s, int l, int step, int m, int k) {
  const float xin = (l == 0) ? layer0_input<WT>(a, s, row_pos(step, m), k)
                             : tag_val(ld_coh64(xb(a, step, l - 1) + (size_t)m * a.dim + k));   // current since the wqkv phase
  return xin + from_fx(accb(a, step, l)[(size_t)m * a.dim + k]);
}

// Scaled dot-product attention of one KV group, causal with offset 0: new
// row m sits at window position first_new + m and sees positions 0..that
// ("Fast-AR codebook decoding ...", section 3).  In LDS: q [M][gh][hd]
// (after q-norm and RoPE), kc / vc [positions][hd] (keys after k-norm and
// RoPE, values).  One wave per (row, head); row m's output of head hh goes
// to out + m * out_ld at the wo GEMV layout position of column hh * hd + d
// of the group's gw columns.
// Straight-line code: every LDS read is unconditional (clamped addresses)
// and masking is done on values, so the reads issue back to back; guarded
// reads would each become a branch with its own wait.  Positions: at most 16.
template <typename WT>
__device__ __forceinline__ void attend_rows(const float* q, const float* kc, const float* vc, int M, int first_new,
                                            int gh, int hd, float* out, int out_ld, int gw) {
  const int wave = tidx() >> 6, lane = tidx() & 63;
  const float scale = 1.0f / sqrtf((float)hd);
  const int g16 = lane >> 4, l16 = lane & 15;   // 16-lane row of the wave, lane in it
  const int d8 = min(8 * l16, hd - 8);          // lane's 8 head dims in the score pass (hd % 8 == 0)
  const bool dlive = 8 * l16 < hd;
  for (int pr = wave; pr < M * gh; pr += NWAVE) {
    const int m = pr / gh, hh = pr % gh;
    const int pos = first_new + m;
    const float* qv = q + (size_t)pr * hd;
    const float4 qa = *reinterpret_cast<const float4*>(qv + d8);
    const float4 qb = *reinterpret_cast<const float4*>(qv + d8 + 4);
    // scores: row g16 of the wave takes positions g16, g16+4, g16+8, g16+12
    float sc4[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = 4 * r + g16;
      const float* kr = kc + (size_t)min(j, pos) * hd + d8;
      const float4 ka = *reinterpret_cast<const float4*>(kr);
      const float4 kb = *reinterpret_cast<const float4*>(kr + 4);
      float part = qa.x * ka.x;
      part = fmaf(qa.y, ka.y, part); part = fmaf(qa.z, ka.z, part); part = fmaf(qa.w, ka.w, part);
      part = fmaf(qb.x, kb.x, part); part = fmaf(qb.y, kb.y, part);
      part = fmaf(qb.z, kb.z, part); part = fmaf(qb.w, kb.w, part);
      part = row16_sum(dlive ? part : 0.0f);
      sc4[r] = (j <= pos) ? part * scale : -INFINITY;
    }
    // softmax over positions 0..pos: exp(s - max) / sum
    float mx = fmaxf(fmaxf(sc4[0], sc4[1]), fmaxf(sc4[2], sc4[3]));
    mx = fmaxf(fmaxf(readlane_f(mx, 0), readlane_f(mx, 16)), fmaxf(readlane_f(mx, 32), readlane_f(mx, 48)));
    float e4[4], es = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      e4[r] = expf(sc4[r] - mx);    // exp(-inf) = 0 for masked positions
      es += e4[r];
    }
    const float den = (readlane_f(es, 0) + readlane_f(es, 16)) + (readlane_f(es, 32) + readlane_f(es, 48));
    // output: lanes over head dims; all 16 positions are read, masked ones
    // with weight 0 (the weights' normalisation is applied once to the output)
    const int c0 = min(lane, hd - 1), c1 = min(lane + 64, hd - 1);
    float o0 = 0.0f, o1 = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float* vr = vc + (size_t)min(j, pos) * hd;
      const float ej = readlane_f(e4[j >> 2], (j & 3) * 16);   // 0 past pos
      o0 = fmaf(ej, vr[c0], o0);
      o1 = fmaf(ej, vr[c1], o1);
    }
    o0 /= den;
    o1 /= den;
    float* o = out + (size_t)m * out_ld;
    if (lane < hd) o[phys<WT>(hh * hd + lane, gw)] = o0;
    if (lane + 64 < hd) o[phys<WT>(hh * hd + lane + 64, gw)] = o1;
  }
}

// Row scales of a phase's int8 matrices: the block's rows [0, nr_a) are
// rows r0.. of matrix a, rows [nr_a, nrows) rows r0.. of matrix b (w1 and
// w3).  row_scale_issue loads thread t's value at the phase start (its
// latency overlaps the activation staging); row_scale_store puts the values
// into LDS before the GEMV.  Without scales (bf16 and f32 models) every row
// scale is 1, which leaves the outputs unchanged.
__device__ __forceinline__ float row_scale_issue(const float* sa, const float* sb, int r0, int nr_a, int nrows) {
  if (!sa || nrows <= 0) return 1.0f;
  const int i = min(tidx(), nrows - 1);
  return i < nr_a ? sa[r0 + i] : sb[r0 + i - nr_a];
}
__device__ __forceinline__ void row_scale_store(float* rsc, float v, const float* sa, const float* sb, int r0,
                                                int nr_a, int nrows) {
  if (tidx() < nrows) rsc[tidx()] = v;
  for (int i = tidx() + NTHREADS; i < nrows; i += NTHREADS) rsc[i] = i < nr_a ? sa[r0 + i] : sb[r0 + i - nr_a];
}

// --------------------------------------------------------------- phases
enum PhaseKind { PH_PROJ = 0, PH_QKV, PH_WO, PH_FFN_UP, PH_FFN_DOWN, PH_HEAD };

struct PhaseId { int step, layer, kind; };

// Phase order of a frame: [fast_project_in], then per decode step 1..ncb-1
// the four phases of every layer and the output head, except that steps
// >= 2 start at layer 0's attention (their one new row's layer-0 q/k/v is a
// row of the qkv0 table).
__device__ __forceinline__ PhaseId first_phase(const FrameArgs& a) {
  PhaseId id;
  id.step = a.has_proj ? 0 : 1;
  id.layer = 0;
  id.kind = a.has_proj ? PH_PROJ : PH_QKV;
  return id;
}

__device__ __forceinline__ PhaseId next_phase(const FrameArgs& a, PhaseId id) {
  if (id.kind == PH_PROJ || id.kind == PH_HEAD) {
    ++id.step;
    id.layer = 0;
    id.kind = (id.step >= 2) ? PH_WO : PH_QKV;   // layer-0 q/k/v of later steps: the qkv0 table
  } else if (id.kind == PH_FFN_DOWN) {
    ++id.layer;
    id.kind = (id.layer == a.n_layer) ? PH_HEAD : PH_QKV;
    if (id.kind == PH_HEAD) id.layer = 0;
  } else {
    ++id.kind;
  }
  return id;
}

__device__ __forceinline__ int phase_count(const FrameArgs& a) {
  return (a.has_proj ? 1 : 0) + a.nsteps * (4 * a.n_layer + 1) - (a.nsteps - 1);
}

// rows of the wo phase: KV group g of this block and its share of the rows
__device__ __forceinline__ void wo_rows(const FrameArgs& a, int& g, int& r0, int& r1) {
  const int P = gridDim.x;
  g = blockIdx.x % a.n_kv;
  const int rg = blockIdx.x / a.n_kv;
  const int Pg = (P - g + a.n_kv - 1) / a.n_kv;
  split_rows(a.dim, rg, Pg, r0, r1);
}

template <typename WT>
__device__ __forceinline__ Plan plan_for(const FrameArgs& a, PhaseId id) {
  const int P = gridDim.x, b = blockIdx.x;
  int r0, r1, g = 0;
  const LayerPtr& L = a.L[id.layer];
  Plan p;
  switch (id.kind) {
    case PH_PROJ:
      split_rows(a.dim, b, P, r0, r1);
      p = make_plan<WT>((const WT*)a.proj, nullptr, a.in_dim, 0, a.in_dim, r0, r1 - r0, r1 - r0);
      break;
    case PH_QKV:
      split_rows(a.qkv_dim, b, P, r0, r1);
      p = make_plan<WT>((const WT*)L.wqkv, nullptr, a.dim, 0, a.dim, r0, r1 - r0, r1 - r0);
      break;
    case PH_WO:
      wo_rows(a, g, r0, r1);
      p = make_plan<WT>((const WT*)L.wo, nullptr, a.attn_dim, g * a.gw, a.gw, r0, r1 - r0, r1 - r0);
      break;
    case PH_FFN_UP:
      split_rows(a.ffn, b, P, r0, r1);
      p = make_plan<WT>((const WT*)L.w1, (const WT*)L.w3, a.dim, 0, a.dim, r0, r1 - r0, 2 * (r1 - r0));
      break;
    case PH_FFN_DOWN:
      split_rows(a.dim, b, P, r0, r1);
      p = make_plan<WT>((const WT*)L.w2, nullptr, a.ffn, 0, a.ffn, r0, r1 - r0, r1 - r0);
      break;
    default:
      split_rows(a.V, b, P, r0, r1);
      p = make_plan<WT>((const WT*)a.outw, nullptr, a.dim, 0, a.dim, r0, r1 - r0, r1 - r0);
      break;
  }
  p.r0 = r0;
  p.r1 = r1;
  p.g = g;
  return p;
}

template <typename WT>
__device__ __forceinline__ void phase_qkv(const FrameArgs& a, const Lds& s, int l, int step, int M, Plan& pl) {
  using VT = typename VecOf<WT>::type;
  const int D = a.dim;
  const int r0 = pl.r0, r1 = pl.r1;
  const float* sq = a.L[l].s_qkv;
  const float scv = row_scale_issue(sq, nullptr, r0, r1 - r0, r1 - r0);
  u32x4 slot[RING];
  const auto pro = [&]() __attribute__((always_inline)) { gemv_prologue(pl, slot); };
  stage_layer_input<WT, false>(a, s, l, step, M, reinterpret_cast<const VT*>(a.L[l].attn_norm), pro);
  row_scale_store(s.rsc, scv, sq, nullptr, r0, r1 - r0, r1 - r0);
  zero_lds(s.red, (r1 - r0) * NWAVE * MMAX);
  __syncthreads();
  mark(a, s.flag[1], 4);
  mark(a, s.flag[1], 2);
  gemv_body<WT>(pl, slot, s.act, a.kmax, M, s.red);
  __syncthreads();
  mark(a, s.flag[1], 3);
  for (int i = tidx(); i < (r1 - r0) * M; i += NTHREADS) {
    const int r = i / M, m = i % M;
    st_tagged(qkvb(a, step, l) + (size_t)m * a.qkv_dim + r0 + r,
              s.rsc[r] * red_sum(s.red, r, m) / norm_den(s.small, m, D, a.eps), out_tag(a));
  }
}

template <typename WT>
__device__ __forceinline__ void phase_attn_wo(const FrameArgs& a, const Lds& s, int l, int step, int M, Plan& pl) {
  const int g = pl.g, r0 = pl.r0, r1 = pl.r1;
  const int rg = blockIdx.x / a.n_kv;
  const int hd = a.hd, H = a.n_head, G = a.n_kv, gh = a.gheads;
  const int first_new = (step == 1) ? 0 : step;   // positions < first_new come from this frame's cache
  const int wave = tidx() >> 6, lane = tidx() & 63;
  const float* qn = s.qkn + (size_t)l * 2 * hd;
  const float* kn = qn + hd;
  float* kvl = a.kv + (size_t)l * a.ctx_len * a.kv_pos;   // [ctx][kv_pos]
  const bool need_attn = (r1 > r0) || rg == 0;
  const float* so = a.L[l].s_wo;
  const float scv = row_scale_issue(so, nullptr, r0, r1 - r0, r1 - r0);
  zero_lds(s.red, (r1 - r0) * NWAVE * MMAX);   // the GEMV's partial sums (read after the barriers below)
  u32x4 slot[RING];
  const auto pro = [&]() __attribute__((always_inline)) { gemv_prologue(pl, slot); };
  {
    // One gather of head vectors (segments of hd floats) into LDS: the cached
    // keys of positions < first_new, their values, then per new row its gh
    // raw query heads (this group's), its key and its value.  Nothing for a
    // block without wo rows outside the first row group.  A wave takes
    // segments wave, wave + NWAVE, ...; the segment arithmetic is
    // wave-uniform and a lane moves one pair of floats.
    constexpr int NS = 4;
    const int F = first_new, hp = hd >> 1;
    // new rows' q/k/v: this step's wqkv phase output (tagged), or at layer 0
    // of steps >= 2 the qkv0 row of the code that produced the row
    const bool table = (l == 0 && step >= 2);
    const float* qkv_tab = a.qkv0 + (size_t)(table ? s.codes[step - 1] : 0) * a.qkv_dim;
    const u64* qkv_new = qkvb(a, step, l);
    const u32 tag = out_tag(a);
    const int nseg = need_attn ? 2 * F + M * (gh + 2) : 0;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int lp = min(lane, hp - 1);
    // segment sg: its LDS destination, and its source as a cache row (src)
    // or as an offset into the new rows' q/k/v (off, with src null)
    auto seg = [&](int sg, const float*& src, long long& off, float*& dst) __attribute__((always_inline)) {
      src = nullptr;
      off = 0;
      if (sg < F) {
        src = kvl + (sg * a.kv_pos + (g * 2 + 0) * hd);
        dst = s.kc + (size_t)sg * hd;
      } else if (sg < 2 * F) {
        src = kvl + ((sg - F) * a.kv_pos + (g * 2 + 1) * hd);
        dst = s.vc + (size_t)(sg - F) * hd;
      } else {
        const int t = sg - 2 * F;
        const int m = t >= gh + 2 ? 1 : 0, r = t - m * (gh + 2);   // M <= 2
        const int pos = row_pos(step, m);
        off = (long long)m * a.qkv_dim;
        if (r < gh) {
          off += (long long)(g * gh + r) * hd;
          dst = s.q + (size_t)(m * gh + r) * hd;
        } else if (r == gh) {
          off += (long long)(H + g) * hd;
          dst = s.kc + (size_t)pos * hd;
        } else {
          off += (long long)(H + G + g) * hd;
          dst = s.vc + (size_t)pos * hd;
        }
        if (table) src = qkv_tab + off;
      }
    };
    auto batch = [&](int base, const auto& after) __attribute__((always_inline)) {
      // two tagged words per lane and segment; a plain pair (cache row or
      // qkv0 row) is given this launch's tag, so only new rows are waited on
      u64 t[2 * NS];
      long long offs[NS];
      float* dst[NS];
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        // a step past the end re-reads segment 0 (a valid row when nseg is 0)
        const int sg = base + wv + NWAVE * j;
        const float* src;
        seg(sg < nseg ? sg : 0, src, offs[j], dst[j]);
        if (src) {
          const u64 v = ld64(src + 2 * lp);
          t[2 * j] = ((u64)tag << 32) | (v & 0xFFFFFFFFull);
          t[2 * j + 1] = ((u64)tag << 32) | (v >> 32);
        } else {
          ld_tagged2(qkv_new + offs[j] + 2 * lp, t[2 * j], t[2 * j + 1]);
        }
      }
      after();
      tag_wait(frame_tw(a, s), t, [&](int i) __attribute__((always_inline)) {
        return qkv_new + offs[i >> 1] + 2 * lp + (i & 1);
      });
      const int nj = steps_opaque(nseg, base, NWAVE);
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        if (j >= nj) break;
        if (base + wv + NWAVE * j < nseg && lane < hp) {
          dst[j][2 * lane] = tag_val(t[2 * j]);
          dst[j][2 * lane + 1] = tag_val(t[2 * j + 1]);
        }
      }
    };
    batch(0, pro);
    for (int base = NWAVE * NS; base < nseg; base += NWAVE * NS) batch(base, NoHook{});
  }
  if (need_attn) {
    __syncthreads();
    mark(a, s.flag[1], 4);
      // q/k RMSNorm + RoPE: one wave per head vector
    const int nvec = M * gh + M;
    for (int v = wave; v < nvec; v += NWAVE) {
      if (v < M * gh) {
        const int m = v / gh;
        head_norm_rope(s.q + (size_t)v * hd, hd, qn, a.has_qkn, a.eps, s.rope, a.ctx_len, row_pos(step, m));
      } else {
        const int m = v - M * gh;
        const int pos = row_pos(step, m);
        head_norm_rope(s.kc + (size_t)pos * hd, hd, kn, a.has_qkn, a.eps, s.rope, a.ctx_len, pos);
      }
    }
    __syncthreads();
    mark(a, s.flag[1], 6);
    // keep this step's keys/values for later steps of the frame
    if (rg == 0) {
      for (int m = 0; m < M; ++m) {
        const int pos = row_pos(step, m);
        for (int d = tidx(); d < hd; d += NTHREADS) {
          st_coh(kvl + (pos * a.kv_pos + (g * 2 + 0) * hd + d), s.kc[(size_t)pos * hd + d]);
          st_coh(kvl + (pos * a.kv_pos + (g * 2 + 1) * hd + d), s.vc[(size_t)pos * hd + d]);
        }
      }
    }
    attend_rows<WT>(s.q, s.kc, s.vc, M, first_new, gh, hd, s.act, a.kmax, a.gw);
    mark(a, s.flag[1], 7);
  }
  row_scale_store(s.rsc, scv, so, nullptr, r0, r1 - r0, r1 - r0);
  __syncthreads();
  mark(a, s.flag[1], 2);
  gemv_body<WT>(pl, slot, s.act, a.kmax, M, s.red);
  __syncthreads();
  mark(a, s.flag[1], 3);
  for (int i = tidx(); i < (r1 - r0) * M; i += NTHREADS) {
    const int r = i / M, m = i % M;
    atomic_add_coh(accb(a, step, l) + (size_t)m * a.dim + r0 + r, to_fx(s.rsc[r] * red_sum(s.red, r, m)));
  }
}

template <typename WT>
__device__ __forceinline__ void phase_ffn_up(const FrameArgs& a, const Lds& s, int l, int step, int M, Plan& pl) {
  using VT = typename VecOf<WT>::type;
  const int D = a.dim;
  const int r0 = pl.r0, r1 = pl.r1;
  const int nr = r1 - r0;
  const LayerPtr& L = a.L[l];
  const float scv = row_scale_issue(L.s_w1, L.s_w3, r0, nr, 2 * nr);
  u32x4 slot[RING];
  const auto pro = [&]() __attribute__((always_inline)) { gemv_prologue(pl, slot); };
  stage_layer_input<WT, true>(a, s, l, step, M, reinterpret_cast<const VT*>(L.ffn_norm), pro);
  row_scale_store(s.rsc, scv, L.s_w1, L.s_w3, r0, nr, 2 * nr);
  zero_lds(s.red, 2 * nr * NWAVE * MMAX);
  __syncthreads();
  mark(a, s.flag[1], 2);
  gemv_body<WT>(pl, slot, s.act, a.kmax, M, s.red);   // rows [0, nr): w1, [nr, 2nr): w3
  __syncthreads();
  mark(a, s.flag[1], 3);
  for (int i = tidx(); i < nr * M; i += NTHREADS) {
    const int r = i / M, m = i % M;
    const float den = norm_den(s.small, m, D, a.eps);
    st_tagged(gb(a, step, l) + (size_t)m * a.ffn + r0 + r,
              silu(s.rsc[r] * red_sum(s.red, r, m) / den) * (s.rsc[nr + r] * red_sum(s.red, nr + r, m) / den),
              out_tag(a));
  }
}

template <typename WT>
__device__ __forceinline__ void phase_ffn_down(const FrameArgs& a, const Lds& s, int l, int step, int M, Plan& pl) {
  const int r0 = pl.r0, r1 = pl.r1;
  const float* s2 = a.L[l].s_w2;
  const float scv = row_scale_issue(s2, nullptr, r0, r1 - r0, r1 - r0);
  u32x4 slot[RING];
  const auto pro = [&]() __attribute__((always_inline)) { gemv_prologue(pl, slot); };
  stage_tagged<WT, 5>(frame_tw(a, s), s.act, gb(a, step, l), a.ffn, pro);
  for (int m = 1; m < M; ++m)
    stage_tagged<WT, 5>(frame_tw(a, s), s.act + (size_t)m * a.kmax, gb(a, step, l) + (size_t)m * a.ffn, a.ffn, NoHook{});
  row_scale_store(s.rsc, scv, s2, nullptr, r0, r1 - r0, r1 - r0);
  zero_lds(s.red, (r1 - r0) * NWAVE * MMAX);
  __syncthreads();
  mark(a, s.flag[1], 2);
  gemv_body<WT>(pl, slot, s.act, a.kmax, M, s.red);
  __syncthreads();
  mark(a, s.flag[1], 3);
  for (int i = tidx(); i < (r1 - r0) * M; i += NTHREADS) {
    const int r = i / M, m = i % M;
    const int k = r0 + r;
    const float xm = x_mid_of<WT>(a, s, l, step, m, k);
    st_tagged(xb(a, step, l) + (size_t)m * a.dim + k, xm + s.rsc[r] * red_sum(s.red, r, m), out_tag(a));
    st_coh(accb(a, step, l) + (size_t)m * a.dim + k, 0ll);   // ready for the next frame
  }
}

template <typename WT>
__device__ __forceinline__ void phase_head(const FrameArgs& a, const Lds& s, int step, int M, Plan& pl) {
  const int D = a.dim;
  const int r0 = pl.r0, r1 = pl.r1;
  const float scv = row_scale_issue(a.out_scale, nullptr, r0, r1 - r0, r1 - r0);
  u32x4 slot[RING];
  const auto pro = [&]() __attribute__((always_inline)) { gemv_prologue(pl, slot); };
  {
    // last row of the final layer, times fast_norm (in LDS); the RMS divides the logits
    constexpr int NS = 2;
    const u64* src = xb(a, step, a.n_layer - 1) + (size_t)(M - 1) * D;
    const int nq = D >> 2;
    float ss = 0.0f;
    auto batch = [&](int base, const auto& after) __attribute__((always_inline)) {
      u64 t[4 * NS];
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        const u64* p = src + 4 * quad_of(base, j, nq);
        ld_tagged2(p, t[4 * j], t[4 * j + 1]);
        ld_tagged2(p + 2, t[4 * j + 2], t[4 * j + 3]);
      }
      after();
      tag_wait(frame_tw(a, s), t, [&](int i) __attribute__((always_inline)) {
        return src + 4 * quad_of(base, i >> 2, nq) + (i & 3);
      });
      const int nj = steps_opaque(nq, base);
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        if (j >= nj) break;
        const int q = base + j * NTHREADS + tidx();
        if (q < nq) {
          v4f o;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float v = tag_val(t[4 * j + e]);
            ss = fmaf(v, v, ss);
            o[e] = v * s.fnw[4 * q + e];
          }
          *reinterpret_cast<v4f*>(s.act + phys<WT>(4 * q, D)) = o;
        }
      }
    };
    batch(0, pro);
    for (int base = NTHREADS * NS; base < nq; base += NTHREADS * NS) batch(base, NoHook{});
    store_ss(s.small, 1, ss, 0.0f);
  }
  row_scale_store(s.rsc, scv, a.out_scale, nullptr, r0, r1 - r0, r1 - r0);
  zero_lds(s.red, (r1 - r0) * NWAVE * MMAX);
  __syncthreads();
  mark(a, s.flag[1], 2);
  gemv_body<WT>(pl, slot, s.act, a.kmax, 1, s.red);
  __syncthreads();
  mark(a, s.flag[1], 3);
  const float hden = norm_den(s.small, 0, D, a.eps);
  for (int r = tidx(); r < r1 - r0; r += NTHREADS) {
    const float v = s.rsc[r] * red_sum(s.red, r, 0) / hden;
    st_tagged(logitsb(a, step) + r0 + r, v, out_tag(a));
    if (a.logits_out && step >= a.lo_first) a.logits_out[(size_t)(step - a.lo_first) * a.V + r0 + r] = v;
  }
}

template <typename WT>
__device__ __forceinline__ void phase_project_in(const FrameArgs& a, const Lds& s, Plan& pl) {
  const int r0 = pl.r0, r1 = pl.r1;
  const float scv = row_scale_issue(a.proj_scale, nullptr, r0, r1 - r0, r1 - r0);
  u32x4 slot[RING];
  gemv_prologue(pl, slot);
  for (int k = tidx(); k < a.in_dim; k += NTHREADS) s.act[phys<WT>(k, a.in_dim)] = a.hidden[k];
  row_scale_store(s.rsc, scv, a.proj_scale, nullptr, r0, r1 - r0, r1 - r0);
  zero_lds(s.red, (r1 - r0) * NWAVE * MMAX);
  __syncthreads();
  mark(a, s.flag[1], 2);
  gemv_body<WT>(pl, slot, s.act, a.kmax, 1, s.red);
  __syncthreads();
  mark(a, s.flag[1], 3);
  for (int r = tidx(); r < r1 - r0; r += NTHREADS) st_coh(a.xin0 + r0 + r, s.rsc[r] * red_sum(s.red, r, 0));
}

template <typename WT>
__global__ void __launch_bounds__(NTHREADS) frame_kernel(FrameArgs a) {
  extern __shared__ float lds_base[];
  const Lds s = carve(lds_base, a);
  // drop any L2/L1 line a previous frame left for the arena's addresses
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  u32 epoch = a.epoch0;
  const int V = a.V;
  if (tidx() == 0) {
    s.flag[4] = 0;
    const int c0 = a.forced ? a.forced[0] : a.sem_code[0];
    s.codes[0] = min(max(c0, 0), V - 1);     // clamp both ways (main loop, section 5.2)
    if (a.forced)
      for (int j = 1; j < a.nsteps; ++j) s.codes[j] = min(max(a.forced[j], 0), V - 1);
  }
  // per-frame constants into LDS: q/k norm weights of every layer, RoPE table
  using VT = typename VecOf<WT>::type;
  if (a.has_qkn) {
    for (int i = tidx(); i < a.n_layer * 2 * a.hd; i += NTHREADS) {
      const int l = i / (2 * a.hd), r = i - l * 2 * a.hd;
      const VT* w = reinterpret_cast<const VT*>(r < a.hd ? a.L[l].q_norm : a.L[l].k_norm);
      s.qkn[i] = WTraits<VT>::one(w, r < a.hd ? r : r - a.hd);
    }
  }
  for (int i = tidx(); i < a.ctx_len * a.hd; i += NTHREADS) s.rope[i] = a.rope[i];
  for (int i = tidx(); i < a.dim; i += NTHREADS) s.fnw[i] = WTraits<VT>::one(reinterpret_cast<const VT*>(a.fnorm), i);
  __syncthreads();
  const int nph = phase_count(a);
  // A phase's plan (row range and chunk split) is plain integers and is
  // computed before the barrier that precedes the phase; its loads are
  // issued only inside the phase.
  PhaseId id = first_phase(a);
  Plan pl = plan_for<WT>(a, id);
  bool ok = true;
  for (int ph = 0; ph < nph; ++ph) {
    const int step = id.step, l = id.layer;
    const int M = (step == 1) ? 2 : 1;
    if (a.tlog && tidx() == 0) s.flag[1] = ph;
    mark(a, ph, 5);
    switch (id.kind) {
      case PH_PROJ: phase_project_in<WT>(a, s, pl); break;
      case PH_QKV: phase_qkv<WT>(a, s, l, step, M, pl); break;
      case PH_WO: phase_attn_wo<WT>(a, s, l, step, M, pl); break;
      case PH_FFN_UP: phase_ffn_up<WT>(a, s, l, step, M, pl); break;
      case PH_FFN_DOWN: phase_ffn_down<WT>(a, s, l, step, M, pl); break;
      default: phase_head<WT>(a, s, step, M, pl); break;
    }
    const PhaseId done = id;
    id = next_phase(a, id);
    pl = plan_for<WT>(a, id);   // past the last phase: a plan that is never used
    mark(a, ph, 0);
    if (done.kind == PH_WO || done.kind == PH_PROJ) {
      // the attention accumulators (device atomics), this step's keys and
      // values and fast_project_in's output are read after a grid sync
      if (!grid_sync<FrameArgs, false>(a, epoch, s.flag)) { ok = false; break; }
    } else {
      // the next phase's loads wait on this phase's tagged outputs: the
      // block only finishes its own use of LDS (the epilogue still reads
      // red and small)
      __syncthreads();
    }
    if (s.flag[4]) { ok = false; break; }
    mark(a, ph, 1);
    if (done.kind == PH_HEAD && !a.forced) {
      const SampScratch sc{s.cval, s.cidx, reinterpret_cast<int*>(s.mark)};
      const int code = sample_from(TaggedLogits{frame_tw(a, s), logitsb(a, step)}, V, a.temp[0], a.top_p[0], a.top_k[0],
                                   a.uniforms[step - 1], sc);
      if (tidx() == 0) s.codes[step] = min(max(code, 0), V - 1);
      __syncthreads();
      if (s.flag[4]) { ok = false; break; }
    }
  }
  if (ok && blockIdx.x == 0 && a.codes_out && tidx() < a.ncb) a.codes_out[tidx()] = s.codes[tidx()];
  // a barrier or tag wait gave up: the frame failed.  The attention accumulators
  // are cleared (the next frame adds into them) and the request's codebooks
  // 1.. are 0, the main loop's convention for a failed fast_decode
  // ("Fast-AR codebook decoding ...", section 5.2).
  launch_exit(a, s.flag, [&]() __attribute__((always_inline)) {
    zero_words64(a.acc, (size_t)(a.ncb - 1) * a.n_layer * a.acc_slot);
    if (a.codes_out && tidx() < a.ncb) st_coh(a.codes_out + tidx(), tidx() == 0 ? s.codes[0] : 0);
  });
}

__global__ void __launch_bounds__(NTHREADS) sample_kernel(int V, const float* logits, const float* temp,
                                                          const float* top_p, const int* top_k, const float* u,
                                                          int* codes) {
  __shared__ float cval[TOPK_MAX];
  __shared__ int cidx[TOPK_MAX];
  __shared__ int red[2 * NWAVE * SAMP_TAU];
  const int b = blockIdx.x;
  const SampScratch sc{cval, cidx, red};
  const int c = sample_request(logits + (size_t)b * V, V, temp[b], top_p[b], top_k[b], u[b], sc);
  if (tidx() == 0) codes[b] = c;
}

// ------------------------------------------------------ test kernels
// The GEMV of the frame kernel on its own: y = W x, with the phase options
// the frame kernel uses (RMSNorm fused into staging and the RMS dividing the
// outputs; w1 / w3 rows run as one GEMV with the SwiGLU epilogue).  Rows of
// W split over the blocks as in a phase; the plan, the weight ring, the
// activation layout and the wave reduction are the frame kernel's own.
struct GemvTestArgs {
  int N, K, M, kmax, rmax;
  const void* W;
  const void* W3;        // second matrix of a SwiGLU pair, or nullptr
  const float* sc;       // row scales of int8 W and W3, or nullptr
  const float* sc3;
  const void* normw;     // RMSNorm weight [K], or nullptr
  float eps;
  const float* x;        // [M][K]
  float* y;              // [M][N]
};

template <typename WT>
__global__ void __launch_bounds__(NTHREADS) gemv_test_kernel(GemvTestArgs a) {
  extern __shared__ float lds_base[];
  float* act = lds_base;                                             // [MMAX][kmax]
  float* red = act + (((size_t)MMAX * a.kmax + 3) & ~(size_t)3);    // [rmax][MMAX][NWAVE]
  float* small = red + (size_t)a.rmax * NWAVE * MMAX;                // [64]
  float* rsc = small + 64;                                            // [rmax]
  using VT = typename VecOf<WT>::type;
  int r0, r1;
  split_rows(a.N, blockIdx.x, gridDim.x, r0, r1);
  const int nr = r1 - r0;
  const WT* W3 = reinterpret_cast<const WT*>(a.W3);
  const int nrows = W3 ? 2 * nr : nr;
  const float scv = row_scale_issue(a.sc, a.sc3, r0, nr, nrows);
  Plan pl = make_plan<WT>(reinterpret_cast<const WT*>(a.W), W3, a.K, 0, a.K, r0, nr, nrows);
  u32x4 slot[RING];
  gemv_prologue(pl, slot);
  float ss0 = 0.0f, ss1 = 0.0f;
  const int nq = a.K >> 2;
  for (int i = tidx(); i < a.M * nq; i += NTHREADS) {
    const int m = i / nq, c = i - m * nq;
    const float4 v = *reinterpret_cast<const float4*>(a.x + (size_t)m * a.K + 4 * c);
    float e[4] = {v.x, v.y, v.z, v.w};
    float t = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      t = fmaf(e[j], e[j], t);
      if (a.normw) e[j] *= WTraits<VT>::one(reinterpret_cast<const VT*>(a.normw), 4 * c + j);
    }
    if (m == 0) ss0 += t; else ss1 += t;
    *reinterpret_cast<float4*>(act + (size_t)m * a.kmax + phys<WT>(4 * c, a.K)) = make_float4(e[0], e[1], e[2], e[3]);
  }
  store_ss(small, a.M, ss0, ss1);
  row_scale_store(rsc, scv, a.sc, a.sc3, r0, nr, nrows);
  zero_lds(red, nrows * NWAVE * MMAX);
  __syncthreads();
  gemv_body<WT>(pl, slot, act, a.kmax, a.M, red);
  __syncthreads();
  for (int i = tidx(); i < nr * a.M; i += NTHREADS) {
    const int r = i / a.M, m = i % a.M;
    const float den = a.normw ? norm_den(small, m, a.K, a.eps) : 1.0f;
    const float d = rsc[r] * red_sum(red, r, m) / den;
    a.y[(size_t)m * a.N + r0 + r] = W3 ? silu(d) * (rsc[nr + r] * red_sum(red, nr + r, m) / den) : d;
  }
}

// q/k RMSNorm + pair RoPE + causal attention of one KV group for the row at
// window position t (block (g, t)) over the raw wqkv outputs of positions
// 0..t, with the frame kernel's device functions (head_norm_rope,
// attend_rows).  out[t][g * gw ..] receives the group's heads.
struct AttnTestArgs {
  int H, G, hd, T, ctx, has_qkn;
  float eps;
  const float* qkv;      // [T][(H + 2G) hd]
  const float* qn;       // [hd] (or any valid pointer without q/k norm)
  const float* kn;
  const float* rope;     // [2][ctx][hd/2]
  float* out;            // [T][H hd]
};

__global__ void __launch_bounds__(NTHREADS) attn_test_kernel(AttnTestArgs a) {
  extern __shared__ float lds_base[];
  const int g = blockIdx.x, t = blockIdx.y;
  const int hd = a.hd, gh = a.H / a.G, gw = gh * hd, qkv_dim = (a.H + 2 * a.G) * hd;
  float* q = lds_base;                        // [gh][hd]
  float* kc = q + (size_t)gh * hd;            // [ctx][hd]
  float* vc = kc + (size_t)a.ctx * hd;        // [ctx][hd]
  float* rope = vc + (size_t)a.ctx * hd;      // [2][ctx][hd/2]
  float* o = rope + (size_t)a.ctx * hd;       // [gw]
  for (int i = tidx(); i < a.ctx * hd; i += NTHREADS) rope[i] = a.rope[i];
  for (int i = tidx(); i < gh * hd; i += NTHREADS) q[i] = a.qkv[(size_t)t * qkv_dim + (size_t)g * gh * hd + i];
  for (int i = tidx(); i < (t + 1) * hd; i += NTHREADS) {
    const int p = i / hd, d = i - p * hd;
    kc[i] = a.qkv[(size_t)p * qkv_dim + (size_t)(a.H + g) * hd + d];
    vc[i] = a.qkv[(size_t)p * qkv_dim + (size_t)(a.H + a.G + g) * hd + d];
  }
  __syncthreads();
  const int wave = tidx() >> 6;
  for (int v = wave; v < gh + t + 1; v += NWAVE) {
    if (v < gh) head_norm_rope(q + (size_t)v * hd, hd, a.qn, a.has_qkn, a.eps, rope, a.ctx, t);
    else head_norm_rope(kc + (size_t)(v - gh) * hd, hd, a.kn, a.has_qkn, a.eps, rope, a.ctx, v - gh);
  }
  __syncthreads();
  attend_rows<float>(q, kc, vc, 1, t, gh, hd, o, 0, gw);
  __syncthreads();
  for (int i = tidx(); i < gw; i += NTHREADS) a.out[(size_t)t * a.H * hd + (size_t)g * gw + i] = o[i];
}

// ------------------------------------------------------ qkv0 table build
// Run once when a context is created.  den[c] = sqrt(mean_k e_c[k]^2 + eps)
// of every embedding row (the layer-0 attention_norm RMS, "Model loading and
// GGUF", section 2.2).
template <typename VT>
__global__ void __launch_bounds__(256) qkv0_den_kernel(const VT* emb, int D, float eps, float* den) {
  __shared__ float red[4];
  const VT* e = emb + (size_t)blockIdx.x * D;
  float ss = 0.0f;
  for (int k = threadIdx.x; k < D; k += 256) {
    const float v = WTraits<VT>::one(e, k);
    ss = fmaf(v, v, ss);
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  if (threadIdx.x == 0) den[blockIdx.x] = sqrtf(((red[0] + red[1]) + (red[2] + red[3])) / (float)D + eps);
}

// out[c][r] = (sum_k W[r][k] * (g[k] * e_c[k])) / den[c]: the layer-0 wqkv
// output of embedding row c, a float32 GEMM in 64 x 64 tiles (16 outputs a
// thread).  An int8 W carries row scales: out = scale[r] * sum / den.
template <typename WT>
__global__ void __launch_bounds__(256) qkv0_gemm_kernel(const WT* W, const float* wscale,
                                                        const typename VecOf<WT>::type* emb,
                                                        const typename VecOf<WT>::type* g, const float* den,
                                                        int V, int R, int D, float* out) {
  using VT = typename VecOf<WT>::type;
  constexpr int TK = 32;
  __shared__ float Es[TK][65];   // [k][c]: g * e
  __shared__ float Ws[TK][65];   // [k][r]
  const int c0 = blockIdx.y * 64, r0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
  for (int k0 = 0; k0 < D; k0 += TK) {
    for (int i = threadIdx.x; i < 64 * TK; i += 256) {
      const int row = i / TK, k = i % TK, kk = k0 + k;
      const int c = c0 + row, r = r0 + row;
      Es[k][row] = (c < V && kk < D) ? WTraits<VT>::one(g, kk) * WTraits<VT>::one(emb + (size_t)c * D, kk) : 0.0f;
      Ws[k][row] = (r < R && kk < D) ? WTraits<WT>::one(W + (size_t)r * D, kk) : 0.0f;
    }
    __syncthreads();
    for (int k = 0; k < TK; ++k) {
      float ev[4], wv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ev[i] = Es[k][ty * 4 + i];
        wv[i] = Ws[k][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(wv[j], ev[i], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = c0 + ty * 4 + i;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = r0 + tx * 4 + j;
      if (c < V && r < R) out[(size_t)c * R + r] = (wscale ? wscale[r] * acc[i][j] : acc[i][j]) / den[c];
    }
  }
}

// ------------------------------------------------- streaming-read probe
// The achievable HBM read rate, measured with the frame kernel's load form:
// workgroup b reads bytes [b n / G, (b + 1) n / G) of src with 16-byte
// non-temporal loads, U in flight a thread, and folds every 32-bit word
// into an XOR; sink[0] receives the XOR of the whole buffer (one atomic a
// workgroup), so a test can check that every byte was read.
template <int U>
__global__ void __launch_bounds__(NTHREADS) stream_read_kernel(const u32x4* src, size_t n16, u32* sink) {
  const size_t G = gridDim.x;
  const size_t s0 = n16 * blockIdx.x / G, s1 = n16 * (blockIdx.x + 1) / G;
  u32 acc = 0u;
  size_t i = s0 + threadIdx.x;
  for (; i + (size_t)(U - 1) * NTHREADS < s1; i += (size_t)U * NTHREADS) {
    u32x4 v[U];
#pragma unroll
    for (int j = 0; j < U; ++j) v[j] = __builtin_nontemporal_load(src + i + (size_t)j * NTHREADS);
#pragma unroll
    for (int j = 0; j < U; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  for (; i < s1; i += NTHREADS) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  __shared__ u32 part[NWAVE];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc ^= (u32)__shfl_xor((int)acc, o);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    u32 t = 0u;
    for (int w = 0; w < NWAVE; ++w) t ^= part[w];
    atomicXor(sink, t);
  }
}

// ------------------------------------------------- static frame scratch
// Scratch of s2fast_decode_frame_static, for callers that cannot allocate:
// the batch-1 frame arena and barrier flags of one launch, in one array per
// GPU that lives until the process ends.  Host code reaches it only through
// the device address hipGetSymbolAddress returns (StaticScratch::ptr).
constexpr size_t STATIC_SCRATCH_BYTES = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[STATIC_SCRATCH_BYTES];

__global__ void __launch_bounds__(256) fill_zero_kernel(u32* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0u;
}

#include "batched.h"
#include "slow_step.h"
#include "prefill.h"

#ifndef KS_DOWN
#define KS_DOWN 4
#endif
static_assert(KS_DOWN >= 1 && KS_DOWN <= 4, "the finalising workgroup adds at most four K slices");

}  // namespace

// =================================================================== host

struct s2fast_ctx {
  s2fast_config cfg;
  s2fast_weights w;
  s2fast_q8_scales q8 = {};   // row scales of an int8 model (copied at creation)
  int device = 0;
  int ncu = 0;
  size_t lds_bytes = 0;
  int kmax = 0, rmax = 0;
  long long x_slot = 0, qkv_slot = 0, acc_slot = 0, g_slot = 0, logits_slot = 0, kv_pos = 0;
  float* rope = nullptr;
  float* qkv0 = nullptr;   // [V][qkv_dim] layer-0 q/k/v of every embedding row
  float* xin0 = nullptr;
  u64* x = nullptr;        // tagged outputs (x, qkv, g, logits): cleared at creation and when the
  u64* qkv = nullptr;      // epoch counter wraps, so no stale tag can match a later launch's
  long long* acc = nullptr;
  u64* g = nullptr;
  float* kv = nullptr;
  u64* logits = nullptr;
  u32* flags = nullptr;
  u32* err = nullptr;
  u32* tlog = nullptr;     // allocated on first s2fast_test_timeline call
  bool tlog_on = false;
  u32 give_up = 0;         // test hook (s2fast_test_watchdog)
  u32 epoch = 0;
  // batched decoding (batch >= 2): requests per launch (0: every request is
  // decoded by its own launch) and the batched arena
  int bq = 0;
  size_t b_lds = 0;
  long long bx_slot = 0, bqkv_slot = 0, batt_slot = 0, bg_slot = 0, blogits_slot = 0;
  float* b_xin0 = nullptr;
  float* b_x = nullptr;
  float* b_xmid = nullptr;
  float* b_qkv = nullptr;
  float* b_att = nullptr;
  float* b_g = nullptr;
  float* b_logits = nullptr;
  float* b_kv = nullptr;
  int* b_codes = nullptr;
  char* b_pk = nullptr;                          // packed weight streams of the batched GEMMs
  float* b_kpart[6] = {};                        // K-split partial sums [slot][ks][kslot]
  long long b_kslot[6] = {};
  float* b_kss[6] = {};                          // slice sums of squares (wqkv) [slot][ks][MP_MAX]
  int* b_kcnt[6] = {};                           // and their per-row-group counts [slot][P]
  int b_ks[6] = {1, 1, 1, 1, 1, 1};              // K split of each batched GEMM kind
  long long b_pk_off[2 + 4 * S2FAST_MAX_LAYERS] = {};
};

namespace {

bool is_gfx950(int dev) {
  hipDeviceProp_t p;
  if (hipGetDeviceProperties(&p, dev) != hipSuccess) return false;
  return std::strncmp(p.gcnArchName, "gfx950", 6) == 0;
}

// The batch-1 frame kernel instantiated for a weight type.
const void* frame_fn(int dtype) {
  if (dtype == S2FAST_BF16) return reinterpret_cast<const void*>(&frame_kernel<uint16_t>);
  if (dtype == S2FAST_Q8) return reinterpret_cast<const void*>(&frame_kernel<q8_t>);
  return reinterpret_cast<const void*>(&frame_kernel<float>);
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

// grid syncs of one launch of `nsteps` decode steps: one per phase (the
// frame kernel's phase_count), less the head's when the prefix is
// teacher-forced
// Grid syncs of a batch-1 launch: after fast_project_in and after every
// layer's attention + wo phase; the other phases hand over tagged values.
int syncs_for(const s2fast_config& c, int nsteps) {
  return (c.has_project_in ? 1 : 0) + nsteps * c.n_layer;
}

void free_ctx(s2fast_ctx* c) {
  if (!c) return;
  void* ptrs[] = {c->rope, c->qkv0, c->xin0, c->x, c->qkv, c->acc, c->g, c->kv, c->logits, c->flags, c->err, c->tlog,
                  c->b_xin0, c->b_x, c->b_xmid, c->b_qkv, c->b_att, c->b_g, c->b_logits, c->b_kv, c->b_codes,
                  c->b_pk, c->b_kpart[BK_WO], c->b_kcnt[BK_WO], c->b_kpart[BK_DOWN], c->b_kcnt[BK_DOWN],
                  c->b_kpart[BK_QKV], c->b_kcnt[BK_QKV], c->b_kss[BK_QKV],
                  c->b_kpart[BK_HEAD], c->b_kcnt[BK_HEAD], c->b_kss[BK_HEAD]};
  for (void* p : ptrs)
    if (p) (void)hipFree(p);
  delete c;
}

template <typename T>
hipError_t dalloc(T** p, size_t n) {
  return hipMalloc(reinterpret_cast<void**>(p), n * sizeof(T) > 0 ? n * sizeof(T) : 16);
}

// One packed weight stream (b_pack_kernel) per job, all in one allocation;
// off[idx] is job idx's byte offset in it.  The streams are cut for grids of
// ncu workgroups.
struct PackJob { int idx; const void* wa; const void* wb; int R, K, S; };

int pack_jobs(int dtype, int ncu, const PackJob* jobs, int nj, char** out, long long* off) {
  const int ksz = dtype == S2FAST_BF16 ? 32 : 16;
  long long total = 0;
  for (int j = 0; j < nj; ++j) {
    off[jobs[j].idx] = total;
    const long long rows = (long long)jobs[j].R * (jobs[j].wb ? 2 : 1) * jobs[j].S;
    total += rows * ((jobs[j].K / jobs[j].S + ksz - 1) / ksz) * 64;
    total = (total + 255) / 256 * 256;
  }
  if (dalloc(out, (size_t)total) != hipSuccess) return S2FAST_ERR_NOMEM;
  for (int j = 0; j < nj; ++j) {
    char* dst = *out + off[jobs[j].idx];
    if (dtype == S2FAST_BF16)
      hipLaunchKernelGGL(b_pack_kernel<uint16_t>, dim3(ncu), dim3(256), 0, 0,
                         static_cast<const uint16_t*>(jobs[j].wa), static_cast<const uint16_t*>(jobs[j].wb),
                         jobs[j].R, jobs[j].K, jobs[j].S, dst);
    else
      hipLaunchKernelGGL(b_pack_kernel<float>, dim3(ncu), dim3(256), 0, 0, static_cast<const float*>(jobs[j].wa),
                         static_cast<const float*>(jobs[j].wb), jobs[j].R, jobs[j].K, jobs[j].S, dst);
  }
  return (hipGetLastError() == hipSuccess && hipDeviceSynchronize() == hipSuccess) ? S2FAST_OK : S2FAST_ERR_HIP;
}

// The batched GEMMs' packed weight streams, one per GEMM and layer, from the
// weights the context was created with.
int pack_batched(s2fast_ctx* c) {
  const s2fast_config& k = c->cfg;
  const int qkv_dim = (k.n_head + 2 * k.n_head_kv) * k.head_dim, attn_dim = k.n_head * k.head_dim;
  PackJob jobs[2 + 4 * S2FAST_MAX_LAYERS];
  int nj = 0;
  if (k.has_project_in) jobs[nj++] = {0, c->w.project_in, nullptr, k.dim, k.in_dim, 1};
  jobs[nj++] = {1, c->w.output, nullptr, k.codebook_size, k.dim, c->b_ks[BK_HEAD]};
  for (int l = 0; l < k.n_layer; ++l) {
    const s2fast_layer_weights& L = c->w.layers[l];
    jobs[nj++] = {2 + 4 * l + 0, L.wqkv, nullptr, qkv_dim, k.dim, c->b_ks[BK_QKV]};
    jobs[nj++] = {2 + 4 * l + 1, L.wo, nullptr, k.dim, attn_dim, c->b_ks[BK_WO]};
    jobs[nj++] = {2 + 4 * l + 2, L.w1, L.w3, k.ffn_dim, k.dim, 1};
    jobs[nj++] = {2 + 4 * l + 3, L.w2, nullptr, k.dim, k.ffn_dim, c->b_ks[BK_DOWN]};
  }
  return pack_jobs(k.weight_dtype, c->ncu, jobs, nj, &c->b_pk, c->b_pk_off);
}

// The qkv0 table from the weights the context was created with (they stay
// unchanged for its life).
int build_qkv0(s2fast_ctx* c) {
  const s2fast_config& k = c->cfg;
  const int R = (k.n_head + 2 * k.n_head_kv) * k.head_dim, V = k.codebook_size, D = k.dim;
  float* den = nullptr;
  if (dalloc(&c->qkv0, (size_t)V * R) != hipSuccess || dalloc(&den, (size_t)V) != hipSuccess) {
    if (den) (void)hipFree(den);
    return S2FAST_ERR_NOMEM;
  }
  const dim3 grid((R + 63) / 64, (V + 63) / 64);
  if (k.weight_dtype != S2FAST_F32) {   // bf16 vectors (bf16 and int8 models)
    const uint16_t* e = static_cast<const uint16_t*>(c->w.embeddings);
    const uint16_t* g = static_cast<const uint16_t*>(c->w.layers[0].attention_norm);
    hipLaunchKernelGGL(qkv0_den_kernel<uint16_t>, dim3(V), dim3(256), 0, 0, e, D, k.norm_eps, den);
    if (k.weight_dtype == S2FAST_Q8)
      hipLaunchKernelGGL(qkv0_gemm_kernel<q8_t>, grid, dim3(256), 0, 0,
                         static_cast<const q8_t*>(c->w.layers[0].wqkv), c->q8.layers[0].wqkv, e, g, den, V, R, D,
                         c->qkv0);
    else
      hipLaunchKernelGGL(qkv0_gemm_kernel<uint16_t>, grid, dim3(256), 0, 0,
                         static_cast<const uint16_t*>(c->w.layers[0].wqkv), (const float*)nullptr, e, g, den, V, R,
                         D, c->qkv0);
  } else {
    const float* e = static_cast<const float*>(c->w.embeddings);
    hipLaunchKernelGGL(qkv0_den_kernel<float>, dim3(V), dim3(256), 0, 0, e, D, k.norm_eps, den);
    hipLaunchKernelGGL(qkv0_gemm_kernel<float>, grid, dim3(256), 0, 0,
                       static_cast<const float*>(c->w.layers[0].wqkv), (const float*)nullptr, e,
                       static_cast<const float*>(c->w.layers[0].attention_norm), den, V, R, D, c->qkv0);
  }
  const bool ok = hipGetLastError() == hipSuccess && hipDeviceSynchronize() == hipSuccess;
  (void)hipFree(den);
  return ok ? S2FAST_OK : S2FAST_ERR_HIP;
}

int zero_device(void* p, size_t bytes, hipStream_t st);

// Before the epoch counter wraps: the barrier flags and the tagged outputs
// go back to their cleared state (tag 0, below every launch's tag) and the
// counter restarts.
int restart_epochs(s2fast_ctx* c, hipStream_t stream) {
  const size_t slots = (size_t)(c->cfg.num_codebooks - 1) * c->cfg.n_layer;
  if (zero_device(c->flags, (size_t)c->ncu * 64 * sizeof(u32), stream) != S2FAST_OK ||
      zero_device(c->x, slots * c->x_slot * sizeof(u64), stream) != S2FAST_OK ||
      zero_device(c->qkv, slots * c->qkv_slot * sizeof(u64), stream) != S2FAST_OK ||
      zero_device(c->g, slots * c->g_slot * sizeof(u64), stream) != S2FAST_OK ||
      zero_device(c->logits, (size_t)(c->cfg.num_codebooks - 1) * c->logits_slot * sizeof(u64), stream) != S2FAST_OK)
    return S2FAST_ERR_HIP;
  c->epoch = 0;
  return S2FAST_OK;
}

int launch_frame(s2fast_ctx* c, const FrameArgs& fa_in, hipStream_t stream) {
  FrameArgs fa = fa_in;
  const u32 n = (u32)syncs_for(c->cfg, fa.nsteps);
  if (c->epoch > 0xF0000000u && restart_epochs(c, stream) != S2FAST_OK) return S2FAST_ERR_HIP;
  fa.epoch0 = c->epoch;
  void* args[] = {&fa};
  hipError_t e = hipLaunchCooperativeKernel(frame_fn(c->cfg.weight_dtype), dim3(c->ncu), dim3(NTHREADS), args,
                                            c->lds_bytes, stream);
  if (e != hipSuccess) return S2FAST_ERR_HIP;
  c->epoch += n;
  return S2FAST_OK;
}

int launch_batched(s2fast_ctx* c, const BatchArgs& ba_in, hipStream_t stream) {
  BatchArgs ba = ba_in;
  const u32 n = (u32)b_syncs(c->cfg.has_project_in, ba.nsteps, c->cfg.n_layer, ba.forced != nullptr,
                            c->b_ks[BK_HEAD] > 1 && ba.logits_out != nullptr,
                            b_merged_draw(ba.Bq, c->cfg.n_head_kv, c->ncu));
  if (c->epoch > 0xF0000000u && restart_epochs(c, stream) != S2FAST_OK) return S2FAST_ERR_HIP;
  ba.epoch0 = c->epoch;
  void* args[] = {&ba};
  const void* fn = c->cfg.weight_dtype == S2FAST_BF16 ? reinterpret_cast<const void*>(&frame_kernel_b<uint16_t>)
                                                       : reinterpret_cast<const void*>(&frame_kernel_b<float>);
  hipError_t e = hipLaunchCooperativeKernel(fn, dim3(c->ncu), dim3(NTHREADS), args, c->b_lds, stream);
  if (e != hipSuccess) return S2FAST_ERR_HIP;
  c->epoch += n;
  return S2FAST_OK;
}

void fill_batch_shape(const s2fast_ctx* c, BatchArgs& ba) {
  const s2fast_config& k = c->cfg;
  std::memset(&ba, 0, sizeof(ba));
  ba.in_dim = k.in_dim; ba.dim = k.dim; ba.n_layer = k.n_layer; ba.n_head = k.n_head; ba.n_kv = k.n_head_kv;
  ba.hd = k.head_dim; ba.ffn = k.ffn_dim; ba.V = k.codebook_size; ba.ncb = k.num_codebooks; ba.ctx_len = k.context;
  ba.eps = k.norm_eps; ba.has_proj = k.has_project_in; ba.has_qkn = k.has_qk_norm; ba.lds_layers = k.n_layer;
  ba.nsteps = k.num_codebooks - 1; ba.forced_ld = k.num_codebooks; ba.lo_first = 1; ba.lo_rows = k.num_codebooks - 1;
  ba.qkv_dim = (k.n_head + 2 * k.n_head_kv) * k.head_dim;
  ba.attn_dim = k.n_head * k.head_dim;
  ba.gheads = k.n_head / k.n_head_kv;
  ba.gw = ba.gheads * k.head_dim;
  ba.proj = c->w.project_in; ba.emb = c->w.embeddings; ba.fnorm = c->w.norm; ba.outw = c->w.output;
  for (int l = 0; l < k.n_layer; ++l) {
    const s2fast_layer_weights& L = c->w.layers[l];
    ba.L[l] = LayerPtr{L.attention_norm, L.wqkv, L.q_norm, L.k_norm, L.wo, L.ffn_norm, L.w1, L.w3, L.w2};
  }
  ba.rope = c->rope;
  ba.qkv0 = c->qkv0;
  for (int i = 0; i < 2 + 4 * S2FAST_MAX_LAYERS; ++i) ba.pk[i] = c->b_pk + c->b_pk_off[i];
  for (int kd = 0; kd < 6; ++kd) {
    ba.ks[kd] = c->b_ks[kd]; ba.kpart[kd] = c->b_kpart[kd]; ba.kslot[kd] = c->b_kslot[kd];
    ba.kcnt[kd] = c->b_kcnt[kd]; ba.kss[kd] = c->b_kss[kd];
  }
  ba.xin0 = c->b_xin0; ba.x = c->b_x; ba.xmid = c->b_xmid; ba.qkv = c->b_qkv; ba.att = c->b_att; ba.g = c->b_g;
  ba.logits = c->b_logits; ba.kv = c->b_kv; ba.codes = c->b_codes;
  ba.x_slot = c->bx_slot; ba.qkv_slot = c->bqkv_slot; ba.att_slot = c->batt_slot; ba.g_slot = c->bg_slot;
  ba.logits_slot = c->blogits_slot;
  ba.flags = c->flags; ba.err = c->err;
  ba.watch.give_up = c->give_up;
  ba.tlog = c->tlog_on ? c->tlog : nullptr;
}

// Can this shape run the batched kernel, and with how many requests per
// launch?  0 when it cannot (then every request gets its own launch).
int batched_group(const s2fast_config& k, int P) {
  const int qkv_dim = (k.n_head + 2 * k.n_head_kv) * k.head_dim;
  const int gh = k.n_head / k.n_head_kv;
  int tmax = 0;
  for (int n : {qkv_dim, k.dim, k.codebook_size}) tmax = std::max(tmax, ((n + P - 1) / P + 15) / 16);
  tmax = std::max(tmax, (2 * ((k.ffn_dim + P - 1) / P) + 15) / 16);
  if (tmax > TMAX || 2 * tmax > RED_TILES) return 0;
  if ((size_t)(2 * gh * k.head_dim + 2 * k.context * k.head_dim) * sizeof(float) > (size_t)XF_BYTES) return 0;
  return BQ_MAX;   // the attention phase loops over (request, KV group) pairs
}

// The sticky status of a context's watchdog words, read (and cleared) after
// the work enqueued on `st` has finished: S2FAST_ERR_HIP if a launch gave up
// a barrier wait since the last read.
int read_status(u32* err, hipStream_t st) {
  u32 v = 0;
  if (hipMemcpyAsync(&v, err + W_STATUS, sizeof(u32), hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return S2FAST_ERR_HIP;
  if (v == 0) return S2FAST_OK;
  if (hipMemsetAsync(err + W_STATUS, 0, sizeof(u32), st) != hipSuccess || hipStreamSynchronize(st) != hipSuccess)
    return S2FAST_ERR_HIP;
  return S2FAST_ERR_HIP;
}

void fill_shape(const s2fast_ctx* c, FrameArgs& fa) {
  const s2fast_config& k = c->cfg;
  std::memset(&fa, 0, sizeof(fa));
  fa.in_dim = k.in_dim; fa.dim = k.dim; fa.n_layer = k.n_layer; fa.n_head = k.n_head; fa.n_kv = k.n_head_kv;
  fa.hd = k.head_dim; fa.ffn = k.ffn_dim; fa.V = k.codebook_size; fa.ncb = k.num_codebooks; fa.ctx_len = k.context;
  fa.eps = k.norm_eps; fa.has_proj = k.has_project_in; fa.has_qkn = k.has_qk_norm;
  fa.nsteps = k.num_codebooks - 1; fa.forced_ld = k.num_codebooks; fa.lo_first = 1; fa.lo_rows = k.num_codebooks - 1;
  fa.qkv_dim = (k.n_head + 2 * k.n_head_kv) * k.head_dim;
  fa.attn_dim = k.n_head * k.head_dim;
  fa.gheads = k.n_head / k.n_head_kv;
  fa.gw = fa.gheads * k.head_dim;
  fa.kmax = c->kmax; fa.rmax = c->rmax;
  fa.proj = c->w.project_in; fa.emb = c->w.embeddings; fa.fnorm = c->w.norm; fa.outw = c->w.output;
  fa.proj_scale = c->q8.project_in; fa.out_scale = c->q8.output;
  for (int l = 0; l < k.n_layer; ++l) {
    const s2fast_layer_weights& L = c->w.layers[l];
    const auto& Q = c->q8.layers[l];
    fa.L[l] = LayerPtr{L.attention_norm, L.wqkv, L.q_norm, L.k_norm, L.wo, L.ffn_norm, L.w1, L.w3, L.w2,
                       Q.wqkv, Q.wo, Q.w1, Q.w3, Q.w2};
  }
  fa.rope = c->rope;
  fa.qkv0 = c->qkv0;
  fa.xin0 = c->xin0; fa.x = c->x; fa.qkv = c->qkv; fa.acc = c->acc; fa.g = c->g; fa.kv = c->kv;
  fa.kv_pos = (int)c->kv_pos;
  fa.x_slot = c->x_slot; fa.qkv_slot = c->qkv_slot; fa.acc_slot = c->acc_slot; fa.g_slot = c->g_slot;
  fa.logits_slot = c->logits_slot;
  fa.logits = c->logits; fa.flags = c->flags; fa.err = c->err;
  fa.watch.give_up = c->give_up;
  fa.tlog = c->tlog_on ? c->tlog : nullptr;
}

// Per-device state of the static scratch: its device address (from
// hipGetSymbolAddress, taken once per device with that device current), the
// barrier epoch its flags have reached, and whether it was cleared.
struct StaticScratch {
  char* ptr = nullptr;
  u32 epoch = 0;
  bool cleared = false;
  size_t layout[3] = {0, 0, 0};   // the arena layout the array was last left in (acc, flags, end)
};
constexpr int STATIC_MAX_DEVICES = 64;
StaticScratch g_static[STATIC_MAX_DEVICES];
std::mutex g_static_mu;

// Byte offsets of the batch-1 frame arena inside the static scratch (the
// layout of the context arena: one 256-byte aligned region per (step,
// layer) output, then the barrier flags); total bytes in `end`.
struct StaticLayout {
  size_t xin0, x, qkv, acc, g, kv, logits, flags, end;
};

StaticLayout static_layout(const s2fast_ctx* c) {
  const s2fast_config& k = c->cfg;
  const size_t slots = (size_t)(k.num_codebooks - 1) * k.n_layer;
  auto r = [](size_t n) { return (n + 255) / 256 * 256; };
  StaticLayout L;
  size_t o = 0;
  L.xin0 = o; o += r(((size_t)k.dim + 63) / 64 * 64 * sizeof(float));
  L.x = o; o += r(slots * c->x_slot * sizeof(u64));
  L.qkv = o; o += r(slots * c->qkv_slot * sizeof(u64));
  L.acc = o; o += r(slots * c->acc_slot * sizeof(long long));
  L.g = o; o += r(slots * c->g_slot * sizeof(u64));
  L.kv = o; o += r((size_t)k.n_layer * k.context * c->kv_pos * sizeof(float));
  L.logits = o; o += r((size_t)(k.num_codebooks - 1) * c->logits_slot * sizeof(u64));
  L.flags = o; o += r((size_t)c->ncu * 64 * sizeof(u32));
  L.end = o;
  return L;
}

int zero_device(void* p, size_t bytes, hipStream_t st) {
  hipLaunchKernelGGL(fill_zero_kernel, dim3(1024), dim3(256), 0, st, static_cast<u32*>(p), bytes / sizeof(u32));
  return hipGetLastError() == hipSuccess ? S2FAST_OK : S2FAST_ERR_HIP;
}

// Teacher-forced launches: B requests with the codes `codes` [B][ld] as
// their prefixes, `nsteps` decode steps, logits of step s >= lo_first into
// row s - lo_first of `logits` [B][lo_rows][V].  Arguments are validated.
int launch_forced(s2fast_ctx* ctx, int B, const float* hidden, const int32_t* codes, int ld, int nsteps,
                  float* logits, int lo_first, int lo_rows, hipStream_t st) {
  const s2fast_config& k = ctx->cfg;
  const size_t lo_req = (size_t)lo_rows * k.codebook_size;
  if (B >= 2 && ctx->bq > 0) {
    BatchArgs ba;
    fill_batch_shape(ctx, ba);
    ba.nsteps = nsteps; ba.forced_ld = ld; ba.lo_first = lo_first; ba.lo_rows = lo_rows;
    for (int b0 = 0; b0 < B; b0 += ctx->bq) {
      ba.Bq = std::min(ctx->bq, B - b0);
      ba.hidden = hidden + (size_t)b0 * k.in_dim;
      ba.sem_code = codes + (size_t)b0 * ld;
      ba.forced = codes + (size_t)b0 * ld;
      ba.codes_out = nullptr;
      ba.logits_out = logits + (size_t)b0 * lo_req;
      const int rc = launch_batched(ctx, ba, st);
      if (rc != S2FAST_OK) return rc;
    }
    return S2FAST_OK;
  }
  FrameArgs fa;
  fill_shape(ctx, fa);
  fa.nsteps = nsteps; fa.forced_ld = ld; fa.lo_first = lo_first; fa.lo_rows = lo_rows;
  for (int b = 0; b < B; ++b) {
    fa.hidden = hidden + (size_t)b * k.in_dim;
    fa.sem_code = codes + (size_t)b * ld;
    fa.forced = codes + (size_t)b * ld;
    fa.codes_out = nullptr;
    fa.logits_out = logits + (size_t)b * lo_req;
    const int rc = launch_frame(ctx, fa, st);
    if (rc != S2FAST_OK) return rc;
  }
  return S2FAST_OK;
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
    case S2FAST_ERR_SCRATCH: return "the shape's frame arena is larger than the library's static scratch";
    default: return "unknown error";
  }
}

int s2fast_create(const s2fast_config* cfg, const s2fast_weights* w, s2fast_ctx** out) {
  if (!cfg || !w || !out) return S2FAST_ERR_ARG;
  *out = nullptr;
  const s2fast_config& k = *cfg;
  const int epl = k.weight_dtype == S2FAST_BF16 ? 8 : (k.weight_dtype == S2FAST_Q8 ? 16 : 4);
  if (k.weight_dtype != S2FAST_BF16 && k.weight_dtype != S2FAST_F32 && k.weight_dtype != S2FAST_Q8)
    return S2FAST_ERR_ARG;
  if (k.n_layer < 1 || k.n_layer > S2FAST_MAX_LAYERS) return S2FAST_ERR_ARG;
  if (k.n_head < 1 || k.n_head_kv < 1 || k.n_head % k.n_head_kv != 0 || k.n_head_kv > 64) return S2FAST_ERR_ARG;
  if (k.head_dim < 8 || k.head_dim > 128 || (k.head_dim % 8)) return S2FAST_ERR_ARG;
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
  // an int8 model's row scales (one per output row of every matrix)
  if ((k.weight_dtype == S2FAST_Q8) != (w->q8_scales != nullptr)) {
    if (k.weight_dtype == S2FAST_Q8) return S2FAST_ERR_NO_FAST_DECODER;
    return S2FAST_ERR_ARG;
  }
  if (w->q8_scales) {
    const s2fast_q8_scales& q = *w->q8_scales;
    if (!q.output || (k.has_project_in && !q.project_in)) return S2FAST_ERR_NO_FAST_DECODER;
    for (int l = 0; l < k.n_layer; ++l) {
      const s2fast_q8_layer_scales& Q = q.layers[l];
      if (!Q.wqkv || !Q.wo || !Q.w1 || !Q.w3 || !Q.w2) return S2FAST_ERR_NO_FAST_DECODER;
    }
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
  c->w.q8_scales = nullptr;
  if (w->q8_scales) {
    c->q8 = *w->q8_scales;
    if (!k.has_project_in) c->q8.project_in = nullptr;
  }
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
  for (int n : {qkv_dim, 2 * k.ffn_dim, k.dim, k.codebook_size}) rmax = std::max(rmax, (n + P - 1) / P);
  rmax = std::max(rmax, 2 * ((k.ffn_dim + P - 1) / P));   // w1 and w3 rows of one block
  rmax = std::max(rmax, (k.dim + groups_min - 1) / std::max(groups_min, 1));
  (void)per_group;
  c->rmax = rmax + 1;
  size_t lds = lds_floats(c->kmax, c->rmax, gheads, k.head_dim, k.context, k.codebook_size, k.dim, k.n_layer) *
               sizeof(float);
  // more than half of the CU's 160 KB: exactly one block per CU
  const size_t one_per_cu = 84 * 1024;
  if (lds < one_per_cu) lds = one_per_cu;
  if (lds > (size_t)prop.sharedMemPerBlock) { free_ctx(c); return S2FAST_ERR_ARG; }
  c->lds_bytes = lds;
  const void* fn = frame_fn(k.weight_dtype);
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess) {
    free_ctx(c); return S2FAST_ERR_HIP;
  }
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, NTHREADS, lds) != hipSuccess) { free_ctx(c); return S2FAST_ERR_HIP; }
  if (nb < 1) { free_ctx(c); return S2FAST_ERR_DEVICE; }

  const int half = k.head_dim / 2;
  std::vector<float> rope((size_t)2 * k.context * half);
  rope_table_host(k.head_dim, k.context, k.rope_base, rope.data(), rope.data() + (size_t)k.context * half);
  // frame arena: one 256-byte aligned region per (decode step, layer)
  auto rup = [](long long n, long long q) { return (n + q - 1) / q * q; };
  const long long slots = (long long)(k.num_codebooks - 1) * k.n_layer;
  c->x_slot = rup((long long)MMAX * k.dim, 64);
  c->qkv_slot = rup((long long)MMAX * qkv_dim, 64);
  c->acc_slot = rup((long long)MMAX * k.dim, 32);
  c->g_slot = rup((long long)MMAX * k.ffn_dim, 64);
  c->logits_slot = rup(k.codebook_size, 64);
  c->kv_pos = rup((long long)k.n_head_kv * 2 * k.head_dim, 32);
  bool ok = dalloc(&c->rope, rope.size()) == hipSuccess && dalloc(&c->xin0, (size_t)rup(k.dim, 64)) == hipSuccess &&
            dalloc(&c->x, (size_t)(slots * c->x_slot)) == hipSuccess &&
            dalloc(&c->qkv, (size_t)(slots * c->qkv_slot)) == hipSuccess &&
            dalloc(&c->acc, (size_t)(slots * c->acc_slot)) == hipSuccess &&
            dalloc(&c->g, (size_t)(slots * c->g_slot)) == hipSuccess &&
            dalloc(&c->kv, (size_t)(k.n_layer * k.context * c->kv_pos)) == hipSuccess &&
            dalloc(&c->logits, (size_t)((k.num_codebooks - 1) * c->logits_slot)) == hipSuccess &&
            dalloc(&c->flags, (size_t)P * 64) == hipSuccess && dalloc(&c->err, W_WORDS) == hipSuccess;
  if (!ok) { free_ctx(c); return S2FAST_ERR_NOMEM; }
  ok = hipMemcpy(c->rope, rope.data(), rope.size() * sizeof(float), hipMemcpyHostToDevice) == hipSuccess &&
       hipMemset(c->acc, 0, (size_t)(slots * c->acc_slot) * sizeof(long long)) == hipSuccess &&
       hipMemset(c->x, 0, (size_t)(slots * c->x_slot) * sizeof(u64)) == hipSuccess &&
       hipMemset(c->qkv, 0, (size_t)(slots * c->qkv_slot) * sizeof(u64)) == hipSuccess &&
       hipMemset(c->g, 0, (size_t)(slots * c->g_slot) * sizeof(u64)) == hipSuccess &&
       hipMemset(c->logits, 0, (size_t)((k.num_codebooks - 1) * c->logits_slot) * sizeof(u64)) == hipSuccess &&
       hipMemset(c->flags, 0, (size_t)P * 64 * sizeof(u32)) == hipSuccess &&
       hipMemset(c->err, 0, W_WORDS * sizeof(u32)) == hipSuccess && hipDeviceSynchronize() == hipSuccess;
  if (!ok) { free_ctx(c); return S2FAST_ERR_HIP; }
  if (build_qkv0(c) != S2FAST_OK) { free_ctx(c); return S2FAST_ERR_HIP; }
  if (k.max_batch >= 2 && k.weight_dtype != S2FAST_Q8) {   // int8 models decode with the batch-1 kernel
    c->bq = batched_group(k, P);
    if (c->bq > 0) {
      c->b_lds = b_lds_bytes(k.n_layer, k.head_dim, k.context);
      const void* fb = k.weight_dtype == S2FAST_BF16 ? reinterpret_cast<const void*>(&frame_kernel_b<uint16_t>)
                                                     : reinterpret_cast<const void*>(&frame_kernel_b<float>);
      int nbb = 0;
      if (c->b_lds > (size_t)prop.sharedMemPerBlock ||
          hipFuncSetAttribute(fb, hipFuncAttributeMaxDynamicSharedMemorySize, (int)c->b_lds) != hipSuccess ||
          hipOccupancyMaxActiveBlocksPerMultiprocessor(&nbb, fb, NTHREADS, c->b_lds) != hipSuccess || nbb < 1) {
        c->bq = 0;   // batches then run one launch per request
      }
    }
    if (c->bq > 0) {
      c->bx_slot = rup((long long)MP_MAX * k.dim, 64);
      c->bqkv_slot = rup((long long)MP_MAX * qkv_dim, 64);
      c->batt_slot = rup((long long)MP_MAX * k.n_head * k.head_dim, 64);
      c->bg_slot = rup((long long)MP_MAX * k.ffn_dim, 64);
      c->blogits_slot = rup((long long)BQ_MAX * k.codebook_size, 64);
      ok = dalloc(&c->b_xin0, (size_t)BQ_MAX * k.dim) == hipSuccess &&
           dalloc(&c->b_x, (size_t)(slots * c->bx_slot)) == hipSuccess &&
           dalloc(&c->b_xmid, (size_t)(slots * c->bx_slot)) == hipSuccess &&
           dalloc(&c->b_qkv, (size_t)(slots * c->bqkv_slot)) == hipSuccess &&
           dalloc(&c->b_att, (size_t)(slots * c->batt_slot)) == hipSuccess &&
           dalloc(&c->b_g, (size_t)(slots * c->bg_slot)) == hipSuccess &&
           dalloc(&c->b_logits, (size_t)((k.num_codebooks - 1) * c->blogits_slot)) == hipSuccess &&
           dalloc(&c->b_kv, (size_t)BQ_MAX * k.n_layer * k.context * k.n_head_kv * 2 * k.head_dim) == hipSuccess &&
           dalloc(&c->b_codes, (size_t)BQ_MAX * 16) == hipSuccess;
      if (!ok) { free_ctx(c); return S2FAST_ERR_NOMEM; }
      // w2 and wo (the widest K: ffn and the attention width) split KS_DOWN
      // ways over K when the row groups and the slices fit the GEMM's tiles
      // (at most TMAX x 16 rows, whole k-steps).  The saved activation reads
      // outweigh the store / count / finalise round trips the split adds
      // (w2 26.5 -> 14.9 us a phase at batch 16; wo about 1 % of a launch).
      const int ksz = k.weight_dtype == S2FAST_BF16 ? 32 : 16;
      const int ks = KS_DOWN;
      const bool rows_fit = P % ks == 0 && (k.dim + P / ks - 1) / (P / ks) <= 16 * TMAX;
      c->b_ks[BK_DOWN] = (rows_fit && k.ffn_dim % (ks * ksz) == 0) ? ks : 1;
      c->b_ks[BK_WO] = (rows_fit && (k.n_head * k.head_dim) % (ks * ksz) == 0) ? ks : 1;
      // wqkv splits two ways (its row groups must also fit TMAX tiles); its
      // consumer, the attention, adds the two slices itself
      constexpr int kq = 2;
      static_assert(kq <= 2, "the attention gather and the sample phase add at most two slices of wqkv / the head");
      c->b_ks[BK_QKV] = (P % kq == 0 && (qkv_dim + P / kq - 1) / (P / kq) <= 16 * TMAX && k.dim % (kq * ksz) == 0)
                            ? kq : 1;
      // the head too, its consumer (the sample phase) adding the slices
      c->b_ks[BK_HEAD] = (P % kq == 0 && (k.codebook_size + P / kq - 1) / (P / kq) <= 16 * TMAX &&
                          k.dim % (kq * ksz) == 0) ? kq : 1;
      c->b_kslot[BK_WO] = c->b_kslot[BK_DOWN] = c->bx_slot;
      c->b_kslot[BK_QKV] = c->bqkv_slot;
      c->b_kslot[BK_HEAD] = c->blogits_slot;
      for (int kd : {(int)BK_QKV, (int)BK_WO, (int)BK_DOWN, (int)BK_HEAD}) {
        if (c->b_ks[kd] == 1) continue;
        ok = dalloc(&c->b_kpart[kd], (size_t)(slots * c->b_ks[kd] * c->b_kslot[kd])) == hipSuccess &&
             dalloc(&c->b_kcnt[kd], (size_t)(slots * P * KCNT_STRIDE)) == hipSuccess &&
             dalloc(&c->b_kss[kd], (size_t)(slots * c->b_ks[kd] * MP_MAX)) == hipSuccess &&
             hipMemset(c->b_kcnt[kd], 0, (size_t)(slots * P * KCNT_STRIDE) * sizeof(int)) == hipSuccess;
        if (!ok) { free_ctx(c); return S2FAST_ERR_NOMEM; }
      }
      const int pst = pack_batched(c);
      if (pst != S2FAST_OK) { free_ctx(c); return pst; }
    }
  }
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
  const int nsteps = ctx->cfg.num_codebooks - 1;
  if (B == 1 || ctx->bq == 0) return B * syncs_for(ctx->cfg, nsteps);
  int n = 0;
  for (int b0 = 0; b0 < B; b0 += ctx->bq) {
    const int Bg = std::min(ctx->bq, B - b0);
    n += b_syncs(ctx->cfg.has_project_in, nsteps, ctx->cfg.n_layer, false, false,
                 b_merged_draw(Bg, ctx->cfg.n_head_kv, ctx->ncu));
  }
  return n;
}

int s2fast_decode_frame(s2fast_ctx* ctx, int32_t B, const float* hidden, const int32_t* sem_code,
                        const float* uniforms, const float* temperature, const float* top_p,
                        const int32_t* top_k, int32_t* codes, void* stream) {
  if (!ctx) return S2FAST_ERR_ARG;
  if (B < 1 || B > ctx->cfg.max_batch) return S2FAST_ERR_BATCH;
  if (!hidden || !sem_code || !uniforms || !temperature || !top_p || !top_k || !codes) return S2FAST_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(hidden) & 15u) return S2FAST_ERR_ARG;   // read in 16-byte quads
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const s2fast_config& k = ctx->cfg;
  int rc = S2FAST_OK;
  int done = 0;   // requests whose launch was enqueued
  if (B >= 2 && ctx->bq > 0) {
    BatchArgs ba;
    fill_batch_shape(ctx, ba);
    for (int b0 = 0; b0 < B && rc == S2FAST_OK; b0 += ctx->bq) {
      ba.Bq = std::min(ctx->bq, B - b0);
      ba.hidden = hidden + (size_t)b0 * k.in_dim;
      ba.sem_code = sem_code + b0;
      ba.uniforms = uniforms + (size_t)b0 * (k.num_codebooks - 1);
      ba.temp = temperature + b0;
      ba.top_p = top_p + b0;
      ba.top_k = top_k + b0;
      ba.forced = nullptr;
      ba.codes_out = codes + (size_t)b0 * k.num_codebooks;
      ba.logits_out = nullptr;
      rc = launch_batched(ctx, ba, st);
      if (rc == S2FAST_OK) done = b0 + ba.Bq;
    }
  }
  FrameArgs fa;
  fill_shape(ctx, fa);
  for (int b = 0; b < B && rc == S2FAST_OK && !(B >= 2 && ctx->bq > 0); ++b) {
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
    if (rc == S2FAST_OK) done = b + 1;
  }
  if (rc != S2FAST_OK) {
    // the requests whose launch could not be enqueued leave codebooks 1.. at
    // 0 ("Fast-AR codebook decoding ...", section 5.2); earlier launches
    // keep their codes
    (void)hipMemset2DAsync(codes + (size_t)done * k.num_codebooks + 1, (size_t)k.num_codebooks * sizeof(int32_t), 0,
                           (size_t)(k.num_codebooks - 1) * sizeof(int32_t), (size_t)(B - done), st);
  }
  return rc;
}

int s2fast_forward_logits(s2fast_ctx* ctx, int32_t B, const float* hidden, const int32_t* codes, float* logits,
                          void* stream) {
  if (!ctx) return S2FAST_ERR_ARG;
  if (B < 1 || B > ctx->cfg.max_batch) return S2FAST_ERR_BATCH;
  if (!hidden || !codes || !logits) return S2FAST_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(hidden) & 15u) return S2FAST_ERR_ARG;   // read in 16-byte quads
  const int n = ctx->cfg.num_codebooks;
  return launch_forced(ctx, B, hidden, codes, n, n - 1, logits, 1, n - 1, reinterpret_cast<hipStream_t>(stream));
}

int s2fast_fast_decode(s2fast_ctx* ctx, int32_t B, const float* hidden, int32_t hidden_dim, const int32_t* prefix,
                       int32_t prefix_len, float* logits, void* stream) {
  if (!ctx) return S2FAST_ERR_ARG;
  if (hidden_dim != ctx->cfg.in_dim) return S2FAST_ERR_HIDDEN_DIM;
  if (prefix_len < 1 || prefix_len >= ctx->cfg.num_codebooks) return S2FAST_ERR_PREFIX_LEN;
  if (B < 1 || B > ctx->cfg.max_batch) return S2FAST_ERR_BATCH;
  if (!hidden || !prefix || !logits) return S2FAST_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(hidden) & 15u) return S2FAST_ERR_ARG;
  return launch_forced(ctx, B, hidden, prefix, prefix_len, prefix_len, logits, prefix_len, 1,
                       reinterpret_cast<hipStream_t>(stream));
}

int s2fast_decode_frame_static(s2fast_ctx* ctx, int32_t B, const float* hidden, const int32_t* sem_code,
                               const float* uniforms, const float* temperature, const float* top_p,
                               const int32_t* top_k, int32_t* codes, void* stream) {
  if (!ctx) return S2FAST_ERR_ARG;
  if (B < 1 || B > ctx->cfg.max_batch) return S2FAST_ERR_BATCH;
  if (!hidden || !sem_code || !uniforms || !temperature || !top_p || !top_k || !codes) return S2FAST_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(hidden) & 15u) return S2FAST_ERR_ARG;
  const StaticLayout L = static_layout(ctx);
  if (L.end > STATIC_SCRATCH_BYTES) return S2FAST_ERR_SCRATCH;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return S2FAST_ERR_HIP;
  if (dev != ctx->device || dev < 0 || dev >= STATIC_MAX_DEVICES) return S2FAST_ERR_DEVICE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const s2fast_config& k = ctx->cfg;
  std::lock_guard<std::mutex> lock(g_static_mu);
  StaticScratch& S = g_static[dev];
  if (!S.ptr) {
    // once per device, with that device current: the array's device address
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return S2FAST_ERR_HIP;
    S.ptr = static_cast<char*>(p);
  }
  // The accumulators must start at zero and the flags below the first
  // epoch.  Every launch leaves its own layout so (a failed one through its
  // recovery), but a context of another shape lays the arena out
  // differently (its accumulators may sit where the last one kept
  // activations): the array is cleared on the first call, when the layout
  // changes, and when the epoch counter would wrap.
  const size_t key[3] = {L.acc, L.flags, L.end};
  if (!S.cleared || S.epoch > 0xF0000000u || std::memcmp(key, S.layout, sizeof(key)) != 0) {
    if (zero_device(S.ptr, STATIC_SCRATCH_BYTES, st) != S2FAST_OK) return S2FAST_ERR_HIP;
    S.cleared = true;
    S.epoch = 0;
    std::memcpy(S.layout, key, sizeof(key));
  }
  FrameArgs fa;
  fill_shape(ctx, fa);
  fa.xin0 = reinterpret_cast<float*>(S.ptr + L.xin0);
  fa.x = reinterpret_cast<u64*>(S.ptr + L.x);
  fa.qkv = reinterpret_cast<u64*>(S.ptr + L.qkv);
  fa.acc = reinterpret_cast<long long*>(S.ptr + L.acc);
  fa.g = reinterpret_cast<u64*>(S.ptr + L.g);
  fa.kv = reinterpret_cast<float*>(S.ptr + L.kv);
  fa.logits = reinterpret_cast<u64*>(S.ptr + L.logits);
  fa.flags = reinterpret_cast<u32*>(S.ptr + L.flags);
  fa.tlog = nullptr;
  const void* fn = frame_fn(k.weight_dtype);
  const u32 n = (u32)syncs_for(k, fa.nsteps);
  int done = 0, rc = S2FAST_OK;
  for (int b = 0; b < B; ++b) {
    fa.hidden = hidden + (size_t)b * k.in_dim;
    fa.sem_code = sem_code + b;
    fa.uniforms = uniforms + (size_t)b * (k.num_codebooks - 1);
    fa.temp = temperature + b;
    fa.top_p = top_p + b;
    fa.top_k = top_k + b;
    fa.forced = nullptr;
    fa.codes_out = codes + (size_t)b * k.num_codebooks;
    fa.logits_out = nullptr;
    fa.epoch0 = S.epoch;
    void* args[] = {&fa};
    if (hipLaunchCooperativeKernel(fn, dim3(ctx->ncu), dim3(NTHREADS), args, ctx->lds_bytes, st) != hipSuccess) {
      rc = S2FAST_ERR_HIP;
      break;
    }
    S.epoch += n;
    done = b + 1;
  }
  if (rc != S2FAST_OK)
    (void)hipMemset2DAsync(codes + (size_t)done * k.num_codebooks + 1, (size_t)k.num_codebooks * sizeof(int32_t), 0,
                           (size_t)(k.num_codebooks - 1) * sizeof(int32_t), (size_t)(B - done), st);
  return rc;
}

int s2fast_status(s2fast_ctx* ctx, void* stream) {
  if (!ctx) return S2FAST_ERR_ARG;
  return read_status(ctx->err, reinterpret_cast<hipStream_t>(stream));
}

int s2fast_test_watchdog(s2fast_ctx* ctx, int32_t give_up) {
  if (!ctx) return S2FAST_ERR_ARG;
  ctx->give_up = give_up ? 1u : 0u;
  return S2FAST_OK;
}

int s2fast_test_timeline(s2fast_ctx* ctx, int32_t enable, uint32_t* host_out, int32_t capacity) {
  if (!ctx) return S2FAST_ERR_ARG;
  const size_t n = (size_t)ctx->ncu * TLOG_MAX * TLOG_W;
  if (!ctx->tlog) {
    if (hipMalloc(reinterpret_cast<void**>(&ctx->tlog), n * sizeof(u32)) != hipSuccess) return S2FAST_ERR_NOMEM;
    if (hipMemset(ctx->tlog, 0, n * sizeof(u32)) != hipSuccess) return S2FAST_ERR_HIP;
  }
  ctx->tlog_on = enable != 0;
  if (host_out) {
    if (capacity < (int64_t)n) return S2FAST_ERR_ARG;
    if (hipDeviceSynchronize() != hipSuccess) return S2FAST_ERR_HIP;
    if (hipMemcpy(host_out, ctx->tlog, n * sizeof(u32), hipMemcpyDeviceToHost) != hipSuccess) return S2FAST_ERR_HIP;
  }
  return S2FAST_OK;
}

int s2fast_test_stream_read(const void* src, uint64_t bytes, int32_t grid, int32_t in_flight, uint32_t* sink,
                            void* stream) {
  if (!src || !sink || (reinterpret_cast<uintptr_t>(src) & 15u) || bytes == 0 || (bytes & 15u) || grid < 1 ||
      grid > 65535 || (in_flight != 4 && in_flight != 8))
    return S2FAST_ERR_ARG;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return S2FAST_ERR_HIP;
  if (!is_gfx950(dev)) return S2FAST_ERR_DEVICE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (hipMemsetAsync(sink, 0, sizeof(u32), st) != hipSuccess) return S2FAST_ERR_HIP;
  const u32x4* p = reinterpret_cast<const u32x4*>(src);
  if (in_flight == 4) hipLaunchKernelGGL(stream_read_kernel<4>, dim3(grid), dim3(NTHREADS), 0, st, p, bytes / 16, sink);
  else hipLaunchKernelGGL(stream_read_kernel<8>, dim3(grid), dim3(NTHREADS), 0, st, p, bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? S2FAST_OK : S2FAST_ERR_HIP;
}

int s2fast_test_rope_table(int32_t head_dim, int32_t context, float rope_base, float* cos_out, float* sin_out) {
  if (!cos_out || !sin_out || head_dim < 2 || (head_dim & 1) || context < 1 || !(rope_base > 0.0f))
    return S2FAST_ERR_ARG;
  rope_table_host(head_dim, context, rope_base, cos_out, sin_out);
  return S2FAST_OK;
}

int s2fast_test_gemv(int32_t weight_dtype, int32_t N, int32_t K, int32_t M, const void* W, const void* W3,
                     const float* scale, const float* scale3, const void* norm_w, float eps, const float* x, float* y,
                     void* stream) {
  const int epl = weight_dtype == S2FAST_BF16 ? 8 : (weight_dtype == S2FAST_Q8 ? 16 : 4);
  if (weight_dtype != S2FAST_BF16 && weight_dtype != S2FAST_F32 && weight_dtype != S2FAST_Q8) return S2FAST_ERR_ARG;
  if (N < 1 || K < epl || K > 16384 || (K % epl) || M < 1 || M > MMAX || !W || !x || !y) return S2FAST_ERR_ARG;
  if ((weight_dtype == S2FAST_Q8) != (scale != nullptr) || (W3 && (scale != nullptr) != (scale3 != nullptr)) ||
      (!W3 && scale3))
    return S2FAST_ERR_ARG;
  auto mis = [](const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u); };
  if (mis(W) || mis(W3) || mis(norm_w) || mis(x)) return S2FAST_ERR_ARG;
  int dev = 0, P = 0;
  if (hipGetDevice(&dev) != hipSuccess) return S2FAST_ERR_HIP;
  if (!is_gfx950(dev)) return S2FAST_ERR_DEVICE;
  if (hipDeviceGetAttribute(&P, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return S2FAST_ERR_HIP;
  GemvTestArgs a;
  a.N = N; a.K = K; a.M = M; a.kmax = (K + 3) & ~3; a.rmax = (W3 ? 2 : 1) * ((N + P - 1) / P) + 1;
  a.W = W; a.W3 = W3; a.sc = scale; a.sc3 = scale3; a.normw = norm_w; a.eps = eps; a.x = x; a.y = y;
  const size_t lds = ((((size_t)MMAX * a.kmax + 3) & ~(size_t)3) + (size_t)a.rmax * NWAVE * MMAX + 64 +
                      (size_t)a.rmax) * sizeof(float);
  const void* fn = weight_dtype == S2FAST_BF16 ? reinterpret_cast<const void*>(&gemv_test_kernel<uint16_t>)
                   : weight_dtype == S2FAST_Q8 ? reinterpret_cast<const void*>(&gemv_test_kernel<q8_t>)
                                               : reinterpret_cast<const void*>(&gemv_test_kernel<float>);
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
    return S2FAST_ERR_ARG;
  void* args[] = {&a};
  if (hipLaunchKernel(fn, dim3(P), dim3(NTHREADS), args, lds, reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return S2FAST_ERR_HIP;
  return S2FAST_OK;
}

int s2fast_test_norm_rope_attn(int32_t n_head, int32_t n_head_kv, int32_t head_dim, int32_t T, int32_t context,
                               float rope_base, float eps, const float* qkv, const float* q_norm, const float* k_norm,
                               float* out, void* stream) {
  if (n_head < 1 || n_head_kv < 1 || n_head % n_head_kv || head_dim < 8 || head_dim > 128 || (head_dim % 8) ||
      context < 1 || context > 16 || T < 1 || T > context || !(rope_base > 0.0f) || !qkv || !out ||
      (!q_norm) != (!k_norm))
    return S2FAST_ERR_ARG;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return S2FAST_ERR_HIP;
  if (!is_gfx950(dev)) return S2FAST_ERR_DEVICE;
  const int half = head_dim / 2;
  std::vector<float> rope((size_t)2 * context * half);
  rope_table_host(head_dim, context, rope_base, rope.data(), rope.data() + (size_t)context * half);
  float* drope = nullptr;
  if (hipMalloc(reinterpret_cast<void**>(&drope), rope.size() * sizeof(float)) != hipSuccess) return S2FAST_ERR_NOMEM;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  AttnTestArgs a;
  a.H = n_head; a.G = n_head_kv; a.hd = head_dim; a.T = T; a.ctx = context; a.has_qkn = q_norm ? 1 : 0;
  a.eps = eps; a.qkv = qkv; a.qn = q_norm ? q_norm : drope; a.kn = k_norm ? k_norm : drope; a.rope = drope;
  a.out = out;
  const int gh = n_head / n_head_kv;
  const size_t lds = ((size_t)gh * head_dim + 3 * (size_t)context * head_dim + (size_t)gh * head_dim) * sizeof(float);
  int rc = S2FAST_OK;
  void* args[] = {&a};
  if (hipMemcpyAsync(drope, rope.data(), rope.size() * sizeof(float), hipMemcpyHostToDevice, st) != hipSuccess ||
      hipLaunchKernel(reinterpret_cast<const void*>(&attn_test_kernel), dim3(n_head_kv, T), dim3(NTHREADS), args,
                      lds, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    rc = S2FAST_ERR_HIP;
  (void)hipFree(drope);
  return rc;
}

int s2fast_test_sample(int32_t B, int32_t V, const float* logits, const float* temperature, const float* top_p,
                       const int32_t* top_k, const float* u, int32_t* codes, void* stream) {
  if (B < 1 || V < 1 || V > 8192 || !logits || !temperature || !top_p || !top_k || !u || !codes) return S2FAST_ERR_ARG;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return S2FAST_ERR_HIP;
  if (!is_gfx950(dev)) return S2FAST_ERR_DEVICE;
  hipLaunchKernelGGL(sample_kernel, dim3(B), dim3(NTHREADS), 0, reinterpret_cast<hipStream_t>(stream), V, logits,
                     temperature, top_p, top_k, u, codes);
  return hipGetLastError() == hipSuccess ? S2FAST_OK : S2FAST_ERR_HIP;
}

}  // extern "C"

// ======================================================= Slow-AR host side
#include "slow_host.h"
