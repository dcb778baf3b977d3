// Slow-AR decode step: one cooperative launch computes one new position of
// one request and draws its main token.  Included by s2fast.hip inside its
// anonymous namespace; it uses the GEMV, grid-barrier and sampler helpers
// defined there.
//
// What one step computes ("Overall architecture & Dual-AR data flow",
// sections 3.2 and 3.4; "Fast-AR codebook decoding and the generation main
// loop", sections 5 and 6):
//   x = sem_scale * embeddings[main] + sum_j codebook_embeddings[j*cbs + c_j]
//   36 x { RMSNorm -> wqkv -> q/k RMSNorm + pair RoPE at position n_past ->
//          attention over the KV cache (positions 0..n_past, the new key and
//          value written at n_past in the cache's precision) -> wo -> + x;
//          RMSNorm -> w1, w3 -> silu * -> w2 -> + x }
//   hidden = RMSNorm(x, norm); logits = embeddings . hidden (tied);
//   main token drawn from logits + sem_mask, redrawn at temperature 1.0 /
//   top_p 0.9 if it is a semantic id already among the last 10 main tokens.
//
// Per layer the blocks run five phases.  The outputs of QKV, ATTN, UP and
// DOWN (and the head's logits) are tagged values that the next phase waits
// on itself; WO is closed by a grid barrier:
//   QKV   RMSNorm(x) -> rows of wqkv
//   ATTN  block (g, c): KV group g, chunk c of the positions.  The group's
//         query heads and the new key/value are normalised and rotated in
//         LDS; the chunk's keys/values stream from the cache once for all
//         the group's query heads; each wave keeps an online softmax over
//         its positions; the block leaves one (max, sum, output) partial per
//         head, and the group's last chunk to finish (a count per group)
//         merges the partials (log-sum-exp weights) into the group's
//         attention output (a two-position launch: a grid barrier, then
//         every WO block merges them itself)
//   WO    block (g, row group): wo rows over the group's columns of the
//         attention output, added across groups in an int64 fixed-point
//         accumulator
//   UP    RMSNorm(x + attn) -> w1, w3 rows -> silu(a1) * a3
//   DOWN  w2 rows; x = x + attn + ffn
// then the head (only the rows sem_mask leaves finite: every other logit is
// -inf and can never be drawn) and, in block 0, the draw.  A prefill
// position before the prompt's last stops after the last layer (do_head 0):
// it only writes its keys and values into the cache.

constexpr int SLOW_MAX_LAYERS = S2FAST_SLOW_MAX_LAYERS;
constexpr int RAS_WIN = 10;     // repetition window (main-loop page, section 6)
constexpr int SPPW = 12;        // attention positions per wave per load batch
constexpr int GH_MAX = 8;       // query heads per KV group

struct SlowArgs {
  int dim, n_layer, n_head, n_kv, hd, ffn, vocab, ncb, cbs;
  int sem_begin, end_id, nsem, n_allowed, end_first;
  float eps, sem_scale;
  int has_qkn, qkv_dim, attn_dim, gheads, gw, kmax, rmax;
  int max_ctx, n_past, nchunk;
  int do_head;        // 0: prefill positions before the prompt's last (no head, no draw)
  int M;              // positions this launch: n_past .. n_past + M - 1 (M <= MMAX)
  const void* emb;    // [vocab][dim]
  const void* cemb;   // [ncb * cbs][dim]
  const void* norm;   // [dim]
  const LayerPtr* L;  // [n_layer] in device memory (the kernel argument stays small)
  const float* rope;  // [2][max_ctx][hd/2]: cos then sin
  void* kv;           // [n_layer][n_kv][max_ctx][2][hd] keys then values, weight type
  // the request
  const int* prev_main;     // [1] the previous frame's main token
  const int* prev_codes;    // [ncb] and its codes
  const int* main1;         // [1], [ncb]: the second position's tokens (M = 2)
  const int* codes1;
  int* window;              // [1 + RAS_WIN]: count, then main tokens oldest first
  const float* u;           // [2]: main draw, repetition redraw
  const float* temp;
  const float* top_p;
  const int* top_k;
  int* main_out;            // [1]
  int* sem_out;             // [1] clamp(main - sem_begin, 0, cbs - 1)
  float* hidden_out;        // [dim]
  float* logits_out;        // [n_allowed] or nullptr
  // per-launch arena: every region is written once per launch.  x, qkv, g
  // and logits are tagged values (the launch's tag beside each float) read
  // with tagged waits; the others are read only after the barrier that
  // follows their writes (see FrameArgs)
  float* x0;                // [MMAX][dim] the positions' input vectors
  u64* x;                   // [n_layer][x_slot]: [MMAX][dim] per layer (tagged)
  u64* qkv;                 // [n_layer][qkv_slot]: [MMAX][qkv_dim] (tagged)
  long long* acc;           // [n_layer][acc_slot]: [MMAX][dim] (zero between launches)
  u64* g;                   // [n_layer][g_slot]: [MMAX][ffn] (tagged)
  float* po;                // [n_layer][n_kv][nchunk][MMAX][gheads][hd] chunk outputs
  float* pml;               // [n_layer][n_kv][nchunk][MMAX][gheads][2] chunk max and sum
  u64* att;                 // [n_layer][att_slot]: [MMAX][attn_dim] merged attention output (tagged)
  int* acnt;                // [n_layer][n_kv][64] chunks of a group done (zero between launches)
  u64* logits;              // [n_allowed] (tagged)
  long long x_slot, qkv_slot, acc_slot, g_slot, po_slot, pml_slot, att_slot;
  u32* flags;
  u32 epoch0;               // epoch0 + 1 tags this launch's outputs
  u32* err;                 // watchdog words (see Watch)
  Watch watch;
  u32* tlog;
  u32 tlog_epoch;
  // head-only launch (not null): the layers are skipped and the head reads
  // this row as the last layer's output (a chunked prefill wrote it)
  const float* x_head;
};

struct SlowLds {
  float* act;    // [MMAX][kmax] GEMV activation rows (phys() layout)
  float* red;    // [rmax][MMAX][NWAVE]
  float* small;  // [64]
  float* q;      // [MMAX][gheads + 2][hd]: per position the group's query heads, its new key and value
  float* qkn;    // [2][hd] q_norm, k_norm
  float* ow;     // [NWAVE][gheads][hd + 2] per-wave attention partials
  float* mrg;    // [NTHREADS][6] chunk-merge partials (max, sum, 4 outputs)
  float* rope1;  // [MMAX][hd]: cos then sin at positions n_past + m
  float* cval;
  int* cidx;
  u32* mark;
  int* flag;     // [8]: [0] grid sync result, [1] timeline record, [2..3] launch exit, [4] a tag wait gave up,
                 // [5] this block merges its group's chunks
  int* tok;      // [64]: row-0 token and codes of position m at 32 m, its codes flag at 32 m + 20; the draw at [16..17]
};

__host__ __device__ inline size_t slow_lds_floats(int kmax, int rmax, int gheads, int hd) {
  const size_t act = (size_t)MMAX * (((size_t)kmax + 3) & ~(size_t)3);
  return act + (size_t)rmax * NWAVE * MMAX + 64 + (size_t)MMAX * (gheads + 2) * hd + 2 * (size_t)hd +
         (size_t)NWAVE * gheads * (hd + 2) + 6 * (size_t)NTHREADS + (size_t)MMAX * hd + 2 * TOPK_MAX + 256 + 8 + 64;
}

__device__ inline SlowLds slow_carve(float* base, const SlowArgs& a) {
  SlowLds s;
  float* p = base;
  s.act = p; p += (size_t)MMAX * (((size_t)a.kmax + 3) & ~(size_t)3);
  s.red = p; p += (size_t)a.rmax * NWAVE * MMAX;
  s.small = p; p += 64;
  s.q = p; p += (size_t)MMAX * (a.gheads + 2) * a.hd;
  s.qkn = p; p += 2 * (size_t)a.hd;
  s.ow = p; p += (size_t)NWAVE * a.gheads * (a.hd + 2);
  s.mrg = p; p += 6 * (size_t)NTHREADS;
  s.rope1 = p; p += (size_t)MMAX * a.hd;
  s.cval = p; p += TOPK_MAX;
  s.cidx = reinterpret_cast<int*>(p); p += TOPK_MAX;
  s.mark = reinterpret_cast<u32*>(p); p += 256;
  s.flag = reinterpret_cast<int*>(p); p += 8;
  s.tok = reinterpret_cast<int*>(p);
  return s;
}

// Layer l's input (l == n_layer: the head's): at layer 0 the step's input
// vectors x0, past the last layer of a head-only launch the row the chunked
// prefill wrote (both plain floats), otherwise the previous layer's tagged
// output.
__device__ __forceinline__ bool slow_in_tagged(const SlowArgs& a, int l) {
  return l > 0 && !(a.x_head && l == a.n_layer);
}
__device__ __forceinline__ const float* slow_in_plain(const SlowArgs& a, int l) { return l == 0 ? a.x0 : a.x_head; }
__device__ __forceinline__ const u64* slow_in_tag(const SlowArgs& a, int l) { return a.x + (size_t)(l - 1) * a.x_slot; }
__device__ __forceinline__ u32 slow_tag(const SlowArgs& a) { return a.epoch0 + 1u; }
__device__ __forceinline__ TagWait slow_tw(const SlowArgs& a, const SlowLds& s) {
  return TagWait{a.err, s.flag + 4, slow_tag(a), a.watch.give_up};
}

// the cache's element type: bf16 (round to nearest even) or f32
template <typename WT> struct KVElem;
template <> struct KVElem<uint16_t> {
  using pair = u32;
  __device__ static __forceinline__ pair load(const uint16_t* p) { return *reinterpret_cast<const u32*>(p); }
  __device__ static __forceinline__ float lo(pair v) { return __uint_as_float(v << 16); }
  __device__ static __forceinline__ float hi(pair v) { return __uint_as_float(v & 0xFFFF0000u); }
  __device__ static __forceinline__ uint16_t enc(float x) {
    const u32 b = __float_as_uint(x);
    return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
  }
  __device__ static __forceinline__ float round(float x) { return __uint_as_float((u32)enc(x) << 16); }
};
template <> struct KVElem<float> {
  using pair = u64;
  __device__ static __forceinline__ pair load(const float* p) { return *reinterpret_cast<const u64*>(p); }
  __device__ static __forceinline__ float lo(pair v) { return lo_f32(v); }
  __device__ static __forceinline__ float hi(pair v) { return hi_f32(v); }
  __device__ static __forceinline__ float enc(float x) { return x; }
  __device__ static __forceinline__ float round(float x) { return x; }
};

// token id of row i of the head (the ids sem_mask leaves finite, ascending)
__device__ __forceinline__ int slow_token(const SlowArgs& a, int i) {
  if (a.end_first) return i == 0 ? a.end_id : a.sem_begin + i - 1;
  return i < a.nsem ? a.sem_begin + i : a.end_id;
}

enum SlowPhase { SP_QKV = 0, SP_ATTN, SP_WO, SP_UP, SP_DOWN, SP_HEAD };

__device__ __forceinline__ void slow_wo_rows(const SlowArgs& a, int& g, int& r0, int& r1) {
  const int P = gridDim.x;
  g = blockIdx.x % a.n_kv;
  const int rg = blockIdx.x / a.n_kv;
  const int Pg = (P - g + a.n_kv - 1) / a.n_kv;
  split_rows(a.dim, rg, Pg, r0, r1);
}

template <typename WT>
__device__ __forceinline__ Plan slow_plan(const SlowArgs& a, int l, int kind) {
  const int P = gridDim.x, b = blockIdx.x;
  const WT* emb = reinterpret_cast<const WT*>(a.emb);
  int r0 = 0, r1 = 0, g = 0;
  Plan p;
  if (kind == SP_HEAD) {
    split_rows(a.n_allowed, b, P, r0, r1);
    const int n = r1 - r0;
    const long long D = a.dim;
    if (a.end_first) {
      if (r0 == 0) p = make_plan<WT>(emb + (long long)a.end_id * D, emb + (long long)a.sem_begin * D, D, 0, a.dim, 0, min(n, 1), n);
      else p = make_plan<WT>(emb + (long long)(a.sem_begin + r0 - 1) * D, nullptr, D, 0, a.dim, 0, n, n);
    } else {
      const int na = max(0, min(r1, a.nsem) - r0);
      const WT* wa = na > 0 ? emb + (long long)(a.sem_begin + r0) * D : emb;
      p = make_plan<WT>(wa, emb + (long long)a.end_id * D, D, 0, a.dim, 0, na, n);
    }
  } else {
    const LayerPtr& L = a.L[l];
    switch (kind) {
      case SP_QKV:
        split_rows(a.qkv_dim, b, P, r0, r1);
        p = make_plan<WT>((const WT*)L.wqkv, nullptr, a.dim, 0, a.dim, r0, r1 - r0, r1 - r0);
        break;
      case SP_WO:
        slow_wo_rows(a, g, r0, r1);
        p = make_plan<WT>((const WT*)L.wo, nullptr, a.attn_dim, g * a.gw, a.gw, r0, r1 - r0, r1 - r0);
        break;
      case SP_UP:
        split_rows(a.ffn, b, P, r0, r1);
        p = make_plan<WT>((const WT*)L.w1, (const WT*)L.w3, a.dim, 0, a.dim, r0, r1 - r0, 2 * (r1 - r0));
        break;
      case SP_DOWN:
        split_rows(a.dim, b, P, r0, r1);
        p = make_plan<WT>((const WT*)L.w2, nullptr, a.ffn, 0, a.ffn, r0, r1 - r0, r1 - r0);
        break;
      default:   // attention: no GEMV
        p = make_plan<WT>(emb, nullptr, a.dim, 0, a.dim, 0, 0, 0);
        break;
    }
  }
  p.r0 = r0;
  p.r1 = r1;
  p.g = g;
  return p;
}

// Layer input into LDS act (GEMV layout over dim columns) times the phase's
// RMSNorm weight; the per-wave sums of squares go to small.  MODE 0: the
// step's input vector built from the embedding tables (block 0 also stores
// it to the arena for the later phases of layer 0); 1: the previous layer's
// output; 2: layer input + the attention accumulator (x_mid).  TAGGED: the
// layer input is tagged (slow_in_tagged).
template <typename WT, int MODE, bool TAGGED, typename Hook>
__device__ __forceinline__ void slow_stage(const SlowArgs& a, const SlowLds& s, int l, int m0, int Mr, const WT* normw,
                                           const Hook& hook) {
  constexpr int NS = MODE == 0 ? 2 : (TAGGED ? 2 : 3);
  constexpr int NT = 11;                    // main token + at most 10 codebook rows per batch step
  const int hq = a.dim >> 2;
  const int nq = Mr * hq;                   // rows m0 .. m0 + Mr - 1 (Mr <= 2), row by row
  const float* src = TAGGED ? nullptr : slow_in_plain(a, l);
  const u64* tsrc = TAGGED ? slow_in_tag(a, l) : nullptr;
  const WT* emb = reinterpret_cast<const WT*>(a.emb);
  const WT* cemb = reinterpret_cast<const WT*>(a.cemb);
  float ss0 = 0.0f, ss1 = 0.0f;
  auto batch = [&](int base, const auto& after) __attribute__((always_inline)) {
    u64 t[TAGGED ? 4 * NS : 1];
    v4f xv[NS];
    v2ll a0[NS], a1[NS];
    typename WQuad<WT>::type wv[NS], ev[NS][NT];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int q = quad_of(base, j, nq);
      const int r = q >= hq ? 1 : 0, c = q - r * hq, m = m0 + r;
      wv[j] = WQuad<WT>::load(normw, c);
      if (MODE == 0) {
        const int* tk = s.tok + 32 * m;
        ev[j][0] = WQuad<WT>::load(emb + (size_t)tk[0] * a.dim, c);
#pragma unroll
        for (int t = 1; t < NT; ++t) {
          const int jj = min(t - 1, a.ncb - 1);
          ev[j][t] = WQuad<WT>::load(cemb + ((size_t)jj * a.cbs + tk[1 + jj]) * a.dim, c);
        }
      } else {
        if constexpr (TAGGED) {
          const u64* p = tsrc + (size_t)m * a.dim + 4 * c;
          ld_tagged2(p, t[4 * j], t[4 * j + 1]);
          ld_tagged2(p + 2, t[4 * j + 2], t[4 * j + 3]);
        } else {
          xv[j] = *reinterpret_cast<const v4f*>(src + (size_t)m * a.dim + 4 * c);
        }
        if (MODE == 2) {
          const long long* ac = a.acc + (size_t)l * a.acc_slot + (size_t)m * a.dim + 4 * c;
          a0[j] = *reinterpret_cast<const v2ll*>(ac);
          a1[j] = *reinterpret_cast<const v2ll*>(ac + 2);
        }
      }
    }
    after();
    if constexpr (MODE != 0 && TAGGED)
      tag_wait(slow_tw(a, s), t, [&](int i) __attribute__((always_inline)) {
        const int q = quad_of(base, i >> 2, nq);
        const int r = q >= hq ? 1 : 0, c = q - r * hq;
        return tsrc + (size_t)(m0 + r) * a.dim + 4 * c + (i & 3);
      });
    const int nj = steps_opaque(nq, base);
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      if (j >= nj) break;
      const int cu = base + j * NTHREADS + tidx();
      const int q = min(cu, nq - 1);
      const int r = q >= hq ? 1 : 0, c = q - r * hq, m = m0 + r;
      float v[4];
      if (MODE == 0) {
        // sem_scale * e_main, then, if the position carries codes (its
        // row-0 token is a semantic id), the codebook rows in codebook order
        const int nadd = s.tok[32 * m + 20] ? a.ncb : 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = a.sem_scale * WQuad<WT>::get(ev[j][0], e);
        // (a masked row adds exactly 0; the mask differs between the rows of
        // a batch, so no lane-dependent loop bound)
#pragma unroll
        for (int t = 1; t < NT; ++t) {
          const bool add = t <= nadd;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] += add ? WQuad<WT>::get(ev[j][t], e) : 0.0f;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = TAGGED ? tag_val(t[4 * j + e]) : xv[j][e];
        if (MODE == 2) {
          v[0] += from_fx(a0[j][0]); v[1] += from_fx(a0[j][1]);
          v[2] += from_fx(a1[j][0]); v[3] += from_fx(a1[j][1]);
        }
      }
      if (cu < nq) {
        float t = r ? ss1 : ss0;
#pragma unroll
        for (int e = 0; e < 4; ++e) t = fmaf(v[e], v[e], t);
        if (r) ss1 = t; else ss0 = t;
        if (MODE == 0 && blockIdx.x == 0)
#pragma unroll
          for (int e = 0; e < 4; ++e) st_coh(a.x0 + (size_t)m * a.dim + 4 * c + e, v[e]);
        v4f o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = v[e] * WQuad<WT>::get(wv[j], e);
        *reinterpret_cast<v4f*>(s.act + (size_t)r * a.kmax + phys<WT>(4 * c, a.dim)) = o;
      }
    }
  };
  batch(0, hook);
  for (int base = NTHREADS * NS; base < nq; base += NTHREADS * NS) batch(base, NoHook{});
  store_ss(s.small, Mr, ss0, ss1);
}

template <typename WT>
__device__ __forceinline__ void slow_qkv(const SlowArgs& a, const SlowLds& s, int l, Plan& pl) {
  const int r0 = pl.r0, r1 = pl.r1;
  u32x4 slot[RING];
  const auto pro = [&]() __attribute__((always_inline)) { gemv_prologue(pl, slot); };
  const WT* nw = reinterpret_cast<const WT*>(a.L[l].attn_norm);
  const int M = a.M;
  if (l == 0) slow_stage<WT, 0, false>(a, s, l, 0, M, nw, pro);
  else slow_stage<WT, 1, true>(a, s, l, 0, M, nw, pro);
  zero_lds(s.red, (r1 - r0) * NWAVE * MMAX);
  __syncthreads();
  mark(a, s.flag[1], 2);
  gemv_body<WT>(pl, slot, s.act, a.kmax, M, s.red);
  __syncthreads();
  mark(a, s.flag[1], 3);
  u64* out = a.qkv + (size_t)l * a.qkv_slot;
  for (int i = tidx(); i < (r1 - r0) * M; i += NTHREADS) {
    const int r = i / M, m = i - r * M;
    st_tagged(out + (size_t)m * a.qkv_dim + r0 + r, red_sum(s.red, r, m) / norm_den(s.small, m, a.dim, a.eps),
              slow_tag(a));
  }
}

// Attention of one block over positions [p0, p1) of its KV group, any
// head_dim / cache type: lane pairs of head dims, one wave reduction per
// (position, head).  Leaves each wave's (output, max, sum) per head in s.ow.
template <typename WT>
__device__ __forceinline__ void attn_lanes(const SlowArgs& a, const SlowLds& s, const WT* kvg, int p0, int p1,
                                           int mq) {
  using KV = KVElem<WT>;
  const int gh = a.gheads, hd = a.hd, rs = (gh + 2) * hd;
  const int wave = tidx() >> 6, lane = tidx() & 63;
  const float* qrow = s.q + (size_t)mq * rs;     // query position n_past + mq
  const bool own = 2 * lane < hd;
  const int lp = own ? lane : 0;
  float qx[GH_MAX][2], m[GH_MAX], ls[GH_MAX], o0[GH_MAX], o1[GH_MAX];
#pragma unroll
  for (int hh = 0; hh < GH_MAX; ++hh) {
    const int h = min(hh, gh - 1);
    qx[hh][0] = own ? qrow[h * hd + 2 * lp] : 0.0f;
    qx[hh][1] = own ? qrow[h * hd + 2 * lp + 1] : 0.0f;
    m[hh] = -INFINITY;
    ls[hh] = 0.0f;
    o0[hh] = 0.0f;
    o1[hh] = 0.0f;
  }
  const float scale = 1.0f / sqrtf((float)hd);
  for (int base = p0 + wave; base < p1; base += NWAVE * SPPW) {
    typename KV::pair kr[SPPW], vr[SPPW];
#pragma unroll
    for (int i = 0; i < SPPW; ++i) {
      const int j = base + NWAVE * i;
      const int jc = j < p1 ? j : p0;     // past the chunk: re-read its first row (in bounds)
      const WT* row = kvg + (size_t)jc * 2 * hd + 2 * lp;
      kr[i] = KV::load(row);
      vr[i] = KV::load(row + hd);
    }
    float kx[SPPW][2], vx[SPPW][2];
#pragma unroll
    for (int i = 0; i < SPPW; ++i) {
      // the launch's new positions come from LDS; a position past the chunk
      // or after the query reads as zeros, so whatever the cache holds past
      // n_past never enters the sums
      const int j = base + NWAVE * i, mm = j - a.n_past;
      const bool nw = mm >= 0 && mm < a.M, live = j < p1 && j <= a.n_past + mq;
      const float* kn = s.q + (size_t)min(max(mm, 0), a.M - 1) * rs + (size_t)gh * hd;
      const float* vn = kn + hd;
      kx[i][0] = !live ? 0.0f : nw ? kn[2 * lp] : KV::lo(kr[i]);
      kx[i][1] = !live ? 0.0f : nw ? kn[2 * lp + 1] : KV::hi(kr[i]);
      vx[i][0] = !live ? 0.0f : nw ? vn[2 * lp] : KV::lo(vr[i]);
      vx[i][1] = !live ? 0.0f : nw ? vn[2 * lp + 1] : KV::hi(vr[i]);
    }
#pragma unroll
    for (int hh = 0; hh < GH_MAX; ++hh) {
      if (hh >= gh) break;
      float sc[SPPW];
      float mb = -INFINITY;
#pragma unroll
      for (int i = 0; i < SPPW; ++i) {
        float part = fmaf(qx[hh][0], kx[i][0], qx[hh][1] * kx[i][1]);
        part = wave_sum(own ? part : 0.0f);
        const int j = base + NWAVE * i;
        sc[i] = (j < p1 && j <= a.n_past + mq) ? part * scale : -INFINITY;
        mb = fmaxf(mb, sc[i]);
      }
      const float mn = fmaxf(m[hh], mb);
      if (mn == -INFINITY) continue;
      const float r = expf(m[hh] - mn);   // 0 while m is -inf
      float l_ = ls[hh] * r, a0 = o0[hh] * r, a1 = o1[hh] * r;
#pragma unroll
      for (int i = 0; i < SPPW; ++i) {
        const float e = expf(sc[i] - mn);   // 0 past the chunk
        l_ += e;
        a0 = fmaf(e, vx[i][0], a0);
        a1 = fmaf(e, vx[i][1], a1);
      }
      m[hh] = mn;
      ls[hh] = l_;
      o0[hh] = a0;
      o1[hh] = a1;
    }
  }
  // per-wave partials
  const int ws = hd + 2;
#pragma unroll
  for (int hh = 0; hh < GH_MAX; ++hh) {
    if (hh >= gh) break;
    float* w = s.ow + ((size_t)wave * gh + hh) * ws;
    if (own) { w[2 * lane] = o0[hh]; w[2 * lane + 1] = o1[hh]; }
    if (lane == 0) { w[hd] = m[hh]; w[hd + 1] = ls[hh]; }
  }
}

// The measured shape's attention: bf16 cache, head_dim 128, four query heads
// per KV group.  A 256-byte key (or value) row is 16 lanes x 16 bytes, so one
// wave load instruction covers four positions; a score is one 16-lane row
// reduction.  Each lane keeps the online-softmax state of its row's
// positions for its 8 head dims; the four rows of a wave are added at the
// end.  Leaves each wave's (output, max, sum) per head in s.ow.
template <typename WT>
__device__ __forceinline__ void attn_rows16(const SlowArgs& a, const SlowLds& s, const WT* kvg, int p0, int p1,
                                            int mq) {
  constexpr int NI = 3;      // load instructions (4 positions each) per wave per batch
  constexpr int GH = 4, HD = 128, RS = (GH + 2) * HD;
  const int wave = tidx() >> 6, lane = tidx() & 63;
  const int r = lane >> 4, sg = lane & 15;     // position row of the instruction, dims 8sg..8sg+7
  const float* qrow = s.q + (size_t)mq * RS;   // query position n_past + mq
  const int jq = a.n_past + mq;
  float qv[GH][8], m[GH], ls[GH], o[GH][8];
#pragma unroll
  for (int hh = 0; hh < GH; ++hh) {
    const float4 q0 = *reinterpret_cast<const float4*>(qrow + hh * HD + 8 * sg);
    const float4 q1 = *reinterpret_cast<const float4*>(qrow + hh * HD + 8 * sg + 4);
    qv[hh][0] = q0.x; qv[hh][1] = q0.y; qv[hh][2] = q0.z; qv[hh][3] = q0.w;
    qv[hh][4] = q1.x; qv[hh][5] = q1.y; qv[hh][6] = q1.z; qv[hh][7] = q1.w;
    m[hh] = -INFINITY;
    ls[hh] = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) o[hh][k] = 0.0f;
  }
  const float scale = 1.0f / sqrtf((float)HD);
  for (int b0 = p0; b0 < p1; b0 += NWAVE * NI * 4) {
    u32x4 kr[NI], vr[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int j = b0 + (i * NWAVE + wave) * 4 + r;
      const int jc = j < p1 ? j : p0;     // past the chunk: re-read its first row (in bounds)
      const WT* row = kvg + (size_t)jc * 2 * HD + 8 * sg;
      kr[i] = *reinterpret_cast<const u32x4*>(row);
      vr[i] = *reinterpret_cast<const u32x4*>(row + HD);
    }
    float kx[NI][8], vx[NI][8], sc[NI][GH];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      // the launch's new positions from LDS; positions past the chunk or
      // after the query read as zeros
      const int j = b0 + (i * NWAVE + wave) * 4 + r, mm = j - a.n_past;
      const bool nw = mm >= 0 && mm < a.M, live = j < p1 && j <= jq;
      const float* kn = s.q + (size_t)min(max(mm, 0), a.M - 1) * RS + GH * HD;
      const float* vn = kn + HD;
      float kf[8], vf[8];
      WTraits<WT>::unpack(make_uint4(kr[i].x, kr[i].y, kr[i].z, kr[i].w), kf);
      WTraits<WT>::unpack(make_uint4(vr[i].x, vr[i].y, vr[i].z, vr[i].w), vf);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        kx[i][k] = !live ? 0.0f : nw ? kn[8 * sg + k] : kf[k];
        vx[i][k] = !live ? 0.0f : nw ? vn[8 * sg + k] : vf[k];
      }
#pragma unroll
      for (int hh = 0; hh < GH; ++hh) {
        float part = qv[hh][0] * kx[i][0];
#pragma unroll
        for (int k = 1; k < 8; ++k) part = fmaf(qv[hh][k], kx[i][k], part);
        part = row16_sum(part);
        sc[i][hh] = live ? part * scale : -INFINITY;
      }
    }
#pragma unroll
    for (int hh = 0; hh < GH; ++hh) {
      float mb = sc[0][hh];
#pragma unroll
      for (int i = 1; i < NI; ++i) mb = fmaxf(mb, sc[i][hh]);
      mb = fmaxf(fmaxf(readlane_f(mb, 0), readlane_f(mb, 16)), fmaxf(readlane_f(mb, 32), readlane_f(mb, 48)));
      const float mn = fmaxf(m[hh], mb);
      if (mn == -INFINITY) continue;
      const float rs = expf(m[hh] - mn);   // 0 while m is -inf
      ls[hh] *= rs;
#pragma unroll
      for (int k = 0; k < 8; ++k) o[hh][k] *= rs;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const float e = expf(sc[i][hh] - mn);   // 0 past the chunk
        ls[hh] += e;
#pragma unroll
        for (int k = 0; k < 8; ++k) o[hh][k] = fmaf(e, vx[i][k], o[hh][k]);
      }
      m[hh] = mn;
    }
  }
  // add the four position rows of the wave
#pragma unroll
  for (int hh = 0; hh < GH; ++hh) {
    ls[hh] += xor_lane_f<16>(ls[hh], lane);
    ls[hh] += xor_lane_f<32>(ls[hh], lane);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      o[hh][k] += xor_lane_f<16>(o[hh][k], lane);
      o[hh][k] += xor_lane_f<32>(o[hh][k], lane);
    }
  }
  const int ws = HD + 2;
  if (r == 0) {
#pragma unroll
    for (int hh = 0; hh < GH; ++hh) {
      float* w = s.ow + ((size_t)wave * GH + hh) * ws;
#pragma unroll
      for (int k = 0; k < 8; ++k) w[8 * sg + k] = o[hh][k];
      if (sg == 0) { w[HD] = m[hh]; w[HD + 1] = ls[hh]; }
    }
  }
}

template <typename WT>
__device__ __forceinline__ void slow_attn(const SlowArgs& a, const SlowLds& s, int l) {
  using KV = KVElem<WT>;
  const int G = a.n_kv, gh = a.gheads, hd = a.hd, H = a.n_head;
  const int g = blockIdx.x % G, c = blockIdx.x / G;
  if (c >= a.nchunk) return;
  const int wave = tidx() >> 6, lane = tidx() & 63;
  const int M = a.M;
  const int N = a.n_past + M;                     // positions 0 .. n_past + M - 1
  const int p0 = (int)(((long long)N * c) / a.nchunk), p1 = (int)(((long long)N * (c + 1)) / a.nchunk);
  const u64* qkv = a.qkv + (size_t)l * a.qkv_slot;
  const int rs = (gh + 2) * hd;
  // per new position: the group's query heads, its new key and value (the
  // QKV phase's tagged outputs, loaded together and waited on); and the q/k
  // norm weights
  {
    constexpr int NI = 3;
    const int n = M * rs;
    auto at = [&](int i) __attribute__((always_inline)) {
      i = min(i, n - 1);
      const int m = i / rs, v = (i - m * rs) / hd, d = i - m * rs - v * hd;
      const int src = v < gh ? (g * gh + v) * hd : (v == gh ? (H + g) * hd : (H + G + g) * hd);
      return qkv + (size_t)m * a.qkv_dim + src + d;
    };
    for (int base = 0; base < n; base += NI * NTHREADS) {
      u64 t[NI];
#pragma unroll
      for (int j = 0; j < NI; ++j) t[j] = ld_tagged(at(base + j * NTHREADS + tidx()));
      tag_wait(slow_tw(a, s), t, [&](int j) __attribute__((always_inline)) { return at(base + j * NTHREADS + tidx()); });
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int i = base + j * NTHREADS + tidx();
        if (i < n) s.q[i] = tag_val(t[j]);
      }
    }
  }
  if (a.has_qkn)
    for (int i = tidx(); i < 2 * hd; i += NTHREADS)
      s.qkn[i] = WTraits<WT>::one(reinterpret_cast<const WT*>(i < hd ? a.L[l].q_norm : a.L[l].k_norm), i % hd);
  __syncthreads();
  for (int v = wave; v < M * (gh + 1); v += NWAVE) {
    const int m = v / (gh + 1), vv = v - m * (gh + 1);
    head_norm_rope(s.q + (size_t)m * rs + (size_t)vv * hd, hd, vv < gh ? s.qkn : s.qkn + hd, a.has_qkn, a.eps,
                   s.rope1 + (size_t)m * hd, 1, 0);
  }
  __syncthreads();
  mark(a, s.flag[1], 6);
  for (int d = tidx(); d < M * 2 * hd; d += NTHREADS) {   // new keys and values in the cache's precision
    const int m = d / (2 * hd);
    float* kv2 = s.q + (size_t)m * rs + (size_t)gh * hd;
    kv2[d - m * 2 * hd] = KV::round(kv2[d - m * 2 * hd]);
  }
  __syncthreads();

  const WT* kvg = reinterpret_cast<const WT*>(a.kv) + (size_t)(l * G + g) * a.max_ctx * 2 * hd;
  const int ws = hd + 2;
  for (int mq = 0; mq < M; ++mq) {
    if (sizeof(WT) == 2 && hd == 128 && gh == 4) attn_rows16<WT>(a, s, kvg, p0, p1, mq);
    else attn_lanes<WT>(a, s, kvg, p0, p1, mq);
    mark(a, s.flag[1], 7);
    __syncthreads();
    const size_t pc = ((size_t)g * a.nchunk + c) * MMAX + mq;   // this chunk's partial of query mq
    float* po = a.po + (size_t)l * a.po_slot + pc * gh * hd;
    float* pml = a.pml + (size_t)l * a.pml_slot + pc * gh * 2;
    for (int t = tidx(); t < gh * hd; t += NTHREADS) {
      const int hh = t / hd, d = t - hh * hd;
      float Mx = -INFINITY;
      for (int w = 0; w < NWAVE; ++w) Mx = fmaxf(Mx, s.ow[((size_t)w * gh + hh) * ws + hd]);
      float O = 0.0f, Ls = 0.0f;
      if (Mx != -INFINITY) {
        for (int w = 0; w < NWAVE; ++w) {
          const float* ww = s.ow + ((size_t)w * gh + hh) * ws;
          const float f = expf(ww[hd] - Mx);   // 0 for a wave without positions
          O = fmaf(f, ww[d], O);
          Ls = fmaf(f, ww[hd + 1], Ls);
        }
      }
      st_coh(po + t, O);
      if (d == 0) {
        st_coh(pml + 2 * hh, Mx);
        st_coh(pml + 2 * hh + 1, Ls);
      }
    }
    if (mq + 1 < M) __syncthreads();   // s.ow is rewritten by the next query's pass
  }
  // the new keys and values into the cache, each by the block whose chunk
  // holds its position
  for (int mm = 0; mm < M; ++mm) {
    const int pos = a.n_past + mm;
    if (pos < p0 || pos >= p1) continue;
    WT* row = reinterpret_cast<WT*>(a.kv) + ((size_t)(l * G + g) * a.max_ctx + pos) * 2 * hd;
    const float* src = s.q + (size_t)mm * rs + (size_t)gh * hd;
    for (int d = tidx(); d < 2 * hd; d += NTHREADS) row[d] = KV::enc(src[d]);
  }
  // One position: the group's last chunk to finish (its partials and every
  // other chunk's stored before the count says so) merges them into the
  // group's tagged attention output; the count is cleared for the next
  // launch.  Two positions: every wo block merges them itself, after a grid
  // sync (one block merging both positions in turn took longer).
  if (M == 1) {
    int* cnt = a.acnt + ((size_t)l * G + g) * 64;
    wait_vmem();
    __syncthreads();
    if (tidx() == 0)
      s.flag[5] = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.nchunk - 1;
    __syncthreads();
    if (s.flag[5]) {
      const u32 tag = slow_tag(a);
      u64* att = a.att + (size_t)l * a.att_slot + (size_t)g * a.gw;
      slow_merge<WT, true>(a, s, l, g, [&](int mq, int col, float v) __attribute__((always_inline)) {
        st_tagged(att + (size_t)mq * a.attn_dim + col, v, tag);
      }, NoHook{});
      if (tidx() == 0) st_coh(cnt, 0);
    }
  }
}

// Merge KV group g's chunk partials of every head (log-sum-exp weights)
// into its attention output: put(mq, column, value) for each of the group's
// gw columns and each position.  A thread takes 4 consecutive output
// elements (two 8-byte loads per chunk) of the chunks cs, cs + S, ...; the S
// subsets of a quad then meet in LDS.  COH: coherent loads (the partials'
// writers are known done only through the group's count); otherwise a grid
// sync came between, and ordinary loads may hit the L2.  hook() runs once,
// right after the first batch of loads is issued.
template <typename WT, bool COH, typename Put, typename Hook>
__device__ __forceinline__ void slow_merge(const SlowArgs& a, const SlowLds& s, int l, int g, const Put& put,
                                           const Hook& hook) {
  const int gh = a.gheads, hd = a.hd, nc = a.nchunk, n = gh * hd;
  const int M = a.M;
  const float* pml0 = a.pml + (size_t)l * a.pml_slot + (size_t)g * nc * MMAX * gh * 2;
  const float* po0 = a.po + (size_t)l * a.po_slot + (size_t)g * nc * MMAX * gh * hd;
  const int nq = n >> 2;                          // hd % 8 == 0
  const int S = max(1, NTHREADS / nq);
  const int iters = S > 1 ? 1 : (nq + NTHREADS - 1) / NTHREADS;
  constexpr int CB = 8;
  for (int mq = 0; mq < M; ++mq) {
  // chunk cc's partial of query mq: pml0 + (cc * MMAX + mq) * gh * 2, po0 + (cc * MMAX + mq) * n
  const float* pml = pml0 + (size_t)mq * gh * 2;
  const float* po = po0 + (size_t)mq * n;
  if (mq > 0) __syncthreads();   // s.mrg of the previous query is read
  for (int it = 0; it < iters; ++it) {
    const int t = tidx();
    const int q = S > 1 ? t % nq : it * NTHREADS + t;
    const int cs = S > 1 ? t / nq : 0;
    const bool live = S > 1 ? cs < S : q < nq;
    const int qq = min(q, nq - 1), hh = (4 * qq) / hd;
    float M = -INFINITY, Ls = 0.0f;
    v4f O = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int c0 = cs; c0 < nc + S * CB; c0 += S * CB) {
      if (c0 >= nc && !(it == 0 && c0 == cs)) break;
      u64 ml[CB], o01[CB], o23[CB];
#pragma unroll
      for (int j = 0; j < CB; ++j) {
        const int cc = min(c0 + j * S, nc - 1);
        const float* mp = pml + ((size_t)cc * MMAX * gh + hh) * 2;
        const float* op = po + (size_t)cc * MMAX * n + 4 * qq;
        ml[j] = COH ? ld_coh64(mp) : ld64(mp);
        o01[j] = COH ? ld_coh64(op) : ld64(op);
        o23[j] = COH ? ld_coh64(op + 2) : ld64(op + 2);
      }
      if (mq == 0 && it == 0 && c0 == cs) hook();
      float mb = -INFINITY;
#pragma unroll
      for (int j = 0; j < CB; ++j)
        if (c0 + j * S < nc) mb = fmaxf(mb, lo_f32(ml[j]));
      const float mn = fmaxf(M, mb);
      if (mn == -INFINITY) continue;
      const float rs = expf(M - mn);
      Ls *= rs;
      O *= rs;
#pragma unroll
      for (int j = 0; j < CB; ++j) {
        if (c0 + j * S < nc) {
          const float f = expf(lo_f32(ml[j]) - mn);   // 0 for an empty chunk
          Ls = fmaf(f, hi_f32(ml[j]), Ls);
          const v4f ov = {lo_f32(o01[j]), hi_f32(o01[j]), lo_f32(o23[j]), hi_f32(o23[j])};
          O += f * ov;
        }
      }
      M = mn;
    }
    if (S > 1) {
      if (live) {
        float* w = s.mrg + (size_t)t * 6;
        w[0] = M; w[1] = Ls; w[2] = O[0]; w[3] = O[1]; w[4] = O[2]; w[5] = O[3];
      }
    } else if (live) {
#pragma unroll
      for (int e = 0; e < 4; ++e) put(mq, 4 * qq + e, O[e] / Ls);
    }
  }
  if (S > 1) {
    __syncthreads();
    for (int q = tidx(); q < nq; q += NTHREADS) {
      float M = -INFINITY;
      for (int j = 0; j < S; ++j) M = fmaxf(M, s.mrg[(size_t)(j * nq + q) * 6]);
      float Ls = 0.0f, O[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      for (int j = 0; j < S; ++j) {
        const float* w = s.mrg + (size_t)(j * nq + q) * 6;
        const float f = expf(w[0] - M);              // 0 for a subset without positions
        Ls = fmaf(f, w[1], Ls);
#pragma unroll
        for (int e = 0; e < 4; ++e) O[e] = fmaf(f, w[2 + e], O[e]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) put(mq, 4 * q + e, O[e] / Ls);
    }
  }
  }
}

template <typename WT>
__device__ __forceinline__ void slow_wo(const SlowArgs& a, const SlowLds& s, int l, Plan& pl) {
  const int g = pl.g, r0 = pl.r0, r1 = pl.r1;
  zero_lds(s.red, (r1 - r0) * NWAVE * MMAX);
  u32x4 slot[RING];
  const auto pro = [&]() __attribute__((always_inline)) { gemv_prologue(pl, slot); };
  const int M = a.M;
  // the group's attention output into LDS, GEMV layout over its gw columns:
  // one position waits on the merged output (tagged); two merge the
  // partials here
  if (M == 1) {
    const u64* att = a.att + (size_t)l * a.att_slot + (size_t)g * a.gw;
    stage_tagged<WT, 1>(slow_tw(a, s), s.act, att, a.gw, pro);
  } else {
    slow_merge<WT, false>(a, s, l, g, [&](int mq, int col, float v) __attribute__((always_inline)) {
      s.act[(size_t)mq * a.kmax + phys<WT>(col, a.gw)] = v;
    }, pro);
  }
  __syncthreads();
  mark(a, s.flag[1], 2);
  gemv_body<WT>(pl, slot, s.act, a.kmax, M, s.red);
  __syncthreads();
  mark(a, s.flag[1], 3);
  long long* acc = a.acc + (size_t)l * a.acc_slot;
  for (int i = tidx(); i < (r1 - r0) * M; i += NTHREADS) {
    const int r = i / M, m = i - r * M;
    atomic_add_coh(acc + (size_t)m * a.dim + r0 + r, to_fx(red_sum(s.red, r, m)));
  }
}

template <typename WT>
__device__ __forceinline__ void slow_up(const SlowArgs& a, const SlowLds& s, int l, Plan& pl) {
  const int r0 = pl.r0, r1 = pl.r1, nr = r1 - r0;
  u32x4 slot[RING];
  const auto pro = [&]() __attribute__((always_inline)) { gemv_prologue(pl, slot); };
  const int M = a.M;
  if (l == 0) slow_stage<WT, 2, false>(a, s, l, 0, M, reinterpret_cast<const WT*>(a.L[l].ffn_norm), pro);
  else slow_stage<WT, 2, true>(a, s, l, 0, M, reinterpret_cast<const WT*>(a.L[l].ffn_norm), pro);
  zero_lds(s.red, 2 * nr * NWAVE * MMAX);
  __syncthreads();
  mark(a, s.flag[1], 2);
  gemv_body<WT>(pl, slot, s.act, a.kmax, M, s.red);   // rows [0, nr): w1, [nr, 2nr): w3
  __syncthreads();
  mark(a, s.flag[1], 3);
  u64* out = a.g + (size_t)l * a.g_slot;
  for (int i = tidx(); i < nr * M; i += NTHREADS) {
    const int r = i / M, m = i - r * M;
    const float den = norm_den(s.small, m, a.dim, a.eps);
    st_tagged(out + (size_t)m * a.ffn + r0 + r, silu(red_sum(s.red, r, m) / den) * (red_sum(s.red, nr + r, m) / den),
              slow_tag(a));
  }
}

template <typename WT>
__device__ __forceinline__ void slow_down(const SlowArgs& a, const SlowLds& s, int l, Plan& pl) {
  const int r0 = pl.r0, r1 = pl.r1;
  u32x4 slot[RING];
  const auto pro = [&]() __attribute__((always_inline)) { gemv_prologue(pl, slot); };
  const int M = a.M;
  stage_tagged<WT, 5>(slow_tw(a, s), s.act, a.g + (size_t)l * a.g_slot, a.ffn, pro);
  for (int m = 1; m < M; ++m)
    stage_tagged<WT, 5>(slow_tw(a, s), s.act + (size_t)m * a.kmax, a.g + (size_t)l * a.g_slot + (size_t)m * a.ffn,
                        a.ffn, NoHook{});
  zero_lds(s.red, (r1 - r0) * NWAVE * MMAX);
  __syncthreads();
  mark(a, s.flag[1], 2);
  gemv_body<WT>(pl, slot, s.act, a.kmax, M, s.red);
  __syncthreads();
  mark(a, s.flag[1], 3);
  u64* xo = a.x + (size_t)l * a.x_slot;
  long long* acc = a.acc + (size_t)l * a.acc_slot;
  for (int i = tidx(); i < (r1 - r0) * M; i += NTHREADS) {
    const int r = i / M, m = i - r * M;
    const size_t k = (size_t)m * a.dim + r0 + r;
    // the layer input (its tagged value is current since this layer's QKV phase)
    const float xin = l == 0 ? a.x0[k] : tag_val(ld_coh64(slow_in_tag(a, l) + k));
    const float xm = xin + from_fx(acc[k]);
    st_tagged(xo + k, xm + red_sum(s.red, r, m), slow_tag(a));
    st_coh(acc + k, 0ll);   // ready for the next launch
  }
}

template <typename WT>
__device__ __forceinline__ void slow_head(const SlowArgs& a, const SlowLds& s, Plan& pl) {
  const int r0 = pl.r0, r1 = pl.r1;
  u32x4 slot[RING];
  const auto pro = [&]() __attribute__((always_inline)) { gemv_prologue(pl, slot); };
  // the final norm reads the last layer's output: the same staging as a
  // layer input one past the last layer
  if (slow_in_tagged(a, a.n_layer))   // the last position
    slow_stage<WT, 1, true>(a, s, a.n_layer, a.M - 1, 1, reinterpret_cast<const WT*>(a.norm), pro);
  else
    slow_stage<WT, 1, false>(a, s, a.n_layer, a.M - 1, 1, reinterpret_cast<const WT*>(a.norm), pro);
  zero_lds(s.red, (r1 - r0) * NWAVE * MMAX);
  __syncthreads();
  mark(a, s.flag[1], 2);
  gemv_body<WT>(pl, slot, s.act, a.kmax, 1, s.red);
  __syncthreads();
  mark(a, s.flag[1], 3);
  const float den = norm_den(s.small, 0, a.dim, a.eps);
  for (int r = tidx(); r < r1 - r0; r += NTHREADS) {
    const float v = red_sum(s.red, r, 0) / den;
    st_tagged(a.logits + r0 + r, v, slow_tag(a));
    if (a.logits_out) a.logits_out[r0 + r] = v;
  }
  // hidden = RMSNorm(x, norm): the normalised state handed to Fast-AR
  if (blockIdx.x == 0)
    for (int k = tidx(); k < a.dim; k += NTHREADS) a.hidden_out[k] = s.act[phys<WT>(k, a.dim)] / den;
}

// Block 0, after the head: the main-token draw (its loads wait on the
// logits' tags), the repetition check against the window, the window update
// (main-loop page, sections 5 and 6).  Nothing is written if a tag wait gave
// up.
__device__ __forceinline__ void slow_draw(const SlowArgs& a, const SlowLds& s) {
  const SampScratch sc{s.cval, s.cidx, reinterpret_cast<int*>(s.mark)};
  const TaggedLogits lg{slow_tw(a, s), a.logits};
  const int i1 = sample_from(lg, a.n_allowed, a.temp[0], a.top_p[0], a.top_k[0], a.u[0], sc);
  if (tidx() == 0) {
    const int tok = slow_token(a, min(max(i1, 0), a.n_allowed - 1));
    const int cnt = min(max(a.window[0], 0), RAS_WIN);
    bool rep = false;
    for (int j = 0; j < cnt; ++j) rep |= a.window[1 + j] == tok;
    s.tok[16] = tok;
    s.tok[17] = (rep && tok >= a.sem_begin && tok < a.sem_begin + a.nsem) ? 1 : 0;
  }
  __syncthreads();
  if (s.flag[4]) return;
  int tok = s.tok[16];
  if (s.tok[17]) {
    const int i2 = sample_from(lg, a.n_allowed, 1.0f, 0.9f, a.top_k[0], a.u[1], sc);
    if (tidx() == 0) s.tok[16] = slow_token(a, min(max(i2, 0), a.n_allowed - 1));
    __syncthreads();
    if (s.flag[4]) return;
    tok = s.tok[16];
  }
  if (tidx() == 0) {
    a.main_out[0] = tok;
    a.sem_out[0] = min(max(tok - a.sem_begin, 0), a.cbs - 1);
    int cnt = min(max(a.window[0], 0), RAS_WIN);
    if (cnt == RAS_WIN) {
      for (int j = 0; j + 1 < RAS_WIN; ++j) a.window[1 + j] = a.window[2 + j];
      a.window[RAS_WIN] = tok;
    } else {
      a.window[1 + cnt] = tok;
      ++cnt;
    }
    a.window[0] = cnt;
  }
}

// MM: positions per launch (1 for decode, 2 for prefill pairs), fixed at
// compile time so that the one-position kernel carries no per-row loops.
template <typename WT, int MM>
__global__ void __launch_bounds__(NTHREADS) slow_kernel(SlowArgs args) {
  SlowArgs a = args;
  a.M = MM;
  extern __shared__ float lds_base[];
  const SlowLds s = slow_carve(lds_base, a);
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  u32 epoch = a.epoch0;
  if (tidx() == 0) s.flag[4] = 0;
  {
    const int m = tidx() >> 5, t = tidx() & 31;   // position m's row-0 token (t = 0) and codes
    if (m < a.M && t <= a.ncb) {
      const int* mt = m ? a.main1 : a.prev_main;
      const int* ct = m ? a.codes1 : a.prev_codes;
      const int v = t == 0 ? min(max(mt[0], 0), a.vocab - 1) : min(max(ct[t - 1], 0), a.cbs - 1);
      s.tok[32 * m + t] = v;
      if (t == 0) s.tok[32 * m + 20] = (v >= a.sem_begin && v < a.sem_begin + a.nsem) ? 1 : 0;
    }
  }
  // cos and sin of positions n_past + m (the same for every layer)
  for (int i = tidx(); i < a.M * a.hd; i += NTHREADS) {
    const int m = i / a.hd, d = i - m * a.hd;
    const int h2 = a.hd >> 1, half = d >= h2 ? 1 : 0;
    s.rope1[i] = a.rope[((size_t)half * a.max_ctx + a.n_past + m) * h2 + (d - half * h2)];
  }
  __syncthreads();
  const int nph = 5 * a.n_layer + (a.do_head ? 1 : 0);
  // A phase's plan (plain integers) is computed before the barrier that
  // precedes the phase.
  // a head-only launch starts at the head phase
  const int ph0 = a.x_head ? 5 * a.n_layer : 0;
  Plan pl = a.x_head ? slow_plan<WT>(a, a.n_layer - 1, SP_HEAD) : slow_plan<WT>(a, 0, SP_QKV);
  bool ok = true;
  for (int ph = ph0; ph < nph; ++ph) {
    const int l = ph / 5;
    const int kind = ph < 5 * a.n_layer ? ph - 5 * l : (int)SP_HEAD;
    if (a.tlog && tidx() == 0) s.flag[1] = ph;
    mark(a, ph, 5);
    switch (kind) {
      case SP_QKV: slow_qkv<WT>(a, s, l, pl); break;
      case SP_ATTN: slow_attn<WT>(a, s, l); break;
      case SP_WO: slow_wo<WT>(a, s, l, pl); break;
      case SP_UP: slow_up<WT>(a, s, l, pl); break;
      case SP_DOWN: slow_down<WT>(a, s, l, pl); break;
      default: slow_head<WT>(a, s, pl); break;
    }
    {
      const int ln = (ph + 1) / 5;
      const int kn = ph + 1 < 5 * a.n_layer ? ph + 1 - 5 * ln : (int)SP_HEAD;
      pl = slow_plan<WT>(a, min(ln, a.n_layer - 1), kn);   // past the last phase: never used
    }
    mark(a, ph, 0);
    if (kind == SP_WO || (kind == SP_ATTN && MM == 2)) {
      // the attention accumulators (and, at two positions, the chunk
      // partials) are read after a grid sync
      if (!grid_sync<SlowArgs, false>(a, epoch, s.flag)) { ok = false; break; }
    } else {
      // the next phase's loads wait on this phase's tagged outputs
      __syncthreads();
    }
    if (s.flag[4]) { ok = false; break; }
    mark(a, ph, 1);
  }
  if (ok && a.do_head && blockIdx.x == 0) slow_draw(a, s);
  // a barrier or tag wait gave up: the step failed (no main token is drawn and the
  // window is left as it was); the attention accumulators and the chunk
  // counts are cleared for the next launch
  launch_exit(a, s.flag, [&]() __attribute__((always_inline)) {
    zero_words64(a.acc, (size_t)a.n_layer * a.acc_slot);
    zero_words32(a.acnt, (size_t)a.n_layer * a.n_kv * 64);
  });
}
