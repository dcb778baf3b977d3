// Batched frame decode: one cooperative launch decodes one frame for up to
// BQ_MAX requests in lockstep, streaming every weight matrix once per decode
// step for all of them.
//
// Per decode step the rows are the requests' new window positions (two per
// request at step 1: positions 0 and 1; one after), M <= 2 * BQ_MAX.  Every
// linear layer is a skinny GEMM Y[M x N] = X[M x K] W^T run on the matrix
// cores: each workgroup owns a range of W's rows (all of K); W (bf16) is the
// MFMA A operand, streamed from HBM with 16-byte loads; X, read from the
// arena by the wave that uses it, is the B operand split into bf16 high and
// low halves (x = hi + lo to about 2^-18 relative; the Slow-AR prefill,
// 36 layers deep, adds a third piece), so that the products keep near
// float32 accuracy; accumulation is float32.  f32 weights use the
// float32 MFMA with float32 X instead.
//
// Phases per step and layer (grid barrier after each):
//   QKV   x_in * attention_norm -> wqkv; the RMS divides the outputs
//   ATTN  one workgroup per (request, KV group): q/k RMSNorm, pair RoPE,
//         causal attention over the request's window (mask offset 0)
//   WO    x_mid = x_in + wo(attn)
//   UP    x_mid * ffn_norm -> w1, w3; g = silu(a1) * a3
//   DOWN  x = x_mid + w2(g)
// then HEAD (fast_norm, untied output) and SAMPLE (workgroup b draws request
// b's code).  ("Fast-AR codebook decoding and the generation main loop",
// sections 2-4.)
//
// Included by s2fast.hip inside its anonymous namespace.

constexpr int BQ_MAX = 64;               // requests per batched launch
constexpr int MP_MAX = 2 * BQ_MAX;       // rows per decode step at most
constexpr int GROUP_ROWS = 32;           // rows of one wave group (two 16-row M-tiles)
constexpr int GM_MAX = 4 * GROUP_ROWS;   // rows of one GEMM pass (up to four wave groups)
constexpr int KCNT_STRIDE = 64;          // ints between K-split counts (each on its own line)
constexpr int XF_BYTES = 128 * 1024;     // LDS for the GEMM partial sums and the attention scratch
constexpr int TMAX = 5;                  // 16-row tiles of W per workgroup and phase
constexpr int RED_TILES = 10;            // tiles x M-tiles the reduction buffer holds

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct BatchArgs {
  int in_dim, dim, n_layer, n_head, n_kv, hd, ffn, V, ncb, ctx_len;
  float eps;
  int has_proj, has_qkn;
  int qkv_dim, attn_dim, gheads, gw;
  const void* proj;
  const void* emb;
  const void* fnorm;
  const void* outw;
  LayerPtr L[S2FAST_MAX_LAYERS];
  const float* rope;        // [2][ctx_len][hd/2]
  const float* qkv0;        // [V][qkv_dim] layer-0 q/k/v of every embedding row (see FrameArgs)
  // each GEMM's weights repacked into one contiguous stream per workgroup
  // (b_pack_kernel), indexed by pk_index(kind, layer)
  const char* pk[2 + 4 * S2FAST_MAX_LAYERS];
  // wo and w2 split over their K columns: ks[kind] workgroups share a row
  // group, each stores its partial sums into its slice of kpart[kind], and
  // the last of them (by the kcnt[kind] count) adds the slices in slice
  // order, writes the phase's output and clears the count for the next
  // frame; ks 1: no split
  // The wqkv phase may split as well; it needs no finalising step: the
  // attention workgroups add the two slices' partial sums of the values
  // they read and divide by the RMS rebuilt from the slices' sums of
  // squares (kss).
  int ks[6];
  float* kpart[6];          // [slot][ks][kslot]
  long long kslot[6];       // elements of one slice: MP_MAX rows of the phase's output width
  int* kcnt[6];             // [slot][P / ks], one count per 256-byte line
  float* kss[6];            // [slot][ks][MP_MAX] sums of squares of a slice's X rows
  int Bq;                   // requests in this launch, 1..BQ_MAX
  const float* hidden;      // [Bq][in_dim]
  const int* sem_code;      // [Bq]
  const float* uniforms;    // [Bq][ncb-1]
  const float* temp;        // [Bq]
  const float* top_p;       // [Bq]
  const int* top_k;         // [Bq]
  const int* forced;        // [Bq][forced_ld] or nullptr
  int* codes_out;           // [Bq][ncb] or nullptr
  float* logits_out;        // [Bq][lo_rows][V] or nullptr
  int nsteps;               // decode steps this launch runs (ncb-1 for a whole frame)
  int forced_ld;            // codes per request in `forced`
  int lo_first, lo_rows;    // logits_out row of step s >= lo_first is s - lo_first
  // arena: every (step, layer) region written once per frame (see FrameArgs)
  float* xin0;              // [BQ_MAX][dim]
  float* x;                 // [slot][MP_MAX][dim] residual after the layer
  float* xmid;              // [slot][MP_MAX][dim] residual after attention
  float* qkv;               // [slot][MP_MAX][qkv_dim]
  float* att;               // [slot][MP_MAX][attn_dim]
  float* g;                 // [slot][MP_MAX][ffn]
  float* logits;            // [step][BQ_MAX][V]
  float* kv;                // [BQ_MAX][n_layer][ctx][n_kv][2][hd]
  int* codes;               // [BQ_MAX][16] sampled codes
  long long x_slot, qkv_slot, att_slot, g_slot, logits_slot;
  u32* flags;
  u32 epoch0;
  u32* err;                 // watchdog words (see Watch)
  Watch watch;
  u32* tlog;
  // Slow-AR prefill launches (prefill = 1): the prompt positions n_past0 ..
  // n_past0 + Bq - 1 are the rows of one step through up to
  // S2FAST_SLOW_MAX_LAYERS layers, whose pointers and packed streams come
  // from device tables
  int prefill;
  int lds_layers;           // layers whose q/k norm weights the LDS holds (n_layer; 1 in prefill)
  const LayerPtr* Lt;       // [n_layer] (prefill)
  const char* const* pkt;   // [2 + 4 n_layer] (prefill)
  int n_past0, max_ctx;
  void* cache;              // the caller's KV cache [n_layer][n_kv][max_ctx][2][hd], weight type
  const int* tokens;        // [Bq][1 + ncb] row-0 token and codes of each position
  float* x0w;               // [Bq][dim] the positions' inputs (hidden reads them)
  const void* cemb;         // codebook embeddings [ncb * cbs][dim]
  int cbs, sem_begin, vocab;
  float sem_scale;
  // the prefill attention on the matrix cores (bf16 caches): work items of
  // pf_qpos positions of one KV group, the cache positions split pf_ps ways
  // (partial results in pf_part, merged in a phase of their own when
  // pf_ps > 1); pf_hdp = head_dim rounded up to whole 32-wide k-steps
  int pf_qpos, pf_nb, pf_ps, pf_hdp;
  float* pf_part;           // [n_kv][pf_nb][pf_ps][64][pf_hdp + 2]: output sums, max, sum
  float* pf_q;              // [Bq][n_head * hd] query vectors after q RMSNorm and RoPE
  int pf_full_last;         // the chunk holds the prompt's last position: the last layer runs in full
};

struct BLds {
  char* xf;      // XF_BYTES: GEMM partial sums; attention scratch
  float* ssp;    // [NWAVE][MP_MAX] per-wave row sums of squares
  float* rms;    // [MP_MAX]
  float* qkn;    // [n_layer][2][hd]
  float* rope;   // [2][ctx][hd/2]
  float* cval;   // [TOPK_MAX]
  int* cidx;     // [TOPK_MAX]
  int* sred;     // [2 * NWAVE * SAMP_TAU]
  int* rcode;    // [MP_MAX] embedding row of each row's layer-0 input (-1: hidden state)
  int* flag;     // [4]
};

// dynamic LDS of a launch whose q/k norm weights of lds_layers layers and
// RoPE table of ctx positions sit in LDS
__host__ __device__ inline size_t b_lds_bytes(int lds_layers, int hd, int ctx) {
  return (size_t)XF_BYTES + sizeof(float) * ((size_t)NWAVE * MP_MAX + MP_MAX + (size_t)lds_layers * 2 * hd + (size_t)ctx * hd +
                                             TOPK_MAX) +
         sizeof(int) * ((size_t)TOPK_MAX + 2 * NWAVE * SAMP_TAU + MP_MAX + 4);
}

__device__ inline BLds b_carve(char* base, const BatchArgs& a) {
  BLds s;
  char* p = base;
  s.xf = p; p += XF_BYTES;
  s.ssp = reinterpret_cast<float*>(p); p += sizeof(float) * NWAVE * MP_MAX;
  s.rms = reinterpret_cast<float*>(p); p += sizeof(float) * MP_MAX;
  s.qkn = reinterpret_cast<float*>(p); p += sizeof(float) * (size_t)a.lds_layers * 2 * a.hd;
  s.rope = reinterpret_cast<float*>(p); p += sizeof(float) * (size_t)a.ctx_len * a.hd;
  s.cval = reinterpret_cast<float*>(p); p += sizeof(float) * TOPK_MAX;
  s.cidx = reinterpret_cast<int*>(p); p += sizeof(int) * TOPK_MAX;
  s.sred = reinterpret_cast<int*>(p); p += sizeof(int) * 2 * NWAVE * SAMP_TAU;
  s.rcode = reinterpret_cast<int*>(p); p += sizeof(int) * MP_MAX;
  s.flag = reinterpret_cast<int*>(p);
  return s;
}

// rows of decode step `step`: request b's positions 0 and 1 are rows b and
// Bq + b at step 1; position `step` is row b afterwards
__device__ __forceinline__ int b_rows(const BatchArgs& a, int step) {
  return (step == 1 && !a.prefill) ? 2 * a.Bq : a.Bq;
}
// layer l's pointers and the packed stream idx (device tables in prefill launches)
__device__ __forceinline__ LayerPtr b_layer(const BatchArgs& a, int l) { return a.prefill ? a.Lt[l] : a.L[l]; }
__device__ __forceinline__ const char* b_pk(const BatchArgs& a, int idx) { return a.prefill ? a.pkt[idx] : a.pk[idx]; }
__device__ __forceinline__ int b_pos(const BatchArgs& a, int step, int m) { return step == 1 ? m / a.Bq : step; }
__device__ __forceinline__ int b_last_row(const BatchArgs& a, int step, int b) { return step == 1 ? a.Bq + b : b; }

__device__ __forceinline__ size_t b_slot(const BatchArgs& a, int step, int l) { return (size_t)(step - 1) * a.n_layer + l; }
__device__ __forceinline__ float* bx(const BatchArgs& a, int step, int l) { return a.x + b_slot(a, step, l) * a.x_slot; }
__device__ __forceinline__ float* bxmid(const BatchArgs& a, int step, int l) { return a.xmid + b_slot(a, step, l) * a.x_slot; }
__device__ __forceinline__ float* bqkv(const BatchArgs& a, int step, int l) { return a.qkv + b_slot(a, step, l) * a.qkv_slot; }
__device__ __forceinline__ float* batt(const BatchArgs& a, int step, int l) { return a.att + b_slot(a, step, l) * a.att_slot; }
__device__ __forceinline__ float* bg(const BatchArgs& a, int step, int l) { return a.g + b_slot(a, step, l) * a.g_slot; }
// slice j of kind's partial sums at (step, layer)
__device__ __forceinline__ float* bkpart(const BatchArgs& a, int kind, int step, int l, int j) {
  return a.kpart[kind] + (b_slot(a, step, l) * a.ks[kind] + j) * a.kslot[kind];
}
__device__ __forceinline__ float* bkss(const BatchArgs& a, int kind, int step, int l, int j) {
  return a.kss[kind] + (b_slot(a, step, l) * a.ks[kind] + j) * MP_MAX;
}
__device__ __forceinline__ float* blogits(const BatchArgs& a, int step) { return a.logits + (size_t)(step - 1) * a.logits_slot; }
__device__ __forceinline__ float* bkv(const BatchArgs& a, int b, int l, int pos, int g) {
  return a.kv + ((((size_t)b * a.n_layer + l) * a.ctx_len + pos) * a.n_kv + g) * 2 * a.hd;
}

// code c_j of request b: the (clamped) semantic code for j = 0, later the
// teacher-forced input or the code sampled at step j
__device__ __forceinline__ int b_code(const BatchArgs& a, int b, int j) {
  int c;
  if (a.forced) c = a.forced[(size_t)b * a.forced_ld + j];
  else if (j == 0) c = a.sem_code[b];
  else c = ld_coh(a.codes + b * 16 + j);   // one line holds codes written at different steps
  return min(max(c, 0), a.V - 1);
}

// ------------------------------------------------------------ skinny GEMM
enum BKind { BK_PROJ = 0, BK_QKV, BK_WO, BK_UP, BK_DOWN, BK_HEAD };

struct GemmDesc {
  const char* pk;      // this workgroup's packed weight stream (b_pack_kernel layout)
  long long kp;        // bytes of one packed row: k-steps * 64
  int R;               // rows (for the SwiGLU phase: w1 rows, then the same w3 rows)
  int K;               // columns (of this workgroup's K slice)
  int k0;              // first column of the slice
  int m0;              // first row of X of this pass
  int M;               // rows of X (<= GM_MAX in a pass)
  int kind, step, l;
  const void* normw;   // RMSNorm weight over K, or nullptr
};

template <typename WT> struct MF;
template <> struct MF<uint16_t> {
  static constexpr int KSZ = 32;      // K per k-step (one 16x16x32 MFMA per X half)
  static constexpr int GE = 8;        // K per lane per k-step
};
template <> struct MF<float> {
  static constexpr int KSZ = 16;      // four 16x16x4 MFMAs
  static constexpr int GE = 4;
};

// Slot of a GEMM's packed stream in BatchArgs::pk.
__host__ __device__ inline int pk_index(int kind, int l) {
  return kind == BK_PROJ ? 0 : (kind == BK_HEAD ? 1 : 2 + 4 * l + (kind - BK_QKV));
}

// Packed weight streams.  Rows are split over the workgroups exactly as the
// GEMM phase splits them (split_rows); the SwiGLU phase's rows are the
// workgroup's w1 rows followed by the same w3 rows.  A workgroup's rows are
// cut into tiles of 16 (the last one may be shorter, rt rows) and each tile
// into k-steps of KSZ columns; the k-step of a tile is rt * 64 contiguous
// bytes, row after row, each row's 64 bytes being the four GE-element pieces
// the MFMA lane groups 0..3 read.  So every weight load of a wave is one
// contiguous run (16 rows x 64 bytes), and a workgroup's whole phase is one
// contiguous stream.  Columns past K are zero.  Workgroup b's stream starts
// at row (or for SwiGLU, 2 x row) r0 of a matrix of k-steps * 64-byte rows.
//
// With a K split S (gridDim.x a multiple of S), workgroup b packs row group
// b / S of gridDim.x / S and the columns [ks Ks, (ks + 1) Ks) of its slice
// ks = b % S, Ks = K / S; the S slices of a row group follow each other, so
// the stream starts at row r0 S + ks nr of a matrix of Ks-column rows.
template <typename WT>
__global__ void __launch_bounds__(256) b_pack_kernel(const WT* wa, const WT* wb, int R, int K, int S, char* dst) {
  constexpr int KSZ = MF<WT>::KSZ, GE = MF<WT>::GE, NG = KSZ / GE;
  const int rg = blockIdx.x / S, ks = blockIdx.x - rg * S;
  int r0, r1;
  split_rows(R, rg, gridDim.x / S, r0, r1);
  const int nr = r1 - r0;
  const int NR = wb ? 2 * nr : nr;
  const int Ks = K / S, c0 = ks * Ks;
  const int KST = (Ks + KSZ - 1) / KSZ;
  const long long kp = (long long)KST * 64;
  char* base = dst + (long long)(wb ? 2 * r0 : r0 * S + ks * nr) * kp;
  const long long n = (long long)NR * KST * NG;
  for (long long idx = threadIdx.x; idx < n; idx += 256) {
    const int i = (int)(idx / (KST * NG));
    const int q = (int)(idx - (long long)i * KST * NG);
    const int st = q / NG, kg = q - st * NG;
    const int c = st * KSZ + kg * GE;
    const WT* src = (wb && i >= nr) ? wb + (long long)(r0 + i - nr) * K : wa + (long long)(r0 + i) * K;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (c < Ks) v = *reinterpret_cast<const uint4*>(src + c0 + c);   // Ks is a multiple of GE
    const int t = i >> 4, ii = i & 15, rt = min(16, NR - 16 * t);
    *reinterpret_cast<uint4*>(base + (long long)16 * t * kp + (long long)st * rt * 64 + ii * 64 + kg * 16) = v;
  }
}

// two floats -> two bf16 (round to nearest even), a in the low half
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32 bf16_pair(float a, float b) {
  const bf16x2 h = __builtin_convertvector(f32x2{a, b}, bf16x2);
  u32 u;
  __builtin_memcpy(&u, &h, 4);
  return u;
}

// GE source values of row m at column k (k a multiple of GE; row and column
// in range).  The loads are unconditional: the phase kind is uniform (scalar
// branches), and at layer 0 the float32 row and the embedding row are both
// read and one is selected, so no load sits behind a per-lane branch.
template <typename WT>
__device__ __forceinline__ void b_fetch(const BatchArgs& a, const BLds& s, const GemmDesc& gd, int m, int k,
                                        float (&v)[8]) {
  constexpr int GE = MF<WT>::GE;
  const float* src;
  switch (gd.kind) {
    case BK_PROJ: src = a.hidden + (size_t)m * a.in_dim; break;
    case BK_QKV:
      if (gd.l > 0) src = bx(a, gd.step, gd.l - 1) + (size_t)m * a.dim;
      else src = a.has_proj ? a.xin0 + (size_t)(m % a.Bq) * a.dim : a.hidden + (size_t)(m % a.Bq) * a.in_dim;
      break;
    case BK_WO: src = batt(a, gd.step, gd.l) + (size_t)m * a.attn_dim; break;
    case BK_UP: src = bxmid(a, gd.step, gd.l) + (size_t)m * a.dim; break;
    case BK_DOWN: src = bg(a, gd.step, gd.l) + (size_t)m * a.ffn; break;
    default: src = bx(a, gd.step, a.n_layer - 1) + (size_t)b_last_row(a, gd.step, m) * a.dim; break;
  }
  const float4 q0 = *reinterpret_cast<const float4*>(src + k);
  v[0] = q0.x; v[1] = q0.y; v[2] = q0.z; v[3] = q0.w;
  if (GE == 8) {
    const float4 q1 = *reinterpret_cast<const float4*>(src + k + 4);
    v[4] = q1.x; v[5] = q1.y; v[6] = q1.z; v[7] = q1.w;
  }
  if (gd.kind == BK_QKV && gd.l == 0) {
    // rows at window positions >= 1 take fast_embeddings[code] instead
    const int c = s.rcode[m];
    const WT* e = reinterpret_cast<const WT*>(a.emb) + (size_t)max(c, 0) * a.dim;
    float ev[8];
    if (GE == 8) {
      const uint4 q = *reinterpret_cast<const uint4*>(e + k);
      ev[0] = __uint_as_float(q.x << 16); ev[1] = __uint_as_float(q.x & 0xFFFF0000u);
      ev[2] = __uint_as_float(q.y << 16); ev[3] = __uint_as_float(q.y & 0xFFFF0000u);
      ev[4] = __uint_as_float(q.z << 16); ev[5] = __uint_as_float(q.z & 0xFFFF0000u);
      ev[6] = __uint_as_float(q.w << 16); ev[7] = __uint_as_float(q.w & 0xFFFF0000u);
    } else {
      const float4 q = *reinterpret_cast<const float4*>(e + k);
      ev[0] = q.x; ev[1] = q.y; ev[2] = q.z; ev[3] = q.w;
    }
#pragma unroll
    for (int t = 0; t < GE; ++t) v[t] = c >= 0 ? ev[t] : v[t];
  }
}

// ------------------------------------------------------------ GEMM core
// Work split: the waves of a wave group split the k-steps (KSZ columns
// each) between them, for every row tile of the workgroup, so each X
// fragment is read and converted by exactly one wave of the group, straight into MFMA B
// operands: no staging in LDS and no barrier inside the phase.  Per k-step a wave loads the
// weight fragment of each row tile (A operand: lane -> row 16 t + lane % 16,
// columns s KSZ + GE (lane / 16) ..) and the X fragment of each M-tile (B
// operand: lane -> row 16 mt + lane % 16, the same columns), applies the
// phase's RMSNorm weight, splits X into bf16 high and low halves (x = hi + lo
// to about 2^-18 relative; a third piece with XS = 3) and accumulates D[t][mt] in float32.  The loads of
// a k-step are issued PD k-steps before it is used (more when a k-step has
// few row tiles; deeper pipelines measured slower).
//
// The two waves that share a SIMD do not progress alike: the first one
// (waves 0..3 of the workgroup) is issued first, and measured 10-25 % faster
// than the second.  A first wave therefore takes a larger share of the
// k-steps (BShare), so the waves of a workgroup finish together.
template <int TT, int MTT> constexpr int bpd() { return TT == 1 ? 4 : (TT == 2 ? 3 : 2); }

template <typename WT, int TT, int MTT>
struct BUnit {
  u32x4 w[TT];
  float x[MTT][8];
  bool ok[MTT];
  uint4 nw;       // the RMSNorm weight of the lane's GE columns (phases with a norm)
};

// A non-temporal 16-byte load of the packed weight stream.  The stream's
// base arrives as a kernel argument, so the compiler already knows it is
// global memory and forms the address from it; an explicit address-space
// cast measured 3 % slower here.
__device__ __forceinline__ void b_load16(u32x4& d, const char* p) {
  d = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Loads of k-step st (past the wave's last k-step: loads of k-step 0, unused)
template <typename WT, int TT, int MTT>
__device__ __forceinline__ void b_load(const BatchArgs& a, const BLds& s, const GemmDesc& gd, int st, int KST,
                                       int lane, BUnit<WT, TT, MTT>& u) {
  constexpr int KSZ = MF<WT>::KSZ, GE = MF<WT>::GE;
  const bool live = st < KST;
  const int col = (live ? st : 0) * KSZ + GE * (lane >> 4);
  const bool colok = col < gd.K;              // past the last column X is zero (weights: column 0)
  const int c = colok ? col : 0;
  // weights from the packed stream: tile t's k-step is rt rows of 64 bytes
  // (lanes past a short tile's rows re-read its last row)
  const int sp = live ? st : 0;
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    const int rt = min(16, gd.R - 16 * t);
    const int i = min(lane & 15, rt - 1);
    b_load16(u.w[t], gd.pk + (long long)16 * t * gd.kp + (long long)sp * rt * 64 + i * 64 + (lane >> 4) * 16);
  }
#pragma unroll
  for (int mt = 0; mt < MTT; ++mt) {
    const int m = 16 * mt + (lane & 15);
    u.ok[mt] = live && colok && m < gd.M;
    b_fetch<WT>(a, s, gd, gd.m0 + (m < gd.M ? m : 0), gd.k0 + c, u.x[mt]);
  }
  // GE norm weights are 16 bytes in either weight format
  if (gd.normw) u.nw = *reinterpret_cast<const uint4*>(reinterpret_cast<const WT*>(gd.normw) + gd.k0 + c);
}

// XS: bf16 pieces of X for bf16 weights (2: x = hi + lo to about 2^-18
// relative; 3: a third piece, to about 2^-27, float32-level)
template <typename WT, int TT, int MTT, int XS>
__device__ __forceinline__ void b_use(const BLds& s, const GemmDesc& gd, int st, int lane, const BUnit<WT, TT, MTT>& u,
                                      f32x4 (&D)[TT][MTT], float (&ss)[MTT]) {
  constexpr int GE = MF<WT>::GE;
  float w[8];
  if (gd.normw) WTraits<WT>::unpack(u.nw, w);   // uniform: the phase's RMSNorm weight
#pragma unroll
  for (int mt = 0; mt < MTT; ++mt) {
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[e] = 0.0f;
      if (e < GE && u.ok[mt]) {
        if (gd.normw) { ss[mt] = fmaf(u.x[mt][e], u.x[mt][e], ss[mt]); x[e] = u.x[mt][e] * w[e]; }
        else x[e] = u.x[mt][e];
      }
    }
    if (GE == 8) {
      u32 h[4], lw[4], l2[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        h[p] = bf16_pair(x[2 * p], x[2 * p + 1]);
        const float r0 = x[2 * p] - __uint_as_float(h[p] << 16), r1 = x[2 * p + 1] - __uint_as_float(h[p] & 0xFFFF0000u);
        lw[p] = bf16_pair(r0, r1);
        if (XS == 3) l2[p] = bf16_pair(r0 - __uint_as_float(lw[p] << 16), r1 - __uint_as_float(lw[p] & 0xFFFF0000u));
      }
      bf16x8 hv, lv, l2v;
      __builtin_memcpy(&hv, h, 16);
      __builtin_memcpy(&lv, lw, 16);
      if (XS == 3) __builtin_memcpy(&l2v, l2, 16);
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        bf16x8 av;
        __builtin_memcpy(&av, &u.w[t], 16);
        D[t][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, hv, D[t][mt], 0, 0, 0);
        D[t][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, lv, D[t][mt], 0, 0, 0);
        if (XS == 3) D[t][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, l2v, D[t][mt], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        const u32x4 q = u.w[t];
        D[t][mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(q.x), x[0], D[t][mt], 0, 0, 0);
        D[t][mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(q.y), x[1], D[t][mt], 0, 0, 0);
        D[t][mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(q.z), x[2], D[t][mt], 0, 0, 0);
        D[t][mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(q.w), x[3], D[t][mt], 0, 0, 0);
      }
    }
  }
}

// One wave's share of a GEMM phase with TT row tiles and MTT M-tiles: its
// range of the k-steps of its wave group's rows (gd.m0.., gd.M <= 32);
// its partial sums go to red[((wave * TT + t) * 2 + mt) * 256 + lane * 4 ..],
// its per-lane sums of squares of X to ssm[mt] (row 16 mt + lane % 16).
// K-steps of wave kw of a group of wpg waves, h = wpg / 2 of them first
// waves of their SIMDs (kw < h).  The k-steps go in rounds of wpg * base +
// h: a round's first wpg * base k-steps are dealt to the waves in turn
// (consecutive k-steps to consecutive waves, the pattern the memory system
// streams best), its last h k-steps one each to the first waves.  So a
// first wave takes base + 1 k-steps a round, a second wave base.
struct BShare {
  int kw, wpg, base, cw, R;
  __device__ __forceinline__ BShare(int KST, int kw_, int wpg_, int base_, int& ns)
      : kw(kw_), wpg(wpg_), base(base_) {
    const int h = wpg >> 1;
    cw = base + (kw < h ? 1 : 0);
    R = wpg * base + h;
    const int nr = KST / R, rem = KST - nr * R;
    int last;   // this wave's k-steps of the partial last round
    if (rem <= wpg * base) last = kw < rem ? (rem - 1 - kw) / wpg + 1 : 0;
    else last = base + (kw < rem - wpg * base ? 1 : 0);
    ns = nr * cw + last;
  }
  // global index of the wave's j-th k-step (j < ns)
  __device__ __forceinline__ int at(int j) const {
    const int r = j / cw, i = j - r * cw;
    return r * R + (i < base ? i * wpg + kw : wpg * base + kw);
  }
};

template <typename WT, int TT, int MTT, int XS>
__device__ __forceinline__ void b_core(const BatchArgs& a, const BLds& s, const GemmDesc& gd, int wave, int kw,
                                       int wpg, int lane, float* red, float (&ssm)[2]) {
  constexpr int KSZ = MF<WT>::KSZ, PD = bpd<TT, MTT>();
  const int KST = (gd.K + KSZ - 1) / KSZ;
  // the SwiGLU phase's first waves measured 25 % faster than the second ones
  // (a first wave takes 5 k-steps to a second's 4), the other phases' about
  // 10 % (9 to 8)
  int ns;
  const BShare sh(KST, kw, wpg, gd.kind == BK_UP ? 4 : 8, ns);
  const auto kstep = [&](int j) __attribute__((always_inline)) { return j < ns ? sh.at(j) : KST; };
  f32x4 D[TT][MTT];
  float ss[MTT];
#pragma unroll
  for (int mt = 0; mt < MTT; ++mt) {
    ss[mt] = 0.0f;
#pragma unroll
    for (int t = 0; t < TT; ++t) D[t][mt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  BUnit<WT, TT, MTT> u[PD];
#pragma unroll
  for (int p = 0; p < PD - 1; ++p) b_load<WT, TT, MTT>(a, s, gd, kstep(p), KST, lane, u[p]);
  for (int i = 0; i < ns; i += PD) {
#pragma unroll
    for (int r = 0; r < PD; ++r) {
      b_load<WT, TT, MTT>(a, s, gd, kstep(i + r + PD - 1), KST, lane, u[(r + PD - 1) % PD]);
      if (i + r < ns) b_use<WT, TT, MTT, XS>(s, gd, kstep(i + r), lane, u[r], D, ss);
    }
  }
#pragma unroll
  for (int mt = 0; mt < MTT; ++mt) {
    ssm[mt] = ss[mt];
#pragma unroll
    for (int t = 0; t < TT; ++t)
      *reinterpret_cast<float4*>(red + (((size_t)wave * TT + t) * 2 + mt) * 256 + lane * 4) =
          make_float4(D[t][mt][0], D[t][mt][1], D[t][mt][2], D[t][mt][3]);
  }
}

// Per-wave partial products of one GEMM phase: row m of the pass belongs to
// wave group g = m / 32 (waves g, g + ng, ...), whose wpg waves' partials
// are summed in wave order.
struct RedView {
  const float* red;
  int T, wpg, ng;
  // the N = wpg partials of element (t, slot ln * 4 + r, M-tile mt) of group
  // g: all N reads issued together, then added in wave order
  template <int N>
  __device__ __forceinline__ float sum_n(int g, int t, int mt, int ln, int r) const {
    float pv[N];
#pragma unroll
    for (int j = 0; j < N; ++j) pv[j] = red[((((size_t)(g + j * ng)) * T + t) * 2 + mt) * 256 + ln * 4 + r];
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < N; ++j) acc += pv[j];
    return acc;
  }
  __device__ __forceinline__ float sum(int v, int m) const {
    // element (v = 16 t + 4 qd + r, row 32 g + 16 mt + j) sits in lane qd * 16 + j, slot r
    const int t = v >> 4, i = v & 15, g = m >> 5, mt = (m >> 4) & 1;
    const int ln = (i >> 2) * 16 + (m & 15), r = i & 3;
    static_assert(NWAVE == 8, "wave groups of 8, 4 or 2 waves");
    if (wpg == 8) return sum_n<8>(g, t, mt, ln, r);
    if (wpg == 4) return sum_n<4>(g, t, mt, ln, r);
    return sum_n<2>(g, t, mt, ln, r);
  }
};

// Run one GEMM phase on this workgroup.  On return (after a barrier) the
// view holds the waves' partial sums and, with a norm weight, rms[m] holds
// sqrt(mean(x_m^2) + eps) over the K columns.
// The pass's rows form up to four wave groups of 32 (1, 2 or 4 groups of
// 8, 4 or 2 waves): each group streams the workgroup's whole weight range
// for its rows, the waves of a group splitting the k-steps.  The groups
// read the same weight fragments at about the same time (one HBM fill
// serves them).
template <typename WT, int XS>
__device__ __forceinline__ RedView b_gemm(const BatchArgs& a, const BLds& s, const GemmDesc& gd) {
  const int tid = tidx();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;   // wave-uniform work split
  const int ng = gd.M <= GROUP_ROWS ? 1 : (gd.M <= 2 * GROUP_ROWS ? 2 : 4);
  const int wpg = NWAVE / ng;
  // group grp = wave % ng: every group holds first and second waves of the SIMDs alike
  const int grp = wave % ng, kw = wave / ng;
  GemmDesc gg = gd;
  gg.m0 = gd.m0 + GROUP_ROWS * grp;
  gg.M = max(0, min(GROUP_ROWS, gd.M - GROUP_ROWS * grp));
  const int MT = gg.M <= 16 ? 1 : 2;
  const int T = gg.M > 0 ? (gd.R + 15) >> 4 : 0;   // a group without rows does nothing
  float* red = reinterpret_cast<float*>(s.xf);
  float ssm[2] = {0.0f, 0.0f};
  mark(a, s.flag[1], 2);
#define B_CORE(TT_)                                                                 \
  case TT_:                                                                         \
    if (MT == 1) b_core<WT, TT_, 1, XS>(a, s, gg, wave, kw, wpg, lane, red, ssm);   \
    else b_core<WT, TT_, 2, XS>(a, s, gg, wave, kw, wpg, lane, red, ssm);           \
    break;
  switch (T) {
    B_CORE(1)
    B_CORE(2)
    B_CORE(3)
    B_CORE(4)
    B_CORE(5)
    default: break;   // no rows in this workgroup
  }
#undef B_CORE
  static_assert(TMAX == 5, "b_gemm dispatches row-tile counts 1..5");
  mark(a, s.flag[1], 3);
  if (gd.normw) {
    // a row's sum of squares: its four lanes (lane % 16 = row) in each wave,
    // then the waves
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      if (mt >= MT || gg.M == 0) break;
      float v = ssm[mt];
      v += xor_lane_f<16>(v, lane);
      v += xor_lane_f<32>(v, lane);
      if (lane < 16) s.ssp[wave * MP_MAX + GROUP_ROWS * grp + 16 * mt + lane] = v;
    }
  }
  __syncthreads();
  if (gd.normw && tid < gd.M) {
    float t2 = 0.0f;
    const int g = tid / GROUP_ROWS;
    for (int j = 0; j < wpg; ++j) t2 += s.ssp[(g + j * ng) * MP_MAX + tid];
    // a K slice keeps its raw sum of squares (the consumer adds the slices')
    s.rms[tid] = a.ks[gd.kind] > 1 ? t2 : sqrtf(t2 / (float)gd.K + a.eps);
  }
  __syncthreads();
  return RedView{red, (gd.R + 15) >> 4, wpg, ng};
}

// ------------------------------------------------------------ phases
template <typename WT>
__device__ __forceinline__ float b_layer0_elem(const BatchArgs& a, const BLds& s, int m, int k) {
  const int c = s.rcode[m];
  if (c < 0) return a.has_proj ? a.xin0[(size_t)(m % a.Bq) * a.dim + k] : a.hidden[(size_t)(m % a.Bq) * a.in_dim + k];
  return WTraits<WT>::one(reinterpret_cast<const WT*>(a.emb) + (size_t)c * a.dim, k);
}

template <typename WT, int XS = 2>
__device__ __forceinline__ void b_phase_gemm(const BatchArgs& a, const BLds& s, int kind, int step, int l) {
  const int P = gridDim.x, blk = blockIdx.x;
  GemmDesc gd;
  gd.kind = kind; gd.step = step; gd.l = l;
  gd.normw = nullptr;
  gd.k0 = 0;
  gd.m0 = 0;
  int r0 = 0, r1 = 0, ks = 0;
  const int S = a.ks[kind];
  const LayerPtr L = b_layer(a, l);
  switch (kind) {
    case BK_PROJ:
      split_rows(a.dim, blk, P, r0, r1);
      gd.K = a.in_dim; gd.M = a.Bq;
      break;
    case BK_QKV:
      ks = blk % S;
      split_rows(a.qkv_dim, blk / S, P / S, r0, r1);
      gd.K = a.dim / S; gd.k0 = ks * gd.K; gd.M = b_rows(a, step);
      gd.normw = L.attn_norm;
      break;
    case BK_WO:
      ks = blk % S;
      split_rows(a.dim, blk / S, P / S, r0, r1);
      gd.K = a.attn_dim / S; gd.k0 = ks * gd.K; gd.M = b_rows(a, step);
      break;
    case BK_UP:
      split_rows(a.ffn, blk, P, r0, r1);
      gd.K = a.dim; gd.M = b_rows(a, step);
      gd.normw = L.ffn_norm;
      break;
    case BK_DOWN:
      ks = blk % S;
      split_rows(a.dim, blk / S, P / S, r0, r1);
      gd.K = a.ffn / S; gd.k0 = ks * gd.K; gd.M = b_rows(a, step);
      break;
    default:
      ks = blk % S;
      split_rows(a.V, blk / S, P / S, r0, r1);
      gd.K = a.dim / S; gd.k0 = ks * gd.K; gd.M = a.Bq;
      gd.normw = a.fnorm;
      break;
  }
  const int nr = r1 - r0;
  gd.R = kind == BK_UP ? 2 * nr : nr;
  gd.kp = (long long)((gd.K + MF<WT>::KSZ - 1) / MF<WT>::KSZ) * 64;
  gd.pk = b_pk(a, pk_index(kind, l)) + (long long)(kind == BK_UP ? 2 * r0 : r0 * S + ks * nr) * gd.kp;
  // rows in passes of at most GM_MAX (the MFMA core's M-tiles): a pass
  // streams this workgroup's weights once
  const int Mt = gd.M;
  for (int m0 = 0; m0 < Mt; m0 += GM_MAX) {
    gd.m0 = m0;
    gd.M = min(GM_MAX, Mt - m0);
    const RedView rv = b_gemm<WT, XS>(a, s, gd);
    mark(a, s.flag[1], 4);
    const int M = gd.M;
    const int nv = kind == BK_UP ? nr : gd.R;
    for (int o = tidx(); o < nv * M; o += NTHREADS) {
      // output column fastest: a wave's stores cover consecutive columns of
      // one row (a few cache lines) rather than one column of many rows
      const int v = o % nv, mp = o / nv;   // output column, row of the pass
      const int m = m0 + mp;
      const float d = rv.sum(v, mp);
      switch (kind) {
        case BK_PROJ: st_coh(a.xin0 + (size_t)m * a.dim + r0 + v, d); break;
        case BK_QKV:
          if (S > 1) st_coh(bkpart(a, kind, step, l, ks) + (size_t)m * a.qkv_dim + r0 + v, d);
          else st_coh(bqkv(a, step, l) + (size_t)m * a.qkv_dim + r0 + v, d / s.rms[mp]);
          break;
        case BK_WO: {
          const int k = r0 + v;
          if (S > 1) {
            st_coh(bkpart(a, kind, step, l, ks) + (size_t)m * a.dim + k, d);
          } else {
            const float xin = l == 0 ? b_layer0_elem<WT>(a, s, m, k) : bx(a, step, l - 1)[(size_t)m * a.dim + k];
            st_coh(bxmid(a, step, l) + (size_t)m * a.dim + k, xin + d);
          }
          break;
        }
        case BK_UP: {
          // rows v < nr are w1 (gate), rows nr + v are w3 (up) of column r0 + v
          const float a1 = d / s.rms[mp], a3 = rv.sum(nr + v, mp) / s.rms[mp];
          st_coh(bg(a, step, l) + (size_t)m * a.ffn + r0 + v, silu(a1) * a3);
          break;
        }
        case BK_DOWN: {
          const int k = r0 + v;
          if (S > 1) st_coh(bkpart(a, kind, step, l, ks) + (size_t)m * a.dim + k, d);
          else st_coh(bx(a, step, l) + (size_t)m * a.dim + k, bxmid(a, step, l)[(size_t)m * a.dim + k] + d);
          break;
        }
        default: {
          if (S > 1) {
            st_coh(bkpart(a, kind, step, l, ks) + (size_t)m * a.V + r0 + v, d);
          } else {
            const float y = d / s.rms[mp];
            st_coh(blogits(a, step) + (size_t)m * a.V + r0 + v, y);
            if (a.logits_out && step >= a.lo_first)
              a.logits_out[((size_t)m * a.lo_rows + (step - a.lo_first)) * a.V + r0 + v] = y;
          }
          break;
        }
      }
    }
    if ((kind == BK_QKV || kind == BK_HEAD) && S > 1 && blk / S == 0 && tidx() < M)   // one row group per slice
      st_coh(bkss(a, kind, step, l, ks) + m0 + tidx(), s.rms[tidx()]);
    if (m0 + GM_MAX < Mt) __syncthreads();   // the next pass reuses the partial sums and rms in LDS
  }
  const int M = Mt;
  if (S > 1 && (kind == BK_WO || kind == BK_DOWN)) {
    // the row group's last contributor: the output from the K slices'
    // partial sums added in slice order (wo: x_mid = x_in + sum; w2: x =
    // x_mid + sum), and the count cleared for the next frame
    int* cnt = a.kcnt[kind] + (b_slot(a, step, l) * (P / S) + blk / S) * KCNT_STRIDE;
    wait_vmem();        // this workgroup's partial sums have been stored
    __syncthreads();
    if (tidx() == 0) s.flag[3] = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == S - 1;
    __syncthreads();
    if (s.flag[3]) {
      // FB elements a thread per batch, every load of a batch issued before
      // any is used (one memory round trip a batch, not one an element)
      constexpr int FB = 4, SMAX = 4;
      const int n = nr * M;
      for (int base = 0; base < n; base += FB * NTHREADS) {
        float pv[FB][SMAX];
        float xv[FB];
#pragma unroll
        for (int j = 0; j < FB; ++j) {
          const int o = min(base + j * NTHREADS + tidx(), n - 1);
          const int k = r0 + o % nr, m = o / nr;   // columns fastest (coalesced)
          const size_t e = (size_t)m * a.dim + k;
#pragma unroll
          for (int q = 0; q < SMAX; ++q) pv[j][q] = q < S ? ld_coh(bkpart(a, kind, step, l, q) + e) : 0.0f;
          xv[j] = kind == BK_WO ? (l == 0 ? b_layer0_elem<WT>(a, s, m, k) : bx(a, step, l - 1)[e])
                                : bxmid(a, step, l)[e];
        }
#pragma unroll
        for (int j = 0; j < FB; ++j) {
          const int o = base + j * NTHREADS + tidx();
          if (o < n) {
            const int k = r0 + o % nr, m = o / nr;   // columns fastest (coalesced)
            float sum = pv[j][0];
#pragma unroll
            for (int q = 1; q < SMAX; ++q)
              if (q < S) sum += pv[j][q];
            st_coh((kind == BK_WO ? bxmid(a, step, l) : bx(a, step, l)) + (size_t)m * a.dim + k, xv[j] + sum);
          }
        }
      }
      if (tidx() == 0) st_coh(cnt, 0);
    }
  }
  mark(a, s.flag[1], 5);
}

// One (request b, KV group g) pair of the attention phase: the request's
// new rows' q (the group's heads), k and v from the wqkv outputs, its cached
// keys/values of earlier positions, q/k RMSNorm + pair RoPE, then causal
// attention with offset 0; the new keys/values are kept for the frame's
// later steps.
template <typename WT>
__device__ __forceinline__ void b_attn_pair(const BatchArgs& a, const BLds& s, int step, int l, int b, int g,
                                            int prev_code) {
  const int hd = a.hd, gh = a.gheads, H = a.n_head, G = a.n_kv;
  const int n_new = step == 1 ? 2 : 1;
  const int first_new = step == 1 ? 0 : step;
  const int tid = tidx(), wave = tid >> 6, lane = tid & 63;
  float* q = reinterpret_cast<float*>(s.xf);                 // [n_new][gh][hd]
  float* kc = q + (size_t)2 * gh * hd;                       // [ctx][hd]
  float* vc = kc + (size_t)a.ctx_len * hd;                   // [ctx][hd]
  // gather: cached keys/values, then the new rows' raw q, k, v (layer 0 of
  // steps >= 2: the qkv0 row of the code that produced the row)
  const float* row0 = (l == 0 && step >= 2)
                          ? a.qkv0 + (size_t)(prev_code >= 0 ? prev_code : b_code(a, b, step - 1)) * a.qkv_dim
                          : nullptr;
  // a wqkv split over K (two slices): the new rows' values are the slices'
  // partial sums added in slice order, divided by the RMS of the whole row,
  // rebuilt from the slices' sums of squares
  const int S = row0 ? 1 : a.ks[BK_QKV];
  // Segments of hd floats: the cached keys of positions < first_new, their
  // values, then per new row its gh query heads, its key and its value.  A
  // wave moves one segment per step (lane i: floats 2i, 2i + 1, one 8-byte
  // load per K-slice); the segment arithmetic is wave-uniform, and a wave
  // issues the loads of all its segments before storing any.
  const int F = first_new;
  const int nseg = 2 * F + n_new * (gh + 2);
  constexpr int NSW = 4;   // segments a wave per batch
  float ssq[2][2];
#pragma unroll
  for (int nr = 0; nr < 2; ++nr) {
    const int m = step == 1 ? min(nr, n_new - 1) * a.Bq + b : b;
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2) ssq[nr][q2] = S > 1 ? bkss(a, BK_QKV, step, l, q2)[m] : 0.0f;
  }
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int hp = hd >> 1, lp = min(lane, hp - 1);
  // segment sg: sources (slice 0, slice 1), LDS destination, and the new
  // row whose RMS divides it (-1: taken as is)
  const auto seg = [&](int sg, const float*& s0, const float*& s1, float*& dst, int& nr) __attribute__((always_inline)) {
    nr = -1;
    if (sg < F) {
      s0 = s1 = bkv(a, b, l, sg, g);
      dst = kc + (size_t)sg * hd;
      return;
    }
    if (sg < 2 * F) {
      s0 = s1 = bkv(a, b, l, sg - F, g) + hd;
      dst = vc + (size_t)(sg - F) * hd;
      return;
    }
    const int t = sg - 2 * F;
    const int r = t >= gh + 2 ? 1 : 0, h = t - r * (gh + 2);   // n_new <= 2
    const int m = step == 1 ? r * a.Bq + b : b;
    const int pos = step == 1 ? r : step;
    int c;   // first column of the segment in the wqkv output row
    if (h < gh) { c = (g * gh + h) * hd; dst = q + (size_t)(r * gh + h) * hd; }
    else if (h == gh) { c = (H + g) * hd; dst = kc + (size_t)pos * hd; }
    else { c = (H + G + g) * hd; dst = vc + (size_t)pos * hd; }
    if (row0) { s0 = s1 = row0 + c; }
    else if (S > 1) {
      s0 = bkpart(a, BK_QKV, step, l, 0) + (size_t)m * a.qkv_dim + c;
      s1 = bkpart(a, BK_QKV, step, l, 1) + (size_t)m * a.qkv_dim + c;
      nr = r;
    } else { s0 = s1 = bqkv(a, step, l) + (size_t)m * a.qkv_dim + c; }
  };
  for (int base = 0; base < nseg; base += NSW * NWAVE) {
    u64 v0[NSW], v1[NSW];
    float* dst[NSW];
    int nrw[NSW];
#pragma unroll
    for (int j = 0; j < NSW; ++j) {
      const int sg = base + wv + NWAVE * j;
      const float *s0, *s1;
      seg(sg < nseg ? sg : 0, s0, s1, dst[j], nrw[j]);   // a step past the end re-reads segment 0
      v0[j] = *reinterpret_cast<const u64*>(s0 + 2 * lp);
      v1[j] = *reinterpret_cast<const u64*>(s1 + 2 * lp);
    }
    float rden[2];
#pragma unroll
    for (int nr = 0; nr < 2; ++nr) rden[nr] = sqrtf((ssq[nr][0] + ssq[nr][1]) / (float)a.dim + a.eps);
#pragma unroll
    for (int j = 0; j < NSW; ++j) {
      if (base + wv + NWAVE * j < nseg && lane < hp) {
        float x0 = __uint_as_float((u32)v0[j]), x1 = __uint_as_float((u32)(v0[j] >> 32));
        if (nrw[j] >= 0) {
          x0 = (x0 + __uint_as_float((u32)v1[j])) / rden[nrw[j]];
          x1 = (x1 + __uint_as_float((u32)(v1[j] >> 32))) / rden[nrw[j]];
        }
        dst[j][2 * lane] = x0;
        dst[j][2 * lane + 1] = x1;
      }
    }
  }
  __syncthreads();
  mark(a, s.flag[1], 2);
  const float* qn = s.qkn + (size_t)l * 2 * hd;
  const float* kn = qn + hd;
  for (int v = wave; v < n_new * gh + n_new; v += NWAVE) {
    if (v < n_new * gh) {
      head_norm_rope(q + (size_t)v * hd, hd, qn, a.has_qkn, a.eps, s.rope, a.ctx_len, first_new + v / gh);
    } else {
      const int pos = first_new + (v - n_new * gh);
      head_norm_rope(kc + (size_t)pos * hd, hd, kn, a.has_qkn, a.eps, s.rope, a.ctx_len, pos);
    }
  }
  __syncthreads();
  mark(a, s.flag[1], 3);
  for (int i = tid; i < n_new * 2 * hd; i += NTHREADS) {
    const int nr = i / (2 * hd), r = i - nr * 2 * hd;
    const int pos = first_new + nr;
    st_coh(bkv(a, b, l, pos, g) + r, r < hd ? kc[(size_t)pos * hd + r] : vc[(size_t)pos * hd + r - hd]);
  }
  mark(a, s.flag[1], 4);
  // one wave per (row, head); same straight-line scheme as the batch-1 kernel
  const float scale = 1.0f / sqrtf((float)hd);
  const int g16 = lane >> 4, l16 = lane & 15;
  const int d8 = min(8 * l16, hd - 8);
  const bool dlive = 8 * l16 < hd;
  const int c0 = min(lane, hd - 1), c1 = min(lane + 64, hd - 1);
  for (int pr = wave; pr < n_new * gh; pr += NWAVE) {
    const int nr = pr / gh, hh = pr % gh;
    const int pos = first_new + nr;
    const int m = step == 1 ? nr * a.Bq + b : b;
    const float* qv = q + (size_t)pr * hd;
    const float4 qa = *reinterpret_cast<const float4*>(qv + d8);
    const float4 qb = *reinterpret_cast<const float4*>(qv + d8 + 4);
    float sc4[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int jp = 4 * r + g16;
      const float* kr = kc + (size_t)min(jp, pos) * hd + d8;
      const float4 ka = *reinterpret_cast<const float4*>(kr);
      const float4 kb = *reinterpret_cast<const float4*>(kr + 4);
      float part = qa.x * ka.x;
      part = fmaf(qa.y, ka.y, part); part = fmaf(qa.z, ka.z, part); part = fmaf(qa.w, ka.w, part);
      part = fmaf(qb.x, kb.x, part); part = fmaf(qb.y, kb.y, part);
      part = fmaf(qb.z, kb.z, part); part = fmaf(qb.w, kb.w, part);
      part = row16_sum(dlive ? part : 0.0f);
      sc4[r] = (jp <= pos) ? part * scale : -INFINITY;
    }
    float mx = fmaxf(fmaxf(sc4[0], sc4[1]), fmaxf(sc4[2], sc4[3]));
    mx = fmaxf(fmaxf(readlane_f(mx, 0), readlane_f(mx, 16)), fmaxf(readlane_f(mx, 32), readlane_f(mx, 48)));
    float e4[4], es = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      e4[r] = expf(sc4[r] - mx);
      es += e4[r];
    }
    const float den = (readlane_f(es, 0) + readlane_f(es, 16)) + (readlane_f(es, 32) + readlane_f(es, 48));
    float o0 = 0.0f, o1 = 0.0f;
#pragma unroll
    for (int jp = 0; jp < 16; ++jp) {
      const float* vr = vc + (size_t)min(jp, pos) * hd;
      const float ej = readlane_f(e4[jp >> 2], (jp & 3) * 16);   // 0 past pos
      o0 = fmaf(ej, vr[c0], o0);
      o1 = fmaf(ej, vr[c1], o1);
    }
    o0 /= den;   // the weights' normalisation, once per output
    o1 /= den;
    float* o = batt(a, step, l) + (size_t)m * a.attn_dim + (size_t)g * a.gw + (size_t)hh * hd;
    if (lane < hd) st_coh(o + lane, o0);
    if (lane + 64 < hd) st_coh(o + lane + 64, o1);
  }
  mark(a, s.flag[1], 5);
}

// Request b's code of step `step`, drawn from that step's logits and
// returned to every thread of the workgroup (with a teacher-forced prefix:
// the prefix's code).  With the head split over K, the workgroup first adds
// request b's two slices of logits in slice order and divides by the RMS
// rebuilt from the slices' sums of squares, into LDS.  With `publish` the
// workgroup also writes the logits to the caller's buffer and the code to
// the codes arrays.
__device__ __forceinline__ int b_draw(const BatchArgs& a, const BLds& s, int step, int b, bool publish) {
  const float* L = blogits(a, step) + (size_t)b * a.V;
  const int S = a.ks[BK_HEAD];
  const bool want_logits = publish && a.logits_out && step >= a.lo_first;
  if (a.forced && !(S > 1 && want_logits)) return b_code(a, b, step);
  if (S > 1) {
    // Every load of a batch (the slices' sums of squares, then SB logits a
    // thread from each slice) is issued before any is used: one memory
    // round trip a batch.  Slices past S read slice 0 and are not added.
    constexpr int SB = 8, SMAX = 4;
    float ssq[SMAX];
#pragma unroll
    for (int q = 0; q < SMAX; ++q) ssq[q] = bkss(a, BK_HEAD, step, 0, q < S ? q : 0)[b];
    float* lg = reinterpret_cast<float*>(s.xf);
    const int V = a.V;
    for (int base = 0; base < V; base += SB * NTHREADS) {
      float pv[SB][SMAX];
#pragma unroll
      for (int j = 0; j < SB; ++j) {
        const int i = min(base + j * NTHREADS + tidx(), V - 1);
#pragma unroll
        for (int q = 0; q < SMAX; ++q) pv[j][q] = bkpart(a, BK_HEAD, step, 0, q < S ? q : 0)[(size_t)b * V + i];
      }
      float ss = ssq[0];
#pragma unroll
      for (int q = 1; q < SMAX; ++q)
        if (q < S) ss += ssq[q];
      const float rd = sqrtf(ss / (float)a.dim + a.eps);
#pragma unroll
      for (int j = 0; j < SB; ++j) {
        const int i = base + j * NTHREADS + tidx();
        if (i < V) {
          float v = pv[j][0];
#pragma unroll
          for (int q = 1; q < SMAX; ++q)
            if (q < S) v += pv[j][q];
          v /= rd;
          lg[i] = v;
          if (want_logits) a.logits_out[((size_t)b * a.lo_rows + (step - a.lo_first)) * V + i] = v;
        }
      }
    }
    __syncthreads();
    L = lg;
  }
  if (a.forced) return b_code(a, b, step);
  const SampScratch sc{s.cval, s.cidx, s.sred};
  const int code = sample_request(L, a.V, a.temp[b], a.top_p[b], a.top_k[b],
                                  a.uniforms[(size_t)b * (a.ncb - 1) + (step - 1)], sc);
  if (tidx() == 0) {
    const int c = min(max(code, 0), a.V - 1);
    s.flag[2] = c;
    if (publish) {
      st_coh(a.codes + b * 16 + step, c);
      if (a.codes_out) a.codes_out[(size_t)b * a.ncb + step] = c;
    }
  }
  __syncthreads();
  return s.flag[2];
}

// The last step's draw: workgroup b < Bq draws and publishes request b's code.
__device__ __forceinline__ void b_phase_sample(const BatchArgs& a, const BLds& s, int step) {
  if ((int)blockIdx.x < a.Bq) b_draw(a, s, step, blockIdx.x, true);
}

// The attention phase: workgroup j takes the pairs j, j + gridDim.x, ...
// With `draw` (layer 0 of steps >= 2), the workgroup of pair (b, g) first
// draws request b's code of the previous step itself (b_draw; every
// workgroup of the request draws the same code), so no grid barrier
// separates the draw from the attention that needs it; the workgroup of
// KV group 0 publishes the code.
template <typename WT>
__device__ __forceinline__ void b_phase_attn(const BatchArgs& a, const BLds& s, int step, int l, bool draw) {
  for (int j = blockIdx.x; j < a.Bq * a.n_kv; j += gridDim.x) {
    if (j != (int)blockIdx.x) __syncthreads();   // the previous pair's LDS scratch is read out
    const int b = j / a.n_kv, g = j - (j / a.n_kv) * a.n_kv;
    int code = -1;
    if (draw) {
      code = b_draw(a, s, step - 1, b, g == 0);
      __syncthreads();   // the draw's LDS scratch is the attention's
    }
    b_attn_pair<WT>(a, s, step, l, b, g, code);
  }
}

// Whether the next step's layer-0 attention phase draws the codes itself:
// when every (request, KV group) pair has a workgroup of its own (a
// workgroup with two pairs of different requests would draw twice: slower
// than a sample phase of one draw a workgroup and its barrier).
__host__ __device__ inline bool b_merged_draw(int Bq, int n_kv, int P) { return Bq * n_kv <= P; }

// grid syncs of one launch; steps >= 2 have no layer-0 wqkv phase.  A
// step's head is followed by one sync; with merged draws the next step's
// layer-0 attention phase then draws the codes (the last step: a sample
// phase with no sync after it), otherwise a sample phase and a second sync
// follow.  With a teacher-forced prefix nothing is drawn, and the head's
// sync remains only when the head is split over K and the caller wants the
// logits (head_logits), which the next phase assembles.
__host__ __device__ inline int b_syncs(int has_proj, int nsteps, int n_layer, bool forced, bool head_logits,
                                       bool merged) {
  return (has_proj ? 1 : 0) + nsteps * (5 * n_layer + (forced ? (head_logits ? 1 : 0) : (merged ? 1 : 2))) -
         (nsteps - 1);
}

// The phases of one launch; false if a barrier wait gave up.
template <typename WT>
__device__ __forceinline__ bool b_frame(const BatchArgs& a, const BLds& s) {
  u32 epoch = a.epoch0;
  if (a.has_qkn) {
    for (int i = tidx(); i < a.n_layer * 2 * a.hd; i += NTHREADS) {
      const int l = i / (2 * a.hd), r = i - l * 2 * a.hd;
      const WT* w = reinterpret_cast<const WT*>(r < a.hd ? a.L[l].q_norm : a.L[l].k_norm);
      s.qkn[i] = WTraits<WT>::one(w, r < a.hd ? r : r - a.hd);
    }
  }
  for (int i = tidx(); i < a.ctx_len * a.hd; i += NTHREADS) s.rope[i] = a.rope[i];
  if (blockIdx.x == 0 && a.codes_out)
    for (int b = tidx(); b < a.Bq; b += NTHREADS) a.codes_out[(size_t)b * a.ncb] = b_code(a, b, 0);
  __syncthreads();
  if (a.has_proj) {
    b_phase_gemm<WT>(a, s, BK_PROJ, 0, 0);
    if (!grid_sync(a, epoch, s.flag)) return false;
  }
  // a step's head is followed by a sync when something reads its output:
  // the draw, or with a teacher-forced prefix the assembly of a split head's
  // logits for the caller
  const bool head_sync = !a.forced || (a.ks[BK_HEAD] > 1 && a.logits_out);
  const bool merged = b_merged_draw(a.Bq, a.n_kv, gridDim.x);
  for (int step = 1; step <= a.nsteps; ++step) {
    const int M = b_rows(a, step);
    if (a.tlog && tidx() == 0) s.flag[1] = (int)(epoch - a.epoch0);
    for (int l = 0; l < a.n_layer; ++l) {
      if (l == 0 && step == 1) {
        // layer-0 input of every row: the hidden state at position 0, else
        // fast_embeddings[c_0] ("Fast-AR codebook decoding ...", section 2)
        for (int m = tidx(); m < M; m += NTHREADS) {
          const int pos = b_pos(a, step, m);
          s.rcode[m] = pos == 0 ? -1 : b_code(a, m % a.Bq, pos - 1);
        }
        __syncthreads();
      }
      if (l > 0 || step == 1) {   // layer 0 of later steps reads the qkv0 table in the attention phase
        b_phase_gemm<WT>(a, s, BK_QKV, step, l);
        if (!grid_sync(a, epoch, s.flag)) return false;
        if (a.tlog && tidx() == 0) s.flag[1] = (int)(epoch - a.epoch0);
      }
      b_phase_attn<WT>(a, s, step, l, merged && l == 0 && step >= 2 && head_sync);
      if (!grid_sync(a, epoch, s.flag)) return false;
      if (a.tlog && tidx() == 0) s.flag[1] = (int)(epoch - a.epoch0);
      if (l == 0 && step >= 2) {
        // the rows' layer-0 inputs (for wo's residual): fast_embeddings of
        // the codes the attention phase drew
        for (int m = tidx(); m < M; m += NTHREADS) s.rcode[m] = b_code(a, m, step - 1);
        __syncthreads();
      }
      b_phase_gemm<WT>(a, s, BK_WO, step, l);
      if (!grid_sync(a, epoch, s.flag)) return false;
      if (a.tlog && tidx() == 0) s.flag[1] = (int)(epoch - a.epoch0);
      b_phase_gemm<WT>(a, s, BK_UP, step, l);
      if (!grid_sync(a, epoch, s.flag)) return false;
      if (a.tlog && tidx() == 0) s.flag[1] = (int)(epoch - a.epoch0);
      b_phase_gemm<WT>(a, s, BK_DOWN, step, l);
      if (!grid_sync(a, epoch, s.flag)) return false;
      if (a.tlog && tidx() == 0) s.flag[1] = (int)(epoch - a.epoch0);
    }
    b_phase_gemm<WT>(a, s, BK_HEAD, step, 0);
    if (!head_sync) continue;
    if (!grid_sync(a, epoch, s.flag)) return false;
    if (a.tlog && tidx() == 0) s.flag[1] = (int)(epoch - a.epoch0);
    if (merged && !a.forced) {
      if (step == a.nsteps) b_phase_sample(a, s, step);
      continue;
    }
    // a sample phase of its own: workgroup b draws (or, teacher-forced,
    // assembles the logits of) request b
    b_phase_sample(a, s, step);
    if (a.forced) continue;
    if (!grid_sync(a, epoch, s.flag)) return false;
    if (a.tlog && tidx() == 0) s.flag[1] = (int)(epoch - a.epoch0);
  }
  return true;
}

template <typename WT>
__global__ void __launch_bounds__(NTHREADS) frame_kernel_b(BatchArgs a) {
  extern __shared__ float lds_base[];
  const BLds s = b_carve(reinterpret_cast<char*>(lds_base), a);
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  b_frame<WT>(a, s);
  // a barrier wait gave up: the K-split counts are cleared (the next frame
  // counts from zero) and every request of the launch keeps its semantic
  // code with codebooks 1.. at 0 ("Fast-AR codebook decoding ...", section
  // 5.2)
  launch_exit(a, s.flag, [&]() __attribute__((always_inline)) {
    const size_t slots = (size_t)(a.ncb - 1) * a.n_layer;
    for (int kd = 0; kd < 6; ++kd)
      if (a.ks[kd] > 1 && a.kcnt[kd]) zero_words32(a.kcnt[kd], slots * (gridDim.x / a.ks[kd]) * KCNT_STRIDE);
    if (a.codes_out)
      for (int i = tidx(); i < a.Bq * a.ncb; i += NTHREADS) {
        const int b = i / a.ncb, j = i - b * a.ncb;
        st_coh(a.codes_out + i, j == 0 ? b_code(a, b, 0) : 0);
      }
  });
}
