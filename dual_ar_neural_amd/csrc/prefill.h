// Slow-AR prefill on the matrix cores: one cooperative launch runs a chunk
// of prompt positions (up to BQ_MAX) through every layer as the rows of the
// batched kernel's skinny GEMMs, so the weights cross HBM once per chunk.
// Included by s2fast.hip after batched.h and slow_step.h, inside its
// anonymous namespace.
//
// What a chunk computes ("Overall architecture & Dual-AR data flow",
// sections 3.2, 3.4 and 4): position n_past0 + i takes the input
//   x = sem_scale * embeddings[m_i] + (m_i semantic ? sum_j codebook_embeddings[j cbs + c_ij] : 0)
// and runs through the layers causally: its keys and values (after q/k
// RMSNorm and RoPE at its position, rounded to the cache's type) go into
// the caller's cache, and its attention sees the cache positions 0 .. its
// own.  Phases, each closed by a grid barrier:
//   COMBINE  every position's input vector
//   per layer: QKV (batched GEMM) | KV (the chunk's keys and values into
//   the cache) | ATTN (one workgroup per position and KV group) | WO | UP |
//   DOWN (batched GEMMs)
// The last layer stops after KV: its attention and FFN feed only the head,
// which a prefill position does not have.  When the chunk holds the
// prompt's last position as its last row (pf_full_last), the last layer
// runs in full and that row's output is left in the arena for a head-only
// Slow-AR launch (the masked head and the draw); otherwise the prompt's
// last position is a Slow-AR step of its own.
// The GEMMs split X into three bf16 pieces (float32-level products): with
// two, the residual stream's error after 36 layers moved keys beyond the
// bf16 rounding band of the float32 step.

// grid syncs of one prefill launch (no sync after the last layer's KV
// phase unless the last layer runs in full; `merge`: the attention's split
// results are merged in a phase of their own)
__host__ __device__ inline int p_syncs(int n_layer, bool merge, bool full_last) {
  const int per = merge ? 7 : 6;
  return 1 + per * (n_layer - 1) + (full_last ? per : 1);
}

constexpr int PF_NQ = 64;       // query vectors of one attention work item (four 16-wide MFMA tiles)
constexpr int PF_TILE = 64;     // cache positions a workgroup stages per iteration
constexpr int PF_PSMAX = 16;    // splits of an item's cache positions at most
constexpr int PF_KPAD = 8, PF_VPAD = 8;   // bf16 row padding of the staged K and transposed V tiles

// query positions of one work item: as many as fill 64 query vectors
__host__ __device__ inline int p_qpos(int gheads) { return PF_NQ / gheads; }

// Position rows' inputs.  The row-0 token is clamped to [0, vocab), codes to
// [0, cbs); codebook rows count only for a semantic row-0 token, and are
// added in codebook order after the scaled embedding (as the step does).
template <typename WT>
__device__ __forceinline__ void p_combine(const BatchArgs& a) {
  const int row = 1 + a.ncb, D = a.dim;
  const size_t n = (size_t)a.Bq * D;
  const WT* emb = reinterpret_cast<const WT*>(a.emb);
  const WT* cemb = reinterpret_cast<const WT*>(a.cemb);
  for (size_t e = (size_t)blockIdx.x * NTHREADS + tidx(); e < n; e += (size_t)gridDim.x * NTHREADS) {
    const int i = (int)(e / D), k = (int)(e - (size_t)i * D);
    const int* tk = a.tokens + (size_t)i * row;
    const int m = min(max(tk[0], 0), a.vocab - 1);
    float v = a.sem_scale * WTraits<WT>::one(emb + (size_t)m * D, k);
    if (m >= a.sem_begin && m < a.sem_begin + a.cbs)
      for (int j = 0; j < a.ncb; ++j) {
        const int c = min(max(tk[1 + j], 0), a.cbs - 1);
        v += WTraits<WT>::one(cemb + ((size_t)j * a.cbs + c) * D, k);
      }
    st_coh(a.x0w + e, v);
  }
}

// Column c0.. of row i of the wqkv output, hd values into dst: the two
// K-slices' partial sums added in slice order and divided by the row's RMS,
// or the unsplit output.  Thread t of the block takes values t, t + NTHREADS, ...
__device__ __forceinline__ void p_qkv_row(const BatchArgs& a, int l, int i, int c0, int n, float* dst) {
  const int S = a.ks[BK_QKV];
  if (S > 1) {
    const float ss = bkss(a, BK_QKV, 1, l, 0)[i] + bkss(a, BK_QKV, 1, l, 1)[i];
    const float rden = sqrtf(ss / (float)a.dim + a.eps);
    const float* p0 = bkpart(a, BK_QKV, 1, l, 0) + (size_t)i * a.qkv_dim + c0;
    const float* p1 = bkpart(a, BK_QKV, 1, l, 1) + (size_t)i * a.qkv_dim + c0;
    for (int d = tidx(); d < n; d += NTHREADS) dst[d] = (p0[d] + p1[d]) / rden;
  } else {
    const float* p0 = bqkv(a, 1, l) + (size_t)i * a.qkv_dim + c0;
    for (int d = tidx(); d < n; d += NTHREADS) dst[d] = p0[d];
  }
}

// Element c of row i of the wqkv output (the two K-slices' partial sums
// added in slice order and divided by the row's RMS, or the unsplit value).
__device__ __forceinline__ float p_qkv_elem(const BatchArgs& a, int l, int i, int c) {
  if (a.ks[BK_QKV] > 1) {
    const float ss = bkss(a, BK_QKV, 1, l, 0)[i] + bkss(a, BK_QKV, 1, l, 1)[i];
    const float rden = sqrtf(ss / (float)a.dim + a.eps);
    const size_t e = (size_t)i * a.qkv_dim + c;
    return (bkpart(a, BK_QKV, 1, l, 0)[e] + bkpart(a, BK_QKV, 1, l, 1)[e]) / rden;
  }
  return bqkv(a, 1, l)[(size_t)i * a.qkv_dim + c];
}

// KV: workgroup j takes (position i, KV group g) pairs j, j + gridDim.x, ...:
// the position's key (k RMSNorm, RoPE) and value, rounded to the cache's
// type, into the cache at n_past0 + i (write-through stores: the attention
// phase reads them from other CUs).  Loads this layer's q/k norm weights
// into LDS for the attention phase too.  With a bf16 cache it also writes
// the pair's gh query heads (q RMSNorm, RoPE) to pf_q for the attention on
// the matrix cores, one wave per vector.
template <typename WT>
__device__ __forceinline__ void p_kv(const BatchArgs& a, const BLds& s, int l) {
  using KV = KVElem<WT>;
  const int hd = a.hd, H = a.n_head, G = a.n_kv;
  const LayerPtr L = b_layer(a, l);
  if (a.has_qkn)
    for (int e = tidx(); e < 2 * hd; e += NTHREADS)
      s.qkn[e] = WTraits<WT>::one(reinterpret_cast<const WT*>(e < hd ? L.q_norm : L.k_norm), e < hd ? e : e - hd);
  constexpr bool QOUT = sizeof(WT) == 2;
  const int gh = a.gheads, nv = QOUT ? 2 + gh : 2;
  float* buf = reinterpret_cast<float*>(s.xf);   // [nv][hd]: key, value, the query heads
  const int wave = tidx() >> 6;
  for (int j = blockIdx.x; j < a.Bq * G; j += gridDim.x) {
    __syncthreads();   // the previous pair's buffer is stored; the norm weights are in LDS
    const int i = j / G, g = j - (j / G) * G, pos = a.n_past0 + i;
    // every load of the pair issued before any is used (up to 10 vectors of
    // 128: three elements a thread)
    constexpr int NE = (2 + GH_MAX) * 128 / NTHREADS + 1;
    const bool split = a.ks[BK_QKV] > 1;
    const float rden = split ? sqrtf((bkss(a, BK_QKV, 1, l, 0)[i] + bkss(a, BK_QKV, 1, l, 1)[i]) / (float)a.dim + a.eps)
                             : 1.0f;
    const float* s0 = split ? bkpart(a, BK_QKV, 1, l, 0) : bqkv(a, 1, l);
    const float* s1 = split ? bkpart(a, BK_QKV, 1, l, 1) : bqkv(a, 1, l);
    float v0[NE], v1[NE];
#pragma unroll
    for (int u = 0; u < NE; ++u) {
      const int e = min(tidx() + u * NTHREADS, nv * hd - 1);
      const int v = e / hd, d = e - v * hd;
      const int c = v == 0 ? (H + g) * hd + d : (v == 1 ? (H + G + g) * hd + d : (g * gh + v - 2) * hd + d);
      const size_t o = (size_t)i * a.qkv_dim + c;
      v0[u] = s0[o];
      v1[u] = s1[o];
    }
#pragma unroll
    for (int u = 0; u < NE; ++u) {
      const int e = tidx() + u * NTHREADS;
      if (e < nv * hd) buf[e] = split ? (v0[u] + v1[u]) / rden : v0[u];
    }
    __syncthreads();
    for (int v = wave; v < nv; v += NWAVE)
      if (v != 1) head_norm_rope(buf + v * hd, hd, v == 0 ? s.qkn + hd : s.qkn, a.has_qkn, a.eps, a.rope, a.max_ctx, pos);
    __syncthreads();
    if (QOUT) {
      float* q = a.pf_q + (size_t)i * a.attn_dim + (size_t)g * gh * hd;
      for (int e = tidx(); e < gh * hd; e += NTHREADS) st_coh(q + e, buf[2 * hd + e]);
    }
    WT* row = reinterpret_cast<WT*>(a.cache) + (((size_t)l * G + g) * a.max_ctx + pos) * 2 * hd;
    // two values a 32-bit store (hd is even)
    for (int d = tidx(); 2 * d < 2 * hd; d += NTHREADS) {
      if constexpr (sizeof(WT) == 2) {
        const u32 w = (u32)KV::enc(buf[2 * d]) | ((u32)KV::enc(buf[2 * d + 1]) << 16);
        st_coh(reinterpret_cast<u32*>(row) + d, w);
      } else {
        float* rf = reinterpret_cast<float*>(row);
        st_coh(rf + 2 * d, buf[2 * d]);
        st_coh(rf + 2 * d + 1, buf[2 * d + 1]);
      }
    }
  }
}

// ATTN: workgroup j takes (position i, KV group g) pairs: the position's gh
// query heads (q RMSNorm, RoPE), scores against the cache positions
// 0 .. n_past0 + i (one thread a position: q from LDS, the key row from the
// cache), a softmax per head over the block, then the output with one wave
// a range of positions and lanes over head dimensions, the waves' partial
// sums added in wave order.  Positions beyond what LDS holds for the scores
// are the host's limit (p_max_positions).
__host__ __device__ inline int p_max_positions(int gheads, int hd) {
  return (XF_BYTES / (int)sizeof(float) - gheads * hd - NWAVE * gheads * hd - 2 * GH_MAX * NWAVE) / gheads;
}

template <typename WT>
__device__ __forceinline__ void p_attn(const BatchArgs& a, const BLds& s, int l) {
  using KV = KVElem<WT>;
  const int hd = a.hd, G = a.n_kv, gh = a.gheads;
  const int tid = tidx(), wave = tid >> 6, lane = tid & 63;
  float* q = reinterpret_cast<float*>(s.xf);         // [gh][hd]
  float* ow = q + gh * hd;                            // [NWAVE][gh][hd] wave partial outputs
  float* red = ow + NWAVE * gh * hd;                  // [2][GH_MAX][NWAVE] max / sum partials
  float* sc = red + 2 * GH_MAX * NWAVE;               // [gh][npos] scores, then weights
  const float scale = 1.0f / sqrtf((float)hd);
  for (int j = blockIdx.x; j < a.Bq * G; j += gridDim.x) {
    __syncthreads();   // the previous pair's LDS is read out
    const int i = j / G, g = j - (j / G) * G, pos = a.n_past0 + i, np = pos + 1;
    p_qkv_row(a, l, i, g * gh * hd, gh * hd, q);
    __syncthreads();
    for (int h = wave; h < gh; h += NWAVE)
      head_norm_rope(q + (size_t)h * hd, hd, s.qkn, a.has_qkn, a.eps, a.rope, a.max_ctx, pos);
    __syncthreads();
    const WT* kvg = reinterpret_cast<const WT*>(a.cache) + ((size_t)l * G + g) * a.max_ctx * 2 * hd;
    // scores: thread t takes positions t, t + NTHREADS, ... (16 bytes of the
    // key row a load, every load of a row issued before any is used)
    for (int p = tid; p < np; p += NTHREADS) {
      const WT* kr = kvg + (size_t)p * 2 * hd;
      float acc[GH_MAX];
#pragma unroll
      for (int h = 0; h < GH_MAX; ++h) acc[h] = 0.0f;
      constexpr int EPL = WTraits<WT>::EPL;
      for (int d0 = 0; d0 < hd; d0 += 4 * EPL) {
        uint4 kq[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int d = min(d0 + u * EPL, hd - EPL);
          kq[u] = *reinterpret_cast<const uint4*>(kr + d);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int d = d0 + u * EPL;
          if (d >= hd) break;
          float kf[EPL];
          WTraits<WT>::unpack(kq[u], kf);
#pragma unroll
          for (int h = 0; h < GH_MAX; ++h) {
            if (h >= gh) break;
            const float* qh = q + (size_t)h * hd + d;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[h] = fmaf(qh[e], kf[e], acc[h]);
          }
        }
      }
#pragma unroll
      for (int h = 0; h < GH_MAX; ++h)
        if (h < gh) sc[(size_t)h * np + p] = acc[h] * scale;
    }
    __syncthreads();
    // softmax per head: block max, weights exp(s - max), block sum
    for (int h = 0; h < gh; ++h) {
      float mx = -INFINITY;
      for (int p = tid; p < np; p += NTHREADS) mx = fmaxf(mx, sc[(size_t)h * np + p]);
      mx = wave_max(mx);
      if (lane == 0) red[h * NWAVE + wave] = mx;
    }
    __syncthreads();
    for (int h = 0; h < gh; ++h) {
      float mx = red[h * NWAVE];
#pragma unroll
      for (int w = 1; w < NWAVE; ++w) mx = fmaxf(mx, red[h * NWAVE + w]);
      float sum = 0.0f;
      for (int p = tid; p < np; p += NTHREADS) {
        const float e = expf(sc[(size_t)h * np + p] - mx);
        sc[(size_t)h * np + p] = e;
        sum += e;
      }
      sum = wave_sum(sum);
      if (lane == 0) red[(GH_MAX + h) * NWAVE + wave] = sum;
    }
    __syncthreads();
    // output: wave w takes positions [p0, p1); lanes over head dimensions
    const int p0 = (int)(((long long)np * wave) / NWAVE), p1 = (int)(((long long)np * (wave + 1)) / NWAVE);
    const int dl = min(2 * lane, hd - 2);   // this lane's two dimensions (hd even, <= 128)
    float o[GH_MAX][2];
#pragma unroll
    for (int h = 0; h < GH_MAX; ++h) o[h][0] = o[h][1] = 0.0f;
    constexpr int NBV = 8;
    for (int b0 = p0; b0 < p1; b0 += NBV) {
      typename KV::pair vv[NBV];
#pragma unroll
      for (int u = 0; u < NBV; ++u) vv[u] = KV::load(kvg + (size_t)min(b0 + u, p1 - 1) * 2 * hd + hd + dl);
#pragma unroll
      for (int u = 0; u < NBV; ++u) {
        if (b0 + u >= p1) break;
        const float v0 = KV::lo(vv[u]), v1 = KV::hi(vv[u]);
#pragma unroll
        for (int h = 0; h < GH_MAX; ++h) {
          if (h >= gh) break;
          const float wgt = sc[(size_t)h * np + b0 + u];
          o[h][0] = fmaf(wgt, v0, o[h][0]);
          o[h][1] = fmaf(wgt, v1, o[h][1]);
        }
      }
    }
    if (2 * lane < hd)
#pragma unroll
      for (int h = 0; h < GH_MAX; ++h)
        if (h < gh) {
          ow[((size_t)wave * gh + h) * hd + dl] = o[h][0];
          ow[((size_t)wave * gh + h) * hd + dl + 1] = o[h][1];
        }
    __syncthreads();
    float* out = batt(a, 1, l) + (size_t)i * a.attn_dim + (size_t)g * gh * hd;
    for (int e = tid; e < gh * hd; e += NTHREADS) {
      const int h = e / hd;
      float sum = 0.0f, acc = 0.0f;
#pragma unroll
      for (int w = 0; w < NWAVE; ++w) {
        sum += red[(GH_MAX + h) * NWAVE + w];
        acc += ow[(size_t)w * gh * hd + e];
      }
      st_coh(out + e, acc / sum);
    }
  }
}

// x = hi + lo + lo2 in bf16 pieces (to about 2^-27 relative), the B or A
// operand pieces of eight values
__device__ __forceinline__ void p_split3(const float (&x)[8], bf16x8 (&o)[3]) {
  u32 h[4], l1[4], l2[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    h[p] = bf16_pair(x[2 * p], x[2 * p + 1]);
    const float r0 = x[2 * p] - __uint_as_float(h[p] << 16), r1 = x[2 * p + 1] - __uint_as_float(h[p] & 0xFFFF0000u);
    l1[p] = bf16_pair(r0, r1);
    l2[p] = bf16_pair(r0 - __uint_as_float(l1[p] << 16), r1 - __uint_as_float(l1[p] & 0xFFFF0000u));
  }
  __builtin_memcpy(&o[0], h, 16);
  __builtin_memcpy(&o[1], l1, 16);
  __builtin_memcpy(&o[2], l2, 16);
}

// ATTN on the matrix cores (bf16 caches).  Work item (g, qb, ps): the gh
// query heads of KV group g at the pf_qpos chunk positions of block qb (up
// to 64 query vectors: four 16-wide tiles), over split ps of the cache
// positions the block attends to.  Per 64-position tile the workgroup
// stages the keys (row-major) and the values (transposed) in LDS; wave w
// takes query tile w % 4 and the tile's half w / 4, and computes
//   S^T = K Q^T (A: key rows, exact bf16; B: q in three bf16 pieces),
// scales and masks it causally (position p is seen by chunk position i
// when p <= n_past0 + i), keeps a running maximum and sum per query
// (online softmax), and accumulates O^T += V^T P^T (A: transposed values;
// B: the probabilities in three bf16 pieces, their k order that of the
// score tile's rows in the lane).  The two halves combine in LDS; one split
// writes the output, several write partial (sums, maximum, total) for the
// merge phase.
__device__ __forceinline__ void p_attn_mfma(const BatchArgs& a, const BLds& s, int l) {
  const int hd = a.hd, G = a.n_kv, gh = a.gheads, HDP = a.pf_hdp, KS = HDP / 32, DT = HDP / 16;
  const int QPOS = a.pf_qpos, NB = a.pf_nb, PS = a.pf_ps, C = a.Bq;
  const int nq = min(PF_NQ, QPOS * gh), QTU = (nq + 15) / 16;
  const int tid = tidx(), wave = tid >> 6, lane = tid & 63;
  const int KR = HDP + PF_KPAD, VR = PF_TILE + PF_VPAD;
  float* qf = reinterpret_cast<float*>(s.xf);                          // [64][HDP] query vectors
  uint16_t* kt = reinterpret_cast<uint16_t*>(qf + PF_NQ * HDP);       // [PF_TILE][KR] keys
  uint16_t* vt = kt + PF_TILE * KR;                                    // [HDP][VR] values, transposed
  float* comb = reinterpret_cast<float*>(vt + HDP * VR);               // [4][34][64] second half's state
  const float scale = 1.0f / sqrtf((float)hd);
  const uint16_t* kvg0 = reinterpret_cast<const uint16_t*>(a.cache);
  const int qt = wave & 3, half = wave >> 2;
  const bool act = qt < QTU;
  const int qcol = qt * 16 + (lane & 15);              // this lane's query vector
  for (int it = blockIdx.x; it < G * NB * PS; it += gridDim.x) {
    const int g = it % G, rest = it / G, ps = rest % PS, qb = rest / PS;
    const int i0 = qb * QPOS, ni = min(QPOS, C - i0);
    const int np_b = a.n_past0 + i0 + ni;              // cache positions the block attends to
    const int itot = (np_b + PF_TILE - 1) / PF_TILE, itp = (itot + PS - 1) / PS;
    const int t0 = ps * itp, t1 = min(itot, t0 + itp);
    const uint16_t* kvg = kvg0 + ((size_t)l * G + g) * a.max_ctx * 2 * hd;
    __syncthreads();                                   // the previous item's LDS is read out
    // the query vectors (normalised and rotated by the KV phase), zero past
    // hd; every load issued before any is used
    {
      constexpr int NE = PF_NQ * 128 / NTHREADS;
      float qv[NE];
#pragma unroll
      for (int u = 0; u < NE; ++u) {
        const int e = tid + u * NTHREADS;
        const int qi = e / HDP, d = e - qi * HDP, j = qi / gh, h = qi - j * gh;
        const bool ok = e < PF_NQ * HDP && qi < nq && j < ni && d < hd;
        qv[u] = a.pf_q[ok ? (size_t)(i0 + j) * a.attn_dim + (size_t)(g * gh + h) * hd + d : 0];
        qv[u] = ok ? qv[u] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < NE; ++u)
        if (tid + u * NTHREADS < PF_NQ * HDP) qf[tid + u * NTHREADS] = qv[u];
    }
    __syncthreads();
    mark(a, s.flag[1], 2);
    bf16x8 bq[4][3];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      if (ks < KS) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = qf[qcol * HDP + ks * 32 + 8 * (lane >> 4) + e];
        p_split3(x, bq[ks]);
      }
    const int jq = qcol / gh;
    const int ilim = (qcol < nq && jq < ni) ? a.n_past0 + i0 + jq : -1;   // the last position it sees
    f32x4 O[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) O[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = -INFINITY, l_run = 0.0f;
    // a tile's keys and values: 16-byte pieces, at most two a thread, loaded
    // one tile ahead into registers (rows past the block's positions repeat
    // its last one and are masked below; columns past hd are zero)
    constexpr int NC = PF_TILE * 128 / 8 / NTHREADS;
    uint4 kq[NC], vq[NC];
    const auto load_tile = [&](int t) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < NC; ++u) {
        const int e = tid + u * NTHREADS;
        const int r = e / (HDP / 8), c8 = (e - r * (HDP / 8)) * 8;
        const int p = min(t * PF_TILE + min(r, PF_TILE - 1), np_b - 1);
        const int cc = min(c8, hd - 8);
        kq[u] = *reinterpret_cast<const uint4*>(kvg + (size_t)p * 2 * hd + cc);
        vq[u] = *reinterpret_cast<const uint4*>(kvg + (size_t)p * 2 * hd + hd + cc);
      }
    };
    if (t0 < t1) load_tile(t0);
    mark(a, s.flag[1], 3);
    for (int t = t0; t < t1; ++t) {
      const int pb = t * PF_TILE;
      __syncthreads();                                 // the previous tile is read out
#pragma unroll
      for (int u = 0; u < NC; ++u) {
        const int e = tid + u * NTHREADS;
        if (e < PF_TILE * (HDP / 8)) {
          const int r = e / (HDP / 8), c8 = (e - r * (HDP / 8)) * 8;
          // columns past hd are zero (component selects keep the pieces in registers)
          const bool in = c8 < hd;
          const uint4 kk = make_uint4(in ? kq[u].x : 0u, in ? kq[u].y : 0u, in ? kq[u].z : 0u, in ? kq[u].w : 0u);
          *reinterpret_cast<uint4*>(kt + r * KR + c8) = kk;
          const u32 vw[4] = {in ? vq[u].x : 0u, in ? vq[u].y : 0u, in ? vq[u].z : 0u, in ? vq[u].w : 0u};
#pragma unroll
          for (int w2 = 0; w2 < 4; ++w2) {
            vt[(c8 + 2 * w2) * VR + r] = (uint16_t)(vw[w2] & 0xFFFFu);
            vt[(c8 + 2 * w2 + 1) * VR + r] = (uint16_t)(vw[w2] >> 16);
          }
        }
      }
      __syncthreads();
      if (t + 1 < t1) load_tile(t + 1);
      if (act) {
        f32x4 S[2];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          S[st] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
          const int r0 = half * 32 + st * 16;
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
            if (ks < KS) {
              bf16x8 ak;
              __builtin_memcpy(&ak, kt + (r0 + (lane & 15)) * KR + ks * 32 + 8 * (lane >> 4), 16);
#pragma unroll
              for (int pc = 0; pc < 3; ++pc) S[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, bq[ks][pc], S[st], 0, 0, 0);
            }
        }
        // lane holds rows 4 (lane / 16) + r of each 16-row score tile, column qcol
        float sv[8], tmax = -INFINITY;
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int p = pb + half * 32 + st * 16 + 4 * (lane >> 4) + r;
            const float v = p <= ilim ? S[st][r] * scale : -INFINITY;
            sv[st * 4 + r] = v;
            tmax = fmaxf(tmax, v);
          }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float m_new = fmaxf(m_run, tmax);
        const bool live = m_new != -INFINITY;
        const float alpha = live ? expf(m_run - m_new) : 1.0f;
        float pv[8], psum = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pv[e] = live ? expf(sv[e] - m_new) : 0.0f;
          psum += pv[e];
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;
        bf16x8 bp[3];
        p_split3(pv, bp);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
          if (dt < DT) {
            O[dt] *= alpha;
            // values of the same eight positions, in the same k order
            const uint16_t* vr = vt + (dt * 16 + (lane & 15)) * VR + half * 32 + 4 * (lane >> 4);
            u32 w4[4];
            __builtin_memcpy(w4, vr, 8);
            __builtin_memcpy(w4 + 2, vr + 16, 8);
            bf16x8 av;
            __builtin_memcpy(&av, w4, 16);
#pragma unroll
            for (int pc = 0; pc < 3; ++pc) O[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bp[pc], O[dt], 0, 0, 0);
          }
      }
    }
    mark(a, s.flag[1], 4);
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    float* cb = comb + (size_t)qt * 34 * 64;
    if (act && half == 1) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        if (dt < DT)
#pragma unroll
          for (int r = 0; r < 4; ++r) cb[(dt * 4 + r) * 64 + lane] = O[dt][r];
      cb[32 * 64 + lane] = m_run;
      cb[33 * 64 + lane] = l_run;
    }
    __syncthreads();
    mark(a, s.flag[1], 5);
    if (act && half == 0) {
      const float m1 = cb[32 * 64 + lane], l1 = cb[33 * 64 + lane];
      const float M = fmaxf(m_run, m1);
      const float a0 = M == -INFINITY ? 0.0f : expf(m_run - M), a1 = M == -INFINITY ? 0.0f : expf(m1 - M);
      const float L = l_run * a0 + l1 * a1;
      if (PS == 1) {
        if (ilim >= 0) {
          const int h = qcol - jq * gh;
          float* out = batt(a, 1, l) + (size_t)(i0 + jq) * a.attn_dim + (size_t)(g * gh + h) * hd;
#pragma unroll
          for (int dt = 0; dt < 8; ++dt)
            if (dt < DT)
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int d = dt * 16 + 4 * (lane >> 4) + r;
                if (d < hd) st_coh(out + d, (O[dt][r] * a0 + cb[(dt * 4 + r) * 64 + lane] * a1) / L);
              }
        }
      } else {
        float* pp = a.pf_part + ((size_t)((g * NB + qb) * PS + ps) * PF_NQ + qcol) * (HDP + 2);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
          if (dt < DT)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              st_coh(pp + dt * 16 + 4 * (lane >> 4) + r, O[dt][r] * a0 + cb[(dt * 4 + r) * 64 + lane] * a1);
        if ((lane >> 4) == 0) {
          st_coh(pp + HDP, M);
          st_coh(pp + HDP + 1, L);
        }
      }
    }
  }
}

// MERGE (pf_ps > 1): one wave per query vector adds its splits' partial
// results, each weighted by exp(max_s - max), in split order.
__device__ __forceinline__ void p_attn_merge(const BatchArgs& a, int l) {
  const int hd = a.hd, G = a.n_kv, gh = a.gheads, HDP = a.pf_hdp;
  const int QPOS = a.pf_qpos, NB = a.pf_nb, PS = a.pf_ps, C = a.Bq;
  const int nq = min(PF_NQ, QPOS * gh);
  const int wave = tidx() >> 6, lane = tidx() & 63;
  const size_t sstride = (size_t)PF_NQ * (HDP + 2);
  for (int w = blockIdx.x * NWAVE + wave; w < G * NB * nq; w += gridDim.x * NWAVE) {
    const int qi = w % nq, rest = w / nq, qb = rest % NB, g = rest / NB;
    const int j = qi / gh, h = qi - j * gh, i = qb * QPOS + j;
    if (i >= C) continue;
    const float* base = a.pf_part + ((size_t)(g * NB + qb) * PS * PF_NQ + qi) * (HDP + 2);
    // every split's loads issued before any is used
    float mv[PF_PSMAX], lv[PF_PSMAX], x0[PF_PSMAX], x1[PF_PSMAX];
#pragma unroll
    for (int s2 = 0; s2 < PF_PSMAX; ++s2) {
      const float* q = base + min(s2, PS - 1) * sstride;
      mv[s2] = q[HDP];
      lv[s2] = q[HDP + 1];
      x0[s2] = q[min(lane, HDP - 1)];
      x1[s2] = q[min(lane + 64, HDP - 1)];
    }
    float M = -INFINITY;
#pragma unroll
    for (int s2 = 0; s2 < PF_PSMAX; ++s2)
      if (s2 < PS) M = fmaxf(M, mv[s2]);
    float L = 0.0f, o0 = 0.0f, o1 = 0.0f;
#pragma unroll
    for (int s2 = 0; s2 < PF_PSMAX; ++s2)
      if (s2 < PS) {
        const float wgt = mv[s2] == -INFINITY ? 0.0f : expf(mv[s2] - M);
        L += lv[s2] * wgt;
        o0 += x0[s2] * wgt;
        o1 += x1[s2] * wgt;
      }
    float* out = batt(a, 1, l) + (size_t)i * a.attn_dim + (size_t)(g * gh + h) * hd;
    if (lane < hd) st_coh(out + lane, o0 / L);
    if (lane + 64 < hd) st_coh(out + lane + 64, o1 / L);
  }
}

template <typename WT>
__device__ __forceinline__ bool p_run(const BatchArgs& a, const BLds& s) {
  u32 epoch = a.epoch0;
  for (int m = tidx(); m < MP_MAX; m += NTHREADS) s.rcode[m] = -1;   // layer-0 input: the combined rows
  p_combine<WT>(a);
  if (!grid_sync(a, epoch, s.flag)) return false;
  for (int l = 0; l < a.n_layer; ++l) {
    if (a.tlog && tidx() == 0) s.flag[1] = (int)(epoch - a.epoch0);
    b_phase_gemm<WT, 3>(a, s, BK_QKV, 1, l);
    if (!grid_sync(a, epoch, s.flag)) return false;
    if (a.tlog && tidx() == 0) s.flag[1] = (int)(epoch - a.epoch0);
    p_kv<WT>(a, s, l);
    if (l == a.n_layer - 1 && !a.pf_full_last) break;   // the last layer's output feeds only the head
    if (!grid_sync(a, epoch, s.flag)) return false;
    if (a.tlog && tidx() == 0) s.flag[1] = (int)(epoch - a.epoch0);
    if constexpr (sizeof(WT) == 2) {
      p_attn_mfma(a, s, l);
      if (a.pf_ps > 1) {
        if (!grid_sync(a, epoch, s.flag)) return false;
        if (a.tlog && tidx() == 0) s.flag[1] = (int)(epoch - a.epoch0);
        p_attn_merge(a, l);
      }
    } else {
      p_attn<WT>(a, s, l);
    }
    if (!grid_sync(a, epoch, s.flag)) return false;
    if (a.tlog && tidx() == 0) s.flag[1] = (int)(epoch - a.epoch0);
    b_phase_gemm<WT, 3>(a, s, BK_WO, 1, l);
    if (!grid_sync(a, epoch, s.flag)) return false;
    if (a.tlog && tidx() == 0) s.flag[1] = (int)(epoch - a.epoch0);
    b_phase_gemm<WT, 3>(a, s, BK_UP, 1, l);
    if (!grid_sync(a, epoch, s.flag)) return false;
    if (a.tlog && tidx() == 0) s.flag[1] = (int)(epoch - a.epoch0);
    b_phase_gemm<WT, 3>(a, s, BK_DOWN, 1, l);
    if (!grid_sync(a, epoch, s.flag)) return false;
  }
  return true;
}

template <typename WT>
__global__ void __launch_bounds__(NTHREADS) prefill_kernel_b(BatchArgs a) {
  extern __shared__ float lds_base[];
  const BLds s = b_carve(reinterpret_cast<char*>(lds_base), a);
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  p_run<WT>(a, s);
  // a barrier wait gave up: the K-split counts are cleared for the next
  // launch (the cache positions of the chunk are the caller's to rewrite)
  launch_exit(a, s.flag, [&]() __attribute__((always_inline)) {
    for (int kd = 0; kd < 6; ++kd)
      if (a.ks[kd] > 1 && a.kcnt[kd]) zero_words32(a.kcnt[kd], (size_t)a.n_layer * (gridDim.x / a.ks[kd]) * KCNT_STRIDE);
  });
}
