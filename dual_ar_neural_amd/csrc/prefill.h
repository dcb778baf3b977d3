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
// which a prefill position does not have.  The prompt's last position, with
// the head and the draw, is a Slow-AR step of its own.
// The GEMMs split X into three bf16 pieces (float32-level products): with
// two, the residual stream's error after 36 layers moved keys beyond the
// bf16 rounding band of the float32 step.

// grid syncs of one prefill launch (no sync after the last layer's KV phase)
__host__ __device__ inline int p_syncs(int n_layer) { return 1 + 6 * (n_layer - 1) + 1; }

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

// KV: workgroup j takes (position i, KV group g) pairs j, j + gridDim.x, ...:
// the position's key (k RMSNorm, RoPE) and value, rounded to the cache's
// type, into the cache at n_past0 + i (write-through stores: the attention
// phase reads them from other CUs).  Loads this layer's q/k norm weights
// into LDS for the attention phase too.
template <typename WT>
__device__ __forceinline__ void p_kv(const BatchArgs& a, const BLds& s, int l) {
  using KV = KVElem<WT>;
  const int hd = a.hd, H = a.n_head, G = a.n_kv;
  const LayerPtr L = b_layer(a, l);
  if (a.has_qkn)
    for (int e = tidx(); e < 2 * hd; e += NTHREADS)
      s.qkn[e] = WTraits<WT>::one(reinterpret_cast<const WT*>(e < hd ? L.q_norm : L.k_norm), e < hd ? e : e - hd);
  float* buf = reinterpret_cast<float*>(s.xf);   // [2][hd]: key, value
  const int wave = tidx() >> 6;
  for (int j = blockIdx.x; j < a.Bq * G; j += gridDim.x) {
    __syncthreads();   // the previous pair's buffer is stored; the norm weights are in LDS
    const int i = j / G, g = j - (j / G) * G, pos = a.n_past0 + i;
    p_qkv_row(a, l, i, (H + g) * hd, hd, buf);
    p_qkv_row(a, l, i, (H + G + g) * hd, hd, buf + hd);
    __syncthreads();
    if (wave == 0) head_norm_rope(buf, hd, s.qkn + hd, a.has_qkn, a.eps, a.rope, a.max_ctx, pos);
    __syncthreads();
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
    if (l == a.n_layer - 1) break;   // the last layer's output feeds only the head
    if (!grid_sync(a, epoch, s.flag)) return false;
    if (a.tlog && tidx() == 0) s.flag[1] = (int)(epoch - a.epoch0);
    p_attn<WT>(a, s, l);
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
