// Host side of the Slow-AR step and the full frame (include/s2fast.h):
// context creation, argument checks and the cooperative launches of
// slow_kernel.  Included once, at the end of s2fast.hip, which defines the
// kernels, the RoPE table builder and the Fast-AR context it relies on.

struct s2fast_slow_ctx {
  s2fast_slow_config cfg;
  s2fast_slow_weights w;
  int device = 0, ncu = 0;
  size_t lds_bytes = 0;
  int kmax = 0, rmax = 0, nchunk = 0, nsem = 0, n_allowed = 0, end_first = 0;
  long long x_slot = 0, qkv_slot = 0, acc_slot = 0, g_slot = 0, po_slot = 0, pml_slot = 0, att_slot = 0;
  LayerPtr* layers = nullptr;   // device copy of the layer pointers
  float* rope = nullptr;
  float* x0 = nullptr;
  u64* x = nullptr;            // tagged outputs (x, qkv, g, logits): cleared at creation and
  u64* qkv = nullptr;          // when the epoch counter wraps
  long long* acc = nullptr;
  u64* g = nullptr;
  float* po = nullptr;
  float* pml = nullptr;
  u64* att = nullptr;          // merged attention outputs (tagged)
  int* acnt = nullptr;         // chunk counts of the attention phase
  u64* logits = nullptr;
  int* sem = nullptr;          // the full frame's semantic code, handed to Fast-AR
  u32* flags = nullptr;
  u32* err = nullptr;
  u32* tlog = nullptr;     // allocated on first s2fast_test_slow_timeline call
  bool tlog_on = false;
  u32 give_up = 0;         // test hook (s2fast_test_slow_watchdog)
  u32 epoch = 0;
  // chunked prefill on the matrix cores (prefill_kernel_b), set up by the
  // first s2fast_slow_prefill: packed weight streams, their device table and
  // an arena of n_layer slots of BQ_MAX position rows
  int prefill_chunks = 1;  // 0: every prefill runs two positions a launch (s2fast_test_slow_prefill_chunks)
  int pf_limit = 0;        // > 0: chunks only below this cache position (the same test hook)
  int pf_state = 0;        // 0: not set up; 1: ready; -1: the shape prefills two positions a launch
  int pf_pmax = 0;         // cache positions whose attention scores fit in LDS
  size_t pf_lds = 0;
  char* pf_pk = nullptr;
  long long pf_pk_off[2 + 4 * S2FAST_SLOW_MAX_LAYERS] = {};
  const char** pf_pkt = nullptr;
  float* pf_x0w = nullptr;
  float* pf_x = nullptr;
  float* pf_xmid = nullptr;
  float* pf_qkv = nullptr;
  float* pf_att = nullptr;
  float* pf_g = nullptr;
  float* pf_part = nullptr;  // the attention's split results (bf16 caches)
  float* pf_q = nullptr;     // the chunk's query vectors (bf16 caches)
  long long pf_x_slot = 0, pf_qkv_slot = 0, pf_att_slot = 0, pf_g_slot = 0;
  int pf_ks[6] = {1, 1, 1, 1, 1, 1};
  float* pf_kpart[6] = {};
  long long pf_kslot[6] = {};
  int* pf_kcnt[6] = {};
  float* pf_kss[6] = {};
};

namespace {

void free_slow(s2fast_slow_ctx* c) {
  if (!c) return;
  void* ptrs[] = {c->layers, c->rope, c->x0, c->x, c->qkv, c->acc, c->g, c->po, c->pml, c->att, c->acnt, c->logits, c->sem,
                  c->flags, c->err, c->tlog, c->pf_pk, c->pf_pkt, c->pf_x0w, c->pf_x, c->pf_xmid, c->pf_qkv,
                  c->pf_att, c->pf_g, c->pf_part, c->pf_q};
  for (void* p : ptrs)
    if (p) (void)hipFree(p);
  for (int kd = 0; kd < 6; ++kd) {
    void* kp[] = {c->pf_kpart[kd], c->pf_kcnt[kd], c->pf_kss[kd]};
    for (void* p : kp)
      if (p) (void)hipFree(p);
  }
  delete c;
}

const void* slow_kernel_fn(int dtype, int M) {
  if (dtype == S2FAST_BF16)
    return M == 2 ? reinterpret_cast<const void*>(&slow_kernel<uint16_t, 2>)
                  : reinterpret_cast<const void*>(&slow_kernel<uint16_t, 1>);
  return M == 2 ? reinterpret_cast<const void*>(&slow_kernel<float, 2>)
                : reinterpret_cast<const void*>(&slow_kernel<float, 1>);
}

}  // namespace

extern "C" {

int s2fast_slow_create(const s2fast_slow_config* cfg, const s2fast_slow_weights* w, s2fast_slow_ctx** out) {
  if (!cfg || !w || !out) return S2FAST_ERR_ARG;
  *out = nullptr;
  const s2fast_slow_config& k = *cfg;
  if (k.weight_dtype != S2FAST_BF16 && k.weight_dtype != S2FAST_F32) return S2FAST_ERR_ARG;
  const int epl = k.weight_dtype == S2FAST_BF16 ? 8 : 4;
  if (k.n_layer < 1 || k.n_layer > S2FAST_SLOW_MAX_LAYERS) return S2FAST_ERR_ARG;
  if (k.n_head < 1 || k.n_head_kv < 1 || k.n_head % k.n_head_kv != 0 || k.n_head / k.n_head_kv > GH_MAX)
    return S2FAST_ERR_ARG;
  if (k.head_dim < 8 || k.head_dim > 128 || (k.head_dim % 8)) return S2FAST_ERR_ARG;
  if (k.dim < epl || k.ffn_dim < epl || k.dim > 16384 || k.ffn_dim > 16384 || k.dim % epl || k.ffn_dim % epl)
    return S2FAST_ERR_ARG;
  if (((k.n_head / k.n_head_kv) * k.head_dim) % epl) return S2FAST_ERR_ARG;
  if (k.num_codebooks < 1 || k.num_codebooks > 10) return S2FAST_ERR_ARG;
  if (k.codebook_size < 1 || k.codebook_size > 8191 || k.vocab < 2) return S2FAST_ERR_ARG;
  if (k.semantic_begin < 0 || (long long)k.semantic_begin + k.codebook_size > k.vocab) return S2FAST_ERR_ARG;
  if (k.end_id < 0 || k.end_id >= k.vocab) return S2FAST_ERR_ARG;
  if (k.max_context < 1 || k.max_context > (1 << 20)) return S2FAST_ERR_ARG;
  if (!(k.norm_eps >= 0.0f) || !(k.rope_base > 0.0f)) return S2FAST_ERR_ARG;
  if (!w->embeddings || !w->codebook_embeddings || !w->norm) return S2FAST_ERR_NO_FAST_DECODER;
  auto misaligned = [](const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u); };
  if (misaligned(w->embeddings) || misaligned(w->codebook_embeddings) || misaligned(w->norm)) return S2FAST_ERR_ARG;
  for (int l = 0; l < k.n_layer; ++l) {
    const s2fast_layer_weights& L = w->layers[l];
    if (!L.attention_norm || !L.wqkv || !L.wo || !L.ffn_norm || !L.w1 || !L.w3 || !L.w2)
      return S2FAST_ERR_NO_FAST_DECODER;
    if (k.has_qk_norm && (!L.q_norm || !L.k_norm)) return S2FAST_ERR_NO_FAST_DECODER;
    for (const void* p : {L.attention_norm, L.wqkv, L.q_norm, L.k_norm, L.wo, L.ffn_norm, L.w1, L.w3, L.w2})
      if (misaligned(p)) return S2FAST_ERR_ARG;
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return S2FAST_ERR_HIP;
  if (!is_gfx950(dev)) return S2FAST_ERR_DEVICE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return S2FAST_ERR_HIP;
  if (!prop.cooperativeLaunch) return S2FAST_ERR_DEVICE;

  s2fast_slow_ctx* c = new (std::nothrow) s2fast_slow_ctx();
  if (!c) return S2FAST_ERR_NOMEM;
  c->cfg = k;
  c->w = *w;
  c->device = dev;
  c->ncu = prop.multiProcessorCount;
  const int P = c->ncu, G = k.n_head_kv;
  if (P < G || P > 1024) { free_slow(c); return S2FAST_ERR_DEVICE; }
  const int gheads = k.n_head / G, gw = gheads * k.head_dim;
  const int qkv_dim = (k.n_head + 2 * G) * k.head_dim;
  c->nsem = k.codebook_size;
  const bool end_inside = k.end_id >= k.semantic_begin && k.end_id < k.semantic_begin + k.codebook_size;
  c->n_allowed = c->nsem + (end_inside ? 0 : 1);
  c->end_first = (!end_inside && k.end_id < k.semantic_begin) ? 1 : 0;
  c->nchunk = P / G;
  c->kmax = (std::max(std::max(k.dim, k.ffn_dim), gw) + 3) & ~3;
  int rmax = 0;
  for (int n : {qkv_dim, k.dim, c->n_allowed}) rmax = std::max(rmax, (n + P - 1) / P);
  rmax = std::max(rmax, 2 * ((k.ffn_dim + P - 1) / P));
  rmax = std::max(rmax, (k.dim + c->nchunk - 1) / c->nchunk);   // wo rows of one block of a group
  c->rmax = rmax + 1;
  size_t lds = slow_lds_floats(c->kmax, c->rmax, gheads, k.head_dim) * sizeof(float);
  const size_t one_per_cu = 84 * 1024;   // more than half the CU's LDS: one block per CU
  if (lds < one_per_cu) lds = one_per_cu;
  if (lds > (size_t)prop.sharedMemPerBlock) { free_slow(c); return S2FAST_ERR_ARG; }
  c->lds_bytes = lds;
  for (int M = 1; M <= MMAX; ++M) {
    const void* fn = slow_kernel_fn(k.weight_dtype, M);
    if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess) {
      free_slow(c); return S2FAST_ERR_HIP;
    }
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, NTHREADS, lds) != hipSuccess) { free_slow(c); return S2FAST_ERR_HIP; }
    if (nb < 1) { free_slow(c); return S2FAST_ERR_DEVICE; }
  }

  const int half = k.head_dim / 2;
  std::vector<float> rope((size_t)2 * k.max_context * half);
  rope_table_host(k.head_dim, k.max_context, k.rope_base, rope.data(), rope.data() + (size_t)k.max_context * half);
  std::vector<LayerPtr> lp(k.n_layer);
  for (int l = 0; l < k.n_layer; ++l) {
    const s2fast_layer_weights& L = w->layers[l];
    lp[l] = LayerPtr{L.attention_norm, L.wqkv, L.q_norm, L.k_norm, L.wo, L.ffn_norm, L.w1, L.w3, L.w2};
  }
  auto rup = [](long long n, long long q) { return (n + q - 1) / q * q; };
  const long long Ln = k.n_layer;
  // every per-layer region holds MMAX position rows (prefill takes two
  // positions per launch)
  c->x_slot = rup((long long)MMAX * k.dim, 64);
  c->qkv_slot = rup((long long)MMAX * qkv_dim, 64);
  c->acc_slot = rup((long long)MMAX * k.dim, 32);
  c->g_slot = rup((long long)MMAX * k.ffn_dim, 64);
  c->po_slot = rup((long long)G * c->nchunk * MMAX * gw, 64);
  c->pml_slot = rup((long long)G * c->nchunk * MMAX * gheads * 2, 64);
  c->att_slot = rup((long long)MMAX * k.n_head * k.head_dim, 32);
  bool ok = dalloc(&c->layers, (size_t)k.n_layer) == hipSuccess && dalloc(&c->rope, rope.size()) == hipSuccess &&
            dalloc(&c->x0, (size_t)c->x_slot) == hipSuccess && dalloc(&c->x, (size_t)(Ln * c->x_slot)) == hipSuccess &&
            dalloc(&c->qkv, (size_t)(Ln * c->qkv_slot)) == hipSuccess &&
            dalloc(&c->acc, (size_t)(Ln * c->acc_slot)) == hipSuccess &&
            dalloc(&c->g, (size_t)(Ln * c->g_slot)) == hipSuccess &&
            dalloc(&c->po, (size_t)(Ln * c->po_slot)) == hipSuccess &&
            dalloc(&c->pml, (size_t)(Ln * c->pml_slot)) == hipSuccess &&
            dalloc(&c->att, (size_t)(Ln * c->att_slot)) == hipSuccess &&
            dalloc(&c->acnt, (size_t)(Ln * G * 64)) == hipSuccess &&
            dalloc(&c->logits, (size_t)rup(c->n_allowed, 64)) == hipSuccess && dalloc(&c->sem, 64) == hipSuccess &&
            dalloc(&c->flags, (size_t)P * 64) == hipSuccess && dalloc(&c->err, W_WORDS) == hipSuccess;
  if (!ok) { free_slow(c); return S2FAST_ERR_NOMEM; }
  ok = hipMemcpy(c->layers, lp.data(), lp.size() * sizeof(LayerPtr), hipMemcpyHostToDevice) == hipSuccess &&
       hipMemcpy(c->rope, rope.data(), rope.size() * sizeof(float), hipMemcpyHostToDevice) == hipSuccess &&
       hipMemset(c->acc, 0, (size_t)(Ln * c->acc_slot) * sizeof(long long)) == hipSuccess &&
       hipMemset(c->x, 0, (size_t)(Ln * c->x_slot) * sizeof(u64)) == hipSuccess &&
       hipMemset(c->qkv, 0, (size_t)(Ln * c->qkv_slot) * sizeof(u64)) == hipSuccess &&
       hipMemset(c->g, 0, (size_t)(Ln * c->g_slot) * sizeof(u64)) == hipSuccess &&
       hipMemset(c->att, 0, (size_t)(Ln * c->att_slot) * sizeof(u64)) == hipSuccess &&
       hipMemset(c->acnt, 0, (size_t)(Ln * G * 64) * sizeof(int)) == hipSuccess &&
       hipMemset(c->logits, 0, (size_t)rup(c->n_allowed, 64) * sizeof(u64)) == hipSuccess &&
       hipMemset(c->flags, 0, (size_t)P * 64 * sizeof(u32)) == hipSuccess &&
       hipMemset(c->err, 0, W_WORDS * sizeof(u32)) == hipSuccess && hipDeviceSynchronize() == hipSuccess;
  if (!ok) { free_slow(c); return S2FAST_ERR_HIP; }
  *out = c;
  return S2FAST_OK;
}

void s2fast_slow_destroy(s2fast_slow_ctx* ctx) {
  if (!ctx) return;
  (void)hipDeviceSynchronize();
  free_slow(ctx);
}

// Grid syncs of one step launch: after every layer's WO phase (a
// two-position launch also after its attention phases).
int s2fast_slow_syncs(const s2fast_slow_ctx* ctx) { return ctx ? ctx->cfg.n_layer : -1; }

// Before the epoch counter wraps: the barrier flags and the tagged outputs
// go back to their cleared state and the counter restarts.
int slow_restart_epochs(s2fast_slow_ctx* c, hipStream_t st) {
  auto rup = [](long long n, long long q) { return (n + q - 1) / q * q; };
  const size_t Ln = (size_t)c->cfg.n_layer;
  if (zero_device(c->flags, (size_t)c->ncu * 64 * sizeof(u32), st) != S2FAST_OK ||
      zero_device(c->x, Ln * c->x_slot * sizeof(u64), st) != S2FAST_OK ||
      zero_device(c->qkv, Ln * c->qkv_slot * sizeof(u64), st) != S2FAST_OK ||
      zero_device(c->g, Ln * c->g_slot * sizeof(u64), st) != S2FAST_OK ||
      zero_device(c->att, Ln * c->att_slot * sizeof(u64), st) != S2FAST_OK ||
      zero_device(c->logits, (size_t)rup(c->n_allowed, 64) * sizeof(u64), st) != S2FAST_OK)
    return S2FAST_ERR_HIP;
  c->epoch = 0;
  return S2FAST_OK;
}

int s2fast_slow_status(s2fast_slow_ctx* ctx, void* stream) {
  if (!ctx) return S2FAST_ERR_ARG;
  return read_status(ctx->err, reinterpret_cast<hipStream_t>(stream));
}

int s2fast_test_slow_watchdog(s2fast_slow_ctx* ctx, int32_t give_up) {
  if (!ctx) return S2FAST_ERR_ARG;
  ctx->give_up = give_up ? 1u : 0u;
  return S2FAST_OK;
}

int s2fast_slow_allowed(const s2fast_slow_ctx* ctx) { return ctx ? ctx->n_allowed : -1; }

int s2fast_test_slow_prefill_chunks(s2fast_slow_ctx* ctx, int32_t enable) {
  if (!ctx || enable < 0) return S2FAST_ERR_ARG;
  ctx->prefill_chunks = enable ? 1 : 0;
  ctx->pf_limit = enable > 1 ? enable : 0;
  return S2FAST_OK;
}

}  // extern "C"

namespace {

// Arguments are already validated; do_head = 0 stops after the last layer.
// One launch of the Slow-AR step kernel at positions n_past .. n_past + M - 1
// (M <= MMAX; the second position's tokens are main1 / codes1).  x_head
// (device, not null): a head-only launch whose head reads that row as the
// last layer's output (M = 1, do_head = 1).
int slow_launch(s2fast_slow_ctx* ctx, void* kv_cache, int32_t n_past, int M, const int32_t* prev_main,
                const int32_t* prev_codes, const int32_t* main1, const int32_t* codes1, int do_head, int32_t* window,
                const float* u, const float* temperature, const float* top_p, const int32_t* top_k,
                int32_t* main_out, int32_t* sem_code_out, float* hidden_out, float* logits_out, hipStream_t st,
                const float* x_head = nullptr) {
  const s2fast_slow_config& k = ctx->cfg;
  SlowArgs a;
  std::memset(&a, 0, sizeof(a));
  a.dim = k.dim; a.n_layer = k.n_layer; a.n_head = k.n_head; a.n_kv = k.n_head_kv; a.hd = k.head_dim;
  a.ffn = k.ffn_dim; a.vocab = k.vocab; a.ncb = k.num_codebooks; a.cbs = k.codebook_size;
  a.sem_begin = k.semantic_begin; a.end_id = k.end_id; a.nsem = ctx->nsem; a.n_allowed = ctx->n_allowed;
  a.end_first = ctx->end_first;
  a.eps = k.norm_eps;
  a.sem_scale = (float)(1.0 / std::sqrt((double)(k.num_codebooks + 1)));
  a.has_qkn = k.has_qk_norm ? 1 : 0;
  a.qkv_dim = (k.n_head + 2 * k.n_head_kv) * k.head_dim;
  a.attn_dim = k.n_head * k.head_dim;
  a.gheads = k.n_head / k.n_head_kv;
  a.gw = a.gheads * k.head_dim;
  a.kmax = ctx->kmax; a.rmax = ctx->rmax;
  a.max_ctx = k.max_context; a.n_past = n_past; a.nchunk = ctx->nchunk; a.do_head = do_head;
  a.M = M;
  a.emb = ctx->w.embeddings; a.cemb = ctx->w.codebook_embeddings; a.norm = ctx->w.norm;
  a.L = ctx->layers; a.rope = ctx->rope; a.kv = kv_cache;
  a.prev_main = prev_main; a.prev_codes = prev_codes; a.window = window; a.u = u;
  a.main1 = main1 ? main1 : prev_main; a.codes1 = codes1 ? codes1 : prev_codes;
  a.temp = temperature; a.top_p = top_p; a.top_k = top_k;
  a.main_out = main_out; a.sem_out = sem_code_out; a.hidden_out = hidden_out; a.logits_out = logits_out;
  a.x0 = ctx->x0; a.x = ctx->x; a.qkv = ctx->qkv; a.acc = ctx->acc; a.g = ctx->g; a.po = ctx->po;
  a.pml = ctx->pml; a.logits = ctx->logits;
  a.x_slot = ctx->x_slot; a.qkv_slot = ctx->qkv_slot; a.acc_slot = ctx->acc_slot; a.g_slot = ctx->g_slot;
  a.po_slot = ctx->po_slot; a.pml_slot = ctx->pml_slot;
  a.att = ctx->att; a.acnt = ctx->acnt; a.att_slot = ctx->att_slot;
  a.flags = ctx->flags; a.err = ctx->err; a.tlog = ctx->tlog_on ? ctx->tlog : nullptr;
  a.watch.give_up = ctx->give_up;
  a.x_head = x_head;
  if (ctx->epoch > 0xF0000000u && slow_restart_epochs(ctx, st) != S2FAST_OK) return S2FAST_ERR_HIP;
  a.epoch0 = ctx->epoch;
  void* args[] = {&a};
  if (hipLaunchCooperativeKernel(slow_kernel_fn(k.weight_dtype, M), dim3(ctx->ncu), dim3(NTHREADS), args,
                                 ctx->lds_bytes, st) != hipSuccess)
    return S2FAST_ERR_HIP;
  // its grid syncs, and at least one: the next launch's outputs need another tag
  ctx->epoch += (u32)(x_head ? 1 : (M == 1 ? 1 : 2) * k.n_layer);
  return S2FAST_OK;
}

const void* prefill_fn(int dtype) {
  return dtype == S2FAST_BF16 ? reinterpret_cast<const void*>(&prefill_kernel_b<uint16_t>)
                              : reinterpret_cast<const void*>(&prefill_kernel_b<float>);
}

// First prefill: can this shape run prefill_kernel_b (the batched GEMM's
// tile limits, the attention's LDS), and if so its packed weights, their
// device table, the arena and the K splits (as the batched Fast-AR kernel
// chooses them).  S2FAST_OK with pf_state -1 when the shape cannot.
int prefill_setup(s2fast_slow_ctx* c) {
  const s2fast_slow_config& k = c->cfg;
  const int P = c->ncu, G = k.n_head_kv, gh = k.n_head / G, hd = k.head_dim;
  const int qkv_dim = (k.n_head + 2 * G) * hd, attn_dim = k.n_head * hd;
  c->pf_state = -1;
  int tmax = 0;
  for (int n : {qkv_dim, k.dim}) tmax = std::max(tmax, ((n + P - 1) / P + 15) / 16);
  tmax = std::max(tmax, (2 * ((k.ffn_dim + P - 1) / P) + 15) / 16);
  if (tmax > TMAX || 2 * tmax > RED_TILES) return S2FAST_OK;
  // bf16 caches: the attention streams the cache in tiles (no bound); f32:
  // the scores of a position's attention are held in LDS
  c->pf_pmax = k.weight_dtype == S2FAST_BF16 ? k.max_context : p_max_positions(gh, hd);
  if (c->pf_pmax < 2) return S2FAST_OK;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, c->device) != hipSuccess) return S2FAST_ERR_HIP;
  c->pf_lds = b_lds_bytes(1, hd, 0);
  const void* fn = prefill_fn(k.weight_dtype);
  int nb = 0;
  if (c->pf_lds > (size_t)prop.sharedMemPerBlock ||
      hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)c->pf_lds) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, NTHREADS, c->pf_lds) != hipSuccess || nb < 1)
    return S2FAST_OK;
  const int ksz = k.weight_dtype == S2FAST_BF16 ? 32 : 16;
  const int ks = KS_DOWN;
  const bool rows_fit = P % ks == 0 && (k.dim + P / ks - 1) / (P / ks) <= 16 * TMAX;
  c->pf_ks[BK_DOWN] = (rows_fit && k.ffn_dim % (ks * ksz) == 0) ? ks : 1;
  c->pf_ks[BK_WO] = (rows_fit && attn_dim % (ks * ksz) == 0) ? ks : 1;
  constexpr int kq = 2;
  c->pf_ks[BK_QKV] = (P % kq == 0 && (qkv_dim + P / kq - 1) / (P / kq) <= 16 * TMAX && k.dim % (kq * ksz) == 0)
                         ? kq : 1;
  auto rup = [](long long n, long long q) { return (n + q - 1) / q * q; };
  const long long slots = k.n_layer;
  c->pf_x_slot = rup((long long)BQ_MAX * k.dim, 64);
  c->pf_qkv_slot = rup((long long)BQ_MAX * qkv_dim, 64);
  c->pf_att_slot = rup((long long)BQ_MAX * attn_dim, 64);
  c->pf_g_slot = rup((long long)BQ_MAX * k.ffn_dim, 64);
  bool ok = dalloc(&c->pf_x0w, (size_t)c->pf_x_slot) == hipSuccess &&
            dalloc(&c->pf_x, (size_t)(slots * c->pf_x_slot)) == hipSuccess &&
            dalloc(&c->pf_xmid, (size_t)(slots * c->pf_x_slot)) == hipSuccess &&
            dalloc(&c->pf_qkv, (size_t)(slots * c->pf_qkv_slot)) == hipSuccess &&
            dalloc(&c->pf_att, (size_t)(slots * c->pf_att_slot)) == hipSuccess &&
            dalloc(&c->pf_g, (size_t)(slots * c->pf_g_slot)) == hipSuccess &&
            dalloc(&c->pf_pkt, (size_t)(2 + 4 * k.n_layer)) == hipSuccess;
  if (!ok) return S2FAST_ERR_NOMEM;
  if (k.weight_dtype == S2FAST_BF16) {
    const int hdp = (hd + 31) / 32 * 32, nbmax = (BQ_MAX + p_qpos(gh) - 1) / p_qpos(gh);
    if (dalloc(&c->pf_part, (size_t)G * nbmax * PF_PSMAX * PF_NQ * (hdp + 2)) != hipSuccess ||
        dalloc(&c->pf_q, (size_t)BQ_MAX * attn_dim) != hipSuccess)
      return S2FAST_ERR_NOMEM;
  }
  c->pf_kslot[BK_QKV] = c->pf_qkv_slot;
  c->pf_kslot[BK_WO] = c->pf_kslot[BK_DOWN] = c->pf_x_slot;
  for (int kd : {(int)BK_QKV, (int)BK_WO, (int)BK_DOWN}) {
    if (c->pf_ks[kd] == 1) continue;
    ok = dalloc(&c->pf_kpart[kd], (size_t)(slots * c->pf_ks[kd] * c->pf_kslot[kd])) == hipSuccess &&
         dalloc(&c->pf_kcnt[kd], (size_t)(slots * P * KCNT_STRIDE)) == hipSuccess &&
         dalloc(&c->pf_kss[kd], (size_t)(slots * c->pf_ks[kd] * MP_MAX)) == hipSuccess;
    if (!ok) return S2FAST_ERR_NOMEM;
    if (hipMemset(c->pf_kcnt[kd], 0, (size_t)(slots * P * KCNT_STRIDE) * sizeof(int)) != hipSuccess)
      return S2FAST_ERR_HIP;
  }
  std::vector<PackJob> jobs;
  for (int l = 0; l < k.n_layer; ++l) {
    const s2fast_layer_weights& L = c->w.layers[l];
    jobs.push_back({pk_index(BK_QKV, l), L.wqkv, nullptr, qkv_dim, k.dim, c->pf_ks[BK_QKV]});
    jobs.push_back({pk_index(BK_WO, l), L.wo, nullptr, k.dim, attn_dim, c->pf_ks[BK_WO]});
    jobs.push_back({pk_index(BK_UP, l), L.w1, L.w3, k.ffn_dim, k.dim, 1});
    jobs.push_back({pk_index(BK_DOWN, l), L.w2, nullptr, k.dim, k.ffn_dim, c->pf_ks[BK_DOWN]});
  }
  const int pst = pack_jobs(k.weight_dtype, P, jobs.data(), (int)jobs.size(), &c->pf_pk, c->pf_pk_off);
  if (pst != S2FAST_OK) return pst;
  std::vector<const char*> tbl(2 + 4 * k.n_layer, nullptr);
  for (const PackJob& j : jobs) tbl[j.idx] = c->pf_pk + c->pf_pk_off[j.idx];
  if (hipMemcpy(c->pf_pkt, tbl.data(), tbl.size() * sizeof(const char*), hipMemcpyHostToDevice) != hipSuccess ||
      hipDeviceSynchronize() != hipSuccess)
    return S2FAST_ERR_HIP;
  c->pf_state = 1;
  return S2FAST_OK;
}

// One launch of prefill_kernel_b over positions n_past0 .. n_past0 + C - 1
// (C <= BQ_MAX, their tokens [C][1 + num_codebooks]); full_last: the last
// of them is the prompt's last position (the last layer runs in full).
int prefill_launch(s2fast_slow_ctx* ctx, void* kv_cache, int32_t n_past0, int C, const int32_t* tokens,
                   hipStream_t st, bool full_last) {
  const s2fast_slow_config& k = ctx->cfg;
  BatchArgs a;
  std::memset(&a, 0, sizeof(a));
  a.in_dim = k.dim; a.dim = k.dim; a.n_layer = k.n_layer; a.n_head = k.n_head; a.n_kv = k.n_head_kv;
  a.hd = k.head_dim; a.ffn = k.ffn_dim; a.V = k.codebook_size; a.ncb = k.num_codebooks; a.ctx_len = 0;
  a.eps = k.norm_eps; a.has_proj = 0; a.has_qkn = k.has_qk_norm ? 1 : 0;
  a.qkv_dim = (k.n_head + 2 * k.n_head_kv) * k.head_dim;
  a.attn_dim = k.n_head * k.head_dim;
  a.gheads = k.n_head / k.n_head_kv;
  a.gw = a.gheads * k.head_dim;
  a.emb = ctx->w.embeddings; a.fnorm = ctx->w.norm;
  a.rope = ctx->rope;
  for (int kd = 0; kd < 6; ++kd) {
    a.ks[kd] = ctx->pf_ks[kd]; a.kpart[kd] = ctx->pf_kpart[kd]; a.kslot[kd] = ctx->pf_kslot[kd];
    a.kcnt[kd] = ctx->pf_kcnt[kd]; a.kss[kd] = ctx->pf_kss[kd];
  }
  a.Bq = C; a.nsteps = 1;
  a.hidden = ctx->pf_x0w; a.xin0 = ctx->pf_x0w;
  a.x = ctx->pf_x; a.xmid = ctx->pf_xmid; a.qkv = ctx->pf_qkv; a.att = ctx->pf_att; a.g = ctx->pf_g;
  a.x_slot = ctx->pf_x_slot; a.qkv_slot = ctx->pf_qkv_slot; a.att_slot = ctx->pf_att_slot; a.g_slot = ctx->pf_g_slot;
  a.flags = ctx->flags; a.err = ctx->err;
  a.watch.give_up = ctx->give_up;
  a.tlog = ctx->tlog_on ? ctx->tlog : nullptr;
  a.prefill = 1; a.lds_layers = 1; a.Lt = ctx->layers; a.pkt = ctx->pf_pkt;
  a.n_past0 = n_past0; a.max_ctx = k.max_context; a.cache = kv_cache; a.tokens = tokens; a.x0w = ctx->pf_x0w;
  a.cemb = ctx->w.codebook_embeddings; a.cbs = k.codebook_size; a.sem_begin = k.semantic_begin;
  a.vocab = k.vocab; a.sem_scale = (float)(1.0 / std::sqrt((double)(k.num_codebooks + 1)));
  // attention work items (bf16): blocks of pf_qpos positions per KV group,
  // their cache positions split so that the items fill the grid (each split
  // at least one 64-position tile)
  const int gh = k.n_head / k.n_head_kv;
  a.pf_qpos = p_qpos(gh);
  a.pf_nb = (C + a.pf_qpos - 1) / a.pf_qpos;
  a.pf_hdp = (k.head_dim + 31) / 32 * 32;
  const int tiles = (n_past0 + C + PF_TILE - 1) / PF_TILE;
  a.pf_ps = std::max(1, std::min(std::min(PF_PSMAX, ctx->ncu / (k.n_head_kv * a.pf_nb)), tiles));
  a.pf_part = ctx->pf_part; a.pf_q = ctx->pf_q;
  a.pf_full_last = full_last ? 1 : 0;
  const bool merge = k.weight_dtype == S2FAST_BF16 && a.pf_ps > 1;
  if (ctx->epoch > 0xF0000000u && slow_restart_epochs(ctx, st) != S2FAST_OK) return S2FAST_ERR_HIP;
  a.epoch0 = ctx->epoch;
  void* args[] = {&a};
  if (hipLaunchCooperativeKernel(prefill_fn(k.weight_dtype), dim3(ctx->ncu), dim3(NTHREADS), args, ctx->pf_lds,
                                 st) != hipSuccess)
    return S2FAST_ERR_HIP;
  ctx->epoch += (u32)p_syncs(k.n_layer, merge, full_last);
  return S2FAST_OK;
}

}  // namespace

extern "C" {

int s2fast_slow_step(s2fast_slow_ctx* ctx, void* kv_cache, int32_t n_past, const int32_t* prev_main,
                     const int32_t* prev_codes, int32_t* window, const float* u, const float* temperature,
                     const float* top_p, const int32_t* top_k, int32_t* main_out, int32_t* sem_code_out,
                     float* hidden_out, float* logits_out, void* stream) {
  if (!ctx || !kv_cache || !prev_main || !prev_codes || !window || !u || !temperature || !top_p || !top_k ||
      !main_out || !sem_code_out || !hidden_out)
    return S2FAST_ERR_ARG;
  const s2fast_slow_config& k = ctx->cfg;
  if (n_past < 0 || n_past >= k.max_context) return S2FAST_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(kv_cache) & 15u) || (reinterpret_cast<uintptr_t>(hidden_out) & 15u))
    return S2FAST_ERR_ARG;
  return slow_launch(ctx, kv_cache, n_past, 1, prev_main, prev_codes, nullptr, nullptr, 1, window, u, temperature,
                     top_p, top_k, main_out, sem_code_out, hidden_out, logits_out,
                     reinterpret_cast<hipStream_t>(stream));
}

int s2fast_slow_prefill(s2fast_slow_ctx* ctx, void* kv_cache, int32_t n_past0, int32_t T, const int32_t* tokens,
                        int32_t* window, const float* u, const float* temperature, const float* top_p,
                        const int32_t* top_k, int32_t* main_out, int32_t* sem_code_out, float* hidden_out,
                        float* logits_out, void* stream) {
  if (!ctx || !kv_cache || !tokens || !window || !u || !temperature || !top_p || !top_k || !main_out ||
      !sem_code_out || !hidden_out)
    return S2FAST_ERR_ARG;
  const s2fast_slow_config& k = ctx->cfg;
  if (T < 1 || n_past0 < 0 || (long long)n_past0 + T > k.max_context) return S2FAST_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(kv_cache) & 15u) || (reinterpret_cast<uintptr_t>(hidden_out) & 15u))
    return S2FAST_ERR_ARG;
  const int row = 1 + k.num_codebooks;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (ctx->prefill_chunks && ctx->pf_state == 0 && T > 1) {
    const int rc = prefill_setup(ctx);
    if (rc != S2FAST_OK) return rc;
  }
  int t = 0;
  const int pmax = ctx->pf_limit > 0 ? std::min(ctx->pf_pmax, ctx->pf_limit) : ctx->pf_pmax;
  const bool chunks = ctx->prefill_chunks && ctx->pf_state == 1;
  // the whole prompt in chunks of up to BQ_MAX, the last chunk holding the
  // last position, then a head-only launch for the head and the draw: when
  // every position's attention fits and the last chunk would hold more
  // than the last position alone (else that position costs a chunk's weight
  // pass; the step launch below is cheaper)
  if (chunks && T >= 2 && (long long)n_past0 + T <= pmax && (T - 1) % BQ_MAX != 0) {
    int C = 0;
    for (; t < T; t += C) {
      C = std::min(BQ_MAX, T - t);
      const int rc = prefill_launch(ctx, kv_cache, n_past0 + t, C, tokens + (size_t)t * row, st, t + C == T);
      if (rc != S2FAST_OK) return rc;
    }
    const float* xh = ctx->pf_x + (size_t)(k.n_layer - 1) * ctx->pf_x_slot + (size_t)(C - 1) * k.dim;
    const int32_t* tk = tokens + (size_t)(T - 1) * row;
    return slow_launch(ctx, kv_cache, n_past0 + T - 1, 1, tk, tk + 1, nullptr, nullptr, 1, window, u, temperature,
                       top_p, top_k, main_out, sem_code_out, hidden_out, logits_out, st, xh);
  }
  // the positions before the last in chunks of up to BQ_MAX a launch (one
  // weight pass a chunk), while their attention fits
  if (chunks)
    while (t < T - 1 && n_past0 + t + 1 <= pmax) {
      const int C = std::min(std::min(BQ_MAX, T - 1 - t), pmax - (n_past0 + t));
      const int rc = prefill_launch(ctx, kv_cache, n_past0 + t, C, tokens + (size_t)t * row, st, false);
      if (rc != S2FAST_OK) return rc;
      t += C;
    }
  // the rest two positions a launch (one weight pass for both), the last
  // one with the head and the draw
  for (; t < T; t += MMAX) {
    const int M = std::min(MMAX, T - t);
    const int32_t* tk = tokens + (size_t)t * row;
    const int32_t* tk1 = tk + (size_t)(M - 1) * row;
    const int rc = slow_launch(ctx, kv_cache, n_past0 + t, M, tk, tk + 1, tk1, tk1 + 1, t + M == T ? 1 : 0, window,
                               u, temperature, top_p, top_k, main_out, sem_code_out, hidden_out, logits_out, st);
    if (rc != S2FAST_OK) return rc;
  }
  return S2FAST_OK;
}

int s2fast_test_slow_timeline(s2fast_slow_ctx* ctx, int32_t enable, uint32_t* host_out, int32_t capacity) {
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

int s2fast_full_frame(s2fast_slow_ctx* slow, s2fast_ctx* fast, void* kv_cache, int32_t n_past,
                      const int32_t* prev_main, const int32_t* prev_codes, int32_t* window, const float* u_slow,
                      const float* u_fast, const float* temperature, const float* top_p, const int32_t* top_k,
                      int32_t* main_out, float* hidden_out, int32_t* codes_out, void* stream) {
  if (!slow || !fast || !codes_out || !u_fast) return S2FAST_ERR_ARG;
  // the hidden state handed over must have the Fast-AR's input width
  // ("Fast-AR codebook decoding ...", section 1)
  if (fast->cfg.in_dim != slow->cfg.dim) return S2FAST_ERR_HIDDEN_DIM;
  if (fast->cfg.codebook_size != slow->cfg.codebook_size || fast->cfg.num_codebooks != slow->cfg.num_codebooks)
    return S2FAST_ERR_ARG;
  int rc = s2fast_slow_step(slow, kv_cache, n_past, prev_main, prev_codes, window, u_slow, temperature, top_p,
                            top_k, main_out, slow->sem, hidden_out, nullptr, stream);
  if (rc != S2FAST_OK) return rc;
  return s2fast_decode_frame(fast, 1, hidden_out, slow->sem, u_fast, temperature, top_p, top_k, codes_out, stream);
}

}  // extern "C"
