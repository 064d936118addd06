// Host side of the C ABI: validation, workspace layout, set-up tables and the
// launch sequence of each entry point. Everything after dflash_create is
// enqueued on the caller's stream with no host synchronisation.
#include "dflash.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "kernels.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

#define HIP_OK(expr)                                                                  \
  do {                                                                                \
    hipError_t e_ = (expr);                                                           \
    if (e_ != hipSuccess) return fail(DFLASH_ERR_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

constexpr int kAttnChunk = 128;   // context keys per attention work item
constexpr int kVerifyChunk = 8192;
constexpr int kKsMax = 8;

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct Layout {
  size_t alpha, rope, rowpos_a, rowseq_a, rowpos_d, rowseq_d, f, x, h, q, o, kblk, vblk, mm, gpart;
  size_t apo, aml, lmpart, vpart, vstate, counters, total;
  int n_ck, n_lm_wg, n_vchunks, m_max, rows_a_max;
};

Layout make_layout(const dflash_config& c) {
  Layout L{};
  const size_t H = c.hidden, D = c.n_layers, T = c.n_target_layers, N = c.block_size;
  const size_t qd = (size_t)c.n_q_heads * c.head_dim;
  const size_t Bm = c.max_batch;
  const size_t R = (size_t)(c.n_q_heads / c.n_kv_heads) * N;
  L.m_max = (int)(Bm * N);
  L.rows_a_max = (int)(Bm * c.max_new);
  L.n_ck = 1 + (c.max_pages_per_seq * 16 + kAttnChunk - 1) / kAttnChunk;
  L.n_lm_wg = (c.vocab / 32 + 3) / 4;
  L.n_vchunks = (c.vocab + kVerifyChunk - 1) / kVerifyChunk;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  L.alpha = take(D * T * 4);
  L.rope = take((size_t)c.max_pos * (c.head_dim / 2) * 2 * 4);
  L.rowpos_a = take(L.rows_a_max * 4);
  L.rowseq_a = take(L.rows_a_max * 4);
  L.rowpos_d = take(L.m_max * 4);
  L.rowseq_d = take(L.m_max * 4);
  L.f = take(D * L.rows_a_max * H * 2);
  L.x = take(L.m_max * H * 4);
  L.h = take(L.m_max * H * 2);
  L.q = take(L.m_max * qd * 2);
  L.o = take(L.m_max * qd * 2);
  L.kblk = take(Bm * c.n_kv_heads * 16 * c.head_dim * 2);
  L.vblk = take(Bm * c.n_kv_heads * 16 * c.head_dim * 2);
  L.mm = take((size_t)L.m_max * c.intermediate * 2);
  L.gpart = take((size_t)kKsMax * L.m_max * H * 4);
  L.apo = take(Bm * c.n_kv_heads * L.n_ck * R * c.head_dim * 4);
  L.aml = take(Bm * c.n_kv_heads * L.n_ck * R * 2 * 4);
  L.lmpart = take((size_t)L.n_lm_wg * L.m_max * sizeof(Top2));
  L.vpart = take(Bm * N * L.n_vchunks * 2 * 4);
  L.vstate = take(Bm * 2 * 4);
  L.counters = take(Bm * 2 * 4);
  L.total = off;
  return L;
}

int check_config(const dflash_config* c) {
  if (!c) return fail(DFLASH_ERR_INVALID_ARG, "config is null");
  if (c->hidden <= 0 || c->n_layers <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 || c->head_dim <= 0 ||
      c->intermediate <= 0 || c->vocab <= 0 || c->n_target_layers <= 0 || c->block_size <= 0 ||
      c->max_seqs <= 0 || c->max_pages_per_seq <= 0 || c->n_pages <= 0 || c->max_pos <= 0 ||
      c->max_batch <= 0 || c->max_new <= 0)
    return fail(DFLASH_ERR_INVALID_ARG, "config sizes must be positive");
  if (c->page_size != 16) return fail(DFLASH_ERR_UNSUPPORTED, "page_size must be 16 (got %d)", c->page_size);
  if (c->head_dim != 64 && c->head_dim != 128) return fail(DFLASH_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (c->hidden % 32 || c->hidden > 8192) return fail(DFLASH_ERR_UNSUPPORTED, "hidden must be a multiple of 32, <= 8192");
  if (c->intermediate % 32) return fail(DFLASH_ERR_UNSUPPORTED, "intermediate must be a multiple of 32");
  if (c->vocab % 32) return fail(DFLASH_ERR_UNSUPPORTED, "vocab must be a multiple of 32");
  if (c->n_q_heads % c->n_kv_heads) return fail(DFLASH_ERR_INVALID_ARG, "n_q_heads must be a multiple of n_kv_heads");
  if (c->block_size < 2 || c->block_size > 16) return fail(DFLASH_ERR_UNSUPPORTED, "block_size must be in [2, 16]");
  const int R = (c->n_q_heads / c->n_kv_heads) * c->block_size;
  if (R % 16 || R > 256)
    return fail(DFLASH_ERR_UNSUPPORTED, "(n_q/n_kv)*block_size must be a multiple of 16 and <= 256 (got %d)", R);
  if (c->mask_token_id < 0 || c->mask_token_id >= c->vocab) return fail(DFLASH_ERR_INVALID_ARG, "mask_token_id out of range");
  if (c->max_pos < c->block_size) return fail(DFLASH_ERR_INVALID_ARG, "max_pos too small");
  if (!(c->rms_eps > 0.f) || !(c->rope_theta > 1.f)) return fail(DFLASH_ERR_INVALID_ARG, "rms_eps > 0 and rope_theta > 1 required");
  return DFLASH_OK;
}

struct Timer {
  bool on = false;
  std::vector<hipEvent_t> ev;  // pairs (start, stop)
  size_t used = 0;             // events in use (2 per launch)
};

}  // namespace

struct dflash_ctx {
  dflash_config c;
  dflash_weights w;
  dflash_kv kv;
  char* ws;
  Layout L;
  Timer timers[DFLASH_K_COUNT];

  template <class T>
  T* at(size_t off) const { return reinterpret_cast<T*>(ws + off); }

  // Launch `fn` (returns hipError_t), with event records around it when
  // kind `kind` is being timed.
  template <class F>
  int launch(int kind, hipStream_t st, F fn) {
    Timer& t = timers[kind];
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (t.on) {
      if (t.used + 2 > 2 * 4096) return fail(DFLASH_ERR_CAPACITY, "kernel timer full: read it first");
      while (t.ev.size() < t.used + 2) {
        hipEvent_t e;
        HIP_OK(hipEventCreate(&e));
        t.ev.push_back(e);
      }
      e0 = t.ev[t.used];
      e1 = t.ev[t.used + 1];
      HIP_OK(hipEventRecord(e0, st));
    }
    hipError_t e = fn();
    if (e != hipSuccess) return fail(DFLASH_ERR_HIP, "kernel launch (kind %d): %s", kind, hipGetErrorString(e));
    if (t.on) {
      HIP_OK(hipEventRecord(e1, st));
      t.used += 2;
    }
    return DFLASH_OK;
  }

  GemmArgs gemm_base(int M, int K) const {
    GemmArgs g;
    std::memset(&g, 0, sizeof(g));
    g.K = K;
    g.M = M;
    g.ks = 1;
    g.head_dim = c.head_dim;
    g.n_kv = c.n_kv_heads;
    g.block = c.block_size;
    g.max_pages_per_seq = c.max_pages_per_seq;
    g.n_pages = c.n_pages;
    g.max_pos = c.max_pos;
    g.page_table = kv.page_table;
    g.kv_pages = kv.kv_pages;
    g.layer_stride = (long long)c.n_pages * 2 * c.n_kv_heads * 16 * c.head_dim;
    g.rope = c.use_rope ? at<float>(L.rope) : nullptr;
    return g;
  }
};

namespace {

void add_seg(GemmArgs& g, const uint16_t* w0, const uint16_t* w1, const uint16_t* act, void* out, int pairs,
             int mode, int epi, int layer) {
  GemmSeg& s = g.seg[g.nseg];
  s.w0 = w0;
  s.w1 = w1;
  s.act = act;
  s.out = out;
  s.pairs = pairs;
  s.mode = mode;
  s.epi = epi;
  s.layer = layer;
  g.seg_start[g.nseg + 1] = g.seg_start[g.nseg] + pairs;
  g.nseg++;
}

int total_pairs(const GemmArgs& g) { return g.seg_start[g.nseg]; }

// Workgroup count and k split for a launch: aim for >= 512 workgroups while
// every wave keeps >= 4 k-steps of 32.
int choose_ks(int pairs, int K, int kw, bool can_split) {
  int ks = 1;
  if (!can_split) return 1;
  while (pairs * ks < 512 && ks * 2 <= kKsMax && (K / 32) / (kw * ks * 2) >= 4) ks *= 2;
  return ks;
}

int gemm_kw(int pairs) { return pairs < 384 ? 8 : 4; }

}  // namespace

extern "C" {

const char* dflash_last_error(void) { return g_last_error.c_str(); }

size_t dflash_workspace_bytes(const dflash_config* cfg) {
  if (check_config(cfg) != DFLASH_OK) return 0;
  return make_layout(*cfg).total;
}

int dflash_create(const dflash_config* cfg, const dflash_weights* w, const dflash_kv* kv, void* workspace,
                  size_t ws_bytes, dflash_ctx** out) {
  if (!out) return fail(DFLASH_ERR_INVALID_ARG, "out is null");
  *out = nullptr;
  int rc = check_config(cfg);
  if (rc) return rc;
  if (!w || !kv || !workspace) return fail(DFLASH_ERR_INVALID_ARG, "weights, kv and workspace are required");
  const dflash_config& c = *cfg;
  if (!w->w_fuse || !w->g_fuse || !w->g_attn || !w->g_mlp || !w->g_final || !w->wq || !w->wk_d || !w->wv_d ||
      !w->wo || !w->wg || !w->wu || !w->wd || !w->embed || !w->lm_head)
    return fail(DFLASH_ERR_INVALID_ARG, "a weight pointer is null");
  if (!c.tied_kv && (!w->wk_t || !w->wv_t)) return fail(DFLASH_ERR_INVALID_ARG, "wk_t/wv_t required unless tied_kv");
  if (!kv->kv_pages || !kv->page_table || !kv->ctx_len || !kv->error_word)
    return fail(DFLASH_ERR_INVALID_ARG, "a kv pointer is null");
  const Layout L = make_layout(c);
  if (ws_bytes < L.total) return fail(DFLASH_ERR_CAPACITY, "workspace %zu bytes < required %zu", ws_bytes, L.total);

  // alpha^(i) = softmax over the T entries of w_fuse[i] (float64 on the host).
  std::vector<float> wf((size_t)c.n_layers * c.n_target_layers);
  HIP_OK(hipMemcpy(wf.data(), w->w_fuse, wf.size() * 4, hipMemcpyDeviceToHost));
  std::vector<float> alpha(wf.size());
  for (int i = 0; i < c.n_layers; ++i) {
    const float* row = &wf[(size_t)i * c.n_target_layers];
    double mx = -INFINITY;
    for (int j = 0; j < c.n_target_layers; ++j) mx = std::fmax(mx, (double)row[j]);
    double sum = 0;
    std::vector<double> e(c.n_target_layers);
    for (int j = 0; j < c.n_target_layers; ++j) sum += (e[j] = std::exp((double)row[j] - mx));
    for (int j = 0; j < c.n_target_layers; ++j) alpha[(size_t)i * c.n_target_layers + j] = (float)(e[j] / sum);
  }
  // RoPE: angle = pos * theta^(-2j/d_h) in float64, cos/sin rounded to fp32.
  const int half = c.head_dim / 2;
  std::vector<float> rope((size_t)c.max_pos * half * 2);
  for (int p = 0; p < c.max_pos; ++p)
    for (int j = 0; j < half; ++j) {
      const double inv = std::pow((double)c.rope_theta, -2.0 * j / c.head_dim);
      const double ang = (double)p * inv;
      rope[((size_t)p * half + j) * 2 + 0] = (float)std::cos(ang);
      rope[((size_t)p * half + j) * 2 + 1] = (float)std::sin(ang);
    }
  char* ws = static_cast<char*>(workspace);
  HIP_OK(hipMemcpy(ws + L.alpha, alpha.data(), alpha.size() * 4, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(ws + L.rope, rope.data(), rope.size() * 4, hipMemcpyHostToDevice));
  std::vector<int32_t> zeros((size_t)c.max_batch * 2, 0);
  HIP_OK(hipMemcpy(ws + L.counters, zeros.data(), zeros.size() * 4, hipMemcpyHostToDevice));

  dflash_ctx* ctx = new dflash_ctx();
  ctx->c = c;
  ctx->w = *w;
  if (c.tied_kv) {
    ctx->w.wk_t = w->wk_d;
    ctx->w.wv_t = w->wv_d;
  }
  ctx->kv = *kv;
  ctx->ws = ws;
  ctx->L = L;
  *out = ctx;
  return DFLASH_OK;
}

void dflash_destroy(dflash_ctx* ctx) {
  if (!ctx) return;
  for (auto& t : ctx->timers)
    for (hipEvent_t e : t.ev) (void)hipEventDestroy(e);
  delete ctx;
}

int dflash_ctx_append(dflash_ctx* ctx, int32_t B, const int32_t* seq_ids, const int32_t* n_new,
                      const uint16_t* target_hidden, int32_t max_new, hipStream_t stream) {
  if (!ctx) return fail(DFLASH_ERR_INVALID_ARG, "ctx is null");
  const dflash_config& c = ctx->c;
  if (B < 1 || B > c.max_batch) return fail(DFLASH_ERR_INVALID_ARG, "B=%d outside [1, max_batch=%d]", B, c.max_batch);
  if (max_new < 1 || max_new > c.max_new)
    return fail(DFLASH_ERR_INVALID_ARG, "max_new=%d outside [1, %d]", max_new, c.max_new);
  if (!seq_ids || !n_new || !target_hidden) return fail(DFLASH_ERR_INVALID_ARG, "null input pointer");
  const Layout& L = ctx->L;
  const int rows = B * max_new;
  const size_t H = c.hidden, kvd = (size_t)c.n_kv_heads * c.head_dim;
  int rc;

  PlanArgs pa{};
  pa.B = B;
  pa.rows_per_seq = max_new;
  pa.seq_ids = seq_ids;
  pa.n_new = n_new;
  pa.ctx_len = ctx->kv.ctx_len;
  pa.page_table = ctx->kv.page_table;
  pa.max_seqs = c.max_seqs;
  pa.max_pages_per_seq = c.max_pages_per_seq;
  pa.n_pages = c.n_pages;
  pa.max_pos = c.max_pos;
  pa.max_new = max_new;
  pa.vocab = c.vocab;
  pa.row_pos = ctx->at<int>(L.rowpos_a);
  pa.row_seq = ctx->at<int>(L.rowseq_a);
  pa.err = ctx->kv.error_word;
  pa.append = 1;
  if ((rc = ctx->launch(DFLASH_K_PLAN, stream, [&] { return dflash_launch_plan(&pa, stream); }))) return rc;

  FuseArgs fa{};
  fa.hidden = target_hidden;
  fa.alpha = ctx->at<float>(L.alpha);
  fa.g_fuse = ctx->w.g_fuse;
  fa.f = ctx->at<uint16_t>(L.f);
  fa.row_pos = pa.row_pos;
  fa.rows = rows;
  fa.T = c.n_target_layers;
  fa.H = c.hidden;
  fa.D = c.n_layers;
  fa.eps = c.rms_eps;
  if ((rc = ctx->launch(DFLASH_K_FUSE, stream, [&] { return dflash_launch_fuse(&fa, stream); }))) return rc;

  // Context K (RoPE pairs) and V of up to 8 layers per launch.
  for (int l0 = 0; l0 < c.n_layers; l0 += GEMM_MAX_SEG / 2) {
    GemmArgs g = ctx->gemm_base(rows, c.hidden);
    g.row_pos = pa.row_pos;
    g.row_seq = pa.row_seq;
    for (int i = l0; i < c.n_layers && i < l0 + GEMM_MAX_SEG / 2; ++i) {
      const uint16_t* act = ctx->at<uint16_t>(L.f) + (size_t)i * rows * H;
      add_seg(g, ctx->w.wk_t + (size_t)i * kvd * H, nullptr, act, nullptr, (int)(kvd / 32), PAIR_ROPE, EPI_CTX_K, i);
      add_seg(g, ctx->w.wv_t + (size_t)i * kvd * H, nullptr, act, nullptr, (int)(kvd / 32), PAIR_PLAIN, EPI_CTX_V, i);
    }
    const int kw = gemm_kw(total_pairs(g));
    if ((rc = ctx->launch(DFLASH_K_CTX_KV, stream, [&] { return dflash_launch_gemm(&g, total_pairs(g), kw, stream); })))
      return rc;
  }
  return DFLASH_OK;
}

int dflash_draft_block(dflash_ctx* ctx, int32_t B, const int32_t* seq_ids, const int32_t* anchor, int32_t* draft,
                       float* top2_gap, float* dbg_hidden, float* dbg_logits, hipStream_t stream) {
  if (!ctx) return fail(DFLASH_ERR_INVALID_ARG, "ctx is null");
  const dflash_config& c = ctx->c;
  if (B < 1 || B > c.max_batch) return fail(DFLASH_ERR_INVALID_ARG, "B=%d outside [1, max_batch=%d]", B, c.max_batch);
  if (!seq_ids || !anchor || !draft) return fail(DFLASH_ERR_INVALID_ARG, "null input/output pointer");
  const Layout& L = ctx->L;
  const int N = c.block_size, M = B * N;
  const size_t H = c.hidden, I = c.intermediate, qd = (size_t)c.n_q_heads * c.head_dim;
  const size_t kvd = (size_t)c.n_kv_heads * c.head_dim;
  int rc;

  PlanArgs pa{};
  pa.B = B;
  pa.rows_per_seq = N;
  pa.seq_ids = seq_ids;
  pa.anchor = anchor;
  pa.ctx_len = ctx->kv.ctx_len;
  pa.page_table = ctx->kv.page_table;
  pa.max_seqs = c.max_seqs;
  pa.max_pages_per_seq = c.max_pages_per_seq;
  pa.n_pages = c.n_pages;
  pa.max_pos = c.max_pos;
  pa.max_new = c.max_new;
  pa.vocab = c.vocab;
  pa.row_pos = ctx->at<int>(L.rowpos_d);
  pa.row_seq = ctx->at<int>(L.rowseq_d);
  pa.err = ctx->kv.error_word;
  pa.append = 0;
  if ((rc = ctx->launch(DFLASH_K_PLAN, stream, [&] { return dflash_launch_plan(&pa, stream); }))) return rc;

  float* x = ctx->at<float>(L.x);
  uint16_t* h = ctx->at<uint16_t>(L.h);
  float* gpart = ctx->at<float>(L.gpart);

  NormArgs na{};
  na.mode = 0;
  na.embed = ctx->w.embed;
  na.anchor = anchor;
  na.mask_id = c.mask_token_id;
  na.N = N;
  na.V = c.vocab;
  na.x = x;
  na.part = gpart;
  na.ks = 0;
  na.g = ctx->w.g_attn;
  na.h = h;
  na.dbg = dbg_hidden;
  na.H = c.hidden;
  na.M = M;
  na.eps = c.rms_eps;
  if ((rc = ctx->launch(DFLASH_K_NORM, stream, [&] { return dflash_launch_norm(&na, stream); }))) return rc;

  AttnArgs aa{};
  aa.q = ctx->at<uint16_t>(L.q);
  aa.kblk = ctx->at<uint16_t>(L.kblk);
  aa.vblk = ctx->at<uint16_t>(L.vblk);
  aa.page_table = ctx->kv.page_table;
  aa.ctx_len = ctx->kv.ctx_len;
  aa.seq_ids = seq_ids;
  aa.part_o = ctx->at<float>(L.apo);
  aa.part_ml = ctx->at<float>(L.aml);
  aa.o = ctx->at<uint16_t>(L.o);
  aa.N = N;
  aa.n_q = c.n_q_heads;
  aa.n_kv = c.n_kv_heads;
  aa.chunk = kAttnChunk;
  aa.n_ck = L.n_ck;
  aa.max_pages_per_seq = c.max_pages_per_seq;
  aa.n_pages = c.n_pages;
  aa.max_seqs = c.max_seqs;
  aa.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)c.head_dim));
  const long long layer_stride = (long long)c.n_pages * 2 * c.n_kv_heads * 16 * c.head_dim;

  for (int i = 0; i < c.n_layers; ++i) {
    {  // Q, block K (RoPE) and block V
      GemmArgs g = ctx->gemm_base(M, c.hidden);
      g.row_pos = pa.row_pos;
      g.row_seq = pa.row_seq;
      g.n_out = (int)qd;
      add_seg(g, ctx->w.wq + (size_t)i * qd * H, nullptr, h, ctx->at<uint16_t>(L.q), (int)(qd / 32), PAIR_ROPE,
              EPI_Q, i);
      add_seg(g, ctx->w.wk_d + (size_t)i * kvd * H, nullptr, h, ctx->at<uint16_t>(L.kblk), (int)(kvd / 32),
              PAIR_ROPE, EPI_KBLK, i);
      add_seg(g, ctx->w.wv_d + (size_t)i * kvd * H, nullptr, h, ctx->at<uint16_t>(L.vblk), (int)(kvd / 32),
              PAIR_PLAIN, EPI_VBLK, i);
      const int kw = gemm_kw(total_pairs(g));
      if ((rc = ctx->launch(DFLASH_K_QKV, stream, [&] { return dflash_launch_gemm(&g, total_pairs(g), kw, stream); })))
        return rc;
    }
    aa.pages = ctx->kv.kv_pages + (size_t)i * layer_stride;
    if ((rc = ctx->launch(DFLASH_K_ATTN, stream, [&] { return dflash_launch_attn(&aa, B, c.head_dim, stream); })))
      return rc;
    if ((rc = ctx->launch(DFLASH_K_ATTN_MERGE, stream,
                          [&] { return dflash_launch_attn_merge(&aa, B, c.head_dim, stream); })))
      return rc;
    int ks_o;
    {  // O projection -> split partials
      GemmArgs g = ctx->gemm_base(M, (int)qd);
      g.n_out = c.hidden;
      add_seg(g, ctx->w.wo + (size_t)i * H * qd, nullptr, aa.o, gpart, c.hidden / 32, PAIR_PLAIN, EPI_PARTIAL, i);
      const int kw = gemm_kw(total_pairs(g));
      g.ks = ks_o = choose_ks(total_pairs(g), (int)qd, kw, true);
      if ((rc = ctx->launch(DFLASH_K_OPROJ, stream, [&] { return dflash_launch_gemm(&g, total_pairs(g), kw, stream); })))
        return rc;
    }
    na.mode = 1;
    na.ks = ks_o;
    na.g = ctx->w.g_mlp + (size_t)i * H;
    na.dbg = nullptr;
    if ((rc = ctx->launch(DFLASH_K_NORM, stream, [&] { return dflash_launch_norm(&na, stream); }))) return rc;
    {  // gate/up + SwiGLU
      GemmArgs g = ctx->gemm_base(M, c.hidden);
      g.n_out = (int)I;
      add_seg(g, ctx->w.wg + (size_t)i * I * H, ctx->w.wu + (size_t)i * I * H, h, ctx->at<uint16_t>(L.mm),
              (int)(I / 16), PAIR_DUAL, EPI_SWIGLU, i);
      const int kw = gemm_kw(total_pairs(g));
      if ((rc = ctx->launch(DFLASH_K_GATE_UP, stream,
                            [&] { return dflash_launch_gemm(&g, total_pairs(g), kw, stream); })))
        return rc;
    }
    int ks_d;
    {  // down -> split partials
      GemmArgs g = ctx->gemm_base(M, (int)I);
      g.n_out = c.hidden;
      add_seg(g, ctx->w.wd + (size_t)i * H * I, nullptr, ctx->at<uint16_t>(L.mm), gpart, c.hidden / 32, PAIR_PLAIN,
              EPI_PARTIAL, i);
      const int kw = gemm_kw(total_pairs(g));
      g.ks = ks_d = choose_ks(total_pairs(g), (int)I, kw, true);
      if ((rc = ctx->launch(DFLASH_K_DOWN, stream, [&] { return dflash_launch_gemm(&g, total_pairs(g), kw, stream); })))
        return rc;
    }
    na.mode = 1;
    na.ks = ks_d;
    na.g = (i + 1 < c.n_layers) ? ctx->w.g_attn + (size_t)(i + 1) * H : ctx->w.g_final;
    na.dbg = dbg_hidden ? dbg_hidden + (size_t)(i + 1) * M * H : nullptr;
    if ((rc = ctx->launch(DFLASH_K_NORM, stream, [&] { return dflash_launch_norm(&na, stream); }))) return rc;
  }

  LmArgs la{};
  la.w = ctx->w.lm_head;
  la.act = h;
  la.M = M;
  la.K = c.hidden;
  la.V = c.vocab;
  la.N = N;
  la.part = ctx->at<Top2>(L.lmpart);
  la.dbg_logits = dbg_logits;
  if ((rc = ctx->launch(DFLASH_K_LM_HEAD, stream, [&] { return dflash_launch_lmhead(&la, stream); }))) return rc;

  ArgmaxArgs ma{};
  ma.part = la.part;
  ma.n_wg = L.n_lm_wg;
  ma.M = M;
  ma.N = N;
  ma.V = c.vocab;
  ma.draft = draft;
  ma.gap = top2_gap;
  ma.err = ctx->kv.error_word;
  return ctx->launch(DFLASH_K_ARGMAX, stream, [&] { return dflash_launch_argmax(&ma, stream); });
}

int dflash_verify(dflash_ctx* ctx, int32_t B, const int32_t* seq_ids, const int32_t* draft, const void* target_logits,
                  int32_t logits_dtype, float temperature, uint64_t seed, uint64_t step, int32_t* accept_len,
                  int32_t* next_token, int32_t* commit_len, hipStream_t stream) {
  if (!ctx) return fail(DFLASH_ERR_INVALID_ARG, "ctx is null");
  const dflash_config& c = ctx->c;
  if (B < 1 || B > c.max_batch) return fail(DFLASH_ERR_INVALID_ARG, "B=%d outside [1, max_batch=%d]", B, c.max_batch);
  if (!seq_ids || !draft || !target_logits || !accept_len || !next_token)
    return fail(DFLASH_ERR_INVALID_ARG, "null input/output pointer");
  if (logits_dtype != DFLASH_DTYPE_BF16 && logits_dtype != DFLASH_DTYPE_F32)
    return fail(DFLASH_ERR_INVALID_ARG, "logits_dtype must be DFLASH_DTYPE_BF16 or DFLASH_DTYPE_F32");
  if (temperature != 0.f && temperature != 1.f)
    return fail(DFLASH_ERR_UNSUPPORTED, "temperature must be 0 (greedy) or 1");
  const Layout& L = ctx->L;
  VerifyArgs va{};
  va.logits = target_logits;
  va.dtype = logits_dtype;
  va.B = B;
  va.N = c.block_size;
  va.V = c.vocab;
  va.chunk = kVerifyChunk;
  va.n_chunks = L.n_vchunks;
  va.seq_ids = seq_ids;
  va.draft = draft;
  va.part = ctx->at<float>(L.vpart);
  va.counters = ctx->at<int>(L.counters);
  va.state = ctx->at<int>(L.vstate);
  va.accept_len = accept_len;
  va.next_token = next_token;
  va.commit_len = commit_len;
  va.temp1 = temperature == 1.f;
  va.seed = seed;
  va.step = step;
  va.err = ctx->kv.error_word;
  return ctx->launch(DFLASH_K_VERIFY, stream, [&] { return dflash_launch_verify(&va, stream); });
}

int dflash_read_error(dflash_ctx* ctx, hipStream_t stream, int32_t* out) {
  if (!ctx || !out) return fail(DFLASH_ERR_INVALID_ARG, "ctx and out are required");
  HIP_OK(hipStreamSynchronize(stream));
  int32_t v = 0;
  HIP_OK(hipMemcpy(&v, ctx->kv.error_word, 4, hipMemcpyDeviceToHost));
  const int32_t z = 0;
  HIP_OK(hipMemcpy(ctx->kv.error_word, &z, 4, hipMemcpyHostToDevice));
  *out = v;
  return DFLASH_OK;
}

int dflash_kernel_timer(dflash_ctx* ctx, int32_t kind, int32_t enable) {
  if (!ctx || kind < 0 || kind >= DFLASH_K_COUNT) return fail(DFLASH_ERR_INVALID_ARG, "bad ctx or kernel kind");
  ctx->timers[kind].on = enable != 0;
  if (enable) ctx->timers[kind].used = 0;
  return DFLASH_OK;
}

int dflash_kernel_timer_read(dflash_ctx* ctx, int32_t kind, double* total_ms, int64_t* launches) {
  if (!ctx || kind < 0 || kind >= DFLASH_K_COUNT || !total_ms || !launches)
    return fail(DFLASH_ERR_INVALID_ARG, "bad arguments");
  Timer& t = ctx->timers[kind];
  double tot = 0;
  for (size_t i = 0; i + 1 < t.used; i += 2) {
    HIP_OK(hipEventSynchronize(t.ev[i + 1]));
    float ms = 0.f;
    HIP_OK(hipEventElapsedTime(&ms, t.ev[i], t.ev[i + 1]));
    tot += ms;
  }
  *total_ms = tot;
  *launches = (int64_t)(t.used / 2);
  t.used = 0;
  return DFLASH_OK;
}

}  // extern "C"
