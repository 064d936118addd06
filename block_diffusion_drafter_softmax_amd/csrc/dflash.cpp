// Host side of the C ABI: validation, workspace layout, set-up (fusion
// weights, RoPE table, weight packing) and the launch sequence of each entry
// point. Everything after dflash_create is enqueued on the caller's stream
// with no host synchronisation.
#include "dflash.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "kernels.h"

thread_local LaunchEvents dflash_launch_events = {nullptr, nullptr};

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

#define HIP_OK(expr)                                                                               \
  do {                                                                                             \
    hipError_t e_ = (expr);                                                                        \
    if (e_ != hipSuccess) return fail(DFLASH_ERR_HIP, "%s: %s", #expr, hipGetErrorString(e_));     \
  } while (0)

constexpr int kAttnChunk = 128;     // context keys per attention chunk
constexpr int kAttnItems = 512;     // attention work items to aim for (two 8-wave workgroups fit a CU: about one
                                    // round of the chip); larger grids take several chunks per item
constexpr int kAttnMaxWaves = 8;    // computing waves of an attention workgroup that takes several blocks of one
                                    // sequence: only the staging-only waves of an 8-wave workgroup are filled (larger
                                    // workgroups were slower: the attention is bound by its compute phase)
constexpr int kVerifyChunk = 32768;       // logits per verification work item (rows pass)
constexpr int kSampleChunkMin = 1024;     // logits per work item of a sampling pass, at least (and a multiple of)
constexpr int kSampleWgs = 512;           // sampling work items to aim for (a batch-1 row still fills the chip)
constexpr int kKsMax = 8;           // largest k split of a streaming GEMM (KS_MAX in common.h)
constexpr int kTargetWaves = 1536;  // streaming waves to aim for (~6 per CU)
constexpr int kMmMinRows = 64;      // from this many activation rows on, GEMMs use the tiled MFMA kernels
constexpr int kMmCols = MM_COL_TILES * 16;  // output columns (vocabulary rows) per tiled-GEMM workgroup
constexpr int kMmRows = MM_ROW_TILES * 16;  // activation rows per tiled-GEMM workgroup
constexpr int kMmTargetWgs = 256;   // tiled-GEMM workgroups to aim for before splitting k (one per CU; more splits cost
                                    // partial-sum traffic in the GEMM and its consumer)
// Partial-sum floats a tiled GEMM may need: a k split is only taken while
// the grid is under 2 * kMmTargetWgs workgroup tiles.
constexpr size_t kMmPartFloats = (size_t)2 * kMmTargetWgs * kMmRows * kMmCols;

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Logits per work item of a sampling pass over `rows` vocabulary rows: about
// kSampleWgs work items, chunks a multiple of kSampleChunkMin.
int sample_chunk(int vocab, long long rows) {
  long long c = (long long)vocab * rows / kSampleWgs;
  c = (c + kSampleChunkMin - 1) / kSampleChunkMin * kSampleChunkMin;
  return (int)std::max<long long>(kSampleChunkMin, std::min<long long>(c, ((long long)vocab + kSampleChunkMin - 1) /
                                                                            kSampleChunkMin * kSampleChunkMin));
}

// Partial top-2 per row that the LM head leaves for the argmax reduction:
// one per 512 vocabulary rows (tiled, many rows) or per 64 (streaming).
int lm_parts(int vocab, int M) { return M >= kMmMinRows ? (vocab + 2 * kMmCols - 1) / (2 * kMmCols) : (vocab / 32 + 1) / 2; }

// Byte offsets of everything the library keeps in the caller's workspace.
struct Layout {
  // set-up tables and packed weights
  size_t alpha, rope, wq, wk_d, wv_d, wk_t, wv_t, wo, wg, wu, wd, lm, wfc;
  // per-call buffers
  size_t rowpos_a, rowseq_a, f, fraw, x, h, q, o, kblk, vblk, mm, gpart, cpart;
  size_t apo, aml, lmpart, vpart, spart, total;
  // dual-pass drafting: second-pass sequences and input blocks, first and
  // second drafts, confidence, cut points; multi-candidate verification
  size_t d_seq, d_tok, d_draft1, d_draft2, d_conf, d_cuts, v_acc, v_next;
  // sampled drafts: drafter rows pass, draft sampling partials
  size_t qpart, dpart;
  // a draft call's plan: per block (sequence, context length), per row RoPE cos/sin
  size_t plan, plan_rope;
  // and each block's page-table row, read by the attention with the plan
  size_t blk_pages;
  // compacted LM-head rows of a dual-pass second pass: block row of each, count
  size_t lm_inv, lm_count, attn_ctr;
  size_t gpart_floats, cpart_floats;
  int n_ck, n_vchunks, n_schunks, m_max, rows_a_max;
};

Layout make_layout(const dflash_config& c) {
  Layout L{};
  const size_t H = c.hidden, D = c.n_layers, T = c.n_target_layers, N = c.block_size, I = c.intermediate;
  const size_t qd = (size_t)c.n_q_heads * c.head_dim, kvd = (size_t)c.n_kv_heads * c.head_dim;
  const size_t Bm = c.max_batch;
  const size_t R = (size_t)(c.n_q_heads / c.n_kv_heads) * N;
  L.m_max = (int)(Bm * N);
  L.rows_a_max = (int)(Bm * c.max_new);
  const size_t mp = pad16(L.m_max), rp = pad16(L.rows_a_max);
  L.n_ck = 1 + (c.max_pages_per_seq * 16 + kAttnChunk - 1) / kAttnChunk;  // the block's keys, then context chunks
  L.n_vchunks = (c.vocab + kVerifyChunk - 1) / kVerifyChunk;
  L.n_schunks = (c.vocab + kSampleChunkMin - 1) / kSampleChunkMin;  // the most chunks a sampling pass uses
  const size_t ncol_d = std::max(qd + 2 * kvd, H), ncol_c = D * 2 * kvd;
  L.gpart_floats = std::max(ncol_d * std::max<size_t>(256, 2 * (size_t)L.m_max), kMmPartFloats);
  L.cpart_floats = std::max(ncol_c * std::max<size_t>(256, 2 * (size_t)L.rows_a_max), kMmPartFloats);
  const bool fc = c.fusion == DFLASH_FUSION_FC;
  if (fc)  // the FC fusion layer's partials [ks][rows][H] share this buffer
    L.cpart_floats = std::max(L.cpart_floats, H * std::max<size_t>(256, 2 * (size_t)L.rows_a_max));

  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  L.alpha = take(D * T * 4);
  L.rope = take((size_t)c.max_pos * (c.head_dim / 2) * 2 * 4);
  L.wq = take(D * qd * H * 2);
  L.wk_d = take(D * kvd * H * 2);
  L.wv_d = take(D * kvd * H * 2);
  L.wk_t = c.tied_kv ? L.wk_d : take(D * kvd * H * 2);
  L.wv_t = c.tied_kv ? L.wv_d : take(D * kvd * H * 2);
  L.wo = take(D * H * qd * 2);
  L.wg = take(D * I * H * 2);
  L.wu = take(D * I * H * 2);
  L.wd = take(D * H * I * 2);
  L.lm = take((size_t)c.vocab * H * 2);
  L.wfc = fc ? take(H * T * H * 2) : 0;
  L.rowpos_a = take(L.rows_a_max * 4);
  L.rowseq_a = take(L.rows_a_max * 4);
  // activations are split hi/lo bf16 pairs: two planes each (FC fusion: one
  // shared context instead of D, and the FC layer's [rows][T*H] input)
  L.f = take((fc ? 1 : D) * 2 * rp * H * 2);
  L.fraw = fc ? take(2 * rp * T * H * 2) : 0;
  L.x = take(L.m_max * H * 4);
  L.h = take(2 * mp * H * 2);
  L.q = take(2 * L.m_max * qd * 2);
  L.o = take(2 * mp * qd * 2);
  L.kblk = take(Bm * kvd * 16 * 2);
  L.vblk = take(Bm * kvd * 16 * 2);
  L.mm = take(2 * mp * I * 2);
  L.gpart = take(L.gpart_floats * 4);
  L.cpart = take(L.cpart_floats * 4);
  L.apo = take(Bm * c.n_kv_heads * L.n_ck * R * c.head_dim * 4);
  L.aml = take(Bm * c.n_kv_heads * L.n_ck * R * 2 * 4);
  L.lmpart = take((size_t)std::max(lm_parts(c.vocab, 1), lm_parts(c.vocab, kMmMinRows)) * L.m_max * sizeof(Top2));
  L.vpart = take(Bm * N * L.n_vchunks * 2 * 4);
  L.spart = take(Bm * L.n_schunks * 2 * 4);
  L.d_seq = take(Bm * 4);
  L.d_tok = take(Bm * N * 4);
  L.d_draft1 = take(Bm * N * 4);
  L.d_draft2 = take(Bm * N * 4);
  L.d_conf = take(Bm * N * 4);
  L.d_cuts = take(Bm * N * 4);
  L.v_acc = take(Bm * 4);
  L.v_next = take(Bm * 4);
  L.qpart = take(Bm * N * L.n_vchunks * 2 * 4);
  L.dpart = take(Bm * N * L.n_schunks * 2 * 4);
  L.plan = take(Bm * 2 * 4);
  L.plan_rope = take(Bm * N * (c.head_dim / 2) * 2 * 4);
  L.blk_pages = take((size_t)Bm * c.max_pages_per_seq * 4);
  L.lm_inv = take(Bm * N * 4);
  L.lm_count = take(4);
  L.attn_ctr = take(8 * 4);
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
  if (c->hidden % 32 || c->hidden > 8192)
    return fail(DFLASH_ERR_UNSUPPORTED, "hidden must be a multiple of 32, <= 8192");
  if (c->intermediate % 32) return fail(DFLASH_ERR_UNSUPPORTED, "intermediate must be a multiple of 32");
  if (c->vocab % 32) return fail(DFLASH_ERR_UNSUPPORTED, "vocab must be a multiple of 32");
  if (c->n_q_heads % c->n_kv_heads) return fail(DFLASH_ERR_INVALID_ARG, "n_q_heads must be a multiple of n_kv_heads");
  if (c->n_target_layers > 16) return fail(DFLASH_ERR_UNSUPPORTED, "n_target_layers must be <= 16");
  if (c->n_layers > 64) return fail(DFLASH_ERR_UNSUPPORTED, "n_layers must be <= 64");
  if (c->block_size < 2 || c->block_size > 16) return fail(DFLASH_ERR_UNSUPPORTED, "block_size must be in [2, 16]");
  const int R = (c->n_q_heads / c->n_kv_heads) * c->block_size;
  if (R % 16 || R > 256)
    return fail(DFLASH_ERR_UNSUPPORTED, "(n_q/n_kv)*block_size must be a multiple of 16 and <= 256 (got %d)", R);
  if ((long long)c->block_size * ((c->vocab + kVerifyChunk - 1) / kVerifyChunk) > VERIFY_MAX_PARTS)
    return fail(DFLASH_ERR_UNSUPPORTED, "block_size * ceil(vocab / %d) must be <= %d", kVerifyChunk, VERIFY_MAX_PARTS);
  if (c->mask_token_id < 0 || c->mask_token_id >= c->vocab)
    return fail(DFLASH_ERR_INVALID_ARG, "mask_token_id out of range");
  if (c->max_pos < c->block_size) return fail(DFLASH_ERR_INVALID_ARG, "max_pos too small");
  if (c->fusion != DFLASH_FUSION_SOFTMAX && c->fusion != DFLASH_FUSION_FC)
    return fail(DFLASH_ERR_INVALID_ARG, "fusion must be DFLASH_FUSION_SOFTMAX or DFLASH_FUSION_FC");
  if (!(c->rms_eps > 0.f) || !(c->rope_theta > 1.f))
    return fail(DFLASH_ERR_INVALID_ARG, "rms_eps > 0 and rope_theta > 1 required");
  return DFLASH_OK;
}

constexpr size_t kTimerCap = 4096;  // timed launches between reads

struct Timer {
  bool on = false;
  std::vector<hipEvent_t> ev;  // pairs (start, stop)
  size_t used = 0;             // launches timed
};

}  // namespace

struct dflash_ctx {
  int device;  // the GPU current at dflash_create
  dflash_config c;
  dflash_weights w;
  dflash_kv kv;
  char* ws;
  Layout L;
  Timer timers[DFLASH_K_COUNT];

  template <class T>
  T* at(size_t off) const { return reinterpret_cast<T*>(ws + off); }

  // Launch `fn` (returns hipError_t). When kind `kind` is being timed, a
  // single-kernel launcher records the kernel's own start/end into a pair
  // of events (dflash_launch_events); verification, which may launch two
  // kernels, gets event records around the launcher instead.
  template <class F>
  int launch(int kind, hipStream_t st, F fn) {
    Timer& t = timers[kind];
    hipEvent_t e0 = nullptr, e1 = nullptr;
    const bool around = kind == DFLASH_K_VERIFY;
    if (t.on) {
      if (t.used >= kTimerCap) return fail(DFLASH_ERR_CAPACITY, "kernel timer full: read it first");
      while (t.ev.size() < 2 * t.used + 2) {
        hipEvent_t e;
        HIP_OK(hipEventCreate(&e));
        t.ev.push_back(e);
      }
      e0 = t.ev[2 * t.used];
      e1 = t.ev[2 * t.used + 1];
      if (around) HIP_OK(hipEventRecord(e0, st));
      else dflash_launch_events = LaunchEvents{e0, e1};
    }
    hipError_t e = fn();
    dflash_launch_events = LaunchEvents{nullptr, nullptr};
    if (e != hipSuccess) return fail(DFLASH_ERR_HIP, "kernel launch (kind %d): %s", kind, hipGetErrorString(e));
    if (t.on) {
      if (around) HIP_OK(hipEventRecord(e1, st));
      t.used += 1;
    }
    return DFLASH_OK;
  }
};

namespace {

void add_seg(WsArgs& a, const uint16_t* w0, const uint16_t* w1, const uint16_t* act, int units, int col0) {
  WsSeg& s = a.seg[a.nseg];
  s.w0 = w0;
  s.w1 = w1;
  s.act = act;
  s.units = units;
  s.col0 = col0;
  a.unit_start[a.nseg + 1] = a.unit_start[a.nseg] + units;
  a.nseg++;
}

WsArgs ws_base(int M, int K, int n_cols) {
  WsArgs a;
  std::memset(&a, 0, sizeof(a));
  a.M = M;
  a.K = K;
  a.ks = 1;
  a.n_cols = n_cols;
  return a;
}

// k split of a streaming GEMM: enough waves to keep ~6 per CU streaming, at
// least 8 k steps per wave, and within the partial buffer.
int pick_ks(int units, int K, int M, int n_cols, size_t cap_floats) {
  int ks = (kTargetWaves + units - 1) / units;
  ks = std::min(ks, std::max(1, (K / 32) / 8));
  ks = std::min(ks, kKsMax);
  ks = std::min<long long>(ks, (long long)(cap_floats / ((size_t)M * n_cols)));
  return std::max(ks, 1);
}

// Few rows: the weight-streaming GEMM with a k split (none for SwiGLU).
// Many rows: the tiled MFMA GEMM (sets g.mm_xt / g.mm_wt, returns the k
// split). By default the 4-wave loop: 128-row tiles while they give every
// CU two workgroups, else 64-row tiles (three fit a CU), then a k split
// while the grid is under its target. The 8-wave loop (one workgroup per
// CU, three LDS stages; 128-row tiles 256, 384 or 512 weight rows wide)
// replaces it where one of its tile widths and k splits fills at least
// three quarters of every round of the chip with k loops of 32 steps or
// more, and is estimated faster. The
// estimate: rounds of the chip times the busiest CU's share of a round
// (workgroups held at once times a tile of work, at the fraction of the
// MFMA rate measured for that loop and occupancy), plus the partial sums a
// k split writes and its consumer reads again.
int gemm_ks(WsArgs& g, int mode, size_t cap_floats) {
  const int units = g.unit_start[g.nseg];
  g.mm_wt = 0;
  if (g.M < kMmMinRows) return mode == WS_SWIGLU ? 1 : pick_ks(units, g.K, g.M, g.n_cols, cap_floats);
  const int m_tiles = pad16(g.M) / 16, steps = g.K / 32;
  const size_t part_cols = (size_t)g.n_cols * (mode == WS_SWIGLU ? 2 : 1);
  const double tile_step_us = 16.0 * 16 * 32 * 2 * 2 / 9.77e6;  // one 16x16x32 hi+lo tile step of a CU at its MFMA peak
  auto col_blocks = [&](int wt) {
    int cb = 0;
    for (int s = 0; s < g.nseg; ++s) cb += (2 * g.seg[s].units + wt - 1) / wt;
    return cb;
  };
  auto ks_cap = [&](int ks) {  // at least 8 k steps per split, within the partial buffer
    ks = std::min(ks, std::max(1, steps / 8));
    ks = std::min(ks, kKsMax);
    ks = std::min<long long>(ks, (long long)(cap_floats / ((size_t)g.M * part_cols)));
    return std::max(ks, 1);
  };
  // measured fraction of the MFMA rate: 4-wave loop by workgroups held per CU
  // (128-row tiles: 1, 2; 64-row tiles: 1, 2, 3), 8-wave loop
  auto eff4 = [](int xt, long long held) {
    if (xt == MM_ROW_TILES) return held >= 2 ? 0.55 : 0.38;
    return held >= 3 ? 0.48 : held == 2 ? 0.45 : 0.33;
  };
  constexpr double kEff8 = 0.52;
  auto estimate = [&](int xt, int wt, int per_cu, long long held, double eff, long long wgs, int ks) {
    const long long rounds = (wgs + 256LL * per_cu - 1) / (256LL * per_cu);
    return rounds * held * (double)xt * wt * ((steps + ks - 1) / ks) * tile_step_us / eff +
           (ks > 1 ? 2.0 * ks * g.M * part_cols * 4 / 6e6 : 0.0);
  };
  // the default plan
  const int cb16 = col_blocks(MM_COL_TILES);
  const int full = cb16 * ((m_tiles + MM_ROW_TILES - 1) / MM_ROW_TILES);
  g.mm_xt = full >= 2 * kMmTargetWgs ? MM_ROW_TILES : MM_ROW_TILES / 2;
  const int blocks = cb16 * ((m_tiles + g.mm_xt - 1) / g.mm_xt);
  const int target = g.mm_xt == MM_ROW_TILES ? kMmTargetWgs : 2 * kMmTargetWgs;
  const int ks = ks_cap((target + blocks - 1) / blocks);  // a split SwiGLU product is finished by swiglu_finish
  {
    const long long wgs = (long long)blocks * ks;
    const int per_cu = g.mm_xt == MM_ROW_TILES ? 2 : 3;
    const long long held = std::min<long long>(per_cu, (wgs + 255) / 256);
    const double base = estimate(g.mm_xt, MM_COL_TILES, per_cu, held, eff4(g.mm_xt, held), wgs, ks);
    double best = base;
    int best_wt = 0, best_ks = ks;
    for (int wt : {16, 24, 32}) {
      const int b8 = col_blocks(wt) * ((m_tiles + MM_ROW_TILES - 1) / MM_ROW_TILES);
      for (int k8 = 1; k8 <= kKsMax; ++k8) {
        if (k8 != ks_cap(k8)) break;
        const long long w8 = (long long)b8 * k8;
        const long long r8 = (w8 + 255) / 256;
        if (w8 * 4 < r8 * 256 * 3) continue;  // at least three quarters of every round
        if (steps / k8 < 32) break;          // the three-stage ring needs a long k loop to pay for its fill
        const double e = estimate(MM_ROW_TILES, wt, 1, 1, kEff8, w8, k8);
        if (e < best) {
          best = e;
          best_wt = wt;
          best_ks = k8;
        }
      }
    }
    if (best_wt) {
      g.mm_xt = MM_ROW_TILES;
      g.mm_wt = best_wt;
      return best_ks;
    }
  }
  return ks;
}

hipError_t launch_gemm(const WsArgs& g, int mode, hipStream_t st) {
  return g.M >= kMmMinRows ? dflash_launch_mm(&g, mode, st) : dflash_launch_ws(&g, mode, st);
}


// ------------------------------------------------------------ context append

// An append's launch arguments: the fusion (and its plan) and the context
// finisher (k split set by append_kv); rows = B * max_new.
struct AppendCall {
  FuseArgs fa;
  CtxFinishArgs ca;
  int rows;
};

int append_check(dflash_ctx* ctx, int32_t B, const int32_t* seq_ids, const int32_t* n_new,
                 const uint16_t* target_hidden, int32_t max_new) {
  if (!ctx) return fail(DFLASH_ERR_INVALID_ARG, "ctx is null");
  const dflash_config& c = ctx->c;
  if (B < 1 || B > c.max_batch) return fail(DFLASH_ERR_INVALID_ARG, "B=%d outside [1, max_batch=%d]", B, c.max_batch);
  if (max_new < 1 || max_new > c.max_new)
    return fail(DFLASH_ERR_INVALID_ARG, "max_new=%d outside [1, %d]", max_new, c.max_new);
  if (!seq_ids || !n_new || !target_hidden) return fail(DFLASH_ERR_INVALID_ARG, "null input pointer");
  return DFLASH_OK;
}

AppendCall append_args(dflash_ctx* ctx, int32_t B, const int32_t* seq_ids, const int32_t* n_new,
                       const uint16_t* target_hidden, int32_t max_new) {
  const dflash_config& c = ctx->c;
  const Layout& L = ctx->L;
  const int rows = B * max_new;
  const int H = c.hidden, D = c.n_layers, kvd = c.n_kv_heads * c.head_dim;
  AppendCall ap{};
  ap.rows = rows;
  FuseArgs& fa = ap.fa;
  fa.hidden = target_hidden;
  fa.alpha = ctx->at<float>(L.alpha);
  fa.g_fuse = ctx->w.g_fuse;
  fa.f = ctx->at<uint16_t>(L.f);
  fa.B = B;
  fa.max_new = max_new;
  fa.seq_ids = seq_ids;
  fa.n_new = n_new;
  fa.ctx_len = ctx->kv.ctx_len;
  fa.page_table = ctx->kv.page_table;
  fa.max_seqs = c.max_seqs;
  fa.max_pages_per_seq = c.max_pages_per_seq;
  fa.n_pages = c.n_pages;
  fa.max_pos = c.max_pos;
  fa.row_pos = ctx->at<int>(L.rowpos_a);
  fa.row_seq = ctx->at<int>(L.rowseq_a);
  fa.err = ctx->kv.error_word;
  fa.rows = rows;
  fa.T = c.n_target_layers;
  fa.H = H;
  fa.D = D;
  fa.eps = c.rms_eps;
  if (c.fusion == DFLASH_FUSION_FC) {
    fa.raw = 1;
    fa.f = ctx->at<uint16_t>(L.fraw);
  }
  CtxFinishArgs& ca = ap.ca;
  ca.part = ctx->at<float>(L.cpart);
  ca.ks = 1;
  ca.M = rows;
  ca.D = D;
  ca.n_kv = c.n_kv_heads;
  ca.d = c.head_dim;
  ca.row_pos = fa.row_pos;
  ca.row_seq = fa.row_seq;
  ca.B = B;
  ca.max_new = max_new;
  ca.n_new = n_new;
  ca.ctx_len = ctx->kv.ctx_len;
  ca.page_table = ctx->kv.page_table;
  ca.max_pages_per_seq = c.max_pages_per_seq;
  ca.n_pages = c.n_pages;
  ca.rope = c.use_rope ? ctx->at<float>(L.rope) : nullptr;
  ca.kv_pages = ctx->kv.kv_pages;
  ca.layer_stride = (long long)c.n_pages * 2 * kvd * 16;
  return ap;
}

// After the fusion: DFlash's FC fusion layer (GEMM, then norm) if so
// configured, then the context K and V of every layer as fp32 split
// partials, columns [layer][K | V]; sets the finisher's k split.
int append_kv(dflash_ctx* ctx, AppendCall& ap, hipStream_t stream) {
  const dflash_config& c = ctx->c;
  const Layout& L = ctx->L;
  const int rows = ap.rows, H = c.hidden, D = c.n_layers, kvd = c.n_kv_heads * c.head_dim;
  const bool fc = c.fusion == DFLASH_FUSION_FC;
  int rc;
  if (fc) {  // DFlash's FC fusion: c = RMSNorm(W_fc [h^(0); ...; h^(T-1)]) * g_fc, one context for all layers
    const int TH = c.n_target_layers * H;
    WsArgs g = ws_base(rows, TH, H);
    g.part = ctx->at<float>(L.cpart);
    add_seg(g, ctx->at<uint16_t>(L.wfc), nullptr, ap.fa.f, H / 32, 0);
    g.ks = gemm_ks(g, WS_PARTIAL, L.cpart_floats);
    if ((rc = ctx->launch(DFLASH_K_CTX_KV, stream, [&] { return launch_gemm(g, WS_PARTIAL, stream); }))) return rc;
    NormArgs na{};
    na.mode = 2;
    na.part = g.part;
    na.ks = g.ks;
    na.g = ctx->w.g_fc;
    na.h = ctx->at<uint16_t>(L.f);
    na.H = H;
    na.M = rows;
    na.eps = c.rms_eps;
    if ((rc = ctx->launch(DFLASH_K_FUSE, stream, [&] { return dflash_launch_norm(&na, stream); }))) return rc;
  }
  const int n_cols = D * 2 * kvd;
  int ks = 1, mm_xt = MM_ROW_TILES, mm_wt = 0;  // of the first launch: every launch writes the same partial layout
  for (int l0 = 0; l0 < D; l0 += WS_MAX_SEG / 2) {
    WsArgs g = ws_base(rows, H, n_cols);
    g.part = ctx->at<float>(L.cpart);
    for (int i = l0; i < D && i < l0 + WS_MAX_SEG / 2; ++i) {
      const uint16_t* act = ctx->at<uint16_t>(L.f) + (fc ? 0 : (size_t)i * 2 * act_plane(rows, H));
      add_seg(g, ctx->at<uint16_t>(L.wk_t) + (size_t)i * kvd * H, nullptr, act, kvd / 32, i * 2 * kvd);
      add_seg(g, ctx->at<uint16_t>(L.wv_t) + (size_t)i * kvd * H, nullptr, act, kvd / 32, i * 2 * kvd + kvd);
    }
    if (l0 == 0) {
      ks = gemm_ks(g, WS_PARTIAL, L.cpart_floats);
      mm_xt = g.mm_xt;
      mm_wt = g.mm_wt;
    }
    g.ks = ks;
    g.mm_xt = mm_xt;
    g.mm_wt = mm_wt;
    if ((rc = ctx->launch(DFLASH_K_CTX_KV, stream, [&] { return launch_gemm(g, WS_PARTIAL, stream); })))
      return rc;
  }
  ap.ca.ks = ks;
  return DFLASH_OK;
}

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
  const bool fc = c.fusion == DFLASH_FUSION_FC;
  if (!w->g_attn || !w->g_mlp || !w->g_final || !w->wq || !w->wk_d || !w->wv_d || !w->wo || !w->wg || !w->wu ||
      !w->wd || !w->embed || !w->lm_head)
    return fail(DFLASH_ERR_INVALID_ARG, "a weight pointer is null");
  if (fc ? (!w->w_fc || !w->g_fc) : (!w->w_fuse || !w->g_fuse))
    return fail(DFLASH_ERR_INVALID_ARG, fc ? "w_fc and g_fc required for FC fusion" : "w_fuse and g_fuse required");
  if (!c.tied_kv && (!w->wk_t || !w->wv_t)) return fail(DFLASH_ERR_INVALID_ARG, "wk_t/wv_t required unless tied_kv");
  if (!kv->kv_pages || !kv->page_table || !kv->ctx_len || !kv->error_word)
    return fail(DFLASH_ERR_INVALID_ARG, "a kv pointer is null");
  const Layout L = make_layout(c);
  if (ws_bytes < L.total) return fail(DFLASH_ERR_CAPACITY, "workspace %zu bytes < required %zu", ws_bytes, L.total);

  // alpha^(i) = softmax over the T entries of w_fuse[i] (float64 on the host;
  // unused, all zero, with FC fusion).
  std::vector<float> wf((size_t)c.n_layers * c.n_target_layers, 0.f);
  if (!fc) HIP_OK(hipMemcpy(wf.data(), w->w_fuse, wf.size() * 4, hipMemcpyDeviceToHost));
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
  int device = 0;
  HIP_OK(hipGetDevice(&device));
  HIP_OK(dflash_verify_scratch_setup(device));  // dflash_verify_noalloc's static scratch on this GPU
  char* ws = static_cast<char*>(workspace);
  HIP_OK(hipMemcpy(ws + L.alpha, alpha.data(), alpha.size() * 4, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(ws + L.rope, rope.data(), rope.size() * 4, hipMemcpyHostToDevice));

  // Pack every streamed matrix into the MFMA-operand layout (layers are
  // stacked along rows, so one pass per matrix).
  const int D = c.n_layers, H = c.hidden, I = c.intermediate;
  const int qd = c.n_q_heads * c.head_dim, kvd = c.n_kv_heads * c.head_dim;
  struct Job {
    const uint16_t* src;
    size_t dst;
    int R, K;
  };
  std::vector<Job> jobs = {{w->wq, L.wq, D * qd, H},   {w->wk_d, L.wk_d, D * kvd, H}, {w->wv_d, L.wv_d, D * kvd, H},
                           {w->wo, L.wo, D * H, qd},   {w->wg, L.wg, D * I, H},       {w->wu, L.wu, D * I, H},
                           {w->wd, L.wd, D * H, I},    {w->lm_head, L.lm, c.vocab, H}};
  if (!c.tied_kv) {
    jobs.push_back({w->wk_t, L.wk_t, D * kvd, H});
    jobs.push_back({w->wv_t, L.wv_t, D * kvd, H});
  }
  if (fc) jobs.push_back({w->w_fc, L.wfc, H, c.n_target_layers * H});
  for (const Job& j : jobs) {
    PackArgs pa{j.src, reinterpret_cast<uint16_t*>(ws + j.dst), j.R, j.K};
    HIP_OK(dflash_launch_pack(&pa, nullptr));
  }
  HIP_OK(hipStreamSynchronize(nullptr));

  dflash_ctx* ctx = new dflash_ctx();
  ctx->device = device;
  ctx->c = c;
  ctx->w = *w;
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
  int rc = append_check(ctx, B, seq_ids, n_new, target_hidden, max_new);
  if (rc) return rc;
  AppendCall ap = append_args(ctx, B, seq_ids, n_new, target_hidden, max_new);
  if ((rc = ctx->launch(DFLASH_K_FUSE, stream, [&] { return dflash_launch_fuse(&ap.fa, stream); }))) return rc;
  if ((rc = append_kv(ctx, ap, stream))) return rc;
  return ctx->launch(DFLASH_K_CTX_FINISH, stream, [&] { return dflash_launch_ctx_finish(&ap.ca, stream); });
}

}  // extern "C"

namespace {

// One drafting pass over B blocks: the block input is the anchor and masks,
// or `tokens` [B][N] when given (the dual-pass drafter's second pass). Each
// run of `grp` consecutive blocks belongs to one sequence (B % grp == 0), so
// the attention reads that sequence's context once for several blocks.
// `row_cut` [B] (device, nullable): block b needs draft positions
// row_cut[b] .. N-1 only (a dual-pass candidate keeps the first draft before
// its cut), so the LM head runs on those rows alone, compacted.
// `app` (nullable): an append of the same call, launched with the draft:
// its fusion shares the draft's first launch (the embedding norm, which
// takes the context length the append leaves), its context K/V projection
// runs before the first QKV projection, and its finisher shares the first
// layer's QKV finisher launch.
int draft_impl(dflash_ctx* ctx, int32_t B, const int32_t* seq_ids, const int32_t* anchor, const int32_t* tokens,
               int32_t* draft, float* top2_gap, float* conf, float* dbg_hidden, float* dbg_logits,
               hipStream_t stream, int grp = 1, const int32_t* row_cut = nullptr, AppendCall* app = nullptr) {
  const dflash_config& c = ctx->c;
  const Layout& L = ctx->L;
  const int N = c.block_size, M = B * N;
  const int H = c.hidden, I = c.intermediate, D = c.n_layers;
  const int qd = c.n_q_heads * c.head_dim, kvd = c.n_kv_heads * c.head_dim;
  int rc;

  float* x = ctx->at<float>(L.x);
  uint16_t* h = ctx->at<uint16_t>(L.h);
  float* gpart = ctx->at<float>(L.gpart);

  NormArgs na{};
  na.mode = 0;
  na.embed = ctx->w.embed;
  na.anchor = anchor;
  na.tokens = tokens;
  na.mask_id = c.mask_token_id;
  na.N = N;
  na.V = c.vocab;
  na.x = x;
  na.part = gpart;
  na.ks = 0;
  na.g = ctx->w.g_attn;
  na.h = h;
  na.dbg = dbg_hidden;
  na.seq_ids = seq_ids;
  na.ctx_len = ctx->kv.ctx_len;
  na.plan = ctx->at<int>(L.plan);
  na.plan_rope = ctx->at<float>(L.plan_rope);
  na.rope = c.use_rope ? ctx->at<float>(L.rope) : nullptr;
  na.half = c.head_dim / 2;
  na.page_table = ctx->kv.page_table;
  na.blk_pages = ctx->at<int>(L.blk_pages);
  na.max_pages_per_seq = c.max_pages_per_seq;
  na.max_seqs = c.max_seqs;
  na.max_pos = c.max_pos;
  na.err = ctx->kv.error_word;
  na.H = H;
  na.M = M;
  na.eps = c.rms_eps;
  if (app) {
    if ((rc = ctx->launch(DFLASH_K_FUSE, stream, [&] { return dflash_launch_fuse_norm(&app->fa, &na, stream); })))
      return rc;
  } else if ((rc = ctx->launch(DFLASH_K_NORM, stream, [&] { return dflash_launch_norm(&na, stream); }))) {
    return rc;
  }

  QkvFinishArgs qa{};
  qa.part = gpart;
  qa.M = M;
  qa.n_q = c.n_q_heads;
  qa.n_kv = c.n_kv_heads;
  qa.d = c.head_dim;
  qa.N = N;
  qa.rope = c.use_rope ? na.plan_rope : nullptr;
  qa.q = ctx->at<uint16_t>(L.q);
  qa.kblk = ctx->at<uint16_t>(L.kblk);
  qa.vblk = ctx->at<uint16_t>(L.vblk);
  qa.attn_ctr = ctx->at<int>(L.attn_ctr);

  AttnArgs aa{};
  aa.q = qa.q;
  aa.kblk = qa.kblk;
  aa.vblk = qa.vblk;
  aa.page_table = ctx->kv.page_table;
  aa.ctx_len = ctx->kv.ctx_len;
  aa.seq_ids = seq_ids;
  aa.plan = na.plan;
  aa.blk_pages = na.blk_pages;
  aa.part_o = ctx->at<float>(L.apo);
  aa.part_ml = ctx->at<float>(L.aml);
  aa.o = ctx->at<uint16_t>(L.o);
  aa.err = ctx->kv.error_word;
  aa.N = N;
  aa.n_q = c.n_q_heads;
  aa.n_kv = c.n_kv_heads;
  aa.chunk = kAttnChunk;
  aa.n_ck = L.n_ck;
  {  // blocks per workgroup, then chunks per work item from the largest grid
     // the batch can have
    const int n_wr = c.n_q_heads / c.n_kv_heads * N / 16;
    aa.grp = grp;
    aa.cand = std::max(1, std::min(grp, kAttnMaxWaves / n_wr));
    const long long wgs_z = (long long)(B / grp) * ((grp + aa.cand - 1) / aa.cand);
    const long long chunks = wgs_z * c.n_kv_heads * L.n_ck;
    const long long cpi = std::min<long long>(8, std::max<long long>(1, (chunks + kAttnItems - 1) / kAttnItems));
    aa.cpi = cpi <= 2 ? (int)cpi : cpi <= 4 ? 4 : 8;  // 1, 2, 4 or 8: the attention's DMA ring is built for these
    aa.n_blocks = B;
    aa.xcd_order = aa.cand == 1;
    aa.xcd_items = 1 + (L.n_ck - 1 + aa.cpi - 1) / aa.cpi;
    aa.xcd_tuples = (B / grp) * c.n_kv_heads;
    aa.attn_ctr = ctx->at<int>(L.attn_ctr);
  }
  aa.max_pages_per_seq = c.max_pages_per_seq;
  aa.n_pages = c.n_pages;
  aa.max_seqs = c.max_seqs;
  qa.q_scale = (float)(1.4426950408889634 / std::sqrt((double)c.head_dim));
  const long long layer_stride = (long long)c.n_pages * 2 * kvd * 16;

  for (int i = 0; i < D; ++i) {
    {  // Q, block K and block V: split partials, then RoPE/layout
      WsArgs g = ws_base(M, H, qd + 2 * kvd);
      g.part = gpart;
      add_seg(g, ctx->at<uint16_t>(L.wq) + (size_t)i * qd * H, nullptr, h, qd / 32, 0);
      add_seg(g, ctx->at<uint16_t>(L.wk_d) + (size_t)i * kvd * H, nullptr, h, kvd / 32, qd);
      add_seg(g, ctx->at<uint16_t>(L.wv_d) + (size_t)i * kvd * H, nullptr, h, kvd / 32, qd + kvd);
      g.ks = gemm_ks(g, WS_PARTIAL, L.gpart_floats);
      qa.ks = g.ks;
      if (i == 0 && app && (rc = append_kv(ctx, *app, stream))) return rc;
      if ((rc = ctx->launch(DFLASH_K_QKV, stream, [&] { return launch_gemm(g, WS_PARTIAL, stream); })))
        return rc;
      if (i == 0 && app) {
        if ((rc = ctx->launch(DFLASH_K_CTX_FINISH, stream,
                              [&] { return dflash_launch_finish2(&app->ca, &qa, stream); })))
          return rc;
      } else if ((rc = ctx->launch(DFLASH_K_QKV_FINISH, stream,
                                   [&] { return dflash_launch_qkv_finish(&qa, stream); }))) {
        return rc;
      }
    }
    aa.pages = ctx->kv.kv_pages + (size_t)i * layer_stride;
    if ((rc = ctx->launch(DFLASH_K_ATTN, stream, [&] { return dflash_launch_attn(&aa, B, c.head_dim, stream); })))
      return rc;
    if ((rc = ctx->launch(DFLASH_K_ATTN_MERGE, stream,
                          [&] { return dflash_launch_attn_merge(&aa, B, c.head_dim, stream); })))
      return rc;
    {  // O projection -> split partials, added by the next norm
      WsArgs g = ws_base(M, qd, H);
      g.part = gpart;
      add_seg(g, ctx->at<uint16_t>(L.wo) + (size_t)i * H * qd, nullptr, aa.o, H / 32, 0);
      g.ks = gemm_ks(g, WS_PARTIAL, L.gpart_floats);
      na.ks = g.ks;
      if ((rc = ctx->launch(DFLASH_K_OPROJ, stream, [&] { return launch_gemm(g, WS_PARTIAL, stream); })))
        return rc;
    }
    na.mode = 1;
    na.g = ctx->w.g_mlp + (size_t)i * H;
    na.dbg = nullptr;
    if ((rc = ctx->launch(DFLASH_K_NORM, stream, [&] { return dflash_launch_norm(&na, stream); }))) return rc;
    {  // gate/up + SwiGLU (full k per wave)
      WsArgs g = ws_base(M, H, I);
      g.out = ctx->at<uint16_t>(L.mm);
      add_seg(g, ctx->at<uint16_t>(L.wg) + (size_t)i * I * H, ctx->at<uint16_t>(L.wu) + (size_t)i * I * H, h,
              I / 16, 0);
      g.ks = gemm_ks(g, WS_SWIGLU, L.gpart_floats);
      g.part = gpart;
      if ((rc = ctx->launch(DFLASH_K_GATE_UP, stream, [&] { return launch_gemm(g, WS_SWIGLU, stream); })))
        return rc;
      if (g.ks > 1 &&
          (rc = ctx->launch(DFLASH_K_GATE_UP, stream, [&] { return dflash_launch_swiglu_finish(&g, stream); })))
        return rc;
    }
    {  // down -> split partials
      WsArgs g = ws_base(M, I, H);
      g.part = gpart;
      add_seg(g, ctx->at<uint16_t>(L.wd) + (size_t)i * H * I, nullptr, ctx->at<uint16_t>(L.mm), H / 32, 0);
      g.ks = gemm_ks(g, WS_PARTIAL, L.gpart_floats);
      na.ks = g.ks;
      if ((rc = ctx->launch(DFLASH_K_DOWN, stream, [&] { return launch_gemm(g, WS_PARTIAL, stream); })))
        return rc;
    }
    na.mode = 1;
    na.g = (i + 1 < D) ? ctx->w.g_attn + (size_t)(i + 1) * H : ctx->w.g_final;
    na.dbg = dbg_hidden ? dbg_hidden + (size_t)(i + 1) * M * H : nullptr;
    if (i + 1 == D && row_cut) {  // the LM head's input: the needed rows, compacted
      na.row_cut = row_cut;
      na.row_inv = ctx->at<int>(L.lm_inv);
      na.row_count = ctx->at<int>(L.lm_count);
    }
    if ((rc = ctx->launch(DFLASH_K_NORM, stream, [&] { return dflash_launch_norm(&na, stream); }))) return rc;
  }

  LmArgs la{};
  la.w = ctx->at<uint16_t>(L.lm);
  la.act = h;
  la.M = M;
  la.K = H;
  la.V = c.vocab;
  la.N = N;
  la.part = ctx->at<Top2>(L.lmpart);
  la.n_parts = lm_parts(c.vocab, M);  // one per LM-head workgroup along the vocabulary
  la.dbg_logits = row_cut ? nullptr : dbg_logits;
  la.row_count = row_cut ? na.row_count : nullptr;
  if ((rc = ctx->launch(DFLASH_K_LM_HEAD, stream, [&] {
         return M >= kMmMinRows ? dflash_launch_lmhead_mm(&la, stream) : dflash_launch_lmhead(&la, stream);
       })))
    return rc;

  ArgmaxArgs ma{};
  ma.part = la.part;
  ma.n_parts = la.n_parts;
  ma.M = M;
  ma.N = N;
  ma.V = c.vocab;
  ma.draft = draft;
  ma.gap = top2_gap;
  ma.conf = conf;
  ma.err = ctx->kv.error_word;
  ma.row_inv = row_cut ? na.row_inv : nullptr;
  ma.row_count = row_cut ? na.row_count : nullptr;
  return ctx->launch(DFLASH_K_ARGMAX, stream, [&] { return dflash_launch_argmax(&ma, stream); });
}

// Greedy or temperature-1 verification; the rows-pass and sampling-pass
// partials go to the workspace, or (noalloc) to the static scratch array of
// the handle's GPU.
int verify_impl(dflash_ctx* ctx, int32_t B, const int32_t* seq_ids, const int32_t* draft, const void* target_logits,
                int32_t logits_dtype, float temperature, uint64_t seed, uint64_t step, int32_t* accept_len,
                int32_t* next_token, int32_t* commit_len, hipStream_t stream, bool noalloc) {
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
  va.s_chunk = sample_chunk(c.vocab, (long long)B);
  va.s_n_chunks = (c.vocab + va.s_chunk - 1) / va.s_chunk;
  va.seq_ids = seq_ids;
  va.draft = draft;
  va.temp1 = temperature == 1.f;
  if (noalloc) {  // partials in the static scratch: rows pass, then (temperature 1) sampling pass
    const size_t part_b = align256((size_t)B * c.block_size * L.n_vchunks * 2 * sizeof(float));
    const size_t spart_b = va.temp1 ? align256((size_t)B * va.s_n_chunks * 2 * sizeof(float)) : 0;
    if (part_b + spart_b > DFLASH_VERIFY_SCRATCH_BYTES)
      return fail(DFLASH_ERR_CAPACITY,
                  "dflash_verify_noalloc: B=%d needs %zu bytes of scratch, the static scratch holds %u "
                  "(dflash_verify takes its partials from the workspace)",
                  B, part_b + spart_b, (unsigned)DFLASH_VERIFY_SCRATCH_BYTES);
    char* scratch = reinterpret_cast<char*>(dflash_verify_scratch(ctx->device));
    if (!scratch) return fail(DFLASH_ERR_HIP, "static scratch of device %d is not set up", ctx->device);
    va.part = reinterpret_cast<float*>(scratch);
    va.spart = reinterpret_cast<float*>(scratch + part_b);
  } else {
    va.part = ctx->at<float>(L.vpart);
    va.spart = ctx->at<float>(L.spart);
  }
  va.accept_len = accept_len;
  va.next_token = next_token;
  va.commit_len = commit_len;
  va.seed = seed;
  va.step = step;
  va.err = ctx->kv.error_word;
  va.inv_scale = 1.f;
  if (noalloc) {  // not routed through the kernel timer, whose events are created on demand
    const hipError_t e = dflash_launch_verify(&va, stream);
    if (e != hipSuccess) return fail(DFLASH_ERR_HIP, "verification launch: %s", hipGetErrorString(e));
    return DFLASH_OK;
  }
  return ctx->launch(DFLASH_K_VERIFY, stream, [&] { return dflash_launch_verify(&va, stream); });
}

}  // namespace

extern "C" {

int dflash_draft_block(dflash_ctx* ctx, int32_t B, const int32_t* seq_ids, const int32_t* anchor, int32_t* draft,
                       float* top2_gap, float* dbg_hidden, float* dbg_logits, hipStream_t stream) {
  if (!ctx) return fail(DFLASH_ERR_INVALID_ARG, "ctx is null");
  const dflash_config& c = ctx->c;
  if (B < 1 || B > c.max_batch) return fail(DFLASH_ERR_INVALID_ARG, "B=%d outside [1, max_batch=%d]", B, c.max_batch);
  if (!seq_ids || !anchor || !draft) return fail(DFLASH_ERR_INVALID_ARG, "null input/output pointer");
  return draft_impl(ctx, B, seq_ids, anchor, nullptr, draft, top2_gap, nullptr, dbg_hidden, dbg_logits, stream);
}

int dflash_append_draft(dflash_ctx* ctx, int32_t B, const int32_t* seq_ids, const int32_t* n_new,
                        const uint16_t* target_hidden, int32_t max_new, const int32_t* anchor, int32_t* draft,
                        float* top2_gap, hipStream_t stream) {
  int rc = append_check(ctx, B, seq_ids, n_new, target_hidden, max_new);
  if (rc) return rc;
  if (!anchor || !draft) return fail(DFLASH_ERR_INVALID_ARG, "null input/output pointer");
  if (ctx->c.fusion == DFLASH_FUSION_FC) {  // its FC layer sits between fusion and projection: the two calls
    if ((rc = dflash_ctx_append(ctx, B, seq_ids, n_new, target_hidden, max_new, stream))) return rc;
    return draft_impl(ctx, B, seq_ids, anchor, nullptr, draft, top2_gap, nullptr, nullptr, nullptr, stream);
  }
  AppendCall ap = append_args(ctx, B, seq_ids, n_new, target_hidden, max_new);
  return draft_impl(ctx, B, seq_ids, anchor, nullptr, draft, top2_gap, nullptr, nullptr, nullptr, stream, 1, nullptr,
                    &ap);
}

int dflash_d2sd_draft(dflash_ctx* ctx, int32_t B, const int32_t* seq_ids, const int32_t* anchor, int32_t K,
                      int32_t* drafts, float* conf, int32_t* cuts, hipStream_t stream) {
  if (!ctx) return fail(DFLASH_ERR_INVALID_ARG, "ctx is null");
  const dflash_config& c = ctx->c;
  const Layout& L = ctx->L;
  const int N = c.block_size;
  if (B < 1 || B > c.max_batch) return fail(DFLASH_ERR_INVALID_ARG, "B=%d outside [1, max_batch=%d]", B, c.max_batch);
  if (K < 1 || K > N - 1) return fail(DFLASH_ERR_INVALID_ARG, "K=%d outside [1, block_size-1=%d]", K, N - 1);
  if ((long long)B * K > c.max_batch)
    return fail(DFLASH_ERR_CAPACITY, "B*K=%lld second-pass blocks > max_batch=%d", (long long)B * K, c.max_batch);
  if (!seq_ids || !anchor || !drafts) return fail(DFLASH_ERR_INVALID_ARG, "null input/output pointer");
  D2sdArgs da{};
  da.B = B;
  da.N = N;
  da.K = K;
  da.V = c.vocab;
  da.mask_id = c.mask_token_id;
  da.seq_ids = seq_ids;
  da.anchor = anchor;
  da.conf = ctx->at<float>(L.d_conf);
  da.draft1 = ctx->at<int>(L.d_draft1);
  da.draft2 = ctx->at<int>(L.d_draft2);
  da.cuts = ctx->at<int>(L.d_cuts);
  da.seq2 = ctx->at<int>(L.d_seq);
  da.tokens = ctx->at<int>(L.d_tok);
  da.drafts = drafts;
  da.cuts_out = cuts;
  da.conf_out = conf;
  int rc = draft_impl(ctx, B, seq_ids, anchor, nullptr, ctx->at<int>(L.d_draft1), nullptr, ctx->at<float>(L.d_conf),
                      nullptr, nullptr, stream);
  if (rc) return rc;
  if ((rc = ctx->launch(DFLASH_K_D2SD, stream, [&] { return dflash_launch_d2sd_select(&da, stream); }))) return rc;
  if ((rc = draft_impl(ctx, B * K, da.seq2, nullptr, da.tokens, ctx->at<int>(L.d_draft2), nullptr, nullptr, nullptr,
                       nullptr, stream, K, da.cuts)))
    return rc;
  return ctx->launch(DFLASH_K_D2SD, stream, [&] { return dflash_launch_d2sd_assemble(&da, stream); });
}

int dflash_verify(dflash_ctx* ctx, int32_t B, const int32_t* seq_ids, const int32_t* draft, const void* target_logits,
                  int32_t logits_dtype, float temperature, uint64_t seed, uint64_t step, int32_t* accept_len,
                  int32_t* next_token, int32_t* commit_len, hipStream_t stream) {
  return verify_impl(ctx, B, seq_ids, draft, target_logits, logits_dtype, temperature, seed, step, accept_len,
                     next_token, commit_len, stream, false);
}

int dflash_verify_noalloc(dflash_ctx* ctx, int32_t B, const int32_t* seq_ids, const int32_t* draft,
                          const void* target_logits, int32_t logits_dtype, float temperature, uint64_t seed,
                          uint64_t step, int32_t* accept_len, int32_t* next_token, int32_t* commit_len,
                          hipStream_t stream) {
  return verify_impl(ctx, B, seq_ids, draft, target_logits, logits_dtype, temperature, seed, step, accept_len,
                     next_token, commit_len, stream, true);
}

int dflash_draft_sample(dflash_ctx* ctx, int32_t B, const int32_t* seq_ids, const int32_t* anchor, float temperature,
                        uint64_t seed, uint64_t step, int32_t* draft, float* draft_logits, hipStream_t stream) {
  if (!ctx) return fail(DFLASH_ERR_INVALID_ARG, "ctx is null");
  const dflash_config& c = ctx->c;
  if (B < 1 || B > c.max_batch) return fail(DFLASH_ERR_INVALID_ARG, "B=%d outside [1, max_batch=%d]", B, c.max_batch);
  if (!seq_ids || !anchor || !draft || !draft_logits) return fail(DFLASH_ERR_INVALID_ARG, "null input/output pointer");
  if (!(temperature > 0.f) || !std::isfinite(temperature) || !std::isfinite(1.f / temperature))
    return fail(DFLASH_ERR_INVALID_ARG, "temperature must be finite and > 0, with a finite reciprocal");
  const Layout& L = ctx->L;
  int rc = draft_impl(ctx, B, seq_ids, anchor, nullptr, ctx->at<int>(L.d_draft1), nullptr, nullptr, nullptr,
                      draft_logits, stream);
  if (rc) return rc;
  VerifyArgs va{};
  va.B = B;
  va.N = c.block_size;
  va.V = c.vocab;
  va.s_chunk = sample_chunk(c.vocab, (long long)B * (c.block_size - 1));
  va.s_n_chunks = (c.vocab + va.s_chunk - 1) / va.s_chunk;
  va.seq_ids = seq_ids;
  va.seed = seed;
  va.step = step;
  va.err = ctx->kv.error_word;
  va.inv_scale = 1.f;
  va.qlogits = draft_logits;
  va.inv_tau = 1.f / temperature;
  va.dpart = ctx->at<float>(L.dpart);
  va.draft_out = draft;
  return ctx->launch(DFLASH_K_ARGMAX, stream, [&] { return dflash_launch_draft_sample(&va, stream); });
}

int dflash_verify_sample(dflash_ctx* ctx, int32_t B, const int32_t* seq_ids, const int32_t* draft,
                         const float* draft_logits, float draft_temperature, const void* target_logits,
                         int32_t logits_dtype, uint64_t seed, uint64_t step, int32_t* accept_len, int32_t* next_token,
                         int32_t* commit_len, hipStream_t stream) {
  if (!ctx) return fail(DFLASH_ERR_INVALID_ARG, "ctx is null");
  const dflash_config& c = ctx->c;
  if (B < 1 || B > c.max_batch) return fail(DFLASH_ERR_INVALID_ARG, "B=%d outside [1, max_batch=%d]", B, c.max_batch);
  if (!seq_ids || !draft || !draft_logits || !target_logits || !accept_len || !next_token)
    return fail(DFLASH_ERR_INVALID_ARG, "null input/output pointer");
  if (logits_dtype != DFLASH_DTYPE_BF16 && logits_dtype != DFLASH_DTYPE_F32)
    return fail(DFLASH_ERR_INVALID_ARG, "logits_dtype must be DFLASH_DTYPE_BF16 or DFLASH_DTYPE_F32");
  if (!(draft_temperature > 0.f) || !std::isfinite(draft_temperature) || !std::isfinite(1.f / draft_temperature))
    return fail(DFLASH_ERR_INVALID_ARG, "draft_temperature must be finite and > 0, with a finite reciprocal");
  const Layout& L = ctx->L;
  VerifyArgs va{};
  va.logits = target_logits;
  va.dtype = logits_dtype;
  va.B = B;
  va.N = c.block_size;
  va.V = c.vocab;
  va.chunk = kVerifyChunk;
  va.n_chunks = L.n_vchunks;
  va.s_chunk = sample_chunk(c.vocab, (long long)B);
  va.s_n_chunks = (c.vocab + va.s_chunk - 1) / va.s_chunk;
  va.seq_ids = seq_ids;
  va.draft = draft;
  va.part = ctx->at<float>(L.vpart);
  va.spart = ctx->at<float>(L.spart);
  va.accept_len = accept_len;
  va.next_token = next_token;
  va.commit_len = commit_len;
  va.temp1 = 1;
  va.seed = seed;
  va.step = step;
  va.err = ctx->kv.error_word;
  va.inv_scale = 1.f;
  va.sampled = 1;
  va.qlogits = draft_logits;
  va.qpart = ctx->at<float>(L.qpart);
  va.inv_tau = 1.f / draft_temperature;
  return ctx->launch(DFLASH_K_VERIFY, stream, [&] { return dflash_launch_verify(&va, stream); });
}

int dflash_verify_multi(dflash_ctx* ctx, int32_t B, int32_t C, const int32_t* seq_ids, const int32_t* drafts,
                        const void* target_logits, int32_t logits_dtype, int32_t* accept_len, int32_t* next_token,
                        int32_t* commit_len, int32_t* chosen, hipStream_t stream) {
  if (!ctx) return fail(DFLASH_ERR_INVALID_ARG, "ctx is null");
  const dflash_config& c = ctx->c;
  if (B < 1 || C < 1) return fail(DFLASH_ERR_INVALID_ARG, "B=%d and C=%d must be >= 1", B, C);
  if ((long long)B * C > c.max_batch)
    return fail(DFLASH_ERR_CAPACITY, "B*C=%lld candidate blocks > max_batch=%d", (long long)B * C, c.max_batch);
  if (!seq_ids || !drafts || !target_logits || !accept_len || !next_token)
    return fail(DFLASH_ERR_INVALID_ARG, "null input/output pointer");
  if (logits_dtype != DFLASH_DTYPE_BF16 && logits_dtype != DFLASH_DTYPE_F32)
    return fail(DFLASH_ERR_INVALID_ARG, "logits_dtype must be DFLASH_DTYPE_BF16 or DFLASH_DTYPE_F32");
  const Layout& L = ctx->L;
  // every candidate block verified greedily as one more sequence (the
  // greedy passes do not read sequence ids), then the longest accept
  VerifyArgs va{};
  va.logits = target_logits;
  va.dtype = logits_dtype;
  va.B = B * C;
  va.N = c.block_size;
  va.V = c.vocab;
  va.chunk = kVerifyChunk;
  va.n_chunks = L.n_vchunks;
  va.s_chunk = sample_chunk(c.vocab, (long long)B * C);
  va.s_n_chunks = (c.vocab + va.s_chunk - 1) / va.s_chunk;
  va.seq_ids = seq_ids;
  va.draft = drafts;
  va.part = ctx->at<float>(L.vpart);
  va.spart = ctx->at<float>(L.spart);
  va.accept_len = ctx->at<int>(L.v_acc);
  va.next_token = ctx->at<int>(L.v_next);
  va.commit_len = nullptr;
  va.temp1 = 0;
  va.err = ctx->kv.error_word;
  va.inv_scale = 1.f;
  int rc = ctx->launch(DFLASH_K_VERIFY, stream, [&] { return dflash_launch_verify(&va, stream); });
  if (rc) return rc;
  PickArgs pa{};
  pa.B = B;
  pa.C = C;
  pa.acc = va.accept_len;
  pa.next = va.next_token;
  pa.accept_len = accept_len;
  pa.next_token = next_token;
  pa.commit_len = commit_len;
  pa.chosen = chosen;
  return ctx->launch(DFLASH_K_D2SD, stream, [&] { return dflash_launch_pick(&pa, stream); });
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
  for (size_t i = 0; i < t.used; ++i) {
    HIP_OK(hipEventSynchronize(t.ev[2 * i + 1]));
    float ms = 0.f;
    HIP_OK(hipEventElapsedTime(&ms, t.ev[2 * i], t.ev[2 * i + 1]));
    tot += ms;
  }
  *total_ms = tot;
  *launches = (int64_t)t.used;
  t.used = 0;
  return DFLASH_OK;
}

}  // extern "C"
