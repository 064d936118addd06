/*
 * dflash.h -- C ABI of the MI355X (gfx950) block-diffusion draft + verify hot path.
 *
 * One decode step of block-diffusion speculative decoding, DFlash style,
 * with DFLARE's per-layer fusion and heterogeneous K/V projections:
 *
 *   dflash_ctx_append   fuse the T target-layer hidden states of the newly
 *                       accepted tokens per draft layer and append their
 *                       context keys/values to the paged cache;
 *   dflash_draft_block  draft a whole block of tokens in one forward pass;
 *   dflash_append_draft the two above as one call, in fewer launches;
 *   dflash_verify       verify the block against the target's logits and
 *                       return the longest accepted prefix.
 *
 * Sources (web summaries; sections, not lines):
 *   [DFLARE] "DFLARE - scaling draft capacity of block-diffusion speculative
 *            decoding", gist.science technical summary: section 1 (problem),
 *            2.1 (adaptive layer fusion), 2.2 (heterogeneous KV projections).
 *   [DFLASH] "DFlash: Block Diffusion for Flash Speculative Decoding",
 *            euno.news summary: Overview, Key contributions, Methodology
 *            steps 1-4.
 *   [D2SD]   "D^2SD: Accelerating Speculative Decoding with Dual Diffusion
 *            Draft Models", euno.news summary: Methodology step 5.
 *
 * Conventions shared by every entry point
 *   - All tensors are device pointers to caller-owned memory (any allocator;
 *     PyTorch in the bundled binding). The library allocates no device
 *     memory and creates no streams; it allocates only the opaque host
 *     handle and, when kernel timing is switched on, HIP events.
 *   - bf16 means IEEE bfloat16 bits (uint16); row-major everywhere; matrices
 *     follow nn.Linear, [out_features, in_features].
 *   - Work is enqueued asynchronously on the caller's stream; nothing syncs
 *     except dflash_create (set-up copies), dflash_read_error and
 *     dflash_kernel_timer_read.
 *   - Arguments are validated on the host before anything is enqueued. On
 *     a negative status nothing was enqueued and dflash_last_error() holds
 *     a message (thread-local).
 *   - Conditions only the device can see (a sequence out of pages, a token
 *     id out of range, ...) OR a DFLASH_DEV_* bit into the caller's device
 *     error word; the affected sequence's results are then unspecified but
 *     every access stays in bounds.
 *   - A handle is not thread-safe. Results are deterministic: the same
 *     inputs give bit-identical outputs (no floating-point atomics).
 *   - Inputs must be finite; behaviour on NaN/Inf inputs is unspecified.
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- status */
#define DFLASH_OK 0
#define DFLASH_ERR_INVALID_ARG (-1) /* null pointer, bad size, B > max_batch ... */
#define DFLASH_ERR_UNSUPPORTED (-2) /* shape this build does not implement */
#define DFLASH_ERR_CAPACITY (-3)    /* workspace too small */
#define DFLASH_ERR_HIP (-4)         /* a HIP runtime call failed */

/* bits of the device error word */
#define DFLASH_DEV_BAD_SEQ 1       /* seq_ids[b] outside [0, max_seqs) */
#define DFLASH_DEV_BAD_N_NEW 2     /* n_new[b] outside [0, max_new] */
#define DFLASH_DEV_NO_PAGES 4      /* ctx_len + rows would exceed max_pages_per_seq*page_size or max_pos */
#define DFLASH_DEV_BAD_PAGE 8      /* a page-table entry outside [0, n_pages) */
#define DFLASH_DEV_BAD_TOKEN 16    /* an anchor or draft token outside [0, vocab) */

#define DFLASH_DTYPE_BF16 0
#define DFLASH_DTYPE_F32 1

/* ----------------------------------------------------------------- model */
typedef struct dflash_config {
  int32_t hidden;          /* H */
  int32_t n_layers;        /* D, draft layers */
  int32_t n_q_heads;       /* n_q */
  int32_t n_kv_heads;      /* n_kv; n_q % n_kv == 0, query head h reads kv head h / (n_q/n_kv) */
  int32_t head_dim;        /* d_h: 64 or 128 */
  int32_t intermediate;    /* I, SwiGLU width */
  int32_t vocab;           /* V */
  int32_t n_target_layers; /* T, target hidden states fused per token [DFLARE 2.1] */
  int32_t block_size;      /* N = 1 anchor + (N-1) mask positions, 2..16 */
  int32_t page_size;       /* tokens per KV page; must be 16 */
  int32_t max_seqs;        /* rows of page_table / entries of ctx_len */
  int32_t max_pages_per_seq;
  int32_t n_pages;         /* pages in kv_pages */
  int32_t max_pos;         /* positions covered by the RoPE table; ctx_len + N <= max_pos */
  int32_t mask_token_id;   /* embedding row used for mask positions */
  int32_t tied_kv;         /* 1: context uses the block projections (DFlash's shared K/V) */
  int32_t use_rope;        /* 1 normally; 0 disables RoPE (tests) */
  int32_t max_batch;       /* largest B of any call (workspace sizing) */
  int32_t max_new;         /* largest rows appended per sequence per call (workspace sizing) */
  float rope_theta;        /* RoPE base, e.g. 1e6 */
  float rms_eps;           /* RMSNorm epsilon, e.g. 1e-6 */
  int32_t fusion;          /* DFLASH_FUSION_SOFTMAX (0): per-layer weighted sum [DFLARE 2.1];
                              DFLASH_FUSION_FC (1): one FC layer, one context for every layer
                              [DFLARE 1: DFlash's conditioning] */
} dflash_config;

#define DFLASH_FUSION_SOFTMAX 0
#define DFLASH_FUSION_FC 1

/* Device pointers to drafter weights, all bf16 except w_fuse (fp32).
 * Stacked over the D draft layers:
 *   wq [D, n_q*d_h, H]          wk_d, wv_d [D, n_kv*d_h, H]  block K/V  [DFLARE 2.2]
 *   wk_t, wv_t [D, n_kv*d_h, H] context K/V [DFLARE 2.2]; ignored when tied_kv
 *   wo [D, H, n_q*d_h]          wg, wu [D, I, H]             wd [D, H, I]
 *   embed, lm_head [V, H]       g_attn, g_mlp [D, H]         g_final [H]
 *   softmax fusion: w_fuse [D, T] fp32, alpha^(i) = softmax(w_fuse[i, :]),
 *                   and g_fuse [D, H]                          [DFLARE 2.1]
 *   FC fusion:      w_fc [H, T*H] (the T states of a token concatenated in
 *                   layer order) and g_fc [H]                  [DFLARE 1]
 * The pointers of the fusion not configured may be null.
 * dflash_create copies every projection matrix (w_fc included) and lm_head
 * into the workspace in the layout the kernels stream (16x32 MFMA operand
 * blocks, 1 KB contiguous each); after it returns only embed and the gains
 * are read again and must stay valid and unchanged until dflash_destroy;
 * the other weight buffers may be freed. */
typedef struct dflash_weights {
  const float* w_fuse;
  const uint16_t *g_fuse, *g_attn, *g_mlp, *g_final;
  const uint16_t *wq, *wk_d, *wv_d, *wk_t, *wv_t, *wo, *wg, *wu, *wd;
  const uint16_t *embed, *lm_head;
  const uint16_t *w_fc, *g_fc;
} dflash_weights;

/* Paged per-sequence context cache, one set of pages per draft layer.
 *   kv_pages   bf16 [D, n_pages, 2, n_kv, 16*d_h]; per page and head, part 0
 *              holds keys slot-major [16 slots][d_h] (already rotated by
 *              RoPE), part 1 holds values dim-major [d_h][16 slots].
 *   page_table int32 [max_seqs, max_pages_per_seq]: position p of sequence
 *              s lives in page page_table[s][p / 16], slot p % 16.
 *   ctx_len    int32 [max_seqs]: cached positions per sequence; advanced
 *              by dflash_ctx_append.
 *   error_word int32 [1]: device error bits (DFLASH_DEV_*), OR-ed.
 * The caller maps pages before a call writes into them. */
typedef struct dflash_kv {
  uint16_t* kv_pages;
  int32_t* page_table;
  int32_t* ctx_len;
  int32_t* error_word;
} dflash_kv;

typedef struct dflash_ctx dflash_ctx;

/* Device workspace the library needs for this config (bytes). */
size_t dflash_workspace_bytes(const dflash_config* cfg);

/* Validate shapes, compute alpha = softmax(w_fuse) rows [DFLARE 2.1] and the
 * RoPE cos/sin table (float64 angles rounded to fp32) on the host, copy them
 * into the workspace and pack the streamed weights into it (synchronous,
 * null stream; the weights must be ready).
 * workspace: device memory of at least dflash_workspace_bytes(cfg) bytes,
 * owned by the caller, exclusively used by this handle until destroy. */
int dflash_create(const dflash_config* cfg, const dflash_weights* w, const dflash_kv* kv,
                  void* workspace, size_t ws_bytes, dflash_ctx** out);

/* Frees the host handle only. */
void dflash_destroy(dflash_ctx* ctx);

/* Append n_new[b] context rows of sequence seq_ids[b], b < B [DFLARE 2.1, 2.2].
 * target_hidden: bf16 [B, max_new, T, H]; row t < n_new[b] of batch entry b
 * holds the T selected target-layer states of the token at position
 * ctx_len[seq] + t. For every draft layer i: f = RMSNorm(sum_j alpha^(i)_j
 * h^(j)) * g_fuse[i] (FC fusion: f = RMSNorm(W_fc [h^(0); ...; h^(T-1)])
 * * g_fc, the same for every layer); K = RoPE(f W^t_K[i]^T) and
 * V = f W^t_V[i]^T go to the cache; then ctx_len[seq] += n_new[b]. seq_ids, n_new: device int32
 * [B]; the B sequences must be distinct. max_new <= cfg.max_new. */
int dflash_ctx_append(dflash_ctx* ctx, int32_t B, const int32_t* seq_ids, const int32_t* n_new,
                      const uint16_t* target_hidden, int32_t max_new, hipStream_t stream);

/* Draft one block per sequence in one forward pass [DFLASH Methodology 2;
 * DFLARE 1, 2.2]. Block tokens [anchor[b], mask x (N-1)] at positions
 * L..L+N-1 (L = ctx_len[seq_ids[b]]). Every draft layer: pre-norm GQA
 * attention with RoPE of the N block queries over [context K/V ; block K/V]
 * (no mask), SwiGLU MLP, residuals; then the final norm, the LM head and an
 * argmax (lowest index on ties) on block rows 1..N-1.
 *   anchor    device int32 [B]
 *   draft     device int32 [B, N-1]                 (out)
 *   top2_gap  device fp32 [B, N-1], nullable         (out) top-1 minus top-2 logit
 *   dbg_hidden device fp32 [D+1, B, N, H], nullable  (out) residual stream: the
 *             embeddings, then after each layer
 *   dbg_logits device fp32 [B, N-1, V], nullable     (out) draft logits */
int dflash_draft_block(dflash_ctx* ctx, int32_t B, const int32_t* seq_ids, const int32_t* anchor,
                       int32_t* draft, float* top2_gap, float* dbg_hidden, float* dbg_logits,
                       hipStream_t stream);

/* dflash_ctx_append followed by dflash_draft_block for the same B sequences
 * [DFLASH Methodology 2, 4; DFLARE 2.1, 2.2], with the same results bit for
 * bit (the draft sees the context the append leaves), in fewer launches:
 * the fusion shares the draft's first launch (the block embedding norm,
 * which applies the append's checks itself to find the context length the
 * append leaves) and the context finisher shares the first draft layer's
 * QKV finisher launch. Arguments as the two calls (draft without debug
 * outputs); validated on the host before anything is enqueued. With FC
 * fusion (an FC layer between fusion and projection) it issues the two
 * calls in turn. Device-side errors set the same bits as the two calls. */
int dflash_append_draft(dflash_ctx* ctx, int32_t B, const int32_t* seq_ids, const int32_t* n_new,
                        const uint16_t* target_hidden, int32_t max_new, const int32_t* anchor, int32_t* draft,
                        float* top2_gap, hipStream_t stream);

/* Verify the drafted blocks [DFLASH Methodology 3, 4; D2SD Methodology 5].
 * target_logits [B, N, V] (bf16 or fp32 per logits_dtype): row r predicts
 * the token after block position r. draft device int32 [B, N-1].
 * temperature 0: t_r = argmax row r (lowest index); a = longest prefix with
 *   draft[j] == t_j; next = t_a.
 * temperature 1: lossless rejection sampling for the one-hot draft: accept
 *   draft[a] while u_a < softmax(row a)[draft[a]], u_a a Philox4x64-10
 *   uniform keyed by (seed; counter k=0, row a | stream 0, seq, step); at
 *   the first rejection sample row a without draft[a], else the bonus row
 *   N-1, by Gumbel-max with per-entry Philox draws (stream 1).
 * Outputs, device int32 [B]: accept_len a in 0..N-1, next_token, and
 * commit_len = a + 1 (nullable). */
int dflash_verify(dflash_ctx* ctx, int32_t B, const int32_t* seq_ids, const int32_t* draft,
                  const void* target_logits, int32_t logits_dtype, float temperature,
                  uint64_t seed, uint64_t step, int32_t* accept_len, int32_t* next_token,
                  int32_t* commit_len, hipStream_t stream);

/* Verification that allocates nothing, for callers that cannot allocate
 * device memory or must not touch the handle's workspace (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).
 * Arguments, outputs and results are exactly those of dflash_verify (the
 * same kernels; bit-identical outputs). The kernels' partial results live
 * in a static device array of DFLASH_VERIFY_SCRATCH_BYTES per GPU (held
 * until the process ends, its address looked up once per device by
 * dflash_create) instead of the workspace; the call needs
 *   8 * B * N * ceil(V / 32768) bytes (greedy), plus about
 *   8 * B * ceil(V / chunk) bytes at temperature 1 (chunk: 1024 .. V logits,
 *   about 512 sampling work items per call),
 * each part rounded up to 256 bytes; a call needing more returns
 * DFLASH_ERR_CAPACITY with a message and enqueues nothing. No hipMalloc,
 * hipFree or allocating library routine is called. Every call on a GPU
 * shares that GPU's array (the last call's partials stay in it; every
 * partial a call reads it wrote first): calls that overlap on one GPU --
 * on different streams, or from several handles -- race and must be
 * ordered by the caller. */
#define DFLASH_VERIFY_SCRATCH_BYTES (1u << 20)
int dflash_verify_noalloc(dflash_ctx* ctx, int32_t B, const int32_t* seq_ids, const int32_t* draft,
                          const void* target_logits, int32_t logits_dtype, float temperature,
                          uint64_t seed, uint64_t step, int32_t* accept_len, int32_t* next_token,
                          int32_t* commit_len, hipStream_t stream);

/* Sampled drafting at temperature > 0 [DFLASH Methodology 2-3, with a
 * sampled proposal]. The forward pass of dflash_draft_block, then for each
 * draft row r (position r + 1) the token d = argmax_k (z[r,k] / temperature
 * + G_k): a draw from q_r = softmax(z[r] / temperature), G_k Gumbel noise from
 * Philox4x64-10 keyed by (seed; counter k / 4, r | 2 << 32, seq, step),
 * word k % 4.
 * temperature: finite, > 0, with a finite fp32 reciprocal
 * (DFLASH_ERR_INVALID_ARG otherwise; the same for draft_temperature below).
 *   draft        device int32 [B, N-1]   (out)
 *   draft_logits device fp32 [B, N-1, V] (out, required): the drafter's
 *                logits z, which dflash_verify_sample needs. */
int dflash_draft_sample(dflash_ctx* ctx, int32_t B, const int32_t* seq_ids, const int32_t* anchor,
                        float temperature, uint64_t seed, uint64_t step, int32_t* draft, float* draft_logits,
                        hipStream_t stream);

/* Lossless verification of sampled drafts at target temperature 1 [DFLASH
 * Methodology 3, key contributions]. p_r = softmax(target_logits[b, r]),
 * q_r = softmax(draft_logits[b, r] / draft_temperature). Accept draft[a]
 * while u_a * q_a(draft[a]) < p_a(draft[a]) (u_a as in dflash_verify); at the
 * first rejection sample max(0, p_a - q_a) renormalised, by Gumbel-max over
 * log(p_k - q_k) + G_k (stream 1) on the entries with p_k > q_k; if all N-1
 * are accepted sample the bonus row N-1 from p. Outputs as dflash_verify. */
int dflash_verify_sample(dflash_ctx* ctx, int32_t B, const int32_t* seq_ids, const int32_t* draft,
                         const float* draft_logits, float draft_temperature, const void* target_logits,
                         int32_t logits_dtype, uint64_t seed, uint64_t step, int32_t* accept_len,
                         int32_t* next_token, int32_t* commit_len, hipStream_t stream);

/* Dual-pass drafting [D2SD Methodology 1-3]. First pass as
 * dflash_draft_block; confidence of draft position j = the drafter's
 * largest softmax probability of block row j, 1 / sum_v exp(z_v - max z);
 * cut points = the K positions of lowest confidence (ties to the lower
 * position), ascending; for each cut point c a second-pass block
 * [anchor, d_1 .. d_{c-1}, mask ...] at the same positions and over the
 * same context (same weights and cache), all B*K blocks in one pass;
 * candidate 0 is the first draft, candidate k keeps d_1 .. d_{c_k - 1} and
 * takes the second pass's argmax from position c_k on.
 *   K         1 .. N-1; B*K <= cfg.max_batch (DFLASH_ERR_CAPACITY)
 *   drafts    device int32 [B, K+1, N-1]      (out) candidates
 *   conf      device fp32 [B, N-1], nullable   (out) first-pass confidence
 *   cuts      device int32 [B, K], nullable    (out) cut positions, 1-based
 * Workspace buffers hold the intermediate blocks; no host synchronisation. */
int dflash_d2sd_draft(dflash_ctx* ctx, int32_t B, const int32_t* seq_ids, const int32_t* anchor,
                      int32_t K, int32_t* drafts, float* conf, int32_t* cuts, hipStream_t stream);

/* Greedy verification of C candidate blocks per sequence [D2SD Methodology
 * 4]: drafts device int32 [B, C, N-1], target_logits [B, C, N, V] (bf16 or
 * fp32), each candidate's own logits. Every candidate is verified as in
 * dflash_verify (temperature 0); the longest accept wins, the lowest
 * candidate index on ties. B*C <= cfg.max_batch (DFLASH_ERR_CAPACITY).
 * Outputs, device int32 [B]: accept_len, next_token, commit_len (nullable),
 * chosen candidate (nullable). */
int dflash_verify_multi(dflash_ctx* ctx, int32_t B, int32_t C, const int32_t* seq_ids, const int32_t* drafts,
                        const void* target_logits, int32_t logits_dtype, int32_t* accept_len,
                        int32_t* next_token, int32_t* commit_len, int32_t* chosen, hipStream_t stream);

/* Message of the last failed call on this thread ("" if none). */
const char* dflash_last_error(void);

/* Synchronise the stream, copy the device error word to *out and clear it.
 * Bits that work on another stream sets between the copy and the clear are
 * lost: call it while no other stream uses the context. */
int dflash_read_error(dflash_ctx* ctx, hipStream_t stream, int32_t* out);

/* ------------------------------------------------------ kernel timing
 * Per-kernel timing with HIP events recorded on the launch stream around
 * every launch of one kernel kind. Off by default; switching it on costs
 * two event records per launch of that kind. */
#define DFLASH_K_FUSE 0      /* append: call plan + layer fusion + RMSNorm */
#define DFLASH_K_CTX_KV 1    /* append: context K/V projection (split-k partials) */
#define DFLASH_K_NORM 2      /* embedding / residual reduce + RMSNorm */
#define DFLASH_K_QKV 3       /* block Q/K/V projection (split-k partials) */
#define DFLASH_K_ATTN 4      /* split-context block attention */
#define DFLASH_K_ATTN_MERGE 5
#define DFLASH_K_OPROJ 6
#define DFLASH_K_GATE_UP 7   /* gate/up projection + SwiGLU (a second launch applies SwiGLU after a k split) */
#define DFLASH_K_DOWN 8
#define DFLASH_K_LM_HEAD 9   /* LM head + per-tile top-2 */
#define DFLASH_K_ARGMAX 10
#define DFLASH_K_VERIFY 11
#define DFLASH_K_QKV_FINISH 12 /* split-k sum + RoPE + layout of Q and block K/V */
#define DFLASH_K_CTX_FINISH 13 /* split-k sum + RoPE + page scatter of context K/V; advances ctx_len */
#define DFLASH_K_D2SD 14     /* dual-pass drafting: cut points + second-pass blocks, candidates; multi-verify pick */
#define DFLASH_K_COUNT 15

/* Start (enable != 0) or stop timing kernel kind `kind`; starting clears
 * the totals. Capacity: 4096 launches between reads. A timed launch of a
 * single-kernel kind records the kernel's own start and end (the events of
 * hipExtLaunchKernel); DFLASH_K_VERIFY is timed between event records on
 * the stream around its two (greedy) or three (temperature 1) kernels.
 * Timing adds a few microseconds
 * of stream idle time around each timed launch; it is meant for eager
 * launches, not for graph capture. */
int dflash_kernel_timer(dflash_ctx* ctx, int32_t kind, int32_t enable);
/* Synchronise the recorded events; *total_ms = summed launch durations,
 * *launches = number of launches timed since the timer was started. */
int dflash_kernel_timer_read(dflash_ctx* ctx, int32_t kind, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif
#endif /* DFLASH_H */
