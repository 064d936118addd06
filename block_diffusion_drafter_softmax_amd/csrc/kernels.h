// Kernel argument structs and launchers shared by the HIP kernels and the
// host library (plain data; the one helper is usable on host and device).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

// Top-2 with index: (v1, i1) is the maximum, lowest index on ties; v2 is
// the largest value among the remaining entries; s = sum of exp(v - v1)
// over all entries merged (so the softmax maximum is 1 / s).
struct Top2 {
  float v1;
  int i1;
  float v2;
  float s;
};

// MFMA-operand packed layout, used for every weight matrix the GEMMs stream
// and for every activation they read. Element (r, k) of an [R][K] matrix
// (R a multiple of 16 after padding, K a multiple of 32) lives at
//   ((r/16 * K/32 + k/32) * 64 + lane) * 8 + k%8,  lane = r%16 + 16*((k%32)/8),
// so the 16x32 operand block of one 16x16x32 MFMA is 1 KB of contiguous
// memory in lane order and a wave loads it with one 16-byte load per lane.
__host__ __device__ inline size_t pk_index(int r, int k, int K) {
  const int lane = (r & 15) | (((k >> 3) & 3) << 4);
  return (((size_t)(r >> 4) * (K >> 5) + (k >> 5)) * 64 + lane) * 8 + (k & 7);
}
__host__ __device__ inline int pad16(int m) { return (m + 15) & ~15; }

// Activations (GEMM inputs, attention queries) are fp32 values carried as a
// bf16 pair: a hi plane holding bf16(x) followed by a lo plane holding
// bf16(x - hi), so x = hi + lo to about 2^-17 relative and a product with a
// bf16 weight, taken as two MFMAs, keeps fp32-level accuracy. In the packed
// layout each plane has act_plane(R, K) elements; only weights and the K/V
// data are single bf16.
__host__ __device__ inline size_t act_plane(int R, int K) { return (size_t)pad16(R) * K; }

// ------------------------------------------------------------ streaming GEMM
enum WsMode : int {
  WS_PARTIAL = 0,  // fp32 partial sums part[split][M][n_cols]
  WS_SWIGLU = 1,   // silu(gate) * up -> bf16, packed activation of the next GEMM (K_next = n_cols)
};

#define WS_MAX_SEG 16

// Output tile of one tiled-GEMM workgroup (many activation rows): 16-row
// activation tiles by 16-row weight tiles.
#define MM_ROW_TILES 8
#define MM_COL_TILES 16

struct WsSeg {
  const uint16_t* w0;   // packed weights [tiles][K/32][512]
  const uint16_t* w1;   // WS_SWIGLU: packed up weights (w0 holds gate)
  const uint16_t* act;  // packed split activation: hi plane, lo plane at + act_plane(M, K)
  int units;            // work units (NT tiles of 16 rows each)
  int col0;             // first output column of this segment
};

struct WsArgs {
  WsSeg seg[WS_MAX_SEG];
  int unit_start[WS_MAX_SEG + 1];
  int nseg;
  int K;        // reduction length (multiple of 32)
  int M;        // activation rows
  int ks;       // k splits (one wave per (unit, split))
  int n_cols;   // row length of the partial buffer / SwiGLU features
  float* part;  // WS_PARTIAL: [ks][M][n_cols]; tiled WS_SWIGLU with ks > 1: [ks][M][2*n_cols] (gate | up)
  uint16_t* out;  // WS_SWIGLU: packed split activation, planes of act_plane(M, n_cols)
  int mm_xt;      // tiled GEMM, 4-wave loop: activation tiles per workgroup (MM_ROW_TILES, or half of it)
  int mm_wt;      // tiled GEMM: 0, or the 8-wave loop with this many weight tiles per workgroup (16, 24, 32)
};

struct PackArgs {
  const uint16_t* src;  // [R][K] row-major
  uint16_t* dst;        // packed
  int R, K;
};

// ------------------------------------------------------------ finishers
struct QkvFinishArgs {
  const float* part;  // [ks][M][n_q*d + 2*n_kv*d]: Q columns, then block K, then block V
  int ks, M, n_q, n_kv, d, N;
  const float* rope;  // the call's plan: cos/sin of every row's position [M][d/2][2], or null (no rotation)
  float q_scale;      // applied to rotated queries: log2(e) / sqrt(d) (attention works in log2 units)
  uint16_t* q;        // split: hi [M][n_q][d], lo at + M*n_q*d
  uint16_t* kblk;     // [B][n_kv][16][d]
  uint16_t* vblk;     // [B][n_kv][d][16]
  int* attn_ctr;      // nullable: the attention's 8 work counters, set to 0 here
};

struct CtxFinishArgs {
  const float* part;  // [ks][M][D * 2 * n_kv*d]: per layer K columns then V columns
  int ks, M, D, n_kv, d;
  int B, max_new;     // the call's sequences: ctx_len[seq] advances by n_new[b]
  const int* n_new;
  int* ctx_len;
  const int* row_pos;  // < 0: row skipped
  const int* row_seq;
  const int* page_table;
  int max_pages_per_seq, n_pages;
  const float* rope;
  uint16_t* kv_pages;
  long long layer_stride;
};

// ------------------------------------------------------------ attention
struct AttnArgs {
  const uint16_t* q;       // split: hi [B*N][n_q][d], lo at + B*N*n_q*d; pre-scaled by log2(e)/sqrt(d)
  const uint16_t* kblk;    // [B][n_kv][16][d]
  const uint16_t* vblk;    // [B][n_kv][d][16]
  const uint16_t* pages;   // this layer's pages [n_pages][2][n_kv][16*d]
  const int* page_table;
  const int* ctx_len;
  const int* seq_ids;
  float* part_o;           // [B][n_kv][n_ck][R][d]: one per work item (item 0: the block's keys; then
                           // context items, < 1 + ceil((n_ck - 1) / cpi))
  float* part_ml;          // [B][n_kv][n_ck][R][2]
  uint16_t* o;             // merge output, packed split activation (planes of act_plane(B*N, n_q*d))
  int32_t* err;
  int N, n_q, n_kv, chunk, n_ck, max_pages_per_seq, n_pages, max_seqs;
  int cpi;                 // chunks of `chunk` context keys per context work item (1 .. 8)
  const int* plan;         // the call's plan [B][2]: sequence (clamped), context length
  const int* blk_pages;    // the call's page-table row of each block [B][max_pages_per_seq]
  int grp;                 // consecutive blocks that share one sequence's context (B % grp == 0)
  int cand;                // blocks of a group one workgroup takes (1 .. grp): a context chunk is read once for them
  int n_blocks;            // B, the blocks of the call
  int xcd_order;           // cand == 1: 1-D grid, all workgroups of a (sequence group, kv head) on one XCD
  int xcd_items, xcd_tuples;  // items per (block, kv head); (B / grp) * n_kv (sequence groups x kv heads)
  int* attn_ctr;           // [8] per-XCD work counters of the persistent ring kernel, zeroed by the Q/K/V
                           // finisher before every attention launch (null: no persistent kernel)
};

// ------------------------------------------------------------ small kernels
// Context append, first kernel: the call's plan (positions, checks) and
// DFLARE fusion + RMSNorm of every appended row for every draft layer.
struct FuseArgs {
  const uint16_t* hidden;  // [rows][T][H], row m = b*max_new + t
  const float* alpha;      // [D][T]
  const uint16_t* g_fuse;  // [D][H]
  uint16_t* f;             // per layer packed split activation, layer stride 2*act_plane(rows, H)
  int B, max_new;
  const int* seq_ids;
  const int* n_new;
  const int* ctx_len;      // read only: the context finisher advances it
  const int* page_table;
  int max_seqs, max_pages_per_seq, n_pages, max_pos;
  int* row_pos;            // [rows]: position, or -1 (row skipped)
  int* row_seq;            // [rows]
  int32_t* err;
  int rows, T, H, D;
  float eps;
  int raw;                 // FC fusion: f is instead the FC layer's input, each row's T*H states as a packed
                           // split activation [rows][T*H] (lo plane 0); no fusion, no norm
};

struct NormArgs {
  int mode;                // 0: x = embedding rows, 1: x += sum of split partials,
                           // 2: x = sum of split partials (no residual; x not written)
  const uint16_t* embed;   // [V][H]
  const int* anchor;       // [B]
  const int* tokens;       // mode 0, nullable: [B][N] block input tokens (else anchor, then masks)
  int mask_id, N, V;
  const int* seq_ids;      // mode 0: checks of the draft call (error word)
  const int* ctx_len;
  int max_seqs, max_pos;
  int32_t* err;
  float* x;                // [M][H] residual stream (fp32)
  const float* part;       // [ks][M][H]
  int ks;
  const uint16_t* g;       // gain [H]
  uint16_t* h;             // packed split activation out (planes of act_plane(M, H))
  float* dbg;              // nullable [M][H]
  int H, M;
  float eps;
  // mode 0 also writes the draft call's plan, read by the later kernels in
  // one load instead of a sequence id -> context length -> table chain
  int* plan;               // [B][2]: sequence (clamped), context length
  float* plan_rope;        // [M][d/2][2]: cos/sin at row m's position (when rope is set)
  const float* rope;       // [max_pos][d/2][2] or null
  int half;                // d/2
  // and block b's row of the page table, copied to blk_pages[b] so that the
  // attention requests its pages together with the plan, not after it
  const int* page_table;   // [max_seqs][max_pages_per_seq]
  int* blk_pages;          // nullable [B][max_pages_per_seq]
  int max_pages_per_seq;
  // Rows the LM head needs (the dual-pass drafter's second pass): block b
  // keeps rows n >= row_cut[b]; those rows are written compacted, in block
  // order, with row_inv[compact] = m and the number of rows in *row_count.
  const int* row_cut;      // nullable [M/N]
  int* row_inv;            // [M]
  int* row_count;          // [1]
};

struct LmArgs {
  const uint16_t* w;    // packed [V/16][K/32][512]
  const uint16_t* act;  // packed split activation of the normed rows
  int M, K, V, N;       // N = block rows per sequence
  Top2* part;           // [M][n_parts]: one top-2 per row and workgroup (64 or 512 vocabulary rows)
  int n_parts;          // workgroups along the vocabulary
  float* dbg_logits;    // nullable [B][N-1][V]
  const int* row_count; // nullable: rows 0 .. *row_count-1 of act are compacted rows; row blocks past it are skipped
};

struct ArgmaxArgs {
  const Top2* part;  // [M][n_parts]
  int n_parts, M, N, V;
  int* draft;        // [B][N-1]
  float* gap;        // nullable [B][N-1]
  float* conf;       // nullable [B][N-1]: largest softmax probability of the drafter's row
  int32_t* err;
  const int* row_inv;    // nullable: compacted rows (row m of the partials is block row row_inv[m])
  const int* row_count;  // with row_inv: rows present
};

// Dual-pass drafting (D2SD): cut points of the first draft and the second
// pass's input blocks; then the candidates' drafts.
struct D2sdArgs {
  int B, N, K, V, mask_id;
  const int* seq_ids;   // [B]
  const int* anchor;    // [B]
  const float* conf;    // [B][N-1] first-pass confidence
  const int* draft1;    // [B][N-1] first draft
  const int* draft2;    // [B*K][N-1] second-pass drafts
  int* cuts;            // [B][K] cut positions (1-based, ascending)
  int* seq2;            // [B*K] sequence of each second-pass block
  int* tokens;          // [B*K][N] second-pass input blocks
  int* drafts;          // [B][K+1][N-1] candidates
  int* cuts_out;        // nullable [B][K]
  float* conf_out;      // nullable [B][N-1]
};

// Longest accept over C candidates of each sequence (lowest index on ties).
struct PickArgs {
  int B, C;
  const int* acc;       // [B*C]
  const int* next;      // [B*C]
  int* accept_len;
  int* next_token;
  int* commit_len;      // nullable
  int* chosen;          // nullable
};

#define VERIFY_MAX_PARTS 2048  // block rows * vocabulary chunks of one sequence

struct VerifyArgs {
  const void* logits;   // [B][N][V]
  int dtype;            // DFLASH_DTYPE_*
  int B, N, V, chunk, n_chunks;  // rows pass: logits per work item, work items per row
  int s_chunk, s_n_chunks;       // temperature-1 sampling pass: the same for the sampled row
  const int* seq_ids;
  const int* draft;     // [B][N-1]
  float* part;          // rows pass [B][N][n_chunks][2]
  float* spart;         // sampling pass [B][s_n_chunks][2]
  int* accept_len;
  int* next_token;
  int* commit_len;      // nullable
  int temp1;
  unsigned long long seed, step;
  int32_t* err;
  // sampled drafts (a general proposal q = softmax(z / tau) per draft row)
  float inv_scale;         // rows pass: logits times this (1 for the target, 1/tau for the drafter)
  int sampled;             // temperature-1 verification against the drafter's q
  const float* qlogits;    // the drafter's logits [B][N-1][V] (fp32)
  const float* qpart;      // rows pass over qlogits / tau: [B][N-1][n_chunks][2]
  float inv_tau;
  float* dpart;            // draft sampling: [B][N-1][s_n_chunks][2]
  int* draft_out;          // draft sampling: [B][N-1]
};

// Kernel timer hook: while `start` is non-null, every single-kernel launcher
// launches through hipExtLaunchKernel with these events, which then hold the
// kernel's own start and end (no dispatch gap in the measured duration).
struct LaunchEvents {
  hipEvent_t start;
  hipEvent_t stop;
};
extern thread_local LaunchEvents dflash_launch_events;


extern "C" {
hipError_t dflash_launch_ws(const WsArgs* a, int mode, hipStream_t st);
hipError_t dflash_launch_mm(const WsArgs* a, int mode, hipStream_t st);
hipError_t dflash_launch_swiglu_finish(const WsArgs* a, hipStream_t st);
hipError_t dflash_launch_pack(const PackArgs* a, hipStream_t st);
hipError_t dflash_launch_qkv_finish(const QkvFinishArgs* a, hipStream_t st);
hipError_t dflash_launch_ctx_finish(const CtxFinishArgs* a, hipStream_t st);
hipError_t dflash_launch_attn(const AttnArgs* a, int B, int head_dim, hipStream_t st);
hipError_t dflash_launch_attn_merge(const AttnArgs* a, int B, int head_dim, hipStream_t st);
hipError_t dflash_launch_fuse(const FuseArgs* a, hipStream_t st);
hipError_t dflash_launch_norm(const NormArgs* a, hipStream_t st);
hipError_t dflash_launch_fuse_norm(const FuseArgs* fa, const NormArgs* na, hipStream_t st);
hipError_t dflash_launch_finish2(const CtxFinishArgs* ca, const QkvFinishArgs* qa, hipStream_t st);
hipError_t dflash_launch_fill(uint32_t* p, size_t n, uint32_t v, hipStream_t st);
hipError_t dflash_launch_lmhead(const LmArgs* a, hipStream_t st);
hipError_t dflash_launch_lmhead_mm(const LmArgs* a, hipStream_t st);
hipError_t dflash_launch_argmax(const ArgmaxArgs* a, hipStream_t st);
hipError_t dflash_launch_verify(const VerifyArgs* a, hipStream_t st);
hipError_t dflash_launch_draft_sample(const VerifyArgs* a, hipStream_t st);
hipError_t dflash_launch_d2sd_select(const D2sdArgs* a, hipStream_t st);
hipError_t dflash_launch_d2sd_assemble(const D2sdArgs* a, hipStream_t st);
hipError_t dflash_launch_pick(const PickArgs* a, hipStream_t st);
hipError_t dflash_verify_scratch_setup(int device);
float* dflash_verify_scratch(int device);
}
