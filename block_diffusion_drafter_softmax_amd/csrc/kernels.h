// Kernel argument structs and launchers shared by the HIP kernels and the
// host library (plain data: no device code here).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

// Top-2 with index: (v1, i1) is the maximum, lowest index on ties; v2 is
// the largest value among the remaining entries.
struct Top2 {
  float v1;
  int i1;
  float v2;
};

// ------------------------------------------------------------ GEMM args
// Tile pairing of the two 16-row weight tiles a wave multiplies.
enum PairMode : int {
  PAIR_PLAIN = 0,  // rows 32p .. 32p+15 and 32p+16 .. 32p+31 of w0
  PAIR_ROPE = 1,   // rows j and j + d_h/2 of one head (rotation partners)
  PAIR_DUAL = 2,   // rows 16p .. 16p+15 of w0 and of w1 (gate, up)
};

enum Epilogue : int {
  EPI_PARTIAL = 0,  // fp32 partial sums [split][M][n_out] (residual added by the next norm)
  EPI_Q = 1,        // RoPE -> bf16 q [M][n_q*d_h]
  EPI_KBLK = 2,     // RoPE -> bf16 block keys [B][n_kv][16][d_h]
  EPI_VBLK = 3,     // bf16 block values, dim-major [B][n_kv][d_h][16]
  EPI_SWIGLU = 4,   // bf16 silu(gate) * up [M][I]
  EPI_CTX_K = 5,    // RoPE -> bf16 into the key part of the row's page slot
  EPI_CTX_V = 6,    // bf16 into the value part of the row's page slot
};

#define GEMM_MAX_SEG 16

struct GemmSeg {
  const uint16_t* w0;
  const uint16_t* w1;
  const uint16_t* act;  // [M][K] bf16
  void* out;
  int pairs;
  int mode;
  int epi;
  int layer;
};

struct GemmArgs {
  GemmSeg seg[GEMM_MAX_SEG];
  int seg_start[GEMM_MAX_SEG + 1];
  int nseg;
  int K;          // reduction length (multiple of 32)
  int M;          // activation rows
  int ks;         // splits of K across workgroups
  int n_out;      // output columns for EPI_PARTIAL
  int head_dim;
  int n_kv;
  int block;      // N, rows per sequence in the draft
  int max_pages_per_seq;
  int n_pages;
  int max_pos;
  const int* row_pos;   // [M] position of each row, < 0: skip the row
  const int* row_seq;   // [M] sequence id of each row
  const int* page_table;
  uint16_t* kv_pages;
  long long layer_stride;  // elements per layer of kv_pages
  const float* rope;       // [max_pos][d_h/2][2] (cos, sin)
};

struct AttnArgs {
  const uint16_t* q;       // [B*N][n_q][d]
  const uint16_t* kblk;    // [B][n_kv][16][d]
  const uint16_t* vblk;    // [B][n_kv][d][16]
  const uint16_t* pages;   // this layer's pages [n_pages][2][n_kv][16*d]
  const int* page_table;
  const int* ctx_len;
  const int* seq_ids;
  float* part_o;           // [B][n_kv][n_ck][R][d]
  float* part_ml;          // [B][n_kv][n_ck][R][2]
  uint16_t* o;             // merge output [B*N][n_q*d]
  int N, n_q, n_kv, chunk, n_ck, max_pages_per_seq, n_pages, max_seqs;
  float scale_log2;        // log2(e) / sqrt(d)
};

struct PlanArgs {
  int B, rows_per_seq;  // max_new (append) or N (draft)
  const int* seq_ids;
  const int* n_new;     // append only
  const int* anchor;    // draft only
  int* ctx_len;
  const int* page_table;
  int max_seqs, max_pages_per_seq, n_pages, max_pos, max_new, vocab;
  int* row_pos;         // [B*rows_per_seq]
  int* row_seq;
  int32_t* err;
  int append;           // 1: append plan (advances ctx_len), 0: draft plan
};

struct FuseArgs {
  const uint16_t* hidden;  // [rows][T][H]
  const float* alpha;      // [D][T]
  const uint16_t* g_fuse;  // [D][H]
  uint16_t* f;             // [D][rows][H]
  const int* row_pos;
  int rows, T, H, D;
  float eps;
};

struct NormArgs {
  int mode;                // 0: x = embedding rows, 1: x += sum of split partials
  const uint16_t* embed;   // [V][H]
  const int* anchor;       // [B]
  int mask_id, N, V;
  float* x;                // [M][H] residual stream (fp32)
  const float* part;       // [ks][M][H]
  int ks;
  const uint16_t* g;       // gain [H]
  uint16_t* h;             // [M][H] bf16 out
  float* dbg;              // nullable [M][H]
  int H, M;
  float eps;
};

struct LmArgs {
  const uint16_t* w;    // [V][K]
  const uint16_t* act;  // [M][K] normed rows
  int M, K, V, N;       // N = block rows per sequence
  Top2* part;           // [n_wg][M]
  float* dbg_logits;    // nullable [B][N-1][V]
};

struct ArgmaxArgs {
  const Top2* part;  // [n_wg][M]
  int n_wg, M, N, V;
  int* draft;        // [B][N-1]
  float* gap;        // nullable [B][N-1]
  int32_t* err;
};

struct VerifyArgs {
  const void* logits;   // [B][N][V]
  int dtype;            // DFLASH_DTYPE_*
  int B, N, V, chunk, n_chunks;
  const int* seq_ids;
  const int* draft;     // [B][N-1]
  float* part;          // [B][N][n_chunks][2]
  int* counters;        // [2*B], zero between calls
  int* state;           // [B][2]: sample row, excluded token
  int* accept_len;
  int* next_token;
  int* commit_len;      // nullable
  int temp1;
  unsigned long long seed, step;
  int32_t* err;
};

extern "C" {
hipError_t dflash_launch_gemm(const GemmArgs* args, int total_pairs, int kw, hipStream_t st);
hipError_t dflash_launch_attn(const AttnArgs* a, int B, int head_dim, hipStream_t st);
hipError_t dflash_launch_attn_merge(const AttnArgs* a, int B, int head_dim, hipStream_t st);
hipError_t dflash_launch_plan(const PlanArgs* a, hipStream_t st);
hipError_t dflash_launch_fuse(const FuseArgs* a, hipStream_t st);
hipError_t dflash_launch_norm(const NormArgs* a, hipStream_t st);
hipError_t dflash_launch_fill(uint32_t* p, size_t n, uint32_t v, hipStream_t st);
hipError_t dflash_launch_lmhead(const LmArgs* a, hipStream_t st);
hipError_t dflash_launch_argmax(const ArgmaxArgs* a, hipStream_t st);
hipError_t dflash_launch_verify(const VerifyArgs* a, hipStream_t st);
}
