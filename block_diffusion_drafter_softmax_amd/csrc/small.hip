// Small per-row kernels: call planning (positions, bounds checks), DFLARE
// layer fusion + RMSNorm, and the residual/embedding + RMSNorm producer of
// every GEMM input.
#include <algorithm>

#include "common.h"
#include "dflash.h"

namespace {
DEV int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }
}


// ------------------------------------------------------------ fusion

#define FUSE_TMAX 16  // target layers
#define FUSE_DMAX 64  // draft layers (the host accepts up to 64)

// One workgroup per (appended row m = b*max_new + t, group of DG draft
// layers), MAXV float4 groups of the row per thread: DG = 1 (a workgroup
// per layer) while rows are few, all layers of a row in one workgroup when
// there are enough rows to fill the chip. While the row's T target states are in flight,
// thread 0 plans the row: sequence b's checks (sequence id, n_new, position
// capacity; its page-table entries are checked by the first threads) give
// position ctx_len + t, or -1 if t >= n_new or a check fails (the whole
// sequence is then skipped and its error bits set once, by row t = 0). The
// positions are recorded for the context finisher, which advances ctx_len.
// The T states stay in registers while, for every draft layer i of the
// group (one workgroup reduction for the group), s = sum_j alpha[i][j] * h_j
// (ascending j) and f = s / sqrt(mean(s^2) + eps) * g are formed and written
// as the packed split activation of the context K/V projection.
// Append plan of sequence b (a whole workgroup takes part; two barriers):
// plan = (sequence, context length before the append (clamped), rows the
// append writes, error bits). A failed check skips the whole append.
DEV void append_plan(const FuseArgs& a, int b, int* plan) {
  if (threadIdx.x == 0) {
    int bad = 0;
    const int s_raw = a.seq_ids[b];
    if (s_raw < 0 || s_raw >= a.max_seqs) bad |= DFLASH_DEV_BAD_SEQ;
    const int seq = clampi(s_raw, 0, a.max_seqs - 1);
    const int L_raw = a.ctx_len[seq];
    const int cap = min(a.max_pages_per_seq * 16, a.max_pos);
    if (L_raw < 0 || L_raw > cap) bad |= DFLASH_DEV_NO_PAGES;
    const int L = clampi(L_raw, 0, cap);
    const int n = a.n_new[b];
    if (n < 0 || n > a.max_new) bad |= DFLASH_DEV_BAD_N_NEW;
    if (!bad && L + n > cap) bad |= DFLASH_DEV_NO_PAGES;
    plan[0] = seq;
    plan[1] = L;
    plan[2] = bad ? 0 : n;
    plan[3] = bad;
  }
  __syncthreads();
  {  // page-table entries the sequence's append writes to (one per thread)
    const int L = plan[1], n = plan[2];
    for (int p = L / 16 + (int)threadIdx.x; n > 0 && p < (L + n + 15) / 16; p += blockDim.x) {
      const int pg = a.page_table[(size_t)plan[0] * a.max_pages_per_seq + p];
      if (pg < 0 || pg >= a.n_pages) atomicOr(&plan[3], DFLASH_DEV_BAD_PAGE);
    }
  }
  __syncthreads();
}

template <int MAXV, int DG>
DEV void fuse_body(const FuseArgs& a, int m, int i0) {
  const int b = m / a.max_new, t = m % a.max_new;
  __shared__ float red[16][DG];
  __shared__ float al_s[FUSE_DMAX * FUSE_TMAX];  // alpha, [layer][j], zero past T
  __shared__ int plan[4];  // seq, L, n, bad
  // the row's target states are requested before the plan, which takes
  // three dependent reads
  const uint16_t* h = a.hidden + (size_t)m * a.T * a.H;
  u16x4 x[MAXV][FUSE_TMAX];
#pragma unroll
  for (int v = 0; v < MAXV; ++v) {
    const int k = min((v * (int)blockDim.x + (int)threadIdx.x) * 4, a.H - 4);  // clamped: no branch around loads
#pragma unroll
    for (int j = 0; j < FUSE_TMAX; ++j) x[v][j] = *reinterpret_cast<const u16x4*>(h + (size_t)min(j, a.T - 1) * a.H + k);
  }
  for (int q = threadIdx.x; q < FUSE_DMAX * FUSE_TMAX; q += blockDim.x) {
    const int i = q / FUSE_TMAX, j = q % FUSE_TMAX;
    al_s[q] = (i < a.D && j < a.T) ? a.alpha[(size_t)i * a.T + j] : 0.f;  // weights past T are 0
  }
  append_plan(a, b, plan);
  const int bad = plan[3];
  const int pos = (!bad && t < plan[2]) ? plan[1] + t : -1;
  if (blockIdx.y == 0 && threadIdx.x == 0) {
    a.row_pos[m] = pos;
    a.row_seq[m] = plan[0];
    if (t == 0 && bad) set_error(a.err, bad);
  }
  if (pos < 0) return;
  if (a.raw) {  // FC fusion: the row's T states, in layer order, are the FC layer's input row
    const int K = a.T * a.H;
    const size_t plane_k = act_plane(a.rows, K);
    const u16x4 zero = {0, 0, 0, 0};
#pragma unroll
    for (int v = 0; v < MAXV; ++v) {
      const int k = (v * blockDim.x + threadIdx.x) * 4;
      if (k >= a.H) continue;
#pragma unroll
      for (int j = 0; j < FUSE_TMAX; ++j) {  // guarded, not `break`: the loop unrolls, x stays in registers
        if (j < a.T) {
          uint16_t* dst = a.f + pk_index(m, j * a.H + k, K);
          *reinterpret_cast<u16x4*>(dst) = x[v][j];
          *reinterpret_cast<u16x4*>(dst + plane_k) = zero;
        }
      }
    }
    return;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const size_t plane = act_plane(a.rows, a.H);
  {
    float s[DG][MAXV][4];
    float ss[DG];
#pragma unroll
    for (int di = 0; di < DG; ++di) {
      ss[di] = 0.f;
      const float* al = al_s + min(i0 + di, FUSE_DMAX - 1) * FUSE_TMAX;
#pragma unroll
      for (int v = 0; v < MAXV; ++v) {
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < FUSE_TMAX; ++j) {  // ascending j; the clamped states past T weigh 0
          const float w = al[j];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] += w * bf2f(x[v][j][e]);
        }
        const bool mine = (v * (int)blockDim.x + (int)threadIdx.x) * 4 < a.H;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s[di][v][e] = acc[e];
          if (mine) ss[di] += acc[e] * acc[e];
        }
      }
    }
    // one reduction for the group's layers (fixed order: waves, then sum)
#pragma unroll
    for (int di = 0; di < DG; ++di) ss[di] = wave_sum(ss[di]);
    if (lane == 0)
#pragma unroll
      for (int di = 0; di < DG; ++di) red[wave][di] = ss[di];
    __syncthreads();
#pragma unroll
    for (int di = 0; di < DG; ++di) {
      const int i = i0 + di;
      if (i >= a.D) break;
      float tot = 0.f;
      for (int w = 0; w < nw; ++w) tot += red[w][di];
      const float rstd = 1.0f / sqrtf(tot / a.H + a.eps);
      uint16_t* out = a.f + (size_t)i * 2 * plane;
      const uint16_t* g = a.g_fuse + (size_t)i * a.H;
#pragma unroll
      for (int v = 0; v < MAXV; ++v) {
        const int k = (v * blockDim.x + threadIdx.x) * 4;
        if (k >= a.H) continue;
        const u16x4 gv = *reinterpret_cast<const u16x4*>(g + k);
        f32x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = s[di][v][e] * rstd * bf2f(gv[e]);
        u16x4 hi, lo;
        split4(y, hi, lo);
        *reinterpret_cast<u16x4*>(out + pk_index(m, k, a.H)) = hi;
        *reinterpret_cast<u16x4*>(out + plane + pk_index(m, k, a.H)) = lo;
      }
    }
  }
}

template <int MAXV, int DG>
__global__ __launch_bounds__(1024) LATENCY_BOUND void fuse_kernel(FuseArgs a) {
  fuse_body<MAXV, DG>(a, blockIdx.x, blockIdx.y * DG);
}

extern "C" hipError_t dflash_launch_fuse(const FuseArgs* a, hipStream_t st) {
  const int threads = std::min(1024, ((a->H / 4 + 63) / 64) * 64);
  constexpr int DG = 8;
  const int gy = a->raw ? 1 : a->D;  // the FC layer's input: one workgroup per row
  if (a->H > 4 * threads) {  // H > 4096: two float4 groups per thread, one layer per workgroup
    launch_kernel((fuse_kernel<2, 1>), dim3(a->rows, gy), dim3(threads), 0, st, *a);
  } else if (a->rows < 128 || a->raw) {  // few rows: a workgroup per (row, layer)
    launch_kernel((fuse_kernel<1, 1>), dim3(a->rows, gy), dim3(threads), 0, st, *a);
  } else {
    launch_kernel((fuse_kernel<1, DG>), dim3(a->rows, (a->D + DG - 1) / DG), dim3(threads), 0, st, *a);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------- norm

#define NORM_MAXV 2  // float4 groups per thread: H <= 1024 * 4 * 2

// One workgroup per row, one float4 of the row per thread: build the
// residual row (embedding gather, or x + the k-split partials of the last
// projection, summed in split order), then h = x / sqrt(mean(x^2) + eps) * g
// as the packed split activation the next projection streams. Mode 2 norms
// the FC fusion layer's output (its partials alone; no residual). Mode 0 (first
// kernel of a draft call) embeds the block's tokens (the anchor and masks,
// or given input tokens) and also checks the call's sequence ids, tokens
// and position capacity.
// `app` (with_app): the block's context length is the one after the
// append of the same call (checked as the append checks it), for a draft
// launched together with that append.
DEV void norm_body(const NormArgs& a, int m, const FuseArgs& app, bool with_app) {
  __shared__ float red[16];
  const int nv = (a.H / 4 + blockDim.x - 1) / blockDim.x;
  float xv[NORM_MAXV][4];
  float ss = 0.f;
  int tok = 0;
  if (a.mode == 0) {
    const int b = m / a.N, n = m % a.N;
    tok = a.tokens ? a.tokens[m] : (n == 0) ? a.anchor[b] : a.mask_id;
    const int s_raw = a.seq_ids[b];
    const int seq = clampi(s_raw, 0, a.max_seqs - 1);
    int L = a.ctx_len[seq];
    if (with_app) {  // the context length after the append, as its finisher will set it
      __shared__ int ap[4];
      append_plan(app, b, ap);
      if (!ap[3]) L = ap[1] + ap[2];
    }
    if (threadIdx.x == 0) {
      int bad = (tok < 0 || tok >= a.V) ? DFLASH_DEV_BAD_TOKEN : 0;
      if (n == 0) {
        if (s_raw < 0 || s_raw >= a.max_seqs) bad |= DFLASH_DEV_BAD_SEQ;
        if (L < 0 || L + a.N > a.max_pos) bad |= DFLASH_DEV_NO_PAGES;
        a.plan[2 * b] = seq;
        a.plan[2 * b + 1] = L;
      }
      if (bad) set_error(a.err, bad);
    }
    if (n == 0 && a.blk_pages)
      for (int p = threadIdx.x; p < a.max_pages_per_seq; p += blockDim.x)
        a.blk_pages[(size_t)b * a.max_pages_per_seq + p] = a.page_table[(size_t)seq * a.max_pages_per_seq + p];
    if (a.rope && (int)threadIdx.x < a.half) {  // this row's RoPE cos/sin (position L + n)
      const int pos = clampi(L + n, 0, a.max_pos - 1);
      const float2 cs = *reinterpret_cast<const float2*>(a.rope + ((size_t)pos * a.half + threadIdx.x) * 2);
      *reinterpret_cast<float2*>(a.plan_rope + ((size_t)m * a.half + threadIdx.x) * 2) = cs;
    }
    tok = clampi(tok, 0, a.V - 1);
  }
  const size_t split_stride = (size_t)a.M * a.H;
  u16x4 gv[NORM_MAXV];  // the gain, requested with the row (not after the reduction's barriers)
#pragma unroll
  for (int v = 0; v < NORM_MAXV; ++v) {
    const int k = min((v * (int)blockDim.x + (int)threadIdx.x) * 4, a.H - 4);
    gv[v] = *reinterpret_cast<const u16x4*>(a.g + k);
  }
#pragma unroll
  for (int v = 0; v < NORM_MAXV; ++v) {
    const int k = (v * blockDim.x + threadIdx.x) * 4;
    if (v >= nv || k >= a.H) continue;
    f32x4 x;
    if (a.mode == 0) {
      const u16x4 e = *reinterpret_cast<const u16x4*>(a.embed + (size_t)tok * a.H + k);
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = bf2f(e[i]);
    } else if (a.mode == 1) {
      x = *reinterpret_cast<const f32x4*>(a.x + (size_t)m * a.H + k);
      x += split_sum4(a.part, a.ks, split_stride, (size_t)m * a.H + k);
    } else {
      x = split_sum4(a.part, a.ks, split_stride, (size_t)m * a.H + k);
    }
    if (a.mode != 2) *reinterpret_cast<f32x4*>(a.x + (size_t)m * a.H + k) = x;
    if (a.dbg) *reinterpret_cast<f32x4*>(a.dbg + (size_t)m * a.H + k) = x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xv[v][i] = x[i];
      ss += x[i] * x[i];
    }
  }
  const float tot = block_sum(ss, red);
  const float rstd = 1.0f / sqrtf(tot / a.H + a.eps);
  int row = m;  // where the normed row goes
  if (a.row_cut) {  // compacted: only rows n >= the block's cut, blocks in order
    const int b = m / a.N, n = m % a.N;
    float before = 0.f;  // rows kept by the earlier blocks (exact in fp32)
    for (int t = threadIdx.x; t < b; t += blockDim.x) before += (float)(a.N - a.row_cut[t]);
    before = block_sum(before, red);
    const int c = a.row_cut[b];
    row = n >= c ? (int)before + n - c : -1;
    if (threadIdx.x == 0 && row >= 0) {
      a.row_inv[row] = m;
      if (m == a.M - 1) *a.row_count = row + 1;  // the last row of the last block is always kept
    }
    if (row < 0) return;
  }
#pragma unroll
  for (int v = 0; v < NORM_MAXV; ++v) {
    const int k = (v * blockDim.x + threadIdx.x) * 4;
    if (v >= nv || k >= a.H) continue;
    f32x4 y;
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = xv[v][i] * rstd * bf2f(gv[v][i]);
    u16x4 hi, lo;
    split4(y, hi, lo);
    *reinterpret_cast<u16x4*>(a.h + pk_index(row, k, a.H)) = hi;
    *reinterpret_cast<u16x4*>(a.h + act_plane(a.M, a.H) + pk_index(row, k, a.H)) = lo;
  }
}

// From 128 rows on, the 16 rows of one tile of the packed output are
// normed on one XCD (the hardware deals workgroups to the 8 XCDs round
// robin): a row's 16-byte pieces share cache lines with the other rows of
// its tile, and those partial-line writes then merge in one L2.
// (A separate instantiation: the plain one-row-per-workgroup kernel of small
// batches stays as it was; the extra branch cost it time.)
template <bool XCD_TILES>
__global__ __launch_bounds__(1024) LATENCY_BOUND void norm_kernel(NormArgs a) {
  int m = blockIdx.x;
  if constexpr (XCD_TILES) {
    const int local = blockIdx.x >> 3;
    m = ((local >> 4) * 8 + (int)(blockIdx.x & 7)) * 16 + (local & 15);
    if (m >= a.M) return;
  }
  norm_body(a, m, FuseArgs{}, false);
}

extern "C" hipError_t dflash_launch_norm(const NormArgs* a, hipStream_t st) {
  const int threads = std::min(1024, ((a->H / 4 + 63) / 64) * 64);
  if (a->M >= 128) launch_kernel(norm_kernel<true>, dim3((a->M + 127) / 128 * 128), dim3(threads), 0, st, *a);
  else launch_kernel(norm_kernel<false>, dim3(a->M), dim3(threads), 0, st, *a);
  return hipGetLastError();
}

// Append and draft launched together: the fusion's workgroups (as
// fuse_kernel, row-major over (row, layer group)) and the draft's first norm
// (embedding; the context length the append leaves) in one launch. Both
// use the same workgroup size (one float4 of a hidden row per thread).
// XCD_TILES (appended rows and block rows multiples of 128): the 16 rows
// of one tile of either packed output on one XCD, as in norm_kernel.
DEV int xcd_tile_row(int i) {
  const int local = i >> 3;
  return ((local >> 4) * 8 + (i & 7)) * 16 + (local & 15);
}

template <int MAXV, int DG, bool XCD_TILES>
__global__ __launch_bounds__(1024) LATENCY_BOUND void fuse_norm_kernel(FuseArgs fa, NormArgs na, int n_fuse) {
  const int x = blockIdx.x;
  if (x < n_fuse) {
    const int r = x % fa.rows;
    fuse_body<MAXV, DG>(fa, XCD_TILES ? xcd_tile_row(r) : r, (x / fa.rows) * DG);
  } else {
    norm_body(na, XCD_TILES ? xcd_tile_row(x - n_fuse) : x - n_fuse, fa, true);
  }
}

extern "C" hipError_t dflash_launch_fuse_norm(const FuseArgs* fa, const NormArgs* na, hipStream_t st) {
  const int threads = std::min(1024, ((fa->H / 4 + 63) / 64) * 64);
  constexpr int DG = 8;
  if (fa->raw || na->mode != 0 || na->H != fa->H) return hipErrorInvalidValue;
  if (fa->H > 4 * threads) {
    const int n_fuse = fa->rows * fa->D;
    launch_kernel((fuse_norm_kernel<2, 1, false>), dim3(n_fuse + na->M), dim3(threads), 0, st, *fa, *na, n_fuse);
  } else if (fa->rows < 128) {
    const int n_fuse = fa->rows * fa->D;
    launch_kernel((fuse_norm_kernel<1, 1, false>), dim3(n_fuse + na->M), dim3(threads), 0, st, *fa, *na, n_fuse);
  } else {
    const int n_fuse = fa->rows * ((fa->D + DG - 1) / DG);
    if (fa->rows % 128 == 0 && na->M % 128 == 0)  // n_fuse a multiple of 8: both parts keep the XCD of their index
      launch_kernel((fuse_norm_kernel<1, DG, true>), dim3(n_fuse + na->M), dim3(threads), 0, st, *fa, *na, n_fuse);
    else
      launch_kernel((fuse_norm_kernel<1, DG, false>), dim3(n_fuse + na->M), dim3(threads), 0, st, *fa, *na, n_fuse);
  }
  return hipGetLastError();
}

// Fill a device buffer with 32-bit words (used at set-up; no memset nodes).
__global__ void fill_u32_kernel(uint32_t* p, size_t n, uint32_t v) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}

extern "C" hipError_t dflash_launch_fill(uint32_t* p, size_t n, uint32_t v, hipStream_t st) {
  if (n == 0) return hipSuccess;
  launch_kernel(fill_u32_kernel, dim3(256), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}
