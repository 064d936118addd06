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

#define FUSE_MAXV 2   // float4 groups per thread: H <= 1024 * 4 * 2
#define FUSE_TMAX 16  // target layers

// One workgroup per (appended row m = b*max_new + t, draft layer i), one
// float4 group of the row per thread. While the row's T target states are
// in flight, thread 0 plans the row: sequence b's checks (sequence id,
// n_new, position capacity; its page-table entries are checked by the first
// threads) give position ctx_len + t, or -1 if t >= n_new or a check fails
// (the whole sequence is then skipped and its error bits set once, by row
// t = 0 of layer 0). Layer 0 records the positions for the context
// finisher, which advances ctx_len. Then s = sum_j alpha[i][j] * h_j
// (ascending j), f = s / sqrt(mean(s^2) + eps) * g, written as the packed
// split activation of the context K/V projection.
__global__ __launch_bounds__(1024) LATENCY_BOUND void fuse_kernel(FuseArgs a) {
  const int m = blockIdx.x, i = blockIdx.y;
  const int b = m / a.max_new, t = m % a.max_new;
  __shared__ float red[16];
  __shared__ int plan[4];  // seq, L, n, bad
  // the row's first 8 target states (this thread's first float4 group) are
  // requested before the plan, which takes three dependent reads
  const uint16_t* h = a.hidden + (size_t)m * a.T * a.H;
  const int kq = min((int)threadIdx.x * 4, a.H - 4);  // clamped: no branch around loads
  u16x4 pre[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) pre[j] = *reinterpret_cast<const u16x4*>(h + (size_t)min(j, a.T - 1) * a.H + kq);
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
  const int bad = plan[3];
  const int pos = (!bad && t < plan[2]) ? plan[1] + t : -1;
  if (i == 0 && threadIdx.x == 0) {
    a.row_pos[m] = pos;
    a.row_seq[m] = plan[0];
    if (t == 0 && bad) set_error(a.err, bad);
  }
  if (pos < 0) return;
  const float* al = a.alpha + (size_t)i * a.T;
  const int nv = (a.H / 4 + blockDim.x - 1) / blockDim.x;
  float s[FUSE_MAXV][4];
  float ss = 0.f;
#pragma unroll
  for (int v = 0; v < FUSE_MAXV; ++v) {
    const int k = min((v * (int)blockDim.x + (int)threadIdx.x) * 4, a.H - 4);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j0 = 0; j0 < FUSE_TMAX; j0 += 8) {  // T <= FUSE_TMAX: at most two batches
      if (j0 >= a.T) break;
      u16x4 x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        x[j] = (v == 0 && j0 == 0) ? pre[j]
                                   : *reinterpret_cast<const u16x4*>(h + (size_t)min(j0 + j, a.T - 1) * a.H + k);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j0 + j >= a.T) break;
        const float w = al[j0 + j];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += w * bf2f(x[j][e]);
      }
    }
    const bool mine = v < nv && (v * (int)blockDim.x + (int)threadIdx.x) * 4 < a.H;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s[v][e] = acc[e];
      if (mine) ss += acc[e] * acc[e];
    }
  }
  const float tot = block_sum(ss, red);
  const float rstd = 1.0f / sqrtf(tot / a.H + a.eps);
  const size_t plane = act_plane(a.rows, a.H);
  uint16_t* out = a.f + (size_t)i * 2 * plane;
  const uint16_t* g = a.g_fuse + (size_t)i * a.H;
#pragma unroll
  for (int v = 0; v < FUSE_MAXV; ++v) {
    const int k = (v * blockDim.x + threadIdx.x) * 4;
    if (v >= nv || k >= a.H) continue;
    const u16x4 gv = *reinterpret_cast<const u16x4*>(g + k);
    f32x4 y;
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = s[v][e] * rstd * bf2f(gv[e]);
    u16x4 hi, lo;
    split4(y, hi, lo);
    *reinterpret_cast<u16x4*>(out + pk_index(m, k, a.H)) = hi;
    *reinterpret_cast<u16x4*>(out + plane + pk_index(m, k, a.H)) = lo;
  }
}

extern "C" hipError_t dflash_launch_fuse(const FuseArgs* a, hipStream_t st) {
  const int threads = std::min(1024, ((a->H / 4 + 63) / 64) * 64);
  launch_kernel(fuse_kernel, dim3(a->rows, a->D), dim3(threads), 0, st, *a);
  return hipGetLastError();
}

// ------------------------------------------------------------- norm

#define NORM_MAXV 2  // float4 groups per thread: H <= 1024 * 4 * 2

// One workgroup per row, one float4 of the row per thread: build the
// residual row (embedding gather, or x + the k-split partials of the last
// projection, summed in split order), then h = x / sqrt(mean(x^2) + eps) * g
// as the packed split activation the next projection streams. Mode 0 (first kernel of a draft call) also checks the call's
// sequence ids, anchors and position capacity.
__global__ __launch_bounds__(1024) LATENCY_BOUND void norm_kernel(NormArgs a) {
  const int m = blockIdx.x;
  __shared__ float red[16];
  const int nv = (a.H / 4 + blockDim.x - 1) / blockDim.x;
  float xv[NORM_MAXV][4];
  float ss = 0.f;
  int tok = 0;
  if (a.mode == 0) {
    const int b = m / a.N;
    tok = (m % a.N == 0) ? a.anchor[b] : a.mask_id;
    if (threadIdx.x == 0 && m % a.N == 0) {
      int bad = 0;
      const int s_raw = a.seq_ids[b];
      if (s_raw < 0 || s_raw >= a.max_seqs) bad |= DFLASH_DEV_BAD_SEQ;
      if (tok < 0 || tok >= a.V) bad |= DFLASH_DEV_BAD_TOKEN;
      const int L = a.ctx_len[clampi(s_raw, 0, a.max_seqs - 1)];
      if (L < 0 || L + a.N > a.max_pos) bad |= DFLASH_DEV_NO_PAGES;
      if (bad) set_error(a.err, bad);
    }
    tok = clampi(tok, 0, a.V - 1);
  }
  const size_t split_stride = (size_t)a.M * a.H;
#pragma unroll
  for (int v = 0; v < NORM_MAXV; ++v) {
    const int k = (v * blockDim.x + threadIdx.x) * 4;
    if (v >= nv || k >= a.H) continue;
    f32x4 x;
    if (a.mode == 0) {
      const u16x4 e = *reinterpret_cast<const u16x4*>(a.embed + (size_t)tok * a.H + k);
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = bf2f(e[i]);
    } else {
      x = *reinterpret_cast<const f32x4*>(a.x + (size_t)m * a.H + k);
      x += split_sum4(a.part, a.ks, split_stride, (size_t)m * a.H + k);
    }
    *reinterpret_cast<f32x4*>(a.x + (size_t)m * a.H + k) = x;
    if (a.dbg) *reinterpret_cast<f32x4*>(a.dbg + (size_t)m * a.H + k) = x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xv[v][i] = x[i];
      ss += x[i] * x[i];
    }
  }
  const float tot = block_sum(ss, red);
  const float rstd = 1.0f / sqrtf(tot / a.H + a.eps);
#pragma unroll
  for (int v = 0; v < NORM_MAXV; ++v) {
    const int k = (v * blockDim.x + threadIdx.x) * 4;
    if (v >= nv || k >= a.H) continue;
    const u16x4 gv = *reinterpret_cast<const u16x4*>(a.g + k);
    f32x4 y;
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = xv[v][i] * rstd * bf2f(gv[i]);
    u16x4 hi, lo;
    split4(y, hi, lo);
    *reinterpret_cast<u16x4*>(a.h + pk_index(m, k, a.H)) = hi;
    *reinterpret_cast<u16x4*>(a.h + act_plane(a.M, a.H) + pk_index(m, k, a.H)) = lo;
  }
}

extern "C" hipError_t dflash_launch_norm(const NormArgs* a, hipStream_t st) {
  const int threads = std::min(1024, ((a->H / 4 + 63) / 64) * 64);
  launch_kernel(norm_kernel, dim3(a->M), dim3(threads), 0, st, *a);
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
