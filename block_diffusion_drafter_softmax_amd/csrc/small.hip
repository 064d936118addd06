// Small per-row kernels: call planning (positions, bounds checks), DFLARE
// layer fusion + RMSNorm, and the residual/embedding + RMSNorm producer of
// every GEMM input.
#include <algorithm>

#include "common.h"
#include "dflash.h"

namespace {
DEV int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }
}


// One thread per batch entry. Append: rows t < n_new[b] get positions
// ctx_len .. ctx_len+n_new-1 and ctx_len advances; a failed check leaves the
// sequence untouched and all its rows skipped. Draft: rows get positions
// L .. L+N-1; checks only flag (positions are clamped into the tables).
__global__ LATENCY_BOUND void plan_kernel(PlanArgs a) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= a.B) return;
  int bad = 0;
  const int s_raw = a.seq_ids[b];
  if (s_raw < 0 || s_raw >= a.max_seqs) bad |= DFLASH_DEV_BAD_SEQ;
  const int seq = clampi(s_raw, 0, a.max_seqs - 1);
  const int L_raw = a.ctx_len[seq];
  const int cap = min(a.max_pages_per_seq * 16, a.max_pos);
  if (L_raw < 0 || L_raw > cap) bad |= DFLASH_DEV_NO_PAGES;
  const int L = clampi(L_raw, 0, cap);
  int n = a.rows_per_seq;
  if (a.append) {
    n = a.n_new[b];
    if (n < 0 || n > a.max_new) bad |= DFLASH_DEV_BAD_N_NEW;
    if (!bad && L + n > cap) bad |= DFLASH_DEV_NO_PAGES;
    if (!bad) {
      for (int p = L / 16; p < (L + n + 15) / 16; ++p) {
        const int pg = a.page_table[(size_t)seq * a.max_pages_per_seq + p];
        if (pg < 0 || pg >= a.n_pages) bad |= DFLASH_DEV_BAD_PAGE;
      }
    }
  } else {
    // context pages are validated by the attention kernel that reads them
    if (L + n > a.max_pos) bad |= DFLASH_DEV_NO_PAGES;
    const int anc = a.anchor[b];
    if (anc < 0 || anc >= a.vocab) bad |= DFLASH_DEV_BAD_TOKEN;
  }
  if (bad) set_error(a.err, bad);
  for (int t = 0; t < a.rows_per_seq; ++t) {
    int pos;
    if (a.append) pos = (!bad && t < n) ? L + t : -1;
    else pos = clampi(L + t, 0, a.max_pos - 1);
    a.row_pos[b * a.rows_per_seq + t] = pos;
    a.row_seq[b * a.rows_per_seq + t] = seq;
  }
  if (a.append && !bad) a.ctx_len[seq] = L + n;
}

extern "C" hipError_t dflash_launch_plan(const PlanArgs* a, hipStream_t st) {
  launch_kernel(plan_kernel, dim3((a->B + 63) / 64), dim3(64), 0, st, *a);
  return hipGetLastError();
}

// ------------------------------------------------------------ fusion

#define FUSE_MAXV 2   // float4 groups per thread: H <= 1024 * 4 * 2
#define FUSE_DMAX 64  // draft layers whose fusion weights fit the LDS table
#define FUSE_TMAX 16  // target layers

// One workgroup per appended row, one float4 group of the row per thread.
// For each draft layer i: s = sum_j alpha[i][j] * h_j (ascending j; the T
// states are re-read per layer from cache, 8 loads in flight per batch),
// f = s / sqrt(mean(s^2) + eps) * g, written as the packed split activation
// of the context K/V projection. The fusion weights are staged in LDS once.
__global__ __launch_bounds__(1024) LATENCY_BOUND void fuse_kernel(FuseArgs a) {
  const int m = blockIdx.x;
  if (a.row_pos[m] < 0) return;
  __shared__ float red[16];
  __shared__ float alpha[FUSE_DMAX * FUSE_TMAX];
  for (int i = threadIdx.x; i < a.D * a.T; i += blockDim.x) alpha[i] = a.alpha[i];
  __syncthreads();
  const uint16_t* h = a.hidden + (size_t)m * a.T * a.H;
  const int nv = (a.H / 4 + blockDim.x - 1) / blockDim.x;
  for (int i = 0; i < a.D; ++i) {
    float s[FUSE_MAXV][4];
    float ss = 0.f;
#pragma unroll
    for (int v = 0; v < FUSE_MAXV; ++v) {
      const int k = (v * (int)blockDim.x + (int)threadIdx.x) * 4;
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
      if (v < nv && k < a.H) {
#pragma unroll 8
        for (int j = 0; j < a.T; ++j) {
          const u16x4 x = *reinterpret_cast<const u16x4*>(h + (size_t)j * a.H + k);
          const float al = alpha[i * a.T + j];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] += al * bf2f(x[e]);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s[v][e] = acc[e];
        ss += acc[e] * acc[e];
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
}

extern "C" hipError_t dflash_launch_fuse(const FuseArgs* a, hipStream_t st) {
  const int threads = std::min(1024, ((a->H / 4 + 63) / 64) * 64);
  launch_kernel(fuse_kernel, dim3(a->rows), dim3(threads), 0, st, *a);
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
