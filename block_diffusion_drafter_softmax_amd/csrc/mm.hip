// Tiled MFMA GEMM for many activation rows: y[m][n] = sum_k x[m][k] * W[n][k],
// x a split (hi + lo) activation, W bf16, both in the packed operand layout.
//
// When a call carries many block rows (a batch of sequences, or a context
// append of hundreds of rows) every weight byte meets M >= 64 activation rows
// and the product is bound by the matrix cores, not by the weight stream.
// Each workgroup of 4 waves computes a 128 x 128 output tile: 8 activation
// tiles, staged through LDS in chunks of MM_KC k steps (double buffered,
// read by every wave), times 8 weight tiles that the waves load straight
// from memory one chunk ahead. Wave (wm, wn) owns activation tiles
// 4wm..4wm+3 and weight tiles 4wn..4wn+3: per k step 8 LDS reads, 4 global
// loads and 32 MFMA 16x16x32 (hi and lo halves of 16 tile products).
// Workgroups of one column block (same weights, different row blocks) are
// placed on one XCD and dispatched together, so the weights leave HBM about
// once per call. Narrow products whose tiles would not fill the chip split
// k (fp32 partials per split, added in split order by the consumer). The
// epilogues are those of the streaming GEMM (fp32 partials, or SwiGLU into
// the next split activation; after a k split the gate and up partials go to
// swiglu_finish_kernel) and the LM head's top-2 reduction.
#include "stream.h"

#define MM_T 8   // activation tiles and weight tiles per workgroup
#define MM_KC 2  // k steps per LDS chunk

namespace {

constexpr int kChunkBlocks = MM_KC * MM_T * 2;  // 1 KB blocks per chunk: (k step, tile, plane)

// Workgroup -> (column block, k split, row block). The grid is a multiple
// of 8 and the hardware deals workgroups to the 8 XCDs round robin;
// renumbering puts the row blocks of one (column block, split) -- the
// workgroups that read the same weights -- next to each other on one XCD.
DEV bool mm_place(int total, int MB, int ks, int& nb, int& split, int& mb) {
  const int per = (int)(gridDim.x >> 3);
  const int L = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
  if (L >= total) return false;
  mb = L % MB;
  split = (L / MB) % ks;
  nb = L / MB / ks;
  return true;
}

struct MmLoop {
  const uint16_t* pw[4];  // this wave's weight tiles at the split's first k step, + lane*8
  const uint16_t* xg[4];  // this thread's activation sources at that k step (see mm_store_x)
  int steps;              // k steps of the split
};

template <int KC>
DEV void mm_load_w(bf16x8 (&w)[KC][4], const MmLoop& p, int c) {
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    const int s = min(c * KC + kc, p.steps - 1);
#pragma unroll
    for (int t = 0; t < 4; ++t)
      w[kc][t] = *reinterpret_cast<const bf16x8*>(p.pw[t] + (size_t)s * 512);
  }
}

template <int KC>
DEV void mm_load_x(u32x4 (&st)[KC][4], const MmLoop& p, int c) {
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    const int s = min(c * KC + kc, p.steps - 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) st[kc][j] = *reinterpret_cast<const u32x4*>(p.xg[j] + (size_t)s * 512);
  }
}

// Chunk block (kc, tile t, plane p) sits at LDS block kc*16 + 2t + p. Thread
// (wave w, lane) moves blocks kc*16 + 4j + w, i.e. tile (w>>1) + 2j, plane w&1.
template <int KC>
DEV void mm_store_x(u32x4* xs, const u32x4 (&st)[KC][4]) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int kc = 0; kc < KC; ++kc)
#pragma unroll
    for (int j = 0; j < 4; ++j) xs[(kc * 16 + 4 * j + w) * 64 + lane] = st[kc][j];
}

template <int KC>
DEV void mm_compute(const u32x4* xs, const bf16x8 (&w)[KC][4], int c, int steps, int wm, f32x4 (&acc)[4][4]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    if (c * KC + kc >= steps) break;
    bf16x8 xh[4], xl[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xh[i] = __builtin_bit_cast(bf16x8, xs[(kc * 16 + (4 * wm + i) * 2) * 64 + lane]);
      xl[i] = __builtin_bit_cast(bf16x8, xs[(kc * 16 + (4 * wm + i) * 2 + 1) * 64 + lane]);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[t][i] = mfma16(w[kc][t], xh[i], acc[t][i]);
        acc[t][i] = mfma16(w[kc][t], xl[i], acc[t][i]);
      }
  }
}

// acc[t][i]: weight tile t of this wave by activation tile i of this wave.
DEV void mm_ksteps(const MmLoop& p, u32x4 (*xs)[kChunkBlocks * 64], int wm, f32x4 (&acc)[4][4]) {
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[t][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int n_chunks = (p.steps + MM_KC - 1) / MM_KC;
  bf16x8 wa[MM_KC][4], wb[MM_KC][4];
  u32x4 st[MM_KC][4];
  mm_load_w(wa, p, 0);
  mm_load_x(st, p, 0);
  mm_store_x(xs[0], st);
  __syncthreads();
  for (int c = 0; c < n_chunks; c += 2) {
    // chunk c: weights in wa, activations in LDS buffer 0
    if (c + 1 < n_chunks) {
      mm_load_w(wb, p, c + 1);
      mm_load_x(st, p, c + 1);
    }
    mm_compute(xs[0], wa, c, p.steps, wm, acc);
    if (c + 1 < n_chunks) mm_store_x(xs[1], st);
    __syncthreads();
    if (c + 1 >= n_chunks) break;
    // chunk c + 1: weights in wb, activations in LDS buffer 1
    if (c + 2 < n_chunks) {
      mm_load_w(wa, p, c + 2);
      mm_load_x(st, p, c + 2);
    }
    mm_compute(xs[1], wb, c + 1, p.steps, wm, acc);
    if (c + 2 < n_chunks) mm_store_x(xs[0], st);
    __syncthreads();
  }
}

// Activation sources of this thread: tile (w>>1) + 2j of the row block
// (clamped to the last real tile), plane w&1, from k step s0 (steps per tile).
DEV void mm_x_sources(MmLoop& p, const uint16_t* act, size_t lo, int mb, int m_tiles, int steps, int s0) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int tm = min(mb * MM_T + (w >> 1) + 2 * j, m_tiles - 1);
    p.xg[j] = act + (w & 1) * lo + ((size_t)tm * steps + s0) * 512 + lane * 8;
  }
}

// Segment of a column block: each segment's units make ceil(units/4) blocks
// (8 tiles of 16 output columns, or 4 SwiGLU feature tiles).
DEV int mm_segment(const WsArgs& a, int& nb) {
  int s = 0;
  while (s + 1 < a.nseg) {
    const int blocks = (a.seg[s].units + 3) >> 2;
    if (nb < blocks) break;
    nb -= blocks;
    ++s;
  }
  return s;
}

}  // namespace

template <int MODE>
__global__ __launch_bounds__(256, 2) void mm_kernel(WsArgs a, int total, int MB) {
  __shared__ u32x4 xs[2][kChunkBlocks * 64];
  int nb, split, mb;
  if (!mm_place(total, MB, a.ks, nb, split, mb)) return;
  const int s = mm_segment(a, nb);
  const WsSeg sg = a.seg[s];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w & 1, wn = w >> 1;
  const int r16 = lane & 15, g4 = (lane >> 4) * 4;
  const int m_tiles = pad16(a.M) >> 4;
  const int steps = a.K >> 5;
  const int s0 = split * steps / a.ks;
  MmLoop p;
  p.steps = (split + 1) * steps / a.ks - s0;
  mm_x_sources(p, sg.act, act_plane(a.M, a.K), mb, m_tiles, steps, s0);
  int col_tile[4];  // PARTIAL: segment tile; SWIGLU: feature tile
  if (MODE == WS_SWIGLU) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      col_tile[t] = nb * 4 + wn * 2 + (t & 1);
      const int f = min(col_tile[t], sg.units - 1);
      p.pw[t] = (t < 2 ? sg.w0 : sg.w1) + ((size_t)f * steps + s0) * 512 + lane * 8;
    }
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      col_tile[t] = nb * 8 + wn * 4 + t;
      const int tl = min(col_tile[t], 2 * sg.units - 1);
      p.pw[t] = sg.w0 + ((size_t)tl * steps + s0) * 512 + lane * 8;
    }
  }
  f32x4 acc[4][4];
  mm_ksteps(p, xs, wm, acc);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tm = mb * MM_T + 4 * wm + i;
    const int m = tm * 16 + r16;
    if (tm >= m_tiles || m >= a.M) continue;
    if (MODE == WS_PARTIAL) {
      float* out = a.part + ((size_t)split * a.M + m) * a.n_cols + sg.col0;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (col_tile[t] < 2 * sg.units) *reinterpret_cast<f32x4*>(out + col_tile[t] * 16 + g4) = acc[t][i];
    } else if (a.ks > 1) {
      float* out = a.part + ((size_t)split * a.M + m) * 2 * a.n_cols + sg.col0;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (col_tile[t] < sg.units)
          *reinterpret_cast<f32x4*>(out + (t >= 2 ? a.n_cols : 0) + col_tile[t] * 16 + g4) = acc[t][i];
    } else {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        if (col_tile[t] >= sg.units) continue;
        f32x4 y;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float gt = acc[t][i][j];
          y[j] = gt / (1.0f + __expf(-gt)) * acc[t + 2][i][j];
        }
        u16x4 hi, lo;
        split4(y, hi, lo);
        uint16_t* dst = a.out + pk_index(m, sg.col0 + col_tile[t] * 16 + g4, a.n_cols);
        *reinterpret_cast<u16x4*>(dst) = hi;
        *reinterpret_cast<u16x4*>(dst + act_plane(a.M, a.n_cols)) = lo;
      }
    }
  }
}

// SwiGLU after a k-split gate/up product: y = silu(sum of gate splits) *
// (sum of up splits), the splits added in order, written as the packed
// split activation of the down projection. One thread per 4 features.
__global__ __launch_bounds__(256) void swiglu_finish_kernel(WsArgs a) {
  const int q = a.n_cols / 4;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= a.M * q) return;
  const int m = idx / q, f = (idx % q) * 4;
  const size_t off = (size_t)m * 2 * a.n_cols + f;
  const size_t stride = (size_t)a.M * 2 * a.n_cols;
  const f32x4 gt = split_sum4(a.part, a.ks, stride, off);
  const f32x4 up = split_sum4(a.part, a.ks, stride, off + a.n_cols);
  f32x4 y;
#pragma unroll
  for (int j = 0; j < 4; ++j) y[j] = gt[j] / (1.0f + __expf(-gt[j])) * up[j];
  u16x4 hi, lo;
  split4(y, hi, lo);
  uint16_t* dst = a.out + pk_index(m, f, a.n_cols);
  *reinterpret_cast<u16x4*>(dst) = hi;
  *reinterpret_cast<u16x4*>(dst + act_plane(a.M, a.n_cols)) = lo;
}

// LM head for many rows: the same tile loop over vocabulary tiles, then a
// top-2 (value, lowest index) per row over the workgroup's 128 vocabulary
// rows, written to part[column block][M]; argmax_reduce_kernel merges them.
__global__ __launch_bounds__(256, 2) void mm_lmhead_kernel(LmArgs a, int total, int MB) {
  __shared__ u32x4 xs[2][kChunkBlocks * 64];
  __shared__ Top2 red[2][MM_T * 16];
  int nb, split, mb;
  if (!mm_place(total, MB, 1, nb, split, mb)) return;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w & 1, wn = w >> 1;
  const int r16 = lane & 15, g4 = (lane >> 4) * 4;
  const int m_tiles = pad16(a.M) >> 4;
  const int v_tiles = a.V >> 4;
  MmLoop p;
  p.steps = a.K >> 5;
  mm_x_sources(p, a.act, act_plane(a.M, a.K), mb, m_tiles, p.steps, 0);
  int vt[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    vt[t] = nb * 8 + wn * 4 + t;
    p.pw[t] = a.w + (size_t)min(vt[t], v_tiles - 1) * p.steps * 512 + lane * 8;
  }
  f32x4 acc[4][4];
  mm_ksteps(p, xs, wm, acc);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    Top2 t2 = top2_empty();
#pragma unroll
    for (int t = 0; t < 4; ++t)
      if (vt[t] < v_tiles)
#pragma unroll
        for (int j = 0; j < 4; ++j) t2 = top2_push(t2, acc[t][i][j], vt[t] * 16 + g4 + j);
    t2 = top2_shfl_xor(t2, 16);
    t2 = top2_shfl_xor(t2, 32);
    if (lane < 16) red[wn][(4 * wm + i) * 16 + lane] = t2;
    const int tm = mb * MM_T + 4 * wm + i;
    const int m = tm * 16 + r16;
    if (a.dbg_logits && tm < m_tiles && m < a.M && (m % a.N) != 0) {
      float* dst = a.dbg_logits + ((size_t)(m / a.N) * (a.N - 1) + (m % a.N) - 1) * a.V;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (vt[t] < v_tiles) *reinterpret_cast<f32x4*>(dst + vt[t] * 16 + g4) = acc[t][i];
    }
  }
  __syncthreads();
  if (threadIdx.x < MM_T * 16) {
    const int m = mb * MM_T * 16 + threadIdx.x;
    if (m < a.M) a.part[(size_t)nb * a.M + m] = top2_merge(red[0][threadIdx.x], red[1][threadIdx.x]);
  }
}

namespace {
int round8(int n) { return (n + 7) & ~7; }
}  // namespace

extern "C" hipError_t dflash_launch_mm(const WsArgs* a, int mode, hipStream_t st) {
  int total_nb = 0;
  for (int s = 0; s < a->nseg; ++s) total_nb += (a->seg[s].units + 3) / 4;
  const int MB = ((pad16(a->M) >> 4) + MM_T - 1) / MM_T;
  const int total = total_nb * a->ks * MB;
  const dim3 grid(round8(total)), block(256);
  if (mode == WS_SWIGLU) launch_kernel(mm_kernel<WS_SWIGLU>, grid, block, 0, st, *a, total, MB);
  else launch_kernel(mm_kernel<WS_PARTIAL>, grid, block, 0, st, *a, total, MB);
  return hipGetLastError();
}

extern "C" hipError_t dflash_launch_swiglu_finish(const WsArgs* a, hipStream_t st) {
  const int n = a->M * (a->n_cols / 4);
  launch_kernel(swiglu_finish_kernel, dim3((n + 255) / 256), dim3(256), 0, st, *a);
  return hipGetLastError();
}

extern "C" hipError_t dflash_launch_lmhead_mm(const LmArgs* a, hipStream_t st) {
  const int NB = ((a->V >> 4) + MM_T - 1) / MM_T;
  const int MB = ((pad16(a->M) >> 4) + MM_T - 1) / MM_T;
  const int total = NB * MB;
  launch_kernel(mm_lmhead_kernel, dim3(round8(total)), dim3(256), 0, st, *a, total, MB);
  return hipGetLastError();
}
