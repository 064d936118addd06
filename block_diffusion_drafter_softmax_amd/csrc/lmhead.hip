// LM head + argmax: z = y W_lm^T over the whole vocabulary, reduced on the fly
// to a top-2 (value, lowest index) per block row for every LM_WAVES*32
// vocabulary rows, so the [rows, V] logits never go to memory (except as an
// optional debug copy). Each wave streams two packed 16-row tiles of W_lm
// over the full hidden size with the pipelined loop of stream.h; the
// workgroup's waves merge their top-2 in LDS and write one per row;
// argmax_reduce_kernel then merges the partial top-2 of each row. The merge
// is order independent, so the draft is deterministic.
#include "dflash.h"
#include "stream.h"

#define LM_WAVES 2  // waves per workgroup (32 vocabulary rows each)

template <int MT, int U>
__global__ __launch_bounds__(64 * LM_WAVES) void lmhead_kernel(LmArgs a) {
  __shared__ Top2 red[LM_WAVES][MT * 16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g4 = (lane >> 4) * 4, r16 = lane & 15;
  const int n_p = a.V / 32;
  const int p = blockIdx.x * LM_WAVES + wave;  // vocabulary rows 32p .. 32p+31
  const bool live = p < n_p;
  const int pc = min(p, n_p - 1);              // idle waves stream nothing
  const int steps = a.K >> 5;
  const uint16_t* pw[2] = {a.w + (size_t)(2 * pc) * steps * 512 + lane * 8,
                           a.w + (size_t)(2 * pc + 1) * steps * 512 + lane * 8};
  const int m_tiles = pad16(a.M) >> 4;
  for (int mg = 0; mg < m_tiles; mg += MT) {
    const uint16_t* px[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) px[mt] = a.act + (size_t)min(mg + mt, m_tiles - 1) * steps * 512 + lane * 8;
    f32x4 acc[2][MT];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (live) stream_ksteps<2, MT, U>(pw, px, act_plane(a.M, a.K), 0, steps, acc);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      Top2 t = top2_empty();
      if (live) {
#pragma unroll
        for (int i = 0; i < 4; ++i) t = top2_push(t, acc[0][mt][i], 32 * p + g4 + i);
#pragma unroll
        for (int i = 0; i < 4; ++i) t = top2_push(t, acc[1][mt][i], 32 * p + 16 + g4 + i);
      }
      t = top2_shfl_xor(t, 16);
      t = top2_shfl_xor(t, 32);
      if (lane < 16) red[wave][mt * 16 + lane] = t;
      const int m = (mg + mt) * 16 + r16;
      if (live && a.dbg_logits && mg + mt < m_tiles && m < a.M && (m % a.N) != 0) {
        float* dst = a.dbg_logits + ((size_t)(m / a.N) * (a.N - 1) + (m % a.N) - 1) * a.V;
        *reinterpret_cast<f32x4*>(dst + 32 * p + g4) = acc[0][mt];
        *reinterpret_cast<f32x4*>(dst + 32 * p + 16 + g4) = acc[1][mt];
      }
    }
    __syncthreads();
    if (threadIdx.x < MT * 16) {
      const int m = mg * 16 + threadIdx.x;
      Top2 t = red[0][threadIdx.x];
      for (int w = 1; w < LM_WAVES; ++w) t = top2_merge(t, red[w][threadIdx.x]);
      if (m < a.M) a.part[(size_t)m * a.n_parts + blockIdx.x] = t;
    }
    __syncthreads();  // red is reused by the next m-group
  }
}

extern "C" hipError_t dflash_launch_lmhead(const LmArgs* a, hipStream_t st) {
  const dim3 grid((a->V / 32 + LM_WAVES - 1) / LM_WAVES), block(64 * LM_WAVES);
  const int m_tiles = pad16(a->M) >> 4;
  hipError_t e;
  if (m_tiles <= 1) e = launch_kernel((lmhead_kernel<1, 4>), grid, block, 0, st, *a);
  else if (m_tiles <= 2) e = launch_kernel((lmhead_kernel<2, 2>), grid, block, 0, st, *a);
  else e = launch_kernel((lmhead_kernel<4, 2>), grid, block, 0, st, *a);
  return e;
}

// One workgroup of ARGMAX_THREADS per block row m (rows with m % N == 0 are
// the anchors and produce nothing): the row's partial top-2 (contiguous)
// are requested in batches of ARGMAX_BATCH loads per thread, then merged
// (the merge is order independent).
#define ARGMAX_THREADS 1024
#define ARGMAX_BATCH 4
__global__ __launch_bounds__(ARGMAX_THREADS) LATENCY_BOUND void argmax_reduce_kernel(ArgmaxArgs a) {
  const int m = blockIdx.x;  // row of the partials
  int mo = m;                // block row it belongs to
  if (a.row_inv) {
    if (m >= *a.row_count) return;
    mo = a.row_inv[m];
  }
  if (mo % a.N == 0) return;
  Top2 t = top2_empty();
  const Top2* row = a.part + (size_t)m * a.n_parts;
  for (int j0 = 0; j0 < a.n_parts; j0 += ARGMAX_THREADS * ARGMAX_BATCH) {
    Top2 v[ARGMAX_BATCH];
#pragma unroll
    for (int u = 0; u < ARGMAX_BATCH; ++u) v[u] = row[min(j0 + u * ARGMAX_THREADS + (int)threadIdx.x, a.n_parts - 1)];
#pragma unroll
    for (int u = 0; u < ARGMAX_BATCH; ++u)  // a clamped duplicate would corrupt the second value: skip it
      if (j0 + u * ARGMAX_THREADS + (int)threadIdx.x < a.n_parts) t = top2_merge(t, v[u]);
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) t = top2_shfl_xor(t, o);
  __shared__ Top2 red[ARGMAX_THREADS / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = t;
  __syncthreads();
  if (threadIdx.x == 0) {
    t = red[0];
    for (int w = 1; w < ARGMAX_THREADS / 64; ++w) t = top2_merge(t, red[w]);
    const int b = mo / a.N, j = mo % a.N - 1;
    int tok = t.i1;
    if (tok < 0 || tok >= a.V) {
      set_error(a.err, DFLASH_DEV_BAD_TOKEN);
      tok = 0;
    }
    a.draft[b * (a.N - 1) + j] = tok;
    if (a.gap) a.gap[b * (a.N - 1) + j] = t.v1 - t.v2;
    if (a.conf) a.conf[b * (a.N - 1) + j] = 1.0f / t.s;
  }
}

extern "C" hipError_t dflash_launch_argmax(const ArgmaxArgs* a, hipStream_t st) {
  launch_kernel(argmax_reduce_kernel, dim3(a->M), dim3(ARGMAX_THREADS), 0, st, *a);
  return hipGetLastError();
}
