// LM head + argmax: z = y W_lm^T over the whole vocabulary, reduced on the fly
// to a per-workgroup top-2 (value, lowest index) for every block row, so the
// [rows, V] logits never go to memory (except as an optional debug copy).
// Same streaming scheme as the projection GEMM: each wave owns 32 vocabulary
// rows over the full hidden size, A operand from HBM, the normed rows as the
// B operand. argmax_reduce_kernel then merges the per-workgroup top-2 of each
// row; the merge is order independent, so the draft is deterministic.
#include "common.h"
#include "dflash.h"


template <int MT, int U>
__global__ __launch_bounds__(256) void lmhead_kernel(LmArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g4 = (lane >> 4) * 4, r16 = lane & 15, kq = (lane >> 4) * 8;
  const int npairs = a.V / 32;
  const int p = blockIdx.x * 4 + wave;
  const bool live = p < npairs;
  const int rowA = 32 * (live ? p : 0), rowB = rowA + 16;
  const int K = a.K, steps = K / 32;
  const uint16_t* pa = a.w + (size_t)(rowA + r16) * K + kq;
  const uint16_t* pb = a.w + (size_t)(rowB + r16) * K + kq;
  __shared__ Top2 red[4][16 * MT];

  const int n_mg = (a.M + 16 * MT - 1) / (16 * MT);
  for (int mg = 0; mg < n_mg; ++mg) {
    const int m0 = mg * 16 * MT;
    f32x4 accA[MT], accB[MT];
    const uint16_t* px[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      accA[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      accB[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      int m = m0 + mt * 16 + r16;
      m = m < a.M ? m : a.M - 1;
      px[mt] = a.act + (size_t)m * K + kq;
    }
    if (live) {
      int st = 0;
      for (; st + U <= steps; st += U) {
        bf16x8 fa[U], fb[U], fx[U][MT];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          fa[u] = ld8(pa + (st + u) * 32);
          fb[u] = ld8(pb + (st + u) * 32);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) fx[u][mt] = ld8(px[mt] + (st + u) * 32);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            accA[mt] = mfma16(fa[u], fx[u][mt], accA[mt]);
            accB[mt] = mfma16(fb[u], fx[u][mt], accB[mt]);
          }
      }
      for (; st < steps; ++st) {
        const bf16x8 fa = ld8(pa + st * 32), fb = ld8(pb + st * 32);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const bf16x8 fx = ld8(px[mt] + st * 32);
          accA[mt] = mfma16(fa, fx, accA[mt]);
          accB[mt] = mfma16(fb, fx, accB[mt]);
        }
      }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      Top2 t = top2_empty();
      if (live) {
#pragma unroll
        for (int i = 0; i < 4; ++i) t = top2_push(t, accA[mt][i], rowA + g4 + i);
#pragma unroll
        for (int i = 0; i < 4; ++i) t = top2_push(t, accB[mt][i], rowB + g4 + i);
      }
      t = top2_shfl_xor(t, 16);
      t = top2_shfl_xor(t, 32);
      if (lane < 16) red[wave][mt * 16 + lane] = t;
      const int m = m0 + mt * 16 + r16;
      if (a.dbg_logits && live && m < a.M && (m % a.N) != 0) {
        float* dst = a.dbg_logits + ((size_t)(m / a.N) * (a.N - 1) + (m % a.N) - 1) * a.V;
        *reinterpret_cast<f32x4*>(dst + rowA + g4) = accA[mt];
        *reinterpret_cast<f32x4*>(dst + rowB + g4) = accB[mt];
      }
    }
    __syncthreads();
    if (threadIdx.x < 16 * MT) {
      const int m = m0 + threadIdx.x;
      Top2 t = red[0][threadIdx.x];
#pragma unroll
      for (int w = 1; w < 4; ++w) t = top2_merge(t, red[w][threadIdx.x]);
      if (m < a.M) a.part[(size_t)blockIdx.x * a.M + m] = t;
    }
    __syncthreads();
  }
}

extern "C" hipError_t dflash_launch_lmhead(const LmArgs* a, hipStream_t st) {
  const int n_wg = (a->V / 32 + 3) / 4;
  if (a->M <= 16) hipLaunchKernelGGL((lmhead_kernel<1, 8>), dim3(n_wg), dim3(256), 0, st, *a);
  else if (a->M <= 32) hipLaunchKernelGGL((lmhead_kernel<2, 4>), dim3(n_wg), dim3(256), 0, st, *a);
  else hipLaunchKernelGGL((lmhead_kernel<4, 4>), dim3(n_wg), dim3(256), 0, st, *a);
  return hipGetLastError();
}


// One workgroup per block row m (rows with m % N == 0 are the anchors and
// produce nothing).
__global__ __launch_bounds__(256) void argmax_reduce_kernel(ArgmaxArgs a) {
  const int m = blockIdx.x;
  if (m % a.N == 0) return;
  Top2 t = top2_empty();
  for (int j = threadIdx.x; j < a.n_wg; j += 256) t = top2_merge(t, a.part[(size_t)j * a.M + m]);
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) t = top2_shfl_xor(t, o);
  __shared__ Top2 red[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = t;
  __syncthreads();
  if (threadIdx.x == 0) {
    t = red[0];
    for (int w = 1; w < 4; ++w) t = top2_merge(t, red[w]);
    const int b = m / a.N, j = m % a.N - 1;
    int tok = t.i1;
    if (tok < 0 || tok >= a.V) {
      set_error(a.err, DFLASH_DEV_BAD_TOKEN);
      tok = 0;
    }
    a.draft[b * (a.N - 1) + j] = tok;
    if (a.gap) a.gap[b * (a.N - 1) + j] = t.v1 - t.v2;
  }
}

extern "C" hipError_t dflash_launch_argmax(const ArgmaxArgs* a, hipStream_t st) {
  hipLaunchKernelGGL(argmax_reduce_kernel, dim3(a->M), dim3(256), 0, st, *a);
  return hipGetLastError();
}
