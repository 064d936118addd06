// Weight-streaming GEMM for few activation rows: out[m][n] = sum_k act[m][k] * W[n][k].
//
// At a decode step the activation has M = B*N rows (16 for one sequence with a
// block of 16) while W has thousands of rows, so every weight byte is used M
// times and the kernel is bound by HBM. Each wave owns a pair of 16-row weight
// tiles and streams them straight from HBM into VGPRs in the MFMA A-operand
// layout (lane l: row l%16, 8 consecutive k at 8*(l/16)), one 16x16x32 bf16
// MFMA per tile and 32-wide k step, with the activation fragment as the B
// operand. The waves of a workgroup split k; their partial tiles are summed
// through LDS in wave order (deterministic). Workgroups can further split k
// (ks > 1) for the EPI_PARTIAL epilogue, whose per-split sums are added by the
// consumer (the next RMSNorm kernel) in split order.
//
// The tile pair is chosen so the epilogue is local to the lane: RoPE partners
// (dims j and j + d_h/2 of a head), or the gate and up rows of one SwiGLU
// feature, land in the same lane and register slot.
#include "common.h"

namespace {

template <int MT>
struct Frag {
  bf16x8 a, b, x[MT];
};

DEV void rope_rotate(float& x1, float& x2, const float* rope, int pos, int half, int j) {
  if (rope == nullptr) return;
  const float c = rope[((size_t)pos * half + j) * 2 + 0];
  const float s = rope[((size_t)pos * half + j) * 2 + 1];
  const float y1 = x1 * c - x2 * s;
  const float y2 = x2 * c + x1 * s;
  x1 = y1;
  x2 = y2;
}

DEV int clamp_page(int p, int n_pages) { return p < 0 ? 0 : (p >= n_pages ? n_pages - 1 : p); }

template <int MT>
DEV void epilogue(const GemmArgs& a, const GemmSeg& sg, int split, int rowA, int rowB, int m0,
                  const f32x4* accA, const f32x4* accB) {
  const int lane = threadIdx.x & 63;
  const int g4 = (lane >> 4) * 4;
  const int d = a.head_dim, half = d / 2;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = m0 + mt * 16 + (lane & 15);
    if (m >= a.M) continue;
    const f32x4 va = accA[mt], vb = accB[mt];
    switch (sg.epi) {
      case EPI_PARTIAL: {
        float* out = (float*)sg.out + ((size_t)split * a.M + m) * a.n_out;
        *reinterpret_cast<f32x4*>(out + rowA + g4) = va;
        *reinterpret_cast<f32x4*>(out + rowB + g4) = vb;
        break;
      }
      case EPI_SWIGLU: {
        u16x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float gt = va[i];
          const float sg_ = gt / (1.0f + __expf(-gt));
          o[i] = f2bf(sg_ * vb[i]);
        }
        *reinterpret_cast<u16x4*>((uint16_t*)sg.out + (size_t)m * a.n_out + rowA + g4) = o;
        break;
      }
      case EPI_Q:
      case EPI_KBLK:
      case EPI_CTX_K: {
        const int pos = a.row_pos[m];
        if (pos < 0) break;
        const int head = rowA / d;
        const int j0 = rowA % d + g4;  // < half
        u16x4 o1, o2;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float x1 = va[i], x2 = vb[i];
          rope_rotate(x1, x2, a.rope, pos, half, j0 + i);
          o1[i] = f2bf(x1);
          o2[i] = f2bf(x2);
        }
        uint16_t* dst;
        if (sg.epi == EPI_Q) {
          dst = (uint16_t*)sg.out + (size_t)m * a.n_out + head * d;
        } else if (sg.epi == EPI_KBLK) {
          const int b = m / a.block, n = m % a.block;
          dst = (uint16_t*)sg.out + (((size_t)b * a.n_kv + head) * 16 + n) * d;
        } else {
          const int seq = a.row_seq[m];
          const int page = clamp_page(a.page_table[(size_t)seq * a.max_pages_per_seq + pos / 16], a.n_pages);
          dst = a.kv_pages + sg.layer * a.layer_stride +
                (((size_t)page * 2 + 0) * a.n_kv + head) * 16 * d + (size_t)(pos % 16) * d;
        }
        *reinterpret_cast<u16x4*>(dst + j0) = o1;
        *reinterpret_cast<u16x4*>(dst + j0 + half) = o2;
        break;
      }
      case EPI_VBLK:
      case EPI_CTX_V: {
        uint16_t* dst;
        int stride_d = 16;
        const int head = rowA / d;
        if (sg.epi == EPI_VBLK) {
          const int b = m / a.block, n = m % a.block;
          dst = (uint16_t*)sg.out + ((size_t)b * a.n_kv + head) * d * 16 + n;
        } else {
          const int pos = a.row_pos[m];
          if (pos < 0) break;
          const int seq = a.row_seq[m];
          const int page = clamp_page(a.page_table[(size_t)seq * a.max_pages_per_seq + pos / 16], a.n_pages);
          dst = a.kv_pages + sg.layer * a.layer_stride +
                (((size_t)page * 2 + 1) * a.n_kv + head) * 16 * d + (pos % 16);
        }
        const int dA = rowA % d + g4, dB = rowB % d + g4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          dst[(size_t)(dA + i) * stride_d] = f2bf(va[i]);
          dst[(size_t)(dB + i) * stride_d] = f2bf(vb[i]);
        }
        break;
      }
      default:
        break;
    }
  }
}

}  // namespace

template <int KW, int MT, int U>
__global__ __launch_bounds__(64 * KW) void gemm_rows_kernel(GemmArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int split = blockIdx.x % a.ks;
  const int gp = blockIdx.x / a.ks;
  int s = 0;
  while (s + 1 < a.nseg && gp >= a.seg_start[s + 1]) ++s;
  const GemmSeg sg = a.seg[s];
  const int p = gp - a.seg_start[s];

  int rowA, rowB;
  const uint16_t *wA, *wB;
  if (sg.mode == PAIR_PLAIN) {
    rowA = 32 * p; rowB = rowA + 16; wA = wB = sg.w0;
  } else if (sg.mode == PAIR_ROPE) {
    const int tph = a.head_dim / 32;
    rowA = (p / tph) * a.head_dim + (p % tph) * 16;
    rowB = rowA + a.head_dim / 2;
    wA = wB = sg.w0;
  } else {
    rowA = rowB = 16 * p; wA = sg.w0; wB = sg.w1;
  }

  const int K = a.K;
  const int steps = K / 32;
  const int s0 = split * steps / a.ks, s1 = (split + 1) * steps / a.ks;
  const int ws0 = s0 + (s1 - s0) * wave / KW, ws1 = s0 + (s1 - s0) * (wave + 1) / KW;
  const int r16 = lane & 15, kq = (lane >> 4) * 8;
  const uint16_t* pa = wA + (size_t)(rowA + r16) * K + kq;
  const uint16_t* pb = wB + (size_t)(rowB + r16) * K + kq;

  __shared__ f32x4 red[(KW > 1 ? KW - 1 : 1)][2 * MT][64];

  const int mg_rows = 16 * MT;
  const int n_mg = (a.M + mg_rows - 1) / mg_rows;
  for (int mg = 0; mg < n_mg; ++mg) {
    const int m0 = mg * mg_rows;
    f32x4 accA[MT], accB[MT];
    const uint16_t* px[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      accA[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      accB[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      int m = m0 + mt * 16 + r16;
      m = m < a.M ? m : a.M - 1;
      px[mt] = sg.act + (size_t)m * K + kq;
    }
    int st = ws0;
    for (; st + U <= ws1; st += U) {
      Frag<MT> f[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        f[u].a = ld8(pa + (st + u) * 32);
        f[u].b = ld8(pb + (st + u) * 32);
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) f[u].x[mt] = ld8(px[mt] + (st + u) * 32);
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          accA[mt] = mfma16(f[u].a, f[u].x[mt], accA[mt]);
          accB[mt] = mfma16(f[u].b, f[u].x[mt], accB[mt]);
        }
    }
    for (; st < ws1; ++st) {
      const bf16x8 fa = ld8(pa + st * 32), fb = ld8(pb + st * 32);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const bf16x8 fx = ld8(px[mt] + st * 32);
        accA[mt] = mfma16(fa, fx, accA[mt]);
        accB[mt] = mfma16(fb, fx, accB[mt]);
      }
    }
    if (KW > 1) {
      if (wave > 0) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          red[wave - 1][2 * mt][lane] = accA[mt];
          red[wave - 1][2 * mt + 1][lane] = accB[mt];
        }
      }
      __syncthreads();
      if (wave == 0) {
        for (int w = 1; w < KW; ++w)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            accA[mt] += red[w - 1][2 * mt][lane];
            accB[mt] += red[w - 1][2 * mt + 1][lane];
          }
      }
    }
    if (wave == 0) epilogue<MT>(a, sg, split, rowA, rowB, m0, accA, accB);
    if (KW > 1) __syncthreads();
  }
}

// Host-side launcher. Chooses the instantiation from the row count.
extern "C" hipError_t dflash_launch_gemm(const GemmArgs* args, int total_pairs, int kw, hipStream_t st) {
  const dim3 grid(total_pairs * args->ks);
  if (args->M <= 16) {
    if (kw == 8) hipLaunchKernelGGL((gemm_rows_kernel<8, 1, 8>), grid, dim3(512), 0, st, *args);
    else hipLaunchKernelGGL((gemm_rows_kernel<4, 1, 8>), grid, dim3(256), 0, st, *args);
  } else if (args->M <= 32) {
    hipLaunchKernelGGL((gemm_rows_kernel<4, 2, 4>), grid, dim3(256), 0, st, *args);
  } else {
    hipLaunchKernelGGL((gemm_rows_kernel<4, 4, 4>), grid, dim3(256), 0, st, *args);
  }
  return hipGetLastError();
}
