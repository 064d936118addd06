// Weight-streaming GEMM for few activation rows: y[m][n] = sum_k x[m][k] * W[n][k],
// x a split (hi + lo) activation, W bf16.
//
// At a decode step the activation has M = B*N rows (16 for one sequence and a
// block of 16) while W has thousands of rows, so every weight byte is used M
// times and the kernel is bound by HBM. Weights are pre-packed (pk_index) so
// that the 16x32 A-operand block of one MFMA is 1 KB of contiguous memory in
// lane order; one wave per workgroup streams NT = 2 tiles (32 output rows)
// over a slice of k with the pipelined loop of stream.h. Narrow matrices
// split k across waves (ks > 1) so that ~1500 waves stream at once; their
// fp32 partial tiles go to part[split][M][n_cols] and the consumer (RMSNorm
// or a finisher) adds the splits in split order, so results are deterministic.
// With ks == 1 the gate/up projection applies SwiGLU in registers: the wave's
// two tiles are the gate and up rows of the same 16 features, and the
// product is written as the split activation of the down projection.
#include "stream.h"

template <int MT, int U, int MODE>
__global__ __launch_bounds__(64) void ws_kernel(WsArgs a) {
  constexpr int NT = 2;
  const int lane = threadIdx.x;
  const int split = blockIdx.x % a.ks;
  const int unit = blockIdx.x / a.ks;
  int s = 0;
  while (s + 1 < a.nseg && unit >= a.unit_start[s + 1]) ++s;
  const WsSeg sg = a.seg[s];
  const int u = unit - a.unit_start[s];
  const int steps = a.K >> 5;
  const int s0 = split * steps / a.ks, s1 = (split + 1) * steps / a.ks;
  const uint16_t* pw[NT];
  if (MODE == WS_SWIGLU) {
    pw[0] = sg.w0 + (size_t)u * steps * 512 + lane * 8;
    pw[1] = sg.w1 + (size_t)u * steps * 512 + lane * 8;
  } else {
#pragma unroll
    for (int t = 0; t < NT; ++t) pw[t] = sg.w0 + (size_t)(u * NT + t) * steps * 512 + lane * 8;
  }
  const int r16 = lane & 15, g4 = (lane >> 4) * 4;
  const int m_tiles = pad16(a.M) >> 4;
  for (int mg = 0; mg < m_tiles; mg += MT) {
    const uint16_t* px[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int tm = min(mg + mt, m_tiles - 1);
      px[mt] = sg.act + (size_t)tm * steps * 512 + lane * 8;
    }
    f32x4 acc[NT][MT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    stream_ksteps<NT, MT, U>(pw, px, act_plane(a.M, a.K), s0, s1, acc);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = (mg + mt) * 16 + r16;
      if (mg + mt >= m_tiles || m >= a.M) continue;
      if (MODE == WS_PARTIAL) {
        float* out = a.part + ((size_t)split * a.M + m) * a.n_cols + sg.col0;
#pragma unroll
        for (int t = 0; t < NT; ++t) *reinterpret_cast<f32x4*>(out + (u * NT + t) * 16 + g4) = acc[t][mt];
      } else {
        f32x4 y;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float gt = acc[0][mt][i];
          y[i] = gt / (1.0f + __expf(-gt)) * acc[1][mt][i];
        }
        u16x4 hi, lo;
        split4(y, hi, lo);
        uint16_t* dst = a.out + pk_index(m, sg.col0 + u * 16 + g4, a.n_cols);
        *reinterpret_cast<u16x4*>(dst) = hi;
        *reinterpret_cast<u16x4*>(dst + act_plane(a.M, a.n_cols)) = lo;
      }
    }
  }
}

extern "C" hipError_t dflash_launch_ws(const WsArgs* a, int mode, hipStream_t st) {
  const dim3 grid(a->unit_start[a->nseg] * a->ks), block(64);
  const int m_tiles = pad16(a->M) >> 4;
  if (mode == WS_SWIGLU) {
    if (m_tiles <= 1) launch_kernel((ws_kernel<1, 4, WS_SWIGLU>), grid, block, 0, st, *a);
    else if (m_tiles <= 2) launch_kernel((ws_kernel<2, 2, WS_SWIGLU>), grid, block, 0, st, *a);
    else launch_kernel((ws_kernel<4, 2, WS_SWIGLU>), grid, block, 0, st, *a);
  } else {
    if (m_tiles <= 1) launch_kernel((ws_kernel<1, 4, WS_PARTIAL>), grid, block, 0, st, *a);
    else if (m_tiles <= 2) launch_kernel((ws_kernel<2, 2, WS_PARTIAL>), grid, block, 0, st, *a);
    else launch_kernel((ws_kernel<4, 2, WS_PARTIAL>), grid, block, 0, st, *a);
  }
  return hipGetLastError();
}

// Row-major [R][K] -> packed layout; one thread moves one 16-byte lane slot.
__global__ __launch_bounds__(256) void pack_kernel(PackArgs a) {
  const size_t n = (size_t)a.R * a.K / 8;
  const int steps = a.K >> 5;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(i & 63);
    const size_t ts = i >> 6;
    const int step = (int)(ts % steps);
    const size_t tile = ts / steps;
    const size_t r = tile * 16 + (lane & 15);
    const int k = step * 32 + (lane >> 4) * 8;
    *reinterpret_cast<u32x4*>(a.dst + i * 8) = *reinterpret_cast<const u32x4*>(a.src + r * a.K + k);
  }
}

extern "C" hipError_t dflash_launch_pack(const PackArgs* a, hipStream_t st) {
  launch_kernel(pack_kernel, dim3(2048), dim3(256), 0, st, *a);
  return hipGetLastError();
}
