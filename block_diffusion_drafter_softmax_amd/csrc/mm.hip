// Tiled MFMA GEMM for many activation rows: y[m][n] = sum_k x[m][k] * W[n][k],
// x a split (hi + lo) activation, W bf16, both in the packed operand layout.
//
// When a call carries many block rows (a batch of sequences, or a context
// append of hundreds of rows) every weight byte meets M >= 64 activation rows
// and the product is bound by the matrix cores, not by the weight stream.
// What limits a tile loop here is the bandwidth from L2 into the CUs: at the
// MFMA rate, every byte a CU loads must serve as many MFMAs as possible.
// So each workgroup of 4 waves computes a 128 x 256 output tile (MM_ROW_TILES
// activation tiles by MM_COL_TILES weight tiles) with both operands staged
// once per workgroup through double-buffered LDS, one k step per stage, and
// each wave owns a 64 x 128 sub-tile (4 activation tiles x 8 weight tiles:
// 16 LDS reads feed 64 MFMA 16x16x32, the hi and lo halves of 32 tile
// products). Per k step a workgroup loads 32 KB for 256 MFMAs, straight
// from memory into LDS (global_load_lds, 1 KB per wave instruction, no
// registers held for staging), issued right after the step's LDS reads.
// Workgroups of one column block (same weights, different row blocks) are
// placed on one XCD and dispatched together, so the weights leave HBM about
// once per call. Narrow products whose tiles would not fill the chip split
// k (fp32 partials per split, added in split order by the consumer). The
// epilogues are those of the streaming GEMM (fp32 partials, or SwiGLU into
// the next split activation; after a k split the gate and up partials go to
// swiglu_finish_kernel) and the LM head's top-2 reduction.
#include "stream.h"

namespace {

// Workgroup tile geometry: XT activation tiles (MM_ROW_TILES, or half of it
// where 128-row tiles would leave CUs without a second workgroup) by WT
// weight tiles; 2 x 2 waves, each XW x WW tiles.
template <int XT>
struct Geo {
  static constexpr int WT = MM_COL_TILES;
  static constexpr int XW = XT / 2, WW = WT / 2;
  static constexpr int kStageBlocks = 2 * XT + WT;  // 1 KB blocks per stage: X tile t plane p at 2t+p, W tile u at 2XT+u
  static constexpr int kLoads = kStageBlocks / 4;   // 16-byte loads per thread and stage (4 waves)
  static_assert(kStageBlocks % 4 == 0 && XT % 4 == 0, "stage blocks are dealt to 4 waves");
};
constexpr int WT = MM_COL_TILES;

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

// Global sources (wave-uniform) of the wave's kLoads blocks of a stage at
// the split's first k step; k step s adds s*512 and lane l reads the 16
// bytes at l*8. Wave w moves stage blocks w + 4j: for j < XT/2 activation
// tile (w>>1) + 2j, plane w&1; after that weight tile w + 4j - 2XT.
template <int XT>
struct MmSrc {
  const uint16_t* p[Geo<XT>::kLoads];
  int steps;  // k steps of the split
};


// 16 bytes per lane from global memory straight into LDS (one 1 KB block per wave instruction).

// Stage k step s into `stage` (kStageBlocks blocks of 1 KB): each wave
// instruction writes one whole block, lane l at byte 16 l.
template <int XT>
DEV void mm_dma(u32x4* stage, const MmSrc<XT>& src, int s, int w) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < Geo<XT>::kLoads; ++j) dma16(src.p[j] + (size_t)s * 512 + lane * 8, stage + (w + 4 * j) * 64);
}

DEV void mm_wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// One k step: the wave's fragments are read from stage `cur` first, then
// the next step's blocks are requested into stage `nxt` (the LDS reads are
// ordered before those writes, and whatever the compiler waits for before
// the next LDS read has already been waited for at the step's barrier),
// then acc[t][i] += W tile (wn*WW + t) x X tile (wm*XW + i), hi and lo.
template <int XT>
DEV void mm_step(const u32x4* cur, u32x4* nxt, const MmSrc<XT>& src, int s, int w,
                 f32x4 (&acc)[Geo<XT>::WW][Geo<XT>::XW]) {
  constexpr int XW = Geo<XT>::XW, WW = Geo<XT>::WW;
  const int lane = threadIdx.x & 63, wm = w & 1, wn = w >> 1;
  bf16x8 xh[XW], xl[XW], wf[WW];
#pragma unroll
  for (int i = 0; i < XW; ++i) {
    xh[i] = __builtin_bit_cast(bf16x8, cur[(2 * (wm * XW + i)) * 64 + lane]);
    xl[i] = __builtin_bit_cast(bf16x8, cur[(2 * (wm * XW + i) + 1) * 64 + lane]);
  }
#pragma unroll
  for (int t = 0; t < WW; ++t) wf[t] = __builtin_bit_cast(bf16x8, cur[(2 * XT + wn * WW + t) * 64 + lane]);
  if (s + 1 < src.steps) mm_dma<XT>(nxt, src, s + 1, w);
#pragma unroll
  for (int t = 0; t < WW; ++t)
#pragma unroll
    for (int i = 0; i < XW; ++i) {
      acc[t][i] = mfma16(wf[t], xh[i], acc[t][i]);
      acc[t][i] = mfma16(wf[t], xl[i], acc[t][i]);
    }
}

template <int XT>
DEV void mm_ksteps(const MmSrc<XT>& src, u32x4 (*stages)[Geo<XT>::kStageBlocks * 64], int w,
                   f32x4 (&acc)[Geo<XT>::WW][Geo<XT>::XW]) {
  constexpr int XW = Geo<XT>::XW, WW = Geo<XT>::WW;
#pragma unroll
  for (int t = 0; t < WW; ++t)
#pragma unroll
    for (int i = 0; i < XW; ++i) acc[t][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  mm_dma<XT>(stages[0], src, 0, w);
  for (int s = 0; s < src.steps; ++s) {
    // the wait sits at the top of the trip, so the MFMAs of step s-1 (which
    // touch no memory and could otherwise sink below it) are issued first
    mm_wait_dma();
    __syncthreads();
    mm_step<XT>(stages[s & 1], stages[(s + 1) & 1], src, s, w, acc);
  }
  __syncthreads();  // every wave's last LDS reads are done before the epilogue reuses LDS
}

template <int XT>
DEV void mm_x_sources(MmSrc<XT>& src, const uint16_t* act, size_t lo, int mb, int m_tiles, int steps, int s0, int w) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < XT / 2; ++j) {
    const int tm = min(mb * XT + (w >> 1) + 2 * j, m_tiles - 1);  // clamped to the last real tile
    src.p[j] = act + (w & 1) * lo + ((size_t)tm * steps + s0) * 512;
  }
}

// Weight tile (within the workgroup's WT) of this thread's load j >= XT/2.
template <int XT>
DEV int mm_w_tile(int j, int w) { return w + 4 * j - 2 * XT; }

// Segment of a column block: each segment's units (2 output tiles each, or
// one SwiGLU feature tile = a gate and an up tile) make ceil(2 units / WT) blocks.
DEV int mm_segment(const WsArgs& a, int& nb) {
  int s = 0;
  while (s + 1 < a.nseg) {
    const int blocks = (2 * a.seg[s].units + WT - 1) / WT;
    if (nb < blocks) break;
    nb -= blocks;
    ++s;
  }
  return s;
}

}  // namespace

// SwiGLU blocks: weight tiles u < WT/2 are the gates of feature tiles
// nb*WT/2 + u, the rest the ups of the same features, so wave (wm, 0) holds
// gate and wave (wm, 1) up of the same rows and features.
template <int MODE, int XT>
__global__ __launch_bounds__(256, XT == 4 ? 3 : 2) void mm_kernel(WsArgs a, int total, int MB) {
  using Gm = Geo<XT>;
  constexpr int XW = Gm::XW, WW = Gm::WW, kStageBlocks = Gm::kStageBlocks, kLoads = Gm::kLoads;
  __shared__ u32x4 stages[2][kStageBlocks * 64];
  int nb, split, mb;
  if (!mm_place(total, MB, a.ks, nb, split, mb)) return;
  const int s = mm_segment(a, nb);
  const WsSeg sg = a.seg[s];
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), wm = w & 1, wn = w >> 1;
  const int r16 = lane & 15, g4 = (lane >> 4) * 4;
  const int m_tiles = pad16(a.M) >> 4;
  const int steps = a.K >> 5;
  const int s0 = split * steps / a.ks;
  MmSrc<XT> src;
  src.steps = (split + 1) * steps / a.ks - s0;
  mm_x_sources<XT>(src, sg.act, act_plane(a.M, a.K), mb, m_tiles, steps, s0, w);
#pragma unroll
  for (int j = XT / 2; j < kLoads; ++j) {
    const int u = mm_w_tile<XT>(j, w);
    const uint16_t* base = sg.w0;
    int tl;
    if (MODE == WS_SWIGLU) {
      if (u >= WT / 2) base = sg.w1;
      tl = min(nb * (WT / 2) + u % (WT / 2), sg.units - 1);
    } else {
      tl = min(nb * WT + u, 2 * sg.units - 1);
    }
    src.p[j] = base + ((size_t)tl * steps + s0) * 512;
  }
  f32x4 acc[WW][XW];
  mm_ksteps<XT>(src, stages, w, acc);

  if (MODE == WS_PARTIAL) {
#pragma unroll
    for (int i = 0; i < XW; ++i) {
      const int tm = mb * XT + wm * XW + i;
      const int m = tm * 16 + r16;
      if (tm >= m_tiles || m >= a.M) continue;
      float* out = a.part + ((size_t)split * a.M + m) * a.n_cols + sg.col0;
#pragma unroll
      for (int t = 0; t < WW; ++t) {
        const int tile = nb * WT + wn * WW + t;
        if (tile < 2 * sg.units) *reinterpret_cast<f32x4*>(out + tile * 16 + g4) = acc[t][i];
      }
    }
    return;
  }

  // SwiGLU: the up wave parks its accumulators in LDS (the stage buffers
  // are free after the k loop's last barrier; row half wm uses stage wm)
  // and the gate wave combines.
  f32x4* park = reinterpret_cast<f32x4*>(stages[wm]);  // [t][i][lane]
  static_assert(WW * XW <= kStageBlocks, "park fits a stage buffer");
  if (wn == 1) {
#pragma unroll
    for (int t = 0; t < WW; ++t)
#pragma unroll
      for (int i = 0; i < XW; ++i) park[(t * XW + i) * 64 + lane] = acc[t][i];
  }
  __syncthreads();
  if (wn == 1) return;
#pragma unroll
  for (int i = 0; i < XW; ++i) {
    const int tm = mb * XT + wm * XW + i;
    const int m = tm * 16 + r16;
    if (tm >= m_tiles || m >= a.M) continue;
#pragma unroll
    for (int t = 0; t < WW; ++t) {
      const int f = nb * (WT / 2) + t;  // feature tile
      if (f >= sg.units) continue;
      const f32x4 up = park[(t * XW + i) * 64 + lane];
      if (a.ks > 1) {
        float* out = a.part + ((size_t)split * a.M + m) * 2 * a.n_cols + sg.col0 + f * 16 + g4;
        *reinterpret_cast<f32x4*>(out) = acc[t][i];
        *reinterpret_cast<f32x4*>(out + a.n_cols) = up;
        continue;
      }
      f32x4 y;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float gt = acc[t][i][j];
        y[j] = gt / (1.0f + __expf(-gt)) * up[j];
      }
      u16x4 hi, lo;
      split4(y, hi, lo);
      uint16_t* dst = a.out + pk_index(m, sg.col0 + f * 16 + g4, a.n_cols);
      *reinterpret_cast<u16x4*>(dst) = hi;
      *reinterpret_cast<u16x4*>(dst + act_plane(a.M, a.n_cols)) = lo;
    }
  }
}

// SwiGLU after a k-split gate/up product: y = silu(sum of gate splits) *
// (sum of up splits), the splits added in order, written as the packed
// split activation of the down projection. One thread per 4 features.
// One workgroup per 16 rows x 64 columns (thread: row tid / 16, columns
// 4 (tid % 16) .. +3; the last block may hold 32): its output is whole 1 KB
// blocks of each plane of the packed activation (16 rows x 32 columns
// each), so no cache line is shared with another workgroup's writes; each
// row's partials are read as 256 contiguous bytes per split.
__global__ __launch_bounds__(256) void swiglu_finish_kernel(WsArgs a) {
  const int cb = (a.n_cols + 63) / 64;  // column blocks (n_cols: a multiple of 32)
  const int m = (blockIdx.x / cb) * 16 + (int)(threadIdx.x >> 4);
  const int f = (blockIdx.x % cb) * 64 + (int)(threadIdx.x & 15) * 4;
  if (m >= a.M || f >= a.n_cols) return;
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

// LM head for many rows: top-2 (value, lowest index) per row over each
// workgroup's vocabulary rows, written to part[M][column block];
// argmax_reduce_kernel merges them.
//
// The vocabulary gives every row block hundreds of column blocks, so this
// product can use wider workgroups than the layer GEMMs: 8 waves, 128
// activation rows x 512 vocabulary rows (each wave the same 64 x 128 as the
// 4-wave loop), three LDS stages of one k step (48 KB each, one workgroup
// per CU). The DMA of k step s+2 is issued during step s, two of the
// workgroup's steps (~1.7 us at the MFMA rate) ahead of its use; the
// two-stage loop keeps one step ahead, less than an L2 or HBM round trip.
// Each step waits for its own stage with a counted vmcnt and a bare
// s_barrier (the compiler's __syncthreads also waits for the DMA still in
// flight); the loop is unrolled by the three stages so that every LDS
// access names its stage statically.
namespace {
// 8 waves (2 row halves x 4 column quarters), 128 activation rows (8 tiles)
// by WT8 weight tiles; each wave 4 x WT8/4 tiles.
template <int WT8>
struct G8 {
  static constexpr int XT = MM_ROW_TILES, WT = WT8;
  static constexpr int XW = XT / 2, WW = WT / 4;
  static constexpr int BLOCKS = 2 * XT + WT;  // 1 KB blocks per stage: X tile t plane p at 2t+p, W tile u at 2XT+u
  static constexpr int LOADS = BLOCKS / 8;    // per wave and stage: wave w moves blocks w + 8j
  static_assert(BLOCKS % 8 == 0 && XT == 8 && WT % 4 == 0 && LOADS <= 6, "8-wave stage geometry");
  typedef u32x4 Stage[BLOCKS * 64];
};

template <int WT8>
DEV void g8_dma(typename G8<WT8>::Stage& st, const uint16_t* const* p, int s, int w) {
#pragma unroll
  for (int j = 0; j < G8<WT8>::LOADS; ++j) dma16(p[j] + (size_t)s * 512, &st[(w + 8 * j) * 64]);
}

// One k step s, read from `cur`; the DMA of step s+2 goes to `nxt2`, the
// stage every wave finished reading in step s-1.
template <int WT8>
DEV void g8_step(const typename G8<WT8>::Stage& cur, typename G8<WT8>::Stage& nxt2, const uint16_t* const* p, int s,
                 int steps, int w, f32x4 (&acc)[G8<WT8>::WW][G8<WT8>::XW]) {
  using G = G8<WT8>;
  // step s landed (step s+1 may not have): s_waitcnt vmcnt(LOADS), or vmcnt(0) at the last step
  if (s + 1 < steps) __builtin_amdgcn_s_waitcnt(0x0F70 | G::LOADS);
  else __builtin_amdgcn_s_waitcnt(0x0F70);
  __builtin_amdgcn_s_barrier();  // every wave's part of step s landed; every wave is past step s-1
  asm volatile("" ::: "memory");
  const int lane = threadIdx.x & 63, wm = w & 1, wn = w >> 1;
  bf16x8 xh[G::XW], xl[G::XW], wf[G::WW];
#pragma unroll
  for (int i = 0; i < G::XW; ++i) {
    xh[i] = __builtin_bit_cast(bf16x8, cur[(2 * (wm * G::XW + i)) * 64 + lane]);
    xl[i] = __builtin_bit_cast(bf16x8, cur[(2 * (wm * G::XW + i) + 1) * 64 + lane]);
  }
#pragma unroll
  for (int t = 0; t < G::WW; ++t) wf[t] = __builtin_bit_cast(bf16x8, cur[(2 * G::XT + wn * G::WW + t) * 64 + lane]);
  if (s + 2 < steps) g8_dma<WT8>(nxt2, p, s + 2, w);
#pragma unroll
  for (int t = 0; t < G::WW; ++t)
#pragma unroll
    for (int i = 0; i < G::XW; ++i) {
      acc[t][i] = mfma16(wf[t], xh[i], acc[t][i]);
      acc[t][i] = mfma16(wf[t], xl[i], acc[t][i]);
    }
}

// The whole k loop over `steps` k steps: two stages requested ahead, the
// loop unrolled by the three stages so every LDS access names its stage.
template <int WT8>
DEV void g8_ksteps(typename G8<WT8>::Stage& st0, typename G8<WT8>::Stage& st1, typename G8<WT8>::Stage& st2,
                   const uint16_t* const* p, int steps, int w, f32x4 (&acc)[G8<WT8>::WW][G8<WT8>::XW]) {
#pragma unroll
  for (int t = 0; t < G8<WT8>::WW; ++t)
#pragma unroll
    for (int i = 0; i < G8<WT8>::XW; ++i) acc[t][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  g8_dma<WT8>(st0, p, 0, w);
  if (steps > 1) g8_dma<WT8>(st1, p, 1, w);
  for (int s = 0; s < steps; s += 3) {
    g8_step<WT8>(st0, st2, p, s, steps, w, acc);
    if (s + 1 < steps) g8_step<WT8>(st1, st0, p, s + 1, steps, w, acc);
    if (s + 2 < steps) g8_step<WT8>(st2, st1, p, s + 2, steps, w, acc);
  }
  __syncthreads();  // every wave's last LDS reads are done before an epilogue reuses LDS
}
}  // namespace

// Layer GEMMs for many rows with the 8-wave loop (one workgroup per CU):
// picked by the host where a tile width of WT8 weight tiles and a k split
// make the grid a whole number of rounds of the chip. SwiGLU blocks: weight
// tiles u < WT8/2 are the gates of feature tiles nb*WT8/2 + u, the rest the
// ups of the same features, so wave (wm, wn) with wn < 2 holds gates and
// wave (wm, wn + 2) the ups of the same rows and features.
template <int MODE, int WT8>
__global__ __launch_bounds__(512, 1) void mm8_kernel(WsArgs a, int total, int MB) {
  using G = G8<WT8>;
  __shared__ typename G::Stage st0, st1, st2;
  int nb, split, mb;
  if (!mm_place(total, MB, a.ks, nb, split, mb)) return;
  int s = 0;  // segment of column block nb (each makes ceil(2 units / WT8) blocks)
  while (s + 1 < a.nseg) {
    const int blocks = (2 * a.seg[s].units + WT8 - 1) / WT8;
    if (nb < blocks) break;
    nb -= blocks;
    ++s;
  }
  const WsSeg sg = a.seg[s];
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), wm = w & 1, wn = w >> 1;
  const int r16 = lane & 15, g4 = (lane >> 4) * 4;
  const int m_tiles = pad16(a.M) >> 4;
  const int steps = a.K >> 5;
  const int s0 = split * steps / a.ks, n_steps = (split + 1) * steps / a.ks - s0;
  const uint16_t* p[G::LOADS];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int tm = min(mb * G::XT + (w >> 1) + 4 * j, m_tiles - 1);
    p[j] = sg.act + (w & 1) * act_plane(a.M, a.K) + ((size_t)tm * steps + s0) * 512 + lane * 8;
  }
#pragma unroll
  for (int j = 2; j < G::LOADS; ++j) {
    const int u = w + 8 * j - 2 * G::XT;  // weight tile within the block
    const uint16_t* base = sg.w0;
    int tl;
    if (MODE == WS_SWIGLU) {
      if (u >= WT8 / 2) base = sg.w1;
      tl = min(nb * (WT8 / 2) + u % (WT8 / 2), sg.units - 1);
    } else {
      tl = min(nb * WT8 + u, 2 * sg.units - 1);
    }
    p[j] = base + ((size_t)tl * steps + s0) * 512 + lane * 8;
  }
  f32x4 acc[G::WW][G::XW];
  g8_ksteps<WT8>(st0, st1, st2, p, n_steps, w, acc);

  if (MODE == WS_PARTIAL || a.ks > 1) {  // fp32 partials (SwiGLU after a k split: gate | up)
    const int up = MODE == WS_SWIGLU && wn >= 2;
#pragma unroll
    for (int i = 0; i < G::XW; ++i) {
      const int tm = mb * G::XT + wm * G::XW + i;
      const int m = tm * 16 + r16;
      if (tm >= m_tiles || m >= a.M) continue;
#pragma unroll
      for (int t = 0; t < G::WW; ++t) {
        if (MODE == WS_PARTIAL) {
          const int tile = nb * WT8 + wn * G::WW + t;
          if (tile < 2 * sg.units)
            *reinterpret_cast<f32x4*>(a.part + ((size_t)split * a.M + m) * a.n_cols + sg.col0 + tile * 16 + g4) =
                acc[t][i];
        } else {
          const int f = nb * (WT8 / 2) + (wn & 1) * G::WW + t;  // feature tile
          if (f < sg.units)
            *reinterpret_cast<f32x4*>(a.part + ((size_t)split * a.M + m) * 2 * a.n_cols + up * a.n_cols + sg.col0 +
                                      f * 16 + g4) = acc[t][i];
        }
      }
    }
    return;
  }

  // SwiGLU in registers: per row half, the two up waves park their
  // accumulators in the (free) stage buffers and the gate waves combine.
  static_assert(G::WW * G::XW * 64 <= G::BLOCKS * 64, "park fits a stage buffer");
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    f32x4* park = reinterpret_cast<f32x4*>((wn & 1) ? st1 : st0);  // [t][i][lane]
    if (wm == half && wn >= 2) {
#pragma unroll
      for (int t = 0; t < G::WW; ++t)
#pragma unroll
        for (int i = 0; i < G::XW; ++i) park[(t * G::XW + i) * 64 + lane] = acc[t][i];
    }
    __syncthreads();
    if (wm == half && wn < 2) {
#pragma unroll
      for (int i = 0; i < G::XW; ++i) {
        const int tm = mb * G::XT + wm * G::XW + i;
        const int m = tm * 16 + r16;
        if (tm >= m_tiles || m >= a.M) continue;
#pragma unroll
        for (int t = 0; t < G::WW; ++t) {
          const int f = nb * (WT8 / 2) + wn * G::WW + t;  // feature tile
          if (f >= sg.units) continue;
          const f32x4 upv = park[(t * G::XW + i) * 64 + lane];
          f32x4 y;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float gt = acc[t][i][j];
            y[j] = gt / (1.0f + __expf(-gt)) * upv[j];
          }
          u16x4 hi, lo;
          split4(y, hi, lo);
          uint16_t* dst = a.out + pk_index(m, sg.col0 + f * 16 + g4, a.n_cols);
          *reinterpret_cast<u16x4*>(dst) = hi;
          *reinterpret_cast<u16x4*>(dst + act_plane(a.M, a.n_cols)) = lo;
        }
      }
    }
    __syncthreads();  // the park area is reused by the second row half
  }
}

namespace {
constexpr int L8_XT = MM_ROW_TILES, L8_WT = 2 * MM_COL_TILES;
constexpr int L8_XW = L8_XT / 2, L8_WW = L8_WT / 4;
}  // namespace

__global__ __launch_bounds__(512, 1) void mm_lmhead_kernel(LmArgs a, int total, int MB) {
  using G = G8<L8_WT>;
  __shared__ G::Stage st0, st1, st2;  // 144 KB
  __shared__ Top2 red[4][L8_XT * 16];
  int nb, split, mb;
  if (!mm_place(total, MB, 1, nb, split, mb)) return;
  if (a.row_count && mb * L8_XT * 16 >= *a.row_count) return;  // compacted rows: nothing in this row block
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), wm = w & 1, wn = w >> 1;
  const int r16 = lane & 15, g4 = (lane >> 4) * 4;
  const int m_tiles = pad16(a.M) >> 4;
  const int v_tiles = a.V >> 4;
  const int steps = a.K >> 5;
  // wave w moves stage blocks w + 8j: j < 2 activation tile (w >> 1) + 4j,
  // plane w & 1; then weight tile w + 8j - 2 XT (clamped to the last real
  // tile: duplicates are computed and never written)
  const uint16_t* p[G::LOADS];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int tm = min(mb * L8_XT + (w >> 1) + 4 * j, m_tiles - 1);
    p[j] = a.act + (w & 1) * act_plane(a.M, a.K) + (size_t)tm * steps * 512 + lane * 8;
  }
#pragma unroll
  for (int j = 2; j < G::LOADS; ++j)
    p[j] = a.w + (size_t)min(nb * L8_WT + w + 8 * j - 2 * L8_XT, v_tiles - 1) * steps * 512 + lane * 8;
  f32x4 acc[L8_WW][L8_XW];
  g8_ksteps<L8_WT>(st0, st1, st2, p, steps, w, acc);
#pragma unroll
  for (int i = 0; i < L8_XW; ++i) {
    Top2 t2 = top2_empty();
#pragma unroll
    for (int t = 0; t < L8_WW; ++t) {
      const int vt = nb * L8_WT + wn * L8_WW + t;
      if (vt < v_tiles)
#pragma unroll
        for (int j = 0; j < 4; ++j) t2 = top2_push(t2, acc[t][i][j], vt * 16 + g4 + j);
    }
    t2 = top2_shfl_xor(t2, 16);
    t2 = top2_shfl_xor(t2, 32);
    if (lane < 16) red[wn][(wm * L8_XW + i) * 16 + lane] = t2;
    const int tm = mb * L8_XT + wm * L8_XW + i;
    const int m = tm * 16 + r16;
    if (a.dbg_logits && tm < m_tiles && m < a.M && (m % a.N) != 0) {
      float* dst = a.dbg_logits + ((size_t)(m / a.N) * (a.N - 1) + (m % a.N) - 1) * a.V;
#pragma unroll
      for (int t = 0; t < L8_WW; ++t) {
        const int vt = nb * L8_WT + wn * L8_WW + t;
        if (vt < v_tiles) *reinterpret_cast<f32x4*>(dst + vt * 16 + g4) = acc[t][i];
      }
    }
  }
  __syncthreads();
  if (threadIdx.x < L8_XT * 16) {
    const int m = mb * L8_XT * 16 + threadIdx.x;
    Top2 t = red[0][threadIdx.x];
#pragma unroll
    for (int q = 1; q < 4; ++q) t = top2_merge(t, red[q][threadIdx.x]);
    if (m < a.M) a.part[(size_t)m * a.n_parts + nb] = t;
  }
}

namespace {
int round8(int n) { return (n + 7) & ~7; }
}  // namespace

template <int WT8>
void launch_mm8(const WsArgs* a, int mode, hipStream_t st) {
  int total_nb = 0;
  for (int s = 0; s < a->nseg; ++s) total_nb += (2 * a->seg[s].units + WT8 - 1) / WT8;
  const int MB = ((pad16(a->M) >> 4) + MM_ROW_TILES - 1) / MM_ROW_TILES;
  const int total = total_nb * a->ks * MB;
  const dim3 grid(round8(total)), block(512);
  if (mode == WS_SWIGLU) launch_kernel(mm8_kernel<WS_SWIGLU, WT8>, grid, block, 0, st, *a, total, MB);
  else launch_kernel(mm8_kernel<WS_PARTIAL, WT8>, grid, block, 0, st, *a, total, MB);
}

extern "C" hipError_t dflash_launch_mm(const WsArgs* a, int mode, hipStream_t st) {
  switch (a->mm_wt) {
    case 16: launch_mm8<16>(a, mode, st); return hipGetLastError();
    case 24: launch_mm8<24>(a, mode, st); return hipGetLastError();
    case 32: launch_mm8<32>(a, mode, st); return hipGetLastError();
    default: break;
  }
  int total_nb = 0;
  for (int s = 0; s < a->nseg; ++s) total_nb += (2 * a->seg[s].units + WT - 1) / WT;
  const int XT = a->mm_xt == MM_ROW_TILES / 2 ? MM_ROW_TILES / 2 : MM_ROW_TILES;
  const int MB = ((pad16(a->M) >> 4) + XT - 1) / XT;
  const int total = total_nb * a->ks * MB;
  const dim3 grid(round8(total)), block(256);
  if (XT == MM_ROW_TILES / 2) {
    if (mode == WS_SWIGLU) launch_kernel(mm_kernel<WS_SWIGLU, MM_ROW_TILES / 2>, grid, block, 0, st, *a, total, MB);
    else launch_kernel(mm_kernel<WS_PARTIAL, MM_ROW_TILES / 2>, grid, block, 0, st, *a, total, MB);
  } else {
    if (mode == WS_SWIGLU) launch_kernel(mm_kernel<WS_SWIGLU, MM_ROW_TILES>, grid, block, 0, st, *a, total, MB);
    else launch_kernel(mm_kernel<WS_PARTIAL, MM_ROW_TILES>, grid, block, 0, st, *a, total, MB);
  }
  return hipGetLastError();
}

extern "C" hipError_t dflash_launch_swiglu_finish(const WsArgs* a, hipStream_t st) {
  launch_kernel(swiglu_finish_kernel, dim3((a->M + 15) / 16 * ((a->n_cols + 63) / 64)), dim3(256), 0, st, *a);
  return hipGetLastError();
}

extern "C" hipError_t dflash_launch_lmhead_mm(const LmArgs* a, hipStream_t st) {
  const int NB = ((a->V >> 4) + L8_WT - 1) / L8_WT;
  const int MB = ((pad16(a->M) >> 4) + L8_XT - 1) / L8_XT;
  const int total = NB * MB;
  launch_kernel(mm_lmhead_kernel, dim3(round8(total)), dim3(512), 0, st, *a, total, MB);
  return hipGetLastError();
}
