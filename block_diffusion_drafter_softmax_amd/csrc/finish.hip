// Finishers of the split-k projections: add the k-split partial sums in split
// order, apply RoPE to keys/queries (rotate-half pairs (j, j + d/2) at the
// row's position, cos/sin from the set-up table) and write the layout the
// consumer wants: the attention's query rows (split hi/lo activation) and
// block K/V (bf16), or the paged context cache (bf16; keys slot-major,
// values dim-major).
#include "common.h"

namespace {
DEV int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// RoPE of 4 consecutive rotate-half pairs (i .. i+3, i+half .. i+half+3; i a
// multiple of 4) at position pos: the 8 cos/sin values are two 16-byte loads
// of the table [pos][half][cos, sin].
DEV void rotate4(f32x4& x1, f32x4& x2, const float* rope, int pos, int half, int i) {
  if (rope == nullptr) return;
  const f32x4* cs = reinterpret_cast<const f32x4*>(rope + ((size_t)pos * half + i) * 2);
  const f32x4 p0 = cs[0], p1 = cs[1];  // (cos, sin) of pairs i, i+1 and i+2, i+3
  const f32x4 c = {p0[0], p0[2], p1[0], p1[2]}, sn = {p0[1], p0[3], p1[1], p1[3]};
  const f32x4 y1 = x1 * c - x2 * sn, y2 = x2 * c + x1 * sn;
  x1 = y1;
  x2 = y2;
}
}  // namespace

// One thread per (row, 4 consecutive rotation pairs of a query or block-key
// head) or per (row, 4 consecutive block-value elements): 16-byte loads of
// every split partial and of the cos/sin pairs, 8-byte query and key
// stores (d_h is 64 or 128: a head holds whole groups of 4).
DEV void qkv_finish_body(const QkvFinishArgs& a, int idx) {
  if (a.attn_ctr && idx < 8) a.attn_ctr[idx] = 0;  // the next attention's work counters
  const int d = a.d, half = d / 2;
  const int pq = a.n_q * half / 4, pk = a.n_kv * half / 4, nv = a.n_kv * d / 4;  // groups of 4 per row
  const int per_row = pq + pk + nv;
  const int n_cols = (a.n_q + 2 * a.n_kv) * d;
  if (idx >= a.M * per_row) return;
  const int m = idx / per_row, j = idx % per_row;
  const int b = m / a.N, n = m % a.N;
  const size_t plane = (size_t)a.M * n_cols, row = (size_t)m * n_cols;
  if (j < pq + pk) {
    const bool isq = j < pq;
    const int jj = (isq ? j : j - pq) * 4;
    const int head = jj / half, i = jj % half;  // pairs (i .. i+3, i+half .. i+half+3)
    const int col = (isq ? 0 : a.n_q * d) + head * d + i;
    f32x4 x1 = split_sum4(a.part, a.ks, plane, row + col);
    f32x4 x2 = split_sum4(a.part, a.ks, plane, row + col + half);
    rotate4(x1, x2, a.rope, m, half, i);  // the call's plan holds row m's cos/sin
    if (isq) {  // query, scaled for a log2-domain softmax: split activation of the attention
      uint16_t* dst = a.q + ((size_t)m * a.n_q + head) * d;
      const size_t lo = (size_t)a.M * a.n_q * d;
      u16x4 h1, l1, h2, l2;
      split4(x1 * a.q_scale, h1, l1);
      split4(x2 * a.q_scale, h2, l2);
      *reinterpret_cast<u16x4*>(dst + i) = h1;
      *reinterpret_cast<u16x4*>(dst + lo + i) = l1;
      *reinterpret_cast<u16x4*>(dst + i + half) = h2;
      *reinterpret_cast<u16x4*>(dst + lo + i + half) = l2;
    } else {  // block key: bf16 storage
      uint16_t* dst = a.kblk + (((size_t)b * a.n_kv + head) * 16 + n) * d;
      *reinterpret_cast<u16x4*>(dst + i) = u16x4{f2bf(x1[0]), f2bf(x1[1]), f2bf(x1[2]), f2bf(x1[3])};
      *reinterpret_cast<u16x4*>(dst + i + half) = u16x4{f2bf(x2[0]), f2bf(x2[1]), f2bf(x2[2]), f2bf(x2[3])};
    }
  } else {  // block value: dim-major, slot n of 16
    const int jj = (j - pq - pk) * 4;
    const int head = jj / d, dd = jj % d;
    const f32x4 v = split_sum4(a.part, a.ks, plane, row + (a.n_q + a.n_kv) * d + jj);
    uint16_t* dst = a.vblk + (((size_t)b * a.n_kv + head) * d + dd) * 16 + n;
#pragma unroll
    for (int t = 0; t < 4; ++t) dst[t * 16] = f2bf(v[t]);
  }
}

__global__ __launch_bounds__(256) LATENCY_BOUND void qkv_finish_kernel(QkvFinishArgs a) {
  qkv_finish_body(a, blockIdx.x * blockDim.x + threadIdx.x);
}

extern "C" hipError_t dflash_launch_qkv_finish(const QkvFinishArgs* a, hipStream_t st) {
  const int per_row = ((a->n_q + a->n_kv) * (a->d / 2) + a->n_kv * a->d) / 4;  // groups of 4
  const int total = a->M * per_row;
  launch_kernel(qkv_finish_kernel, dim3((total + 255) / 256), dim3(256), 0, st, *a);
  return hipGetLastError();
}

// One thread per (appended row, layer, 4 consecutive key rotation pairs or
// value elements of a head); the first B threads also advance the context
// length of the call's sequences (the append's last kernel: nothing after it
// reads the old one).
DEV void ctx_finish_body(const CtxFinishArgs& a, int idx) {
  const int d = a.d, half = d / 2, kvd = a.n_kv * d;
  const int pk = a.n_kv * half / 4, pv = kvd / 4;  // groups of 4
  const int per_layer = pk + pv;
  const int per_row = a.D * per_layer;
  const int n_cols = a.D * 2 * kvd;
  if (idx < a.B) {
    const int m0 = idx * a.max_new;
    if (a.row_pos[m0] >= 0) a.ctx_len[a.row_seq[m0]] = a.row_pos[m0] + a.n_new[idx];
  }
  if (idx >= a.M * per_row) return;
  const int m = idx / per_row, rem = idx % per_row;
  const int pos = a.row_pos[m];
  if (pos < 0) return;
  const int layer = rem / per_layer, j = rem % per_layer;
  const int seq = a.row_seq[m];
  const int page = clampi(a.page_table[(size_t)seq * a.max_pages_per_seq + pos / 16], 0, a.n_pages - 1);
  const int slot = pos % 16;
  uint16_t* base = a.kv_pages + layer * a.layer_stride + (size_t)page * 2 * kvd * 16;
  const size_t plane = (size_t)a.M * n_cols, row = (size_t)m * n_cols;
  if (j < pk) {  // key: rotated, slot-major
    const int jj = j * 4, head = jj / half, i = jj % half;
    const int col = layer * 2 * kvd + head * d + i;
    f32x4 x1 = split_sum4(a.part, a.ks, plane, row + col);
    f32x4 x2 = split_sum4(a.part, a.ks, plane, row + col + half);
    rotate4(x1, x2, a.rope, pos, half, i);
    uint16_t* dst = base + ((size_t)head * 16 + slot) * d;
    *reinterpret_cast<u16x4*>(dst + i) = u16x4{f2bf(x1[0]), f2bf(x1[1]), f2bf(x1[2]), f2bf(x1[3])};
    *reinterpret_cast<u16x4*>(dst + i + half) = u16x4{f2bf(x2[0]), f2bf(x2[1]), f2bf(x2[2]), f2bf(x2[3])};
  } else {  // value: dim-major
    const int jj = (j - pk) * 4, head = jj / d, dd = jj % d;
    const f32x4 v = split_sum4(a.part, a.ks, plane, row + layer * 2 * kvd + kvd + jj);
    uint16_t* dst = base + (size_t)kvd * 16 + ((size_t)head * d + dd) * 16 + slot;
#pragma unroll
    for (int t = 0; t < 4; ++t) dst[t * 16] = f2bf(v[t]);
  }
}

__global__ __launch_bounds__(256) LATENCY_BOUND void ctx_finish_kernel(CtxFinishArgs a) {
  ctx_finish_body(a, blockIdx.x * blockDim.x + threadIdx.x);
}

extern "C" hipError_t dflash_launch_ctx_finish(const CtxFinishArgs* a, hipStream_t st) {
  const int per_row = a->D * ((a->n_kv * (a->d / 2) + a->n_kv * a->d) / 4);  // groups of 4
  const int total = a->M * per_row;
  launch_kernel(ctx_finish_kernel, dim3((total + 255) / 256), dim3(256), 0, st, *a);
  return hipGetLastError();
}

// Append and draft launched together: the context finisher (all layers;
// it also advances ctx_len) and the first draft layer's query/key/value
// finisher in one launch of independent workgroups.
__global__ __launch_bounds__(256) LATENCY_BOUND void finish2_kernel(CtxFinishArgs ca, QkvFinishArgs qa, int n_ctx) {
  const int x = blockIdx.x;
  if (x < n_ctx) ctx_finish_body(ca, x * blockDim.x + threadIdx.x);
  else qkv_finish_body(qa, (x - n_ctx) * blockDim.x + threadIdx.x);
}

extern "C" hipError_t dflash_launch_finish2(const CtxFinishArgs* ca, const QkvFinishArgs* qa, hipStream_t st) {
  const int n_ctx = (ca->M * ca->D * ((ca->n_kv * (ca->d / 2) + ca->n_kv * ca->d) / 4) + 255) / 256;
  const int n_qkv = (qa->M * (((qa->n_q + qa->n_kv) * (qa->d / 2) + qa->n_kv * qa->d) / 4) + 255) / 256;
  launch_kernel(finish2_kernel, dim3(n_ctx + n_qkv), dim3(256), 0, st, *ca, *qa, n_ctx);
  return hipGetLastError();
}
