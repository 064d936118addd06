// Block attention: the N block queries of every head attend, with no mask,
// to all L context keys of their sequence plus the N block keys (the draft
// is not autoregressive; the fused target context enters each draft layer
// as keys/values only).
//
// Work item = (key chunk, kv head, sequence). Chunk 0 is the block's own N
// keys; chunks 1.. cover the context in pieces of CH = 128 keys (8 pages).
// A workgroup holds all R = (n_q/n_kv)*N query rows of one kv head (GQA: a
// K/V tile is read from HBM once for the whole query group), one wave per 16
// rows. The chunk's page indices are read first, then every K and V byte of
// the chunk is requested at once and staged in LDS, so a workgroup waits for
// two memory latencies in total. Per 32-key step a wave computes S^T = K Q^T
// with MFMA (keys as rows, the lane's query as column), runs an online
// softmax in the log2 domain, and accumulates O^T += V^T P^T with MFMA: V is
// stored dim-major per page ([d_h][16 slots]), so its A-operand fragments are
// contiguous, and P^T comes straight from the S^T accumulators (both MFMAs use
// the same permutation of the 32 keys). Q and P are fp32 values entering
// the MFMAs as hi/lo bf16 pairs (two MFMAs each); K and V are bf16 storage.
// Unnormalised O, the running max and the sum go to a partial buffer;
// attn_merge_kernel combines the chunks.
#include "common.h"
#include "dflash.h"

namespace {
DEV int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }
constexpr int CH = 128;  // context keys per work item
}  // namespace

template <int D>
__global__ __launch_bounds__(1024) LATENCY_BOUND void attn_chunk_kernel(AttnArgs a) {
  constexpr int KP = D + 8;          // padded LDS row of one key (bf16 elements)
  constexpr int PAGES = CH / 16;
  __shared__ uint16_t k_lds[CH * KP];
  __shared__ uint16_t v_lds[PAGES * D * 16];
  __shared__ int pg[PAGES];

  const int c = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int seq = clampi(a.seq_ids[b], 0, a.max_seqs - 1);
  const int L = clampi(a.ctx_len[seq], 0, a.max_pages_per_seq * 16);
  int key_begin, key_end;
  if (c == 0) {
    key_begin = 0;
    key_end = a.N;
  } else {
    key_begin = (c - 1) * CH;
    key_end = min(L, c * CH);
    if (key_begin >= key_end) return;
  }
  const int nkeys = key_end - key_begin;
  const int np = (nkeys + 15) / 16;
  const int tid = threadIdx.x, nthreads = blockDim.x;
  const size_t page_elems = (size_t)2 * a.n_kv * 16 * D;

  if (tid < np) {
    int p = 0;
    if (c > 0) {
      const int raw = a.page_table[(size_t)seq * a.max_pages_per_seq + key_begin / 16 + tid];
      if (raw < 0 || raw >= a.n_pages) set_error(a.err, DFLASH_DEV_BAD_PAGE);
      p = clampi(raw, 0, a.n_pages - 1);
    }
    pg[tid] = p;
  }
  __syncthreads();

  // Stage K (slot-major rows) and V (dim-major) of the chunk's pages in LDS:
  // per page, 2*D*16 bf16 = 4*D 16-byte units (K units first, then V units).
  // Batches of 8 loads per thread, all in flight before the LDS stores: unit
  // indices are clamped (a clamped duplicate loads valid memory and is not
  // stored), so no branch separates the loads.
  constexpr int UNITS_PER_PAGE = 4 * D;
  const int total_units = np * UNITS_PER_PAGE;
  const uint16_t* blk_k = a.kblk + ((size_t)b * a.n_kv + kvh) * 16 * D;
  const uint16_t* blk_v = a.vblk + ((size_t)b * a.n_kv + kvh) * D * 16;
  for (int base = 0; base < total_units; base += 8 * nthreads) {
    int uu[8], pgv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) uu[j] = min(base + j * nthreads + tid, total_units - 1);
#pragma unroll
    for (int j = 0; j < 8; ++j) pgv[j] = pg[uu[j] / UNITS_PER_PAGE];
    u32x4 buf[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int p = uu[j] / UNITS_PER_PAGE, w = uu[j] % UNITS_PER_PAGE;
      const uint16_t* kb = (c == 0) ? blk_k : a.pages + pgv[j] * page_elems + (size_t)kvh * 16 * D;
      const uint16_t* vb = (c == 0) ? blk_v : kb + (size_t)a.n_kv * 16 * D;
      const uint16_t* src = (w < 2 * D) ? kb + (w / (D / 8)) * D + (w % (D / 8)) * 8 : vb + (w - 2 * D) * 8;
      buf[j] = *reinterpret_cast<const u32x4*>(src);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (base + j * nthreads + tid >= total_units) continue;
      const int p = uu[j] / UNITS_PER_PAGE, w = uu[j] % UNITS_PER_PAGE;
      if (w < 2 * D) {  // K: 16 slots x D, 8 elements per unit
        *reinterpret_cast<u32x4*>(&k_lds[(p * 16 + w / (D / 8)) * KP + (w % (D / 8)) * 8]) = buf[j];
      } else {
        *reinterpret_cast<u32x4*>(&v_lds[p * D * 16 + (w - 2 * D) * 8]) = buf[j];
      }
    }
  }
  __syncthreads();

  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int G = a.n_q / a.n_kv, R = G * a.N;
  const int r = wave * 16 + r16;
  const int hq = kvh * G + r / a.N, n = r % a.N;
  constexpr int KD = D / 32, DT = D / 16;

  bf16x8 qh[KD], ql[KD];
  const uint16_t* qp = a.q + ((size_t)(b * a.N + n) * a.n_q + hq) * D + 8 * g;
  const size_t q_lo = (size_t)gridDim.z * a.N * a.n_q * D;
#pragma unroll
  for (int kd = 0; kd < KD; ++kd) {
    qh[kd] = ld8(qp + kd * 32);
    ql[kd] = ld8(qp + q_lo + kd * 32);
  }

  f32x4 acc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  for (int k0 = 0; k0 < nkeys; k0 += 32) {  // chunk-relative keys
    const bool t1 = k0 + 16 < nkeys;
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kd = 0; kd < KD; ++kd) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(&k_lds[(k0 + r16) * KP + kd * 32 + 8 * g]);
      s0 = mfma16(kf, qh[kd], s0);
      s0 = mfma16(kf, ql[kd], s0);
    }
    if (t1) {
#pragma unroll
      for (int kd = 0; kd < KD; ++kd) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(&k_lds[(k0 + 16 + r16) * KP + kd * 32 + 8 * g]);
        s1 = mfma16(kf, qh[kd], s1);
        s1 = mfma16(kf, ql[kd], s1);
      }
    }
    // lane holds keys k0 + 4g + i (s0) and k0 + 16 + 4g + i (s1) for query r
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = (k0 + 4 * g + i < nkeys) ? s0[i] * a.scale_log2 : -INFINITY;
      x[4 + i] = (t1 && k0 + 16 + 4 * g + i < nkeys) ? s1[i] * a.scale_log2 : -INFINITY;
    }
    float mt = x[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) mt = fmaxf(mt, x[j]);
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m_run, mt);
    const float corr = exp2f(m_run - m_new);
    f32x4 p0, p1;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p0[i] = exp2f(x[i] - m_new);
      p1[i] = exp2f(x[4 + i] - m_new);
      psum += p0[i] + p1[i];
    }
    l_run = l_run * corr + psum;
    m_run = m_new;
    u16x4 h0, l0, h1, l1;
    split4(p0, h0, l0);
    split4(p1, h1, l1);
    const bf16x8 ph = __builtin_bit_cast(bf16x8, __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7));
    const bf16x8 pl = __builtin_bit_cast(bf16x8, __builtin_shufflevector(l0, l1, 0, 1, 2, 3, 4, 5, 6, 7));
    const uint16_t* vp0 = &v_lds[(k0 / 16) * D * 16];
    const uint16_t* vp1 = vp0 + D * 16;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      u16x4 v0 = *reinterpret_cast<const u16x4*>(vp0 + (t * 16 + r16) * 16 + 4 * g);
      u16x4 v1 = {0, 0, 0, 0};
      if (t1) v1 = *reinterpret_cast<const u16x4*>(vp1 + (t * 16 + r16) * 16 + 4 * g);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (k0 + 4 * g + i >= nkeys) v0[i] = 0;
        if (k0 + 16 + 4 * g + i >= nkeys) v1[i] = 0;
      }
      const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
      acc[t] = acc[t] * corr;
      acc[t] = mfma16(vf, ph, acc[t]);
      acc[t] = mfma16(vf, pl, acc[t]);
    }
  }
  float l = l_run + __shfl_xor(l_run, 16, 64);
  l += __shfl_xor(l, 32, 64);

  const size_t unit = ((size_t)b * a.n_kv + kvh) * a.n_ck + c;
  float* po = a.part_o + (unit * R + r) * D;
#pragma unroll
  for (int t = 0; t < DT; ++t) *reinterpret_cast<f32x4*>(po + t * 16 + 4 * g) = acc[t];
  if (g == 0) {
    a.part_ml[(unit * R + r) * 2 + 0] = m_run;
    a.part_ml[(unit * R + r) * 2 + 1] = l;
  }
}

// One thread per (sequence, kv head, query row, 4 dims): single-pass
// log-sum-exp merge of the chunk partials in chunk order, normalise, and
// write the O-projection's packed split activation.
template <int D>
__global__ __launch_bounds__(256) LATENCY_BOUND void attn_merge_kernel(AttnArgs a, int B) {
  const int G = a.n_q / a.n_kv, R = G * a.N;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  const int dq = idx % (D / 4);
  const int r = (idx / (D / 4)) % R;
  const int kvh = (idx / (D / 4) / R) % a.n_kv;
  const int b = idx / (D / 4) / R / a.n_kv;
  if (b >= B) return;
  const int seq = clampi(a.seq_ids[b], 0, a.max_seqs - 1);
  const int L = clampi(a.ctx_len[seq], 0, a.max_pages_per_seq * 16);
  const int nc = min(a.n_ck, 1 + (L + CH - 1) / CH);
  const size_t unit0 = ((size_t)b * a.n_kv + kvh) * a.n_ck;
  float M = -INFINITY, den = 0.f;
  f32x4 num = {0.f, 0.f, 0.f, 0.f};
  constexpr int GRP = 8;  // chunks whose loads are in flight together (more costs time on gfx950)
  for (int c0 = 0; c0 < nc; c0 += GRP) {
    float2 ml[GRP];
    f32x4 ov[GRP];
#pragma unroll
    for (int j = 0; j < GRP; ++j) {
      const size_t row = (unit0 + min(c0 + j, nc - 1)) * R + r;
      ml[j] = *reinterpret_cast<const float2*>(a.part_ml + row * 2);
      ov[j] = *reinterpret_cast<const f32x4*>(a.part_o + row * D + dq * 4);
    }
#pragma unroll
    for (int j = 0; j < GRP; ++j) {
      if (c0 + j >= nc) break;
      const float Mn = fmaxf(M, ml[j].x);
      const float wo = exp2f(M - Mn), wn = exp2f(ml[j].x - Mn);
      den = den * wo + ml[j].y * wn;
      num = num * wo + ov[j] * wn;
      M = Mn;
    }
  }
  const float inv = 1.0f / den;
  const int hq = kvh * G + r / a.N, n = r % a.N;
  const int m = b * a.N + n, qd = a.n_q * D;
  u16x4 hi, lo;
  split4(num * inv, hi, lo);
  uint16_t* dst = a.o + pk_index(m, hq * D + dq * 4, qd);
  *reinterpret_cast<u16x4*>(dst) = hi;
  *reinterpret_cast<u16x4*>(dst + act_plane(B * a.N, qd)) = lo;
}

extern "C" hipError_t dflash_launch_attn(const AttnArgs* a, int B, int head_dim, hipStream_t st) {
  const int G = a->n_q / a->n_kv, R = G * a->N;
  const dim3 grid(a->n_ck, a->n_kv, B), block(64 * (R / 16));
  if (head_dim == 128) launch_kernel(attn_chunk_kernel<128>, grid, block, 0, st, *a);
  else launch_kernel(attn_chunk_kernel<64>, grid, block, 0, st, *a);
  return hipGetLastError();
}

extern "C" hipError_t dflash_launch_attn_merge(const AttnArgs* a, int B, int head_dim, hipStream_t st) {
  const int G = a->n_q / a->n_kv, R = G * a->N;
  const int total = B * a->n_kv * R * (head_dim / 4);
  const dim3 grid((total + 255) / 256), block(256);
  if (head_dim == 128) launch_kernel(attn_merge_kernel<128>, grid, block, 0, st, *a, B);
  else launch_kernel(attn_merge_kernel<64>, grid, block, 0, st, *a, B);
  return hipGetLastError();
}
