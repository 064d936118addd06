// Parallel verification of the drafted blocks against the target's logits
// (greedy, or temperature-1 rejection sampling of an argmax draft or of a
// draft sampled at temperature tau), and the sampling of such drafts.
//
// verify_rows_kernel streams every logit once: work item = (vocabulary chunk
// of up to 32768 logits, block row, sequence). Greedy keeps (max, lowest
// index); temperature 1 keeps (max, sum of exp(z - max)). A second kernel
// merges each row's chunks in chunk order and runs the accept scan
// (verify_greedy_kernel, one workgroup per sequence). Temperature 1 also
// samples from one row: verify_sample_kernel repeats the scan in every
// work item (vocabulary chunk, sequence; chunks sized per call so that a
// batch-1 row still spreads over ~512 work items) -- it is a few dozen
// loads -- and takes a Gumbel-max over its chunk with a counter-based
// Philox4x64-10 draw per vocabulary entry, which gives the same sample
// whatever the order; verify_pick_kernel merges the chunks. Kernel
// boundaries order the passes: a device-scope hand-off inside a kernel
// costs an L2 write-back per workgroup, which thousands of workgroups (32
// sequences x 16 rows x 5 chunks) cannot afford.
#include <mutex>

#include "common.h"
#include "dflash.h"


namespace {
DEV float load_logit(const VerifyArgs& a, size_t i) {
  if (a.dtype == DFLASH_DTYPE_F32) return ((const float*)a.logits)[i];
  return bf2f(((const uint16_t*)a.logits)[i]);
}

// Philox4x64-10 (Salmon et al., SC 2011), published multipliers and Weyl
// constants.
DEV void philox4x64_10(unsigned long long c[4], unsigned long long k0, unsigned long long k1) {
  const unsigned long long M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const unsigned long long W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const unsigned long long lo0 = M0 * c[0], hi0 = __umul64hi(M0, c[0]);
    const unsigned long long lo1 = M1 * c[2], hi1 = __umul64hi(M1, c[2]);
    const unsigned long long n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
    k0 += W0; k1 += W1;
  }
}

// Word 0 of Philox at counter (k, row | stream << 32, seq, step), key (seed, 0).
DEV unsigned long long rng_word(const VerifyArgs& a, int seq, int row, int k, int stream) {
  unsigned long long c[4] = {(unsigned long long)(unsigned)k,
                             (unsigned long long)(unsigned)row | ((unsigned long long)stream << 32),
                             (unsigned long long)(unsigned)seq, a.step};
  philox4x64_10(c, a.seed, 0ull);
  return c[0];
}

DEV int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

struct ArgMax {
  float v;
  int i;
};
DEV ArgMax am_merge(ArgMax x, ArgMax y) { return better(x.v, x.i, y.v, y.i) ? x : y; }
DEV ArgMax am_shfl(ArgMax x, int o) {
  ArgMax y{__shfl_xor(x.v, o, 64), __shfl_xor(x.i, o, 64)};
  return am_merge(x, y);
}

// max and sum of exp(z - max) pairs
DEV float2 ms_merge(float2 x, float2 y) {
  const float m = fmaxf(x.x, y.x);
  if (m == -INFINITY) return make_float2(m, 0.f);
  return make_float2(m, x.y * __expf(x.x - m) + y.y * __expf(y.x - m));
}
}  // namespace

namespace {
// Eight consecutive logits k .. k+7 (k % 8 == 0) as fp32.
template <int DTYPE>
DEV void load8(const VerifyArgs& a, size_t i, float (&z)[8]) {
  if (DTYPE == DFLASH_DTYPE_F32) {
    const f32x4 lo = *reinterpret_cast<const f32x4*>((const float*)a.logits + i);
    const f32x4 hi = *reinterpret_cast<const f32x4*>((const float*)a.logits + i + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      z[e] = lo[e];
      z[4 + e] = hi[e];
    }
  } else {
    const u32x4 v = *reinterpret_cast<const u32x4*>((const uint16_t*)a.logits + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      z[2 * e] = __uint_as_float(v[e] << 16);
      z[2 * e + 1] = __uint_as_float(v[e] & 0xFFFF0000u);
    }
  }
}
}  // namespace

// Work item = (vocabulary chunk, block row, sequence); chunk % 8 == 0 and
// V % 8 == 0, so every thread reads whole 8-logit groups, 8 groups in
// flight per batch.
#define VERIFY_THREADS 1024
#define VG 4  // 8-logit groups per thread in flight: a 32768-logit chunk in one batch
template <int DTYPE>
__global__ __launch_bounds__(VERIFY_THREADS) LATENCY_BOUND void verify_rows_kernel(VerifyArgs a) {
  const int c = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
  const size_t row_off = ((size_t)b * a.N + r) * a.V;
  const int k0 = c * a.chunk, k1 = min(a.V, k0 + a.chunk);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int NW = VERIFY_THREADS / 64;
  __shared__ float2 red[NW];
  float2 res = make_float2(0.f, 0.f);
  if (!a.temp1) {
    ArgMax t{-INFINITY, 0x7FFFFFFF};
    for (int base = k0; base < k1; base += VERIFY_THREADS * 8 * VG) {
      float zs[VG][8];
#pragma unroll
      for (int j = 0; j < VG; ++j) {  // clamped loads, all in flight; unused past k1
        const int k = min(base + (int)(threadIdx.x + VERIFY_THREADS * j) * 8, k1 - 8);
        load8<DTYPE>(a, row_off + k, zs[j]);
      }
#pragma unroll
      for (int j = 0; j < VG; ++j) {
        const int k = base + (threadIdx.x + VERIFY_THREADS * j) * 8;
        if (k < k1) {
#pragma unroll
          for (int e = 0; e < 8; ++e) t = am_merge(t, ArgMax{zs[j][e], k + e});
        }
      }
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) t = am_shfl(t, o);
    if (lane == 0) red[wave] = make_float2(t.v, __int_as_float(t.i));
    __syncthreads();
    if (threadIdx.x == 0) {
      ArgMax u{red[0].x, __float_as_int(red[0].y)};
      for (int w = 1; w < NW; ++w) u = am_merge(u, ArgMax{red[w].x, __float_as_int(red[w].y)});
      res = make_float2(u.v, __int_as_float(u.i));
    }
  } else {
    float2 ms = make_float2(-INFINITY, 0.f);  // (max, sum of exp(z - max)) of this thread's logits
    for (int base = k0; base < k1; base += VERIFY_THREADS * 8 * VG) {
      float zs[VG][8];
#pragma unroll
      for (int j = 0; j < VG; ++j) {
        const int k = min(base + (int)(threadIdx.x + VERIFY_THREADS * j) * 8, k1 - 8);
        load8<DTYPE>(a, row_off + k, zs[j]);
      }
#pragma unroll
      for (int j = 0; j < VG; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) zs[j][e] *= a.inv_scale;  // 1 for the target; 1/tau for the drafter
      float m = -INFINITY;
#pragma unroll
      for (int j = 0; j < VG; ++j) {
        if (base + (int)(threadIdx.x + VERIFY_THREADS * j) * 8 >= k1) continue;
#pragma unroll
        for (int e = 0; e < 8; ++e) m = fmaxf(m, zs[j][e]);
      }
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < VG; ++j) {
        if (base + (int)(threadIdx.x + VERIFY_THREADS * j) * 8 >= k1) continue;
#pragma unroll
        for (int e = 0; e < 8; ++e) sum += __expf(zs[j][e] - m);
      }
      ms = ms_merge(ms, make_float2(m, sum));
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1)
      ms = ms_merge(ms, make_float2(__shfl_xor(ms.x, o, 64), __shfl_xor(ms.y, o, 64)));
    if (lane == 0) red[wave] = ms;
    __syncthreads();
    if (threadIdx.x == 0) {
      float2 u = red[0];
      for (int w = 1; w < NW; ++w) u = ms_merge(u, red[w]);
      res = u;
    }
  }
  if (threadIdx.x == 0) *reinterpret_cast<float2*>(a.part + ((((size_t)b * a.N + r) * a.n_chunks + c) * 2)) = res;
}

namespace {
// Accept scan of sequence b from the rows pass: every (row, chunk) result
// is loaded in one batch into LDS, thread `row` merges its row's chunks in
// chunk order, then every thread reads the scan's outcome. Greedy: acc and
// the target's argmax of row acc (next token). Temperature 1: acc, and the
// token excluded when sampling row acc (the rejected draft token, or -1).
struct Scan {
  int acc, next, excl;
  float lse_p, lse_q;  // sampled drafts: log-normalisers of row acc (target, drafter / tau)
};

template <int NT>
DEV Scan verify_scan(const VerifyArgs& a, int b) {
  __shared__ float2 parts[VERIFY_MAX_PARTS];
  __shared__ float2 rowres[32];
  __shared__ float prob[32], unif[32], qprob[32], lsep[32], lseq[32];
  __shared__ Scan out;
  const int* d = a.draft + (size_t)b * (a.N - 1);
  const int n_parts = a.N * a.n_chunks;  // <= VERIFY_MAX_PARTS (host check)
  const float2* src = reinterpret_cast<const float2*>(a.part) + (size_t)b * n_parts;
  for (int p0 = 0; p0 < n_parts; p0 += NT * 8) {
    float2 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = src[min(p0 + j * NT + (int)threadIdx.x, n_parts - 1)];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (p0 + j * NT + (int)threadIdx.x < n_parts) parts[p0 + j * NT + threadIdx.x] = v[j];
  }
  __syncthreads();
  const int row = threadIdx.x;
  if (row < a.N) {
    if (!a.temp1) {
      ArgMax u{-INFINITY, 0x7FFFFFFF};
      for (int cc = 0; cc < a.n_chunks; ++cc) {
        const float2 p = parts[row * a.n_chunks + cc];
        u = am_merge(u, ArgMax{p.x, __float_as_int(p.y)});
      }
      rowres[row] = make_float2(u.v, __int_as_float(u.i));
    } else if (row < a.N - 1) {
      float2 ms = make_float2(-INFINITY, 0.f);
      for (int cc = 0; cc < a.n_chunks; ++cc) ms = ms_merge(ms, parts[row * a.n_chunks + cc]);
      const float lse = ms.x + __logf(ms.y);
      int tok = d[row];
      if (tok < 0 || tok >= a.V) {
        set_error(a.err, DFLASH_DEV_BAD_TOKEN);
        tok = clampi(tok, 0, a.V - 1);
      }
      const float zt = load_logit(a, ((size_t)b * a.N + row) * a.V + tok);
      prob[row] = expf(zt - lse);
      unif[row] = (float)(rng_word(a, a.seq_ids[b], row, 0, 0) >> 40) * 5.9604644775390625e-08f;
      if (a.sampled) {  // the drafter's probability of its own token: q = softmax(z / tau)
        float2 mq = make_float2(-INFINITY, 0.f);
        const float2* qp = reinterpret_cast<const float2*>(a.qpart) + ((size_t)b * (a.N - 1) + row) * a.n_chunks;
        for (int cc = 0; cc < a.n_chunks; ++cc) mq = ms_merge(mq, qp[cc]);
        const float lq = mq.x + __logf(mq.y);
        qprob[row] = expf(a.qlogits[((size_t)b * (a.N - 1) + row) * a.V + tok] * a.inv_tau - lq);
        lsep[row] = lse;
        lseq[row] = lq;
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    Scan r;
    if (!a.temp1) {
      while (acc < a.N - 1 && d[acc] == __float_as_int(rowres[acc].y)) ++acc;
      r = Scan{acc, __float_as_int(rowres[acc].y), -1, 0.f, 0.f};
    } else if (!a.sampled) {
      while (acc < a.N - 1 && unif[acc] < prob[acc]) ++acc;
      r = Scan{acc, -1, acc < a.N - 1 ? d[acc] : -1};
    } else {  // accept with probability min(1, p/q)
      while (acc < a.N - 1 && unif[acc] * qprob[acc] < prob[acc]) ++acc;
      r = Scan{acc, -1, -1, acc < a.N - 1 ? lsep[acc] : 0.f, acc < a.N - 1 ? lseq[acc] : 0.f};
    }
    out = r;
  }
  __syncthreads();
  return out;
}
}  // namespace

#define SCAN_THREADS 256

__global__ __launch_bounds__(SCAN_THREADS) LATENCY_BOUND void verify_greedy_kernel(VerifyArgs a) {
  const int b = blockIdx.x;
  const Scan r = verify_scan<SCAN_THREADS>(a, b);
  if (threadIdx.x != 0) return;
  a.accept_len[b] = r.acc;
  a.next_token[b] = r.next;
  if (a.commit_len) a.commit_len[b] = r.acc + 1;
}

// Gumbel-max sample over vocabulary chunk c of row acc, the excluded token
// skipped; the chunk's (value, index) goes to spart[b][c].
__global__ __launch_bounds__(SCAN_THREADS) LATENCY_BOUND void verify_sample_kernel(VerifyArgs a) {
  const int c = blockIdx.x, b = blockIdx.y;
  const Scan r = verify_scan<SCAN_THREADS>(a, b);
  if (c == 0 && threadIdx.x == 0) {
    a.accept_len[b] = r.acc;
    if (a.commit_len) a.commit_len[b] = r.acc + 1;
  }
  const int row = r.acc, excl = r.excl;
  const int seq = a.seq_ids[b];
  const size_t row_off = ((size_t)b * a.N + row) * a.V;
  const int k0 = c * a.s_chunk, k1 = min(a.V, k0 + a.s_chunk);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  ArgMax t{-INFINITY, 0x7FFFFFFF};
  const bool residual = a.sampled && row < a.N - 1;  // max(0, p - q) of a sampled draft
  const float* qrow = residual ? a.qlogits + ((size_t)b * (a.N - 1) + row) * a.V : nullptr;
  for (int k = k0 + threadIdx.x; k < k1; k += SCAN_THREADS) {
    if (k == excl) continue;
    const unsigned long long w = rng_word(a, seq, row, k, 1);
    const float u = ((float)(w >> 41) + 0.5f) * 1.1920928955078125e-07f;
    const float gmb = -logf(-logf(u));
    float key = load_logit(a, row_off + k) + gmb;
    if (residual) {
      const float rw = expf(load_logit(a, row_off + k) - r.lse_p) - expf(qrow[k] * a.inv_tau - r.lse_q);
      key = rw > 0.f ? logf(rw) + gmb : -INFINITY;
    }
    t = am_merge(t, ArgMax{key, k});
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) t = am_shfl(t, o);
  __shared__ ArgMax red[SCAN_THREADS / 64];
  if (lane == 0) red[wave] = t;
  __syncthreads();
  if (threadIdx.x != 0) return;
  ArgMax u = red[0];
  for (int w = 1; w < SCAN_THREADS / 64; ++w) u = am_merge(u, red[w]);
  *reinterpret_cast<float2*>(a.spart + (((size_t)b * a.s_n_chunks + c) * 2)) = make_float2(u.v, __int_as_float(u.i));
}

// Next token of sequence b (temperature 1): merge of the sampling chunks in
// chunk order (one wave per sequence, loads in one batch).
__global__ __launch_bounds__(64) void verify_pick_kernel(VerifyArgs a) {
  const int b = blockIdx.x, lane = threadIdx.x;
  ArgMax t{-INFINITY, 0x7FFFFFFF};
  for (int c0 = 0; c0 < a.s_n_chunks; c0 += 64) {
    const int c = c0 + lane;
    if (c < a.s_n_chunks) {
      const float2 p = *reinterpret_cast<const float2*>(a.spart + (((size_t)b * a.s_n_chunks + c) * 2));
      t = am_merge(t, ArgMax{p.x, __float_as_int(p.y)});
    }
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) t = am_shfl(t, o);
  if (lane == 0) a.next_token[b] = t.i;
}

// Sampled drafts: Gumbel-max over vocabulary chunk c of draft row r,
// argmax_k (z[r, k] / tau + G_k) with noise of stream 2: one Philox block
// at counter (k / 4, r | 2 << 32, seq, step) serves entries k .. k+3, word
// j for entry k + j. The chunk's (value, index) goes to dpart[b][r][c].
__global__ __launch_bounds__(SCAN_THREADS) LATENCY_BOUND void draft_sample_kernel(VerifyArgs a) {
  const int c = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
  const int seq = a.seq_ids[b];
  const float* zr = a.qlogits + ((size_t)b * (a.N - 1) + r) * a.V;
  const int k0 = c * a.s_chunk, k1 = min(a.V, k0 + a.s_chunk);  // multiples of 4
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  ArgMax t{-INFINITY, 0x7FFFFFFF};
  for (int k = k0 + 4 * (int)threadIdx.x; k < k1; k += 4 * SCAN_THREADS) {
    unsigned long long w[4] = {(unsigned long long)(unsigned)(k >> 2),
                               (unsigned long long)(unsigned)r | (2ull << 32),
                               (unsigned long long)(unsigned)seq, a.step};
    philox4x64_10(w, a.seed, 0ull);
    const f32x4 z = *reinterpret_cast<const f32x4*>(zr + k);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float u = ((float)(w[e] >> 41) + 0.5f) * 1.1920928955078125e-07f;
      t = am_merge(t, ArgMax{z[e] * a.inv_tau - logf(-logf(u)), k + e});
    }
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) t = am_shfl(t, o);
  __shared__ ArgMax red[SCAN_THREADS / 64];
  if (lane == 0) red[wave] = t;
  __syncthreads();
  if (threadIdx.x != 0) return;
  ArgMax u = red[0];
  for (int w = 1; w < SCAN_THREADS / 64; ++w) u = am_merge(u, red[w]);
  *reinterpret_cast<float2*>(a.dpart + ((((size_t)b * (a.N - 1) + r) * a.s_n_chunks + c) * 2)) =
      make_float2(u.v, __int_as_float(u.i));
}

// Draft token of (row r, sequence b): merge of the row's chunks in chunk order.
__global__ __launch_bounds__(64) void draft_pick_kernel(VerifyArgs a) {
  const int r = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const float2* src = reinterpret_cast<const float2*>(a.dpart) + ((size_t)b * (a.N - 1) + r) * a.s_n_chunks;
  ArgMax t{-INFINITY, 0x7FFFFFFF};
  for (int c = lane; c < a.s_n_chunks; c += 64) t = am_merge(t, ArgMax{src[c].x, __float_as_int(src[c].y)});
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) t = am_shfl(t, o);
  if (lane == 0) a.draft_out[(size_t)b * (a.N - 1) + r] = t.i;
}

extern "C" hipError_t dflash_launch_draft_sample(const VerifyArgs* a, hipStream_t st) {
  hipError_t e = launch_kernel(draft_sample_kernel, dim3(a->s_n_chunks, a->N - 1, a->B), dim3(SCAN_THREADS), 0, st, *a);
  if (e != hipSuccess) return e;
  return launch_kernel(draft_pick_kernel, dim3(a->N - 1, a->B), dim3(64), 0, st, *a);
}

extern "C" hipError_t dflash_launch_verify(const VerifyArgs* a, hipStream_t st) {
  const dim3 grid(a->n_chunks, a->N, a->B), block(VERIFY_THREADS);
  hipError_t e;
  if (a->dtype == DFLASH_DTYPE_F32) e = launch_kernel(verify_rows_kernel<DFLASH_DTYPE_F32>, grid, block, 0, st, *a);
  else e = launch_kernel(verify_rows_kernel<DFLASH_DTYPE_BF16>, grid, block, 0, st, *a);
  if (e != hipSuccess) return e;
  if (a->sampled) {  // rows pass over the drafter's logits / tau: (max, sum) per row chunk into qpart
    VerifyArgs q = *a;
    q.logits = a->qlogits;
    q.dtype = DFLASH_DTYPE_F32;
    q.N = a->N - 1;
    q.part = const_cast<float*>(a->qpart);
    q.inv_scale = a->inv_tau;
    e = launch_kernel(verify_rows_kernel<DFLASH_DTYPE_F32>, dim3(a->n_chunks, a->N - 1, a->B), block, 0, st, q);
    if (e != hipSuccess) return e;
  }
  if (!a->temp1) return launch_kernel(verify_greedy_kernel, dim3(a->B), dim3(SCAN_THREADS), 0, st, *a);
  e = launch_kernel(verify_sample_kernel, dim3(a->s_n_chunks, a->B), dim3(SCAN_THREADS), 0, st, *a);
  if (e != hipSuccess) return e;
  return launch_kernel(verify_pick_kernel, dim3(a->B), dim3(64), 0, st, *a);
}

// ------------------------------------------------------- static scratch
// The partials of dflash_verify_noalloc, the verification for callers that
// cannot allocate device memory: a file-scope array, one copy per GPU, held
// until the process ends. On the host the array's name is only a stand-in
// for the device variable, never a device address: the set-up below looks
// up each device's address once (hipGetSymbolAddress) and the launches
// take that pointer.
static __device__ __align__(256) float scratch[DFLASH_VERIFY_SCRATCH_BYTES / sizeof(float)];

namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch[kScratchDevices];  // address of `scratch` on each device; null until set up
}  // namespace

// Called by dflash_create with `device` current; later calls on the same
// device return at once.
extern "C" hipError_t dflash_verify_scratch_setup(int device) {
  if (device < 0 || device >= kScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[device]) return hipSuccess;
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  g_scratch[device] = static_cast<float*>(p);
  return hipSuccess;
}

// Device address of the scratch array on `device`, or null if not set up.
extern "C" float* dflash_verify_scratch(int device) {
  if (device < 0 || device >= kScratchDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  return g_scratch[device];
}
