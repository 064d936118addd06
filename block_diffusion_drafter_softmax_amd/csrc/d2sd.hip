// Dual-pass drafting (D2SD): from the first draft's per-position confidence
// (the drafter's largest softmax probability), pick the K positions where a
// rejection is likeliest, build the second pass's input blocks re-anchored
// on each prefix, and assemble the K+1 candidate drafts; after verifying all
// candidates, keep the longest accepted one.
#include "common.h"

// One wave per sequence b; lane j < N-1 holds draft position j+1. A
// position is cut if fewer than K positions rank before it by (confidence,
// position); the cuts, in position order, are candidates 1..K. Block
// b*K + k of the second pass is [anchor, d_1 .. d_{c-1}, mask ...] at
// sequence seq_ids[b].
__global__ __launch_bounds__(64) void d2sd_select_kernel(D2sdArgs a) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int n = a.N - 1;
  const float c = lane < n ? a.conf[b * n + lane] : INFINITY;
  int rank = 0;
  for (int i = 0; i < n; ++i) {
    const float ci = __shfl(c, i, 64);
    rank += (ci < c || (ci == c && i < lane)) ? 1 : 0;
  }
  const bool cut = lane < n && rank < a.K;
  const unsigned long long mask = __ballot(cut);
  const int k = __popcll(mask & ((1ull << lane) - 1));  // this cut's candidate index - 1
  __shared__ int cuts[64];
  if (cut) {
    const int cp = lane + 1;  // cut position, 1-based
    cuts[k] = cp;
    a.cuts[b * a.K + k] = cp;
    if (a.cuts_out) a.cuts_out[b * a.K + k] = cp;
  }
  if (a.conf_out && lane < n) a.conf_out[b * n + lane] = c;
  __syncthreads();
  // second-pass blocks: thread (k, n) for the K blocks of this sequence
  for (int idx = lane; idx < a.K * a.N; idx += 64) {
    const int kk = idx / a.N, pos = idx % a.N;
    const int cp = cuts[kk];
    const int tok = pos == 0 ? a.anchor[b] : pos < cp ? a.draft1[b * n + pos - 1] : a.mask_id;
    a.tokens[(size_t)(b * a.K + kk) * a.N + pos] = tok;
    if (pos == 0) a.seq2[b * a.K + kk] = a.seq_ids[b];
  }
}

// Candidate drafts [B][K+1][N-1]: candidate 0 is the first draft; candidate
// k keeps d_1 .. d_{c_k - 1} and takes the second pass from position c_k.
__global__ __launch_bounds__(64) void d2sd_assemble_kernel(D2sdArgs a) {
  const int b = blockIdx.x, k = blockIdx.y, j = threadIdx.x;  // j: draft position j+1
  const int n = a.N - 1;
  if (j >= n) return;
  int tok = a.draft1[b * n + j];
  if (k > 0 && j + 1 >= a.cuts[b * a.K + k - 1]) tok = a.draft2[(size_t)(b * a.K + k - 1) * n + j];
  a.drafts[((size_t)b * (a.K + 1) + k) * n + j] = tok;
}

// One wave per sequence: the candidate with the longest accept, the lowest
// index on ties.
__global__ __launch_bounds__(64) void pick_kernel(PickArgs a) {
  const int b = blockIdx.x, lane = threadIdx.x;
  int best = -1, bi = 0;
  for (int c = lane; c < a.C; c += 64) {
    const int acc = a.acc[b * a.C + c];
    if (acc > best) {
      best = acc;
      bi = c;
    }
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int ob = __shfl_xor(best, o, 64), oi = __shfl_xor(bi, o, 64);
    if (ob > best || (ob == best && oi < bi)) {
      best = ob;
      bi = oi;
    }
  }
  if (lane != 0) return;
  a.accept_len[b] = best;
  a.next_token[b] = a.next[b * a.C + bi];
  if (a.commit_len) a.commit_len[b] = best + 1;
  if (a.chosen) a.chosen[b] = bi;
}

extern "C" hipError_t dflash_launch_d2sd_select(const D2sdArgs* a, hipStream_t st) {
  launch_kernel(d2sd_select_kernel, dim3(a->B), dim3(64), 0, st, *a);
  return hipGetLastError();
}

extern "C" hipError_t dflash_launch_d2sd_assemble(const D2sdArgs* a, hipStream_t st) {
  launch_kernel(d2sd_assemble_kernel, dim3(a->B, a->K + 1), dim3(64), 0, st, *a);
  return hipGetLastError();
}

extern "C" hipError_t dflash_launch_pick(const PickArgs* a, hipStream_t st) {
  launch_kernel(pick_kernel, dim3(a->B), dim3(64), 0, st, *a);
  return hipGetLastError();
}
