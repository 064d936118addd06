// Software-pipelined k loop of the weight-streaming kernels.
//
// One wave multiplies NT packed 16-row weight tiles by MT packed 16-row
// split activation tiles (hi and lo bf16 planes) over k steps [s0, s1) of
// 32: per step and lane, one 16-byte non-temporal load per weight tile (a
// whole wave reads 1 KB of contiguous HBM), two 16-byte loads per activation
// tile (L2 resident), and 2*NT*MT MFMA 16x16x32 bf16 (W*hi + W*lo). Loads for
// steps s+U .. s+2U-1 are issued before the MFMAs of steps s .. s+U-1, so a
// wave always has U steps of loads in flight; with one wave per workgroup
// this keeps HBM busy without relying on many co-resident waves.
#pragma once
#include "common.h"

template <int NT, int MT, int U>
struct StreamFrag {
  bf16x8 w[U][NT];
  bf16x8 xh[U][MT];
  bf16x8 xl[U][MT];
};

template <int NT, int MT, int U>
DEV void stream_load(StreamFrag<NT, MT, U>& f, const uint16_t* const* pw, const uint16_t* const* px, size_t lo,
                     int s) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
      f.w[u][t] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(pw[t] + (size_t)(s + u) * 512));
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      f.xh[u][m] = *reinterpret_cast<const bf16x8*>(px[m] + (size_t)(s + u) * 512);
      f.xl[u][m] = *reinterpret_cast<const bf16x8*>(px[m] + lo + (size_t)(s + u) * 512);
    }
  }
}

template <int NT, int MT, int U>
DEV void stream_mfma(const StreamFrag<NT, MT, U>& f, f32x4 (&acc)[NT][MT]) {
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        acc[t][m] = mfma16(f.w[u][t], f.xh[u][m], acc[t][m]);
        acc[t][m] = mfma16(f.w[u][t], f.xl[u][m], acc[t][m]);
      }
}

// pw[t]: tile t's packed block for k step 0, offset by lane*8 (step stride 512);
// px[m]: the same for the hi plane of activation tile m; lo: elements from a
// hi-plane address to the matching lo-plane address.
template <int NT, int MT, int U>
DEV void stream_ksteps(const uint16_t* const* pw, const uint16_t* const* px, size_t lo, int s0, int s1,
                       f32x4 (&acc)[NT][MT]) {
  const int s_end = s0 + (s1 - s0) / U * U;
  int s = s0;
  StreamFrag<NT, MT, U> fa, fb;
  if (s < s_end) stream_load(fa, pw, px, lo, s);
  while (s < s_end) {
    if (s + U < s_end) stream_load(fb, pw, px, lo, s + U);
    stream_mfma(fa, acc);
    s += U;
    if (s >= s_end) break;
    if (s + U < s_end) stream_load(fa, pw, px, lo, s + U);
    stream_mfma(fb, acc);
    s += U;
  }
  for (; s < s1; ++s) {
    StreamFrag<NT, MT, 1> f1;
    stream_load(f1, pw, px, lo, s);
    stream_mfma(f1, acc);
  }
}
