// Shared device helpers for the gfx950 kernels: bf16 storage, MFMA operand
// types, wave-level reductions and the kernel argument structs.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define DEV __device__ __forceinline__

// Host: launch kernel k with the given arguments, timed into
// dflash_launch_events when the kernel timer is on.
template <typename... Args>
inline hipError_t launch_args(void (*k)(Args...), dim3 g, dim3 b, uint32_t shmem, hipStream_t st, Args... args) {
  void* ptrs[] = {(void*)&args...};
  const LaunchEvents ev = dflash_launch_events;
  if (ev.start) return hipExtLaunchKernel((const void*)k, g, b, ptrs, shmem, st, ev.start, ev.stop, 0);
  return hipLaunchKernel((const void*)k, g, b, ptrs, shmem, st);
}

template <typename... Args, typename... P>
inline hipError_t launch_kernel(void (*k)(Args...), dim3 g, dim3 b, uint32_t shmem, hipStream_t st, P... p) {
  return launch_args<Args...>(k, g, b, shmem, st, static_cast<Args>(p)...);
}

// Kernels with small grids whose time is memory latency: let the scheduler
// use up to 128 VGPRs (<= 4 waves per SIMD) so that independent loads are all
// issued before the first wait, instead of serialising them to reach an
// occupancy these grids never use.
#define LATENCY_BOUND __attribute__((amdgpu_waves_per_eu(1, 4)))

// bf16 bits -> fp32 (exact).
DEV float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16 bits, round to nearest even (the hardware conversion).
DEV uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f)); }

// fp32 -> bf16 pair (hi, lo) with hi + lo = x to about 2^-17 relative.
DEV void split_bf16(float x, uint16_t& hi, uint16_t& lo) {
  hi = f2bf(x);
  lo = f2bf(x - bf2f(hi));
}

// Two values at a time with the packed hardware conversion.
DEV void split2(f32x2 x, uint32_t& hi, uint32_t& lo) {
  const bf16x2 h = __builtin_convertvector(x, bf16x2);
  const bf16x2 l = __builtin_convertvector(x - __builtin_convertvector(h, f32x2), bf16x2);
  hi = __builtin_bit_cast(uint32_t, h);
  lo = __builtin_bit_cast(uint32_t, l);
}

DEV void split4(const f32x4& x, u16x4& hi, u16x4& lo) {
  uint32_t h0, l0, h1, l1;
  split2(f32x2{x[0], x[1]}, h0, l0);
  split2(f32x2{x[2], x[3]}, h1, l1);
  hi = __builtin_bit_cast(u16x4, (uint32_t __attribute__((ext_vector_type(2)))){h0, h1});
  lo = __builtin_bit_cast(u16x4, (uint32_t __attribute__((ext_vector_type(2)))){l0, l1});
}

// Direct-to-LDS load (global_load_lds, 16 bytes per lane): lane l's 16
// bytes from src land at byte 16 l of the wave's LDS block dst (dst must be
// wave-uniform). Counted by vmcnt like any load.
typedef __attribute__((address_space(3))) void* lds_ptr;
DEV void dma16(const uint16_t* src, u32x4* dst) { __builtin_amdgcn_global_load_lds(src, (lds_ptr)dst, 16, 0, 0); }

// 16 bytes = 8 bf16 from global memory.
DEV bf16x8 ld8(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

DEV bf16x8 zero8() {
  u32x4 z = {0u, 0u, 0u, 0u};
  return __builtin_bit_cast(bf16x8, z);
}

// D(16x16, fp32) += A(16x32) * B(32x16), bf16 operands.
// Lane l: A row l%16, B column l%16, each holding k = 8*(l/16) .. +7;
// D rows 4*(l/16) + i (i < 4), column l%16.
DEV f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Sum over a whole workgroup (blockDim.x a multiple of 64, <= 1024).
// Every thread gets the total; the order of summation is fixed.
DEV float block_sum(float v, float* lds /* >= 16 floats */) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) lds[wave] = v;
  __syncthreads();
  float t = 0.f;
  for (int w = 0; w < nw; ++w) t += lds[w];
  return t;
}

DEV void set_error(int32_t* err, int bits) { atomicOr(err, bits); }

// Largest k split a streaming GEMM uses; reducers unroll over it (one batch
// of at most 8 loads per thread: bigger batches cost time on gfx950).
#define KS_MAX 8

// Sum of the ks split partials part[k*stride + off], k = 0..ks-1, in k
// order. All loads are issued before the first add, so the reduction costs
// one memory latency instead of ks.
DEV float split_sum1(const float* part, int ks, size_t stride, size_t off) {
  float v[KS_MAX];
#pragma unroll
  for (int k = 0; k < KS_MAX; ++k) v[k] = k < ks ? part[k * stride + off] : 0.f;
  float s = v[0];
#pragma unroll
  for (int k = 1; k < KS_MAX; ++k)
    if (k < ks) s += v[k];
  return s;
}

DEV f32x4 split_sum4(const float* part, int ks, size_t stride, size_t off) {
  f32x4 v[KS_MAX];
#pragma unroll
  for (int k = 0; k < KS_MAX; ++k)
    v[k] = k < ks ? *reinterpret_cast<const f32x4*>(part + k * stride + off) : f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 s = v[0];
#pragma unroll
  for (int k = 1; k < KS_MAX; ++k)
    if (k < ks) s += v[k];
  return s;
}


DEV Top2 top2_empty() { return {-INFINITY, 0x7FFFFFFF, -INFINITY, 0.f}; }

DEV bool better(float va, int ia, float vb, int ib) { return va > vb || (va == vb && ia < ib); }

// exp of the loser's maximum against the winner's, 0 for an empty loser
DEV float top2_rescale(float s, float v, float v1) { return s > 0.f ? s * __expf(v - v1) : 0.f; }

DEV Top2 top2_merge(Top2 a, Top2 b) {
  Top2 r;
  if (better(a.v1, a.i1, b.v1, b.i1)) {
    r.v1 = a.v1; r.i1 = a.i1; r.v2 = fmaxf(a.v2, b.v1);
    r.s = a.s + top2_rescale(b.s, b.v1, a.v1);
  } else {
    r.v1 = b.v1; r.i1 = b.i1; r.v2 = fmaxf(b.v2, a.v1);
    r.s = b.s + top2_rescale(a.s, a.v1, b.v1);
  }
  return r;
}

DEV Top2 top2_push(Top2 a, float v, int i) { return top2_merge(a, Top2{v, i, -INFINITY, 1.f}); }

DEV Top2 top2_shfl_xor(Top2 a, int o) {
  Top2 b;
  b.v1 = __shfl_xor(a.v1, o, 64);
  b.i1 = __shfl_xor(a.i1, o, 64);
  b.v2 = __shfl_xor(a.v2, o, 64);
  b.s = __shfl_xor(a.s, o, 64);
  return top2_merge(a, b);
}
