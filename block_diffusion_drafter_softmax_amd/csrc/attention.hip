// Block attention: the N block queries of every head attend, with no mask,
// to all L context keys of their sequence plus the N block keys (the draft
// is not autoregressive; the fused target context enters each draft layer
// as keys/values only).
//
// Work item = (key set, kv head, sequence). Item 0 is the block's own N
// keys (laid out like one cache page; slots >= N are invalid): a short
// item, two key tiles of compute. Item i >= 1 is the context chunk of CH =
// 128 keys from 128 * (i - 1) (page p of the sequence holds keys 16p ..
// 16p+15), so a context of 128 * n keys gives 1 + n items per kv head; the
// one workgroup past a CU each (at 4096 keys) is a light block item. A
// workgroup holds all R = (n_q/n_kv)*N query rows of one kv head (GQA: a
// K/V tile is read from HBM once for the whole query group), one computing
// wave per 16 rows, and at least 8 waves for staging. The chunk's page
// indices and the queries are loaded together; then every K and V byte of
// the chunk is requested at once (one batch of <= 8 16-byte loads per
// thread) and staged in LDS, V values of invalid slots written as zeros.
// A computing wave then takes the whole chunk in one pass: S^T = K Q^T with
// MFMA (keys as rows, the lane's query as column; hi and lo products in
// separate accumulators where registers allow), one softmax in the log2
// domain (the scale
// log2(e)/sqrt(d_h) is applied to Q when it is written), and O^T += V^T P^T:
// V is staged per page as [half][d_h][8 slots], so an A-operand fragment
// is one 16-byte read, and P^T comes straight from the S^T
// accumulators (both MFMAs use the same permutation of the keys, chosen so
// that every LDS read is a conflict-free 16-byte read). Q and P
// are fp32 values entering the MFMAs as hi/lo bf16 pairs (two MFMAs each);
// K and V are bf16 storage. Unnormalised O, the chunk's max and sum go to a
// partial buffer, and attn_merge_kernel combines the chunks.
//
// Large batches and long contexts have far more chunks than the chip holds
// at once (about 512 workgroups, two per CU). There a work item is cpi > 1
// consecutive chunks, taken one after the other by the
// same workgroup (stage, compute, stage, ...) with the running max, sum and
// O rescaled per half chunk as in any online softmax, and one partial per
// item goes to the merge: cpi times fewer partial bytes. With 8-wave
// workgroups and cpi = 2, 4 or 8 every context item streams its chunks
// through a direct-to-LDS ring of two stages (ring_item), and at d_h 128
// with two key groups one persistent workgroup per CU slot takes item after
// item from a per-XCD list, longest first (attn_persist_kernel).
//
// Blocks that share a sequence (the dual-pass drafter's candidates: grp
// consecutive blocks) share its context: a workgroup takes `cand` of them
// for a context item, with cand * R / 16 computing waves, so each context
// chunk is read from HBM once for all of them. Item 0, the block keys,
// differs per candidate: it gets one workgroup per candidate.
#include <algorithm>

#include "common.h"
#include "dflash.h"

namespace {
DEV int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

constexpr int CH = 128;  // context keys per chunk (a context item takes cpi chunks)
constexpr int PAGES = CH / 16;
constexpr int MIN_WAVES = 8;  // staging waves per workgroup
constexpr int CPI_MAX = 8;    // chunks per work item, at most

// LDS row of chunk key k. Within each 32-key group (two pages), key 8a + b
// goes to row 4a + b of the group's first 16-row tile for b < 4 and of its
// second tile for b >= 4. A lane then holds S for keys 8g .. 8g+3 (first
// tile) and 8g+4 .. 8g+7 (second tile): its 8 P values of a k-step are 8
// consecutive slots of one page, so the matching V fragment is one 16-byte
// LDS read (V is kept per page as [half][dim][8 slots]).
DEV int krow(int k) {
  const int b = k & 7;
  return (k & ~31) + (b & 4) * 4 + ((k >> 3) & 3) * 4 + (b & 3);
}
// Chunk key held by lane group g, accumulator i, of key tile j.
DEV int tile_key(int j, int g, int i) { return (j >> 1) * 32 + 8 * g + (j & 1) * 4 + i; }
// Chunk key held in LDS row `row` (the inverse of krow).
DEV int kinv(int row) {
  const int r = row & 31;
  return (row & ~31) + ((r >> 2) & 3) * 8 + (r >> 4) * 4 + (r & 3);
}
// DMA layout: key rows of D elements with no padding; the 16-byte units of
// row r are XOR-permuted by kswz(r), so that the 16 lanes that read one unit
// of 16 consecutive rows hit 16 distinct bank groups.
template <int D>
DEV int kswz(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
}  // namespace

// Reductions over the four lane groups g that hold one query's keys (lanes
// l, l ^ 16, l ^ 32, l ^ 48): the gfx950 row swaps, no lane-index
// arithmetic; every lane ends with the same value, summed in the same
// order (groups 0 + 1, then 2 + 3, then the two pairs).
DEV float group_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
DEV float group_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Growth of a row's max (log2 units) that the running max absorbs without
// a rescale: numerators exp2(S - max) stay below 2^8.
constexpr float MAX_SLACK = 8.0f;

// Masking of invalid keys (masked: the block item, or the context's last
// chunk) and the online-softmax update of one half of S held by a wave: S
// becomes its numerators exp2(S - max), the running max and sum advance,
// and (MULTI) the O accumulators are rescaled. shifted: S arrives as S -
// max (the MFMAs started from -max; every row of the wave has a finite
// max), and the max moves only when some row's S exceeds it by more than
// MAX_SLACK -- the (max, sum, O) triple stays exact for any max it keeps,
// and most halves then skip the rescale.
template <int D, int NTH, bool MULTI>
DEV void softmax_update(f32x4 (&s)[NTH], const int* ccnt, bool masked, bool shifted, int hv, int g, float& mx,
                        float& l, f32x4 (&acc)[D / 16]) {
  constexpr int DT = D / 16;
  if (masked) {
#pragma unroll
    for (int j = 0; j < NTH; ++j) {
      const int k0 = tile_key(hv * NTH + j, g, 0);  // 4 keys k0 .. k0+3 of one page
      const int nj = ccnt[k0 >> 4] - (k0 & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) s[j][i] = i < nj ? s[j][i] : -INFINITY;
    }
  }
  float cm = -INFINITY;
#pragma unroll
  for (int j = 0; j < NTH; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) cm = fmaxf(cm, s[j][i]);
  cm = group_max(cm);  // -inf for a half with no valid key
  // a new running max: the first update (mx -inf: sub keeps the exponents
  // defined while a wave has met no valid key -- the second key group can
  // meet none), or a row's S beyond the slack (wave-uniform choice)
  float sub = 0.f, scale = 1.f;
  const bool move = !shifted || __ballot(cm > MAX_SLACK);
  if (move) {
    if (!shifted) {
      const float mn = fmaxf(mx, cm);
      sub = mn == -INFINITY ? 0.f : mn;
      scale = exp2f(mx - sub);  // 0 at the first update
      mx = mn;
    } else {
      sub = fmaxf(cm, 0.f);
      scale = __builtin_amdgcn_exp2f(-sub);
      mx += sub;
    }
#pragma unroll
    for (int j = 0; j < NTH; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) s[j][i] -= sub;
    l *= scale;
    if (MULTI) {
#pragma unroll
      for (int t = 0; t < DT; ++t) acc[t] *= scale;
    }
  }
  float cs = 0.f;
#pragma unroll
  for (int j = 0; j < NTH; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[j][i] = __builtin_amdgcn_exp2f(s[j][i]);  // <= 2^MAX_SLACK; results under 2^-126 flush to 0
      cs += s[j][i];
    }
  l += group_sum(cs);
}

// P of key tiles j, j + 1 (32 keys: the lane's 8 slots of one page) as a
// split hi/lo MFMA operand.
DEV void p_operand(const f32x4& s0, const f32x4& s1, bf16x8& ph, bf16x8& pl) {
  u16x4 h0, l0, h1, l1;
  split4(s0, h0, l0);
  split4(s1, h1, l1);
  ph = __builtin_bit_cast(bf16x8, __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7));
  pl = __builtin_bit_cast(bf16x8, __builtin_shufflevector(l0, l1, 0, 1, 2, 3, 4, 5, 6, 7));
}

// S = K Q^T, the online-softmax update and O^T += V^T P^T of one chunk (or
// of the block item) for one computing wave: key row r of the LDS stage at
// kb + r * KP (units swizzled with SWZ), V at vb as [page slot][half][d][8
// slots]; ccnt: valid keys of each page slot of the chunk.
template <int D, int NACC, bool MULTI, int KS, int KP, bool SWZ>
DEV void chunk_compute(const uint16_t* kb, const uint16_t* vb, const int* ccnt, bool blk_item, int nv, int kh,
                       int r16, int g, const bf16x8 (&qh)[D / 32], const bf16x8 (&ql)[D / 32],
                       f32x4 (&acc)[D / 16], float& mx, float& l) {
  constexpr int KD = D / 32, DT = D / 16, NT = CH / 16;
  // Key tile j = LDS rows 16j .. 16j+15; the lane holds S for keys
  // tile_key(j, g, 0..3) of its query. Multi-chunk items take a chunk as
  // HV = 2 halves of 64 keys, each with its own online-softmax update, so
  // that the O accumulators kept across chunks fit the registers; with
  // KS = 2 each key group takes its own half.
  constexpr int HV = MULTI || KS == 2 ? 2 : 1, NTH = NT / HV;
  // key tiles with work: the block item's two (its keys, then a masked
  // page), all of a context chunk's (wave-uniform)
  const int nt_act = blk_item ? 2 : NTH;
#pragma unroll
  for (int hh = 0; hh < (KS == 2 ? 1 : HV); ++hh) {
    const int hv = KS == 2 ? kh : hh;  // the half: a key group's own one with KS = 2
    if (blk_item && hv > 0) break;
    f32x4 s[NTH];
    // once every row of the wave has a finite running max (multi-chunk
    // items after their first half), S - max straight from the MFMAs
    const bool shifted = MULTI && !__ballot(mx == -INFINITY);
    {
      const float c0 = shifted ? -mx : 0.f;
      f32x4 sa[NACC][NTH];
#pragma unroll
      for (int h = 0; h < NACC; ++h)
#pragma unroll
        for (int j = 0; j < NTH; ++j) sa[h][j] = h == 0 ? f32x4{c0, c0, c0, c0} : f32x4{0.f, 0.f, 0.f, 0.f};
      // the ring's d_h-128 kernel (registers to spare): every K fragment of
      // the half requested at once, so LDS latency is paid once, not per kd
      constexpr bool PF = SWZ && D == 128;
      constexpr int KB = PF ? KD : 1;  // kd steps whose fragments are read together
#pragma unroll
      for (int kd0 = 0; kd0 < KD; kd0 += KB) {
        bf16x8 kf[KB][NTH];
#pragma unroll
        for (int kk = 0; kk < KB; ++kk)
#pragma unroll
          for (int j = 0; j < NTH; ++j) {
            const int row = 16 * (hv * NTH + j) + r16, u = (kd0 + kk) * 4 + g;
            kf[kk][j] = *reinterpret_cast<const bf16x8*>(kb + row * KP + (SWZ ? (u ^ kswz<D>(row)) : u) * 8);
          }
#pragma unroll
        for (int kk = 0; kk < KB; ++kk)
#pragma unroll
          for (int j = 0; j < NTH; ++j) {
            sa[0][j] = mfma16(kf[kk][j], qh[kd0 + kk], sa[0][j]);
            sa[NACC - 1][j] = mfma16(kf[kk][j], ql[kd0 + kk], sa[NACC - 1][j]);
          }
      }
#pragma unroll
      for (int j = 0; j < NTH; ++j) s[j] = NACC == 2 ? sa[0][j] + sa[NACC - 1][j] : sa[0][j];
    }
    // the ring's d_h-128 kernel: the half's V fragments requested before
    // the softmax (they do not depend on it), in flight while it runs
    constexpr bool VPF_ON = SWZ && D == 128;
    constexpr int VPF = VPF_ON ? NTH / 2 : 1;
    bf16x8 vpre[VPF][VPF_ON ? DT : 1];
    if constexpr (VPF_ON) {
#pragma unroll
      for (int jj = 0; jj < VPF; ++jj) {
        const uint16_t* vp = vb + (hv * NTH + 2 * jj + (g >> 1)) * D * 16 + (g & 1) * D * 8 + r16 * 8;
#pragma unroll
        for (int t = 0; t < DT; ++t) vpre[jj][t] = *reinterpret_cast<const bf16x8*>(vp + t * 128);
      }
    }
    softmax_update<D, NTH, MULTI>(s, ccnt, blk_item || nv < CH, shifted, hv, g, mx, l, acc);

#pragma unroll
    for (int j = 0; j < NTH; j += 2) {  // k-step: key tiles j and j+1 (32 keys, 2 pages)
      if (j < nt_act) {
        // lane's keys: slots 8*(g&1) .. +7 of the step's page g>>1
        const uint16_t* vp = vb + (hv * NTH + j + (g >> 1)) * D * 16 + (g & 1) * D * 8 + r16 * 8;
        bf16x8 ph, pl;
        p_operand(s[j], s[j + 1], ph, pl);
        if constexpr (VPF_ON) {
#pragma unroll
          for (int t = 0; t < DT; ++t) {
            acc[t] = mfma16(vpre[j / 2][t], ph, acc[t]);
            acc[t] = mfma16(vpre[j / 2][t], pl, acc[t]);
          }
        } else {
          constexpr int TB = MULTI ? DT / 2 : DT;  // V fragments read at once
#pragma unroll
          for (int t0 = 0; t0 < DT; t0 += TB) {
            bf16x8 vf[TB];
#pragma unroll
            for (int t = 0; t < TB; ++t) vf[t] = *reinterpret_cast<const bf16x8*>(vp + (t0 + t) * 128);
#pragma unroll
            for (int t = 0; t < TB; ++t) {
              acc[t0 + t] = mfma16(vf[t], ph, acc[t0 + t]);
              acc[t0 + t] = mfma16(vf[t], pl, acc[t0 + t]);
            }
          }
        }
      }
    }
  }
}

// Stage K (rows krow(key)) and V ([page slot][half][d][8 slots]) of the
// PAGES page slots of a chunk in LDS through registers: per page, 2*D*16
// bf16 = UPP = 4*D 16-byte units, K units first. Thread t moves unit t %
// UPP of page slots t / UPP + SP*i, so the unit -- K or V, its source
// offset, its LDS place -- is fixed per thread and a whole wave works on
// one page slot (UPP is a multiple of 64): page lookups and the K/V choice
// are wave-uniform. Slots past the chunk's pages read the block (valid
// memory) and count 0 valid keys, so every V value of an invalid key is
// stored as 0 and the MFMAs never meet stale values; K of invalid keys is
// masked in S. The block item stages its one page (one load per thread)
// and the masked page's V as zeros.
template <int D, bool MULTI, int KP, bool SWZ>
DEV void stage_regs(uint16_t* kst, uint16_t* vst, const long long* cpo, const int* ccnt, bool blk_item, bool isk,
                    int tid, int nthreads, const uint16_t* blk_k, const uint16_t* blk_v, const uint16_t* pages,
                    int n_kv) {
  constexpr int UPP = 4 * D;
  constexpr int UB = MULTI ? 4 : 8;  // loads per thread and batch (registers: O is live across chunks)
  const int SP = nthreads / UPP;     // page slots per pass (nthreads >= 512 >= UPP)
  const int passes = (PAGES + SP - 1) / SP;
  const int w = tid % UPP;
  const int p0 = __builtin_amdgcn_readfirstlane(tid / UPP);
  const int e = w - 2 * D;  // V unit: dim e/2, slots 8*(e&1) .. +7
  const int kslot = w / (D / 8), kunit = w % (D / 8);
  const int src_off = isk ? kslot * D + kunit * 8 : e * 8;
  const int v_off = (e & 1) * D * 8 + (e >> 1) * 8;
  auto k_off = [&](int pi) {  // this thread's K unit of page slot pi
    const int row = krow(pi * 16 + kslot);
    return row * KP + (SWZ ? (kunit ^ kswz<D>(row)) : kunit) * 8;
  };
  const uint16_t* blk = (isk ? blk_k : blk_v) + src_off;
  const uint16_t* pgs = pages + (isk ? 0 : (size_t)n_kv * 16 * D) + src_off;
  if (blk_item) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (p0 == 0) v = *reinterpret_cast<const u32x4*>(blk);
    for (int pi = p0; pi < 2; pi += SP) {
      if (isk) {
        if (pi == 0) *reinterpret_cast<u32x4*>(&kst[k_off(0)]) = v;
      } else {
        const int valid = ccnt[pi] - (e & 1) * 8;
        u32x4 m;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          m[q] = (2 * q < valid ? 0xFFFFu : 0u) | (2 * q + 1 < valid ? 0xFFFF0000u : 0u);
        *reinterpret_cast<u32x4*>(&vst[pi * D * 16 + v_off]) = v & m;
      }
    }
  } else if (p0 < SP) {
    for (int i0 = 0; i0 < passes; i0 += UB) {
      u32x4 buf[UB];
#pragma unroll
      for (int u = 0; u < UB; ++u) {  // clamped slots: duplicate loads, not stored
        const long long o = cpo[min((i0 + u) * SP + p0, PAGES - 1)];
        buf[u] = *reinterpret_cast<const u32x4*>(o < 0 ? blk : pgs + o);
      }
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        const int pi = (i0 + u) * SP + p0;
        if (i0 + u >= passes || pi >= PAGES) break;
        if (isk) {
          *reinterpret_cast<u32x4*>(&kst[k_off(pi)]) = buf[u];
        } else {
          const int valid = ccnt[pi] - (e & 1) * 8;
          u32x4 m;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            m[q] = (2 * q < valid ? 0xFFFFu : 0u) | (2 * q + 1 < valid ? 0xFFFF0000u : 0u);
          *reinterpret_cast<u32x4*>(&vst[pi * D * 16 + v_off]) = buf[u] & m;
        }
      }
    }
  }
}

// Direct-to-LDS staging of one chunk (DMA layout) by a workgroup of 8 waves
// into a stage's K array (CH rows of D) and V array ([page slot][half][d][8
// slots]): each wave instruction moves one 1 KB block, lane l to byte 16l
// of it, from wherever that unit lives in the cache pages. The first half
// of a thread's instructions fill K, the second half V; a block is all of
// one page slot (K: 4 rows of d_h 128 or 8 rows of 64 in one 8-key run of
// krow's order; V: 64 dims of one half page), so the page lookup is one
// broadcast LDS read per instruction. Slots past the chunk's pages read the
// block (valid memory); their V is zeroed once landed.
template <int D>
DEV void stage_dma(uint16_t* kst, uint16_t* vst, const long long* cpo, int wave, int lane, const uint16_t* blk_k,
                   const uint16_t* blk_v, const uint16_t* pages, int n_kv) {
  constexpr int KU = CH * D / 8, LPC = 2 * KU / 64 / 8;  // K units (= V units), loads per thread
  static_assert(KU == 64 * 8 * (LPC / 2), "K blocks are the first half of every wave's loads");
  const uint16_t* pages_v = pages + (size_t)n_kv * 16 * D;
#pragma unroll
  for (int i = 0; i < LPC; ++i) {
    const int blk = (i % (LPC / 2)) * 8 + wave;  // block of the K or V array
    const int u = blk * 64 + lane;
    if (i < LPC / 2) {
      const int row = u / (D / 8), key = kinv(row), c = (u % (D / 8)) ^ kswz<D>(row);
      const long long o = cpo[key >> 4];
      dma16((o < 0 ? blk_k : pages + o) + (key & 15) * D + c * 8, reinterpret_cast<u32x4*>(kst) + blk * 64);
    } else {
      const int pi = u / (2 * D), half = (u / D) & 1, dim = u % D;
      const long long o = cpo[pi];
      dma16((o < 0 ? blk_v : pages_v + o) + dim * 16 + half * 8, reinterpret_cast<u32x4*>(vst) + blk * 64);
    }
  }
}

// V values of invalid key slots of a landed DMA stage set to 0 (P is 0
// there, but a stale value could be a NaN or an infinity); 512 threads,
// straight-line code (a loop here would cost the ring its precise waits).
template <int D>
DEV void zero_invalid_v(uint16_t* vb, const int* ccnt, int tid) {
  constexpr int UNITS = PAGES * 2 * D;
  static_assert(UNITS % 512 == 0, "whole passes");
#pragma unroll
  for (int i = 0; i < UNITS / 512; ++i) {
    const int u = i * 512 + tid;
    const int valid = ccnt[u / (2 * D)] - ((u / D) & 1) * 8;
    if (valid < 8) {
      u32x4* p = reinterpret_cast<u32x4*>(vb) + u;
      u32x4 m;
#pragma unroll
      for (int q = 0; q < 4; ++q) m[q] = (2 * q < valid ? 0xFFFFu : 0u) | (2 * q + 1 < valid ? 0xFFFF0000u : 0u);
      *p = *p & m;
    }
  }
}

// One context item of NR chunks through the DMA ring of two LDS stages
// (k0, v0) and (k1, v1): chunks 0 and 1 requested at once; then per chunk,
// wait for its own loads (the next chunk's stay in flight), compute it, and
// request the chunk after next into the stage it leaves. Fully unrolled
// with every load request and wait fixed at compile time: only then does
// the compiler let the reads of one stage run while the other stage's loads
// are in flight (a request or a wait under a run-time condition makes it
// wait for all of them before every read). Waits are explicit vmcnt counts
// and bare barriers (the compiler's __syncthreads would also wait for the
// loads in flight). The caller has written the page slots and synchronised.
template <int D, int NACC, int KS, int NR>
DEV void ring_item(uint16_t* k0, uint16_t* v0, uint16_t* k1, uint16_t* v1, const long long* poff, const int* cnt,
                   int item_nv, bool computing, int wave, int lane, int tid, int kh, int r16, int g,
                   const uint16_t* blk_k, const uint16_t* blk_v, const uint16_t* pages, int n_kv,
                   const bf16x8 (&qh)[D / 32], const bf16x8 (&ql)[D / 32], f32x4 (&acc)[D / 16], float& mx,
                   float& l) {
  constexpr int LPC = 2 * CH * D / 8 / 64 / 8;  // DMA loads per thread and chunk
  stage_dma<D>(k0, v0, poff, wave, lane, blk_k, blk_v, pages, n_kv);
  if constexpr (NR > 1) stage_dma<D>(k1, v1, poff + PAGES, wave, lane, blk_k, blk_v, pages, n_kv);
#pragma unroll
  for (int ci = 0; ci < NR; ++ci) {
    uint16_t* kst = (ci & 1) ? k1 : k0;
    uint16_t* vst = (ci & 1) ? v1 : v0;
    if (ci + 1 < NR) __builtin_amdgcn_s_waitcnt(0x0F70 | LPC);
    else __builtin_amdgcn_s_waitcnt(0x0F70);
    __builtin_amdgcn_s_barrier();  // chunk ci landed for every wave
    const int nv = min(item_nv - ci * CH, CH);
    if (nv < CH) {  // the context's last chunk: V of its invalid slots to 0
      zero_invalid_v<D>(vst, cnt + ci * PAGES, tid);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
    }
    if (computing)
      chunk_compute<D, NACC, true, KS, D, true>(kst, vst, cnt + ci * PAGES, false, nv, kh, r16, g, qh, ql, acc, mx, l);
    __builtin_amdgcn_s_barrier();  // every wave is done with this stage
    if (ci + 2 < NR) stage_dma<D>(kst, vst, poff + (ci + 2) * PAGES, wave, lane, blk_k, blk_v, pages, n_kv);
  }
}

// One work item of one kv head: item 0 = the block's own keys for block b0
// (n_cand = 1), item i >= 1 = context chunks from cpi * CH * (i - 1) for
// blocks b0 .. b0 + n_cand - 1; stages the keys into the workgroup's LDS
// arrays, computes every query row's (max, sum, O) over them and writes
// them as the item's partials. Called by the whole workgroup (every
// thread; the non-computing waves return at the end).
//
// NACC: accumulator sets for the S products (2: hi and lo separately, more
// independent MFMA chains; 1 where 1024-thread workgroups cap the registers).
// MULTI: work items of up to CPI_MAX chunks.
// KS = 2 (multi-chunk items, where the workgroup's staging-only waves
// allow it): twice as many computing waves as query row groups; the second
// group takes the second half of every chunk's keys for the same rows,
// with its own online softmax, and hands (max, sum, O) to its partner
// through LDS at the end.
// DMA (multi-chunk items, 8 waves): a ring of two LDS stages filled by
// direct-to-LDS loads; chunk i + 1 lands while chunk i is computed. Its
// 128 KB at d_h 128 leave one workgroup per CU (two at d_h 64).
// The ring's workgroup is 8 waves and LDS holds it to one per CU at d_h 128,
// so it may take 256 VGPRs there (a spill reload would be counted with the
// loads in flight and wait for them all); two per CU at d_h 64, 128 VGPRs.
template <int D, int NACC, bool MULTI, int KS, int RING>
DEV void attn_item(const AttnArgs& a, int b0, int kvh, int item, int n_cand, uint16_t* lds, uint16_t* ldv0,
                   uint16_t* ldk1, uint16_t* ldv1, long long* poff, int* cnt) {
  constexpr bool DMA = RING > 0;
  constexpr int KP = DMA ? D : D + 8;  // LDS row of one key (bf16 elements): padded, or swizzled
  constexpr int K_ELEMS = CH * KP, V_ELEMS = PAGES * D * 16;
  const bool blk_item = item == 0;
  const int cpi = MULTI ? a.cpi : 1;
  // the thread index as an opaque value: in the persistent kernel's item loop
  // the compiler would otherwise keep every per-lane offset derived from it
  // (staging and fragment addresses) live across the loop, and spill
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int nthreads = blockDim.x;
  // page-table entry of page slot tid (< SLOTS <= nthreads), requested with
  // the plan from the call's per-block copy; clamped, used only if valid
  int raw_slot = 0;
  if (!blk_item && tid < cpi * PAGES)
    raw_slot = a.blk_pages[(size_t)b0 * a.max_pages_per_seq +
                           clampi((item - 1) * cpi * PAGES + tid, 0, a.max_pages_per_seq - 1)];
  const int2 pl = *reinterpret_cast<const int2*>(a.plan + 2 * b0);  // (sequence, context length)
  const int seq = clampi(pl.x, 0, a.max_seqs - 1);
  const int L = clampi(pl.y, 0, a.max_pages_per_seq * 16);
  const int c_begin = (item - 1) * cpi * CH;  // context items: first key
  const int item_nv = blk_item ? a.N : min(L, c_begin + cpi * CH) - c_begin;  // keys in this item
  if (item_nv <= 0) return;
  const int n_chunks = MULTI && !blk_item ? (item_nv + CH - 1) / CH : 1;
  const size_t page_elems = (size_t)2 * a.n_kv * 16 * D;

  // Page slots of the item (the block item's slot 0 is the block; slots
  // past the keys point at the block, valid memory, and hold 0 valid keys).
  const uint16_t* blk_k = a.kblk + ((size_t)b0 * a.n_kv + kvh) * 16 * D;
  const uint16_t* blk_v = a.vblk + ((size_t)b0 * a.n_kv + kvh) * D * 16;
  if (tid < n_chunks * PAGES) {  // n_chunks * PAGES <= SLOTS <= nthreads: one slot per thread
    const int t = tid;
    long long off = -1;
    int n_ok = 0;
    if (blk_item) {
      n_ok = t == 0 ? a.N : 0;
    } else if (16 * t < item_nv) {
      const int raw = raw_slot;
      if (raw < 0 || raw >= a.n_pages) set_error(a.err, DFLASH_DEV_BAD_PAGE);
      off = (long long)clampi(raw, 0, a.n_pages - 1) * page_elems + (long long)kvh * 16 * D;
      n_ok = min(16, item_nv - 16 * t);
    }
    poff[t] = off;
    cnt[t] = n_ok;
  }

  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  // the divisors as opaque scalars: a division's reciprocal would otherwise
  // be computed once before the persistent kernel's item loop and held in
  // vector registers across it
  int n_q = a.n_q, n_kv = a.n_kv, N = a.N;
  asm volatile("" : "+s"(n_q), "+s"(n_kv), "+s"(N));
  const int G = n_q / n_kv, R = G * N, n_wr = R / 16;
  const int n_comp = n_cand * n_wr;  // computing waves per key group
  const bool computing = wave < KS * n_comp;
  const int kh = KS == 2 && wave >= n_comp ? 1 : 0;  // the wave's key group (wave-uniform)
  // staging: thread t moves unit t % (4D) of its page slots, K units first
  const bool isk_wave = __builtin_amdgcn_readfirstlane((int)(tid % (4 * D) < 2 * D));
  const int wc = min(wave - kh * n_comp, n_comp - 1);
  const int cand = wc / n_wr, b = b0 + cand;  // the wave's block
  const int r = (wc % n_wr) * 16 + r16;
  const int hq = kvh * G + r / N, n = r % N;
  constexpr int KD = D / 32, DT = D / 16;

  // queries (softmax scale already applied): in flight with the page reads
  bf16x8 qh[KD], ql[KD];
  {
    const uint16_t* qp = a.q + ((size_t)(b * a.N + n) * a.n_q + hq) * D + 8 * g;
    const size_t q_lo = (size_t)a.n_blocks * a.N * a.n_q * D;
#pragma unroll
    for (int kd = 0; kd < KD; ++kd) {
      qh[kd] = ld8(qp + kd * 32);
      ql[kd] = ld8(qp + q_lo + kd * 32);
    }
  }

  f32x4 acc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mx = -INFINITY, l = 0.f;
  if (!DMA || blk_item) {
    // stage a chunk through registers, then compute it (the block item: its
    // keys and one masked page, two key tiles)
    uint16_t* kst = lds;
    uint16_t* vst = DMA ? ldv0 : lds + K_ELEMS;
    for (int ci = 0; ci < n_chunks; ++ci) {
      const int nv = min(item_nv - ci * CH, CH);  // keys in this chunk
      __syncthreads();  // page slots written; the previous chunk's LDS reads done
      stage_regs<D, MULTI, KP, DMA>(kst, vst, poff + ci * PAGES, cnt + ci * PAGES, blk_item, isk_wave, tid, nthreads,
                                    blk_k, blk_v, a.pages, a.n_kv);
      __syncthreads();
      if (computing)
        chunk_compute<D, NACC, MULTI, KS, KP, DMA>(kst, vst, cnt + ci * PAGES, blk_item, nv, kh, r16, g, qh, ql, acc,
                                                   mx, l);
    }
  } else if constexpr (DMA) {
    // a context item: the ring, unrolled for its chunk count (1 .. RING; a
    // sequence's last item may have fewer chunks than the others)
    __syncthreads();  // page slots written
#define RING_CASE(NR)                                                                                      \
  case NR:                                                                                                 \
    if constexpr (NR <= RING)                                                                              \
      ring_item<D, NACC, KS, NR>(lds, ldv0, ldk1, ldv1, poff, cnt, item_nv, computing, wave, lane, tid, kh, \
                                 r16, g, blk_k, blk_v, a.pages, a.n_kv, qh, ql, acc, mx, l);               \
    break;
    switch (n_chunks) {
      RING_CASE(1)
      RING_CASE(2)
      RING_CASE(3)
      RING_CASE(4)
      RING_CASE(5)
      RING_CASE(6)
      RING_CASE(7)
      RING_CASE(8)
      default: break;
    }
#undef RING_CASE
  }
  if (KS == 2) {  // the second key group's (max, sum, O) to its partner, lane by lane
    // O parts [wave][t][lane] and (max, sum) [wave][lane]; wc < n_comp <= 4
    static_assert(DMA ? (4 * DT * 64 * 16 <= V_ELEMS * 2 && 4 * 64 * 16 <= K_ELEMS * 2)
                      : 4 * (DT + 1) * 64 * 16 <= (K_ELEMS + V_ELEMS) * 2,
                  "hand-off area");
    f32x4* xl = reinterpret_cast<f32x4*>(DMA ? ldv0 : lds) + (size_t)wc * DT * 64 + lane;
    f32x4* xm = reinterpret_cast<f32x4*>(lds) + (DMA ? 0 : 4 * DT * 64) + (size_t)wc * 64 + lane;
    __syncthreads();  // every LDS read of the last chunk done
    if (computing && kh == 1) {
#pragma unroll
      for (int t = 0; t < DT; ++t) xl[t * 64] = acc[t];
      *xm = f32x4{mx, l, 0.f, 0.f};
    }
    __syncthreads();
    if (computing && kh == 0) {
      const f32x4 ml1 = *xm;
      const float M = fmaxf(mx, ml1[0]);  // finite: the first group's first half holds a valid key
      const float w0 = exp2f(mx - M), w1 = exp2f(ml1[0] - M);
      l = l * w0 + ml1[1] * w1;
#pragma unroll
      for (int t = 0; t < DT; ++t) acc[t] = acc[t] * w0 + xl[t * 64] * w1;
      mx = M;
    }
  }
  if (!computing || kh == 1) return;

  const size_t unit = ((size_t)b * a.n_kv + kvh) * a.n_ck + item;
  float* po = a.part_o + (unit * R + r) * D;
#pragma unroll
  for (int t = 0; t < DT; ++t) *reinterpret_cast<f32x4*>(po + t * 16 + 4 * g) = acc[t];
  if (g == 0) {
    a.part_ml[(unit * R + r) * 2 + 0] = mx;
    a.part_ml[(unit * R + r) * 2 + 1] = l;
  }
}

template <int D, int NACC, bool MULTI, int KS, int RING>
__global__ __launch_bounds__(RING ? 512 : 1024)
__attribute__((amdgpu_waves_per_eu(RING && D == 128 ? 1 : 4, RING && D == 128 ? 2 : 4)))
void attn_chunk_kernel(AttnArgs a) {
  constexpr bool DMA = RING > 0;
  static_assert(!DMA || (MULTI && RING >= 2 && RING <= CPI_MAX), "the DMA ring takes multi-chunk items");
  constexpr int KP = DMA ? D : D + 8;  // LDS row of one key (bf16 elements): padded, or swizzled
  constexpr int K_ELEMS = CH * KP, V_ELEMS = PAGES * D * 16;
  constexpr int SLOTS = (MULTI ? CPI_MAX : 1) * PAGES;
  // register staging: one stage, lds = K then V. The ring: stage 0 = (lds,
  // ldv0), stage 1 = (ldk1, ldv1), four arrays, so that every LDS access is
  // a short index off its own array: the compiler then keeps the alias
  // information that lets a read of one stage proceed while the other
  // stage's loads are in flight (with long address chains it drops it and
  // waits for all of them).
  __shared__ __attribute__((aligned(16))) uint16_t lds[DMA ? K_ELEMS : K_ELEMS + V_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t ldv0[DMA ? V_ELEMS : 8];
  __shared__ __attribute__((aligned(16))) uint16_t ldk1[DMA ? K_ELEMS : 8];
  __shared__ __attribute__((aligned(16))) uint16_t ldv1[DMA ? V_ELEMS : 8];
  __shared__ long long poff[SLOTS];  // element offset in `pages` of each page slot's K block (this kv head); -1: block
  __shared__ int cnt[SLOTS];         // valid key slots of each page slot

  // Grid position (x: item slot, y: kv head, z: sequence group * splits + split).
  // With one block per workgroup (cand == 1) the grid is 1-D instead and
  // numbered so that all workgroups of one (sequence group, kv head) -- every
  // item of every candidate block -- are dealt to the same XCD (the hardware
  // deals workgroups to the 8 XCDs round robin), one after the other: the
  // head's query rows then come from memory once, not once per XCD, and a
  // context chunk that several candidate blocks attend to once, then from
  // that XCD's L2.
  int bx = blockIdx.x, by = blockIdx.y, bz = blockIdx.z;
  if (a.xcd_order) {
    // the context items first, tuple by tuple; the (short) block items of
    // every tuple last, where they fill the final round of workgroups
    const int L = blockIdx.x, local = L >> 3, J = (a.xcd_tuples + 7) / 8;
    const int per = (a.xcd_items - 1) * a.grp;  // context item slots of a tuple
    int j, rem;
    if (local < J * per) {
      j = local / per;
      rem = local % per + a.grp;  // slot (item 1 + rem / grp - 1, candidate rem % grp)
    } else {
      j = (local - J * per) / a.grp;
      rem = (local - J * per) % a.grp;
    }
    const int T = j * 8 + (L & 7);  // (sequence group, kv head), head fastest
    if (T >= a.xcd_tuples) return;
    bx = rem / a.grp;
    by = T % a.n_kv;
    bz = T / a.n_kv * a.grp + rem % a.grp;
  }
  const int kvh = by;
  const int splits = (a.grp + a.cand - 1) / a.cand;  // workgroups per group along z
  int c0 = (bz % splits) * a.cand;                   // first candidate of this split
  int n_cand = min(a.cand, a.grp - c0);              // candidates of this split
  // x < cand: item 0 (the block keys) for candidate c0 + x alone;
  // x >= cand: context item x - cand + 1 for all n_cand candidates
  int item = 0;
  if (bx < a.cand) {
    if (bx >= n_cand) return;
    c0 += bx;
    n_cand = 1;
  } else {
    item = bx - a.cand + 1;
  }
  const int b0 = bz / splits * a.grp + c0;   // the workgroup's first block
  attn_item<D, NACC, MULTI, KS, RING>(a, b0, kvh, item, n_cand, lds, ldv0, ldk1, ldv1, poff, cnt);
}

// The work list of one XCD for the persistent ring kernel: its tuples are
// (sequence group, kv head) T = 8j + x, j < J <= 64. Longest first: every
// full item (cpi chunks) of every tuple, tuple by tuple; then each tuple's
// last, partial item, the most chunks first; then the block items. A
// position is pos = u * grp + candidate.
struct AttnList {
  int F, Tt, J;
};

// The job at list position pos: (first block, kv head, item), or b0 = -1
// past the end. s_pref[j]: full items of the tuples before j; s_f[j]: full
// items of tuple j; s_tail[k]: tuple of the k-th partial item.
DEV int3 attn_job(const AttnArgs& a, const AttnList& w, int pos, int x, const int* s_pref, const int* s_f,
                  const int* s_tail) {
  int grp = a.grp, n_kv = a.n_kv;  // opaque: no reciprocal held across the item loop
  asm volatile("" : "+s"(grp), "+s"(n_kv));
  const int u = pos / grp, gi = pos % grp;
  int j, item;
  if (pos < 0) {
    return int3{-1, 0, 0};
  } else if (u < w.F) {  // the last tuple whose full items start at or before u
    int lo = 0, hi = w.J - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_pref[mid] <= u) lo = mid;
      else hi = mid - 1;
    }
    j = lo;
    item = 1 + u - s_pref[j];
  } else if (u < w.F + w.Tt) {
    j = s_tail[u - w.F];
    item = 1 + s_f[j];
  } else if (u < w.F + w.Tt + w.J) {
    j = u - w.F - w.Tt;
    item = 0;
  } else {
    return int3{-1, 0, 0};
  }
  const int T = 8 * j + x;
  return int3{T / n_kv * grp + gi, T % n_kv, item};
}

// The DMA ring as a persistent kernel (one block per work item, cand == 1):
// gridDim.x = 8 * P workgroups, all resident at once; workgroup i serves
// XCD x = i % 8 (the hardware deals workgroups to the XCDs round robin)
// and takes the items of x's work list: position i / 8 first, then the
// position a per-XCD counter hands out (P + its count), until the list
// ends. Versus one workgroup per item slot: no workgroups for the slots
// that a short sequence leaves empty, no workgroup launch per item, and the
// longest items first so that the last ones to finish are short. The
// counters (attn_ctr[8]) are zeroed by the kernel before the attention in
// the stream (the Q/K/V finisher). Which workgroup computes an item does
// not change its partials: the results are the same in any order.
template <int D, int NACC, int KS, int RING>
__global__ __launch_bounds__(512)
__attribute__((amdgpu_waves_per_eu(D == 128 ? 1 : 4, D == 128 ? 2 : 4)))
void attn_persist_kernel(AttnArgs a) {
  static_assert(RING >= 2 && RING <= CPI_MAX, "the DMA ring takes multi-chunk items");
  constexpr int K_ELEMS = CH * D, V_ELEMS = PAGES * D * 16, SLOTS = CPI_MAX * PAGES;
  __shared__ __attribute__((aligned(16))) uint16_t lds[K_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t ldv0[V_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t ldk1[K_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t ldv1[V_ELEMS];
  __shared__ long long poff[SLOTS];
  __shared__ int cnt[SLOTS];
  __shared__ int s_pref[64], s_f[64], s_tail[64];
  __shared__ int s_list[3];
  __shared__ int3 s_job[2];
  const int x = blockIdx.x & 7, P = gridDim.x >> 3, tid = threadIdx.x;
  if (tid < 64) {  // the list, in wave 0: lane t = tuple t of this XCD
    const int t = tid, J = min(64, (a.xcd_tuples - x + 7) / 8);
    const int ik = a.cpi * CH;  // keys per full item
    int f = 0, tc = 0;
    if (t < J) {
      const int T = 8 * t + x, b = T / a.n_kv * a.grp;
      const int L = clampi(a.plan[2 * b + 1], 0, a.max_pages_per_seq * 16);
      f = L / ik;
      tc = (L % ik + CH - 1) / CH;  // chunks of the partial item (0: none)
    }
    int incl = f;  // inclusive prefix over the lanes
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d);
      if (t >= d) incl += v;
    }
    int rank = 0, n_tail = 0;  // partial items: the most chunks first, then by tuple
#pragma unroll
    for (int c = CPI_MAX; c >= 1; --c) {
      const unsigned long long m = __ballot(tc == c);
      if (tc == c) rank = n_tail + __popcll(m & ((1ull << t) - 1));
      n_tail += __popcll(m);
    }
    if (t < J) {
      s_pref[t] = incl - f;
      s_f[t] = f;
    }
    if (tc > 0) s_tail[rank] = t;
    if (t == 63) {
      s_list[0] = incl;
      s_list[1] = n_tail;
      s_list[2] = J;
    }
  }
  __syncthreads();
  const AttnList w{s_list[0], s_list[1], s_list[2]};
  if (tid == 0) s_job[0] = attn_job(a, w, blockIdx.x >> 3, x, s_pref, s_f, s_tail);
  __syncthreads();
  for (int it = 0;; ++it) {
    // the job is the same for every thread: wave-uniform values (scalar
    // registers, uniform branches) for everything derived from it
    const int3 job = s_job[it & 1];
    const int b0 = __builtin_amdgcn_readfirstlane(job.x);
    if (b0 < 0) break;
    const int kvh = __builtin_amdgcn_readfirstlane(job.y), item = __builtin_amdgcn_readfirstlane(job.z);
    int nxt = 0;
    if (tid == 0) nxt = P + atomicAdd(a.attn_ctr + x, 1);
    attn_item<D, NACC, true, KS, RING>(a, b0, kvh, item, 1, lds, ldv0, ldk1, ldv1, poff, cnt);
    if (tid == 0) s_job[(it + 1) & 1] = attn_job(a, w, nxt, x, s_pref, s_f, s_tail);
    __syncthreads();  // the item's LDS reads done; the next job visible
  }
}

// One workgroup per RW query rows of one (sequence, kv head): thread (row,
// cg, dq) merges work items cg, cg + CG, ... of its row for dims 4*dq ..
// 4*dq+3 (all its loads in one batch of <= 8), then the CG partial merges
// of the row are combined in cg order through LDS; the result is
// normalised and written as the O projection's packed split activation.
// Deterministic (fixed order). CG is sized by the host to the items a row
// can have (about eight per thread, one load batch), RW = 256 / (CG *
// D/4): rows with few items (long items at large batches) share a
// workgroup instead of leaving most of its item groups idle.
template <int D, int CG>
__global__ __launch_bounds__(256) LATENCY_BOUND void attn_merge_kernel(AttnArgs a, int B) {
  constexpr int TPR = D / 4, RW = 256 / (TPR * CG);
  static_assert(RW >= 1 && RW * TPR * CG == 256, "whole rows per workgroup");
  __shared__ float sm[RW][CG], sd[RW][CG];
  __shared__ f32x4 sn[RW][CG][TPR];
  const int G = a.n_q / a.n_kv, R = G * a.N, RB = R / RW;  // row groups per (block, kv head)
  // The row groups of one (block, kv head) are dealt to one XCD, the XCD whose
  // attention workgroups wrote the head's partials when the attention grid
  // is XCD-ordered (tuple (block, head) -> XCD tuple % 8 there too, with one
  // block per sequence group): the partials are read from that XCD's L2.
  const int local = blockIdx.x >> 3;
  const int T = (local / RB) * 8 + (blockIdx.x & 7);  // b * n_kv + kvh
  if (T >= B * a.n_kv) return;
  const int rr = threadIdx.x / (TPR * CG);
  const int r = (local % RB) * RW + rr;
  const int kvh = T % a.n_kv;
  const int b = T / a.n_kv;
  const int dq = threadIdx.x % TPR, cg = (threadIdx.x / TPR) % CG;
  const size_t unit0 = ((size_t)b * a.n_kv + kvh) * a.n_ck;
  constexpr int GRP = 8;  // loads in flight per thread (more costs time on gfx950)
  // One chunk per item (small batches): the first batch is requested before
  // the sequence's item count is known (every slot below n_ck is in the
  // buffer; slots past the sequence's items are dropped unread), so the plan
  // load does not delay it. With several chunks per item the sequence's
  // items are far fewer than n_ck: there the batch waits for the count.
  const bool spec = a.cpi == 1;
  float2 ml0[GRP];
  f32x4 ov0[GRP];
  if (spec) {
#pragma unroll
    for (int j = 0; j < GRP; ++j) {
      const size_t row = (unit0 + min(cg + j * CG, a.n_ck - 1)) * R + r;
      ml0[j] = *reinterpret_cast<const float2*>(a.part_ml + row * 2);
      ov0[j] = *reinterpret_cast<const f32x4*>(a.part_o + row * D + dq * 4);
    }
  }
  const int L = clampi(a.plan[2 * b + 1], 0, a.max_pages_per_seq * 16);
  const int nc = min(a.n_ck, 1 + (L + a.cpi * CH - 1) / (a.cpi * CH));  // work items of the block (item 0: its keys)
  float M = -INFINITY, den = 0.f;
  f32x4 num = {0.f, 0.f, 0.f, 0.f};
  if (spec) {
#pragma unroll
    for (int j = 0; j < GRP; ++j) {
      if (cg + j * CG < nc) {
        const float Mn = fmaxf(M, ml0[j].x);
        const float wo = exp2f(M - Mn), wn = exp2f(ml0[j].x - Mn);
        den = den * wo + ml0[j].y * wn;
        num = num * wo + ov0[j] * wn;
        M = Mn;
      }
    }
  }
  for (int c0 = cg + (spec ? GRP * CG : 0); c0 < nc; c0 += GRP * CG) {
    float2 ml[GRP];
    f32x4 ov[GRP];
#pragma unroll
    for (int j = 0; j < GRP; ++j) {
      const size_t row = (unit0 + min(c0 + j * CG, nc - 1)) * R + r;
      ml[j] = *reinterpret_cast<const float2*>(a.part_ml + row * 2);
      ov[j] = *reinterpret_cast<const f32x4*>(a.part_o + row * D + dq * 4);
    }
#pragma unroll
    for (int j = 0; j < GRP; ++j) {
      if (c0 + j * CG >= nc) break;
      const float Mn = fmaxf(M, ml[j].x);
      const float wo = exp2f(M - Mn), wn = exp2f(ml[j].x - Mn);
      den = den * wo + ml[j].y * wn;
      num = num * wo + ov[j] * wn;
      M = Mn;
    }
  }
  if (dq == 0) {
    sm[rr][cg] = M;
    sd[rr][cg] = den;
  }
  sn[rr][cg][dq] = num;
  __syncthreads();
  if (cg != 0) return;
  for (int k = 1; k < CG && k < nc; ++k) {  // group k holds >= 1 chunk
    const float Mn = fmaxf(M, sm[rr][k]);
    const float wo = exp2f(M - Mn), wn = exp2f(sm[rr][k] - Mn);
    den = den * wo + sd[rr][k] * wn;
    num = num * wo + sn[rr][k][dq] * wn;
    M = Mn;
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

template <int D, int NACC, int KS>
void launch_ring(const AttnArgs* a, dim3 grid, dim3 block, hipStream_t st) {
  if (a->cpi == 2) launch_kernel((attn_chunk_kernel<D, NACC, true, KS, 2>), grid, block, 0, st, *a);
  else if (a->cpi == 4) launch_kernel((attn_chunk_kernel<D, NACC, true, KS, 4>), grid, block, 0, st, *a);
  else launch_kernel((attn_chunk_kernel<D, NACC, true, KS, 8>), grid, block, 0, st, *a);
}

// Workgroups of the persistent ring kernel: every CU's resident count, whole
// XCD rounds (0 if the device cannot be queried: the item-slot grid then).
template <int D, int NACC, int KS, int RING>
int persist_wgs() {
  static const int n = [] {
    int dev = 0, cus = 0, occ = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, attn_persist_kernel<D, NACC, KS, RING>, 512, 0) !=
            hipSuccess)
      return 0;
    return cus >= 8 && occ >= 1 ? cus / 8 * 8 * occ : 0;
  }();
  return n;
}

template <int D, int NACC, int KS>
bool launch_persist(const AttnArgs* a, hipStream_t st) {
  int n = 0;
  if (a->cpi == 2) n = persist_wgs<D, NACC, KS, 2>();
  else if (a->cpi == 4) n = persist_wgs<D, NACC, KS, 4>();
  else n = persist_wgs<D, NACC, KS, 8>();
  if (n <= 0) return false;
  const dim3 grid(n), block(512);
  if (a->cpi == 2) launch_kernel((attn_persist_kernel<D, NACC, KS, 2>), grid, block, 0, st, *a);
  else if (a->cpi == 4) launch_kernel((attn_persist_kernel<D, NACC, KS, 4>), grid, block, 0, st, *a);
  else launch_kernel((attn_persist_kernel<D, NACC, KS, 8>), grid, block, 0, st, *a);
  return true;
}

extern "C" hipError_t dflash_launch_attn(const AttnArgs* a, int B, int head_dim, hipStream_t st) {
  const int G = a->n_q / a->n_kv, n_wr = G * a->N / 16;
  const int waves = std::max(a->cand * n_wr, MIN_WAVES);
  // idle staging waves take the second half of the keys: where work items
  // are chunk sequences (at one chunk per item the hand-off did not pay)
  const bool ks2 = a->cpi > 1 && 2 * a->cand * n_wr <= waves;
  const int wgs_z = B / a->grp * ((a->grp + a->cand - 1) / a->cand);
  const int items = 1 + (a->n_ck - 1 + a->cpi - 1) / a->cpi + a->cand - 1;
  dim3 grid(items, a->n_kv, wgs_z);
  if (a->xcd_order) grid = dim3((a->xcd_tuples + 7) / 8 * 8 * a->xcd_items * a->grp);  // whole XCD rounds
  const dim3 block(64 * waves);
  // multi-chunk items of 2, 4 or 8 chunks with 8 waves: the DMA ring; as a
  // persistent kernel where one block per workgroup lets it take the XCD
  // work lists (at most 64 tuples per XCD), at d_h 128 with two key groups
  // (at d_h 64, two workgroups per CU, the item-slot grid was faster)
  const bool dma = waves == 8 && (a->cpi == 2 || a->cpi == 4 || a->cpi == 8);
  if (dma && ks2 && head_dim == 128 && a->xcd_order && a->attn_ctr && (a->xcd_tuples + 7) / 8 <= 64 &&
      launch_persist<128, 1, 2>(a, st))
    return hipGetLastError();
  if (head_dim == 128) {
    if (a->cpi > 1) {
      if (dma && ks2) launch_ring<128, 1, 2>(a, grid, block, st);
      else if (dma) launch_ring<128, 1, 1>(a, grid, block, st);
      else if (ks2) launch_kernel((attn_chunk_kernel<128, 1, true, 2, 0>), grid, block, 0, st, *a);
      else launch_kernel((attn_chunk_kernel<128, 1, true, 1, 0>), grid, block, 0, st, *a);
    } else if (waves <= 8) {
      launch_kernel((attn_chunk_kernel<128, 2, false, 1, 0>), grid, block, 0, st, *a);
    } else {
      launch_kernel((attn_chunk_kernel<128, 1, false, 1, 0>), grid, block, 0, st, *a);
    }
  } else if (a->cpi > 1) {
    if (dma && ks2) launch_ring<64, 1, 2>(a, grid, block, st);  // one S accumulator set: no spills
    else if (dma) launch_ring<64, 1, 1>(a, grid, block, st);  // one S accumulator set: 128 VGPRs, two workgroups per CU
    else if (ks2) launch_kernel((attn_chunk_kernel<64, 2, true, 2, 0>), grid, block, 0, st, *a);
    else launch_kernel((attn_chunk_kernel<64, 2, true, 1, 0>), grid, block, 0, st, *a);
  } else if (waves <= 8) {
    launch_kernel((attn_chunk_kernel<64, 2, false, 1, 0>), grid, block, 0, st, *a);
  } else {
    launch_kernel((attn_chunk_kernel<64, 1, false, 1, 0>), grid, block, 0, st, *a);
  }
  return hipGetLastError();
}

extern "C" hipError_t dflash_launch_attn_merge(const AttnArgs* a, int B, int head_dim, hipStream_t st) {
  const int G = a->n_q / a->n_kv, R = G * a->N;
  // item groups per row: about eight items per thread (one load batch) for
  // the most a block can have, at most a whole workgroup per row; RW rows
  // per workgroup
  const int max_items = 1 + (a->n_ck - 1 + a->cpi - 1) / a->cpi;
  const int tpr = head_dim / 4;
  int cg = 1;
  while (cg < 256 / tpr && cg * 8 < max_items) cg *= 2;
  cg = std::max(cg, 2);
  while (R % (256 / (tpr * cg))) cg *= 2;  // whole row groups per (block, head)
  const int rw = 256 / (tpr * cg);
  const dim3 grid((B * a->n_kv + 7) / 8 * 8 * (R / rw)), block(256);  // whole XCD rounds of (block, kv head) tuples
  if (head_dim == 128) {
    if (cg == 2) launch_kernel((attn_merge_kernel<128, 2>), grid, block, 0, st, *a, B);
    else if (cg == 4) launch_kernel((attn_merge_kernel<128, 4>), grid, block, 0, st, *a, B);
    else launch_kernel((attn_merge_kernel<128, 8>), grid, block, 0, st, *a, B);
  } else {
    if (cg == 2) launch_kernel((attn_merge_kernel<64, 2>), grid, block, 0, st, *a, B);
    else if (cg == 4) launch_kernel((attn_merge_kernel<64, 4>), grid, block, 0, st, *a, B);
    else if (cg == 8) launch_kernel((attn_merge_kernel<64, 8>), grid, block, 0, st, *a, B);
    else launch_kernel((attn_merge_kernel<64, 16>), grid, block, 0, st, *a, B);
  }
  return hipGetLastError();
}
