// Exact per-chunk top-k of a 64x64 coefficient block held by one wave64.
//
// DeMo ("DeMo: Decoupled Momentum Optimization", §3.4 Top-k Sparsification)
// keeps the k largest-magnitude transform coefficients of every chunk and
// zeroes the rest; §3.4 Momentum Subtraction then removes alpha times the
// inverse transform of what was kept from the momentum.  The selection writes
// the payload and leaves Q_hat in place of the block: every kept coefficient
// unchanged, every other one zero, ready for the inverse transform of the
// subtraction.
//
// Ranking is on float32 magnitudes; equal magnitudes go to the lower
// chunk-local index u*64 + v.  Layout: row layout, lane u holds q[v] = Q[u][v].
//
// Fast path (keff <= 64):
//   1. every lane takes the maximum magnitude of its row;
//   2. T0 = the keff-th largest of those 64 row maxima, found bit by bit with
//      wave ballots (at least keff coefficients are >= T0, so the keff-th
//      largest coefficient K satisfies K >= T0);
//   3. the coefficients >= T0 (the candidates; a few dozen for Gaussian
//      blocks) are compacted into LDS in index order;
//   4. K is found bit by bit over the candidates, again with ballots;
//   5. every candidate > K is kept, and of those == K the first ones in index
//      order up to k.
// If the candidates do not fit (more than kMaxCand, e.g. a block of equal
// magnitudes) or keff > 64, the block falls back to the same bitwise search
// run over all 4096 coefficients.  Both paths give the identical set.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "common.h"

namespace demo {
namespace tk {

constexpr int kMaxCand = 256;  // candidates held in LDS, 4 per lane

__device__ __forceinline__ int ballot_count(bool p) { return __popcll(__ballot(p)); }

// number of set lanes of `mask` below this lane
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(uint32_t(mask >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(mask), 0));
}

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

// Bitwise search over all 4096 magnitudes: K = largest T with #(|q| >= T) >= keff.
// Magnitudes are compared as floats through the |x| operand modifier (the
// order of non-negative floats is the order of their bit patterns).  The
// lane's 64 coefficients go to `row` (its 64 floats of LDS, free during the
// call) and the searches read them there, so their registers are free for
// the search: this rarely taken path then does not set the kernel's register
// count.  q is rewritten from `row` at the end.
__device__ __forceinline__ void topk_full_search(float (&q)[64], int keff, int lane, float* __restrict__ outv,
                                                 uint16_t* __restrict__ outi, float* __restrict__ row) {
#pragma unroll
  for (int v = 0; v < 64; ++v) row[v] = q[v];
  float lmax = 0.f;
#pragma unroll
  for (int v = 0; v < 64; ++v) lmax = fmaxf(lmax, fabsf(row[v]));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) lmax = fmaxf(lmax, __shfl_xor(lmax, o));
  const uint32_t hi = __float_as_uint(lmax);
  uint32_t T = 0;
#pragma unroll 1
  for (int b = 30; b >= 0; --b) {
    const uint32_t cand = T | (1u << b);
    if (cand > hi) continue;
    const float cf = __uint_as_float(cand);
    int c = 0;
#pragma unroll
    for (int v = 0; v < 64; ++v) c += fabsf(row[v]) >= cf ? 1 : 0;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o);
    if (c >= keff) T = cand;
  }
  const float kf = __uint_as_float(T);
  int gt = 0, eq = 0;
#pragma unroll
  for (int v = 0; v < 64; ++v) {
    gt += fabsf(row[v]) > kf ? 1 : 0;
    eq += fabsf(row[v]) == kf ? 1 : 0;
  }
  int gt_all = gt;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) gt_all += __shfl_xor(gt_all, o);
  const int quota = keff - gt_all;  // ties at K still to take, in index order
  const int eq_before = wave_incl_scan(eq, lane) - eq;
  const int kept = gt + min(max(quota - eq_before, 0), eq);
  int off = wave_incl_scan(kept, lane) - kept;
  int eqr = eq_before;
#pragma unroll
  for (int v = 0; v < 64; ++v) {
    const float a = fabsf(row[v]);
    const bool is_eq = a == kf;
    const bool keep = a > kf || (is_eq && eqr < quota);
    eqr += is_eq ? 1 : 0;
    const float qv = row[v];
    if (keep) {
      outv[off] = qv;
      outi[off] = static_cast<uint16_t>(lane * 64 + v);
      ++off;
    }
    q[v] = keep ? qv : 0.f;
  }
}

// One wave owns the block (LDS accesses ordered with wave_sync).
// cand: LDS scratch of 2 * kMaxCand words; row: this lane's 64 floats of
// LDS (both free during the call; they may overlap, the fast path uses cand
// and the full search row).
__device__ __forceinline__ void topk_chunk(float (&q)[64], int keff, int lane, float* __restrict__ outv,
                                           uint16_t* __restrict__ outi, uint32_t* __restrict__ cand,
                                           float* __restrict__ row) {
  if (keff >= 4096) {  // lossless: every coefficient, already in index order, all kept
#pragma unroll
    for (int v = 0; v < 64; ++v) {
      outv[lane * 64 + v] = q[v];
      outi[lane * 64 + v] = static_cast<uint16_t>(lane * 64 + v);
    }
    return;
  }
  if (keff > 64) {
    topk_full_search(q, keff, lane, outv, outi, row);
    return;
  }

  // 1-2. T0 = keff-th largest row maximum
  float lm = 0.f;
#pragma unroll
  for (int v = 0; v < 64; ++v) lm = fmaxf(lm, fabsf(q[v]));
  const uint32_t lmb = __float_as_uint(lm);
  uint32_t T0 = 0;
  for (int b = 30; b >= 0; --b) {
    const uint32_t c = T0 | (1u << b);
    if (ballot_count(lmb >= c) >= keff) T0 = c;
  }
  // 3. candidates |q| >= T0, compacted in index order
  int cnt = 0;
  {
    // T0 == 0 counts every coefficient: 4096 > kMaxCand takes the full search
    const float t0 = __uint_as_float(T0);
#pragma unroll
    for (int v = 0; v < 64; ++v) cnt += fabsf(q[v]) >= t0 ? 1 : 0;
  }
  const int incl = wave_incl_scan(cnt, lane);
  const int total = __shfl(incl, 63);
  if (T0 == 0 || total > kMaxCand) {
    topk_full_search(q, keff, lane, outv, outi, row);
    return;
  }
  uint32_t* cmag = cand;             // magnitude bits
  uint32_t* cid = cand + kMaxCand;   // (index << 1) | sign
  {
    const float t0 = __uint_as_float(T0);
    int pos = incl - cnt;
#pragma unroll
    for (int v = 0; v < 64; ++v) {
      if (fabsf(q[v]) >= t0) {
        const uint32_t bits = __float_as_uint(q[v]);
        cmag[pos] = bits & 0x7fffffffu;
        cid[pos] = (uint32_t(lane * 64 + v) << 1) | (bits >> 31);
        ++pos;
      }
    }
  }
  wave_sync();
  const int slots = (total + 63) >> 6;  // 1..4, wave-uniform
  uint32_t m[4], id[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int s = r * 64 + lane;
    const bool live = r < slots && s < total;
    m[r] = live ? cmag[s] : 0u;
    id[r] = live ? cid[s] : 0u;
  }
  wave_sync();
  // 4. K over the candidates.  Every candidate is >= T0 >= 1 and empty slots
  //    hold 0, so empty slots never count for a threshold >= 1.
  uint32_t K = 0;
  if (slots == 1) {
    for (int b = 30; b >= 0; --b) {
      const uint32_t c = K | (1u << b);
      if (ballot_count(m[0] >= c) >= keff) K = c;
    }
  } else {
    for (int b = 30; b >= 0; --b) {
      const uint32_t c = K | (1u << b);
      const int n = ballot_count(m[0] >= c) + ballot_count(m[1] >= c) + ballot_count(m[2] >= c) +
                    ballot_count(m[3] >= c);
      if (n >= keff) K = c;
    }
  }
  // 5. keep > K, and ties == K in index order (slot order is index order)
  const int gt = ballot_count(m[0] > K) + ballot_count(m[1] > K) + ballot_count(m[2] > K) + ballot_count(m[3] > K);
  const int quota = keff - gt;
  int eq_before = 0, out_before = 0, eq_total = 0;
  uint32_t last_tie = 0;  // index of the last tie taken
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (r < slots) {
      const uint64_t eqm = __ballot(m[r] == K);
      const int my_eq = eq_before + lanes_below(eqm);
      const bool keep = m[r] > K || (m[r] == K && my_eq < quota);
      if (m[r] == K && my_eq == quota - 1) last_tie = id[r] >> 1;
      const uint64_t km = __ballot(keep);
      if (keep) {
        const int o = out_before + lanes_below(km);
        outv[o] = __uint_as_float(m[r] | (id[r] << 31));
        outi[o] = static_cast<uint16_t>(id[r] >> 1);
      }
      eq_before += __popcll(eqm);
      out_before += __popcll(km);
    }
  }
  eq_total = eq_before;
  const float kf = __uint_as_float(K);
  if (eq_total == quota) {
    // no tie is dropped: kept <=> |q| >= K
#pragma unroll
    for (int v = 0; v < 64; ++v) q[v] = fabsf(q[v]) >= kf ? q[v] : 0.f;
  } else {
    // some coefficients equal to K are dropped: keep those up to the last tie taken
    uint32_t lt = last_tie;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) lt = max(lt, uint32_t(__shfl_xor(int(lt), o)));
#pragma unroll
    for (int v = 0; v < 64; ++v) {
      const float a = fabsf(q[v]);
      const bool keep = a > kf || (a == kf && uint32_t(lane * 64 + v) <= lt);
      q[v] = keep ? q[v] : 0.f;
    }
  }
}

// Top-k of one 64-element vector chunk held in one lane (vector chunks: lane
// = chunk).  Same rule; writes only when `write` (lanes past the tensor's last
// chunk hold zeros and write nothing).  Leaves Q_hat in q.
__device__ __forceinline__ void topk_lane(float (&q)[64], int keff, bool write, float* __restrict__ outv,
                                          uint16_t* __restrict__ outi) {
  if (keff >= 64) {
#pragma unroll
    for (int v = 0; v < 64; ++v) {
      if (write) {
        outv[v] = q[v];
        outi[v] = static_cast<uint16_t>(v);
      }
    }
    return;
  }
  float lmax = 0.f;
#pragma unroll
  for (int v = 0; v < 64; ++v) lmax = fmaxf(lmax, fabsf(q[v]));
  const uint32_t hi = __float_as_uint(lmax);
  uint32_t T = 0;
#pragma unroll 1
  for (int b = 30; b >= 0; --b) {
    const uint32_t cand = T | (1u << b);
    const float cf = __uint_as_float(cand);
    int c = 0;
#pragma unroll
    for (int v = 0; v < 64; ++v) c += fabsf(q[v]) >= cf ? 1 : 0;
    if (cand <= hi && c >= keff) T = cand;
  }
  const float kf = __uint_as_float(T);
  int gt = 0;
#pragma unroll
  for (int v = 0; v < 64; ++v) gt += fabsf(q[v]) > kf ? 1 : 0;
  const int quota = keff - gt;
  int eqr = 0, off = 0;
#pragma unroll
  for (int v = 0; v < 64; ++v) {
    const float a = fabsf(q[v]);
    const bool is_eq = a == kf;
    const bool keep = a > kf || (is_eq && eqr < quota);
    eqr += is_eq ? 1 : 0;
    if (keep) {
      if (write) {
        outv[off] = q[v];
        outi[off] = static_cast<uint16_t>(v);
      }
      ++off;
    }
    q[v] = keep ? q[v] : 0.f;
  }
}

}  // namespace tk
}  // namespace demo
