// HIP kernels of the DeMo codec for chunk edge s = 128 on CDNA4 (gfx950).
//
// The pages run DeMo with 64x64 and with 128x128 chunks ("DeMo: Decoupled
// Momentum Optimization", summary §3.4 Tensor Chunking; Ablation Studies and
// Robustness Checks, chunk size s = 64 vs s = 128).  The method is the same
// as for s = 64 (see kernels.hip); only the transform length and the chunk
// size change.
//
// Transform.  The orthonormal 128-point DCT-II splits into two 64-point
// halves: the even frequencies 2m are a 64-point DCT-II of the sums
// x[n] + x[127-n], the odd frequencies 2m+1 a 64-point DCT-IV of the
// differences x[n] - x[127-n], both scaled by sqrt(2/128).  On both
// dimensions of a 128x128 block this makes four independent 64x64
// transforms: sub-block (a, b) holds the coefficients Q[2u+a][2v+b] and is
// the (C_a x C_b) transform (C_0 = DCT-II, C_1 = DCT-IV) of
//   S_ab[i][j] = sum over quadrants (qa, qb) of (-1)^(a qa + b qb) B_q[i][j],
// where B_q[i][j] is chunk element (qa ? 127-i : i, qb ? 127-j : j).  The
// inverse applies the transposed halves and the same sign combination (the
// factor 1/2 of the butterfly's inverse is inside the sqrt(2/128) scaling).
//
// Work split.  A 256-thread workgroup (four wave64) owns one 128x128 chunk.
// Wave q loads quadrant q already in those (i, j) coordinates (row and lane
// order reversed in the second halves; each row segment is still one
// contiguous 256-byte access), the waves exchange quadrants through LDS to
// form S_ab (wave w = 2a + b takes sub-block (a, b)), and each wave then runs
// its 64x64 sub-block exactly like a 64x64 chunk: column pass in registers,
// LDS transpose, row pass.  Top-k is workgroup-wide over the 16384
// coefficients of the chunk; in the decode each wave scatters the W
// payloads' entries of its own sub-block into its own quarter of the LDS, in
// worker order, so sums are deterministic.
//
// A vector is cut into 128-element chunks; a workgroup item is 128 chunks,
// 32 per wave.  A lane pair holds one chunk (lane 2g + h: half h of chunk g),
// the halves are exchanged between the two lanes with DPP, and lane h runs
// the 64-point half transform h.
#include "common.h"
#include "launch.h"
#include "xform.h"

namespace demo {
namespace {

using xf::Ortho;
using xf::Unit;

constexpr int kS = 128;
constexpr int kLd = 65;             // per-wave transpose tile row stride (floats)
constexpr int kTile = 64 * kLd;     // floats of one wave's transpose tile
constexpr int kQuad = 64 * 64;      // floats of one quadrant in the butterfly exchange
constexpr int kWorkerBatch = 16;
constexpr int kVecChunksPerWave = 32;
constexpr int kVecChunksPerItem = 4 * kVecChunksPerWave;

// encode LDS: four transpose tiles (the butterfly exchange reuses them), then
// the top-k scratch
constexpr int kTilesWords = 4 * kTile;
constexpr int kSlots = 1;                 // top-k candidate slots per lane and wave
constexpr int kCandPerWave = 64 * kSlots;  // candidates each wave may put in LDS
// top-k scratch: 16 header words, 512 kept-mask words, candidate values and
// indices, the kept list (64 values, 64 indices)
constexpr int kScrWords = 16 + 512 + 2 * 4 * kCandPerWave + 128;
constexpr int kEncLdsWords = kTilesWords + kScrWords;
// decode LDS: 128 x 128 fp32 sums + 128 x 32 words of 8-bit counts, as four
// per-wave quarters; the tiles, the butterfly exchange and the vector path
// reuse it
constexpr int kDecLdsWords = kS * kS + kS * kS / 4;
static_assert(kTilesWords <= kDecLdsWords && 4 * kQuad <= kTilesWords, "LDS regions");
static_assert(kDecLdsWords * 4 <= 81920, "two decode workgroups per CU");
static_assert((kEncLdsWords * 4) * 2 <= 160 * 1024, "two encode workgroups per CU");

// ---------------------------------------------------------------- halves of the 128-point DCT

// h = 0: even frequencies from the sums; h = 1: odd frequencies from the differences.
__device__ __forceinline__ void fwd_half(float (&x)[64], int h) {
  if (h == 0)
    xf::dct2<64, Ortho<128>>(x);
  else
    xf::dct4<64, Unit, Ortho<128>>(x);
}

__device__ __forceinline__ void inv_half(float (&x)[64], int h) {
  if (h == 0)
    xf::dct3<64, Ortho<128>>(x);
  else
    xf::dct4<64, Ortho<128>, Unit>(x);
}

// ---------------------------------------------------------------- wave / workgroup helpers

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ int ballot_count(bool p) { return __popcll(__builtin_amdgcn_ballot_w64(p)); }

// Sum over the four waves of one wave-uniform value.  `buf` holds two sets of
// four words used alternately (`parity`), so one barrier per call suffices: a
// wave can only overwrite a set after every wave has passed the next call's
// barrier, i.e. after all of them have read it.
__device__ __forceinline__ int wg_sum(int v, uint32_t* buf, int& parity, int w, int lane) {
  uint32_t* b = buf + parity * 4;
  if (lane == 0) b[w] = uint32_t(v);
  __syncthreads();
  parity ^= 1;
  return int(b[0] + b[1] + b[2] + b[3]);
}

// value of the other lane of this lane's pair (lanes 2g and 2g+1)
__device__ __forceinline__ float pair_swap(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ int pair_swap(int v) { return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false); }
__device__ __forceinline__ uint64_t pair_swap(uint64_t v) {
  return (uint64_t(uint32_t(pair_swap(int(v >> 32)))) << 32) | uint32_t(pair_swap(int(uint32_t(v))));
}

__device__ __forceinline__ int popc64(uint64_t v) { return __popcll(v); }

// bits below position n (n in 0..64)
__device__ __forceinline__ uint64_t below(int n) { return n >= 64 ? ~0ull : ((1ull << n) - 1ull); }

// Per-wave LDS transposes through the wave's own tile.  col_to_row only
// synchronises the wave: its tile is its own, and whatever LDS the workgroup
// used before was released by a workgroup barrier.  row_to_col ends with a
// workgroup barrier because a butterfly exchange, which spans every wave's
// tile, may follow it.
__device__ __forceinline__ void col_to_row(float* tile, float (&x)[64], int lane) {
#pragma unroll
  for (int i = 0; i < 64; ++i) tile[i * kLd + lane] = x[i];
  wave_sync();
#pragma unroll
  for (int v = 0; v < 64; ++v) x[v] = tile[lane * kLd + v];
  wave_sync();
}

__device__ __forceinline__ void row_to_col(float* tile, float (&x)[64], int lane) {
#pragma unroll
  for (int v = 0; v < 64; ++v) tile[lane * kLd + v] = x[v];
  wave_sync();
#pragma unroll
  for (int i = 0; i < 64; ++i) x[i] = tile[i * kLd + lane];
  __syncthreads();
}

// Wave W's share of the exchange: x <- (x_0 + sb x_1) + sa (x_2 + sb x_3),
// sa = (-1)^a, sb = (-1)^b for W = 2a + b, x_q the rows of wave q (x_W is
// this wave's own registers).  The same operations, in the same order, as a
// two-point butterfly along dimension 1 followed by one along dimension 0.
template <int W>
__device__ __forceinline__ void butterfly_combine(float (&x)[64], const float* xq, int lane) {
  constexpr float sa = (W & 2) ? -1.f : 1.f, sb = (W & 1) ? -1.f : 1.f;
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    float v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = q == W ? x[i] : xq[q * kQuad + i * 64 + lane];
    x[i] = fmaf(sa, fmaf(sb, v[3], v[2]), fmaf(sb, v[1], v[0]));
  }
}

// One butterfly stage between wave w and wave w ^ bit: the wave without `bit`
// keeps own + partner, the one with it partner - own.
__device__ __forceinline__ void butterfly_stage(float (&x)[64], float* xq, int w, int lane, int bit) {
#pragma unroll
  for (int i = 0; i < 64; ++i) xq[w * kQuad + i * 64 + lane] = x[i];
  __syncthreads();
  const float sg = (w & bit) ? -1.f : 1.f;
  const float* __restrict__ px = xq + (w ^ bit) * kQuad + lane;
#pragma unroll
  for (int i = 0; i < 64; ++i) x[i] = fmaf(sg, x[i], px[i * 64]);
  __syncthreads();
}

// The same exchange as butterfly() in two stages (along dimension 1, then 0),
// each through LDS: two more barriers, fewer live registers, bitwise the same
// result.  Used where the registers are full (decode updating X and M).
__device__ __forceinline__ void butterfly_staged(float (&x)[64], float* xq, int w, int lane) {
  butterfly_stage(x, xq, w, lane, 1);
  butterfly_stage(x, xq, w, lane, 2);
}

// x <- sum over the four waves' x (same i, same lane) with sign (-1)^(a qa + b qb),
// (a, b) the bits of this wave, (qa, qb) those of the other.
// Forward: quadrants -> S_ab; inverse: S'_ab -> quadrants.  One exchange
// through LDS; leaves the exchange area free.
template <bool kRelease = true>
__device__ __forceinline__ void butterfly(float (&x)[64], float* xq, int w, int lane) {
#pragma unroll
  for (int i = 0; i < 64; ++i) xq[w * kQuad + i * 64 + lane] = x[i];
  __syncthreads();
  switch (w) {
    case 0: butterfly_combine<0>(x, xq, lane); break;
    case 1: butterfly_combine<1>(x, xq, lane); break;
    case 2: butterfly_combine<2>(x, xq, lane); break;
    default: butterfly_combine<3>(x, xq, lane); break;
  }
  if constexpr (kRelease) __syncthreads();
}

struct Chunk128 {
  int local;     // chunk ordinal within its tensor
  int vr, vc;    // valid rows / columns
  int64_t base;  // element offset of the chunk's (0, 0)
  bool full;
};

__device__ __forceinline__ Chunk128 chunk_pos128(const TensorSlot& ts, int item) {
  Chunk128 c;
  c.local = item - ts.item_begin;
  const int grid1 = int((uint32_t(ts.cols) + 127u) >> 7);
  const int cr = c.local / grid1;
  const int cc = c.local - cr * grid1;
  c.vr = min(kS, ts.rows - cr * kS);
  c.vc = min(kS, ts.cols - cc * kS);
  c.base = int64_t(cr) * kS * ts.cols + int64_t(cc) * kS;
  c.full = (c.vr == kS) && (c.vc == kS);
  return c;
}

// The workgroup's wave number, in a scalar register (the compiler cannot see
// that threadIdx.x >> 6 is the same on every lane of a wave).
__device__ __forceinline__ int wave_index() { return __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6)); }

// quadrant coordinates -> chunk coordinates
__device__ __forceinline__ int quad_row(int qa, int i) { return qa ? (kS - 1 - i) : i; }

// ---------------------------------------------------------------- top-k over a 128x128 chunk

// Wave w = 2a + b holds sub-block (a, b) in row layout: lane u, q[v] =
// Q[2u+a][2v+b], chunk-local index (2u+a)*128 + 2v + b.  Keeps the keff
// largest magnitudes (float32; equal magnitudes: lower index first), writes
// them in index order and leaves Q_hat in q (kept coefficients unchanged,
// the others zero).
//
// Fast path (keff <= 64), one workgroup barrier:
//   1. each wave finds T_w = the keff-th largest of its 64 lane maxima (wave
//      ballots, as for a 64x64 chunk) and puts its coefficients >= T_w (the
//      candidates) into its own LDS region;
//   2. every wave reads all four regions and finds, redundantly, the
//      threshold K and the tie cut over the union.  The union holds every
//      coefficient >= K: K >= each wave's own keff-th largest >= T_w;
//   3. wave 0 ranks the keff kept candidates by index and writes the payload;
//      every wave zeroes its own coefficients that were not kept.
// Otherwise (keff > 64, or a region overflows, e.g. a block of equal
// magnitudes) the same bitwise searches run over all 16384 coefficients with
// workgroup-wide counts, and the payload positions come from kept-bit masks.

// Returns true when the payload is still to be written by emit_kept (fast
// path: wave 0 holds the kept list in LDS scratch that nothing else reuses).
template <bool kSmallK>
__device__ __forceinline__ bool topk128(float (&q)[64], int keff, int w, int lane, float* __restrict__ outv,
                                        uint16_t* __restrict__ outi, uint32_t* scr, float* tile) {
  const int a = w >> 1, b = w & 1;
  const uint32_t idx0 = uint32_t((2 * lane + a) * kS + b);  // index of q[0]; q[v] sits at idx0 + 2v
  uint32_t* hdr = scr;                             // [0, 4): candidates per wave (~0u: none)
  uint32_t* red = scr + 8;                         // two sets of four words: workgroup sums
  uint32_t* kmask = scr + 16;                      // kept bits, 2 words per lane and wave
  uint32_t* cval = scr + 528;                      // candidate value bits, kCandPerWave per wave
  uint32_t* cid = cval + 4 * kCandPerWave;         // candidate indices
  uint32_t* kl = cid + 4 * kCandPerWave;           // wave 0: kept list (64 values, 64 indices)

  if (!kSmallK && keff >= kS * kS) {  // lossless: every coefficient, at its own index
    // one base per lane, constant offsets per v (no 64 separate addresses)
    float* __restrict__ ov = outv + idx0;
    uint16_t* __restrict__ oi = outi + idx0;
#pragma unroll
    for (int v = 0; v < 64; ++v) {
      ov[2 * v] = q[v];
      oi[2 * v] = static_cast<uint16_t>(idx0 + 2 * v);
    }
    return false;
  }

  float lm = 0.f;
#pragma unroll
  for (int v = 0; v < 64; ++v) lm = fmaxf(lm, fabsf(q[v]));
  uint32_t K = 0, cut = 0xffffffffu;  // cut: largest index admitted among |q| == K
  bool fast = kSmallK || keff <= 64;
  if (fast) {
    const uint32_t lmb = __float_as_uint(lm);
    uint32_t T = 0;
    for (int bit = 30; bit >= 0; --bit) {
      const uint32_t c = T | (1u << bit);
      if (ballot_count(lmb >= c) >= keff) T = c;
    }
    // Candidates in column order: column v's ballot places them after the
    // ones already found (a wave-uniform running count), so no per-lane
    // count and scan come first.  The order within a region does not matter:
    // the tie cut searches indices and emit_kept ranks by index.
    uint32_t cw = 0;
    if (T != 0) {
      const float t = __uint_as_float(T);
      uint32_t* cv = cval + w * kCandPerWave;
      uint32_t* ci = cid + w * kCandPerWave;
#pragma unroll
      for (int v = 0; v < 64; ++v) {
        const bool is_c = fabsf(q[v]) >= t;
        const uint64_t m = __builtin_amdgcn_ballot_w64(is_c);
        if (m != 0) {  // wave-uniform
          if (is_c) {
            const uint32_t pos = cw + uint32_t(lanes_below_mask(m));
            if (pos < uint32_t(kCandPerWave)) {
              cv[pos] = __float_as_uint(q[v]);
              ci[pos] = idx0 + 2 * v;
            }
          }
          cw += uint32_t(__popcll(m));
        }
      }
    }
    if (lane == 0) hdr[w] = T != 0 ? cw : 0xffffffffu;
    __syncthreads();
    uint32_t C[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      C[r] = hdr[r];
      fast = fast && C[r] <= uint32_t(kCandPerWave);
    }
    if (fast) {  // the same decision in every wave
      // slot j = (region r = j / kSlots, entry (j % kSlots) * 64 + lane); empty slots hold 0, never counted
      uint32_t mg[4 * kSlots];
#pragma unroll
      for (int j = 0; j < 4 * kSlots; ++j) {
        const uint32_t e = uint32_t((j % kSlots) * 64 + lane);
        mg[j] = e < C[j / kSlots] ? (cval[(j / kSlots) * kCandPerWave + e] & 0x7fffffffu) : 0u;
      }
      for (int bit = 30; bit >= 0; --bit) {
        const uint32_t c = K | (1u << bit);
        int n = 0;
#pragma unroll
        for (int j = 0; j < 4 * kSlots; ++j) n += ballot_count(mg[j] >= c);
        if (n >= keff) K = c;
      }
      int gt = 0, eq = 0;
#pragma unroll
      for (int j = 0; j < 4 * kSlots; ++j) {
        gt += ballot_count(mg[j] > K);
        eq += ballot_count(mg[j] == K);
      }
      const int quota = keff - gt;
      if (eq > quota) {  // the quota-th smallest index among the ties
        uint32_t L = 0;
        for (int bit = 13; bit >= 0; --bit) {
          const uint32_t c = L | (1u << bit);
          int n = 0;
#pragma unroll
          for (int j = 0; j < 4 * kSlots; ++j) {
            const uint32_t e = uint32_t((j % kSlots) * 64 + lane);
            const uint32_t id = e < C[j / kSlots] ? cid[(j / kSlots) * kCandPerWave + e] : 0xffffffffu;
            n += ballot_count(mg[j] == K && id < c);
          }
          if (n < quota) L = c;
        }
        cut = L;
      }
      if (w == 0) {
        // compact the keff kept candidates into the kept list; emit_kept ranks
        // and writes them at the end of the chunk (the other waves do not wait)
        int off = 0;
#pragma unroll
        for (int j = 0; j < 4 * kSlots; ++j) {
          const int r = j / kSlots;
          const uint32_t e = uint32_t((j % kSlots) * 64 + lane);
          const bool live = e < C[r];
          const uint32_t id = live ? cid[r * kCandPerWave + e] : 0u;
          const bool keep = live && (mg[j] > K || (mg[j] == K && id <= cut));
          const uint64_t km = __builtin_amdgcn_ballot_w64(keep);
          if (keep) {
            const int o = off + lanes_below_mask(km);
            kl[o] = cval[r * kCandPerWave + e];
            kl[64 + o] = id;
          }
          off += __popcll(km);
        }
      }
      const float kf = __uint_as_float(K);
      if (cut == 0xffffffffu) {  // no tie dropped: kept <=> |q| >= K (the same branch in every wave)
#pragma unroll
        for (int v = 0; v < 64; ++v) q[v] = fabsf(q[v]) >= kf ? q[v] : 0.f;
      } else {
#pragma unroll
        for (int v = 0; v < 64; ++v) {
          const float m = fabsf(q[v]);
          const bool keep = m > kf || (m == kf && idx0 + 2 * v <= cut);
          q[v] = keep ? q[v] : 0.f;
        }
      }
      return true;
    }
  }

  // bitwise searches over all 16384 magnitudes, counted across the workgroup.
  // The lane's 64 coefficients go to the wave's transpose tile (unused during
  // top-k) and the searches read them there, one lane its own row: their
  // registers are then free for the search, which keeps this rarely taken
  // path from setting the kernel's register count.
  float* __restrict__ row = tile + lane * kLd;
#pragma unroll
  for (int v = 0; v < 64; ++v) row[v] = q[v];
  int parity = 0;
  float hmax = lm;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) hmax = fmaxf(hmax, __shfl_xor(hmax, o));
  if (lane == 0) red[w] = __float_as_uint(hmax);
  __syncthreads();
  const uint32_t hi = max(max(red[0], red[1]), max(red[2], red[3]));
  parity = 1;  // set 0 of `red` is still being read
  uint32_t T = 0;
  for (int bit = 30; bit >= 0; --bit) {
    const uint32_t c = T | (1u << bit);
    if (c > hi) continue;  // the same for every wave
    const float cf = __uint_as_float(c);
    int n = 0;
#pragma unroll
    for (int v = 0; v < 64; ++v) n += fabsf(row[v]) >= cf ? 1 : 0;
    if (wg_sum(wave_sum(n), red, parity, w, lane) >= keff) T = c;
  }
  K = T;
  const float kf = __uint_as_float(K);
  {
    int gt = 0, eq = 0;
#pragma unroll
    for (int v = 0; v < 64; ++v) {
      gt += fabsf(row[v]) > kf ? 1 : 0;
      eq += fabsf(row[v]) == kf ? 1 : 0;
    }
    const int quota = keff - wg_sum(wave_sum(gt), red, parity, w, lane);
    if (wg_sum(wave_sum(eq), red, parity, w, lane) > quota) {
      uint64_t eqm = 0;  // ties of this lane; row[v] has index idx0 + 2v
#pragma unroll
      for (int v = 0; v < 64; ++v) eqm |= fabsf(row[v]) == kf ? (1ull << v) : 0ull;
      uint32_t L = 0;
      for (int bit = 13; bit >= 0; --bit) {
        const uint32_t c = L | (1u << bit);
        const int nv = min(64, max(0, (int(c) - int(idx0) + 1) >> 1));  // v with idx0 + 2v < c
        if (wg_sum(wave_sum(popc64(eqm & below(nv))), red, parity, w, lane) < quota) L = c;
      }
      cut = L;
    }
  }

  // kept masks; the payload position of a kept coefficient is the number of
  // kept coefficients of smaller index: rows before its row (rows 2u and
  // 2u+1 belong to lane u of waves 0,1 and 2,3), plus, in its row, its own
  // wave's kept entries of smaller v and its partner wave's (other b) ones
  // of smaller column.
  uint64_t mine = 0;
#pragma unroll
  for (int v = 0; v < 64; ++v) {
    const float m = fabsf(row[v]);
    const bool keep = m > kf || (m == kf && idx0 + 2 * v <= cut);
    mine |= keep ? (1ull << v) : 0ull;
  }
  kmask[(w * 64 + lane) * 2] = uint32_t(mine);
  kmask[(w * 64 + lane) * 2 + 1] = uint32_t(mine >> 32);
  __syncthreads();
  uint64_t mk[4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
    mk[r] = (uint64_t(kmask[(r * 64 + lane) * 2 + 1]) << 32) | kmask[(r * 64 + lane) * 2];
  const int c0 = popc64(mk[0]) + popc64(mk[1]);  // row 2u
  const int c1 = popc64(mk[2]) + popc64(mk[3]);  // row 2u + 1
  const int tot = c0 + c1;
  const int rbase = wave_incl_scan(tot, lane) - tot + (a ? c0 : 0);
  const uint64_t partner = mk[w ^ 1];
  // positions by running counts: this lane's kept entries before v, and the
  // partner's before column 2v + b (bits below v + b of its mask)
  int pos = rbase + (b ? int(partner & 1ull) : 0);
#pragma unroll
  for (int v = 0; v < 64; ++v) {
    const bool keep = (mine >> v) & 1ull;
    const float qv = row[v];
    if (keep) {
      outv[pos] = qv;
      outi[pos] = static_cast<uint16_t>(idx0 + 2 * v);
    }
    q[v] = keep ? qv : 0.f;
    pos += int(keep) + ((v + b < 64) ? int((partner >> (v + b)) & 1ull) : 0);
  }
  return false;
}

// Wave 0, after the fast path: the keff (<= 64) kept candidates of the kept
// list, ranked by index, into the payload.
__device__ __forceinline__ void emit_kept(int keff, int lane, float* __restrict__ outv, uint16_t* __restrict__ outi,
                                          const uint32_t* scr) {
  const uint32_t* kl = scr + 528 + 2 * 4 * kCandPerWave;
  const bool mine = lane < keff;
  const uint32_t myv = mine ? kl[lane] : 0u;
  const uint32_t myid = mine ? kl[64 + lane] : 0xffffffffu;
  int rank = 0;
  for (int j = 0; j < keff; ++j) rank += uint32_t(__builtin_amdgcn_readlane(int(myid), j)) < myid ? 1 : 0;
  if (mine) {
    outv[rank] = __uint_as_float(myv);
    outi[rank] = static_cast<uint16_t>(myid);
  }
}

// ---------------------------------------------------------------- top-k over a 128-element vector chunk

// The chunk is held by a lane pair: lane h has y[m] = coefficient 2m + h.
// Same rule as above over the pair; `write` is false for lanes past the
// tensor's last chunk.  Leaves the pair's half of Q_hat in y.
__device__ __forceinline__ void topk_pair(float (&y)[64], int keff, int h, bool write, float* __restrict__ outv,
                                          uint16_t* __restrict__ outi) {
  float lm = 0.f;
#pragma unroll
  for (int m = 0; m < 64; ++m) lm = fmaxf(lm, fabsf(y[m]));
  const uint32_t hi = max(__float_as_uint(lm), __float_as_uint(pair_swap(lm)));
  uint32_t T = 0;
#pragma unroll 1
  for (int bit = 30; bit >= 0; --bit) {
    const uint32_t c = T | (1u << bit);
    const float cf = __uint_as_float(c);
    int n = 0;
#pragma unroll
    for (int m = 0; m < 64; ++m) n += fabsf(y[m]) >= cf ? 1 : 0;
    n += pair_swap(n);
    if (c <= hi && n >= keff) T = c;
  }
  const float kf = __uint_as_float(T);
  int gt = 0, eq = 0;
#pragma unroll
  for (int m = 0; m < 64; ++m) {
    gt += fabsf(y[m]) > kf ? 1 : 0;
    eq += fabsf(y[m]) == kf ? 1 : 0;
  }
  gt += pair_swap(gt);
  eq += pair_swap(eq);
  const int quota = keff - gt;
  uint32_t cut = 0xffffffffu;
  if (eq > quota) {
    uint64_t eqm = 0;  // ties of this lane; y[m] is coefficient 2m + h
#pragma unroll
    for (int m = 0; m < 64; ++m) eqm |= fabsf(y[m]) == kf ? (1ull << m) : 0ull;
    uint32_t L = 0;
#pragma unroll 1
    for (int bit = 6; bit >= 0; --bit) {
      const uint32_t c = L | (1u << bit);
      int n = popc64(eqm & below(min(64, max(0, (int(c) - h + 1) >> 1))));  // m with 2m + h < c
      n += pair_swap(n);
      if (n < quota) L = c;
    }
    cut = L;
  }
  uint64_t mine = 0;
#pragma unroll
  for (int m = 0; m < 64; ++m) {
    const float v = fabsf(y[m]);
    const bool keep = v > kf || (v == kf && uint32_t(2 * m + h) <= cut);
    mine |= keep ? (1ull << m) : 0ull;
  }
  const uint64_t partner = pair_swap(mine);
#pragma unroll
  for (int m = 0; m < 64; ++m) {
    if ((mine >> m) & 1ull) {
      if (write) {
        const int pos = popc64(mine & below(m)) + popc64(partner & below(m + h));
        outv[pos] = y[m];
        outi[pos] = static_cast<uint16_t>(2 * m + h);
      }
    }
    y[m] = ((mine >> m) & 1ull) ? y[m] : 0.f;
  }
}

// ---------------------------------------------------------------- encode

// Element offset of quadrant q's (0, lane) inside the chunk, and the
// (wave-uniform) offset from one quadrant row to the next.
__device__ __forceinline__ int64_t quad_origin(int q, int lane, int64_t ld) {
  return int64_t((q >> 1) ? kS - 1 : 0) * ld + ((q & 1) ? kS - 1 - lane : lane);
}
__device__ __forceinline__ int64_t quad_step(int q, int64_t ld) { return (q >> 1) ? -ld : ld; }

// Quadrant q's row i of a full chunk through buffer instructions: chunk row
// quad_row(q >> 1, i) (a scalar offset; q is wave-uniform), the lane's
// column (q & 1 ? 127 - lane : lane) the vector offset.
__device__ __forceinline__ void load_quad_rows(float (&x)[64], const float* __restrict__ chunk, int64_t ld, int q,
                                               int lane) {
  const RowBuf b = row_buf(chunk, ld * 4);
  const int col = (q & 1) ? kS - 1 - lane : lane;
#pragma unroll
  for (int i = 0; i < 64; ++i) x[i] = buf_load_f32(b, quad_row(q >> 1, i), col * 4);
}

template <bool kFull, bool kBf16, bool kKeep = false>
__device__ __forceinline__ void load_quadrant(float (&x)[64], const TensorSlot& ts, const Chunk128& c, int q,
                                              int lane, float beta, float gcoef) {
  const int64_t ld = ts.cols, step = quad_step(q, ld), o = c.base + quad_origin(q, lane, ld);
  const int col = (q & 1) ? kS - 1 - lane : lane;
  if (kFull && !kKeep && buf_rows_fit(kS, ld * 4)) {
    const RowBuf bm = row_buf(ts.dst + c.base, ld * 4);
    const RowBuf bg = row_buf(static_cast<const char*>(ts.aux) + c.base * (kBf16 ? 2 : 4), ld * (kBf16 ? 2 : 4));
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      const int r = quad_row(q >> 1, i);
      const float gv = kBf16 ? buf_load_bf16(bg, r, col * 2) : buf_load_f32(bg, r, col * 4);
      x[i] = fmaf(beta, buf_load_f32(bm, r, col * 4), gcoef * gv);
    }
    return;
  }
  const float* __restrict__ m = ts.dst + o;
  const char* __restrict__ g = static_cast<const char*>(ts.aux) + o * (kBf16 ? 2 : 4);
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    float gv = 0.f, mv = 0.f;
    if (kFull || (quad_row(q >> 1, i) < c.vr && col < c.vc)) {
      gv = load_src<kBf16, kKeep>(g, i * step);
      mv = kKeep ? m[i * step] : stream_load(&m[i * step]);
    }
    x[i] = fmaf(beta, mv, gcoef * gv);
  }
}

template <bool kFull>
__device__ __forceinline__ void store_quadrant(const float (&x)[64], float* __restrict__ dst, int64_t ld,
                                               const Chunk128& c, int q, int lane) {
  const int64_t step = quad_step(q, ld);
  const int col = (q & 1) ? kS - 1 - lane : lane;
  if (kFull && buf_rows_fit(kS, ld * 4)) {
    const RowBuf b = row_buf(dst, ld * 4);
#pragma unroll
    for (int i = 0; i < 64; ++i) buf_store_f32(b, quad_row(q >> 1, i), col * 4, x[i]);
    return;
  }
  float* __restrict__ d = dst + quad_origin(q, lane, ld);
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    if (kFull || (quad_row(q >> 1, i) < c.vr && col < c.vc)) stream_store(x[i], &d[i * step]);
  }
}

template <bool kBf16, bool kSmallK>
__device__ __forceinline__ void encode_matrix128(const TensorSlot& ts, const EncodeParams& p, float* lds,
                                                 uint32_t* scr) {
  const int w = wave_index(), lane = threadIdx.x & 63;
  const int a = w >> 1, b = w & 1;
  const Chunk128 c = chunk_pos128(ts, blockIdx.x);
  float* __restrict__ mdst = ts.dst + c.base;

  float x[64];
  if (c.full)
    load_quadrant<true, kBf16>(x, ts, c, w, lane, p.beta, p.gcoef);
  else
    load_quadrant<false, kBf16>(x, ts, c, w, lane, p.beta, p.gcoef);
  if (!p.subtract_local) {  // aggregated subtraction: M = M' now, the decode side subtracts
    if (c.full)
      store_quadrant<true>(x, mdst, ts.cols, c, w, lane);
    else
      store_quadrant<false>(x, mdst, ts.cols, c, w, lane);
  }
  float mp[64];  // the quadrant's M', held for the subtraction
#pragma unroll
  for (int i = 0; i < 64; ++i) mp[i] = x[i];

  butterfly(x, lds, w, lane);  // quadrants -> S_ab
  fwd_half(x, a);
  col_to_row(lds + w * kTile, x, lane);
  fwd_half(x, b);

  const int64_t e0 = ts.entry_begin + int64_t(c.local) * p.keff2;
  const bool deferred = topk128<kSmallK>(x, p.keff2, w, lane, p.pay_val + e0, p.pay_idx + e0, scr, lds + w * kTile);
  if (!p.subtract_local) {
    if (deferred && w == 0) emit_kept(p.keff2, lane, p.pay_val + e0, p.pay_idx + e0, scr);
    return;
  }

  inv_half(x, b);  // x holds Q_hat: R = P^T Q_hat P, quadrant by quadrant
  row_to_col(lds + w * kTile, x, lane);
  inv_half(x, a);
  butterfly<false>(x, lds, w, lane);  // S'_ab -> quadrants; the tiles are not used again

  // M = M' - alpha R
#pragma unroll
  for (int i = 0; i < 64; ++i) x[i] = fmaf(-p.alpha, x[i], mp[i]);
  if (c.full)
    store_quadrant<true>(x, mdst, ts.cols, c, w, lane);
  else
    store_quadrant<false>(x, mdst, ts.cols, c, w, lane);
  if (deferred && w == 0) emit_kept(p.keff2, lane, p.pay_val + e0, p.pay_idx + e0, scr);
}

// Lane pair (2g, 2g+1) holds chunk g of this wave's 32: x[e] = position 64h + e.
// In place, x becomes the sums x_n + x_{127-n} (h = 0) or the differences
// x_n - x_{127-n} (h = 1), n = 0..63.
__device__ __forceinline__ void pair_butterfly(float (&x)[64], int h) {
#pragma unroll
  for (int n = 0; n < 32; ++n) {
    const float on = x[n], om = x[63 - n];
    const float pn = pair_swap(on), pm = pair_swap(om);
    x[n] = h ? pn - om : on + pm;
    x[63 - n] = h ? pm - on : om + pn;
  }
}

// Inverse of pair_butterfly after the inverse half transforms (lane h holds
// the even part a_n or the odd part b_n): in place, lane h gets positions
// 64h + e of its chunk, x_n = a_n + b_n and x_{127-n} = a_n - b_n.
__device__ __forceinline__ void pair_unbutterfly(float (&y)[64], int h) {
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    const float ye = y[e], ym = y[63 - e];
    const float pe = pair_swap(ye), pm = pair_swap(ym);
    y[e] = h ? pm - ym : ye + pe;
    y[63 - e] = h ? pe - ye : ym + pm;
  }
}

template <bool kBf16>
__device__ __forceinline__ void encode_vector128(const TensorSlot& ts, const EncodeParams& p, float* lds) {
  const int w = wave_index(), lane = threadIdx.x & 63;
  const int slab = blockIdx.x - ts.item_begin;
  const int chunk0 = slab * kVecChunksPerItem + w * kVecChunksPerWave;  // this wave's first chunk
  const int64_t first = int64_t(chunk0) * kS + lane;  // column layout: x[r] = element first + 64 r
  const int64_t rem = int64_t(ts.rows) - first;       // element r exists iff 64 r < rem
  float* __restrict__ m = ts.dst + first;
  const char* __restrict__ g = static_cast<const char*>(ts.aux) + first * (kBf16 ? 2 : 4);

  float x[64];
#pragma unroll
  for (int r = 0; r < 64; ++r) {
    float gv = 0.f, mv = 0.f;
    if (r * 64 < rem) {
      gv = load_src<kBf16>(g, r * 64);
      mv = stream_load(&m[r * 64]);
    }
    x[r] = fmaf(p.beta, mv, p.gcoef * gv);
  }
  if (!p.subtract_local) {
#pragma unroll
    for (int r = 0; r < 64; ++r) {
      if (r * 64 < rem) stream_store(x[r], &m[r * 64]);
    }
  }
  float* tile = lds + w * kTile;
  col_to_row(tile, x, lane);  // lane 2g + h: positions 64h + e of chunk g
  const int h = lane & 1;
  pair_butterfly(x, h);
  fwd_half(x, h);  // lane h: coefficients 2m + h

  const int chunk = chunk0 + (lane >> 1);
  const int nchunks = int((uint32_t(ts.rows) + 127u) >> 7);
  const bool live = chunk < nchunks;
  const int64_t e0 = ts.entry_begin + int64_t(live ? chunk : 0) * p.keff1;
  topk_pair(x, p.keff1, h, live, p.pay_val + e0, p.pay_idx + e0);
  if (!p.subtract_local) return;

  inv_half(x, h);  // R = P^T q_hat per chunk
  pair_unbutterfly(x, h);
  row_to_col(tile, x, lane);
#pragma unroll
  for (int r = 0; r < 64; ++r) {
    if (r * 64 < rem) {
      const float mp = fmaf(p.beta, stream_load(&m[r * 64]), p.gcoef * load_src<kBf16>(g, r * 64));  // M' again
      stream_store(fmaf(-p.alpha, x[r], mp), &m[r * 64]);
    }
  }
}

// kSmallK: every matrix chunk keeps at most 64 coefficients (keff2 <= 64),
// the common case; the lossless branch is then compiled out, which keeps the
// kernel within 256 VGPRs while it holds M' (two workgroups per CU).
template <bool kBf16, bool kSmallK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void encode128_kernel(LaunchTable tab,
                                                                                               EncodeParams p) {
  __shared__ __align__(16) uint32_t lds[kEncLdsWords];
  const TensorSlot& ts = tab.t[find_tensor(tab, blockIdx.x)];
  if (ts.cols == 0)
    encode_vector128<kBf16>(ts, p, reinterpret_cast<float*>(lds));
  else
    encode_matrix128<kBf16, kSmallK>(ts, p, reinterpret_cast<float*>(lds), lds + kTilesWords);
}

// ---------------------------------------------------------------- decode

// Per-wave sub-block accumulator (wave w = 2a + b owns the coefficients
// (2u + a, 2v + b)): its 20 KB quarter of the decode LDS holds the sum of
// (u, v) at v*64 + u and its 8-bit count in byte v & 3 of word
// 4096 + (v >> 2)*64 + u.  Stored transposed, so that lane u reads its row
// at constant offsets from one address, lanes on distinct banks.
constexpr int kQWords = kDecLdsWords / 4;
static_assert(64 * 64 + 64 * 16 <= kQWords && kTile <= kQWords, "sub-block accumulator and tile in a quarter");
__device__ __forceinline__ void accumulate_sub(float* acc, uint32_t* cntw, uint32_t u, uint32_t v, float x) {
  scatter_add_nowait(&acc[v * 64 + u], &cntw[(v >> 2) * 64 + u], v & 3u, x);
}
// the sub-block (wave) of chunk coefficient id = r*128 + c
__device__ __forceinline__ int sub_of(uint32_t id) { return int(((id >> 6) & 2u) | (id & 1u)); }

// Quadrant q's rows of X (and, for the momentum-only target, of M) for the
// decode: clamped addresses, so every load is valid; clamped lanes are not
// stored.
template <int kTargets>
__device__ __forceinline__ void decode_rows128(float (&x)[64], float (&m)[64], const float* __restrict__ xp,
                                               const float* __restrict__ mp, int64_t ld, const Chunk128& c, int q,
                                               int lane, int col) {
  if (c.full && buf_rows_fit(kS, ld * 4)) {
    if constexpr ((kTargets & kToParams) != 0) load_quad_rows(x, xp, ld, q, lane);
    if constexpr (kTargets == kToMomentum) load_quad_rows(m, mp, ld, q, lane);
  } else if (c.full) {
    const int64_t o = quad_origin(q, lane, ld), step = quad_step(q, ld);
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      if constexpr ((kTargets & kToParams) != 0) x[i] = stream_load(&xp[o + i * step]);
      if constexpr (kTargets == kToMomentum) m[i] = stream_load(&mp[o + i * step]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      const int64_t off = int64_t(min(quad_row(q >> 1, i), c.vr - 1)) * ld + col;
      if constexpr ((kTargets & kToParams) != 0) x[i] = stream_load(&xp[off]);
      if constexpr (kTargets == kToMomentum) m[i] = stream_load(&mp[off]);
    }
  }
}

// Entry f of worker w's payload: the float32 arrays, or the compact wire
// format (bfloat16 value in the high half of a float; 14-bit position).
template <bool kWire>
__device__ __forceinline__ void load_entry128(const DecodeParams& p, int64_t w, int64_t f, float& v, uint32_t& ix) {
  if constexpr (kWire) {
    v = __uint_as_float(uint32_t(p.wire_val[w * p.entries + f]) << 16);
    ix = WireFormat<14>::index(p.wire_idx + w * p.wire_words, f);
  } else {
    v = p.pay_val[w * p.entries + f];
    ix = p.pay_idx[w * p.entries + f];
  }
}

template <int kTargets, bool kWire>
__device__ __forceinline__ void decode_matrix128(const TensorSlot& ts, const DecodeParams& p, uint32_t* lds) {
  const int w = wave_index(), lane = threadIdx.x & 63;
  const int a = w >> 1, b = w & 1;
  const Chunk128 c = chunk_pos128(ts, blockIdx.x);

  // Every wave requests all payload entries of the chunk first and then its
  // quadrant's rows of X (of M for the momentum-only target), which land
  // during the scatter and the inverse passes.  Every load is unconditional
  // (clamped addresses), so no wait is placed between the two groups and the
  // payloads, issued first, arrive first.  With both X and M to update, the
  // momentum rows follow the exchange (registers).
  const int64_t e0 = ts.entry_begin + int64_t(c.local) * p.keff2;
  const bool one_batch = p.keff2 <= 64 && p.workers <= kWorkerBatch;
  float val[kWorkerBatch];
  uint32_t ix[kWorkerBatch];
  {
    const uint32_t e = uint32_t(min(lane, p.keff2 - 1));
#pragma unroll
    for (int j = 0; j < kWorkerBatch; ++j) {
      if constexpr (kWire) {
        load_entry128<true>(p, min(j, p.workers - 1), e0 + e, val[j], ix[j]);
      } else {
        const int64_t w0 = int64_t(min(j, p.workers - 1)) * p.entries + e0;
        val[j] = (p.pay_val + w0)[e];
        ix[j] = (p.pay_idx + w0)[e];
      }
    }
  }
  const int64_t ld = ts.cols;
  float* __restrict__ xp = ts.dst + c.base;
  float* __restrict__ mp = static_cast<float*>(ts.aux) + c.base;
  const int col = min((w & 1) ? kS - 1 - lane : lane, c.vc - 1);
  float x[64], m[64];
  decode_rows128<kTargets>(x, m, xp, mp, ld, c, w, lane, col);

  // Each wave scatters the entries of its own sub-block into its own quarter
  // of the LDS, in worker order 0..W-1 (a fixed summation order), and reads
  // the averages back: no workgroup barrier until the transposes.
  uint32_t* my = lds + w * kQWords;
  float* acc = reinterpret_cast<float*>(my);
  uint32_t* cntw = my + 64 * 64;
  {
    uint4* l4 = reinterpret_cast<uint4*>(my);
    const uint4 z = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int i = 0; i < kQWords / (64 * 4); ++i) l4[i * 64 + lane] = z;
  }
  wave_sync();
  if (one_batch) {
#pragma unroll
    for (int j = 0; j < kWorkerBatch; ++j) {
      const uint32_t id = ix[j] & 16383u;
      if (lane < p.keff2 && j < p.workers && sub_of(id) == w) accumulate_sub(acc, cntw, id >> 8, (id & 127u) >> 1, val[j]);
    }
  } else {
    // (worker, 64-entry block) steps worker-major, kWorkerBatch loads at a
    // time: every entry of worker wk is added before any of worker wk + 1
    const int nb = (p.keff2 + 63) >> 6;
    const int steps = p.workers * nb;
    int wk = 0, eb = 0;
    for (int t0 = 0; t0 < steps; t0 += kWorkerBatch) {
      float v2[kWorkerBatch];
      uint32_t i2[kWorkerBatch];
      bool on[kWorkerBatch];
#pragma unroll
      for (int j = 0; j < kWorkerBatch; ++j) {
        const int e = eb * 64 + lane;
        on[j] = t0 + j < steps && e < p.keff2;
        v2[j] = 0.f;
        i2[j] = 0u;
        if (on[j]) load_entry128<kWire>(p, wk, e0 + e, v2[j], i2[j]);
        if (++eb == nb) {
          eb = 0;
          ++wk;
        }
      }
#pragma unroll
      for (int j = 0; j < kWorkerBatch; ++j) {
        const uint32_t id = i2[j] & 16383u;
        if (on[j] && sub_of(id) == w) accumulate_sub(acc, cntw, id >> 8, (id & 127u) >> 1, v2[j]);
      }
    }
  }
  wave_sync();

  // this wave's sub-block (a, b) in row layout: lane u, q[v] = Q_bar[2u+a][2v+b]
  float q[64];
  if (p.avg_workers) {
#pragma unroll
    for (int v = 0; v < 64; ++v) q[v] = acc[v * 64 + lane] * p.inv_workers;
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) {  // one count word covers v = 4j .. 4j + 3
      const uint32_t cw = cntw[j * 64 + lane];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        // n == 0: no worker sent the coefficient and its sum is 0 as well
        const float n = float((cw >> (8 * t)) & 255u);
        q[4 * j + t] = acc[(4 * j + t) * 64 + lane] * __builtin_amdgcn_rcpf(fmaxf(n, 1.f));
      }
    }
  }
  wave_sync();  // the quarter is reused as this wave's transpose tile
  inv_half(q, b);
  row_to_col(reinterpret_cast<float*>(my), q, lane);
  inv_half(q, a);
  if constexpr (kTargets == (kToParams | kToMomentum))
    butterfly_staged(q, reinterpret_cast<float*>(lds), w, lane);  // -> M* of quadrant w
  else
    butterfly<false>(q, reinterpret_cast<float*>(lds), w, lane);  // the LDS is not used again

  if constexpr ((kTargets & kToSigns) != 0) {
    // Chunk row r's sign bits fill words 2r (columns 0..63) and 2r + 1
    // (64..127), bit = column within the half.  Quadrant row i is chunk row
    // r(i) = quad_row(a, i) and half b; in the second column half lane j holds
    // column 127 - j, bit 63 - j, so the ballot is bit-reversed.  Row i's word
    // goes into lane i, which stores it; rows and columns past the chunk's
    // valid ones give 0 bits.
    const int colq = b ? kS - 1 - lane : lane;
    const uint64_t cols = __builtin_amdgcn_ballot_w64(colq < c.vc);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      uint64_t bb = quad_row(a, i) < c.vr ? __builtin_amdgcn_ballot_w64(q[i] < 0.f) & cols : 0ull;
      bb = b ? __builtin_bitreverse64(bb) : bb;
      write_lane(lo, uint32_t(bb), i);
      write_lane(hi, uint32_t(bb >> 32), i);
    }
    const uint64_t word = (uint64_t(hi) << 32) | lo;
    stream_store(word, static_cast<uint64_t*>(ts.aux) + int64_t(c.local) * 256 + 2 * quad_row(a, lane) + b);
  }
  if constexpr ((kTargets & kToParams) != 0) {
    update_all(x, q, p);
    if (c.full)
      store_quadrant<true>(x, xp, ld, c, w, lane);
    else
      store_quadrant<false>(x, xp, ld, c, w, lane);
  }
  if constexpr ((kTargets & kToMomentum) != 0) {  // aggregated subtraction: M = M - alpha M*
    if constexpr (kTargets != kToMomentum) {
      if (c.full && buf_rows_fit(kS, ld * 4)) {
        load_quad_rows(m, mp, ld, w, lane);
      } else if (c.full) {
        const int64_t o = quad_origin(w, lane, ld), step = quad_step(w, ld);
#pragma unroll
        for (int i = 0; i < 64; ++i) m[i] = stream_load(&mp[o + i * step]);
      } else {
#pragma unroll
        for (int i = 0; i < 64; ++i) m[i] = stream_load(&mp[int64_t(min(quad_row(w >> 1, i), c.vr - 1)) * ld + col]);
      }
    }
#pragma unroll
    for (int i = 0; i < 64; ++i) m[i] = fmaf(-p.alpha, q[i], m[i]);
    if (c.full)
      store_quadrant<true>(m, mp, ld, c, w, lane);
    else
      store_quadrant<false>(m, mp, ld, c, w, lane);
  }
}

// Vector item: each wave owns 32 chunks and its own quarter of the LDS:
// accumulator (chunk g, coefficient c) at c*32 + g, counts in byte c & 3 of
// word (c >> 2)*32 + g (transposed: lane 2g + h reads its coefficients
// 2m + h at constant offsets, lanes on distinct banks).
template <int kTargets, bool kWire>
__device__ __forceinline__ void decode_vector128(const TensorSlot& ts, const DecodeParams& p, uint32_t* lds) {
  const int w = wave_index(), lane = threadIdx.x & 63;
  constexpr int kWaveWords = kDecLdsWords / 4;
  static_assert(kVecChunksPerWave * kS + kVecChunksPerWave * kS / 4 <= kWaveWords && kTile <= kWaveWords,
                "per-wave vector LDS");
  uint32_t* my = lds + w * kWaveWords;
  float* acc = reinterpret_cast<float*>(my);
  uint32_t* cntw = my + kVecChunksPerWave * kS;
  const int slab = blockIdx.x - ts.item_begin;
  const int chunk0 = slab * kVecChunksPerItem + w * kVecChunksPerWave;
  const int nchunks = int((uint32_t(ts.rows) + 127u) >> 7);
  const int nc = max(0, min(kVecChunksPerWave, nchunks - chunk0));  // chunks of this wave
  const int64_t first = int64_t(chunk0) * kS + lane;
  const int64_t rem = int64_t(ts.rows) - first;

  uint4* l4 = reinterpret_cast<uint4*>(my);
  const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
  for (int i = 0; i < kWaveWords / 256; ++i) l4[i * 64 + lane] = z4;
  wave_sync();
  const int keff = p.keff1;
  const int n = nc * keff;
  const int64_t e0 = ts.entry_begin + int64_t(chunk0) * keff;
  for (int wk = 0; wk < p.workers; ++wk) {
    for (int f0 = 0; f0 < n; f0 += 64 * 8) {
      float vv[8];
      uint32_t ii[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int f = f0 + 64 * j + lane;
        vv[j] = 0.f;
        ii[j] = 0u;
        if (f < n) load_entry128<kWire>(p, wk, e0 + f, vv[j], ii[j]);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int f = f0 + 64 * j + lane;
        if (f < n) {
          const uint32_t g = uint32_t(f / keff), cc = ii[j] & 127u;
          scatter_add_nowait(&acc[cc * 32 + g], &cntw[(cc >> 2) * 32 + g], cc & 3u, vv[j]);
        }
      }
    }
  }
  wave_sync();
  const int h = lane & 1;
  const uint32_t g = uint32_t(lane >> 1);
  float y[64];  // lane h: coefficients 2m + h of chunk g
  const float* __restrict__ mine = acc + 32 * h + g;  // coefficient 2m + h at mine[64 m]
  if (p.avg_workers) {
#pragma unroll
    for (int m = 0; m < 64; ++m) y[m] = mine[64 * m] * p.inv_workers;
  } else {
#pragma unroll
    for (int m2 = 0; m2 < 32; ++m2) {
      const uint32_t cw = cntw[m2 * 32 + g];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const float n = float((cw >> (8 * (2 * t + h))) & 255u);
        y[2 * m2 + t] = mine[64 * (2 * m2 + t)] * __builtin_amdgcn_rcpf(fmaxf(n, 1.f));
      }
    }
  }
  wave_sync();
  inv_half(y, h);
  pair_unbutterfly(y, h);
  float (&x)[64] = y;
  row_to_col(reinterpret_cast<float*>(my), x, lane);  // column layout: x[r] = M* at element first + 64 r

  if constexpr ((kTargets & kToSigns) != 0) {
    // A 128-element chunk's signs are two words (its elements 0..63 and
    // 64..127), so this wave's 32 chunks own words 2 chunk0 + r, r < 64:
    // word r covers elements chunk0 * 128 + 64 r + j, which is x[r] of lane
    // j.  Only the words of existing chunks are stored.
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int r = 0; r < 64; ++r) {
      const uint64_t bb = __builtin_amdgcn_ballot_w64(r * 64 < rem && x[r] < 0.f);
      write_lane(lo, uint32_t(bb), r);
      write_lane(hi, uint32_t(bb >> 32), r);
    }
    if (lane < 2 * nc)
      stream_store((uint64_t(hi) << 32) | lo, static_cast<uint64_t*>(ts.aux) + int64_t(chunk0) * 2 + lane);
  }
  if constexpr ((kTargets & kToParams) != 0) {
    update_strided(ts.dst + first, x, rem, p);
  }
  if constexpr ((kTargets & kToMomentum) != 0) {
    float* __restrict__ mp = static_cast<float*>(ts.aux) + first;
#pragma unroll
    for (int r = 0; r < 64; ++r) {
      if (r * 64 < rem) stream_store(fmaf(-p.alpha, x[r], stream_load(&mp[r * 64])), &mp[r * 64]);
    }
  }
}

template <int kTargets, bool kWire = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void decode128_kernel(LaunchTable tab,
                                                                                               DecodeParams p) {
  __shared__ __align__(16) uint32_t lds[kDecLdsWords];
  const TensorSlot& ts = tab.t[find_tensor(tab, blockIdx.x)];
  if (ts.cols == 0)
    decode_vector128<kTargets, kWire>(ts, p, lds);
  else
    decode_matrix128<kTargets, kWire>(ts, p, lds);
}

// ---------------------------------------------------------------- one-bit sign apply

// X = X - eta (s + lambda X), s = -1 where the element's bit is set, else +1.
// A workgroup (four waves) takes one 128x128 chunk, wave 2 rb + h its 64x64
// sub-block of rows 64 rb .. and columns 64 h ..: chunk row r's bit for
// column 64 h + j is bit j of word 2 r + h.  Or, for a vector, 128 chunks,
// wave w the 64 words of elements 4096 w .. 4096 w + 4095 of the item (word
// = 64 consecutive elements, as at chunk edge 64).  Words arrive through
// wave-uniform (scalar) loads.
__global__ __launch_bounds__(256) void apply_signs128_kernel(LaunchTable tab, ApplyParams p) {
  const TensorSlot& ts = tab.t[find_tensor(tab, blockIdx.x)];
  const int w = wave_index(), lane = threadIdx.x & 63;
  const uint64_t* __restrict__ words = static_cast<const uint64_t*>(ts.aux);
  if (ts.cols == 0) {
    const int slab = blockIdx.x - ts.item_begin;
    const int64_t base = int64_t(slab) * kVecChunksPerItem * kS + int64_t(w) * 64 * 64;  // the wave's first element
    const int64_t nwords = 2 * ((int64_t(ts.rows) + kS - 1) / kS);                        // words of the tensor
    const int64_t rem = int64_t(ts.rows) - (base + lane);
    float* __restrict__ x = ts.dst + base + lane;
    for (int c = 0; c < 64 && base / 64 + c < nwords; ++c) {
      const uint64_t wd = words[base / 64 + c];
      if (c * 64 < rem) {
        const float s = ((wd >> lane) & 1u) ? -1.f : 1.f;
        const float xv = stream_load(&x[c * 64]);
        stream_store(fmaf(-p.eta, fmaf(p.lam, xv, s), xv), &x[c * 64]);
      }
    }
    return;
  }
  const Chunk128 c = chunk_pos128(ts, blockIdx.x);
  const int rb = w >> 1, h = w & 1;
  const int vr = min(64, c.vr - 64 * rb), vc = min(64, c.vc - 64 * h);  // valid rows / columns of the sub-block
  if (vr <= 0 || vc <= 0) return;
  const uint64_t* __restrict__ wp = words + int64_t(c.local) * 256 + 2 * 64 * rb + h;
  const int64_t ld = ts.cols;
  float* __restrict__ xp = ts.dst + c.base + int64_t(64 * rb) * ld + 64 * h;
  // all 64 rows are requested before the first store (a store may alias a
  // later row as far as the compiler knows, so loads are not moved past it)
  float x[64];
  const bool full = vr == 64 && vc == 64 && buf_rows_fit(64, ld * 4);
  const int col = min(lane, vc - 1);
  if (full) {
    const RowBuf b = row_buf(xp, ld * 4);
#pragma unroll
    for (int i = 0; i < 64; ++i) x[i] = buf_load_f32(b, i, lane * 4);
  } else {
#pragma unroll
    for (int i = 0; i < 64; ++i) x[i] = stream_load(&xp[min(i, vr - 1) * ld + col]);
  }
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    const float s = ((wp[2 * i] >> lane) & 1u) ? -1.f : 1.f;
    x[i] = fmaf(-p.eta, fmaf(p.lam, x[i], s), x[i]);
  }
  if (full) {
    const RowBuf b = row_buf(xp, ld * 4);
#pragma unroll
    for (int i = 0; i < 64; ++i) buf_store_f32(b, i, lane * 4, x[i]);
  } else {
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      if (lane < vc && i < vr) stream_store(x[i], &xp[i * ld + lane]);
    }
  }
}

}  // namespace

hipError_t launch_encode128(const LaunchTable& tab, const EncodeParams& p, bool g_bf16, hipStream_t stream) {
  if (tab.items <= 0) return hipSuccess;
  const dim3 grid(tab.items), block(256);
  const bool small = p.keff2 <= 64;
  if (g_bf16 && small)
    encode128_kernel<true, true><<<grid, block, 0, stream>>>(tab, p);
  else if (g_bf16)
    encode128_kernel<true, false><<<grid, block, 0, stream>>>(tab, p);
  else if (small)
    encode128_kernel<false, true><<<grid, block, 0, stream>>>(tab, p);
  else
    encode128_kernel<false, false><<<grid, block, 0, stream>>>(tab, p);
  return hipGetLastError();
}

hipError_t launch_decode128(const LaunchTable& tab, const DecodeParams& p, hipStream_t stream) {
  if (tab.items <= 0) return hipSuccess;
  const dim3 grid(tab.items), block(256);
  if (p.wire)
    decode128_kernel<kToParams, true><<<grid, block, 0, stream>>>(tab, p);
  else if (p.pack_signs)
    decode128_kernel<kToSigns><<<grid, block, 0, stream>>>(tab, p);
  else if (p.update_x && p.update_m)
    decode128_kernel<kToParams | kToMomentum><<<grid, block, 0, stream>>>(tab, p);
  else if (p.update_m)
    decode128_kernel<kToMomentum><<<grid, block, 0, stream>>>(tab, p);
  else
    decode128_kernel<kToParams><<<grid, block, 0, stream>>>(tab, p);
  return hipGetLastError();
}

hipError_t launch_apply_signs128(const LaunchTable& tab, const ApplyParams& p, hipStream_t stream) {
  if (tab.items <= 0) return hipSuccess;
  apply_signs128_kernel<<<dim3(tab.items), dim3(256), 0, stream>>>(tab, p);
  return hipGetLastError();
}

}  // namespace demo
