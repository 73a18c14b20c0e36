// HIP kernels of the DeMo per-step momentum codec for CDNA4 (gfx950).
//
// One launch covers a batch of tensors of both kinds.  A work item is one
// 64x64 chunk of a matrix, or one slab of up to 64 consecutive 64-element
// chunks of a vector; the host puts the vector slabs first so their longer,
// serial lanes start early and finish under the matrix chunks.  One wave64
// owns one item.
//
// Data move between two register layouts:
//   column layout: lane j holds column j, x[i] = element (i, j);
//   row layout:    lane u holds row u,    x[v] = element (u, v).
// A coalesced global access of one 256-byte row segment per instruction
// fills the column layout directly; a 64x65-float LDS tile (row stride 65:
// row and column accesses are both bank-conflict free) converts between the
// two.  Each 64-point transform runs inside one lane's registers.  G, M and X
// are streamed once, so their loads and stores carry the non-temporal hint.
//
// encode (DeMo summary, §3.4 Decoupled Local Momentum Updates, Tensor
// Chunking, Blockwise Linear Projection, Top-k Sparsification, Momentum
// Subtraction):
//   load G, M -> M' = beta M + c G (registers, column layout)
//   Q = P0 M' P1^T  (column pass, LDS transpose, row pass)
//   exact top-k of |Q| over the chunk, lower index wins ties; payload
//   (value, index) in index order
//   R = P0^T Q_hat P1 (row pass, LDS transpose, column pass);
//   M = M' - alpha R, with M' held in registers since the load (vector
//   chunks under a caller basis, whose per-lane products need the registers,
//   load G and M again and form M' bit for bit).  Only the selected part goes
//   through the float32 transforms, so the rounding of the rest of M' does
//   not accumulate in the momentum from step to step.
// decode/apply (§3.4 Server-Side Aggregation, Inverse DCT and Unchunking,
// Base Optimizer Update):
//   scatter-add W payloads into an LDS accumulator with 8-bit contributor
//   counts, atomic-free: one load-add-store per worker in worker order
//   0..W-1 (indices are distinct within one payload, so the lanes of one
//   step never collide and the sum order is fixed); average;
//   M* = P0^T Q_bar P1; X = X - eta (phi(M*) + lambda X).
#include "common.h"
#include "launch.h"
#include "topk.h"
#include "xform.h"

namespace demo {
namespace {

using xf::DctBasis;
using xf::DenseBasis;
using xf::IdentityBasis;

constexpr int kLd = 65;     // LDS tile row stride in floats
constexpr int kCntLd = 15;  // count rows: words 0..14 of a row's 8-bit counts (word 15: see count_word)
constexpr int kWorkerBatch = 16;


// Every workgroup here is one wave: LDS accesses are ordered with wave_sync,
// not with workgroup barriers.

// column layout -> row layout through the LDS tile
__device__ __forceinline__ void col_to_row(float* tile, float (&x)[64], int lane) {
#pragma unroll
  for (int i = 0; i < 64; ++i) tile[i * kLd + lane] = x[i];
  wave_sync();
#pragma unroll
  for (int v = 0; v < 64; ++v) x[v] = tile[lane * kLd + v];
  wave_sync();
}

// row layout -> column layout through the LDS tile
__device__ __forceinline__ void row_to_col(float* tile, float (&x)[64], int lane) {
#pragma unroll
  for (int v = 0; v < 64; ++v) tile[lane * kLd + v] = x[v];
  wave_sync();
#pragma unroll
  for (int i = 0; i < 64; ++i) x[i] = tile[i * kLd + lane];
  wave_sync();
}

struct ChunkPos {
  int local;     // chunk ordinal within its tensor
  int vr, vc;    // valid rows / columns of the chunk
  int64_t base;  // element offset of the chunk's (0, 0)
  bool full;
};

__device__ __forceinline__ ChunkPos chunk_pos(const TensorSlot& ts, int item) {
  ChunkPos c;
  c.local = item - ts.item_begin;
  const int grid1 = int((uint32_t(ts.cols) + 63u) >> 6);  // chunks along dimension 1
  const int cr = c.local / grid1;
  const int cc = c.local - cr * grid1;
  c.vr = min(64, ts.rows - cr * 64);
  c.vc = min(64, ts.cols - cc * 64);
  c.base = int64_t(cr) * 64 * ts.cols + int64_t(cc) * 64;
  c.full = (c.vr == 64) && (c.vc == 64);
  return c;
}

template <bool kFull>
__device__ __forceinline__ void store_rows(const float (&q)[64], float* __restrict__ dst, int64_t ld,
                                           const ChunkPos& c, int lane) {
  if (kFull && buf_rows_fit(64, ld * 4)) {
    const RowBuf b = row_buf(dst, ld * 4);
#pragma unroll
    for (int i = 0; i < 64; ++i) buf_store_f32(b, i, lane * 4, q[i]);
    return;
  }
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    if (kFull || (lane < c.vc && i < c.vr)) stream_store(q[i], &dst[i * ld + lane]);
  }
}

// Rows 0..63 of a full chunk at src (row stride ld), lane = column.
__device__ __forceinline__ void load_rows_full(float (&x)[64], const float* __restrict__ src, int64_t ld, int lane) {
  if (buf_rows_fit(64, ld * 4)) {
    const RowBuf b = row_buf(src, ld * 4);
#pragma unroll
    for (int i = 0; i < 64; ++i) x[i] = buf_load_f32(b, i, lane * 4);
  } else {
#pragma unroll
    for (int i = 0; i < 64; ++i) x[i] = stream_load(&src[i * ld + lane]);
  }
}

// ---------------------------------------------------------------- encode, 64x64 chunk

template <bool kFull, bool kBf16>
__device__ __forceinline__ void load_momentum(float (&q)[64], const TensorSlot& ts, const ChunkPos& c, int lane,
                                              float beta, float gcoef) {
  const int64_t ld = ts.cols;
  const float* __restrict__ m = ts.dst + c.base;
  const char* __restrict__ g = static_cast<const char*>(ts.aux) + c.base * (kBf16 ? 2 : 4);
  if (kFull && buf_rows_fit(64, ld * 4)) {
    const RowBuf bm = row_buf(m, ld * 4), bg = row_buf(g, ld * (kBf16 ? 2 : 4));
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      const float gv = kBf16 ? buf_load_bf16(bg, i, lane * 2) : buf_load_f32(bg, i, lane * 4);
      q[i] = fmaf(beta, buf_load_f32(bm, i, lane * 4), gcoef * gv);
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    float gv = 0.f, mv = 0.f;
    if (kFull || (lane < c.vc && i < c.vr)) {
      gv = load_src<kBf16>(g, i * ld + lane);
      mv = stream_load(&m[i * ld + lane]);
    }
    q[i] = fmaf(beta, mv, gcoef * gv);
  }
}

template <class Basis, bool kBf16>
__device__ __forceinline__ void encode_matrix(const TensorSlot& ts, const EncodeParams& p, const Basis& basis,
                                              float* tile, int item) {
  const int lane = threadIdx.x;
  const ChunkPos c = chunk_pos(ts, item);

  float q[64];
  if (c.full)
    load_momentum<true, kBf16>(q, ts, c, lane, p.beta, p.gcoef);
  else
    load_momentum<false, kBf16>(q, ts, c, lane, p.beta, p.gcoef);
  if (!p.subtract_local) {  // aggregated subtraction: M = M' now, the decode side subtracts
    if (c.full)
      store_rows<true>(q, ts.dst + c.base, ts.cols, c, lane);
    else
      store_rows<false>(q, ts.dst + c.base, ts.cols, c, lane);
  }
  float mp[64];  // M' (column layout), held for the subtraction
#pragma unroll
  for (int i = 0; i < 64; ++i) mp[i] = q[i];

  if constexpr (Basis::kMatrixCores) {
    basis.template forward2d<kLd>(q, tile, lane);
  } else {
    basis.fwd0(q);
    col_to_row(tile, q, lane);
    basis.fwd1(q);
  }

  const int64_t e0 = ts.entry_begin + int64_t(c.local) * p.keff2;
  tk::topk_chunk(q, p.keff2, lane, p.pay_val + e0, p.pay_idx + e0, reinterpret_cast<uint32_t*>(tile),
                 tile + lane * kLd);
  if (!p.subtract_local) return;
  wave_sync();

  // q holds Q_hat (row layout); R = P0^T Q_hat P1 in column layout
  if constexpr (Basis::kMatrixCores) {
    basis.template inverse2d<kLd>(q, tile, lane);
  } else {
    basis.inv1(q);
    row_to_col(tile, q, lane);
    basis.inv0(q);
  }

#pragma unroll
  for (int i = 0; i < 64; ++i) q[i] = fmaf(-p.alpha, q[i], mp[i]);  // M = M' - alpha R
  if (c.full)
    store_rows<true>(q, ts.dst + c.base, ts.cols, c, lane);
  else
    store_rows<false>(q, ts.dst + c.base, ts.cols, c, lane);
}

// ---------------------------------------------------------------- encode, vector slab

// Slab view of a vector: V[c][e] = vec[(64 * slab + c) * 64 + e], chunk c of
// the slab is row c.  Column layout after the load (lane e), row layout
// (lane c = one chunk) after the transpose; each lane then transforms and
// selects its own chunk.
template <class Basis, bool kBf16>
__device__ __forceinline__ void encode_vector(const TensorSlot& ts, const EncodeParams& p, const Basis& basis,
                                              float* tile, int item) {
  const int lane = threadIdx.x;
  const int slab = item - ts.item_begin;
  const int64_t first = int64_t(slab) * 64 * 64 + lane;  // this lane's element of the slab's chunk 0
  const int64_t rem = int64_t(ts.rows) - first;          // elements c * 64 < rem exist
  float* __restrict__ m = ts.dst + first;
  const char* __restrict__ g = static_cast<const char*>(ts.aux) + first * (kBf16 ? 2 : 4);

  // M' is held for the subtraction, except with the caller basis (whose
  // per-lane products need the registers), which forms it again at the end.
  constexpr bool kHold = !Basis::kMatrixCores;
  float q[64], mp[kHold ? 64 : 1];
#pragma unroll
  for (int c = 0; c < 64; ++c) {
    float gv = 0.f, mv = 0.f;
    if (c * 64 < rem) {
      gv = load_src<kBf16>(g, c * 64);
      mv = stream_load(&m[c * 64]);
    }
    q[c] = fmaf(p.beta, mv, p.gcoef * gv);
    if constexpr (kHold) mp[c] = q[c];
  }
  if (!p.subtract_local) {  // aggregated subtraction: M = M' now, the decode side subtracts
#pragma unroll
    for (int c = 0; c < 64; ++c) {
      if (c * 64 < rem) stream_store(q[c], &m[c * 64]);
    }
  }
  col_to_row(tile, q, lane);
  basis.fwd0(q);

  const int chunk = slab * 64 + lane;  // this lane's chunk within the tensor
  const bool live = chunk < int((uint32_t(ts.rows) + 63u) >> 6);
  const int64_t e0 = ts.entry_begin + int64_t(live ? chunk : 0) * p.keff1;
  tk::topk_lane(q, p.keff1, live, p.pay_val + e0, p.pay_idx + e0);
  if (!p.subtract_local) return;

  basis.inv0(q);  // R = P0^T q_hat per chunk
  row_to_col(tile, q, lane);
#pragma unroll
  for (int c = 0; c < 64; ++c) {
    if (c * 64 < rem) {
      float mc;
      if constexpr (kHold)
        mc = mp[c];
      else
        mc = fmaf(p.beta, stream_load(&m[c * 64]), p.gcoef * load_src<kBf16>(g, c * 64));  // M' again
      stream_store(fmaf(-p.alpha, q[c], mc), &m[c * 64]);
    }
  }
}

template <class Basis, bool kBf16>
__device__ __forceinline__ void encode_item(const LaunchTable& tab, const EncodeParams& p, const Basis& basis,
                                            float* tile) {
  const int item = xcd_item(blockIdx.x, gridDim.x);
  const TensorSlot& ts = tab.t[find_tensor(tab, item)];
  if (ts.cols == 0)
    encode_vector<Basis, kBf16>(ts, p, basis, tile, item);
  else
    encode_matrix<Basis, kBf16>(ts, p, basis, tile, item);
}

// The DCT and identity kernels hold M' next to the block: up to 256 VGPRs,
// two waves per SIMD (eight per CU; the 16.6 KB LDS tile alone allows nine).
template <class Basis, bool kBf16>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void encode_kernel(LaunchTable tab,
                                                                                             EncodeParams p) {
  __shared__ float tile[64 * kLd];
  encode_item<Basis, kBf16>(tab, p, Basis{}, tile);
}

template <bool kBf16>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void encode_dense_kernel(LaunchTable tab, EncodeParams p, DenseBasis basis) {
  __shared__ float tile[64 * kLd];
  encode_item<DenseBasis, kBf16>(tab, p, basis, tile);
}

// ---------------------------------------------------------------- decode / apply

// The decode's LDS: the 64 x kLd fp32 accumulator, then 64 x kCntLd words of
// 8-bit counts; the 16th count word of row u sits in the accumulator row's
// padding slot (column 64, which no transform touches).  20 KB: eight waves
// per CU.
constexpr int kDecodeLdsWords = 64 * kLd + 64 * kCntLd;
static_assert(kDecodeLdsWords % 256 == 0 && kDecodeLdsWords * 4 == 20480, "cleared in whole 16-byte stores");
// The decode that updates both X and M streams twice the bytes per chunk and
// ran 1 % faster with seven waves per CU: its allocation is 1 KB larger
// (unused) to keep it there.
template <int kTargets>
constexpr int decode_lds_words() {
  return kTargets == (kToParams | kToMomentum) ? kDecodeLdsWords + 256 : kDecodeLdsWords;
}

// Count word j (counts of columns 4j .. 4j + 3) of row u.  Rows of 15 words
// and the padding slots both put 64 lanes' reads of their own rows on 64
// banks (15 u and 65 u are distinct mod 64).
template <class F, class W>
__device__ __forceinline__ W* count_word(F* acc, W* cntw, uint32_t u, uint32_t j) {
  return j < 15u ? cntw + u * kCntLd + j : reinterpret_cast<W*>(acc + u * kLd + 64);
}

// Zero the accumulator tile and the count rows: unguarded 16-byte stores.
__device__ __forceinline__ void clear_acc(uint32_t* lds, int lane) {
  uint4* l4 = reinterpret_cast<uint4*>(lds);
  const uint4 z = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
  for (int i = 0; i < kDecodeLdsWords / 256; ++i) l4[i * 64 + lane] = z;
}

// Add one payload entry (value v at coefficient (u, col)) to the accumulator
// and to its 8-bit contributor count (byte col of count row u).
__device__ __forceinline__ void accumulate(float* acc, uint32_t* cntw, uint32_t u, uint32_t col, float v) {
  scatter_add(acc + u * kLd + col, reinterpret_cast<uint8_t*>(count_word(acc, cntw, u, col >> 2)) + (col & 3u), v);
}

// Entry f of worker w's payload: the float32 arrays, or the compact wire
// format (value = bfloat16 bits in the high half of a float; index = bits
// 12f .. 12f + 11 of the worker's little-endian word string, which may
// straddle two words of f's 8-entry, three-word group).
template <bool kWire>
__device__ __forceinline__ void load_entry(const DecodeParams& p, int64_t w, int64_t f, float& v, uint32_t& ix) {
  if constexpr (kWire) {
    v = __uint_as_float(uint32_t(p.wire_val[w * p.entries + f]) << 16);
    ix = WireFormat<12>::index(p.wire_idx + w * p.wire_words, f);
  } else {
    const int64_t off = w * p.entries + f;
    v = p.pay_val[off];
    ix = p.pay_idx[off];
  }
}

// Scatter-add the W payload segments of one 64x64 chunk (entries e0 ..
// e0 + keff of every worker).  The (worker, 64-entry block) steps run
// worker-major: every entry of worker w is added before any of worker w + 1,
// so each coefficient receives its terms in worker order 0..W-1.  Loads are
// issued kWorkerBatch steps at a time; inside one step the indices are
// distinct (one worker's payload), so no lanes collide.
template <bool kWire>
__device__ __forceinline__ void scatter_chunk(float* acc, uint32_t* cntw, const DecodeParams& p, int64_t e0,
                                              int lane) {
  const int keff = p.keff2;
  const int nb = (keff + 63) >> 6;  // entry blocks per worker
  const int steps = p.workers * nb;
  int w = 0, eb = 0;  // worker and block of step t0 (wave-uniform)
  for (int t0 = 0; t0 < steps; t0 += kWorkerBatch) {
    float val[kWorkerBatch];
    uint32_t ix[kWorkerBatch];
    bool on[kWorkerBatch];
#pragma unroll
    for (int j = 0; j < kWorkerBatch; ++j) {
      const int e = eb * 64 + lane;
      on[j] = t0 + j < steps && e < keff;
      val[j] = 0.f;
      ix[j] = 0u;
      if (on[j]) load_entry<kWire>(p, w, e0 + e, val[j], ix[j]);
      if (++eb == nb) {
        eb = 0;
        ++w;
      }
    }
#pragma unroll
    for (int j = 0; j < kWorkerBatch; ++j) {
      if (on[j]) {
        const uint32_t id = ix[j] & 4095u;
        accumulate(acc, cntw, id >> 6, id & 63u, val[j]);
      }
    }
  }
}

// Scatter-add the W payload segments of the nc <= 64 vector chunks of a slab
// (entries e0 .. e0 + nc * keff of every worker, chunk r of the slab into
// accumulator row r).  Entry f of a segment belongs to chunk f / keff; one
// instruction covers 64 consecutive entries of one worker, whose (chunk,
// index) pairs are distinct.
template <bool kWire>
__device__ __forceinline__ void scatter_slab(float* acc, uint32_t* cntw, const DecodeParams& p, int64_t e0, int nc,
                                             int lane) {
  const int keff = p.keff1;
  const int n = nc * keff;
  for (int w = 0; w < p.workers; ++w) {
    for (int f0 = 0; f0 < n; f0 += 64 * 8) {
      float val[8];
      uint32_t ix[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int f = f0 + 64 * j + lane;
        val[j] = 0.f;
        ix[j] = 0u;
        if (f < n) load_entry<kWire>(p, w, e0 + f, val[j], ix[j]);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int f = f0 + 64 * j + lane;
        if (f < n) accumulate(acc, cntw, uint32_t(f / keff), ix[j] & 63u, val[j]);
      }
    }
  }
}

// Row `lane` of the average into q (row layout).
__device__ __forceinline__ void average_row(float (&q)[64], const float* acc, const uint32_t* cntw,
                                            const DecodeParams& p, int lane) {
  if (p.avg_workers) {
#pragma unroll
    for (int v = 0; v < 64; ++v) q[v] = acc[lane * kLd + v] * p.inv_workers;
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t w = *count_word(acc, cntw, uint32_t(lane), uint32_t(j));
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const float n = float((w >> (8 * b)) & 255u);
        // n == 0 means no worker sent the coefficient; its sum is 0 as well
        q[4 * j + b] = acc[lane * kLd + 4 * j + b] * __builtin_amdgcn_rcpf(fmaxf(n, 1.f));
      }
    }
  }
}

template <class Basis, int kTargets, bool kWire>
__device__ __forceinline__ void decode_matrix(const TensorSlot& ts, const DecodeParams& p, const Basis& basis,
                                              float* acc, uint32_t* cntw, int item) {
  const int lane = threadIdx.x;
  const ChunkPos c = chunk_pos(ts, item);

  // Memory order matters: a wave's loads complete in issue order, so the
  // payload entries (needed first) are requested before the tensors to
  // update, which then land while the payloads are averaged and
  // inverse-transformed.  Both sets of loads are issued without branches
  // (addresses clamped into the valid range, results of clamped lanes
  // unused), so no wait separates them.
  const int64_t e0 = ts.entry_begin + int64_t(c.local) * p.keff2;
  const bool one_batch = p.keff2 <= 64 && p.workers <= kWorkerBatch;
  float val[kWorkerBatch];
  uint32_t ix[kWorkerBatch];
  if (one_batch) {
    // wave-uniform worker pointers plus a 32-bit lane index
    const uint32_t e = uint32_t(min(lane, p.keff2 - 1));
#pragma unroll
    for (int j = 0; j < kWorkerBatch; ++j) {
      if constexpr (kWire) {
        load_entry<true>(p, min(j, p.workers - 1), e0 + e, val[j], ix[j]);
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
  const uint32_t col = uint32_t(min(lane, c.vc - 1));
  // with both targets the momentum rows are fetched after the transforms
  // (registers: X, M and the transform together would halve occupancy)
  constexpr bool kEarlyM = kTargets == kToMomentum;
  // the matrix-core transform needs those registers too: there the parameter
  // rows follow the transform (a second wave per SIMD hides them instead)
  constexpr bool kEarlyX = !Basis::kMatrixCores;
  float x[64], m[64];
  if (c.full) {
    if constexpr ((kTargets & kToParams) != 0 && kEarlyX) load_rows_full(x, xp, ld, lane);
    if constexpr (kEarlyM) load_rows_full(m, mp, ld, lane);
  } else {
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      const int64_t row = int64_t(min(i, c.vr - 1)) * ld;
      if constexpr ((kTargets & kToParams) != 0 && kEarlyX) x[i] = stream_load(&(xp + row)[col]);
      if constexpr (kEarlyM) m[i] = stream_load(&(mp + row)[col]);
    }
  }

  clear_acc(reinterpret_cast<uint32_t*>(acc), lane);
  wave_sync();
  if (one_batch) {
#pragma unroll
    for (int j = 0; j < kWorkerBatch; ++j) {
      if (lane < p.keff2 && j < p.workers) {
        const uint32_t id = ix[j] & 4095u;
        accumulate(acc, cntw, id >> 6, id & 63u, val[j]);
      }
    }
  } else {
    scatter_chunk<kWire>(acc, cntw, p, e0, lane);
  }
  wave_sync();

  float q[64];
  average_row(q, acc, cntw, p, lane);
  wave_sync();
  if constexpr (Basis::kMatrixCores) {
    basis.template inverse2d<kLd>(q, acc, lane);
  } else {
    basis.inv1(q);
    row_to_col(acc, q, lane);
    basis.inv0(q);
  }

  if constexpr ((kTargets & kToParams) != 0) {
    if constexpr (!kEarlyX) {
      if (c.full) {
        load_rows_full(x, xp, ld, lane);
      } else {
#pragma unroll
        for (int i = 0; i < 64; ++i) x[i] = stream_load(&(xp + int64_t(min(i, c.vr - 1)) * ld)[col]);
      }
    }
    update_all(x, q, p);
    if (c.full)
      store_rows<true>(x, xp, ld, c, lane);
    else
      store_rows<false>(x, xp, ld, c, lane);
  }
  if constexpr ((kTargets & kToMomentum) != 0) {  // aggregated subtraction: M = M - alpha M*
    if constexpr (!kEarlyM) {
      if (c.full) {
        load_rows_full(m, mp, ld, lane);
      } else {
#pragma unroll
        for (int i = 0; i < 64; ++i) m[i] = stream_load(&(mp + int64_t(min(i, c.vr - 1)) * ld)[col]);
      }
    }
#pragma unroll
    for (int i = 0; i < 64; ++i) m[i] = fmaf(-p.alpha, q[i], m[i]);
    if (c.full)
      store_rows<true>(m, mp, ld, c, lane);
    else
      store_rows<false>(m, mp, ld, c, lane);
  }
  if constexpr ((kTargets & kToMstar) != 0) {
    float* __restrict__ sp = static_cast<float*>(ts.aux) + c.base;
    if (c.full)
      store_rows<true>(q, sp, ld, c, lane);
    else
      store_rows<false>(q, sp, ld, c, lane);
  }
  if constexpr ((kTargets & kToSigns) != 0) {
    // Row i of the chunk is one ballot (bit j = lane j = column j), written
    // into lane i (rows past the chunk's valid ones stay 0); the 64 words go
    // out as one coalesced 512-byte store.
    const uint64_t cols = __builtin_amdgcn_ballot_w64(lane < c.vc);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      const uint64_t b = i < c.vr ? __builtin_amdgcn_ballot_w64(q[i] < 0.f) & cols : 0ull;
      write_lane(lo, uint32_t(b), i);
      write_lane(hi, uint32_t(b >> 32), i);
    }
    const uint64_t word = (uint64_t(uint32_t(hi)) << 32) | uint32_t(lo);
    stream_store(word, static_cast<uint64_t*>(ts.aux) + int64_t(c.local) * 64 + lane);
  }
}

template <class Basis, int kTargets, bool kWire>
__device__ __forceinline__ void decode_vector(const TensorSlot& ts, const DecodeParams& p, const Basis& basis,
                                              float* acc, uint32_t* cntw, int item) {
  const int lane = threadIdx.x;
  const int slab = item - ts.item_begin;
  const int64_t first = int64_t(slab) * 64 * 64 + lane;  // this lane's element of the slab's chunk 0
  const int64_t rem = int64_t(ts.rows) - first;          // elements c * 64 < rem exist
  const int nc = min(64, int((uint32_t(ts.rows) + 63u) >> 6) - slab * 64);  // chunks in this slab

  clear_acc(reinterpret_cast<uint32_t*>(acc), lane);
  wave_sync();
  scatter_slab<kWire>(acc, cntw, p, ts.entry_begin + int64_t(slab) * 64 * p.keff1, nc, lane);
  wave_sync();
  float q[64];
  average_row(q, acc, cntw, p, lane);
  wave_sync();
  basis.inv0(q);
  row_to_col(acc, q, lane);

  if constexpr ((kTargets & kToParams) != 0) {
    update_strided(ts.dst + first, q, rem, p);
  }
  if constexpr ((kTargets & kToMomentum) != 0) {  // aggregated subtraction: M = M - alpha M*
    float* __restrict__ m = static_cast<float*>(ts.aux) + first;
#pragma unroll
    for (int c = 0; c < 64; ++c) {
      if (c * 64 < rem) stream_store(fmaf(-p.alpha, q[c], stream_load(&m[c * 64])), &m[c * 64]);
    }
  }
  if constexpr ((kTargets & kToMstar) != 0) {
    float* __restrict__ sp = static_cast<float*>(ts.aux) + first;
#pragma unroll
    for (int c = 0; c < 64; ++c) {
      if (c * 64 < rem) stream_store(q[c], &sp[c * 64]);
    }
  }
  if constexpr ((kTargets & kToSigns) != 0) {  // one word per vector chunk: chunk c's ballot goes to lane c
    uint64_t word = 0;
#pragma unroll
    for (int c = 0; c < 64; ++c) {
      const uint64_t b = __builtin_amdgcn_ballot_w64(c * 64 < rem && q[c] < 0.f);
      word = lane == c ? b : word;
    }
    if (lane < nc) stream_store(word, static_cast<uint64_t*>(ts.aux) + int64_t(slab) * 64 + lane);
  }
}

template <class Basis, int kTargets, bool kWire>
__device__ __forceinline__ void decode_item(const LaunchTable& tab, const DecodeParams& p, const Basis& basis,
                                            float* acc, uint32_t* cntw) {
  const int item = xcd_item(blockIdx.x, gridDim.x);
  const TensorSlot& ts = tab.t[find_tensor(tab, item)];
  if (ts.cols == 0)
    decode_vector<Basis, kTargets, kWire>(ts, p, basis, acc, cntw, item);
  else
    decode_matrix<Basis, kTargets, kWire>(ts, p, basis, acc, cntw, item);
}

template <class Basis, int kTargets, bool kWire = false>
__global__ __launch_bounds__(64) void decode_kernel(LaunchTable tab, DecodeParams p) {
  __shared__ __align__(16) uint32_t lds[decode_lds_words<kTargets>()];
  decode_item<Basis, kTargets, kWire>(tab, p, Basis{}, reinterpret_cast<float*>(lds), lds + 64 * kLd);
}

template <int kTargets, bool kWire = false>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void decode_dense_kernel(LaunchTable tab, DecodeParams p, DenseBasis basis) {
  __shared__ __align__(16) uint32_t lds[decode_lds_words<kTargets>()];
  decode_item<DenseBasis, kTargets, kWire>(tab, p, basis, reinterpret_cast<float*>(lds), lds + 64 * kLd);
}

template <int kTargets, bool kWire = false>
void launch_decode_targets(const LaunchTable& tab, const DecodeParams& p, BasisKind kind, const float* basis_p0,
                           const float* basis_p1, hipStream_t stream) {
  const dim3 grid(tab.items), block(64);
  switch (kind) {
    case BasisKind::kDct:
      decode_kernel<DctBasis, kTargets, kWire><<<grid, block, 0, stream>>>(tab, p);
      break;
    case BasisKind::kIdentity:
      decode_kernel<IdentityBasis, kTargets, kWire><<<grid, block, 0, stream>>>(tab, p);
      break;
    case BasisKind::kUser:
      decode_dense_kernel<kTargets, kWire><<<grid, block, 0, stream>>>(tab, p, DenseBasis{basis_p0, basis_p1});
      break;
  }
}

// ---------------------------------------------------------------- compact wire format

// float32 -> bfloat16 bits, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t b = __float_as_uint(x);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// One thread per group of one worker's entries (8 at 12 bits, 16 at 14):
// the group's bfloat16 values, and its positions as whole little-endian
// 32-bit words (entry j at bits kBits * j); entries past the end count as
// position 0 and store no value.
template <int kBits>
__global__ __launch_bounds__(256) void pack_wire_kernel(const float* __restrict__ pay_val,
                                                        const uint16_t* __restrict__ pay_idx, int64_t entries,
                                                        int64_t groups, int64_t total, uint16_t* __restrict__ wire_val,
                                                        uint32_t* __restrict__ wire_idx) {
  using F = WireFormat<kBits>;
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (t >= total) return;
  const int64_t w = t / groups;
  const int64_t g = t - w * groups;
  const int64_t base = w * entries;
  uint32_t* __restrict__ out = wire_idx + t * F::kWords;  // worker w's words start at w * groups * kWords
  uint64_t bits = 0;  // pending bits, low first
  int nb = 0, o = 0;
#pragma unroll
  for (int j = 0; j < F::kGroup; ++j) {
    const int64_t e = g * F::kGroup + j;
    uint32_t f = 0u;
    if (e < entries) {
      f = pay_idx[base + e] & ((1u << kBits) - 1u);
      wire_val[base + e] = uint16_t(bf16_rne(pay_val[base + e]));
    }
    bits |= uint64_t(f) << nb;
    nb += kBits;
    if (nb >= 32) {  // resolved at compile time: j is a constant
      out[o++] = uint32_t(bits);
      bits >>= 32;
      nb -= 32;
    }
  }
}

// ---------------------------------------------------------------- one-bit sign apply

// X = X - eta (s + lambda X), s = -1 where the element's bit is set, else +1.
__device__ __forceinline__ float apply_bit(float x, uint64_t word, int bit, const ApplyParams& p) {
  const float s = ((word >> bit) & 1u) ? -1.f : 1.f;
  return fmaf(-p.eta, fmaf(p.lam, x, s), x);
}

// Same work items as the decode, four to a workgroup (one per wave): a
// 64x64 chunk (word i = row i, bit j = column j = lane j) or a slab of 64
// vector chunks (word c = chunk c, bit j = element j = lane j).  The word
// index is wave-uniform, so the words arrive through scalar loads while the
// rows stream through vector loads.
__global__ __launch_bounds__(256) void apply_signs_kernel(LaunchTable tab, ApplyParams p) {
  // four items per workgroup, one per wave
  const int item = xcd_item(blockIdx.x, gridDim.x) * 4 + int(__builtin_amdgcn_readfirstlane(threadIdx.x >> 6));
  if (item >= tab.items) return;
  const TensorSlot& ts = tab.t[find_tensor(tab, item)];
  const int lane = threadIdx.x & 63;
  const uint64_t* __restrict__ words = static_cast<const uint64_t*>(ts.aux);
  if (ts.cols == 0) {
    const int slab = item - ts.item_begin;
    const int64_t first = int64_t(slab) * 64 * 64 + lane;
    const int64_t rem = int64_t(ts.rows) - first;
    const int nc = min(64, int((uint32_t(ts.rows) + 63u) >> 6) - slab * 64);
    const uint64_t* __restrict__ wp = words + int64_t(slab) * 64;
    float* __restrict__ x = ts.dst + first;
    for (int c = 0; c < nc; ++c) {
      const uint64_t w = wp[c];
      if (c * 64 < rem) stream_store(apply_bit(stream_load(&x[c * 64]), w, lane, p), &x[c * 64]);
    }
    return;
  }
  const ChunkPos c = chunk_pos(ts, item);
  const uint64_t* __restrict__ wp = words + int64_t(c.local) * 64;
  float* __restrict__ xp = ts.dst + c.base;
  const int64_t ld = ts.cols;
  const int col = min(lane, c.vc - 1);
  // all 64 rows are requested before the first store (a store may alias a
  // later row as far as the compiler knows, so loads are not moved past it)
  float x[64];
  if (c.full) {
    load_rows_full(x, xp, ld, lane);
  } else {
#pragma unroll
    for (int i = 0; i < 64; ++i) x[i] = stream_load(&xp[min(i, c.vr - 1) * ld + col]);
  }
#pragma unroll
  for (int i = 0; i < 64; ++i) x[i] = apply_bit(x[i], wp[i], lane, p);
  if (c.full)
    store_rows<true>(x, xp, ld, c, lane);
  else
    store_rows<false>(x, xp, ld, c, lane);
}

}  // namespace

// ---------------------------------------------------------------- host-side launchers

hipError_t launch_encode(const LaunchTable& tab, const EncodeParams& p, bool g_bf16, BasisKind kind,
                         const float* basis_p0, const float* basis_p1, hipStream_t stream) {
  if (tab.items <= 0) return hipSuccess;
  const dim3 grid(tab.items), block(64);
  switch (kind) {
    case BasisKind::kDct:
      if (g_bf16)
        encode_kernel<DctBasis, true><<<grid, block, 0, stream>>>(tab, p);
      else
        encode_kernel<DctBasis, false><<<grid, block, 0, stream>>>(tab, p);
      break;
    case BasisKind::kIdentity:
      if (g_bf16)
        encode_kernel<IdentityBasis, true><<<grid, block, 0, stream>>>(tab, p);
      else
        encode_kernel<IdentityBasis, false><<<grid, block, 0, stream>>>(tab, p);
      break;
    case BasisKind::kUser: {
      const DenseBasis b{basis_p0, basis_p1};
      if (g_bf16)
        encode_dense_kernel<true><<<grid, block, 0, stream>>>(tab, p, b);
      else
        encode_dense_kernel<false><<<grid, block, 0, stream>>>(tab, p, b);
      break;
    }
  }
  return hipGetLastError();
}

hipError_t launch_decode(const LaunchTable& tab, const DecodeParams& p, BasisKind kind, const float* basis_p0,
                         const float* basis_p1, hipStream_t stream) {
  if (tab.items <= 0) return hipSuccess;
  if (p.wire)
    launch_decode_targets<kToParams, true>(tab, p, kind, basis_p0, basis_p1, stream);
  else if (p.pack_signs)
    launch_decode_targets<kToSigns>(tab, p, kind, basis_p0, basis_p1, stream);
  else if (p.write_mstar)
    launch_decode_targets<kToMstar>(tab, p, kind, basis_p0, basis_p1, stream);
  else if (p.update_x && p.update_m)
    launch_decode_targets<kToParams | kToMomentum>(tab, p, kind, basis_p0, basis_p1, stream);
  else if (p.update_m)
    launch_decode_targets<kToMomentum>(tab, p, kind, basis_p0, basis_p1, stream);
  else
    launch_decode_targets<kToParams>(tab, p, kind, basis_p0, basis_p1, stream);
  return hipGetLastError();
}

hipError_t launch_pack_wire(int32_t bits, const float* pay_val, const uint16_t* pay_idx, int64_t entries,
                            int32_t workers, uint16_t* wire_val, uint32_t* wire_idx, hipStream_t stream) {
  const int64_t per = bits == 12 ? WireFormat<12>::kGroup : WireFormat<14>::kGroup;
  const int64_t groups = (entries + per - 1) / per;
  const int64_t total = groups * workers;
  if (total <= 0) return hipSuccess;
  if ((total + 255) / 256 > int64_t(UINT32_MAX)) return hipErrorInvalidValue;
  const dim3 grid(uint32_t((total + 255) / 256)), block(256);
  if (bits == 12)
    pack_wire_kernel<12><<<grid, block, 0, stream>>>(pay_val, pay_idx, entries, groups, total, wire_val, wire_idx);
  else
    pack_wire_kernel<14><<<grid, block, 0, stream>>>(pay_val, pay_idx, entries, groups, total, wire_val, wire_idx);
  return hipGetLastError();
}

hipError_t launch_apply_signs(const LaunchTable& tab, const ApplyParams& p, hipStream_t stream) {
  if (tab.items <= 0) return hipSuccess;
  apply_signs_kernel<<<dim3((tab.items + 3) / 4), dim3(256), 0, stream>>>(tab, p);
  return hipGetLastError();
}

}  // namespace demo
