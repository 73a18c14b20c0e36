// HIP kernels of the DeMo per-step momentum codec for CDNA4 (gfx950).
//
// One wave64 owns one 64x64 chunk (2-D) or one slab of 64 consecutive
// 64-element chunks (1-D).  Data move between two register layouts:
//   column layout: lane j holds column j, x[i] = element (i, j);
//   row layout:    lane u holds row u,    x[v] = element (u, v).
// A coalesced global access of one 256-byte row segment per instruction
// fills the column layout directly; a 64x65-float LDS tile (row stride 65:
// row and column accesses are both bank-conflict free) converts between the
// two.  Each 64-point transform runs inside one lane's registers.
//
// encode (DeMo summary, §3.4 Decoupled Local Momentum Updates, Tensor
// Chunking, Blockwise Linear Projection, Top-k Sparsification, Momentum
// Subtraction):
//   load G, M -> M' = beta M + c G (registers, column layout)
//   Q = P0 M' P1^T  (column pass, LDS transpose, row pass)
//   exact top-k of |Q| over the chunk, lower index wins ties; payload
//   (value, index) in index order
//   M = P0^T (Q - alpha Q_hat) P1 (row pass, LDS transpose, column pass),
//   which equals M' - alpha P0^T Q_hat P1 because P0, P1 are orthonormal
// decode/apply (§3.4 Server-Side Aggregation, Inverse DCT and Unchunking,
// Base Optimizer Update):
//   scatter-add W payloads into an LDS accumulator with 8-bit contributor
//   counts, one LDS atomic instruction per worker in worker order 0..W-1
//   (indices are distinct within one payload, so the lanes of one
//   instruction never collide and the sum order is fixed); average;
//   M* = P0^T Q_bar P1; X = X - eta (phi(M*) + lambda X).
#include "launch.h"
#include "topk.h"
#include "xform.h"

namespace demo {
namespace {

using xf::DctBasis;
using xf::DenseBasis;

constexpr int kLd = 65;     // LDS tile row stride in floats
constexpr int kCntLd = 17;  // count rows: 16 words of 8-bit counts + 1 pad word
constexpr int kWorkerBatch = 16;

// ---------------------------------------------------------------- helpers

__device__ __forceinline__ int find_tensor(const LaunchTable& tab, int item) {
  int lo = 0, hi = tab.n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tab.t[mid].item_begin <= item)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

template <bool kBf16>
__device__ __forceinline__ float load_src(const void* p, int64_t off) {
  if constexpr (kBf16) {
    const uint32_t b = static_cast<const uint16_t*>(p)[off];
    return __uint_as_float(b << 16);
  } else {
    return static_cast<const float*>(p)[off];
  }
}

__device__ __forceinline__ float sign_of(float m) { return m > 0.f ? 1.f : (m < 0.f ? -1.f : 0.f); }

// column layout -> row layout through the LDS tile
__device__ __forceinline__ void col_to_row(float* tile, float (&x)[64], int lane) {
#pragma unroll
  for (int i = 0; i < 64; ++i) tile[i * kLd + lane] = x[i];
  __syncthreads();
#pragma unroll
  for (int v = 0; v < 64; ++v) x[v] = tile[lane * kLd + v];
  __syncthreads();
}

// row layout -> column layout through the LDS tile
__device__ __forceinline__ void row_to_col(float* tile, float (&x)[64], int lane) {
#pragma unroll
  for (int v = 0; v < 64; ++v) tile[lane * kLd + v] = x[v];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 64; ++i) x[i] = tile[i * kLd + lane];
  __syncthreads();
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
  const int cr = c.local / ts.grid1;
  const int cc = c.local - cr * ts.grid1;
  c.vr = min(64, ts.rows - cr * 64);
  c.vc = min(64, ts.cols - cc * 64);
  c.base = int64_t(cr) * 64 * ts.cols + int64_t(cc) * 64;
  c.full = (c.vr == 64) && (c.vc == 64);
  return c;
}

// ---------------------------------------------------------------- encode, 2-D chunks

template <bool kFull, bool kBf16>
__device__ __forceinline__ void load_momentum(float (&q)[64], const TensorSlot& ts, const ChunkPos& c, int lane,
                                              float beta, float gcoef) {
  const int64_t ld = ts.cols;
  const float* __restrict__ m = ts.dst + c.base;
  const char* __restrict__ g = static_cast<const char*>(ts.src) + c.base * (kBf16 ? 2 : 4);
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    float gv = 0.f, mv = 0.f;
    if (kFull || (lane < c.vc && i < c.vr)) {
      gv = load_src<kBf16>(g, i * ld + lane);
      mv = m[i * ld + lane];
    }
    q[i] = fmaf(beta, mv, gcoef * gv);
  }
}

template <bool kFull>
__device__ __forceinline__ void store_rows(const float (&q)[64], float* __restrict__ dst, int64_t ld,
                                           const ChunkPos& c, int lane) {
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    if (kFull || (lane < c.vc && i < c.vr)) dst[i * ld + lane] = q[i];
  }
}

template <class Basis, bool kBf16>
__global__ __launch_bounds__(64) void encode2d_kernel(LaunchTable tab, EncodeParams p, Basis basis) {
  __shared__ float tile[64 * kLd];
  const int lane = threadIdx.x;
  const TensorSlot& ts = tab.t[find_tensor(tab, blockIdx.x)];
  const ChunkPos c = chunk_pos(ts, blockIdx.x);

  float q[64];
  if (c.full)
    load_momentum<true, kBf16>(q, ts, c, lane, p.beta, p.gcoef);
  else
    load_momentum<false, kBf16>(q, ts, c, lane, p.beta, p.gcoef);

  basis.fwd0(q);
  col_to_row(tile, q, lane);
  basis.fwd1(q);

  const int64_t e0 = ts.entry_begin + int64_t(c.local) * p.keff;
  tk::topk_chunk(q, p.keff, lane, p.alpha, p.pay_val + e0, p.pay_idx + e0, reinterpret_cast<uint32_t*>(tile));
  __syncthreads();

  basis.inv1(q);
  row_to_col(tile, q, lane);
  basis.inv0(q);

  if (c.full)
    store_rows<true>(q, ts.dst + c.base, ts.cols, c, lane);
  else
    store_rows<false>(q, ts.dst + c.base, ts.cols, c, lane);
}

// ---------------------------------------------------------------- encode, 1-D chunks

// Slab view of a vector: V[c][e] = vec[(64 * slab + c) * 64 + e], chunk c of
// the slab is row c.  Column layout after the load (lane e), row layout
// (lane c = one chunk) after the transpose.
template <class Basis, bool kBf16>
__global__ __launch_bounds__(64) void encode1d_kernel(LaunchTable tab, EncodeParams p, Basis basis) {
  __shared__ float tile[64 * kLd];
  const int lane = threadIdx.x;
  const int item = blockIdx.x;
  const TensorSlot& ts = tab.t[find_tensor(tab, item)];
  const int slab = item - ts.item_begin;
  const int64_t first = int64_t(slab) * 64 * 64;  // element offset of the slab
  const int64_t len = ts.rows;
  float* __restrict__ m = ts.dst;

  float q[64];
#pragma unroll
  for (int c = 0; c < 64; ++c) {
    const int64_t off = first + int64_t(c) * 64 + lane;
    float g = 0.f, mv = 0.f;
    if (off < len) {
      g = load_src<kBf16>(ts.src, off);
      mv = m[off];
    }
    q[c] = fmaf(p.beta, mv, p.gcoef * g);
  }
  col_to_row(tile, q, lane);
  basis.fwd0(q);

  const int chunk = slab * 64 + lane;  // this lane's chunk within the tensor
  const bool live = chunk < ts.grid1;
  const int64_t e0 = ts.entry_begin + int64_t(live ? chunk : 0) * p.keff;
  tk::topk_lane(q, p.keff, live, p.alpha, p.pay_val + e0, p.pay_idx + e0);

  basis.inv0(q);
  row_to_col(tile, q, lane);
#pragma unroll
  for (int c = 0; c < 64; ++c) {
    const int64_t off = first + int64_t(c) * 64 + lane;
    if (off < len) m[off] = q[c];
  }
}

// ---------------------------------------------------------------- decode / apply

__device__ __forceinline__ float update(float x, float m, const DecodeParams& p) {
  const float ph = p.phi_sign ? sign_of(m) : m;
  return fmaf(-p.eta, fmaf(p.lam, x, ph), x);
}

// Zero the accumulator tile and the count rows.
__device__ __forceinline__ void clear_acc(float* acc, uint32_t* cntw, int lane) {
  for (int i = lane; i < 64 * kLd; i += 64) acc[i] = 0.f;
  for (int i = lane; i < 64 * kCntLd; i += 64) cntw[i] = 0u;
}

// Scatter-add the W payload segments of one 64x64 chunk (entries e0 ..
// e0 + keff of every worker).  One LDS atomic instruction per (worker, entry
// block); within it the indices are distinct, so no lanes collide and every
// coefficient receives its terms in worker order.
__device__ __forceinline__ void scatter_chunk(float* acc, uint32_t* cntw, const DecodeParams& p, int64_t e0,
                                              int lane) {
  for (int eb = 0; eb < p.keff; eb += 64) {
    const int e = eb + lane;
    const bool on = e < p.keff;
    for (int w0 = 0; w0 < p.workers; w0 += kWorkerBatch) {
      float val[kWorkerBatch];
      uint32_t ix[kWorkerBatch];
#pragma unroll
      for (int j = 0; j < kWorkerBatch; ++j) {
        const int64_t off = int64_t(w0 + j) * p.entries + e0 + e;
        const bool ok = on && (w0 + j) < p.workers;
        val[j] = ok ? p.pay_val[off] : 0.f;
        ix[j] = ok ? p.pay_idx[off] : 0u;
      }
#pragma unroll
      for (int j = 0; j < kWorkerBatch; ++j) {
        if (on && (w0 + j) < p.workers) {
          const uint32_t id = ix[j] & 4095u;
          const uint32_t u = id >> 6, v = id & 63u;
          atomicAdd(&acc[u * kLd + v], val[j]);
          atomicAdd(&cntw[u * kCntLd + (v >> 2)], 1u << ((v & 3u) * 8u));
        }
      }
    }
  }
}

// Row u of the average into q (row layout).
__device__ __forceinline__ void average_row(float (&q)[64], const float* acc, const uint32_t* cntw,
                                            const DecodeParams& p, int lane) {
  if (p.avg_workers) {
#pragma unroll
    for (int v = 0; v < 64; ++v) q[v] = acc[lane * kLd + v] * p.inv_workers;
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t w = cntw[lane * kCntLd + j];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const float n = float((w >> (8 * b)) & 255u);
        // n == 0 means no worker sent the coefficient; its sum is 0 as well
        q[4 * j + b] = acc[lane * kLd + 4 * j + b] * __builtin_amdgcn_rcpf(fmaxf(n, 1.f));
      }
    }
  }
}

template <class Basis>
__global__ __launch_bounds__(64) void decode2d_kernel(LaunchTable tab, DecodeParams p, Basis basis) {
  __shared__ float acc[64 * kLd];
  __shared__ uint32_t cntw[64 * kCntLd];
  const int lane = threadIdx.x;
  const TensorSlot& ts = tab.t[find_tensor(tab, blockIdx.x)];
  const ChunkPos c = chunk_pos(ts, blockIdx.x);

  clear_acc(acc, cntw, lane);
  __syncthreads();
  scatter_chunk(acc, cntw, p, ts.entry_begin + int64_t(c.local) * p.keff, lane);
  __syncthreads();

  // parameters are fetched now; they land while the average and the inverse transform run
  const int64_t ld = ts.cols;
  float* __restrict__ xp = ts.dst + c.base;
  float x[64];
  if (c.full) {
#pragma unroll
    for (int i = 0; i < 64; ++i) x[i] = xp[i * ld + lane];
  } else {
#pragma unroll
    for (int i = 0; i < 64; ++i) x[i] = (lane < c.vc && i < c.vr) ? xp[i * ld + lane] : 0.f;
  }

  float q[64];
  average_row(q, acc, cntw, p, lane);
  __syncthreads();
  basis.inv1(q);
  row_to_col(acc, q, lane);
  basis.inv0(q);

#pragma unroll
  for (int i = 0; i < 64; ++i) x[i] = update(x[i], q[i], p);
  if (c.full)
    store_rows<true>(x, xp, ld, c, lane);
  else
    store_rows<false>(x, xp, ld, c, lane);
}

template <class Basis>
__global__ __launch_bounds__(64) void decode1d_kernel(LaunchTable tab, DecodeParams p, Basis basis) {
  __shared__ float acc[64 * kLd];
  __shared__ uint32_t cntw[64 * kCntLd];
  const int lane = threadIdx.x;
  const int item = blockIdx.x;
  const TensorSlot& ts = tab.t[find_tensor(tab, item)];
  const int slab = item - ts.item_begin;
  const int64_t first = int64_t(slab) * 64 * 64;
  const int64_t len = ts.rows;

  clear_acc(acc, cntw, lane);
  __syncthreads();
  // lane c gathers the payload entries of its own chunk into LDS row c
  const int chunk = slab * 64 + lane;
  if (chunk < ts.grid1) {
    const int64_t e0 = ts.entry_begin + int64_t(chunk) * p.keff;
    for (int w = 0; w < p.workers; ++w) {
      const float* __restrict__ pv = p.pay_val + w * p.entries + e0;
      const uint16_t* __restrict__ pi = p.pay_idx + w * p.entries + e0;
      for (int e = 0; e < p.keff; ++e) {
        const uint32_t id = pi[e] & 63u;
        acc[lane * kLd + id] += pv[e];
        cntw[lane * kCntLd + (id >> 2)] += 1u << ((id & 3u) * 8u);
      }
    }
  }
  __syncthreads();
  float q[64];
  average_row(q, acc, cntw, p, lane);
  __syncthreads();
  basis.inv0(q);
  row_to_col(acc, q, lane);

  float* __restrict__ x = ts.dst;
#pragma unroll
  for (int c = 0; c < 64; ++c) {
    const int64_t off = first + int64_t(c) * 64 + lane;
    if (off < len) x[off] = update(x[off], q[c], p);
  }
}

}  // namespace

// ---------------------------------------------------------------- host-side launchers

hipError_t launch_encode2d(const LaunchTable& tab, const EncodeParams& p, bool g_bf16, const float* basis_p0,
                           const float* basis_p1, hipStream_t stream) {
  if (tab.items <= 0) return hipSuccess;
  const dim3 grid(tab.items), block(64);
  if (basis_p0 == nullptr) {
    if (g_bf16)
      encode2d_kernel<DctBasis, true><<<grid, block, 0, stream>>>(tab, p, DctBasis{});
    else
      encode2d_kernel<DctBasis, false><<<grid, block, 0, stream>>>(tab, p, DctBasis{});
  } else {
    const DenseBasis b{basis_p0, basis_p1};
    if (g_bf16)
      encode2d_kernel<DenseBasis, true><<<grid, block, 0, stream>>>(tab, p, b);
    else
      encode2d_kernel<DenseBasis, false><<<grid, block, 0, stream>>>(tab, p, b);
  }
  return hipGetLastError();
}

hipError_t launch_encode1d(const LaunchTable& tab, const EncodeParams& p, bool g_bf16, const float* basis_p0,
                           hipStream_t stream) {
  if (tab.items <= 0) return hipSuccess;
  const dim3 grid(tab.items), block(64);
  if (basis_p0 == nullptr) {
    if (g_bf16)
      encode1d_kernel<DctBasis, true><<<grid, block, 0, stream>>>(tab, p, DctBasis{});
    else
      encode1d_kernel<DctBasis, false><<<grid, block, 0, stream>>>(tab, p, DctBasis{});
  } else {
    const DenseBasis b{basis_p0, basis_p0};
    if (g_bf16)
      encode1d_kernel<DenseBasis, true><<<grid, block, 0, stream>>>(tab, p, b);
    else
      encode1d_kernel<DenseBasis, false><<<grid, block, 0, stream>>>(tab, p, b);
  }
  return hipGetLastError();
}

hipError_t launch_decode2d(const LaunchTable& tab, const DecodeParams& p, const float* basis_p0,
                           const float* basis_p1, hipStream_t stream) {
  if (tab.items <= 0) return hipSuccess;
  const dim3 grid(tab.items), block(64);
  if (basis_p0 == nullptr)
    decode2d_kernel<DctBasis><<<grid, block, 0, stream>>>(tab, p, DctBasis{});
  else
    decode2d_kernel<DenseBasis><<<grid, block, 0, stream>>>(tab, p, DenseBasis{basis_p0, basis_p1});
  return hipGetLastError();
}

hipError_t launch_decode1d(const LaunchTable& tab, const DecodeParams& p, const float* basis_p0,
                           hipStream_t stream) {
  if (tab.items <= 0) return hipSuccess;
  const dim3 grid(tab.items), block(64);
  if (basis_p0 == nullptr)
    decode1d_kernel<DctBasis><<<grid, block, 0, stream>>>(tab, p, DctBasis{});
  else
    decode1d_kernel<DenseBasis><<<grid, block, 0, stream>>>(tab, p, DenseBasis{basis_p0, basis_p0});
  return hipGetLastError();
}

}  // namespace demo
