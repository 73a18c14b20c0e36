// HIP kernels of the DeMo per-step momentum codec for CDNA4 (gfx950).
//
// One wave64 owns one 64x64 chunk (2-D) or one slab of 64 consecutive
// 64-element chunks (1-D).  Data move between two register layouts:
//   column layout: lane j holds column j, x[i] = element (i, j);
//   row layout:    lane u holds row u,    x[v] = element (u, v).
// A coalesced global access of one row per instruction (64 lanes x 4 bytes)
// fills the column layout directly; a 64x65-float LDS tile (row stride 65:
// row and column accesses are both bank-conflict free) converts between the
// two.  Each 64-point transform runs inside one lane's registers.
//
// encode (DeMo summary, §3.4 Decoupled Local Momentum Updates, Tensor
// Chunking, Blockwise Linear Projection, Top-k Sparsification, Momentum
// Subtraction):
//   load G, M -> M' = beta M + c G (registers, column layout)
//   Q = P0 M' P1^T  (column pass, LDS transpose, row pass)
//   exact top-k of |Q| over the chunk, lower index wins ties
//   payload (value, index) in index order
//   R = P0^T Q_hat P1 (row pass, LDS transpose, column pass); M = M' - alpha R
// decode/apply (§3.4 Server-Side Aggregation, Inverse DCT and Unchunking,
// Base Optimizer Update):
//   scatter-add W payloads into an LDS accumulator with 8-bit counts, in
//   worker order 0..W-1 (indices are distinct within one payload, so no
//   atomics); average; M* = P0^T Q_bar P1; X = X - eta (phi(M*) + lambda X).
#include "launch.h"
#include "xform.h"

namespace demo {
namespace {

using xf::DctBasis;
using xf::DenseBasis;

constexpr int kLd = 65;  // LDS tile row stride in floats

// ---------------------------------------------------------------- wave helpers

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ int wave_excl_scan(int v, int lane) {
  int s = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(s, o);
    if (lane >= o) s += t;
  }
  return s - v;
}

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

// ---------------------------------------------------------------- top-k of one 64x64 chunk

// Row layout in q (lane u holds Q[u][0..63]).  Keeps the keff largest |Q|
// (ties: lower index u*64+v first), writes them in index order to outv/outi
// and zeroes every other entry of q (q becomes Q_hat).
//
// Exact selection: K, the keff-th largest magnitude, is built bit by bit
// from the top (a candidate T is kept when at least keff magnitudes are
// >= T).  Then every |Q| > K is taken, and of the |Q| == K the first
// keff - #(|Q| > K) in index order.
__device__ __forceinline__ void topk_chunk(float (&q)[64], int keff, int lane, float* __restrict__ outv,
                                           uint16_t* __restrict__ outi) {
  if (keff >= 4096) {
#pragma unroll
    for (int v = 0; v < 64; ++v) {
      outv[lane * 64 + v] = q[v];
      outi[lane * 64 + v] = static_cast<uint16_t>(lane * 64 + v);
    }
    return;
  }
  float lmax = 0.f;
#pragma unroll
  for (int v = 0; v < 64; ++v) lmax = fmaxf(lmax, fabsf(q[v]));
  const uint32_t hi = __float_as_uint(wave_max(lmax));
  uint32_t T = 0;
  for (int b = 30; b >= 0; --b) {
    const uint32_t cand = T | (1u << b);
    if (cand > hi) continue;
    const float cf = __uint_as_float(cand);
    int c = 0;
#pragma unroll
    for (int v = 0; v < 64; ++v) c += fabsf(q[v]) >= cf ? 1 : 0;
    if (wave_sum(c) >= keff) T = cand;
  }
  const float K = __uint_as_float(T);
  int gt = 0, eq = 0;
#pragma unroll
  for (int v = 0; v < 64; ++v) {
    const float a = fabsf(q[v]);
    gt += a > K ? 1 : 0;
    eq += a == K ? 1 : 0;
  }
  const int quota = keff - wave_sum(gt);
  const int eq_before = wave_excl_scan(eq, lane);
  const int take_eq = min(max(quota - eq_before, 0), eq);
  int off = wave_excl_scan(gt + take_eq, lane);
  int eqr = eq_before;
#pragma unroll
  for (int v = 0; v < 64; ++v) {
    const float a = fabsf(q[v]);
    const bool is_eq = a == K;
    const bool keep = a > K || (is_eq && eqr < quota);
    eqr += is_eq ? 1 : 0;
    if (keep) {
      outv[off] = q[v];
      outi[off] = static_cast<uint16_t>(lane * 64 + v);
      ++off;
    } else {
      q[v] = 0.f;
    }
  }
}

// Per-lane top-k of one 64-element chunk held in q (1-D chunks, lane = chunk).
__device__ __forceinline__ void topk_lane(float (&q)[64], int keff, bool write, float* __restrict__ outv,
                                          uint16_t* __restrict__ outi) {
  if (keff >= 64) {
    if (write) {
#pragma unroll
      for (int v = 0; v < 64; ++v) {
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
  for (int b = 30; b >= 0; --b) {
    const uint32_t cand = T | (1u << b);
    const float cf = __uint_as_float(cand);
    int c = 0;
#pragma unroll
    for (int v = 0; v < 64; ++v) c += fabsf(q[v]) >= cf ? 1 : 0;
    if (cand <= hi && c >= keff) T = cand;
  }
  const float K = __uint_as_float(T);
  int gt = 0;
#pragma unroll
  for (int v = 0; v < 64; ++v) gt += fabsf(q[v]) > K ? 1 : 0;
  const int quota = keff - gt;
  int eqr = 0, off = 0;
#pragma unroll
  for (int v = 0; v < 64; ++v) {
    const float a = fabsf(q[v]);
    const bool is_eq = a == K;
    const bool keep = a > K || (is_eq && eqr < quota);
    eqr += is_eq ? 1 : 0;
    if (keep) {
      if (write) {
        outv[off] = q[v];
        outi[off] = static_cast<uint16_t>(v);
      }
      ++off;
    } else {
      q[v] = 0.f;
    }
  }
}

// ---------------------------------------------------------------- encode, 2-D chunks

template <bool kFull, bool kBf16>
__device__ __forceinline__ void load_momentum(float (&mp)[64], const TensorSlot& ts, int64_t base, int vr,
                                              int vc, int lane, float beta, float gcoef) {
  const int64_t ld = ts.cols;
  const float* __restrict__ m = ts.dst;
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    float g = 0.f, mv = 0.f;
    if (kFull || (lane < vc && i < vr)) {
      const int64_t off = base + i * ld + lane;
      g = load_src<kBf16>(ts.src, off);
      mv = m[off];
    }
    mp[i] = fmaf(beta, mv, gcoef * g);
  }
}

template <bool kFull>
__device__ __forceinline__ void store_residual(const float (&mp)[64], const float (&r)[64], const TensorSlot& ts,
                                               int64_t base, int vr, int vc, int lane, float alpha) {
  const int64_t ld = ts.cols;
  float* __restrict__ m = ts.dst;
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    if (kFull || (lane < vc && i < vr)) m[base + i * ld + lane] = fmaf(-alpha, r[i], mp[i]);
  }
}

template <class Basis, bool kBf16>
__global__ __launch_bounds__(64) void encode2d_kernel(LaunchTable tab, EncodeParams p, Basis basis) {
  __shared__ float tile[64 * kLd];
  const int lane = threadIdx.x;
  const int item = blockIdx.x;
  const TensorSlot& ts = tab.t[find_tensor(tab, item)];
  const int local = item - ts.item_begin;
  const int cr = local / ts.grid1;
  const int cc = local - cr * ts.grid1;
  const int vr = min(64, ts.rows - cr * 64);
  const int vc = min(64, ts.cols - cc * 64);
  const int64_t base = int64_t(cr) * 64 * ts.cols + int64_t(cc) * 64;
  const bool full = (vr == 64) && (vc == 64);

  float mp[64];
  if (full)
    load_momentum<true, kBf16>(mp, ts, base, vr, vc, lane, p.beta, p.gcoef);
  else
    load_momentum<false, kBf16>(mp, ts, base, vr, vc, lane, p.beta, p.gcoef);

  float q[64];
#pragma unroll
  for (int i = 0; i < 64; ++i) q[i] = mp[i];
  basis.fwd0(q);
  col_to_row(tile, q, lane);
  basis.fwd1(q);

  const int64_t e0 = ts.entry_begin + int64_t(local) * p.keff;
  topk_chunk(q, p.keff, lane, p.pay_val + e0, p.pay_idx + e0);

  basis.inv1(q);
  row_to_col(tile, q, lane);
  basis.inv0(q);

  if (full)
    store_residual<true>(mp, q, ts, base, vr, vc, lane, p.alpha);
  else
    store_residual<false>(mp, q, ts, base, vr, vc, lane, p.alpha);
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
  const float* __restrict__ m = ts.dst;

  float mp[64];
#pragma unroll
  for (int c = 0; c < 64; ++c) {
    const int64_t off = first + int64_t(c) * 64 + lane;
    float g = 0.f, mv = 0.f;
    if (off < len) {
      g = load_src<kBf16>(ts.src, off);
      mv = m[off];
    }
    mp[c] = fmaf(p.beta, mv, p.gcoef * g);
  }
  float q[64];
#pragma unroll
  for (int c = 0; c < 64; ++c) q[c] = mp[c];
  col_to_row(tile, q, lane);
  basis.fwd0(q);

  const int chunk = slab * 64 + lane;  // this lane's chunk within the tensor
  const bool live = chunk < ts.grid1;
  const int64_t e0 = ts.entry_begin + int64_t(live ? chunk : 0) * p.keff;
  topk_lane(q, p.keff, live, p.pay_val + e0, p.pay_idx + e0);

  basis.inv0(q);
  row_to_col(tile, q, lane);
  float* __restrict__ mo = ts.dst;
#pragma unroll
  for (int c = 0; c < 64; ++c) {
    const int64_t off = first + int64_t(c) * 64 + lane;
    if (off < len) mo[off] = fmaf(-p.alpha, q[c], mp[c]);
  }
}

// ---------------------------------------------------------------- decode / apply

__device__ __forceinline__ float average(float s, int c, const DecodeParams& p) {
  if (p.avg_workers) return s * p.inv_workers;
  return c ? s * __builtin_amdgcn_rcpf(float(c)) : 0.f;
}

__device__ __forceinline__ float update(float x, float m, const DecodeParams& p) {
  const float ph = p.phi_sign ? sign_of(m) : m;
  return fmaf(-p.eta, fmaf(p.lam, x, ph), x);
}

template <class Basis>
__global__ __launch_bounds__(64) void decode2d_kernel(LaunchTable tab, DecodeParams p, Basis basis) {
  __shared__ float acc[64 * kLd];
  __shared__ uint32_t cntw[1024];
  uint8_t* cnt = reinterpret_cast<uint8_t*>(cntw);
  const int lane = threadIdx.x;
  const int item = blockIdx.x;
  const TensorSlot& ts = tab.t[find_tensor(tab, item)];
  const int local = item - ts.item_begin;
  const int cr = local / ts.grid1;
  const int cc = local - cr * ts.grid1;
  const int vr = min(64, ts.rows - cr * 64);
  const int vc = min(64, ts.cols - cc * 64);
  const int64_t base = int64_t(cr) * 64 * ts.cols + int64_t(cc) * 64;

  for (int i = lane; i < 64 * kLd; i += 64) acc[i] = 0.f;
  for (int i = lane; i < 1024; i += 64) cntw[i] = 0u;
  __syncthreads();

  const int64_t e0 = ts.entry_begin + int64_t(local) * p.keff;
  for (int w = 0; w < p.workers; ++w) {
    const float* __restrict__ pv = p.pay_val + w * p.entries + e0;
    const uint16_t* __restrict__ pi = p.pay_idx + w * p.entries + e0;
    for (int e = lane; e < p.keff; e += 64) {
      const int id = pi[e] & 4095;
      acc[(id >> 6) * kLd + (id & 63)] += pv[e];
      cnt[id] += 1;
    }
    __syncthreads();
  }

  float q[64];
#pragma unroll
  for (int v = 0; v < 64; ++v) q[v] = average(acc[lane * kLd + v], cnt[lane * 64 + v], p);
  __syncthreads();
  basis.inv1(q);
  row_to_col(acc, q, lane);
  basis.inv0(q);

  float* __restrict__ x = ts.dst;
  const int64_t ld = ts.cols;
  if (vr == 64 && vc == 64) {
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      const int64_t off = base + i * ld + lane;
      x[off] = update(x[off], q[i], p);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      if (lane < vc && i < vr) {
        const int64_t off = base + i * ld + lane;
        x[off] = update(x[off], q[i], p);
      }
    }
  }
}

template <class Basis>
__global__ __launch_bounds__(64) void decode1d_kernel(LaunchTable tab, DecodeParams p, Basis basis) {
  __shared__ float acc[64 * kLd];
  __shared__ uint32_t cntw[1024];
  uint8_t* cnt = reinterpret_cast<uint8_t*>(cntw);
  const int lane = threadIdx.x;
  const int item = blockIdx.x;
  const TensorSlot& ts = tab.t[find_tensor(tab, item)];
  const int slab = item - ts.item_begin;
  const int64_t first = int64_t(slab) * 64 * 64;
  const int64_t len = ts.rows;

  for (int i = lane; i < 64 * kLd; i += 64) acc[i] = 0.f;
  for (int i = lane; i < 1024; i += 64) cntw[i] = 0u;
  __syncthreads();

  // lane c gathers the payload entries of its own chunk into LDS row c
  const int chunk = slab * 64 + lane;
  if (chunk < ts.grid1) {
    const int64_t e0 = ts.entry_begin + int64_t(chunk) * p.keff;
    for (int w = 0; w < p.workers; ++w) {
      const float* __restrict__ pv = p.pay_val + w * p.entries + e0;
      const uint16_t* __restrict__ pi = p.pay_idx + w * p.entries + e0;
      for (int e = 0; e < p.keff; ++e) {
        const int id = pi[e] & 63;
        acc[lane * kLd + id] += pv[e];
        cnt[lane * 64 + id] += 1;
      }
    }
  }
  __syncthreads();
  float q[64];
#pragma unroll
  for (int v = 0; v < 64; ++v) q[v] = average(acc[lane * kLd + v], cnt[lane * 64 + v], p);
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
