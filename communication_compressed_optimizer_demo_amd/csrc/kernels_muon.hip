// phi = Muon on CDNA4 (gfx950): phi(M) = M (M^T M + eps I)^(-1/2) on every
// whole tensor ("DeMo: Decoupled Momentum Optimization", summary §3.4 Base
// Optimizer Update, Muon), followed by X = X - eta (phi(M*) + lambda X).
//
// A matrix M (r x c, n = min(r, c)) goes through its smaller Gram matrix
// A = M M^T (r <= c) or M^T M, n x n, since (M M^T + eps I)^(-1/2) M and
// M (M^T M + eps I)^(-1/2) are the same matrix.  The inverse square root
// comes from the coupled Newton-Schulz iteration
//   Y0 = (A + eps I) / s,  Z0 = I,
//   T = (3 I - Z Y) / 2,  Y <- Y T,  Z <- T Z,
// with s = ||A + eps I||_F (so every eigenvalue of Y0 is in (0, 1]); Z then
// converges to (A + eps I)^(-1/2) sqrt(s).  Every product is a dense fp32
// GEMM on the matrix cores; the last one, Z M / sqrt(s) (or M Z / sqrt(s)),
// carries the parameter update in its epilogue.  A vector is one column:
// m / sqrt(m.m + eps).
//
// GEMM on v_mfma_f32_32x32x2f32.  Operand layout of that instruction: lane l
// supplies A[l % 32][l / 32] and B[l / 32][l % 32]; the accumulator holds
// D[8 (v / 4) + 4 (l / 32) + (v % 4)][l % 32] in register v.  Two kernels:
//  - gemm_kernel (any shape): 128 x 128 (or 64 x 64) output tile per
//    256-thread workgroup, 2 x 2 waves; K advances kBK per LDS stage,
//    double-buffered, bounds-checked 4-byte loads of the next stage issued
//    before the current stage's MFMAs;
//  - gemm_tile_kernel (whole tiles): the same tiles with 4 x 2 waves at
//    128 x 128, K stages of kSK, 16-byte loads two stages ahead.
// Both take a batch of same-shape products (grid z), which the Newton-Schulz
// steps of several matrices with equal n share.
#include <mutex>

#include "common.h"
#include "launch.h"

namespace demo {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kBK = 16, kPad = 4;

// Product blockIdx.z of a batch: move the operand pointers to it.
__device__ __forceinline__ void select_product(GemmArgs& g) {
  const int64_t z = blockIdx.z;
  g.A += z * g.sA;
  g.B += z * g.sB;
  if (g.C) g.C += z * g.sC;
  g.D += z * g.sD;
}

// kT: workgroup tile edge (128 or 64); the four waves form a 2 x 2 grid of
// kT/2 x kT/2 wave tiles, each (kT/64) x (kT/64) MFMA tiles of 32 x 32.
template <bool kTA, bool kTB, int kT>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g) {
  select_product(g);
  constexpr int E = kT / 16;    // floats each thread stages per operand and K stage
  constexpr int kMT = kT / 64;  // MFMA tiles per wave and dimension
  __shared__ float As[2][kBK][kT + kPad];
  __shared__ float Bs[2][kBK][kT + kPad];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int m0 = blockIdx.y * kT, n0 = blockIdx.x * kT;
  const int M = g.M, N = g.N, K = g.K;

  // Staging: E consecutive elements per thread, along K for an operand whose
  // rows run along M (N), along M (N) for a transposed one.
  float ra[E], rb[E];
  auto load_a = [&](int k0) {
    if constexpr (!kTA) {  // A row-major M x K
      const int m = m0 + tid / (16 / E), kb = k0 + (tid % (16 / E)) * E;
#pragma unroll
      for (int q = 0; q < E; ++q) ra[q] = (m < M && kb + q < K) ? g.A[int64_t(m) * g.lda + kb + q] : 0.f;
    } else {  // A = S^T, S row-major K x M
      const int k = k0 + tid / (kT / E), mb = m0 + (tid % (kT / E)) * E;
#pragma unroll
      for (int q = 0; q < E; ++q) ra[q] = (k < K && mb + q < M) ? g.A[int64_t(k) * g.lda + mb + q] : 0.f;
    }
  };
  auto load_b = [&](int k0) {
    if constexpr (!kTB) {  // B row-major K x N
      const int k = k0 + tid / (kT / E), nb = n0 + (tid % (kT / E)) * E;
#pragma unroll
      for (int q = 0; q < E; ++q) rb[q] = (k < K && nb + q < N) ? g.B[int64_t(k) * g.ldb + nb + q] : 0.f;
    } else {  // B = S^T, S row-major N x K
      const int n = n0 + tid / (16 / E), kb = k0 + (tid % (16 / E)) * E;
#pragma unroll
      for (int q = 0; q < E; ++q) rb[q] = (n < N && kb + q < K) ? g.B[int64_t(n) * g.ldb + kb + q] : 0.f;
    }
  };
  auto store_ab = [&](int buf) {
    if constexpr (!kTA) {
      const int m = tid / (16 / E), kb = (tid % (16 / E)) * E;
#pragma unroll
      for (int q = 0; q < E; ++q) As[buf][kb + q][m] = ra[q];
    } else {
      const int k = tid / (kT / E), mb = (tid % (kT / E)) * E;
#pragma unroll
      for (int q = 0; q < E; ++q) As[buf][k][mb + q] = ra[q];
    }
    if constexpr (!kTB) {
      const int k = tid / (kT / E), nb = (tid % (kT / E)) * E;
#pragma unroll
      for (int q = 0; q < E; ++q) Bs[buf][k][nb + q] = rb[q];
    } else {
      const int n = tid / (16 / E), kb = (tid % (16 / E)) * E;
#pragma unroll
      for (int q = 0; q < E; ++q) Bs[buf][kb + q][n] = rb[q];
    }
  };

  floatx16 acc[kMT][kMT];
#pragma unroll
  for (int i = 0; i < kMT; ++i)
#pragma unroll
    for (int j = 0; j < kMT; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int nk = (K + kBK - 1) / kBK;
  load_a(0);
  load_b(0);
  store_ab(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      load_a((kt + 1) * kBK);
      load_b((kt + 1) * kBK);
    }
#pragma unroll
    for (int kk = 0; kk < kBK / 2; ++kk) {
      const int kr = 2 * kk + (lane >> 5);
      float a[kMT], b[kMT];
#pragma unroll
      for (int t = 0; t < kMT; ++t) {
        a[t] = As[cur][kr][wm * (kT / 2) + t * 32 + (lane & 31)];
        b[t] = Bs[cur][kr][wn * (kT / 2) + t * 32 + (lane & 31)];
      }
#pragma unroll
      for (int i = 0; i < kMT; ++i)
#pragma unroll
        for (int j = 0; j < kMT; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_ab(cur ^ 1);
    __syncthreads();
  }

  // D = alpha * acc + beta * C + gamma * I (C may alias D: each element is
  // read and written by the same lane)
  const float alpha = g.alpha * (g.alpha_scale ? *g.alpha_scale : 1.f);
#pragma unroll
  for (int ti = 0; ti < kMT; ++ti) {
#pragma unroll
    for (int tj = 0; tj < kMT; ++tj) {
      const int col = n0 + wn * (kT / 2) + tj * 32 + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wm * (kT / 2) + ti * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (row < M && col < N) {
          float r = alpha * acc[ti][tj][v];
          if (g.beta != 0.f) r = fmaf(g.beta, g.C[int64_t(row) * g.ldc + col], r);
          if (row == col) r += g.gamma;
          g.D[int64_t(row) * g.ldd + col] = r;
        }
      }
    }
  }
}

// ---------------------------------------------------------------- whole-tile GEMM
//
// For products whose M and N are multiples of the tile edge and K of 2 kSK, with
// 16-byte aligned operands.  Same 2 x 2 wave grid and MFMA tiles as above;
// what differs is how operands reach the matrix cores:
//  - K advances kSK = 32 per stage; each thread moves its share of a stage
//    with 16-byte global loads, eight lanes per 128-byte row segment;
//  - two register sets hold stages s+1 and s+2 while stage s is multiplied,
//    so a global load has two stages of MFMA work to arrive;
//  - MFMA k-slot h (lane half) takes the k values 16h .. 16h + 15 of a stage,
//    so an operand whose rows run along K in memory is kept that way in LDS
//    (pitch kSK + 4) and read with 16-byte LDS loads, and one whose rows run
//    along M or N is kept k-major (pitch kT + 2: the two lane halves, 16 rows
//    apart, fall on opposite halves of the banks).
constexpr int kSK = 32;

// Native vectors (not HIP's float4 struct) so the staging registers stay registers.
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// One operand's stage: kT rows (along M for A, N for B) by kSK values of k,
// moved by kThreads threads.  kKc: element (row, k) sits at X[row * ld + k]
// (rows along K in memory); otherwise at X[k * ld + row].
template <bool kKc, int kT, int kThreads>
struct TileOperand {
  static constexpr int kV = kT * kSK / 4 / kThreads;  // f32x4 per thread and stage
  static constexpr int kPitch = kKc ? kSK + 4 : kT + 2;
  static constexpr int kFloats = kKc ? kT * kPitch : kSK * kPitch;

  __device__ static void load(f32x4 (&r)[kV], const float* __restrict__ X, int64_t ld, int r0, int k0, int tid) {
#pragma unroll
    for (int j = 0; j < kV; ++j) {
      const int f = tid + kThreads * j;
      if constexpr (kKc) {
        const int c4 = f & 7, row = f >> 3;
        r[j] = *reinterpret_cast<const f32x4*>(X + int64_t(r0 + row) * ld + k0 + 4 * c4);
      } else {
        const int c4 = f % (kT / 4), k = f / (kT / 4);
        r[j] = *reinterpret_cast<const f32x4*>(X + int64_t(k0 + k) * ld + r0 + 4 * c4);
      }
    }
  }

  __device__ static void store(const f32x4 (&r)[kV], float* s, int tid) {
#pragma unroll
    for (int j = 0; j < kV; ++j) {
      const int f = tid + kThreads * j;
      if constexpr (kKc) {
        const int c4 = f & 7, row = f >> 3;
        *reinterpret_cast<f32x4*>(s + row * kPitch + 4 * c4) = r[j];
      } else {
        const int c4 = f % (kT / 4), k = f / (kT / 4);
        f32x2* p = reinterpret_cast<f32x2*>(s + k * kPitch + 4 * c4);
        p[0] = r[j].xy;
        p[1] = r[j].zw;
      }
    }
  }
};

// kWM x 2 waves; wave tile (kT / kWM) x (kT / 2), i.e. kMI x kMJ MFMA tiles.
template <bool kTA, bool kTB, int kT, int kWM>
__global__ __launch_bounds__(128 * kWM) void gemm_tile_kernel(GemmArgs g) {
  select_product(g);
  constexpr int kThreads = 128 * kWM;
  using OA = TileOperand<!kTA, kT, kThreads>;
  using OB = TileOperand<kTB, kT, kThreads>;
  constexpr int kMI = kT / kWM / 32, kMJ = kT / 64;
  constexpr int kAcc = kMI * kMJ == 1 ? 2 : 1;  // a lone 32 x 32 tile alternates two accumulators
  __shared__ __align__(16) float As[2][OA::kFloats];
  __shared__ __align__(16) float Bs[2][OB::kFloats];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, i32 = lane & 31;
  const int wm = w >> 1, wn = w & 1;
  const int m0 = blockIdx.y * kT, n0 = blockIdx.x * kT;
  const int nk = g.K / kSK;

  floatx16 acc[kMI][kMJ][kAcc];
#pragma unroll
  for (int i = 0; i < kMI; ++i)
#pragma unroll
    for (int j = 0; j < kMJ; ++j)
#pragma unroll
      for (int a = 0; a < kAcc; ++a)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][a][v] = 0.f;

  // Multiply one LDS stage: 16 MFMA k-steps, step kk uses k = 16h + kk.
  auto compute = [&](const float* sa, const float* sb) {
    f32x4 av[kMI][4], bv[kMJ][4];
#pragma unroll
    for (int t = 0; t < kMI; ++t) {
      if constexpr (!kTA) {
        const float* p = sa + (wm * (kT / kWM) + t * 32 + i32) * OA::kPitch + 16 * h;
#pragma unroll
        for (int q = 0; q < 4; ++q) av[t][q] = *reinterpret_cast<const f32x4*>(p + 4 * q);
      }
    }
#pragma unroll
    for (int t = 0; t < kMJ; ++t) {
      if constexpr (kTB) {
        const float* p = sb + (wn * (kT / 2) + t * 32 + i32) * OB::kPitch + 16 * h;
#pragma unroll
        for (int q = 0; q < 4; ++q) bv[t][q] = *reinterpret_cast<const f32x4*>(p + 4 * q);
      }
    }
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[kMI], b[kMJ];
#pragma unroll
      for (int t = 0; t < kMI; ++t) {
        if constexpr (!kTA)
          a[t] = av[t][kk >> 2][kk & 3];
        else
          a[t] = sa[(16 * h + kk) * OA::kPitch + wm * (kT / kWM) + t * 32 + i32];
      }
#pragma unroll
      for (int t = 0; t < kMJ; ++t) {
        if constexpr (kTB)
          b[t] = bv[t][kk >> 2][kk & 3];
        else
          b[t] = sb[(16 * h + kk) * OB::kPitch + wn * (kT / 2) + t * 32 + i32];
      }
#pragma unroll
      for (int i = 0; i < kMI; ++i)
#pragma unroll
        for (int j = 0; j < kMJ; ++j)
          acc[i][j][kk % kAcc] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[j], acc[i][j][kk % kAcc], 0, 0, 0);
    }
  };

  f32x4 ra0[OA::kV], rb0[OB::kV], ra1[OA::kV], rb1[OB::kV];
  auto load = [&](f32x4 (&ra)[OA::kV], f32x4 (&rb)[OB::kV], int kt) {
    OA::load(ra, g.A, g.lda, m0, kt * kSK, tid);
    OB::load(rb, g.B, g.ldb, n0, kt * kSK, tid);
  };
  auto store = [&](const f32x4 (&ra)[OA::kV], const f32x4 (&rb)[OB::kV], int buf) {
    OA::store(ra, As[buf], tid);
    OB::store(rb, Bs[buf], tid);
  };

  // nk is even and >= 2.  Loads past the last stage re-read the last stage
  // and are never multiplied: with no branch around a load, the compiler's
  // wait before a store counts only the younger register set.
  load(ra0, rb0, 0);
  store(ra0, rb0, 0);
  load(ra0, rb0, 1);
  load(ra1, rb1, min(2, nk - 1));
  __syncthreads();
  for (int kt = 0; kt < nk; kt += 2) {
    // stage kt from buffer 0; set 0 holds stage kt + 1, set 1 stage kt + 2
    compute(As[0], Bs[0]);
    store(ra0, rb0, 1);
    load(ra0, rb0, min(kt + 3, nk - 1));
    __syncthreads();
    compute(As[1], Bs[1]);
    store(ra1, rb1, 0);
    load(ra1, rb1, min(kt + 4, nk - 1));
    __syncthreads();
  }

  // D = alpha * acc + beta * C + gamma * I (C may alias D: each element is
  // read and written by the same lane)
  const float alpha = g.alpha * (g.alpha_scale ? *g.alpha_scale : 1.f);
#pragma unroll
  for (int ti = 0; ti < kMI; ++ti) {
#pragma unroll
    for (int tj = 0; tj < kMJ; ++tj) {
      const int col = n0 + wn * (kT / 2) + tj * 32 + i32;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wm * (kT / kWM) + ti * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
        float sum = acc[ti][tj][0][v];
        if constexpr (kAcc == 2) sum += acc[ti][tj][1][v];
        float r = alpha * sum;
        if (g.beta != 0.f) r = fmaf(g.beta, g.C[int64_t(row) * g.ldc + col], r);
        if (row == col) r += g.gamma;
        g.D[int64_t(row) * g.ldd + col] = r;
      }
    }
  }
}

// ||A + eps I||_F^2, first level: per-block partial sums in float64 (a fixed
// order, so the result does not change from run to run).
constexpr int kNormBlocks = 256;

__global__ __launch_bounds__(256) void fro_partial_kernel(const float* __restrict__ A, int n, float eps,
                                                          double* __restrict__ partial) {
  __shared__ double red[256];
  const int64_t total = int64_t(n) * n;
  double s = 0.0;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < total; i += int64_t(kNormBlocks) * 256) {
    double v = A[i];
    if (i / n == i % n) v += eps;
    s += v * v;
  }
  red[threadIdx.x] = s;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) partial[blockIdx.x] = red[0];
}

// scal[0] = 1 / s, scal[1] = 1 / sqrt(s), s = ||A + eps I||_F
__global__ __launch_bounds__(256) void fro_final_kernel(const double* __restrict__ partial,
                                                        float* __restrict__ scal) {
  __shared__ double red[256];
  red[threadIdx.x] = threadIdx.x < kNormBlocks ? partial[threadIdx.x] : 0.0;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double s = sqrt(red[0]);
    scal[0] = float(1.0 / s);
    scal[1] = float(1.0 / sqrt(s));
  }
}

// Y0 = (A + eps I) / s, Z0 = I
__global__ __launch_bounds__(256) void ns_init_kernel(const float* __restrict__ A, int n, float eps,
                                                      const float* __restrict__ scal, float* __restrict__ Y,
                                                      float* __restrict__ Z) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= int64_t(n) * n) return;
  const bool diag = i / n == i % n;
  Y[i] = (A[i] + (diag ? eps : 0.f)) * scal[0];
  Z[i] = diag ? 1.f : 0.f;
}

// One vector: X = X - eta (m / sqrt(m.m + eps) + lambda X)
__global__ __launch_bounds__(256) void muon_vector_kernel(const float* __restrict__ m, float* __restrict__ x,
                                                          int64_t len, float eps, float eta, float lam) {
  __shared__ double red[256];
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < len; i += 256) s += double(m[i]) * double(m[i]);
  red[threadIdx.x] = s;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  const float inv = float(1.0 / sqrt(red[0] + double(eps)));
  for (int64_t i = threadIdx.x; i < len; i += 256) x[i] = fmaf(-eta, fmaf(lam, x[i], m[i] * inv), x[i]);
}

template <int kT>
void launch_gemm_tile(const GemmArgs& g, bool trans_a, bool trans_b, bool whole, int32_t batch, hipStream_t stream) {
  const dim3 grid((g.N + kT - 1) / kT, (g.M + kT - 1) / kT, batch), block(256);
  if (whole) {
    // 128 x 128 tiles: 4 x 2 waves (two per SIMD at one workgroup per CU)
    constexpr int kWM = kT == 128 ? 4 : 2;
    const dim3 wblock(128 * kWM);
    if (!trans_a && !trans_b)
      gemm_tile_kernel<false, false, kT, kWM><<<grid, wblock, 0, stream>>>(g);
    else if (!trans_a && trans_b)
      gemm_tile_kernel<false, true, kT, kWM><<<grid, wblock, 0, stream>>>(g);
    else if (trans_a && !trans_b)
      gemm_tile_kernel<true, false, kT, kWM><<<grid, wblock, 0, stream>>>(g);
    else
      gemm_tile_kernel<true, true, kT, kWM><<<grid, wblock, 0, stream>>>(g);
    return;
  }
  if (!trans_a && !trans_b)
    gemm_kernel<false, false, kT><<<grid, block, 0, stream>>>(g);
  else if (!trans_a && trans_b)
    gemm_kernel<false, true, kT><<<grid, block, 0, stream>>>(g);
  else if (trans_a && !trans_b)
    gemm_kernel<true, false, kT><<<grid, block, 0, stream>>>(g);
  else
    gemm_kernel<true, true, kT><<<grid, block, 0, stream>>>(g);
}

bool aligned16(const void* p, int64_t ld) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0 && ld % 4 == 0;
}

}  // namespace

// 128 x 128 workgroup tiles when the batch has at least one such workgroup
// per CU, 64 x 64 tiles otherwise.  Whole tiles (M, N multiples of the edge,
// K of 64, 16-byte aligned operands and strides) take gemm_tile_kernel,
// anything else the bounds-checked gemm_kernel.
hipError_t launch_gemm(const GemmArgs& g, bool trans_a, bool trans_b, int32_t batch, hipStream_t stream) {
  if (g.M <= 0 || g.N <= 0 || batch <= 0) return hipSuccess;
  const int64_t big = int64_t((g.M + 127) / 128) * ((g.N + 127) / 128) * batch;
  const int t = big >= 256 ? 128 : 64;
  const bool whole = g.M % t == 0 && g.N % t == 0 && g.K > 0 && g.K % (2 * kSK) == 0 && aligned16(g.A, g.lda) &&
                     aligned16(g.B, g.ldb) && (batch == 1 || (g.sA % 4 == 0 && g.sB % 4 == 0));
  if (t == 128)
    launch_gemm_tile<128>(g, trans_a, trans_b, whole, batch, stream);
  else
    launch_gemm_tile<64>(g, trans_a, trans_b, whole, batch, stream);
  return hipGetLastError();
}

hipError_t launch_ns_prepare(const float* A, int n, float eps, double* partial, float* scal, float* Y, float* Z,
                             hipStream_t stream) {
  fro_partial_kernel<<<kNormBlocks, 256, 0, stream>>>(A, n, eps, partial);
  fro_final_kernel<<<1, 256, 0, stream>>>(partial, scal);
  const int64_t total = int64_t(n) * n;
  ns_init_kernel<<<dim3(unsigned((total + 255) / 256)), 256, 0, stream>>>(A, n, eps, scal, Y, Z);
  return hipGetLastError();
}

hipError_t launch_muon_vector(const float* m, float* x, int64_t len, float eps, float eta, float lam,
                              hipStream_t stream) {
  muon_vector_kernel<<<1, 256, 0, stream>>>(m, x, len, eps, eta, lam);
  return hipGetLastError();
}

// ---------------------------------------------------------------- static scratch

}  // namespace demo

// The Muon decode's workspace for callers that cannot allocate device memory
// (graph capture, tight serving loops): one array per device, held until the
// process ends.  Host code must not pass `scratch` itself to a kernel (in
// host code it names a host-side stand-in); it uses the device address that
// muon_scratch looks up.
static __device__ __align__(256) float scratch[demo::kMuonScratchBytes / sizeof(float)];

namespace demo {

hipError_t muon_scratch(int device, float** out) {
  static std::mutex mu;
  static float* address[kMaxDevices] = {};
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (address[device] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    address[device] = static_cast<float*>(p);
  }
  *out = address[device];
  return hipSuccess;
}

}  // namespace demo
