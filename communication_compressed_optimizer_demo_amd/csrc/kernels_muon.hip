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
// converges to (A + eps I)^(-1/2) sqrt(s).  Every product is a dense GEMM
// on the matrix cores at float32 accuracy; the last one, Z M / sqrt(s) (or
// M Z / sqrt(s)), carries the parameter update in its epilogue.  A vector is one column:
// m / sqrt(m.m + eps).
//
// Two GEMM kernels; a 32 x 32 MFMA accumulator holds
// D[8 (v / 4) + 4 (l / 32) + (v % 4)][l % 32] in register v of lane l:
//  - gemm_kernel (any shape): v_mfma_f32_32x32x2f32 (lane l supplies
//    A[l % 32][l / 32] and B[l / 32][l % 32]); 128 x 128 (or 64 x 64)
//    output tile per 256-thread workgroup, 2 x 2 waves; K advances kBK per
//    LDS stage, double-buffered, bounds-checked 4-byte loads of the next
//    stage issued before the current stage's MFMAs;
//  - gemm_tile_kernel (whole tiles, where all of the Newton-Schulz work
//    runs): the same tiles and waves on the bfloat16 matrix cores, every
//    float32 operand split exactly into three bfloat16 parts (below).
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
// For products whose M and N are multiples of the tile edge and K of
// kWholeK, with 16-byte aligned operands.  Float32-accurate products on the bfloat16 matrix
// cores (v_mfma_f32_32x32x16_bf16, 16 k values per step): every operand value
// is split exactly into three bfloat16 parts (8 + 8 + 8 significant bits,
// each the rounding of what the previous parts leave) as it is staged into
// LDS, and each MFMA tile accumulates the six part products down to the third
// order (a1b1, a1b2, a2b1, a1b3, a2b2, a3b1; each of the three dropped ones
// is at most 2^-24 |ab|) in float32, smallest first.
//  - K advances kSK per stage (one MFMA k-step at 128 x 128 tiles, two at
//    64 x 64); each thread loads its share of a stage with two 16-byte
//    global loads, two register sets holding stages s+1 and s+2 while stage
//    s is multiplied, and splits it as it stores it to LDS (double-buffered,
//    so two workgroups fit a CU);
//  - in LDS each part is kept k-contiguous per row of the tile (row along M
//    for A, along N for B), so that a lane reads the eight k values it feeds
//    to one MFMA step with one 16-byte load: lane l gives
//    A[l % 32][8 (l / 32) + j] and B[8 (l / 32) + j][l % 32], j = 0..7;
//  - an operand whose rows run along K in memory is staged eight k values
//    per thread and row (one 16-byte store per part); one whose rows run
//    along M or N two k values for four rows, eight lanes reading one
//    128-byte row segment.
// Whole tiles need K to be a multiple of this (two stages of the deepest kSK).
constexpr int kWholeK = 64;

// Native vectors (not HIP's float4 struct) so the staging registers stay registers.
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// (x, y) rounded to bfloat16 in one packed conversion, x in the low half.
__device__ __forceinline__ uint32_t pack_pair(float x, float y) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x, y}, bf16x2));
}

// The packed rounding of (x, y), leaving what it left out in x and y (exact
// in float32).
__device__ __forceinline__ uint32_t peel_pair(float& x, float& y) {
  const uint32_t bits = pack_pair(x, y);
  x -= __uint_as_float(bits << 16);
  y -= __uint_as_float(bits & 0xffff0000u);
  return bits;
}

// The three packed parts of (x, y), high part first.
__device__ __forceinline__ void split_pair(float x, float y, uint32_t (&w)[3]) {
  w[0] = peel_pair(x, y);
  w[1] = peel_pair(x, y);
  w[2] = pack_pair(x, y);
}

// One operand's stage: kT rows (along M for A, N for B) by kSK values of k,
// moved by 256 threads (kT * kSK / 4 = 512 16-byte loads, two per thread).
// kKc: element (row, k) sits at X[row * ld + k] (rows along K in memory);
// otherwise at X[k * ld + row].  LDS: part p, row r, k pair q at word
// p * kPart + slot(r) * kPitch + q.  The pitch of kSK / 2 + 4 words puts the
// 16-byte reads of 16 consecutive rows on distinct banks; slot(r) swaps
// rows r and r ^ 2 in every second block of 16 rows, which keeps that and
// puts the 4-byte stores of the k-major staging (eight row groups of four
// rows, eight k pairs) on distinct banks too.
template <bool kKc, int kT, int kSK>
struct SplitOperand {
  static_assert(kT * kSK / 4 == 512, "two 16-byte loads per thread and stage");
  static constexpr int kPitch = kSK / 2 + 4;
  static constexpr int kPart = kT * kPitch;
  static constexpr int kWords = 3 * kPart;
  static constexpr int kQ = kSK / 2;  // k pairs per row and stage
  static constexpr int kG = kSK / 8;  // groups of eight k per row and stage

  static __device__ __forceinline__ int slot(int r) { return r ^ ((r >> 3) & 2); }

  __device__ static void load(f32x4 (&r)[2], const float* __restrict__ X, int64_t ld, int r0, int k0, int tid) {
    if constexpr (kKc) {
      // row tid / kG, k 8 (tid % kG) .. + 7
      const float* p = X + int64_t(r0 + tid / kG) * ld + k0 + 8 * (tid % kG);
      r[0] = *reinterpret_cast<const f32x4*>(p);
      r[1] = *reinterpret_cast<const f32x4*>(p + 4);
    } else {
      // rows 4 r4 .. 4 r4 + 3 at k = 2 q (j = 0) and 2 q + 1 (j = 1); eight
      // lanes read one 128-byte row segment
      const int r4 = tid / (8 * kQ) * 8 + (tid & 7), q = (tid >> 3) % kQ;
#pragma unroll
      for (int j = 0; j < 2; ++j) r[j] = *reinterpret_cast<const f32x4*>(X + int64_t(k0 + 2 * q + j) * ld + r0 + 4 * r4);
    }
  }

  __device__ static void store(const f32x4 (&r)[2], uint32_t* s, int tid) {
    if constexpr (kKc) {
      uint32_t w[4][3];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        split_pair(r[j][0], r[j][1], w[2 * j]);
        split_pair(r[j][2], r[j][3], w[2 * j + 1]);
      }
      uint32_t* p = s + slot(tid / kG) * kPitch + 4 * (tid % kG);
#pragma unroll
      for (int part = 0; part < 3; ++part)
        *reinterpret_cast<u32x4*>(p + part * kPart) = u32x4{w[0][part], w[1][part], w[2][part], w[3][part]};
    } else {
      const int r4 = tid / (8 * kQ) * 8 + (tid & 7), q = (tid >> 3) % kQ;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint32_t w[3];
        split_pair(r[0][c], r[1][c], w);
#pragma unroll
        for (int part = 0; part < 3; ++part) s[part * kPart + slot(4 * r4 + c) * kPitch + q] = w[part];
      }
    }
  }

  // The three parts of this lane's eight k values of step st for tile row r.
  __device__ static void fragment(const uint32_t* s, int r, int st, int h, u32x4 (&f)[3]) {
    const uint32_t* p = s + slot(r) * kPitch + 8 * st + 4 * h;
#pragma unroll
    for (int part = 0; part < 3; ++part) f[part] = *reinterpret_cast<const u32x4*>(p + part * kPart);
  }
};

// Four waves in a 2 x 2 grid; wave tile (kT / 2) x (kT / 2), i.e. kMT x kMT
// MFMA tiles.  K advances kSK per stage: 16 at kT = 128 (one MFMA k-step;
// 72 KB of LDS, two workgroups per CU), 32 at kT = 64.
template <bool kTA, bool kTB, int kT>
__global__ __launch_bounds__(256) void gemm_tile_kernel(GemmArgs g) {
  select_product(g);
  constexpr int kSK = kT == 128 ? 16 : 32;
  using OA = SplitOperand<!kTA, kT, kSK>;
  using OB = SplitOperand<kTB, kT, kSK>;
  constexpr int kMT = kT / 64;
  constexpr int kAcc = kMT == 1 ? 2 : 1;  // a lone 32 x 32 tile alternates two accumulators
  __shared__ __align__(16) uint32_t As[2][OA::kWords];
  __shared__ __align__(16) uint32_t Bs[2][OB::kWords];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, i32 = lane & 31;
  const int wm = w >> 1, wn = w & 1;
  // Workgroups reach the eight XCDs round-robin by linear id.  When the tile
  // grid splits into a 4 x 2 arrangement of equal blocks, XCD k gets block
  // (k / 2, k % 2), so each XCD's L2 serves a quarter of A's row blocks and
  // half of B's column blocks instead of all of A.
  int tx = blockIdx.x, ty = blockIdx.y;
  if (gridDim.x % 2 == 0 && gridDim.y % 4 == 0) {
    const int l = blockIdx.x + gridDim.x * blockIdx.y, k = l & 7, m = l >> 3;
    const int bw = gridDim.x / 2, bh = gridDim.y / 4;
    tx = (k & 1) * bw + m % bw;
    ty = (k >> 1) * bh + m / bw;
  }
  const int m0 = ty * kT, n0 = tx * kT;
  const int nk = g.K / kSK;

  floatx16 acc[kMT][kMT][kAcc];
#pragma unroll
  for (int i = 0; i < kMT; ++i)
#pragma unroll
    for (int j = 0; j < kMT; ++j)
#pragma unroll
      for (int a = 0; a < kAcc; ++a)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][a][v] = 0.f;

  // Multiply one LDS stage: kSK / 16 k-steps of six part products each.
  auto compute = [&](const uint32_t* sa, const uint32_t* sb) {
#pragma unroll
    for (int st = 0; st < kSK / 16; ++st) {
      u32x4 a[kMT][3], b[kMT][3];
#pragma unroll
      for (int t = 0; t < kMT; ++t) {
        OA::fragment(sa, wm * (kT / 2) + t * 32 + i32, st, h, a[t]);
        OB::fragment(sb, wn * (kT / 2) + t * 32 + i32, st, h, b[t]);
      }
      constexpr int kPa[6] = {2, 1, 0, 1, 0, 0}, kPb[6] = {0, 1, 2, 0, 1, 0};
#pragma unroll
      for (int p = 0; p < 6; ++p)
#pragma unroll
        for (int i = 0; i < kMT; ++i)
#pragma unroll
          for (int j = 0; j < kMT; ++j)
            acc[i][j][p % kAcc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, a[i][kPa[p]]), __builtin_bit_cast(bf16x8, b[j][kPb[p]]),
                acc[i][j][p % kAcc], 0, 0, 0);
    }
  };

  f32x4 ra0[2], rb0[2], ra1[2], rb1[2];
  auto load = [&](f32x4 (&ra)[2], f32x4 (&rb)[2], int kt) {
    OA::load(ra, g.A, g.lda, m0, kt * kSK, tid);
    OB::load(rb, g.B, g.ldb, n0, kt * kSK, tid);
  };
  auto store = [&](const f32x4 (&ra)[2], const f32x4 (&rb)[2], int buf) {
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
  for (int ti = 0; ti < kMT; ++ti) {
#pragma unroll
    for (int tj = 0; tj < kMT; ++tj) {
      const int col = n0 + wn * (kT / 2) + tj * 32 + i32;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wm * (kT / 2) + ti * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
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
    if (!trans_a && !trans_b)
      gemm_tile_kernel<false, false, kT><<<grid, block, 0, stream>>>(g);
    else if (!trans_a && trans_b)
      gemm_tile_kernel<false, true, kT><<<grid, block, 0, stream>>>(g);
    else if (trans_a && !trans_b)
      gemm_tile_kernel<true, false, kT><<<grid, block, 0, stream>>>(g);
    else
      gemm_tile_kernel<true, true, kT><<<grid, block, 0, stream>>>(g);
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
  const bool whole = g.M % t == 0 && g.N % t == 0 && g.K > 0 && g.K % kWholeK == 0 && aligned16(g.A, g.lda) &&
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
