// In-register transforms of one 64-element vector per lane.
//
// The orthonormal DCT-II basis of the DeMo codec ("DeMo: Decoupled Momentum
// Optimization", §3.4 Blockwise Linear Projection (DCT)) is applied with a
// fast factorisation instead of a 64x64 matrix product:
//   * DCT-II of length N splits into a DCT-II of length N/2 on the sums
//     x[n] + x[N-1-n] (even outputs) and a DCT-IV of length N/2 on the
//     differences x[n] - x[N-1-n] (odd outputs);
//   * a DCT-IV of length M is a complex DFT of length M/2 between a pre- and
//     a post-rotation (pairs x[2n] + i x[M-1-2n]);
//   * the DFT is radix-2 decimation in time.
// DCT-III (the transpose, used for the inverse) runs the same graph backwards.
// The orthonormal scale factors are folded into the rotation constants.
// Every twiddle is a compile-time constant computed in double precision and
// rounded once to float; all loops are unrolled at compile time so the
// arrays live in VGPRs.
//
// A caller-supplied basis (random orthonormal projection, same section) has
// no fast form; DenseBasis applies it to 64x64 blocks as two matrix products
// on the matrix cores, float32-accurate through a three-way bfloat16 split
// of both operands, and to vectors as a plain matrix-vector product whose
// rows are read through uniform (scalar) loads.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

namespace demo {
namespace xf {

// ---------------------------------------------------------------- compile-time trig

constexpr double kPi = 3.14159265358979323846264338327950288;

constexpr double taylor_sin(double x) {  // |x| <= pi/4
  double x2 = x * x, term = x, sum = x;
  for (int n = 1; n < 14; ++n) {
    term *= -x2 / double((2 * n) * (2 * n + 1));
    sum += term;
  }
  return sum;
}

constexpr double taylor_cos(double x) {  // |x| <= pi/4
  double x2 = x * x, term = 1.0, sum = 1.0;
  for (int n = 1; n < 14; ++n) {
    term *= -x2 / double((2 * n - 1) * (2 * n));
    sum += term;
  }
  return sum;
}

// cos(pi * p / q), q > 0, by reduction to [0, pi/4]
constexpr double cospi(long p, long q) {
  long t = p % (2 * q);
  if (t < 0) t += 2 * q;
  if (t > q) t = 2 * q - t;  // angle in [0, pi]
  double sign = 1.0;
  if (2 * t > q) {  // angle in (pi/2, pi]
    t = q - t;
    sign = -1.0;
  }
  if (4 * t > q) return sign * taylor_sin(kPi * double(q - 2 * t) / double(2 * q));
  return sign * taylor_cos(kPi * double(t) / double(q));
}

// sin(pi p / q) = cos(pi (2p - q) / (2q))
constexpr double sinpi(long p, long q) { return cospi(2 * p - q, 2 * q); }

// tan(theta / 2) = sin(theta) / (1 + cos(theta)), theta = pi p / q in [0, pi/2]
constexpr double tanhalfpi(long p, long q) { return sinpi(p, q) / (1.0 + cospi(p, q)); }

constexpr double csqrt(double v) {
  double r = v > 1.0 ? v : 1.0;
  for (int i = 0; i < 64; ++i) r = 0.5 * (r + v / r);
  return r;
}

// Scale tags (C++17 has no floating-point template parameters).
struct Unit {
  static constexpr double v = 1.0;
};
template <int N>
struct Ortho {  // sqrt(2 / N): the non-DC row scale of the orthonormal DCT-II of length N
  static constexpr double v = csqrt(2.0 / double(N));
};

// ---------------------------------------------------------------- compile-time loop

template <int B, int E, class F>
__host__ __device__ __forceinline__ void sfor(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    sfor<B + 1, E>(f);
  }
}

// ---------------------------------------------------------------- complex DFT, radix 2

// Z[k] = sum_n z[n] exp(-2 pi i n k / L), natural order in and out.
template <int L>
__host__ __device__ __forceinline__ void fft(float (&re)[L], float (&im)[L]) {
  if constexpr (L == 1) {
    return;
  } else if constexpr (L == 2) {
    const float r0 = re[0], i0 = im[0];
    re[0] = r0 + re[1];
    im[0] = i0 + im[1];
    re[1] = r0 - re[1];
    im[1] = i0 - im[1];
  } else {
    constexpr int H = L / 2;
    float er[H], ei[H], orr[H], oi[H];
    sfor<0, H>([&](auto I) {
      constexpr int n = decltype(I)::value;
      er[n] = re[2 * n];
      ei[n] = im[2 * n];
      orr[n] = re[2 * n + 1];
      oi[n] = im[2 * n + 1];
    });
    fft<H>(er, ei);
    fft<H>(orr, oi);
    sfor<0, H>([&](auto I) {
      constexpr int k = decltype(I)::value;
      float tr, ti;
      if constexpr (k == 0) {
        tr = orr[k];
        ti = oi[k];
      } else if constexpr (4 * k == L) {  // times -i
        tr = oi[k];
        ti = -orr[k];
      } else {
        // (orr + i oi) exp(-i theta), theta = 2 pi k / L, folded into the
        // butterfly: with theta = phi (k < L/4) or phi + pi/2 (a free factor
        // -i), and g = cos phi, w = tan phi for phi <= pi/4, else g = sin phi,
        // w = cot phi, the product is g (p + i q) with p, q one FMA each;
        // the four outputs are then one FMA each (6 instead of 8).
        constexpr bool kRot = 4 * k > L;  // theta > pi/2
        constexpr int k2 = kRot ? k - L / 4 : k;  // phi = 2 pi k2 / L
        constexpr bool kLow = 8 * k2 <= L;        // phi <= pi/4
        constexpr float g = float(kLow ? cospi(2 * k2, L) : sinpi(2 * k2, L));
        constexpr float w = float(kLow ? sinpi(2 * k2, L) / cospi(2 * k2, L) : cospi(2 * k2, L) / sinpi(2 * k2, L));
        float p, q;
        if constexpr (kLow) {
          p = fmaf(w, oi[k], orr[k]);
          q = fmaf(-w, orr[k], oi[k]);
        } else {
          p = fmaf(w, orr[k], oi[k]);
          q = fmaf(w, oi[k], -orr[k]);
        }
        if constexpr (kRot) {  // times -i: (p, q) -> (q, -p)
          re[k] = fmaf(g, q, er[k]);
          re[k + H] = fmaf(-g, q, er[k]);
          im[k] = fmaf(-g, p, ei[k]);
          im[k + H] = fmaf(g, p, ei[k]);
        } else {
          re[k] = fmaf(g, p, er[k]);
          re[k + H] = fmaf(-g, p, er[k]);
          im[k] = fmaf(g, q, ei[k]);
          im[k + H] = fmaf(-g, q, ei[k]);
        }
        return;
      }
      re[k] = er[k] + tr;
      im[k] = ei[k] + ti;
      re[k + H] = er[k] - tr;
      im[k + H] = ei[k] - ti;
    });
  }
}

// ---------------------------------------------------------------- DCT-IV

// (u, v) = (a cos t + b sin t, b cos t - a sin t), t = pi P / Q in (0, pi/2):
// the rotation as three shears (lifting steps) of tan(t/2), sin(t),
// tan(t/2), each one FMA.
template <long P, long Q>
__host__ __device__ __forceinline__ void rotate_lift(float a, float b, float& u, float& v) {
  constexpr float h = float(tanhalfpi(P, Q));
  constexpr float s = float(sinpi(P, Q));
  const float x1 = fmaf(h, b, a);
  v = fmaf(-s, x1, b);
  u = fmaf(h, v, x1);
}

// y[m] = Pre*Post * sum_n x[n] cos(pi (2n+1)(2m+1) / (4M)).
// Pre and Post are scale tags; only their product matters mathematically,
// they say on which side of the graph the factor is folded in.
template <int M, class Pre, class Post>
__host__ __device__ __forceinline__ void dct4(float (&x)[M]) {
  constexpr double g = Pre::v * Post::v;
  if constexpr (M == 1) {
    x[0] *= float(g * cospi(1, 4));
  } else if constexpr (M == 2) {
    constexpr float c1 = float(g * cospi(1, 8));
    constexpr float c3 = float(g * cospi(3, 8));
    const float a = x[0], b = x[1];
    x[0] = fmaf(a, c1, b * c3);
    x[1] = fmaf(a, c3, -(b * c1));
  } else {
    constexpr int L = M / 2;
    float re[L], im[L];
    sfor<0, L>([&](auto I) {
      constexpr int n = decltype(I)::value;
      const float a = x[2 * n], b = x[M - 1 - 2 * n];
      if constexpr (Pre::v == 1.0) {
        // unscaled rotation by theta < pi/2 as three lifting steps
        // (tan(theta/2), sin(theta), tan(theta/2)): 3 FMAs instead of 4 ops
        rotate_lift<4 * n + 1, 4 * M>(a, b, re[n], im[n]);
      } else {
        constexpr float c = float(Pre::v * cospi(4 * n + 1, 4 * M));
        constexpr float s = float(Pre::v * sinpi(4 * n + 1, 4 * M));
        re[n] = fmaf(a, c, b * s);
        im[n] = fmaf(b, c, -(a * s));
      }
    });
    fft<L>(re, im);
    sfor<0, L>([&](auto I) {
      constexpr int k = decltype(I)::value;
      constexpr float c = float(Post::v * cospi(k, M));
      constexpr float s = float(Post::v * sinpi(k, M));
      float ur, ui;
      if constexpr (k == 0) {
        if constexpr (Post::v == 1.0) {
          ur = re[0];
          ui = im[0];
        } else {
          ur = re[0] * c;
          ui = im[0] * c;
        }
      } else if constexpr (Post::v == 1.0) {
        rotate_lift<k, M>(re[k], im[k], ur, ui);
      } else {
        ur = fmaf(re[k], c, im[k] * s);
        ui = fmaf(im[k], c, -(re[k] * s));
      }
      x[2 * k] = ur;
      x[M - 1 - 2 * k] = -ui;
    });
  }
}

// ---------------------------------------------------------------- DCT-II / DCT-III

// Forward: X[k] = S_k * sum_n x[n] cos(pi (2n+1) k / (2N)), with S_k = Sig::v
// for k > 0 and Sig::v / sqrt(2) for k = 0.  Sig = Ortho<N> gives the
// orthonormal DCT-II.
template <int N, class Sig>
__host__ __device__ __forceinline__ void dct2(float (&x)[N]) {
  constexpr double r2 = 0.70710678118654752440084436210484904;
  if constexpr (N == 1) {
    x[0] *= float(Sig::v * r2);
  } else if constexpr (N == 2) {
    constexpr float h = float(Sig::v * r2);
    const float a = x[0], b = x[1];
    x[0] = (a + b) * h;
    x[1] = (a - b) * h;
  } else {
    constexpr int H = N / 2;
    float a[H], b[H];
    sfor<0, H>([&](auto I) {
      constexpr int n = decltype(I)::value;
      a[n] = x[n] + x[N - 1 - n];
      b[n] = x[n] - x[N - 1 - n];
    });
    dct2<H, Sig>(a);
    dct4<H, Unit, Sig>(b);
    sfor<0, H>([&](auto I) {
      constexpr int m = decltype(I)::value;
      x[2 * m] = a[m];
      x[2 * m + 1] = b[m];
    });
  }
}

// Inverse (transpose of dct2 with the same scaling): x[n] = sum_k S_k X[k] cos(pi (2n+1) k / (2N)).
template <int N, class Sig>
__host__ __device__ __forceinline__ void dct3(float (&x)[N]) {
  constexpr double r2 = 0.70710678118654752440084436210484904;
  if constexpr (N == 1) {
    x[0] *= float(Sig::v * r2);
  } else if constexpr (N == 2) {
    constexpr float h = float(Sig::v * r2);
    const float a = x[0], b = x[1];
    x[0] = (a + b) * h;
    x[1] = (a - b) * h;
  } else {
    constexpr int H = N / 2;
    float a[H], b[H];
    sfor<0, H>([&](auto I) {
      constexpr int m = decltype(I)::value;
      a[m] = x[2 * m];
      b[m] = x[2 * m + 1];
    });
    dct3<H, Sig>(a);
    dct4<H, Sig, Unit>(b);
    sfor<0, H>([&](auto I) {
      constexpr int n = decltype(I)::value;
      x[n] = a[n] + b[n];
      x[N - 1 - n] = a[n] - b[n];
    });
  }
}

// ---------------------------------------------------------------- bases as kernel policies

// Orthonormal DCT-II on both dimensions (P0 = P1 = P).
struct DctBasis {
  static constexpr bool kMatrixCores = false;
  // y = P x
  __host__ __device__ __forceinline__ void fwd0(float (&x)[64]) const { dct2<64, Ortho<64>>(x); }
  __host__ __device__ __forceinline__ void fwd1(float (&x)[64]) const { dct2<64, Ortho<64>>(x); }
  // y = P^T x
  __host__ __device__ __forceinline__ void inv0(float (&x)[64]) const { dct3<64, Ortho<64>>(x); }
  __host__ __device__ __forceinline__ void inv1(float (&x)[64]) const { dct3<64, Ortho<64>>(x); }
};

// P0 = P1 = I: the chunk is ranked and sparsified in the parameter domain.
struct IdentityBasis {
  static constexpr bool kMatrixCores = false;
  __host__ __device__ __forceinline__ void fwd0(float (&)[64]) const {}
  __host__ __device__ __forceinline__ void fwd1(float (&)[64]) const {}
  __host__ __device__ __forceinline__ void inv0(float (&)[64]) const {}
  __host__ __device__ __forceinline__ void inv1(float (&)[64]) const {}
};

// Caller-supplied orthonormal P0 / P1 (64 x 64, row-major, rows are basis vectors).
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct DenseBasis {
  const float* __restrict__ p0;
  const float* __restrict__ p1;
  // A 64x64 block goes through the matrix cores (two 64x64x64 products per
  // direction) instead of one matrix-vector product per lane.
  static constexpr bool kMatrixCores = true;

  static __device__ __forceinline__ void apply(const float* __restrict__ P, float (&x)[64]) {
    float y[64];
#pragma unroll
    for (int u = 0; u < 64; ++u) {
      float acc = 0.f;
#pragma unroll
      for (int n = 0; n < 64; ++n) acc = fmaf(P[u * 64 + n], x[n], acc);
      y[u] = acc;
    }
#pragma unroll
    for (int u = 0; u < 64; ++u) x[u] = y[u];
  }
  static __device__ __forceinline__ void apply_t(const float* __restrict__ P, float (&x)[64]) {
    float y[64];
#pragma unroll
    for (int n = 0; n < 64; ++n) y[n] = 0.f;
#pragma unroll
    for (int u = 0; u < 64; ++u) {
#pragma unroll
      for (int n = 0; n < 64; ++n) y[n] = fmaf(P[u * 64 + n], x[u], y[n]);
    }
#pragma unroll
    for (int n = 0; n < 64; ++n) x[n] = y[n];
  }
  __device__ __forceinline__ void fwd0(float (&x)[64]) const { apply(p0, x); }
  __device__ __forceinline__ void fwd1(float (&x)[64]) const { apply(p1, x); }
  __device__ __forceinline__ void inv0(float (&x)[64]) const { apply_t(p0, x); }
  __device__ __forceinline__ void inv1(float (&x)[64]) const { apply_t(p1, x); }

  // --- 64x64 blocks on the matrix cores (one wave; `tile` is 64 rows of kLd
  // floats in LDS).  A 32x32 result sits in register v of lane l at row
  // 8 (v / 4) + 4 (l / 32) + v % 4, column l % 32.  Each lane half feeds
  // one contiguous half of the 64-deep k range: k = kk + 32 (l / 32),
  // kk = 0..31, so a lane walks one half of a row or column.

  // (x, y) rounded to bfloat16 in one packed conversion, x in the low half.
  static __device__ __forceinline__ uint32_t pack_pair(float x, float y) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x, y}, bf16x2));
  }
  // The packed rounding of (x, y), leaving what it left out in x and y (exact
  // in float32).
  static __device__ __forceinline__ uint32_t peel_pair(float& x, float& y) {
    const uint32_t bits = pack_pair(x, y);
    x -= __uint_as_float(bits << 16);
    y -= __uint_as_float(bits & 0xffff0000u);
    return bits;
  }

  // D = A * B for 64x64 operands given as functions (m, k) -> A, (k, n) -> B
  // of this lane's (row / column within a 32-tile, kk), k = kk + 32 (lane / 32).
  // Float32-accurate products on the bfloat16 matrix cores: every operand is
  // split exactly into three bfloat16 parts (8 + 8 + 8 significant bits,
  // each the rounding of what the previous parts leave) and the six part
  // products down to the third order (a1b1, a1b2, a2b1, a1b3, a2b2, a3b1;
  // each of the three dropped ones is at most 2^-24 |ab|) are accumulated in
  // float32, smallest first.  v_mfma_f32_32x32x16_bf16: lane l gives
  // A[l % 32][8 (l / 32) + j] and B[8 (l / 32) + j][l % 32], j = 0..7; step
  // s of four takes kk = 8 s + j, so both operands pair the same k.
  template <class FA, class FB>
  static __device__ __forceinline__ void product(f32x16 (&d)[2][2], FA a_of, FB b_of) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) d[i][j][v] = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 a[2][3], b[2][3];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float x0 = a_of(t, 8 * s + 2 * j), x1 = a_of(t, 8 * s + 2 * j + 1);
          a[t][0][j] = peel_pair(x0, x1);
          a[t][1][j] = peel_pair(x0, x1);
          a[t][2][j] = pack_pair(x0, x1);
          float y0 = b_of(t, 8 * s + 2 * j), y1 = b_of(t, 8 * s + 2 * j + 1);
          b[t][0][j] = peel_pair(y0, y1);
          b[t][1][j] = peel_pair(y0, y1);
          b[t][2][j] = pack_pair(y0, y1);
        }
      constexpr int kTa[6] = {2, 1, 0, 1, 0, 0}, kTb[6] = {0, 1, 2, 0, 1, 0};
#pragma unroll
      for (int p = 0; p < 6; ++p)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            d[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[i][kTa[p]]),
                                                              __builtin_bit_cast(bf16x8, b[j][kTb[p]]), d[i][j], 0, 0,
                                                              0);
    }
  }

  // Power-of-two factor applied to a block before its products and undone
  // after them: 1 unless the block's largest magnitude is below 2^-90, where
  // the bfloat16 parts of its values and their part products would reach
  // the subnormal range and be lost on the matrix cores (a block at 1e-36
  // otherwise comes out with errors near 1e-5 of its norm).  Scaling by a
  // power of two is exact and the products are linear, so the result is
  // the one without scaling wherever nothing underflows.  Returns the
  // exponent of the factor (0: none).
  static __device__ __forceinline__ int block_scale(const float (&x)[64]) {
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 64; ++i) m = fmaxf(m, fabsf(x[i]));
    if (__builtin_amdgcn_ballot_w64(m >= 0x1p-90f) != 0) return 0;  // the common case
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if (m == 0.f) return 0;
    const int e = int(__builtin_amdgcn_readfirstlane(__float_as_uint(m) >> 23));  // biased exponent
    return 127 - e;  // m 2^(127 - e) is in [1, 2)
  }

  // The 64x64 result into the tile, row-major.
  template <int kLd>
  static __device__ __forceinline__ void store_result(const f32x16 (&d)[2][2], float* tile, int lane) {
    const int h = lane >> 5, c = lane & 31;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) tile[(32 * i + 8 * (v >> 2) + 4 * h + (v & 3)) * kLd + 32 * j + c] = d[i][j][v];
  }

  // The tile belongs to this one wave: its LDS accesses only need ordering
  // (a wave's LDS operations complete in issue order).
  static __device__ __forceinline__ void lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // Forward: x holds column `lane` of the block B (x[i] = B[i][lane]); on
  // return x holds row `lane` of Q = P0 B P1^T.
  template <int kLd>
  __device__ __forceinline__ void forward2d(float (&x)[64], float* tile, int lane) const {
    const int h = lane >> 5, c = lane & 31;
    const int sc = block_scale(x);
    if (sc != 0) {
#pragma unroll
      for (int i = 0; i < 64; ++i) x[i] = ldexpf(x[i], sc);
    }
#pragma unroll
    for (int i = 0; i < 64; ++i) tile[i * kLd + lane] = x[i];
    // this lane's rows of P0 (A of the first product) and P1 (B^T of the second): 32 contiguous k each
    f32x4 pr[2][8];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int q = 0; q < 8; ++q) pr[t][q] = *reinterpret_cast<const f32x4*>(p0 + (32 * t + c) * 64 + 32 * h + 4 * q);
    lds_sync();
    f32x16 d[2][2];
    // C = P0 B
    product(d, [&](int t, int kk) { return pr[t][kk >> 2][kk & 3]; },
            [&](int t, int kk) { return tile[(kk + 32 * h) * kLd + 32 * t + c]; });
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int q = 0; q < 8; ++q) pr[t][q] = *reinterpret_cast<const f32x4*>(p1 + (32 * t + c) * 64 + 32 * h + 4 * q);
    lds_sync();
    store_result<kLd>(d, tile, lane);
    lds_sync();
    // Q = C P1^T: B[k][n] = P1[n][k]
    product(d, [&](int t, int kk) { return tile[(32 * t + c) * kLd + kk + 32 * h]; },
            [&](int t, int kk) { return pr[t][kk >> 2][kk & 3]; });
    lds_sync();
    store_result<kLd>(d, tile, lane);
    lds_sync();
#pragma unroll
    for (int v = 0; v < 64; ++v) x[v] = tile[lane * kLd + v];
    lds_sync();
    if (sc != 0) {
#pragma unroll
      for (int v = 0; v < 64; ++v) x[v] = ldexpf(x[v], -sc);
    }
  }

  // Inverse: x holds row `lane` of Q (x[v] = Q[lane][v]); on return x holds
  // column `lane` of P0^T Q P1.
  template <int kLd>
  __device__ __forceinline__ void inverse2d(float (&x)[64], float* tile, int lane) const {
    const int h = lane >> 5, c = lane & 31;
    const int sc = block_scale(x);
    if (sc != 0) {
#pragma unroll
      for (int v = 0; v < 64; ++v) x[v] = ldexpf(x[v], sc);
    }
#pragma unroll
    for (int v = 0; v < 64; ++v) tile[lane * kLd + v] = x[v];
    lds_sync();
    f32x16 d[2][2];
    // D = Q P1 (rows of P1 read a coalesced 128 bytes per lane half)
    product(d, [&](int t, int kk) { return tile[(32 * t + c) * kLd + kk + 32 * h]; },
            [&](int t, int kk) { return p1[(kk + 32 * h) * 64 + 32 * t + c]; });
    lds_sync();
    store_result<kLd>(d, tile, lane);
    lds_sync();
    // X = P0^T D: A[m][k] = P0[k][m]
    product(d, [&](int t, int kk) { return p0[(kk + 32 * h) * 64 + 32 * t + c]; },
            [&](int t, int kk) { return tile[(kk + 32 * h) * kLd + 32 * t + c]; });
    lds_sync();
    store_result<kLd>(d, tile, lane);
    lds_sync();
#pragma unroll
    for (int i = 0; i < 64; ++i) x[i] = tile[i * kLd + lane];
    lds_sync();
    if (sc != 0) {
#pragma unroll
      for (int i = 0; i < 64; ++i) x[i] = ldexpf(x[i], -sc);
    }
  }
};

}  // namespace xf
}  // namespace demo
