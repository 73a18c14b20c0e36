// Device helpers shared by the kernel files: tensor lookup in a launch
// table, streaming (non-temporal) loads and stores, gradient widening.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "launch.h"

namespace demo {
namespace {

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

template <class T>
__device__ __forceinline__ T stream_load(const T* p) {
  return __builtin_nontemporal_load(p);
}

__device__ __forceinline__ void stream_store(float v, float* p) { __builtin_nontemporal_store(v, p); }

// A gradient element widened to float32; kKeep: a plain load (the line may
// stay cached for a second read), otherwise a streaming one.
template <bool kBf16, bool kKeep = false>
__device__ __forceinline__ float load_src(const void* p, int64_t off) {
  if constexpr (kBf16) {
    const uint16_t* q = static_cast<const uint16_t*>(p) + off;
    const uint32_t b = kKeep ? uint32_t(*q) : uint32_t(stream_load(q));
    return __uint_as_float(b << 16);
  } else {
    const float* q = static_cast<const float*>(p) + off;
    return kKeep ? *q : stream_load(q);
  }
}

// Rows of one chunk through buffer instructions: the chunk origin sits in a
// buffer resource (scalar registers), row i is the scalar offset i * ldb and
// the lane's column the vector offset, so a row access needs no vector
// address arithmetic (a global access would spend a 64-bit vector add per
// row).  Offsets are 32-bit: usable while the chunk's rows span fewer than
// 2^31 bytes (buf_rows_fit); the range check of the resource is left open,
// addresses stay inside the tensor as with the global accesses.
struct RowBuf {
  __amdgpu_buffer_rsrc_t r;
  int32_t ldb;  // row stride in bytes
};
constexpr int kBufNt = 2;                 // cache policy: non-temporal
constexpr int kBufWord3 = 0x00020000;     // resource word 3: 32-bit data format
__device__ __forceinline__ bool buf_rows_fit(int64_t rows, int64_t ld_bytes) {
  return rows * ld_bytes < (int64_t(1) << 31);
}
__device__ __forceinline__ RowBuf row_buf(const void* base, int64_t ld_bytes) {
  RowBuf b;
  b.r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, kBufWord3);
  b.ldb = int32_t(ld_bytes);
  return b;
}
__device__ __forceinline__ float buf_load_f32(const RowBuf& b, int row, int32_t voff) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(b.r, voff, row * b.ldb, kBufNt));
}
__device__ __forceinline__ float buf_load_bf16(const RowBuf& b, int row, int32_t voff) {
  return __uint_as_float(uint32_t(__builtin_amdgcn_raw_buffer_load_b16(b.r, voff, row * b.ldb, kBufNt)) << 16);
}
__device__ __forceinline__ void buf_store_f32(const RowBuf& b, int row, int32_t voff, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), b.r, voff, row * b.ldb, kBufNt);
}

__device__ __forceinline__ float sign_of(float m) { return m > 0.f ? 1.f : (m < 0.f ? -1.f : 0.f); }

__device__ __forceinline__ void stream_store(uint64_t v, uint64_t* p) { __builtin_nontemporal_store(v, p); }

// What a decode launch writes: the parameters, a momentum (aggregated
// subtraction), both, the packed sign of M* (one-bit download), or M* itself
// (Muon, whose phi needs whole tensors).
constexpr int kToParams = 1;
constexpr int kToMomentum = 2;
constexpr int kToSigns = 4;
constexpr int kToMstar = 8;

// X <- X - eta (phi(m) + lambda X) for one element, phi = sign (kSign) or
// the identity.
template <bool kSign>
__device__ __forceinline__ float update(float x, float m, const DecodeParams& p) {
  const float ph = kSign ? sign_of(m) : m;
  return fmaf(-p.eta, fmaf(p.lam, x, ph), x);
}

// The update of a lane's 64 elements, phi chosen once for all of them (a
// per-element choice would spend the sign's instructions on the identity
// path as well).
__device__ __forceinline__ void update_all(float (&x)[64], const float (&m)[64], const DecodeParams& p) {
  if (p.phi_sign) {
#pragma unroll
    for (int i = 0; i < 64; ++i) x[i] = update<true>(x[i], m[i], p);
  } else {
#pragma unroll
    for (int i = 0; i < 64; ++i) x[i] = update<false>(x[i], m[i], p);
  }
}

// The same in place for a vector slab: elements 64 r of xp, those with
// 64 r < rem.
__device__ __forceinline__ void update_strided(float* __restrict__ xp, const float (&m)[64], int64_t rem,
                                               const DecodeParams& p) {
  if (p.phi_sign) {
#pragma unroll
    for (int r = 0; r < 64; ++r) {
      if (r * 64 < rem) stream_store(update<true>(stream_load(&xp[r * 64]), m[r], p), &xp[r * 64]);
    }
  } else {
#pragma unroll
    for (int r = 0; r < 64; ++r) {
      if (r * 64 < rem) stream_store(update<false>(stream_load(&xp[r * 64]), m[r], p), &xp[r * 64]);
    }
  }
}

// Scatter-add of one payload entry into a wave's LDS accumulator: the sum
// gains v and the 8-bit contributor count (byte *cnt) gains 1.  Plain LDS
// loads and stores, no atomic read-modify-write instruction: the lanes of one
// call hold distinct coefficients, and one wave's LDS operations complete in
// issue order, so the next call (the next worker) reads what this one wrote
// and every coefficient sums its terms in worker order.  The relaxed
// wave-scope atomic load/store only tell the compiler that other lanes touch
// these locations; they compile to ordinary ds_read / ds_write.
__device__ __forceinline__ void scatter_add(float* sum, uint8_t* cnt, float v) {
  const float s = __hip_atomic_load(sum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
  const uint8_t n = __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
  __hip_atomic_store(sum, s + v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
  __hip_atomic_store(cnt, uint8_t(n + 1u), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
}

// The same through LDS atomic adds whose results are not read (ds_add_f32,
// ds_add_u32 on the count's word): no wait between calls, and the order
// argument above still holds, so the sums are bitwise those of scatter_add.
// A count stays below 256 (at most 255 workers), so no byte carries into its
// neighbour.  Faster where a wave's calls have few active lanes (the
// per-sub-block scatter at chunk edge 128); slower than scatter_add for a
// full 64x64 chunk.
__device__ __forceinline__ void scatter_add_nowait(float* sum, uint32_t* cntw, uint32_t byte, float v) {
  __hip_atomic_fetch_add(sum, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
  __hip_atomic_fetch_add(cntw, 1u << (8u * byte), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
}

// Work item of workgroup b of n.  Workgroups go to the 8 XCDs round-robin
// (workgroup b to XCD b mod 8); this gives each XCD one contiguous range of
// items, so neighbouring chunks, whose payload entries share cache lines,
// meet in the same L2.  A bijection of 0 .. n-1.
__device__ __forceinline__ int xcd_item(int b, int n) {
  constexpr int kXcds = 8;
  const int x = b % kXcds, j = b / kXcds;
  const int q = n / kXcds, r = n % kXcds;  // XCDs below r take q + 1 items
  return x * q + min(x, r) + j;
}

// Orders one wave's LDS stores before its later LDS loads (other lanes of the
// same wave read what a lane wrote).  A wave's LDS operations complete in
// issue order, so no wait is needed; the fences keep the compiler from
// moving loads above the stores.  In a one-wave workgroup this replaces a
// workgroup barrier, which would also wait for every LDS operation in flight.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Lane i of v takes the wave-uniform value x (v_writelane: no compare, no
// select; i is a compile-time lane number).  x is read from the first active
// lane, which moves it into a scalar register where the compiler cannot
// prove it uniform (it is free where x already is one).
__device__ __forceinline__ void write_lane(uint32_t& v, uint32_t x, int i) {
  asm volatile("v_writelane_b32 %0, %1, %2" : "+v"(v) : "s"(__builtin_amdgcn_readfirstlane(x)), "i"(i));
}

// Compact wire format: chunk positions of kBits bits (12 at chunk edge 64,
// 14 at 128) packed as one little-endian bit string per worker, in groups of
// kWireGroup entries that fill whole 32-bit words.
template <int kBits>
struct WireFormat {
  static constexpr int kGroup = kBits == 12 ? 8 : 16;        // entries per group
  static constexpr int kWords = kGroup * kBits / 32;          // 32-bit words per group
  static_assert(kBits == 12 || kBits == 14, "positions of 12 or 14 bits");
  static_assert(kGroup * kBits == 32 * kWords, "groups fill whole words");
  // position of entry f from a worker's words (two words of f's group)
  static __device__ __forceinline__ uint32_t index(const uint32_t* __restrict__ s, int64_t f) {
    const int64_t bit = f * kBits;
    const int64_t d = bit >> 5;
    const int64_t last = (f / kGroup) * kWords + kWords - 1;
    const uint64_t pair = (uint64_t(s[d < last ? d + 1 : d]) << 32) | s[d];
    return uint32_t(pair >> (bit & 31)) & ((1u << kBits) - 1u);
  }
};

// number of set lanes of `mask` below this lane
__device__ __forceinline__ int lanes_below_mask(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(uint32_t(mask >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(mask), 0));
}

}  // namespace
}  // namespace demo
