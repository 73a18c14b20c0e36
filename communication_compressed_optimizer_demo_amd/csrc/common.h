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

template <bool kBf16>
__device__ __forceinline__ float load_src(const void* p, int64_t off) {
  if constexpr (kBf16) {
    const uint32_t b = stream_load(static_cast<const uint16_t*>(p) + off);
    return __uint_as_float(b << 16);
  } else {
    return stream_load(static_cast<const float*>(p) + off);
  }
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

__device__ __forceinline__ float update(float x, float m, const DecodeParams& p) {
  const float ph = p.phi_sign ? sign_of(m) : m;
  return fmaf(-p.eta, fmaf(p.lam, x, ph), x);
}

// number of set lanes of `mask` below this lane
__device__ __forceinline__ int lanes_below_mask(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(uint32_t(mask >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(mask), 0));
}

}  // namespace
}  // namespace demo
