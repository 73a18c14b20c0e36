// Kernel-argument layout shared by the host side (codec.cpp) and the kernels.
//
// A launch covers up to kMaxTensorsPerLaunch tensors of both kinds.  The
// tensor table travels by value in the kernel arguments, so no device-side
// table is allocated or copied.  A work item is one 64x64 chunk of a matrix,
// or one slab of up to 64 consecutive 64-element chunks of a vector; items
// are numbered consecutively over the launch's tensors in table order (the
// host lists the vectors first).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace demo {

constexpr int kChunk = 64;       // default chunk edge
constexpr int kChunkLarge = 128;  // the other chunk edge built
constexpr int kMaxTensorsPerLaunch = 96;
constexpr int kMaxWorkers = 255;  // counts are kept in 8 bits

struct TensorSlot {
  void* aux;            // encode: gradient (fp32 or bf16, read only); decode: momentum (in/out), the
                        // tensor's packed sign words or M* (out), or null; sign apply: sign words (in)
  float* dst;           // encode: momentum (in/out); decode, sign apply: parameters (in/out) or null
  int64_t entry_begin;  // payload entry of the tensor's first chunk
  int32_t rows;         // 2-D: dim 0; 1-D: length
  int32_t cols;         // 2-D: dim 1 (>= 1); 1-D: 0, which marks a vector
  int32_t item_begin;   // first work item of this tensor within the launch
};

struct LaunchTable {
  int32_t n;
  int32_t items;
  TensorSlot t[kMaxTensorsPerLaunch];
};
// Kernel arguments are limited to 4 KiB; the table leaves room for the
// parameter structs and the basis pointers.
static_assert(sizeof(TensorSlot) == 40, "tensor slot layout");
static_assert(sizeof(LaunchTable) <= 3856, "launch table too large for the kernel argument segment");

struct EncodeParams {
  float* pay_val;
  uint16_t* pay_idx;
  float beta;
  float gcoef;  // (1 - beta) or 1
  float alpha;
  int32_t keff2;           // entries per s x s chunk
  int32_t keff1;           // entries per s-element chunk
  int32_t subtract_local;  // 1: M = M' - alpha (own part); 0: M = M'
};

struct DecodeParams {
  const float* pay_val;
  const uint16_t* pay_idx;
  int64_t entries;  // entries per worker payload
  int32_t workers;
  int32_t keff2;  // entries per s x s chunk
  int32_t keff1;  // entries per s-element chunk
  float eta;
  float lam;
  float inv_workers;
  int32_t phi_sign;     // 1: sign, 0: identity
  int32_t avg_workers;  // 1: divide by W, 0: by contributor count
  int32_t update_x;     // 1: X = X - eta (phi(M*) + lambda X)
  int32_t update_m;     // 1: M = M - alpha M* (aggregated subtraction)
  int32_t pack_signs;   // 1: write sign(M*) as bits (no parameter or momentum update)
  int32_t write_mstar;  // 1: write M* itself (the Muon path applies phi afterwards)
  float alpha;
  // compact wire payload (read instead of pay_val / pay_idx when wire is 1):
  // bfloat16 values and 12-bit (chunk edge 64) or 14-bit (128) positions in
  // a little-endian bit string,
  // wire_words 32-bit words per worker
  int32_t wire;
  const uint16_t* wire_val;
  const uint32_t* wire_idx;
  int64_t wire_words;
};

struct ApplyParams {
  float eta;
  float lam;
};

enum class BasisKind { kDct, kUser, kIdentity };

// Host entry points into the kernels (kernels.hip).  basis_p0/p1 are used
// for BasisKind::kUser only.  Return the hipError_t of the launch.
hipError_t launch_encode(const LaunchTable& tab, const EncodeParams& p, bool g_bf16, BasisKind kind,
                         const float* basis_p0, const float* basis_p1, hipStream_t stream);
hipError_t launch_decode(const LaunchTable& tab, const DecodeParams& p, BasisKind kind, const float* basis_p0,
                         const float* basis_p1, hipStream_t stream);
hipError_t launch_apply_signs(const LaunchTable& tab, const ApplyParams& p, hipStream_t stream);
// workers x entries payload entries -> wire values (workers x entries) and
// wire index words (workers x 3 * ceil(entries / 8) at 12 bits, workers x
// 7 * ceil(entries / 16) at 14 bits)
hipError_t launch_pack_wire(int32_t bits, const float* pay_val, const uint16_t* pay_idx, int64_t entries,
                            int32_t workers, uint16_t* wire_val, uint32_t* wire_idx, hipStream_t stream);
// Packed signs at chunk edge 128 (kernels128.hip): X update from sign words.
hipError_t launch_apply_signs128(const LaunchTable& tab, const ApplyParams& p, hipStream_t stream);
// phi = Muon (kernels_muon.hip).  D = alpha * (*alpha_scale if given) *
// op(A) op(B) + beta * C + gamma * I, fp32, row-major; op(A) is M x K (the
// transpose of a row-major K x M matrix when trans_a), op(B) K x N.  C may
// alias D.
struct GemmArgs {
  const float* A;
  const float* B;
  const float* C;
  float* D;
  int32_t M, N, K;
  int64_t lda, ldb, ldc, ldd;
  float alpha, beta, gamma;
  const float* alpha_scale;
  int64_t sA, sB, sC, sD;  // element strides between the products of a batch
};
// `batch` products of the same shape: product z reads A + z sA, B + z sB,
// C + z sC and writes D + z sD.
hipError_t launch_gemm(const GemmArgs& g, bool trans_a, bool trans_b, int32_t batch, hipStream_t stream);
// partial: 256 doubles; scal: 2 floats (1/s, 1/sqrt(s)), s = ||A + eps I||_F;
// Y = (A + eps I) / s, Z = I (all n x n)
hipError_t launch_ns_prepare(const float* A, int n, float eps, double* partial, float* scal, float* Y, float* Z,
                             hipStream_t stream);
hipError_t launch_muon_vector(const float* m, float* x, int64_t len, float eps, float eta, float lam,
                              hipStream_t stream);
// The Muon decode's static device scratch (kernels_muon.hip), for callers
// that cannot allocate: kMuonScratchBytes per device.  muon_scratch returns
// its device address on `device`, which must be the current device; the
// address is looked up once per device and kept.
constexpr int64_t kMuonScratchBytes = int64_t(64) << 20;
constexpr int kMaxDevices = 64;
hipError_t muon_scratch(int device, float** out);

// Chunk edge 128 (kernels128.hip): DCT basis; a work item is one 128x128
// chunk or 128 vector chunks, 256 threads each.
hipError_t launch_encode128(const LaunchTable& tab, const EncodeParams& p, bool g_bf16, hipStream_t stream);
hipError_t launch_decode128(const LaunchTable& tab, const DecodeParams& p, hipStream_t stream);

}  // namespace demo
