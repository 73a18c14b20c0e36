// Issue cost of single VALU instruction forms on gfx950, for the VALU
// rooflines of the codec kernels.
//
// Each kernel runs one instruction form, written out through inline asm so
// that the exact encoding is measured (no memory instruction is written in
// asm), on 8 independent register chains per lane, 128 instructions per
// loop iteration, over 8192 workgroups of four waves (eight waves per SIMD).
// The figure printed is cycles per wave64 instruction per SIMD at the
// 2.4 GHz peak engine clock: total wave-instructions over 1024 SIMDs x
// 2.4 GHz x the measured time.
//
//   valu_issue_probe            (built by the package's build step)
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <utility>

namespace {

constexpr int kBlocks = 8192;
constexpr int kIters = 200;
constexpr int kPerIter = 128;

#define CHAINS(stmt) stmt(a0) stmt(a1) stmt(a2) stmt(a3) stmt(a4) stmt(a5) stmt(a6) stmt(a7)

// One instruction form per kernel, selected by kOp; see kForms for the text.
template <int kOp>
__global__ __launch_bounds__(256) void probe(float* out, int iters, float sv) {
  float a0 = 1.f + threadIdx.x * 1e-3f, a1 = a0 + 1.f, a2 = a0 + 2.f, a3 = a0 + 3.f, a4 = a0 + 4.f,
        a5 = a0 + 5.f, a6 = a0 + 6.f, a7 = a0 + 7.f;
  const float bv = 1.0f + 1e-7f * float(threadIdx.x), cv = 0.25f * bv;
  const uint64_t mask = __builtin_amdgcn_ballot_w64((threadIdx.x & 1) != 0);
  const uint32_t su = __builtin_amdgcn_readfirstlane(threadIdx.x);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < kPerIter / 8; ++r) {
      if constexpr (kOp == 0) {
#define S(x) asm volatile("v_add_f32_e32 %0, %0, %1" : "+v"(x) : "v"(bv));
        CHAINS(S)
#undef S
      } else if constexpr (kOp == 1) {
#define S(x) asm volatile("v_mul_f32_e32 %0, %0, %1" : "+v"(x) : "v"(bv));
        CHAINS(S)
#undef S
      } else if constexpr (kOp == 2) {
#define S(x) asm volatile("v_mul_f32_e32 %0, 0x3f800347, %0" : "+v"(x));
        CHAINS(S)
#undef S
      } else if constexpr (kOp == 3) {
#define S(x) asm volatile("v_fmac_f32_e32 %0, %1, %2" : "+v"(x) : "v"(bv), "v"(cv));
        CHAINS(S)
#undef S
      } else if constexpr (kOp == 4) {
#define S(x) asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(x) : "v"(bv), "v"(cv));
        CHAINS(S)
#undef S
      } else if constexpr (kOp == 5) {
#define S(x) asm volatile("v_fmamk_f32 %0, %0, 0x3f800347, %1" : "+v"(x) : "v"(bv));
        CHAINS(S)
#undef S
      } else if constexpr (kOp == 6) {
#define S(x) asm volatile("v_and_b32_e32 %0, 0x7fffffff, %0" : "+v"(x));
        CHAINS(S)
#undef S
      } else if constexpr (kOp == 7) {
#define S(x) asm volatile("v_lshrrev_b32_e32 %0, 1, %0" : "+v"(x));
        CHAINS(S)
#undef S
      } else if constexpr (kOp == 8) {
#define S(x) asm volatile("v_add_u32_e32 %0, %0, %1" : "+v"(x) : "v"(bv));
        CHAINS(S)
#undef S
      } else if constexpr (kOp == 9) {
#define S(x) asm volatile("v_mul_f32_e32 %0, %1, %0" : "+v"(x) : "s"(sv));
        CHAINS(S)
#undef S
      } else if constexpr (kOp == 10) {
#define S(x) asm volatile("v_fma_f32 %0, %1, %0, %2" : "+v"(x) : "s"(sv), "v"(cv));
        CHAINS(S)
#undef S
      } else if constexpr (kOp == 11) {
#define S(x) asm volatile("v_max_f32_e32 %0, %0, %1" : "+v"(x) : "v"(bv));
        CHAINS(S)
#undef S
      } else if constexpr (kOp == 12) {
#define S(x) asm volatile("v_cvt_f32_ubyte1_e32 %0, %0" : "+v"(x));
        CHAINS(S)
#undef S
      } else if constexpr (kOp == 13) {
#define S(x) asm volatile("v_bfe_u32 %0, %0, 8, 8" : "+v"(x));
        CHAINS(S)
#undef S
      } else if constexpr (kOp == 14) {
#define S(x) asm volatile("v_lshl_add_u32 %0, %0, 2, %1" : "+v"(x) : "v"(bv));
        CHAINS(S)
#undef S
      } else if constexpr (kOp == 15) {
#define S(x) asm volatile("v_cmp_gt_f32_e64 s[40:41], %0, %1" : : "v"(x), "v"(bv) : "s40", "s41");
        CHAINS(S)
#undef S
      } else if constexpr (kOp == 16) {
#define S(x) asm volatile("v_cndmask_b32_e64 %0, %0, %1, %2" : "+v"(x) : "v"(bv), "s"(mask));
        CHAINS(S)
#undef S
      } else if constexpr (kOp == 17) {
#define S(x) asm volatile("v_writelane_b32 %0, %1, 5" : "+v"(x) : "s"(su));
        CHAINS(S)
#undef S
      } else if constexpr (kOp == 18) {
#define S(x) asm volatile("v_rcp_f32_e32 %0, %0" : "+v"(x));
        CHAINS(S)
#undef S
      } else if constexpr (kOp == 19) {
#define S(x) asm volatile("v_exp_f32_e32 %0, %0" : "+v"(x));
        CHAINS(S)
#undef S
      }
    }
  }
  out[blockIdx.x * 256 + threadIdx.x] = a0 + a1 + a2 + a3 + a4 + a5 + a6 + a7;
}

constexpr const char* kForms[] = {
    "v_add_f32_e32 v, v, v",        "v_mul_f32_e32 v, v, v",      "v_mul_f32_e32 v, literal, v",
    "v_fmac_f32_e32 v, v, v",       "v_fma_f32 v, v, v, v",       "v_fmamk_f32 v, v, literal, v",
    "v_and_b32_e32 v, literal, v",  "v_lshrrev_b32_e32 v, 1, v",  "v_add_u32_e32 v, v, v",
    "v_mul_f32_e32 v, s, v",        "v_fma_f32 v, s, v, v",       "v_max_f32_e32 v, v, v",
    "v_cvt_f32_ubyte1_e32 v, v",    "v_bfe_u32 v, v, 8, 8",       "v_lshl_add_u32 v, v, 2, v",
    "v_cmp_gt_f32_e64 s[2], v, v",  "v_cndmask_b32_e64 v, v, v, s[2]", "v_writelane_b32 v, s, 5",
    "v_rcp_f32_e32 v, v",           "v_exp_f32_e32 v, v",
};

template <int kOp>
bool run(float* out, hipEvent_t e0, hipEvent_t e1) {
  probe<kOp><<<kBlocks, 256>>>(out, kIters, 1.0001f);  // warm-up
  if (hipEventRecord(e0) != hipSuccess) return false;
  probe<kOp><<<kBlocks, 256>>>(out, kIters, 1.0001f);
  if (hipEventRecord(e1) != hipSuccess || hipEventSynchronize(e1) != hipSuccess) return false;
  float ms = 0.f;
  if (hipEventElapsedTime(&ms, e0, e1) != hipSuccess) return false;
  const double inst = double(kBlocks) * 4 * kIters * kPerIter;  // wave64 instructions
  const double rate = inst / (ms * 1e-3);
  std::printf("| `%s` | %.3f | %.1f | %.2f |\n", kForms[kOp], ms, rate / 1e9, 1024.0 * 2.4e9 / rate);
  return true;
}

template <int... kOps>
bool run_all(float* out, hipEvent_t e0, hipEvent_t e1, std::integer_sequence<int, kOps...>) {
  return (run<kOps>(out, e0, e1) && ...);
}

}  // namespace

int main() {
  float* out = nullptr;
  if (hipMalloc(&out, sizeof(float) * kBlocks * 256) != hipSuccess) return 1;
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return 1;
  std::printf("| instruction form | ms | G wave-instructions/s | cycles per instruction per SIMD |\n|---|---|---|---|\n");
  const bool ok = run_all(out, e0, e1, std::make_integer_sequence<int, sizeof(kForms) / sizeof(kForms[0])>{});
  if (hipFree(out) != hipSuccess || !ok) return 1;
  return 0;
}
