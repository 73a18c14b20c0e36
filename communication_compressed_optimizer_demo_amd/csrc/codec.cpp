// C ABI of the DeMo momentum codec: argument validation, chunk planning and
// launch batching.  Every check runs on the host before anything is enqueued;
// the kernels themselves live in kernels.hip.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <string>
#include <vector>

#include "demo_codec.h"
#include "launch.h"

struct demo_ctx {
  int device;
  float* scratch;  // the device's static Muon scratch (demo::kMuonScratchBytes), looked up at creation
};

namespace {

using demo::kChunk;
using demo::kChunkLarge;
using demo::kMaxTensorsPerLaunch;
static_assert(kMaxTensorsPerLaunch == DEMO_MAX_TENSORS_PER_LAUNCH, "header and launch table disagree");
static_assert(demo::kMaxWorkers == DEMO_MAX_WORKERS, "header and kernels disagree");
static_assert(kChunk == DEMO_CHUNK && kChunkLarge == DEMO_CHUNK_LARGE, "header and kernels disagree on chunk edges");
static_assert(demo::kMuonScratchBytes == DEMO_MUON_SCRATCH_BYTES, "header and kernels disagree on the scratch size");
using demo::LaunchTable;

thread_local std::string g_last_error;

demo_status fail(demo_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

struct TensorPlan {
  int ndim;
  int64_t rows, cols;   // 1-D: rows = length, cols = 1
  int64_t chunks;       // chunks of the tensor
  int32_t keff;         // entries per chunk
  int64_t entry_begin;  // payload offset of the first chunk
  int64_t items;        // work items: chunks (2-D) or 64-chunk slabs (1-D)
  int64_t word_begin;   // first 64-bit word of the tensor's packed sign
};

// Packed-sign words per chunk: one per 64 elements of the (padded) chunk.
int64_t words_per_chunk(int32_t chunk, int ndim) { return ndim == 2 ? int64_t(chunk) * chunk / 64 : chunk / 64; }

// Vector chunks per work item: 64 (one wave, one chunk per lane) at chunk
// edge 64, 128 (four waves, one chunk per lane pair) at chunk edge 128.
int64_t vector_chunks_per_item(int32_t chunk) { return chunk == kChunk ? 64 : 128; }

demo_status plan_list(const demo_shape* shapes, int32_t n, int32_t chunk, int32_t k, std::vector<TensorPlan>* out,
                      int64_t* entries, int64_t* chunks, int64_t* words = nullptr) {
  if (n < 0) return fail(DEMO_ERR_RANGE, "tensor count is negative");
  if (n > 0 && shapes == nullptr) return fail(DEMO_ERR_INVALID, "shapes is NULL");
  if (chunk != kChunk && chunk != kChunkLarge) return fail(DEMO_ERR_RANGE, "chunk size must be 64 or 128");
  if (k < 1) return fail(DEMO_ERR_RANGE, "k must be >= 1");
  int64_t e = 0, c = 0, w = 0;
  if (out) out->clear();
  for (int32_t i = 0; i < n; ++i) {
    const demo_shape& s = shapes[i];
    TensorPlan t{};
    t.ndim = s.ndim;
    if (s.ndim != 1 && s.ndim != 2)
      return fail(DEMO_ERR_SHAPE, "tensor " + std::to_string(i) + ": ndim must be 1 or 2");
    for (int d = 0; d < s.ndim; ++d) {
      if (s.dims[d] < 1 || s.dims[d] > INT32_MAX)
        return fail(DEMO_ERR_SHAPE, "tensor " + std::to_string(i) + ": dimension out of 1..2^31-1");
    }
    if (s.ndim == 2) {
      t.rows = s.dims[0];
      t.cols = s.dims[1];
      const int64_t g0 = (t.rows + chunk - 1) / chunk, g1 = (t.cols + chunk - 1) / chunk;
      t.chunks = g0 * g1;
      t.keff = k < chunk * chunk ? k : chunk * chunk;
      t.items = t.chunks;
    } else {
      t.rows = s.dims[0];
      t.cols = 1;
      t.chunks = (t.rows + chunk - 1) / chunk;
      t.keff = k < chunk ? k : chunk;
      const int64_t per = vector_chunks_per_item(chunk);
      t.items = (t.chunks + per - 1) / per;
    }
    if (t.items > INT32_MAX) return fail(DEMO_ERR_SHAPE, "tensor " + std::to_string(i) + ": too many chunks");
    t.entry_begin = e;
    t.word_begin = w;
    e += t.chunks * t.keff;
    c += t.chunks;
    w += t.chunks * words_per_chunk(chunk, t.ndim);
    if (out) out->push_back(t);
  }
  if (entries) *entries = e;
  if (chunks) *chunks = c;
  if (words) *words = w;
  return DEMO_OK;
}

demo_status check_device(const demo_ctx* ctx) {
  if (ctx == nullptr) return fail(DEMO_ERR_INVALID, "context is NULL");
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return fail(DEMO_ERR_HIP, "hipGetDevice failed");
  if (cur != ctx->device)
    return fail(DEMO_ERR_DEVICE, "current device " + std::to_string(cur) + " is not the context's device " +
                                     std::to_string(ctx->device));
  return DEMO_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

demo_status check_basis(const demo_codec_cfg* cfg, const std::vector<TensorPlan>& plan, demo::BasisKind* kind,
                        const float** p0, const float** p1) {
  *p0 = nullptr;
  *p1 = nullptr;
  if (cfg->basis == DEMO_BASIS_DCT) {
    *kind = demo::BasisKind::kDct;
    return DEMO_OK;
  }
  if (cfg->basis == DEMO_BASIS_IDENTITY) {
    *kind = demo::BasisKind::kIdentity;
    return DEMO_OK;
  }
  if (cfg->basis != DEMO_BASIS_USER) return fail(DEMO_ERR_INVALID, "unknown basis");
  bool any2d = false;
  for (const auto& t : plan) any2d = any2d || t.ndim == 2;
  if (cfg->P0 == nullptr) return fail(DEMO_ERR_INVALID, "user basis without P0");
  if (any2d && cfg->P1 == nullptr) return fail(DEMO_ERR_INVALID, "user basis without P1 for a matrix");
  if (!aligned(cfg->P0, 16) || (cfg->P1 && !aligned(cfg->P1, 16)))
    return fail(DEMO_ERR_ALIGN, "basis misaligned (16 bytes)");
  *kind = demo::BasisKind::kUser;
  *p0 = cfg->P0;
  *p1 = cfg->P1 ? cfg->P1 : cfg->P0;
  return DEMO_OK;
}

// Fills launch tables (vectors first, then matrices, each kind in list order)
// and calls `launch` for each batch of up to kMaxTensorsPerLaunch tensors.
template <class Fill, class Launch>
demo_status for_each_batch(const std::vector<TensorPlan>& plan, Fill&& fill, Launch&& launch) {
  LaunchTable tab;
  std::memset(&tab, 0, sizeof(tab));
  auto flush = [&]() -> demo_status {
    if (tab.n == 0) return DEMO_OK;
    const hipError_t err = launch(tab);
    if (err != hipSuccess) return fail(DEMO_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(err));
    std::memset(&tab, 0, sizeof(tab));
    return DEMO_OK;
  };
  for (int ndim : {1, 2}) {
    for (size_t i = 0; i < plan.size(); ++i) {
      const TensorPlan& t = plan[i];
      if (t.ndim != ndim) continue;
      if (tab.n == kMaxTensorsPerLaunch || int64_t(tab.items) + t.items > INT32_MAX) {
        const demo_status s = flush();
        if (s != DEMO_OK) return s;
      }
      demo::TensorSlot& slot = tab.t[tab.n++];
      slot.entry_begin = t.entry_begin;
      slot.rows = int32_t(t.rows);
      slot.cols = t.ndim == 2 ? int32_t(t.cols) : 0;
      slot.item_begin = tab.items;
      fill(slot, i);
      tab.items += int32_t(t.items);
    }
  }
  return flush();
}

// Bits of a wire position: 12 inside a 64x64 chunk, 14 inside a 128x128 one.
int32_t wire_bits(int32_t chunk) { return chunk == kChunkLarge ? 14 : 12; }

// 32-bit words of one worker's wire indices: whole groups of 32 positions'
// worth of words, 3 words per 8 positions (12 bits) or 7 per 16 (14 bits).
int64_t wire_idx_words(int32_t chunk, int64_t entries) {
  return chunk == kChunkLarge ? (entries + 15) / 16 * 7 : (entries + 7) / 8 * 3;
}

// Shared body of the decode entry points: params and/or moms (either may be
// NULL) receive X - eta (phi(M*) + lambda X) and M - alpha M*; or, with
// `signs` given (params and moms NULL), sign(M*) is packed into n_words words.
// With `wire` the payload is read from the wire arrays instead of pay_values /
// pay_idx (parameter update only).
demo_status decode_common(demo_ctx* ctx, int32_t n, const demo_shape* shapes, float* const* params,
                          float* const* moms, const demo_codec_cfg* cfg, int32_t workers, const float* pay_values,
                          const uint16_t* pay_idx, int64_t n_entries, demo_phi phi, float eta, float lambda,
                          demo_average avg, hipStream_t stream, uint64_t* signs = nullptr, int64_t n_words = 0,
                          float* const* mstar = nullptr, bool wire = false, const uint16_t* wire_values = nullptr,
                          const void* wire_idx = nullptr) {
  if (cfg == nullptr) return fail(DEMO_ERR_INVALID, "cfg is NULL");
  std::vector<TensorPlan> plan;
  int64_t entries = 0, words = 0;
  demo_status s = plan_list(shapes, n, cfg->chunk, cfg->k, &plan, &entries, nullptr, &words);
  if (s != DEMO_OK) return s;
  const bool to_signs = params == nullptr && moms == nullptr && mstar == nullptr;
  if (to_signs) {
    if (n_words != words)
      return fail(DEMO_ERR_PAYLOAD, "sign buffer holds " + std::to_string(n_words) + " words, plan needs " +
                                        std::to_string(words));
    if (words > 0 && signs == nullptr) return fail(DEMO_ERR_INVALID, "sign buffer is NULL");
    if (!aligned(signs, 8)) return fail(DEMO_ERR_ALIGN, "sign buffer misaligned");
  }
  if (workers < 1 || workers > demo::kMaxWorkers) return fail(DEMO_ERR_RANGE, "workers must be in 1..255");
  if (phi != DEMO_PHI_SIGN && phi != DEMO_PHI_IDENTITY) return fail(DEMO_ERR_INVALID, "unknown phi");
  if (avg != DEMO_AVG_CONTRIBUTORS && avg != DEMO_AVG_WORKERS) return fail(DEMO_ERR_INVALID, "unknown average");
  if (!std::isfinite(eta) || !std::isfinite(lambda)) return fail(DEMO_ERR_INVALID, "eta/lambda not finite");
  if (moms != nullptr && !std::isfinite(cfg->alpha)) return fail(DEMO_ERR_INVALID, "alpha not finite");
  if (n_entries != entries)
    return fail(DEMO_ERR_PAYLOAD, "payload holds " + std::to_string(n_entries) + " entries per worker, plan needs " +
                                      std::to_string(entries));
  for (float* const* list : {params, moms}) {
    if (list == nullptr) continue;
    for (int32_t i = 0; i < n; ++i) {
      if (list[i] == nullptr) return fail(DEMO_ERR_INVALID, "tensor " + std::to_string(i) + ": NULL device pointer");
      if (!aligned(list[i], 4)) return fail(DEMO_ERR_ALIGN, "tensor " + std::to_string(i) + ": misaligned pointer");
    }
  }
  if (wire) {
    if (entries > 0 && (wire_values == nullptr || wire_idx == nullptr))
      return fail(DEMO_ERR_INVALID, "wire payload is NULL");
    if (!aligned(wire_values, 2) || !aligned(wire_idx, 4)) return fail(DEMO_ERR_ALIGN, "wire payload misaligned");
  } else {
    if (entries > 0 && (pay_values == nullptr || pay_idx == nullptr))
      return fail(DEMO_ERR_INVALID, "payload is NULL");
    if (!aligned(pay_values, 4) || !aligned(pay_idx, 2)) return fail(DEMO_ERR_ALIGN, "payload misaligned");
  }
  const float *p0, *p1;
  demo::BasisKind kind;
  if ((s = check_basis(cfg, plan, &kind, &p0, &p1)) != DEMO_OK) return s;
  if (cfg->chunk == kChunkLarge && kind != demo::BasisKind::kDct)
    return fail(DEMO_ERR_RANGE, "chunk 128 is built for the DCT basis");
  if ((s = check_device(ctx)) != DEMO_OK) return s;

  demo::DecodeParams p{};
  p.pay_val = pay_values;
  p.pay_idx = pay_idx;
  p.entries = entries;
  p.workers = workers;
  p.eta = eta;
  p.lam = lambda;
  p.inv_workers = float(1.0 / double(workers));
  p.phi_sign = phi == DEMO_PHI_SIGN ? 1 : 0;
  p.avg_workers = avg == DEMO_AVG_WORKERS ? 1 : 0;
  p.update_x = params != nullptr ? 1 : 0;
  p.update_m = moms != nullptr ? 1 : 0;
  p.pack_signs = to_signs ? 1 : 0;
  p.write_mstar = mstar != nullptr ? 1 : 0;
  p.alpha = cfg->alpha;
  p.wire = wire ? 1 : 0;
  p.wire_val = wire_values;
  p.wire_idx = static_cast<const uint32_t*>(wire_idx);
  p.wire_words = wire_idx_words(cfg->chunk, entries);
  auto fill = [&](demo::TensorSlot& slot, size_t i) {
    slot.aux = moms != nullptr    ? static_cast<void*>(moms[i])
               : mstar != nullptr ? static_cast<void*>(mstar[i])
               : to_signs         ? static_cast<void*>(signs + plan[i].word_begin)
                                  : nullptr;
    slot.dst = params != nullptr ? params[i] : nullptr;
  };
  const int32_t S = cfg->chunk;
  p.keff2 = cfg->k < S * S ? cfg->k : S * S;
  p.keff1 = cfg->k < S ? cfg->k : S;
  if (S == kChunkLarge)
    return for_each_batch(plan, fill, [&](const LaunchTable& t) { return demo::launch_decode128(t, p, stream); });
  return for_each_batch(plan, fill,
                        [&](const LaunchTable& t) { return demo::launch_decode(t, p, kind, p0, p1, stream); });
}

// Workspace of the Muon decode: M* of every tensor (offsets rounded up to 64
// floats), then `slots` Newton-Schulz slots, one per matrix of a batch, each
// six n x n fp32 matrices (A, Y, Y', Z, Z', T) for n up to n_max (rounded up
// to 64 floats), 256 doubles of partial sums and 64 floats (two used).
constexpr int64_t kMuonBatch = 8;  // matrices whose iterations share launches

struct MuonLayout {
  std::vector<int64_t> mstar;  // float offset of each tensor's M*
  int64_t nmax = 0, slots = 0;
  int64_t ns = 0, slot = 0, partial = 0, scal = 0, bytes = 0;  // float offsets / sizes; total bytes
};

MuonLayout muon_layout(const std::vector<TensorPlan>& plan) {
  MuonLayout L;
  int64_t off = 0, matrices = 0;
  for (const auto& t : plan) {
    L.mstar.push_back(off);
    off += (t.rows * t.cols + 63) / 64 * 64;
    if (t.ndim == 2) {
      L.nmax = std::max(L.nmax, std::min(t.rows, t.cols));
      ++matrices;
    }
  }
  L.ns = off;
  L.slots = std::min(matrices, kMuonBatch);
  L.partial = (6 * L.nmax * L.nmax + 63) / 64 * 64;  // inside a slot
  L.scal = L.partial + 2 * 256;
  L.slot = L.scal + 64;
  L.bytes = (L.ns + L.slots * L.slot) * 4;
  return L;
}

}  // namespace

extern "C" {

const char* demo_last_error(void) { return g_last_error.c_str(); }

demo_status demo_ctx_create(int32_t device, demo_ctx** out) {
  if (out == nullptr) return fail(DEMO_ERR_INVALID, "out is NULL");
  *out = nullptr;
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) return fail(DEMO_ERR_DEVICE, "no HIP device");
  if (device < 0 || device >= count) return fail(DEMO_ERR_DEVICE, "device ordinal out of range");
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess) return fail(DEMO_ERR_HIP, "hipGetDeviceProperties failed");
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(DEMO_ERR_DEVICE, std::string("device is ") + prop.gcnArchName + ", this library is built for gfx950");
  if (device >= demo::kMaxDevices) return fail(DEMO_ERR_DEVICE, "device ordinal beyond the library's device table");
  // The static Muon scratch's address on this device, looked up with the
  // device current (once per device; later contexts reuse it).
  int prev = -1;
  if (hipGetDevice(&prev) != hipSuccess) return fail(DEMO_ERR_HIP, "hipGetDevice failed");
  if (prev != device && hipSetDevice(device) != hipSuccess) return fail(DEMO_ERR_HIP, "hipSetDevice failed");
  float* scratch = nullptr;
  const hipError_t se = demo::muon_scratch(device, &scratch);
  if (prev != device && hipSetDevice(prev) != hipSuccess) return fail(DEMO_ERR_HIP, "hipSetDevice failed");
  if (se != hipSuccess)
    return fail(DEMO_ERR_HIP, std::string("hipGetSymbolAddress of the Muon scratch failed: ") + hipGetErrorString(se));
  demo_ctx* c = new (std::nothrow) demo_ctx;
  if (c == nullptr) return fail(DEMO_ERR_INVALID, "out of host memory");
  c->device = device;
  c->scratch = scratch;
  *out = c;
  return DEMO_OK;
}

void demo_ctx_destroy(demo_ctx* ctx) { delete ctx; }

demo_status demo_plan(const demo_shape* shapes, int32_t n, int32_t chunk, int32_t k, int64_t* n_chunks,
                      int64_t* n_entries, int64_t* entry_begin) {
  std::vector<TensorPlan> plan;
  int64_t e = 0, c = 0;
  const demo_status s = plan_list(shapes, n, chunk, k, &plan, &e, &c);
  if (s != DEMO_OK) return s;
  if (n_chunks) *n_chunks = c;
  if (n_entries) *n_entries = e;
  if (entry_begin) {
    for (int32_t i = 0; i < n; ++i) entry_begin[i] = plan[i].entry_begin;
    entry_begin[n] = e;
  }
  return DEMO_OK;
}

demo_status demo_encode(demo_ctx* ctx, int32_t n, const demo_shape* shapes, const void* const* grads,
                        demo_dtype grad_dtype, float* const* moms, const demo_codec_cfg* cfg, float* pay_values,
                        uint16_t* pay_idx, int64_t n_entries, hipStream_t stream) {
  if (cfg == nullptr) return fail(DEMO_ERR_INVALID, "cfg is NULL");
  std::vector<TensorPlan> plan;
  int64_t entries = 0;
  demo_status s = plan_list(shapes, n, cfg->chunk, cfg->k, &plan, &entries, nullptr);
  if (s != DEMO_OK) return s;
  if (grad_dtype != DEMO_F32 && grad_dtype != DEMO_BF16) return fail(DEMO_ERR_INVALID, "unknown gradient dtype");
  if (cfg->momentum_form != DEMO_MOMENTUM_DAMPED && cfg->momentum_form != DEMO_MOMENTUM_PLAIN)
    return fail(DEMO_ERR_INVALID, "unknown momentum form");
  if (cfg->subtraction != DEMO_SUBTRACT_LOCAL && cfg->subtraction != DEMO_SUBTRACT_AGGREGATED)
    return fail(DEMO_ERR_INVALID, "unknown subtraction mode");
  if (!std::isfinite(cfg->beta) || !std::isfinite(cfg->alpha)) return fail(DEMO_ERR_INVALID, "beta/alpha not finite");
  if (n_entries != entries)
    return fail(DEMO_ERR_PAYLOAD, "payload holds " + std::to_string(n_entries) + " entries, plan needs " +
                                      std::to_string(entries));
  if (n > 0 && (grads == nullptr || moms == nullptr)) return fail(DEMO_ERR_INVALID, "tensor pointer list is NULL");
  const size_t gsz = grad_dtype == DEMO_BF16 ? 2 : 4;
  for (int32_t i = 0; i < n; ++i) {
    if (grads[i] == nullptr || moms[i] == nullptr)
      return fail(DEMO_ERR_INVALID, "tensor " + std::to_string(i) + ": NULL device pointer");
    if (!aligned(grads[i], gsz) || !aligned(moms[i], 4))
      return fail(DEMO_ERR_ALIGN, "tensor " + std::to_string(i) + ": misaligned pointer");
  }
  if (entries > 0 && (pay_values == nullptr || pay_idx == nullptr)) return fail(DEMO_ERR_INVALID, "payload is NULL");
  if (!aligned(pay_values, 4) || !aligned(pay_idx, 2)) return fail(DEMO_ERR_ALIGN, "payload misaligned");
  const float *p0, *p1;
  demo::BasisKind kind;
  if ((s = check_basis(cfg, plan, &kind, &p0, &p1)) != DEMO_OK) return s;
  if (cfg->chunk == kChunkLarge && kind != demo::BasisKind::kDct)
    return fail(DEMO_ERR_RANGE, "chunk 128 is built for the DCT basis");
  if ((s = check_device(ctx)) != DEMO_OK) return s;

  demo::EncodeParams p{};
  p.pay_val = pay_values;
  p.pay_idx = pay_idx;
  p.beta = cfg->beta;
  p.gcoef = cfg->momentum_form == DEMO_MOMENTUM_PLAIN ? 1.0f : float(1.0 - double(cfg->beta));
  p.alpha = cfg->alpha;
  p.subtract_local = cfg->subtraction == DEMO_SUBTRACT_LOCAL ? 1 : 0;
  const bool bf16 = grad_dtype == DEMO_BF16;
  auto fill = [&](demo::TensorSlot& slot, size_t i) {
    slot.aux = const_cast<void*>(grads[i]);  // read only in the kernels
    slot.dst = moms[i];
  };
  const int32_t S = cfg->chunk;
  p.keff2 = cfg->k < S * S ? cfg->k : S * S;
  p.keff1 = cfg->k < S ? cfg->k : S;
  if (S == kChunkLarge)
    return for_each_batch(plan, fill,
                          [&](const LaunchTable& t) { return demo::launch_encode128(t, p, bf16, stream); });
  return for_each_batch(plan, fill,
                        [&](const LaunchTable& t) { return demo::launch_encode(t, p, bf16, kind, p0, p1, stream); });
}

demo_status demo_decode_apply(demo_ctx* ctx, int32_t n, const demo_shape* shapes, float* const* params,
                              const demo_codec_cfg* cfg, int32_t workers, const float* pay_values,
                              const uint16_t* pay_idx, int64_t n_entries, demo_phi phi, float eta, float lambda,
                              demo_average avg, hipStream_t stream) {
  if (n > 0 && params == nullptr) return fail(DEMO_ERR_INVALID, "parameter pointer list is NULL");
  return decode_common(ctx, n, shapes, params, nullptr, cfg, workers, pay_values, pay_idx, n_entries, phi, eta,
                       lambda, avg, stream);
}

demo_status demo_wire_size(int32_t chunk, int64_t n_entries, int64_t* value_bytes, int64_t* idx_bytes) {
  if (chunk != kChunk && chunk != kChunkLarge) return fail(DEMO_ERR_RANGE, "chunk size must be 64 or 128");
  if (n_entries < 0 || n_entries > (int64_t(1) << 40)) return fail(DEMO_ERR_RANGE, "entry count out of range");
  if (value_bytes != nullptr) *value_bytes = 2 * n_entries;
  if (idx_bytes != nullptr) *idx_bytes = 4 * wire_idx_words(chunk, n_entries);
  return DEMO_OK;
}

demo_status demo_pack_wire(demo_ctx* ctx, int32_t chunk, int32_t workers, const float* pay_values,
                           const uint16_t* pay_idx, int64_t n_entries, uint16_t* wire_values, void* wire_idx,
                           hipStream_t stream) {
  if (chunk != kChunk && chunk != kChunkLarge) return fail(DEMO_ERR_RANGE, "chunk size must be 64 or 128");
  if (workers < 1 || workers > demo::kMaxWorkers) return fail(DEMO_ERR_RANGE, "workers must be in 1..255");
  if (n_entries < 0 || n_entries > (int64_t(1) << 40)) return fail(DEMO_ERR_RANGE, "entry count out of range");
  if (n_entries > 0 && (pay_values == nullptr || pay_idx == nullptr || wire_values == nullptr || wire_idx == nullptr))
    return fail(DEMO_ERR_INVALID, "payload or wire buffer is NULL");
  if (!aligned(pay_values, 4) || !aligned(pay_idx, 2) || !aligned(wire_values, 2) || !aligned(wire_idx, 4))
    return fail(DEMO_ERR_ALIGN, "payload or wire buffer misaligned");
  demo_status s = check_device(ctx);
  if (s != DEMO_OK) return s;
  const hipError_t e = demo::launch_pack_wire(wire_bits(chunk), pay_values, pay_idx, n_entries, workers, wire_values,
                                              static_cast<uint32_t*>(wire_idx), stream);
  return e == hipSuccess ? DEMO_OK : fail(DEMO_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
}

demo_status demo_decode_apply_wire(demo_ctx* ctx, int32_t n, const demo_shape* shapes, float* const* params,
                                   const demo_codec_cfg* cfg, int32_t workers, const uint16_t* wire_values,
                                   const void* wire_idx, int64_t n_entries, demo_phi phi, float eta, float lambda,
                                   demo_average avg, hipStream_t stream) {
  if (n > 0 && params == nullptr) return fail(DEMO_ERR_INVALID, "parameter pointer list is NULL");
  return decode_common(ctx, n, shapes, params, nullptr, cfg, workers, nullptr, nullptr, n_entries, phi, eta, lambda,
                       avg, stream, nullptr, 0, nullptr, true, wire_values, wire_idx);
}

demo_status demo_decode_apply_subtract(demo_ctx* ctx, int32_t n, const demo_shape* shapes, float* const* params,
                                       float* const* moms, const demo_codec_cfg* cfg, int32_t workers,
                                       const float* pay_values, const uint16_t* pay_idx, int64_t n_entries,
                                       demo_phi phi, float eta, float lambda, demo_average avg, hipStream_t stream) {
  if (params == nullptr && moms == nullptr) return fail(DEMO_ERR_INVALID, "neither parameters nor momenta given");
  return decode_common(ctx, n, shapes, params, moms, cfg, workers, pay_values, pay_idx, n_entries, phi, eta, lambda,
                       avg, stream);
}

demo_status demo_plan_signs(const demo_shape* shapes, int32_t n, int32_t chunk, int64_t* n_words,
                            int64_t* word_begin) {
  std::vector<TensorPlan> plan;
  int64_t w = 0;
  const demo_status s = plan_list(shapes, n, chunk, 1, &plan, nullptr, nullptr, &w);
  if (s != DEMO_OK) return s;
  if (n_words) *n_words = w;
  if (word_begin) {
    for (int32_t i = 0; i < n; ++i) word_begin[i] = plan[i].word_begin;
    word_begin[n] = w;
  }
  return DEMO_OK;
}

demo_status demo_decode_signs(demo_ctx* ctx, int32_t n, const demo_shape* shapes, const demo_codec_cfg* cfg,
                              int32_t workers, const float* pay_values, const uint16_t* pay_idx, int64_t n_entries,
                              demo_average avg, uint64_t* signs, int64_t n_words, hipStream_t stream) {
  return decode_common(ctx, n, shapes, nullptr, nullptr, cfg, workers, pay_values, pay_idx, n_entries,
                       DEMO_PHI_SIGN, 0.0f, 0.0f, avg, stream, signs, n_words);
}

demo_status demo_apply_signs(demo_ctx* ctx, int32_t n, const demo_shape* shapes, float* const* params,
                             int32_t chunk, const uint64_t* signs, int64_t n_words, float eta, float lambda,
                             hipStream_t stream) {
  std::vector<TensorPlan> plan;
  int64_t words = 0;
  demo_status s = plan_list(shapes, n, chunk, 1, &plan, nullptr, nullptr, &words);
  if (s != DEMO_OK) return s;
  if (!std::isfinite(eta) || !std::isfinite(lambda)) return fail(DEMO_ERR_INVALID, "eta/lambda not finite");
  if (n_words != words)
    return fail(DEMO_ERR_PAYLOAD, "sign buffer holds " + std::to_string(n_words) + " words, plan needs " +
                                      std::to_string(words));
  if (words > 0 && signs == nullptr) return fail(DEMO_ERR_INVALID, "sign buffer is NULL");
  if (!aligned(signs, 8)) return fail(DEMO_ERR_ALIGN, "sign buffer misaligned");
  if (n > 0 && params == nullptr) return fail(DEMO_ERR_INVALID, "parameter pointer list is NULL");
  for (int32_t i = 0; i < n; ++i) {
    if (params[i] == nullptr) return fail(DEMO_ERR_INVALID, "tensor " + std::to_string(i) + ": NULL device pointer");
    if (!aligned(params[i], 4)) return fail(DEMO_ERR_ALIGN, "tensor " + std::to_string(i) + ": misaligned pointer");
  }
  if ((s = check_device(ctx)) != DEMO_OK) return s;
  const demo::ApplyParams p{eta, lambda};
  auto fill = [&](demo::TensorSlot& slot, size_t i) {
    slot.aux = const_cast<uint64_t*>(signs) + plan[i].word_begin;  // read only in the kernel
    slot.dst = params[i];
  };
  if (chunk == kChunkLarge)
    return for_each_batch(plan, fill, [&](const LaunchTable& t) { return demo::launch_apply_signs128(t, p, stream); });
  return for_each_batch(plan, fill, [&](const LaunchTable& t) { return demo::launch_apply_signs(t, p, stream); });
}

demo_status demo_muon_workspace(const demo_shape* shapes, int32_t n, int64_t* ws_bytes) {
  std::vector<TensorPlan> plan;
  const demo_status s = plan_list(shapes, n, kChunk, 1, &plan, nullptr, nullptr);
  if (s != DEMO_OK) return s;
  if (ws_bytes == nullptr) return fail(DEMO_ERR_INVALID, "ws_bytes is NULL");
  *ws_bytes = muon_layout(plan).bytes;
  return DEMO_OK;
}

}  // extern "C"

namespace {

// The Muon decode over a caller workspace, or (from_scratch) over the
// context's static scratch: then workspace and ws_bytes are ignored, and a
// NULL context is still reported last, after every other check.
demo_status muon_decode(demo_ctx* ctx, int32_t n, const demo_shape* shapes, float* const* params,
                        const demo_codec_cfg* cfg, int32_t workers, const float* pay_values, const uint16_t* pay_idx,
                        int64_t n_entries, float eta, float lambda, float eps, int32_t iters, demo_average avg,
                        void* workspace, int64_t ws_bytes, hipStream_t stream, bool from_scratch = false) {
  if (from_scratch) {
    workspace = ctx != nullptr ? ctx->scratch : nullptr;
    ws_bytes = demo::kMuonScratchBytes;
  }
  if (cfg == nullptr) return fail(DEMO_ERR_INVALID, "cfg is NULL");
  if (cfg->chunk != kChunk) return fail(DEMO_ERR_RANGE, "the Muon decode is built for chunk 64");
  if (n > 0 && params == nullptr) return fail(DEMO_ERR_INVALID, "parameter pointer list is NULL");
  if (!std::isfinite(eps) || eps < 0.f) return fail(DEMO_ERR_INVALID, "eps must be finite and >= 0");
  if (iters < 1 || iters > 64) return fail(DEMO_ERR_RANGE, "iters must be in 1..64");
  std::vector<TensorPlan> plan;
  demo_status s = plan_list(shapes, n, cfg->chunk, cfg->k, &plan, nullptr, nullptr);
  if (s != DEMO_OK) return s;
  const MuonLayout L = muon_layout(plan);
  if (ws_bytes < L.bytes)
    return fail(DEMO_ERR_RANGE, "workspace holds " + std::to_string(ws_bytes) + " bytes, the list needs " +
                                    std::to_string(L.bytes));
  if (!from_scratch && L.bytes > 0 && workspace == nullptr) return fail(DEMO_ERR_INVALID, "workspace is NULL");
  if (!aligned(workspace, 16)) return fail(DEMO_ERR_ALIGN, "workspace misaligned (16 bytes)");
  for (int32_t i = 0; i < n; ++i) {
    if (params[i] == nullptr) return fail(DEMO_ERR_INVALID, "tensor " + std::to_string(i) + ": NULL device pointer");
    if (!aligned(params[i], 4)) return fail(DEMO_ERR_ALIGN, "tensor " + std::to_string(i) + ": misaligned pointer");
  }
  float* ws = static_cast<float*>(workspace);
  std::vector<float*> mstar(size_t(n > 0 ? n : 0));
  // addresses inside the workspace (integer arithmetic: with from_scratch and
  // no context the base is NULL, and decode_common fails before any launch)
  for (int32_t i = 0; i < n; ++i)
    mstar[i] = reinterpret_cast<float*>(reinterpret_cast<uintptr_t>(workspace) + uintptr_t(L.mstar[i]) * 4u);
  // rows a7, a8: M* of every tensor into the workspace (validates the rest,
  // the context last; nothing is enqueued unless all of it passes)
  s = decode_common(ctx, n, shapes, nullptr, nullptr, cfg, workers, pay_values, pay_idx, n_entries, DEMO_PHI_IDENTITY,
                    eta, lambda, avg, stream, nullptr, 0, mstar.data());
  if (s != DEMO_OK) return s;
  auto check = [&](hipError_t e) -> demo_status {
    if (e != hipSuccess) return fail(DEMO_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
    return DEMO_OK;
  };
  // Vectors now; matrices in list order, batched while they share n: their
  // Newton-Schulz products go out as one launch per step with one slot each.
  std::vector<int32_t> mats;
  for (int32_t i = 0; i < n; ++i) {
    const TensorPlan& t = plan[i];
    if (t.ndim == 1) {
      if ((s = check(demo::launch_muon_vector(mstar[i], params[i], t.rows, eps, eta, lambda, stream))) != DEMO_OK)
        return s;
    } else {
      mats.push_back(i);
    }
  }
  auto small_dim = [&](int32_t i) { return int32_t(std::min(plan[i].rows, plan[i].cols)); };
  for (size_t b0 = 0; b0 < mats.size();) {
    const int32_t nn = small_dim(mats[b0]);
    size_t b1 = b0 + 1;
    while (b1 < mats.size() && int64_t(b1 - b0) < L.slots && small_dim(mats[b1]) == nn) ++b1;
    const int32_t nb = int32_t(b1 - b0);
    const int64_t sq = int64_t(nn) * nn;
    float* base = ws + L.ns;  // slot j starts at base + j * L.slot
    // per matrix: Gram A = M M^T (wide) or M^T M, then Y0, Z0 and the scale
    for (int32_t j = 0; j < nb; ++j) {
      const TensorPlan& t = plan[mats[b0 + j]];
      const int32_t r = int32_t(t.rows), c = int32_t(t.cols);
      const bool wide = r <= c;
      float* slot = base + j * L.slot;
      demo::GemmArgs g{};
      g.A = mstar[mats[b0 + j]];
      g.B = g.A;
      g.D = slot;
      g.M = g.N = nn;
      g.K = wide ? c : r;
      g.lda = g.ldb = c;
      g.ldd = nn;
      g.alpha = 1.f;
      if ((s = check(demo::launch_gemm(g, !wide, wide, 1, stream))) != DEMO_OK) return s;
      if ((s = check(demo::launch_ns_prepare(slot, nn, eps, reinterpret_cast<double*>(slot + L.partial),
                                             slot + L.scal, slot + sq, slot + 3 * sq, stream))) != DEMO_OK)
        return s;
    }
    float *Y = base + sq, *Y2 = base + 2 * sq, *Z = base + 3 * sq, *Z2 = base + 4 * sq, *T = base + 5 * sq;
    for (int32_t it = 0; it < iters; ++it) {
      demo::GemmArgs h{};
      h.M = h.N = h.K = nn;
      h.lda = h.ldb = h.ldd = nn;
      h.sA = h.sB = h.sD = L.slot;
      // T = 1.5 I - 0.5 Z Y
      h.A = Z;
      h.B = Y;
      h.D = T;
      h.alpha = -0.5f;
      h.gamma = 1.5f;
      if ((s = check(demo::launch_gemm(h, false, false, nb, stream))) != DEMO_OK) return s;
      h.gamma = 0.f;
      h.alpha = 1.f;
      h.A = Y;  // Y' = Y T
      h.B = T;
      h.D = Y2;
      if ((s = check(demo::launch_gemm(h, false, false, nb, stream))) != DEMO_OK) return s;
      h.A = T;  // Z' = T Z
      h.B = Z;
      h.D = Z2;
      if ((s = check(demo::launch_gemm(h, false, false, nb, stream))) != DEMO_OK) return s;
      std::swap(Y, Y2);
      std::swap(Z, Z2);
    }
    // per matrix: X = (1 - eta lambda) X - eta / sqrt(s) * (Z M  or  M Z), Z ~ (A + eps I)^(-1/2) sqrt(s)
    for (int32_t j = 0; j < nb; ++j) {
      const int32_t i = mats[b0 + j];
      const TensorPlan& t = plan[i];
      const int32_t r = int32_t(t.rows), c = int32_t(t.cols);
      const bool wide = r <= c;
      const float* Zj = Z + j * L.slot;
      demo::GemmArgs f{};
      f.A = wide ? Zj : mstar[i];
      f.B = wide ? mstar[i] : Zj;
      f.C = params[i];
      f.D = params[i];
      f.M = r;
      f.N = c;
      f.K = wide ? r : c;
      f.lda = wide ? nn : c;
      f.ldb = wide ? c : nn;
      f.ldc = f.ldd = c;
      f.alpha = -eta;
      f.alpha_scale = base + j * L.slot + L.scal + 1;
      f.beta = 1.f - eta * lambda;
      if ((s = check(demo::launch_gemm(f, false, false, 1, stream))) != DEMO_OK) return s;
    }
    b0 = b1;
  }
  return DEMO_OK;
}

}  // namespace

extern "C" {

demo_status demo_decode_apply_muon(demo_ctx* ctx, int32_t n, const demo_shape* shapes, float* const* params,
                                   const demo_codec_cfg* cfg, int32_t workers, const float* pay_values,
                                   const uint16_t* pay_idx, int64_t n_entries, float eta, float lambda, float eps,
                                   int32_t iters, demo_average avg, void* workspace, int64_t ws_bytes,
                                   hipStream_t stream) {
  return muon_decode(ctx, n, shapes, params, cfg, workers, pay_values, pay_idx, n_entries, eta, lambda, eps, iters,
                     avg, workspace, ws_bytes, stream);
}

demo_status demo_decode_apply_muon_noalloc(demo_ctx* ctx, int32_t n, const demo_shape* shapes, float* const* params,
                                           const demo_codec_cfg* cfg, int32_t workers, const float* pay_values,
                                           const uint16_t* pay_idx, int64_t n_entries, float eta, float lambda,
                                           float eps, int32_t iters, demo_average avg, hipStream_t stream) {
  std::vector<TensorPlan> plan;
  demo_status s = plan_list(shapes, n, kChunk, 1, &plan, nullptr, nullptr);
  if (s != DEMO_OK) return s;
  const int64_t need = muon_layout(plan).bytes;
  if (need > demo::kMuonScratchBytes)
    return fail(DEMO_ERR_RANGE, "the list needs " + std::to_string(need) + " bytes of Muon workspace; the static " +
                                    "scratch holds " + std::to_string(demo::kMuonScratchBytes) +
                                    " (use demo_decode_apply_muon with a workspace)");
  return muon_decode(ctx, n, shapes, params, cfg, workers, pay_values, pay_idx, n_entries, eta, lambda, eps, iters,
                     avg, nullptr, 0, stream, true);
}

}  // extern "C"
