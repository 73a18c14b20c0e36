/*
 * demo_codec.h -- C ABI of the MI355X (gfx950) DeMo per-step momentum codec.
 *
 * The codec is the data-parallel hot path of DeMo ("DeMo: Decoupled Momentum
 * Optimization", paper-graph-ui summary of arXiv 2411.19870, §3.4 Detailed,
 * sentence-based technical breakdown).  It is split where the pages place the
 * all-gather between workers (§3.4 Top-k Sparsification, last paragraph):
 *
 *   demo_encode        one worker, before communication: momentum update,
 *                      chunking, DCT, per-chunk top-k, payload, momentum
 *                      subtraction.
 *   demo_decode_apply  after communication: sparse averaging of W payloads,
 *                      inverse DCT, phi, parameter update.
 *   demo_decode_signs / demo_apply_signs
 *                      the same decode split once more for the Signum
 *                      variant's one-bit download (server side / worker side).
 *   demo_pack_wire / demo_decode_apply_wire
 *                      the payload in a compact wire format (bfloat16 values,
 *                      12-bit indices) and the decode that reads it.
 *   demo_decode_apply_muon
 *                      the decode with phi = Muon.
 *
 * Conventions for every call:
 *   - Tensors are dense, row-major, contiguous device buffers.  Matrices
 *     (ndim 2) are cut into s x s chunks, vectors (ndim 1) into s-element
 *     chunks, s = 64 (default) or 128 (DeMo summary §3.4 Tensor Chunking;
 *     Ablation Studies, chunk size s = 64 vs 128); trailing chunks are zero-padded for the
 *     transform and cropped on store.  Chunks are numbered tensor by tensor in
 *     list order, row-major inside a matrix.
 *   - A payload holds, for every chunk in that order, keff = min(k, chunk
 *     element count) entries: a float32 value array and a uint16 index array
 *     (index = u*s + v inside an s x s chunk, u the dimension-0 frequency;
 *     the frequency itself for a vector chunk), entries of a chunk in
 *     ascending index order.  demo_plan gives the entry count and offsets.
 *   - The caller owns every buffer.  Device pointers must be device memory of
 *     the context's device; host arrays (shape lists, pointer lists, the
 *     config) are read during the call only.
 *   - Calls enqueue kernels on `stream` and return without synchronising.
 *     They allocate no device memory and touch none before validation has
 *     passed: a non-DEMO_OK status means nothing was enqueued, except
 *     DEMO_ERR_HIP from a failed launch (earlier launches of the same call
 *     may then have been enqueued).
 *   - Inputs must be finite; NaN or Inf give unspecified (but memory-safe)
 *     results.  Payload indices outside a chunk are masked into it.
 *   - Calls are thread-safe; concurrent calls that write the same buffers race.
 *   - demo_last_error() returns a thread-local message for the last failure.
 */
#ifndef DEMO_CODEC_H
#define DEMO_CODEC_H

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DEMO_CHUNK 64        /* default chunk edge s (the pages' default) */
#define DEMO_CHUNK_LARGE 128 /* the other chunk edge built: DCT basis only, no Muon */
#define DEMO_MAX_WORKERS 255 /* decode keeps per-coefficient contributor counts in 8 bits */
#define DEMO_MAX_TENSORS_PER_LAUNCH 96 /* longer lists are split into several launches per call */

typedef enum demo_status {
  DEMO_OK = 0,
  DEMO_ERR_INVALID = 1, /* null pointer, unknown enum value, non-finite scalar */
  DEMO_ERR_SHAPE = 2,   /* ndim not 1 or 2, a zero or too large dimension */
  DEMO_ERR_RANGE = 3,   /* k < 1, chunk not 64 or 128 (or 128 where not built), workers outside 1..255, n < 0 */
  DEMO_ERR_PAYLOAD = 4, /* payload entry count differs from the plan */
  DEMO_ERR_DEVICE = 5,  /* no gfx950 device, or the current device is not the context's */
  DEMO_ERR_HIP = 6,     /* a HIP runtime call or launch failed */
  DEMO_ERR_ALIGN = 7    /* a device pointer is not aligned to its element size */
} demo_status;

/* Element type of the gradients (momentum, parameters and payload values are float32). */
typedef enum demo_dtype { DEMO_F32 = 0, DEMO_BF16 = 1 } demo_dtype;

/* Local momentum update, DeMo summary §3.4 Decoupled Local Momentum Updates:
 * DAMPED  M <- beta M + (1 - beta) G   (that section's equation)
 * PLAIN   M <- beta M + G              (the papernotes.org note's flowchart) */
typedef enum demo_momentum_form { DEMO_MOMENTUM_DAMPED = 0, DEMO_MOMENTUM_PLAIN = 1 } demo_momentum_form;

/* Projection, DeMo summary §3.4 Blockwise Linear Projection (DCT):
 * DCT       orthonormal DCT-II on both chunk dimensions (P0 = P1 = P, P^T = P^-1)
 * USER      caller-supplied orthonormal P0, P1 (e.g. the random orthonormal
 *           projection re-drawn every step, identical on all workers)
 * IDENTITY  P0 = P1 = I: top-k in the parameter domain (the identity choice
 *           that section compares against) */
typedef enum demo_basis { DEMO_BASIS_DCT = 0, DEMO_BASIS_USER = 1, DEMO_BASIS_IDENTITY = 2 } demo_basis;

/* phi of DeMo summary §3.4 Base Optimizer Update: sign (Signum) or identity (SGD). */
typedef enum demo_phi { DEMO_PHI_SIGN = 0, DEMO_PHI_IDENTITY = 1 } demo_phi;

/* Denominator of the sparse average, DeMo summary §3.4 Server-Side Aggregation:
 * CONTRIBUTORS  number of workers whose payload holds the index (default)
 * WORKERS       W (a worker without the index contributes a zero) */
typedef enum demo_average { DEMO_AVG_CONTRIBUTORS = 0, DEMO_AVG_WORKERS = 1 } demo_average;

/* What the momentum subtraction removes (DeMo summary §3.4 Momentum
 * Subtraction as Implicit Error Feedback, which writes the aggregated
 * coefficients; the papernotes.org note's 关键设计 3 subtracts what the worker
 * itself sent, before the all-gather):
 * LOCAL       demo_encode leaves M' - alpha * unchunk(P0^T Q_hat P1), Q_hat the
 *             worker's own selected coefficients (default)
 * AGGREGATED  demo_encode leaves M' untouched; demo_decode_apply_subtract then
 *             removes alpha * unchunk(P0^T Q_bar P1) = alpha * M*, Q_bar the
 *             average of all W payloads */
typedef enum demo_subtraction { DEMO_SUBTRACT_LOCAL = 0, DEMO_SUBTRACT_AGGREGATED = 1 } demo_subtraction;

typedef struct demo_shape {
  int32_t ndim;    /* 1 or 2 */
  int64_t dims[2]; /* dims[1] ignored for ndim 1; each in 1 .. 2^31-1 */
} demo_shape;

typedef struct demo_codec_cfg {
  int32_t chunk;         /* chunk edge s: DEMO_CHUNK, or DEMO_CHUNK_LARGE with the DCT basis */
  int32_t k;             /* coefficients kept per chunk, >= 1; clamped to the chunk's element count */
  float beta;            /* momentum decay (DeMo summary §3.4 Decoupled Local Momentum Updates) */
  float alpha;           /* momentum-subtraction coefficient (§3.4 Momentum Subtraction) */
  int32_t momentum_form; /* demo_momentum_form */
  int32_t basis;         /* demo_basis */
  const float* P0;       /* DEMO_BASIS_USER: device 64x64 fp32 row-major, rows are the basis
                            vectors, 16-byte aligned; acts on dimension 0 and on vectors */
  const float* P1;       /* DEMO_BASIS_USER with any matrix: device 64x64, 16-byte aligned, acts on
                            dimension 1 */
  int32_t subtraction;   /* demo_subtraction */
} demo_codec_cfg;

typedef struct demo_ctx demo_ctx;

/* Bind a context to HIP device `device`; fails with DEMO_ERR_DEVICE unless it is gfx950.
 * Every later call must run with that device current. */
demo_status demo_ctx_create(int32_t device, demo_ctx** out);
void demo_ctx_destroy(demo_ctx* ctx);

/* Thread-local description of the last non-DEMO_OK status of this thread ("" if none). */
const char* demo_last_error(void);

/* Host-only planning (no device work, no context needed).
 * n_chunks:    total chunks of the list (may be NULL)
 * n_entries:   payload entries per worker, sum over chunks of keff (may be NULL)
 * entry_begin: if not NULL, n+1 entries: payload offset of every tensor's first
 *              chunk, and the total at [n]. */
demo_status demo_plan(const demo_shape* shapes, int32_t n, int32_t chunk, int32_t k, int64_t* n_chunks,
                      int64_t* n_entries, int64_t* entry_begin);

/* One worker's encode of a tensor list (DeMo summary §3.4: Decoupled Local
 * Momentum Updates, Tensor Chunking, Blockwise Linear Projection, Top-k
 * Sparsification, Momentum Subtraction as Implicit Error Feedback).
 *   grads[i]:  device, shapes[i], element type grad_dtype; read only
 *   moms[i]:   device float32, shapes[i]; read and overwritten with
 *              M' - alpha * unchunk(P0^T Q_hat P1), where M' is the updated
 *              momentum and Q_hat this worker's own selected coefficients
 *              (with cfg->subtraction == DEMO_SUBTRACT_AGGREGATED: with M')
 *   pay_values / pay_idx: device arrays of n_entries entries, written
 * Top-k ranks float32 magnitudes; equal magnitudes go to the lower index. */
demo_status demo_encode(demo_ctx* ctx, int32_t n, const demo_shape* shapes, const void* const* grads,
                        demo_dtype grad_dtype, float* const* moms, const demo_codec_cfg* cfg, float* pay_values,
                        uint16_t* pay_idx, int64_t n_entries, hipStream_t stream);

/* Decode W payloads and apply the update to a tensor list (DeMo summary §3.4:
 * Server-Side Aggregation and Momentum Reconstruction, Inverse DCT and
 * Unchunking, Base Optimizer Update).
 *   params[i]:  device float32, shapes[i]; read and overwritten with
 *               X - eta * (phi(M*) + lambda * X), X the pre-update value
 *   pay_values / pay_idx: device, workers x n_entries entries (worker-major, as
 *               an all-gather lays them out); read only
 * cfg supplies chunk, k and the basis; its beta, alpha, momentum_form and
 * subtraction are unused.  Coefficients are summed in worker order 0..W-1;
 * the result is deterministic. */
demo_status demo_decode_apply(demo_ctx* ctx, int32_t n, const demo_shape* shapes, float* const* params,
                              const demo_codec_cfg* cfg, int32_t workers, const float* pay_values,
                              const uint16_t* pay_idx, int64_t n_entries, demo_phi phi, float eta, float lambda,
                              demo_average avg, hipStream_t stream);

/* The decode of DEMO_SUBTRACT_AGGREGATED (DeMo summary §3.4 Momentum
 * Subtraction as Implicit Error Feedback, with the aggregated coefficients):
 * the same M* as demo_decode_apply, applied to the parameters and/or to one
 * worker's momentum in one pass.
 *   params: as for demo_decode_apply, or NULL to leave the parameters alone
 *   moms:   NULL, or device float32 tensors (shapes[i]) overwritten with
 *           M - cfg->alpha * M*
 * At least one of params and moms must be given.  A worker runs it once with
 * both; a single-device simulation of W workers passes the parameters with
 * one worker's momenta and then each other worker's momenta alone. */
demo_status demo_decode_apply_subtract(demo_ctx* ctx, int32_t n, const demo_shape* shapes, float* const* params,
                                       float* const* moms, const demo_codec_cfg* cfg, int32_t workers,
                                       const float* pay_values, const uint16_t* pay_idx, int64_t n_entries,
                                       demo_phi phi, float eta, float lambda, demo_average avg, hipStream_t stream);

/* ---- One-bit download of the Signum variant (DeMo summary §3.4 Base Optimizer
 * Update: with phi = sign the server broadcasts only sign(M*), one bit per
 * parameter, and every worker applies it to its own copy of X).
 * Built for both chunk edges (64, and 128 with the DCT basis).
 * Packed-sign layout: uint64 words, chunk after chunk in the chunk order of the
 * payload; inside a chunk its elements in row-major order, 64 to a word, bit j
 * the j-th of them.  A 64x64 chunk takes 64 words (word i = chunk row i, bit
 * j = column j), a 128x128 chunk 256 (word 2i + h = chunk row i, columns
 * 64h .. 64h + 63), a vector chunk s / 64 words.  A bit is set
 * where M* < 0; M* = 0 reads as +1, since one bit cannot carry sign(0) = 0.
 * Padding positions hold 0.
 * This differs from demo_decode_apply with DEMO_PHI_SIGN exactly where M* = 0:
 * there the Signum decode leaves X <- X (1 - eta lambda), this path applies
 * X <- X - eta (1 + lambda X).  M* is exactly 0 only where no worker sent a
 * non-zero coefficient for the element's chunk (e.g. a tensor whose gradients
 * are all zero); everywhere else the two paths give the same parameters. */

/* Host-only: words of the packed sign of a list (n_words, may be NULL) and, if
 * word_begin is not NULL, the first word of every tensor (n+1 entries, the
 * total at [n]). */
demo_status demo_plan_signs(const demo_shape* shapes, int32_t n, int32_t chunk, int64_t* n_words,
                            int64_t* word_begin);

/* Server side: the sparse average of W payloads, inverse transform and
 * unchunking of demo_decode_apply, then sign(M*) packed as above.
 *   signs: device, n_words uint64 words (8-byte aligned); every word is written
 * cfg supplies chunk, k and the basis; the other fields are unused. */
demo_status demo_decode_signs(demo_ctx* ctx, int32_t n, const demo_shape* shapes, const demo_codec_cfg* cfg,
                              int32_t workers, const float* pay_values, const uint16_t* pay_idx, int64_t n_entries,
                              demo_average avg, uint64_t* signs, int64_t n_words, hipStream_t stream);

/* Worker side: X <- X - eta * (s + lambda * X) with the pre-update X, s = -1
 * where the tensor's bit is set and +1 elsewhere.
 *   params[i]: device float32, shapes[i]; read and overwritten
 *   signs:     device, n_words words laid out as demo_decode_signs writes them;
 *              read only */
demo_status demo_apply_signs(demo_ctx* ctx, int32_t n, const demo_shape* shapes, float* const* params,
                             int32_t chunk, const uint64_t* signs, int64_t n_words, float eta, float lambda,
                             hipStream_t stream);

/* ---- Compact wire format (teaching deck "Training over Slow Links", top-k
 * and DeMo slides: a kept value travels as 2 bytes of bfloat16 plus its
 * position).  A position takes b bits, enough for a matrix chunk's s*s
 * positions: b = 12 at chunk edge 64, b = 14 at chunk edge 128.
 * A worker's wire payload of E entries is two arrays:
 *   values:  E uint16 bfloat16 bit patterns, entry order kept; float32 ->
 *            bfloat16 rounds to nearest, ties to even
 *   indices: entry j's b-bit position sits at bits bj .. bj + b - 1 of the
 *            array read as one little-endian bit string (bit t = bit t mod 8
 *            of byte t / 8).  The array is whole groups of 32-bit words, 12
 *            bytes per 8 entries (b = 12) or 28 bytes per 16 (b = 14), so
 *            idx_bytes = 12 ceil(E / 8) or 28 ceil(E / 16); the bits past the
 *            last entry are zero.
 * W wire payloads lie worker-major: values as W x E uint16, indices as
 * W x demo_wire_size's idx_bytes. */

/* Host-only: bytes of one worker's wire values (2E) and indices at chunk
 * edge `chunk` (64 or 128, else DEMO_ERR_RANGE). */
demo_status demo_wire_size(int32_t chunk, int64_t n_entries, int64_t* value_bytes, int64_t* idx_bytes);

/* Convert `workers` payloads (worker-major, n_entries each, as demo_encode
 * writes them at chunk edge `chunk`) into the wire format.  Indices are sent
 * modulo 2^b (a chunk's indices are below that).
 *   wire_values: device, workers x n_entries uint16 (2-byte aligned); written
 *   wire_idx:    device, workers x idx_bytes bytes (4-byte aligned); written,
 *                padding included */
demo_status demo_pack_wire(demo_ctx* ctx, int32_t chunk, int32_t workers, const float* pay_values,
                           const uint16_t* pay_idx, int64_t n_entries, uint16_t* wire_values, void* wire_idx,
                           hipStream_t stream);

/* demo_decode_apply reading W wire payloads directly (values widened from
 * bfloat16, indices unpacked in the kernel; nothing is unpacked into memory).
 * Arguments as for demo_decode_apply, the payload given as wire arrays
 * (read only) packed at cfg->chunk. */
demo_status demo_decode_apply_wire(demo_ctx* ctx, int32_t n, const demo_shape* shapes, float* const* params,
                                   const demo_codec_cfg* cfg, int32_t workers, const uint16_t* wire_values,
                                   const void* wire_idx, int64_t n_entries, demo_phi phi, float eta, float lambda,
                                   demo_average avg, hipStream_t stream);

/* ---- phi = Muon (DeMo summary §3.4 Base Optimizer Update: phi(M) =
 * M (M^T M + eps I)^(-1/2), Newton-Schulz normalization).  phi acts on each
 * whole tensor, so the decode first writes M* of every tensor into a
 * workspace; a matrix then goes through its smaller Gram matrix and the
 * coupled Newton-Schulz iteration for the inverse square root (products on
 * the matrix cores at float32 accuracy), a vector (one column) through
 * m / sqrt(m.m + eps).  Built for chunk edge 64. */

/* Host-only: bytes of device workspace demo_decode_apply_muon needs for a list:
 * M* of every tensor, then one slot of Newton-Schulz matrices (six n x n,
 * n the largest smaller dimension) per matrix of a batch, up to 8 matrices
 * with equal smaller dimension sharing each iteration launch. */
demo_status demo_muon_workspace(const demo_shape* shapes, int32_t n, int64_t* ws_bytes);

/* demo_decode_apply with phi = Muon: X <- X - eta * (phi(M*) + lambda * X).
 *   eps:       the eps of the formula (absolute), finite and >= 0
 *   iters:     Newton-Schulz iterations, 1..64 (each costs three n x n x n
 *              products, n the smaller dimension of the matrix)
 *   workspace: device, at least demo_muon_workspace bytes, 16-byte aligned;
 *              scratch owned by the caller, contents undefined afterwards
 * Other arguments as for demo_decode_apply; cfg->chunk must be 64. */
demo_status demo_decode_apply_muon(demo_ctx* ctx, int32_t n, const demo_shape* shapes, float* const* params,
                                   const demo_codec_cfg* cfg, int32_t workers, const float* pay_values,
                                   const uint16_t* pay_idx, int64_t n_entries, float eta, float lambda, float eps,
                                   int32_t iters, demo_average avg, void* workspace, int64_t ws_bytes,
                                   hipStream_t stream);

/* ---- The Muon decode without allocation, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).
 *
 * demo_decode_apply_muon with the workspace taken from a static device array
 * of DEMO_MUON_SCRATCH_BYTES that the library holds on every device it runs
 * on, until the process ends.  Nothing is allocated by the call.
 *   - A list whose workspace (demo_muon_workspace) exceeds
 *     DEMO_MUON_SCRATCH_BYTES is refused with DEMO_ERR_RANGE before anything
 *     is enqueued.
 *   - All calls on one GPU share that GPU's scratch.  Calls that overlap on
 *     one GPU (different streams, or different threads without ordering)
 *     race; calls ordered on one stream do not.  The scratch keeps the last
 *     call's contents; no part of it has to start at zero.
 * Other arguments, validation and errors as for demo_decode_apply_muon. */
#define DEMO_MUON_SCRATCH_BYTES (64ll << 20)

demo_status demo_decode_apply_muon_noalloc(demo_ctx* ctx, int32_t n, const demo_shape* shapes, float* const* params,
                                           const demo_codec_cfg* cfg, int32_t workers, const float* pay_values,
                                           const uint16_t* pay_idx, int64_t n_entries, float eta, float lambda,
                                           float eps, int32_t iters, demo_average avg, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DEMO_CODEC_H */
