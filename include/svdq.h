/*
 * svdq.h -- C ABI of the SVDQuant linear layer for AMD Instinct MI355X (gfx950).
 *
 * The layer computes, for activations X (M x K) and a weight W (K x N),
 *
 *     Y = (X diag(lambda)^-1) L1 L2  +  Q(X diag(lambda)^-1) Q(R)  (+ bias)
 *
 * SVDQuant paper ("SVDQuant: Absorbing Outliers by Low-Rank Components for
 * 4-Bit Diffusion Models", translated article on developer.volcengine.com):
 *   - smoothing by per-channel factors lambda            §4.2, Fig. 4
 *   - rank-r SVD split W_hat = L1 L2 + R                 §4.2, Eq. 5, Fig. 5
 *   - symmetric group quantizer Q, INT4 / FP4            §3; §5.1 impl. details
 *   - down-projection fused with the activation quantizer,
 *     up-projection fused with the 4-bit product         §4.3, Fig. 6b
 *   - LoRA concatenated into the low-rank branch         §5.2 (LoRA), §1
 *
 * Conventions for every entry point:
 *   - Every call returns an svdq_status; nothing throws or aborts across
 *     the ABI.  Argument and shape errors are reported synchronously before
 *     anything is launched.
 *   - All device memory (packed blob, X, Y, workspace) is allocated and owned
 *     by the caller.  The library never allocates device memory; the one
 *     exception, svdq_linear_forward_noalloc, uses a fixed array that is part
 *     of the library's device code object.
 *   - Row-major storage.  X is M x K with row stride ldx elements, Y is
 *     M x N with row stride ldy elements, both in the layer's 16-bit dtype.
 *   - Host buffers passed to synchronous calls may be freed on return.
 *   - Forward calls are asynchronous on the caller's stream; forwards on
 *     different streams may run concurrently.  Attaching/detaching a LoRA
 *     must not race with forwards of the same layer.
 */
#ifndef SVDQ_H
#define SVDQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SVDQ_OK = 0,
  SVDQ_ERR_INVALID_ARG = 1,  /* null pointer, bad enum, negative size, bad rank */
  SVDQ_ERR_SHAPE = 2,        /* K not a multiple of 128, N of 128, strides too small */
  SVDQ_ERR_UNSUPPORTED = 3,  /* valid request the library does not implement */
  SVDQ_ERR_CAPACITY = 4,     /* buffer too small, LoRA rank beyond the capacity */
  SVDQ_ERR_NUMERIC = 5,      /* non-finite weights or calibration maxima */
  SVDQ_ERR_HIP = 6           /* a HIP runtime call or kernel launch failed */
} svdq_status;

typedef enum {
  SVDQ_FMT_INT4_G64 = 0,     /* signed INT4 codes in [-7, 7], group 64 along K, fp16 scales */
  SVDQ_FMT_MXFP4_G32 = 1,    /* E2M1 codes, group 32 along K, e8m0 (power-of-two) scales */
  SVDQ_FMT_INT8_W8A8 = 2,    /* the 8-bit setting (SVDQuant §5.1 implementation details): signed
                                INT8 codes in [-127, 127], one fp32 scale per output channel of
                                the residual and, computed on the fly, per token of X_hat */
  /* range markers (not formats): they make every int a value of the type, so
     an unknown value passed in is reported (SVDQ_ERR_INVALID_ARG), not
     undefined behaviour of the C++ implementation */
  SVDQ_FMT_RANGE_MIN_ = -2147483647 - 1,
  SVDQ_FMT_RANGE_MAX_ = 2147483647
} svdq_format;

typedef enum {
  SVDQ_F16 = 0,
  SVDQ_BF16 = 1,
  SVDQ_DTYPE_RANGE_MIN_ = -2147483647 - 1,   /* range markers, as for svdq_format */
  SVDQ_DTYPE_RANGE_MAX_ = 2147483647
} svdq_dtype;

enum {
  SVDQ_FLAG_GELU = 1u,            /* apply x * Phi(x) (erf GELU) to Y before rounding */
  SVDQ_FLAG_UNFUSED_LOWRANK = 2u, /* baseline for measuring the fusion: run the low-rank
                                     branch as separate passes (a second read of X for T,
                                     then Y is read back and rewritten with T L2 added),
                                     as an engine without the fusion would; Y is rounded
                                     twice.  svdq_linear_forward only. */
  SVDQ_FLAG_TRACE = 4u            /* record the GEMM's per-workgroup start / end times and
                                     shader-clock cycles (svdq_trace_read); results are
                                     unchanged.  svdq_linear_forward, svdq_gemm_forward,
                                     svdq_linear_forward_noalloc. */
};

#define SVDQ_MAX_RANK_CAPACITY 128

/* Descriptor of one packed layer (plain data, caller-owned).  It points into
 * the caller's blob; all offsets are bytes from `blob`.  The blob holds no
 * absolute pointers, so copying its bytes moves the layer (save/restore). */
typedef struct {
  int64_t K, N;
  int32_t rank;            /* SVD rank r of the split */
  int32_t rank_active;     /* r + rank of the attached LoRA */
  int32_t rank_capacity;   /* factor slots reserved at pack time (>= rank) */
  int32_t rank_slots;      /* rank_capacity rounded up to a multiple of 32 */
  int32_t fmt;             /* svdq_format */
  int32_t dtype;           /* svdq_dtype */
  int32_t has_bias;
  int32_t blob_on_device;  /* 1: blob is device memory, 0: host memory */
  void* blob;
  size_t blob_bytes;
  size_t off_invlam, off_lam, off_l1x, off_l2, off_wq, off_sw, off_bias;
} svdq_layer;

const char* svdq_status_string(svdq_status s);

/* ---------------------------------------------------------------- pack --- */

/* Bytes of the packed blob for a K x N layer with `rank_capacity` factor
 * slots.  Layout: header, 1/lambda and lambda (fp32 [K]), L1x (16-bit,
 * K x slots, tiled for the activation kernel), L2 (16-bit, slots x N, tiled
 * for the GEMM epilogue), residual codes (4-bit, K x N, tiled as matrix-core
 * fragments), group scales, bias (fp32 [N]). */
svdq_status svdq_packed_size(int64_t K, int64_t N, int rank_capacity, svdq_format fmt,
                             svdq_dtype dtype, size_t* bytes);

/* Offline post-training quantization of one linear layer (SVDQuant §4.2):
 *   lambda_j = sqrt(act_absmax[j] / max_n |W[j,n]|) (fp32; 1 for a zero
 *     channel or when act_absmax is NULL),
 *   W_hat = diag(lambda) W, truncated SVD W_hat ~ L1 L2 with L1 = U_r S_r,
 *   L1x = 16-bit(diag(1/lambda) L1), L2 = 16-bit(V_r^T),
 *   R = fp32(W_hat - diag(lambda) L1x L2), quantized per output column in
 *   K-groups (INT4 g64 / MXFP4 g32), all tiled for the GEMM.
 * W_host: K x N, 16-bit `dtype`, row stride ldw.  act_absmax_host: [K] fp32
 * per-channel calibration maxima of |X| or NULL.  bias_host: [N] 16-bit or
 * NULL.  0 <= rank <= min(K, N, rank_capacity), rank_capacity <=
 * SVDQ_MAX_RANK_CAPACITY.  Requires K % 128 == 0 and N % 128 == 0.
 * svdq_pack_weights writes the blob to device memory blob_dev (>=
 * svdq_packed_size bytes) and returns after the copy finished on `stream`;
 * svdq_pack_weights_host writes it to host memory.  `out` receives the
 * descriptor.  Synchronous. */
svdq_status svdq_pack_weights(const void* W_host, int64_t K, int64_t N, int64_t ldw, svdq_dtype dtype,
                              const float* act_absmax_host, int rank, int rank_capacity, svdq_format fmt,
                              const void* bias_host, void* blob_dev, size_t blob_bytes, hipStream_t stream,
                              svdq_layer* out);
svdq_status svdq_pack_weights_host(const void* W_host, int64_t K, int64_t N, int64_t ldw, svdq_dtype dtype,
                                   const float* act_absmax_host, int rank, int rank_capacity, svdq_format fmt,
                                   const void* bias_host, void* blob_host, size_t blob_bytes, svdq_layer* out);

/* svdq_pack_weights with iterative refinement of the low-rank split
 * [SVDQuant §4.2, the closing remark on the low-rank branch]: after the
 * one-shot split, each of refine_iters rounds splits W_hat - deq(Q(R)) at
 * rank `rank` again (deq(Q(R)): the previous round's quantized residual),
 * rounds the factors to 16 bits, re-derives R and its codes, and measures
 * err = ||W_hat - diag(lambda) L1x L2 - deq(Q(R))||_F^2 (float64).  The split
 * with the smallest err is packed.  0 <= refine_iters <=
 * SVDQ_MAX_REFINE_ITERS; refine_iters = 0 packs exactly what
 * svdq_pack_weights packs.  errors_out: NULL or [refine_iters + 1] doubles,
 * err of the one-shot split first.  blob_on_device: 1 = blob is device
 * memory (copied on `stream`), 0 = host memory.  Synchronous; each round
 * costs about one pack. */
#define SVDQ_MAX_REFINE_ITERS 16
svdq_status svdq_pack_weights_ex(const void* W_host, int64_t K, int64_t N, int64_t ldw, svdq_dtype dtype,
                                 const float* act_absmax_host, int rank, int rank_capacity, svdq_format fmt,
                                 const void* bias_host, int refine_iters, double* errors_out, void* blob,
                                 size_t blob_bytes, int blob_on_device, hipStream_t stream, svdq_layer* out);

/* Copy a packed layer's blob (host or device) to another buffer (host or
 * device) and describe the copy in `out` (restore / upload).  dst_on_device
 * selects the destination kind.  Synchronous on `stream`. */
svdq_status svdq_layer_copy(const svdq_layer* src, void* dst, size_t dst_bytes, int dst_on_device,
                            hipStream_t stream, svdq_layer* out);

/* Concatenate a LoRA (A: K x rL, B: rL x N, 16-bit host matrices, row-major)
 * into the low-rank branch: L1x[:, rank:rank+rL] = A, L2[rank:rank+rL, :] =
 * 16-bit(alpha * B).  The residual and its codes are untouched (no
 * re-quantization, SVDQuant §5.2).  Replaces any LoRA attached before.
 * Error SVDQ_ERR_CAPACITY if rank + rL > rank_capacity.  Synchronous. */
svdq_status svdq_attach_lora(svdq_layer* layer, const void* A_host, const void* B_host, int rL,
                             float alpha, hipStream_t stream);
/* Zero the LoRA slots and set rank_active = rank.  Synchronous. */
svdq_status svdq_detach_lora(svdq_layer* layer, hipStream_t stream);

/* ------------------------------------------------------------- forward --- */

/* Bytes of device workspace a forward of M tokens needs (4-bit activation
 * codes and scales, and the 16-bit down-projection T = X L1x). */
svdq_status svdq_workspace_size(const svdq_layer* layer, int64_t M, size_t* bytes);

/* Y = X_hat L1x L2 + Q(X_hat) Q(R) + bias [-> GELU], rounded to the layer's
 * dtype (SVDQuant §4.2 Eq. 5, fused as in §4.3).  flags: SVDQ_FLAG_GELU,
 * SVDQ_FLAG_UNFUSED_LOWRANK (see above).  Two kernels on `stream`:
 * the activation kernel (smoothing, group quantization, down-projection,
 * one pass over X) and the 4-bit GEMM with the up-projection, bias and
 * optional GELU in its epilogue.  X_dev: M x K (ldx >= K, ldx % 8 == 0,
 * 16-byte aligned); Y_dev: M x N (ldy >= N, ldy % 8 == 0, 16-byte aligned);
 * ws_dev: >= svdq_workspace_size bytes, 256-byte aligned.  M >= 0 (M == 0
 * is a no-op).  SVDQ_ERR_UNSUPPORTED if an operand span the GEMM addresses
 * with 31-bit offsets reaches 2 GiB: MXFP4 and INT8, the workspace or the
 * blob's span from L2 to the bias; INT4, the weight codes (N K / 2 bytes)
 * or the activation codes (M rounded up to 256, times K / 2 bytes).
 * Asynchronous. */
svdq_status svdq_linear_forward(const svdq_layer* layer, const void* X_dev, int64_t M, int64_t ldx,
                                void* Y_dev, int64_t ldy, void* ws_dev, size_t ws_bytes, unsigned flags,
                                hipStream_t stream);

/* svdq_linear_forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the workspace is a library-owned device array of
 * SVDQ_NOALLOC_SCRATCH_BYTES per GPU (each GPU the library runs on holds it
 * until the process ends).  Same arguments, kernels and results as
 * svdq_linear_forward, minus ws_dev / ws_bytes.  Calls no allocating routine.
 * SVDQ_ERR_CAPACITY if svdq_workspace_size(layer, M) exceeds the array (32 MiB
 * covers the 4-bit formats at 4608 tokens with K up to 12288 and rank
 * capacity 128).
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (several streams, or several host threads) race and must be serialised
 * by the caller.  Nothing in the array needs to start at zero (each kernel
 * writes what the next reads).  Asynchronous. */
#define SVDQ_NOALLOC_SCRATCH_BYTES (32u << 20)
svdq_status svdq_linear_forward_noalloc(const svdq_layer* layer, const void* X_dev, int64_t M, int64_t ldx,
                                        void* Y_dev, int64_t ldy, unsigned flags, hipStream_t stream);

/* The two stages of svdq_linear_forward, callable on their own (the second
 * reads what the first wrote into ws_dev).  Asynchronous. */
svdq_status svdq_quantize_activations(const svdq_layer* layer, const void* X_dev, int64_t M, int64_t ldx,
                                      void* ws_dev, size_t ws_bytes, hipStream_t stream);
svdq_status svdq_gemm_forward(const svdq_layer* layer, int64_t M, void* Y_dev, int64_t ldy,
                              const void* ws_dev, size_t ws_bytes, unsigned flags, hipStream_t stream);

/* Epilogue chaining of two layers where the output of `first` is the input
 * of `next` (an MLP's fc1 -> fc2).  The pages' engine keeps operations that
 * share an input in one kernel (SVDQuant §4.3, Fig. 6); here the same idea
 * runs across a layer boundary: the 4-bit GEMM of `first` computes, in its
 * epilogue and from the 16-bit output bits it would store, `next`'s
 * smoothing, group quantization (codes and scales into ws_next_dev) and
 * fp32 partial down-projections (one slab per GEMM column tile of `first`:
 * 192 output columns for MXFP4 with GELU, 256 without, 128 for INT4; in
 * ws_dev, sized by svdq_chain_workspace_size for the narrowest); a small kernel
 * then sums the slabs in a fixed order and rounds T once into ws_next_dev.
 * The activation pass of `next` over `first`'s output is gone;
 * svdq_gemm_forward(next, M, ..., ws_next_dev, ...) finishes `next`.  Codes
 * and scales are identical to what svdq_quantize_activations writes for that
 * output; T differs only in fp32 summation order.
 * Requires: both layers MXFP4 or both INT4 (else SVDQ_ERR_UNSUPPORTED), the
 * same dtype (else SVDQ_ERR_INVALID_ARG), first->N == next->K (else
 * SVDQ_ERR_SHAPE).
 * X_dev as for svdq_linear_forward on `first`; Y_dev may be NULL (the
 * output of `first` is then not stored; else as for svdq_linear_forward);
 * flags: SVDQ_FLAG_GELU for `first`.  ws_dev: >= svdq_chain_workspace_size
 * bytes; ws_next_dev: >= svdq_workspace_size(next, M) bytes; both 256-byte
 * aligned and not overlapping.  Deterministic.  Asynchronous. */
svdq_status svdq_chain_workspace_size(const svdq_layer* first, const svdq_layer* next, int64_t M, size_t* bytes);
svdq_status svdq_linear_forward_chain(const svdq_layer* first, const svdq_layer* next, const void* X_dev,
                                      int64_t M, int64_t ldx, void* Y_dev, int64_t ldy, void* ws_dev,
                                      size_t ws_bytes, void* ws_next_dev, size_t ws_next_bytes, unsigned flags,
                                      hipStream_t stream);

/* Calibration statistic for smoothing (SVDQuant §4.2): absmax_dev[k] =
 * max(absmax_dev[k], max_m |X[m,k]|), fp32, exact.  Initialise absmax_dev to
 * zero before the first batch.  Asynchronous. */
svdq_status svdq_activation_absmax(const void* X_dev, int64_t M, int64_t K, int64_t ldx, svdq_dtype dtype,
                                   float* absmax_dev, hipStream_t stream);

/* --------------------------------------------------------- inspection --- */

/* Canonical (untiled) copies of a packed layer, written to host buffers;
 * any output pointer may be NULL.  lam, invlam: [K] fp32.  l1x: K x
 * rank_active 16-bit.  l2: rank_active x N 16-bit.  codes: K x N bytes
 * (INT4: int8 value in [-7, 7]; MXFP4: E2M1 code 0..15; INT8: int8 value
 * in [-127, 127]).  scales: (K/G) x N (INT4: fp16 bits as uint16; MXFP4:
 * e8m0 bytes; INT8: 1 x N fp32).  bias: [N] fp32.
 * Synchronous (copies the blob from the device when it lives there). */
svdq_status svdq_layer_export(const svdq_layer* layer, float* lam, float* invlam, void* l1x, void* l2,
                              void* codes, void* scales, float* bias, hipStream_t stream);

/* Canonical copies of what svdq_quantize_activations wrote for M tokens:
 * codes M x K bytes (as above), scales M x (K/G) (INT8: M x 1 fp32), t: M x rank_active
 * 16-bit (the rounded down-projection).  Synchronous. */
svdq_status svdq_workspace_export(const svdq_layer* layer, const void* ws_dev, size_t ws_bytes, int64_t M,
                                  void* codes, void* scales, void* t, hipStream_t stream);

/* The fp64 factors of the truncated SVD the pack uses, before any 16-bit
 * rounding: L1 (K x rank) = U_r S_r, L2 (rank x N) = V_r^T, sigma[rank] the
 * top singular values, and lambda [K].  Host only, synchronous. */
svdq_status svdq_svd_factors(const void* W_host, int64_t K, int64_t N, int64_t ldw, svdq_dtype dtype,
                             const float* act_absmax_host, int rank, double* L1, double* L2, double* sigma,
                             float* lam);

/* INT4 layers only: the per-group integer products P_g[m,n] = sum over the
 * 64 k of group g of code_x[m,k] code_w[k,n] for the window m in
 * [m0, m0+nm), n in [n0, n0+nn), g in [g0, g0+ng).  A separate test kernel
 * computes them; it is not the GEMM, but it forms each product the way the
 * GEMM does -- the same nibble widening of the packed codes and the same
 * 16 x 16 x 64 int8 matrix instruction on the same operand layout -- so
 * the GEMM's partials equal these by construction (the GEMM feeds its own
 * straight into the fp32 scale multiply-add and never stores them).
 * out_dev: int32 [ng][nm][nn] device buffer.  Reads the codes
 * svdq_quantize_activations left in ws_dev.
 * Requires m0 % 16 == 0, n0 % 16 == 0, nm % 16 == 0, nn % 16 == 0.
 * Asynchronous. */
svdq_status svdq_int4_group_partials(const svdq_layer* layer, const void* ws_dev, size_t ws_bytes, int64_t M,
                                     int64_t m0, int64_t nm, int64_t n0, int64_t nn, int64_t g0, int64_t ng,
                                     int32_t* out_dev, hipStream_t stream);

/* ---------------------------------------------------- measurement hooks --- */

/* The trace of the last GEMM launched with SVDQ_FLAG_TRACE on the current
 * device: for each of its *n_records workgroups (at most 65536 are kept),
 * four counters -- wall clock and shader clock when the workgroup started,
 * wall clock and shader clock after its last store was issued.  The wall
 * clock runs at *wall_hz; cycles / wall time is the shader clock the
 * workgroup ran at.  An MXFP4 or INT8 GEMM of more than three rounds of
 * tiles launches workgroups past some XCDs' tile shares; those run no tile
 * and record start and end a fraction of a microsecond apart.  Writes
 * min(*n_records, max_records) records (4 x uint64 each) to host memory
 * `records`.  Synchronizes the device.  A
 * library-owned array per device holds the trace: traced launches that
 * overlap on one device overwrite each other's records. */
svdq_status svdq_trace_read(unsigned long long* records, int max_records, int* n_records, double* wall_hz);

/* Shader clock of the current device right now, in MHz: a short spin on
 * every compute unit timed by the shader-clock counter (s_memtime) and the
 * constant-rate wall counter (s_memrealtime).  Run right after a workload,
 * it reports the clock the power management settled on under that load.
 * Synchronous on `stream`.  Not thread-safe against itself on one device
 * (a lock inside serialises host threads). */
svdq_status svdq_probe_clock(hipStream_t stream, double* mhz);

/* Sustained rate of the scaled FP4 matrix instruction the MXFP4 GEMM uses
 * (V_MFMA_SCALE_F32_32X32X64_F8F6F4, E2M1 operands): eight waves on every
 * compute unit, `iters` x 9 independent instructions each, no memory
 * traffic.  random_operands = 0 feeds zero codes, else pseudo-random codes
 * (the matrix core's power, and with it the clock the chip can hold,
 * depends on the operand bits).  tflops: achieved dense rate; mhz: the
 * mean shader clock over the loop.  1 <= iters <= 2^24.  Synchronous. */
svdq_status svdq_probe_mfma_rate(int random_operands, int iters, hipStream_t stream, double* tflops, double* mhz);

/* Kinds of kernel launch that svdq_timing_stop reports. */
typedef enum {
  SVDQ_KERNEL_ACT = 1,     /* activation kernel: smoothing, quantization, down-projection */
  SVDQ_KERNEL_GEMM = 2,    /* the 4-bit (8-bit) GEMM with its fused epilogue */
  SVDQ_KERNEL_OTHER = 3,   /* separate low-rank pass, chained T finalisation */
  SVDQ_KERNEL_RANGE_MIN_ = -2147483647 - 1,   /* range markers, as for svdq_format */
  SVDQ_KERNEL_RANGE_MAX_ = 2147483647
} svdq_kernel_kind;

/* Kernel durations taken from the kernels' own dispatch timestamps.
 * svdq_timing_start(capacity): from this call on, the first `capacity`
 * kernel launches that the calling host thread makes through this library
 * (svdq_linear_forward, svdq_quantize_activations, svdq_gemm_forward, the
 * chained forward; absmax and test hooks excepted) are made with
 * hipExtLaunchKernel and an event pair of their own, which brackets that
 * kernel alone -- nothing is inserted in the stream between kernels.
 * Later launches run untimed.  1 <= capacity <= 2^20; the events are
 * created here (the call allocates; a second start replaces the first).
 * svdq_timing_stop(kinds, ms, max_launches, n_launches): ends recording,
 * waits for the recorded kernels, and writes for the first
 * min(*n_launches, max_launches) recorded launches, in launch order, their
 * svdq_kernel_kind and duration in milliseconds; *n_launches = the number
 * recorded.  Both act on the calling thread only; stop without start
 * reports zero launches.  The events belong to the device current at
 * svdq_timing_start: time launches on that device only. */
svdq_status svdq_timing_start(int capacity);
svdq_status svdq_timing_stop(int* kinds, float* ms, int max_launches, int* n_launches);

#ifdef __cplusplus
}
#endif
#endif /* SVDQ_H */
