/*
 * fp4attn.h -- C ABI of the MI355X (gfx950) FP4 attention library.
 *
 * Method: "Hardware-Aware FP4 FlashAttention-4" (arXiv:2609.04105), as described by the
 * gist.science technical summary of the paper (Methodology 1 "Direct-P for Forward
 * Inference", Methodology 2 "Quantized Causal Backward") and by its arXiv abstract.
 *
 * Conventions shared by every entry point
 *  - Every tensor pointer is a DEVICE pointer (HBM of the current HIP device). The caller
 *    owns every buffer, including the quantized operands, LSE and the workspace; the
 *    library never allocates, frees, prints, or keeps mutable global state, except for the
 *    static scratch array of fp4attn_bwd_noalloc (see there).
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL is the null stream) and
 *    returns after enqueueing. Argument errors are detected on the host, before anything
 *    is enqueued, and returned as a status; launch failures return FP4ATTN_ERR_LAUNCH.
 *    Device faults surface at the caller's next synchronization on the stream.
 *  - Shapes: bf16 activations are [B, heads, N, D] row-major (D contiguous). Query heads
 *    number H, key/value heads Hkv (H % Hkv == 0; query head h reads KV head
 *    h / (H / Hkv)). Supported: D in {64, 128}; N % 32 == 0 (N == 0 or B == 0 enqueue
 *    nothing and return FP4ATTN_OK); B * heads * N * D < 2^31 elements per tensor.
 *    Every pointer must be 16-byte aligned.
 *  - The softmax scale is 1/sqrt(D). LSE is the natural-log log-sum-exp of the scaled
 *    scores, fp32 [B, H, N].
 *  - Non-finite inputs violate a precondition: outputs are then undefined and no status
 *    reports it.
 *  - Calls on different streams may run concurrently; the library is thread-safe.
 */
#ifndef FP4ATTN_H_
#define FP4ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FP4ATTN_OK = 0,
  FP4ATTN_ERR_NULL = 1,        /* a required pointer is NULL */
  FP4ATTN_ERR_SHAPE = 2,       /* negative sizes, H % Hkv != 0, N % 32 != 0, too large */
  FP4ATTN_ERR_UNSUPPORTED = 3, /* D not in {64, 128}, or a mode this build does not have */
  FP4ATTN_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
  FP4ATTN_ERR_FORMAT = 5,      /* an operand's format or blocking axis is not the one required */
  FP4ATTN_ERR_LAUNCH = 6,      /* the HIP runtime refused a launch */
  FP4ATTN_ERR_SCRATCH = 7      /* the sizes need more than fp4attn_bwd_noalloc's static scratch */
} fp4attn_status;

/* Element formats of an MX tensor (OCP Microscaling v1.0): 32 consecutive elements along
 * the blocking axis share one E8M0 scale byte (value 2^(byte - 127)). */
enum {
  FP4ATTN_MXFP4 = 1, /* E2M1 elements, two per byte: lower index in the low nibble */
  FP4ATTN_MXFP8 = 2  /* E4M3 (OCP "FN") elements, one per byte */
};

/* Blocking axis of an MX tensor, and with it the physical layout:
 *  ALONG_D:   codes [B, heads, N, D * bits / 8]   (row-major, element (n, d) in row n)
 *             scales [B, heads, N, D / 32]
 *  ALONG_SEQ: codes [B, heads, D, N * bits / 8]   (transposed: the sequence is contiguous)
 *             scales [B, heads, D, N / 32]
 * with bits = 4 for MXFP4 and 8 for MXFP8. */
enum { FP4ATTN_ALONG_D = 0, FP4ATTN_ALONG_SEQ = 1 };

/* A view of one MX-quantized [B, heads, N, D] tensor. */
typedef struct {
  int32_t fmt;     /* FP4ATTN_MXFP4 or FP4ATTN_MXFP8 */
  int32_t axis;    /* FP4ATTN_ALONG_D or FP4ATTN_ALONG_SEQ */
  void* codes;     /* device pointer, layout above */
  uint8_t* scales; /* device pointer, layout above */
} fp4attn_mx;

/* Bytes of the codes / scales arrays of an MX tensor of shape [B, heads, N, D]. */
size_t fp4attn_mx_codes_bytes(int fmt, int64_t B, int64_t heads, int64_t N, int64_t D);
size_t fp4attn_mx_scales_bytes(int64_t B, int64_t heads, int64_t N, int64_t D);

/* MX quantization of a bf16 tensor x [B, heads, N, D] into `out` (its fmt and axis chosen
 * by the caller). Scale of each 32-element block: floor(log2(amax)) - emax (emax 2 for
 * E2M1, 8 for E4M3), clamped to [-127, 127] (an all-zero block gets -127); elements are
 * x / 2^scale rounded to nearest even on the element grid, saturating at the largest
 * magnitude, keeping the sign (negative values that round to zero give -0).
 * Source: summary, Methodology 1 "Format Selection" (MXFP4 with power-of-two block scales
 * for P and V), Methodology 2 "Reconstruction" and "Gradient Formats" (the saved quantized
 * Q/K payload and scales; the row/column-oriented FP8 views of Q, K, V); the pages put this
 * step in the projection epilogues, this library runs it as its own HBM-streaming kernel.
 * Errors: NULL, SHAPE, UNSUPPORTED, ALIGN, FORMAT (unknown fmt/axis), LAUNCH. */
int fp4attn_quantize_mx(const void* x_bf16, const fp4attn_mx* out, int64_t B, int64_t heads, int64_t N, int64_t D,
                        void* stream);

/* Several MX quantizations in one launch, for callers that quantize a group of tensors
 * together (the forward's Q and K along D and V along the sequence). Job i quantizes the bf16
 * tensor jobs[i].x_bf16 [B, jobs[i].heads, N, D] into jobs[i].out by the rule of
 * fp4attn_quantize_mx; the results are identical to count separate fp4attn_quantize_mx calls.
 * All jobs share B, N and D; 1 <= count <= FP4ATTN_MAX_QUANT_JOBS. Outputs must not overlap
 * each other or any input. The caller owns `jobs`, which is read before the call returns.
 * Errors: NULL (jobs, or a pointer of a job), SHAPE (count out of range, or sizes), UNSUPPORTED,
 * ALIGN, FORMAT, LAUNCH. */
#define FP4ATTN_MAX_QUANT_JOBS 4
typedef struct {
  const void* x_bf16; /* device pointer, bf16 [B, heads, N, D] */
  int64_t heads;
  fp4attn_mx out;     /* format and blocking axis chosen by the caller */
} fp4attn_quant_job;
int fp4attn_quantize_mx_batch(const fp4attn_quant_job* jobs, int count, int64_t B, int64_t N, int64_t D,
                              void* stream);

/* NVFP4-style block quantization of a bf16 tensor x [B, heads, N, D] along D, for Q and K.
 * Source: summary, Methodology 1 "Format Selection" (the pages quantize Q and K to NVFP4: E2M1
 * elements with finer block scales than MXFP4). Reading: blocks of 16 consecutive elements along D;
 * scale s = RNE_E4M3(amax / 6 / 2^tensor_exp), saturating at 448 (zero when it rounds to zero);
 * element code = RNE_E2M1(x / (s 2^tensor_exp)), saturating, sign kept (magnitude 0 for every
 * element of a block with s = 0); the per-tensor scale is the power of two 2^tensor_exp chosen by
 * the caller (0 suits unit-scale data; the block scales then cover block maxima from about 0.003 to
 * 2688).
 * Outputs (all caller-owned device buffers, 16-byte aligned):
 *  codes: [B, heads, N, D/2] bytes, two E2M1 codes per byte, the lower index in the low nibble;
 *  scales: [B, heads, N, D/16] E4M3 bytes;
 *  xhat_bf16: [B, heads, N, D] bf16, the represented values E2M1(code) s 2^tensor_exp, which are
 *    exact in bf16 (at most 6 significant bits): the operands of fp4attn_fwd_nvfp4.
 * Constraints: D in {64, 128}; N a multiple of 32; -100 <= tensor_exp <= 100.
 * Errors: NULL, SHAPE (sizes, tensor_exp), UNSUPPORTED (D), ALIGN, LAUNCH. */
int fp4attn_quantize_nvfp4(const void* x_bf16, void* codes, void* scales, void* xhat_bf16, int tensor_exp,
                           int64_t B, int64_t heads, int64_t N, int64_t D, void* stream);

/* Direct-P forward (noncausal) with NVFP4-style Q and K. q_hat [B, H, N, D] and k_hat [B, Hkv, N, D]
 * are bf16 tensors, normally the xhat outputs of fp4attn_quantize_nvfp4 for Q and K; v is MXFP4
 * ALONG_SEQ. S = q_hat k_hat^T on the BF16 MFMA with fp32 accumulation (gfx950's block-scaled MFMA
 * takes E8M0 scales per 32 elements, not E4M3 scales per 16); P and P.V as the integer-log2-anchor
 * reading of fp4attn_fwd_ex with FP4ATTN_FWD_ANCHORED (summary, Methodology 1 "Direct Mapping",
 * "Consistent Normalization", "Range Guarding"). start_event and stop_event: as in fp4attn_fwd_ex.
 * Outputs: o_bf16 [B, H, N, D], lse [B, H, N].
 * Errors: NULL, SHAPE, UNSUPPORTED, ALIGN, FORMAT (v not MXFP4 ALONG_SEQ), LAUNCH. */
int fp4attn_fwd_nvfp4(const void* q_hat_bf16, const void* k_hat_bf16, const fp4attn_mx* v, void* o_bf16, float* lse,
                      int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t D, void* stream, void* start_event,
                      void* stop_event);

/* The attention block's QKV projection with the MX quantization in its epilogue: computes
 * Q = X Wq^T, K = X Wk^T, V = X Wv^T with bf16 operands and fp32 accumulation, and writes them
 * straight from the fp32 sums as the quantized tensors the attention calls take (no bf16 copy of
 * Q, K, V is formed; the rule of fp4attn_quantize_mx applied to the fp32 values).
 * Source: summary, Methodology 2 "Gradient Formats" (the projection epilogues publish the
 * quantized operands and the row/column-oriented FP8 views) and Results "Training Performance".
 *  x_bf16: [B, N, Dm] bf16, row-major. w_bf16: [(H + 2 Hkv) D, Dm] bf16, row-major, the weight of
 *    one linear layer (output features by input features): the rows of Wq (H heads of D rows),
 *    then of Wk (Hkv heads), then of Wv (Hkv heads).
 *  q, k: MXFP4 ALONG_D views of [B, H, N, D] and [B, Hkv, N, D]. v: ALONG_SEQ of [B, Hkv, N, D],
 *    MXFP4 (Direct-P) or MXFP8 (the FP8 routes).
 *  q8, k8, v8: all NULL, or the backward's views: q8, k8 MXFP8 ALONG_SEQ, v8 MXFP8 ALONG_D.
 * Constraints: D in {64, 128}; N a positive multiple of 32; Dm a positive multiple of 64, at most
 * 65536; H a multiple of Hkv; x, w and every codes and scales buffer 16-byte aligned; outputs
 * must not overlap each other or the inputs.
 * Errors: NULL, SHAPE, UNSUPPORTED, ALIGN, FORMAT (a view of the wrong format or axis, or some but
 * not all of q8, k8, v8), LAUNCH. */
int fp4attn_project_qkv(const void* x_bf16, const void* w_bf16, const fp4attn_mx* q, const fp4attn_mx* k,
                        const fp4attn_mx* v, const fp4attn_mx* q8, const fp4attn_mx* k8, const fp4attn_mx* v8,
                        int64_t B, int64_t N, int64_t Dm, int64_t H, int64_t Hkv, int64_t D, void* stream);

/* fp4attn_project_qkv with the workgroup tile chosen by the caller. tile: 0 chooses by the launch's
 * size (what fp4attn_project_qkv does), 128 takes tiles of 256 tokens x 128 features, 256 tiles of
 * 256 tokens x 256 features (fewer LDS reads per MFMA, half as many workgroups). Every tile gives
 * bit-identical outputs: each fp32 sum takes the same MFMA steps in the same order.
 * Errors: those of fp4attn_project_qkv; UNSUPPORTED also for any other tile. */
int fp4attn_project_qkv_ex(const void* x_bf16, const void* w_bf16, const fp4attn_mx* q, const fp4attn_mx* k,
                           const fp4attn_mx* v, const fp4attn_mx* q8, const fp4attn_mx* k8, const fp4attn_mx* v8,
                           int64_t B, int64_t N, int64_t Dm, int64_t H, int64_t Hkv, int64_t D, int tile,
                           void* stream);

/* Forward attention with 4-bit operands. q, k are MXFP4 ALONG_D; the route follows causal and
 * v's format:
 *  causal == 0, v MXFP4 ALONG_SEQ (Direct-P, the inference route; summary, Methodology 1
 *    "Direct Mapping" and "Consistent Normalization"; arXiv abstract): S = Q K^T on
 *    block-scaled MFMA; per 32-key block the scores are mapped straight to E2M1 probability
 *    codes with a shared E8M0 scale; the normalizer accumulates the same represented values
 *    that the P.V product consumes.
 *  causal == 0, v MXFP8 ALONG_SEQ (the FP8 P/V route the pages compare Direct-P with; summary,
 *    Results "Accuracy"): P is formed in E4M3 with one E8M0 scale per 32 keys, no mask.
 *  causal == 1, v MXFP8 ALONG_SEQ (the training route; summary, Methodology 2 "Stability
 *    Constraint"): as the FP8 route with key j visible to query i iff j <= i; q, k are the
 *    state saved for fp4attn_bwd.
 * Keys are consumed in blocks of fp4attn_key_block(D, causal) keys, in increasing order,
 * with the running max updated once per key block.
 * Outputs: o_bf16 [B, H, N, D] (bf16), lse [B, H, N] (fp32).
 * Errors: NULL, SHAPE, UNSUPPORTED, ALIGN, FORMAT (wrong fmt/axis for the route), LAUNCH. */
int fp4attn_fwd(const fp4attn_mx* q, const fp4attn_mx* k, const fp4attn_mx* v, void* o_bf16, float* lse, int64_t B,
                int64_t H, int64_t Hkv, int64_t N, int64_t D, int causal, void* stream);

/* fp4attn_fwd with options: `flags` selects a variant of the route, and two optional HIP events
 * time the attention kernel.
 *  FP4ATTN_FWD_ANCHORED (noncausal Direct-P only; summary, Methodology 1 "Direct Mapping" and
 *    "Range Guarding"): the integer-log2 anchor. Each 32-key block's codes are those of
 *    2^(S c - t_b + 2), t_b = floor(fp32(S_bmax c)), one fused multiply-add, and P = E2M1 code *
 *    2^(t_b - 2): the MX quantization of the unnormalized exponentials 2^(S c). There is no
 *    running max: the kernel keeps O and l relative to a per-query integer anchor taken from the
 *    first key block (a sample of the scores) and moves it, by an exact power-of-two rescale, only
 *    when a later block exceeds it by more than 64 binades (the range guard). LSE = ln sum P.
 *    Blocks more than 125 binades below the anchor (below 2^-120 of the normalizer) are dropped.
 *  Events: start_event and stop_event (hipEvent_t, created by the caller on the current device,
 *    timing enabled; both NULL for none) are bound to the attention kernel's own dispatch
 *    (hipExtLaunchKernel), so hipEventElapsedTime gives the kernel's duration on `stream`. The
 *    runtime records the start event as a marker before the kernel, which lengthens the stream's
 *    work by a few microseconds. The events are recorded only when the call returns FP4ATTN_OK.
 * Errors: those of fp4attn_fwd; UNSUPPORTED for unknown flags or FP4ATTN_FWD_ANCHORED with causal
 * or an MXFP8 V; NULL when exactly one event is NULL. */
#define FP4ATTN_FWD_ANCHORED 1u
int fp4attn_fwd_ex(const fp4attn_mx* q, const fp4attn_mx* k, const fp4attn_mx* v, void* o_bf16, float* lse,
                   int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t D, int causal, unsigned flags, void* stream,
                   void* start_event, void* stop_event);

/* The same forward loop with bf16 operands on the bf16 MFMA: P = 2^((S - m) * c) in fp32,
 * rounded to bf16 for the P.V product, normalizer from the unrounded P. It exists to form
 * the FP4/BF16 throughput ratio the pages report against a BF16 FlashAttention baseline
 * (summary, Key Contributions and Results "Throughput").
 * Inputs (device, bf16, 16-byte aligned, caller-owned, only read): q [B, H, N, D], k [B, Hkv, N, D],
 * and V transposed, vt [B, Hkv, D, N] (the sequence contiguous, as the FP4 routes' V along the
 * sequence); key j visible to query i iff causal == 0 or j <= i.
 * Outputs as fp4attn_fwd. Constraints as fp4attn_fwd: D in {64, 128}; N a multiple of 32.
 * Errors: NULL, SHAPE, UNSUPPORTED (D, causal not 0/1), ALIGN, LAUNCH. */
int fp4attn_fwd_bf16(const void* q_bf16, const void* k_bf16, const void* vt_bf16, void* o_bf16, float* lse, int64_t B,
                     int64_t H, int64_t Hkv, int64_t N, int64_t D, int causal, void* stream);

/* Workspace bytes fp4attn_bwd needs for these sizes (device memory, caller-owned, no
 * initialization required, not retained between calls): Delta (fp32 [B, H, N]) and dO's
 * MXFP8 views along D and along the queries. Returns 0 for invalid sizes. */
size_t fp4attn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t D);

/* Backward of the causal route (summary, Methodology 2 "Reconstruction" and "Gradient
 * Formats"; arXiv abstract): P is rebuilt from the saved MXFP4 q, k and the forward's LSE,
 * P = 2^(S * c - LSE * log2(e)), with no separate score path; the four gradient products run
 * on MXFP8 operands:
 *   dP = dO . V^T     dO, V blocked along D     (v8: MXFP8 ALONG_D)
 *   dS = P (dP - Delta),  Delta_i = sum_d dO_id O_id
 *   dV = P^T . dO     P, dO blocked along queries
 *   dQ = scale dS . K     dS, K blocked along keys    (k8: MXFP8 ALONG_SEQ)
 *   dK = scale dS^T . Q   dS, Q blocked along queries (q8: MXFP8 ALONG_SEQ)
 * dO's two MXFP8 views and P's and dS's are formed inside. dK and dV of a KV head sum over
 * its H / Hkv query heads.
 * Inputs: q, k (MXFP4 ALONG_D, as given to the forward), q8, k8, v8 (views above), o_bf16
 * and lse (the forward's outputs), do_bf16 [B, H, N, D]. Outputs: dq [B, H, N, D],
 * dk, dv [B, Hkv, N, D], bf16. workspace: fp4attn_bwd_workspace_bytes bytes.
 * causal: 1 applies the mask key <= query; 0 uses every key (the same gradient formats).
 * Kernels, in stream order: Delta and dO's two MXFP8 views into the workspace, then dK/dV
 * (one workgroup per 128 keys of a KV head), then dQ (one workgroup per 128 queries).
 * Errors: NULL, SHAPE, UNSUPPORTED, ALIGN, FORMAT, LAUNCH. */
int fp4attn_bwd(const fp4attn_mx* q, const fp4attn_mx* k, const fp4attn_mx* q8, const fp4attn_mx* k8,
                const fp4attn_mx* v8, const void* o_bf16, const void* do_bf16, const float* lse, void* dq_bf16,
                void* dk_bf16, void* dv_bf16, void* workspace, int64_t B, int64_t H, int64_t Hkv, int64_t N,
                int64_t D, int causal, void* stream);

/* fp4attn_bwd for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): the same computation and kernels, with
 * the workspace taken from a static device array of FP4ATTN_NOALLOC_SCRATCH_BYTES (72 MiB) that
 * every device the library runs on holds until the process ends. The call allocates and frees
 * nothing; the caller still passes every input and output. The workspace needs no initial
 * contents, so nothing is cleared between calls.
 * Calls on one device share its scratch array: calls that overlap on one device (concurrent
 * streams, or threads) race and give undefined results; serialize them.
 * Limit: fp4attn_bwd_workspace_bytes(B, H, Hkv, N, D) <= FP4ATTN_NOALLOC_SCRATCH_BYTES, which holds
 * B * H * N <= 262144 rows at D = 128 (the 8B training shape B1 H32 N8192) and more at D = 64.
 * Errors: those of fp4attn_bwd; SCRATCH when the sizes need more scratch (nothing is enqueued);
 * LAUNCH also when the scratch array's device address cannot be obtained. */
#define FP4ATTN_NOALLOC_SCRATCH_BYTES (72u << 20)
int fp4attn_bwd_noalloc(const fp4attn_mx* q, const fp4attn_mx* k, const fp4attn_mx* q8, const fp4attn_mx* k8,
                        const fp4attn_mx* v8, const void* o_bf16, const void* do_bf16, const float* lse,
                        void* dq_bf16, void* dk_bf16, void* dv_bf16, int64_t B, int64_t H, int64_t Hkv, int64_t N,
                        int64_t D, int causal, void* stream);

/* Keys per running-max update used by fp4attn_fwd for this head size and route: the
 * key-block parameter of the method's online softmax: 128 for D = 128 and 64 for D = 64, on both
 * routes. Returns 0 for unsupported D. */
int fp4attn_key_block(int64_t D, int causal);

/* Static, NUL-terminated description of a status code. */
const char* fp4attn_status_str(int status);

/* Measurement: the shader clock under load, for the fraction of peak at the clock the GPU runs
 * (the MI355X's published MFMA peaks assume 2.4 GHz). Runs nblocks workgroups of four waves, two
 * workgroups per CU, each wave `iters` iterations of one FP4 MFMA and sixteen VALU instructions
 * (fused multiply-adds and exponentials, about the proportion of the Direct-P forward's block
 * loop), and writes per workgroup the shader cycles (s_memtime) and real-time counter ticks
 * (s_memrealtime) its loop took; the clock is cycles / ticks x *realtime_khz.
 * Arguments: counts -- device, 2 * nblocks uint64 (cycles, ticks per workgroup), written;
 * nblocks in [1, 4096] (512 fills the MI355X); iters in [1, 2^24]; realtime_khz -- host, receives
 * the real-time counter's rate in kHz; stream -- hipStream_t or NULL.
 * Errors: NULL, SHAPE (nblocks or iters out of range), LAUNCH. */
int fp4attn_clock_probe(uint64_t* counts, int nblocks, int iters, int* realtime_khz, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP4ATTN_H_ */
