/*
 * w4a8.h -- C ABI of the W4A8 block-32 linear layer for AMD Instinct MI355X (gfx950).
 *
 * The operation (ML Drift pages: explainer on tech.dede.sh, section
 * "Stage-aware optimization for large language models"; x-techcon article,
 * section on moving less data for large models): an LLM linear layer whose
 * weights are 4-bit in blocks of 32 and whose activations the kernel
 * quantises itself, with one kernel for the decode stage (few tokens,
 * memory-bound) and another for the prefill stage (hundreds of tokens,
 * compute-bound).  The numeric scheme pinned by this library:
 *
 *   weights      qw in [-8, 7] (int4, symmetric), one fp16 scale sw[n][b] per
 *                output column n and block b of 32 consecutive inputs;
 *   activations  per token row m and block b: sx[m][b] = fp32(max|x| / 127),
 *                qx = clamp(round_half_even(fp32(x / sx)), -127, 127);
 *                an all-zero block gives sx = 0, qx = 0;
 *   output       out[m][n] = sum_b sx[m][b] * sw[n][b] * I[m][n][b],
 *                I[m][n][b] = sum_{j<32} qx[m][32b+j] * qw[n][32b+j]  (exact int32).
 *
 * Conventions for every entry point:
 *   - tensor pointers are HIP device pointers to row-major, contiguous data;
 *     fp16 tensors are passed as uint16_t bit patterns;
 *   - the caller owns every tensor; the library owns only its scratch memory
 *     (per device): w4a8_init reserves 64 MiB of it, and only
 *     w4a8_reserve_scratch adds more.  No other call allocates, frees or
 *     synchronises: a call that needs more scratch than is reserved fails
 *     with W4A8_EINVAL before launching anything, and the *_scratch_bytes
 *     queries below give the size each call needs;
 *   - calls are asynchronous on `stream` (0 = the null stream); none
 *     synchronises and none returns results on the host, except as noted;
 *   - calls that share a device share its scratch and its argmax slots:
 *     issue them on one stream, or serialise them yourself;
 *   - outputs must not alias inputs;
 *   - arguments are validated before any HIP call, so a rejected call has no
 *     effect; no C++ exception crosses this boundary.
 *
 * Shape limits: M >= 1, K >= 32 with K % 32 == 0, N >= 64 with N % 64 == 0,
 * all three below 2^31, and K * N / 2 bytes of packed weights below 2^40.
 * Inputs must be finite (NaN and Inf activations give unspecified results).
 */
#ifndef W4A8_H
#define W4A8_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#if defined(__GNUC__)
#define W4A8_API __attribute__((visibility("default")))
#else
#define W4A8_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes: 0 on success, negative on failure. */
#define W4A8_OK            0
#define W4A8_EINVAL       -1  /* null pointer, bad shape, misaligned pointer, bad path/option */
#define W4A8_EUNSUPPORTED -2  /* the device is not gfx950 */
#define W4A8_EHIP         -3  /* a HIP runtime call or kernel launch failed; see w4a8_last_error() */
#define W4A8_ENOINIT      -4  /* w4a8_init has not succeeded on the current device */

/* Kernel selection for w4a8_linear_path / w4a8_block_sums. */
#define W4A8_PATH_AUTO 0  /* decode GEMV, small-batch kernel or prefill MFMA GEMM by shape: w4a8_auto_path */
#define W4A8_PATH_GEMV 1  /* force the decode GEMV (any M; slow for large M) */
#define W4A8_PATH_GEMM 2  /* force the quantise pre-pass + MFMA GEMM (any M) */
#define W4A8_PATH_BATCH 3 /* force the small-batch kernel: M <= 16 rows on the int8 MFMA, every weight read
                             once, activations quantised in the kernel (K a multiple of 256) */

/*
 * Select `device`, check that it is gfx950 and allocate the library's scratch
 * (completion tickets, argmax slots, and a 64 MiB work area for
 * quantised-activation staging and split-K partials).  Idempotent per device.
 * Synchronises the device.  Returns W4A8_EUNSUPPORTED on other GPUs.
 */
W4A8_API int w4a8_init(int device);

/*
 * Make the current device's scratch work area at least `bytes` long
 * (hipMalloc; rounded up to 1 MiB).  The area it replaces is kept, never
 * freed, because a HIP graph captured while it was in use still reads and
 * writes it; so reserve the largest size once, before capturing or timing.
 * Not for use while kernels of this library run on another stream.
 * W4A8_ENOINIT before w4a8_init; W4A8_EHIP when the allocation fails.
 */
W4A8_API int w4a8_reserve_scratch(size_t bytes);

/* Bytes in the current device's scratch work area (after w4a8_init). */
W4A8_API int w4a8_scratch_capacity(size_t* bytes);

/*
 * Scratch each call needs, host-only (no device, no w4a8_init): the bytes of
 * work area that w4a8_linear_path (and w4a8_block_sums with the same path),
 * w4a8_decoder_layer, w4a8_norm_linear_argmax, w4a8_mx_linear and
 * w4a8_decode_attention need for these shapes.  Shapes are validated as the
 * calls validate them (W4A8_EINVAL).  The decode GEMV paths need 0.
 */
W4A8_API int w4a8_linear_scratch_bytes(int64_t M, int64_t K, int64_t N, int path, size_t* bytes);
struct w4a8_weights;
W4A8_API int w4a8_decoder_layer_scratch_bytes(int64_t M, int64_t H, const struct w4a8_weights* qkv,
                                              const struct w4a8_weights* gate_up, size_t* bytes);
W4A8_API int w4a8_norm_linear_argmax_scratch_bytes(int64_t M, int64_t K, int64_t N, size_t* bytes);
W4A8_API int w4a8_mx_linear_scratch_bytes(int64_t M, int64_t K, int64_t N, size_t* bytes);
W4A8_API int w4a8_decode_attention_scratch_bytes(int64_t n_heads, int64_t n_kv_heads, int64_t head_dim,
                                                 int64_t length, size_t* bytes);

/*
 * Pack int4 weights into the K-block-major layout read by every kernel
 * (the pages fix 4-bit weights in blocks of 32; the layout is this library's).
 *   q         int8  [N][K], values in [-8, 7] (out-of-range values are masked to 4 bits)
 *   s         fp16  [N][K/32] weight scales
 *   packed_w  uint8 [K/32][N][16], 16-byte aligned: byte j of (block b, column n)
 *             = (q[n][32b+j] & 0xF) | (q[n][32b+16+j] & 0xF) << 4
 *   w_scales  fp16  [K/32][N]: w_scales[b][n] = s[n][b]
 */
W4A8_API int w4a8_pack_weights(const int8_t* q, const uint16_t* s, int64_t K, int64_t N,
                      uint8_t* packed_w, uint16_t* w_scales, hipStream_t stream);

/*
 * out = W4A8 linear of x (see the header comment), fp32 [M][N], 16-byte aligned.
 *   x         fp16 [M][K], 16-byte aligned
 *   packed_w, w_scales as produced by w4a8_pack_weights, both 16-byte aligned
 * Stage choice (w4a8_auto_path): few rows run the decode GEMV, which quantises
 * the activations inside the kernel; up to 16 rows the small-batch kernel,
 * which also quantises in the kernel and forms the block sums on the int8
 * matrix instruction; more rows run a quantise pre-pass into library scratch
 * followed by the int8-MFMA prefill GEMM.
 */
W4A8_API int w4a8_linear(const uint16_t* x, const uint8_t* packed_w, const uint16_t* w_scales,
                int64_t M, int64_t K, int64_t N, float* out, hipStream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): w4a8_linear
 * with the same arguments, kernels and results, whose scratch (prefill
 * staging, split-K partials, completion tickets) is a static device array of
 * the library instead of memory the library allocates.  It allocates and
 * frees nothing; the array (32 MiB per GPU, held from the library's load to
 * the process end) is set up by w4a8_init.  A call whose scratch need
 * (w4a8_linear_scratch_bytes with W4A8_PATH_AUTO) exceeds
 * w4a8_noalloc_scratch_bytes fails with W4A8_EINVAL before launching
 * anything.  Every call on a GPU shares that GPU's array, which keeps the last
 * call's contents: calls that overlap on one GPU (other streams, other host
 * threads) race; issue them on one stream.
 */
W4A8_API int w4a8_linear_noalloc(const uint16_t* x, const uint8_t* packed_w, const uint16_t* w_scales,
                                 int64_t M, int64_t K, int64_t N, float* out, hipStream_t stream);

/* Work-area bytes of the static scratch that w4a8_linear_noalloc uses (host-only). */
W4A8_API int w4a8_noalloc_scratch_bytes(size_t* bytes);

/* w4a8_linear with an explicit kernel choice (W4A8_PATH_*), for tests and tuning. */
W4A8_API int w4a8_linear_path(const uint16_t* x, const uint8_t* packed_w, const uint16_t* w_scales,
                     int64_t M, int64_t K, int64_t N, float* out, int path,
                     hipStream_t stream);

/*
 * Linear layer followed by argmax over each output row (the pages' benchmark
 * samples with argmax).  argmax[m] = lowest n with out[m][n] maximal, -0.0 and
 * +0.0 compare equal.  `logits` (fp32 [M][N], 16-byte aligned) may be NULL, in
 * which case the logits are never written to memory.  argmax is int32 [M].
 * M must not exceed 64.  Runs the decode GEMV for any M.
 */
W4A8_API int w4a8_linear_argmax(const uint16_t* x, const uint8_t* packed_w, const uint16_t* w_scales,
                       int64_t M, int64_t K, int64_t N, float* logits, int32_t* argmax,
                       hipStream_t stream);

/*
 * Verification export: the in-kernel activation quantiser run on its own.
 *   x 16-byte aligned; qx int8 [M][K] 8-byte and sx fp32 [M][K/32] 4-byte aligned
 *   (the same device function the GEMV and the GEMM pre-pass use)
 */
W4A8_API int w4a8_quantize_act(const uint16_t* x, int64_t M, int64_t K, int8_t* qx, float* sx,
                      hipStream_t stream);

/*
 * Verification export: the unscaled integer block sums I[m][n][b] as the chosen
 * kernel forms them (same quantiser, unpacking and integer arithmetic as
 * w4a8_linear_path with that path), int32 [M][N][K/32], 16-byte aligned.
 * M must not exceed 65536.  The weight scales are not needed for this export.
 */
W4A8_API int w4a8_block_sums(const uint16_t* x, const uint8_t* packed_w, int64_t M, int64_t K,
                    int64_t N, int32_t* sums, int path, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Synthetic decoder layer around the linear (the pages' LLM benchmark runs
 * prefill 512 / decode 128 with argmax sampling and a sync every token: ML
 * Drift explainer on tech.dede.sh, section "Stage-aware optimization for large
 * language models").  Layer wiring, with x an fp32 residual stream [M][H],
 * rms(x) = sqrt(mean(x^2) + eps) per row and s the residual scale:
 *   n1 = fp16(x / rms(x)); q = L(n1; qkv); a = fp16(q[:, :H]); o = L(a; o)
 *   x += s*o; n2 = fp16(x / rms(x)); g = L(n2; gate_up)
 *   u = fp16(g[:, :F] * g[:, F:]) with F = gate_up.N / 2; d = L(u; down); x += s*d
 * Every L is w4a8_linear (decode GEMV or prefill GEMM by M).
 * ------------------------------------------------------------------------ */

/* One packed weight matrix as produced by w4a8_pack_weights (device pointers). */
struct w4a8_weights {
  const uint8_t* packed_w;   /* uint8 [K/32][N][16], 16-byte aligned */
  const uint16_t* w_scales;  /* fp16  [K/32][N], 16-byte aligned */
  int64_t K;
  int64_t N;
};
typedef struct w4a8_weights w4a8_weights;

/*
 * Per row m of x (fp32 [M][H]): if d is not NULL, x[m][h] = RN(x[m][h] + alpha *
 * d[m * ld_d + h]) (one fused multiply-add); then, if y is not NULL,
 * y[m][h] = fp16(x[m][h] * r) with r = fp32(1 / sqrt(mean_h x[m][h]^2 + eps))
 * and the sum of squares formed in fp64: the same fp16 values every
 * normalising kernel of this library forms from that row.
 * H >= 1; y fp16 [M][H].
 */
W4A8_API int w4a8_residual_norm_cast(float* x, const float* d, int64_t ld_d, float alpha, float eps,
                                     int64_t M, int64_t H, uint16_t* y, hipStream_t stream);

/* Bytes of caller-owned workspace that w4a8_decoder_layer needs for these shapes. */
W4A8_API int w4a8_decoder_layer_workspace(int64_t M, int64_t H, const w4a8_weights* qkv,
                                          const w4a8_weights* gate_up, size_t* bytes);

/*
 * Byte offsets in that workspace of the layer's intermediates, in this order:
 *   q fp32 [M][qkv.N], a fp16 [M][H], o fp32 [M][H], n fp16 [M][H],
 *   g fp32 [M][2F], u fp16 [M][F], d fp32 [M][H].
 * When every projection of the call runs the decode GEMV (M = 1 among them),
 * the call leaves q, a = fp16(q[:, :H]), o = L(a; o), g = L(n2; gate_up),
 * u and d = L(u; down) there (n only on the nine-launch path), so each
 * projection can be checked on its own inputs.  The prefill path keeps
 * quantised GEMM staging in a and g and writes none of o, n, u, d.
 */
W4A8_API int w4a8_decoder_layer_workspace_offsets(int64_t M, int64_t H, const w4a8_weights* qkv,
                                                  const w4a8_weights* gate_up, size_t offsets[7]);

/*
 * One decoder layer (wiring above), in place on x (fp32 [M][H], 16-byte aligned).
 * Shapes: qkv.K = H <= qkv.N; o.K = o.N = H; gate_up.K = H; gate_up.N = 2 * down.K;
 * down.N = H; H % 64 == 0.  workspace: device memory of at least
 * w4a8_decoder_layer_workspace bytes, 256-byte aligned, owned by the caller and
 * not touched by other calls in flight.  Allocates nothing (the linears use the
 * library scratch as w4a8_linear does: w4a8_decoder_layer_scratch_bytes), so
 * the call can be captured in a HIP graph.  M must not exceed 65536.
 * With M = 1, when the GEMV tiles of qkv and gate/up cover all of K = H in one
 * chunk (H <= 2048 for N >= 32768, H <= 4096 for N >= 16384, H <= 8192
 * otherwise), the layer runs as four GEMV launches: the normalisation sits in the prologue of qkv and
 * gate/up, the fp16 cast of q[:, :H], the residual adds and the gated product
 * in the epilogues (the pages fold such element-wise work into neighbouring
 * operators: sciencestack summary of the ML Drift paper, Figure 4).  Every
 * normalisation sums its squares in fp64, so the fused prologue and the glue
 * kernel form the same fp16 inputs and the result equals the nine-launch
 * chain; q, o, g and d are still written to the workspace.
 * When every projection runs the prefill GEMM, the layer is six launches: the
 * two normalisations quantise straight into GEMM staging; the qkv GEMM
 * quantises fp16(q[:, :H]) into the o projection's staging (its other columns
 * are written to the workspace); the o and down GEMMs add 0.01 times their
 * result into x in their epilogues; and, where the gate/up GEMM runs 128 x 128
 * tiles without a K split, it quantises fp16(gate * up) into the down
 * projection's staging (otherwise g is written and a glue kernel quantises
 * it).  Those stagings live in the workspace.  Each fused epilogue forms
 * the same fp16 values as the glue kernel it replaces and quantises them with
 * the same routine, so its codes and scales are those the glue kernel wrote.
 * With M = 1 at hidden 2048, feed-forward 8192 (gate_up.N = 16384) and
 * 2048 <= qkv.N <= 4096, on a device that holds 256 of its 768-thread
 * workgroups at once, the four projections run in ONE launch
 * (W4A8_LAYER_RESIDENT): each workgroup owns the columns the four GEMV launches
 * would give it, requests the weights of all four projections at its start,
 * and hands each projection's output to the next through flagged words in
 * the library's exchange area (the pages overlap transfers with compute:
 * aigridhq article on the WebGPU kernel studio).  The outputs and the
 * workspace values equal the four-launch layer's bit for bit.  Calls of this
 * kind on one device share the exchange area: they must not overlap (one
 * stream, or streams ordered by events).  Its waits are bounded: if the
 * workgroups cannot all be resident (another process occupying the GPU), a
 * wait gives up after about a second, the outputs are undefined and
 * w4a8_take_device_errors reports it.  W4A8_OPTION_RESIDENT_LAYER = 0 selects
 * the four launches instead.
 */
W4A8_API int w4a8_decoder_layer(float* x, int64_t M, int64_t H, const w4a8_weights* qkv,
                                const w4a8_weights* o, const w4a8_weights* gate_up,
                                const w4a8_weights* down, float residual_scale, float eps,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * n_layers decoder layers in order on x (the wiring above, layer l with the
 * weights layers[4 l .. 4 l + 3] = qkv, o, gate_up, down; a host array read
 * during the call).  Every layer must have the shapes of layer 0; each is
 * checked as by w4a8_decoder_layer before anything runs.  The result equals
 * n_layers calls of w4a8_decoder_layer bit for bit, and the workspace holds
 * the last layer's intermediates.  Where w4a8_decoder_layer would run the
 * one-launch layer (W4A8_LAYER_RESIDENT), up to 32 layers run in one launch:
 * each layer's output stream is handed to the next layer inside the launch,
 * and the next layer's qkv weights are requested while the current layer's
 * down projection waits for its input (the pages overlap transfers with
 * compute: aigridhq article on the WebGPU kernel studio; and decode a whole
 * token per step: ML Drift explainer on tech.dede.sh, section "Stage-aware
 * optimization for large language models").  Otherwise the layers run one
 * after another as w4a8_decoder_layer runs them.  Allocates nothing.
 */
W4A8_API int w4a8_decoder_stack(float* x, int64_t M, int64_t H, const w4a8_weights* layers, int64_t n_layers,
                                float residual_scale, float eps, void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/*
 * One decode token through a decoder layer with attention between the qkv
 * and o projections (the pages decode an LLM with an fp16 KV cache at context
 * 640: ML Drift explainer on tech.dede.sh, section "Stage-aware optimization
 * for large language models"):
 *   n1 = fp16(x / rms(x)); q = L(n1; qkv) (fp32, qkv.N = (n_heads + 2 n_kv_heads)
 *   head_dim values: the query heads, then one key and one value per KV head)
 *   a  = w4a8_decode_attention(queries, key, value over the caches at `length`)
 *   x += s * L(a; o); then the feed-forward half as in w4a8_decoder_layer.
 * x fp32 [1][H] with H = n_heads * head_dim; caches, limits and errors as for
 * w4a8_decode_attention (the call writes the new key and value at position
 * length - 1).  Three launches: the qkv GEMV with the normalisation in its
 * prologue, decode attention, and o, gate/up and down in one launch of
 * resident workgroups where w4a8_layer_kernel gives W4A8_LAYER_RESIDENT for
 * the shape (otherwise as three one-token GEMVs; the same values either
 * way).  The workspace (w4a8_decoder_layer_workspace for M = 1)
 * receives q, a (the attention output), o, g, u and d.  The one-token GEMV
 * launches must support the shape (as for W4A8_LAYER_GEMV4).
 */
W4A8_API int w4a8_decoder_layer_attention(float* x, int64_t H, const w4a8_weights* qkv, const w4a8_weights* o,
                                          const w4a8_weights* gate_up, const w4a8_weights* down,
                                          float residual_scale, float eps, uint16_t* k_cache, uint16_t* v_cache,
                                          int64_t n_heads, int64_t n_kv_heads, int64_t head_dim, int64_t length,
                                          int64_t capacity, void* workspace, size_t workspace_bytes,
                                          hipStream_t stream);

/* How w4a8_decoder_layer runs a layer of this shape on the current device. */
#define W4A8_LAYER_CHAIN 0     /* separate linears with glue kernels (nine launches) */
#define W4A8_LAYER_GEMM 1      /* prefill GEMMs with fused glue (six launches) */
#define W4A8_LAYER_GEMV4 2     /* one token, four fused GEMV launches */
#define W4A8_LAYER_RESIDENT 3  /* one token, one launch of resident workgroups */
W4A8_API int w4a8_layer_kernel(int64_t M, int64_t H, const w4a8_weights* qkv, const w4a8_weights* gate_up,
                               int* kernel);

/*
 * Library options (process-wide):
 *   W4A8_OPTION_RESIDENT_LAYER  1 (default): the one-token layer runs in one
 *                               launch where it can (and the attention layer's
 *                               o, gate/up and down in one); 0: as four
 *                               launches (three).
 * W4A8_EINVAL for an unknown option or value.  Not for calls in flight.
 */
#define W4A8_OPTION_RESIDENT_LAYER 1
W4A8_API int w4a8_set_option(int option, int value);
W4A8_API int w4a8_get_option(int option, int* value);

/*
 * Errors that kernels of the current device raised since the last call
 * (0: none; nonzero: a one-launch decoder layer gave up waiting for an input,
 * so that call's outputs are undefined), then cleared.  Synchronises the
 * device.
 */
W4A8_API int w4a8_take_device_errors(uint32_t* errors);

/*
 * LM-head argmax on the residual stream: argmax[m] = first index of the
 * maximum over n of w4a8_linear(fp16(x[m] / rms(x[m])))[n], with rms as in
 * w4a8_residual_norm_cast; logits (nullable) receive the fp32 row.
 *   x       fp32 [M][K], 16-byte aligned, not modified
 *   others  as w4a8_linear_argmax (M <= 64)
 * M = 1 runs one GEMV launch with the normalisation in its prologue when K
 * fits one GEMV chunk; otherwise the rows are normalised into library scratch
 * first.
 */
W4A8_API int w4a8_norm_linear_argmax(const float* x, float eps, const uint8_t* packed_w,
                                     const uint16_t* w_scales, int64_t M, int64_t K, int64_t N,
                                     float* logits, int32_t* argmax, hipStream_t stream);

/* Largest M that W4A8_PATH_AUTO sends to the decode GEMV (for any shape). */
W4A8_API int w4a8_gemv_max_m(void);

/*
 * Kernel that W4A8_PATH_AUTO runs for an M x K by K x N linear
 * (W4A8_PATH_GEMV, W4A8_PATH_BATCH or W4A8_PATH_GEMM).  The pages run one
 * kernel per inference stage (ML Drift explainer on tech.dede.sh, section
 * "Stage-aware optimization for large language models"); the row thresholds
 * are measured on MI355X: the decode GEMV for M = 1, for M = 2 too where
 * the small-batch kernel does not run, and up to M = w4a8_gemv_max_m() for
 * weight matrices of at most 2^25 values; then up to M = 16 the small-batch
 * kernel where it runs (K a multiple of 256, N of 64) and either N >= 8192 or
 * K <= 4096; the prefill GEMM otherwise.  The
 * environment variable W4A8_GEMV_MAX_M replaces the rule by the plain
 * threshold M <= W4A8_GEMV_MAX_M between GEMV and GEMM.  Host-only; no error
 * cases.
 */
W4A8_API int w4a8_auto_path(int64_t M, int64_t K, int64_t N);

/*
 * MX variant (the pages' 4-bit weights in blocks of 32 -- ML Drift explainer on
 * tech.dede.sh, section "Stage-aware optimization for large language models" --
 * in the OCP Microscaling v1.0 formats that gfx950's block-scaled matrix
 * instruction consumes).  Every block of 32 values along K shares an E8M0 scale
 * byte c (value 2^(c - 127)), c = floor(log2(max |v|)) - emax + 127 (0 for an
 * all-zero block); each value / scale is rounded to the element format, nearest
 * with ties to even, saturating at the largest normal.  Weights use FP4 E2M1
 * elements (emax 2, largest 6), activations FP8 E4M3 (emax 8, largest 448).
 * A different numeric scheme from w4a8_linear: not interchangeable with it.
 * K must be a multiple of 64, N of 64.  Errors as for w4a8_linear.
 *
 * w4a8_mx_pack_weights: w fp16 [N][K] (16-byte aligned, finite) ->
 *   packed [K/32][N][16] (byte j of (block b, column n): element 32b+2j in the
 *   low nibble, 32b+2j+1 in the high; 16-byte aligned) and
 *   scales [K/32][N] E8M0 bytes.  Both outputs are caller-owned device memory.
 */
W4A8_API int w4a8_mx_pack_weights(const uint16_t* w, int64_t K, int64_t N, uint8_t* packed,
                                  uint8_t* scales, hipStream_t stream);

/*
 * MXFP8 conversion of activations x fp16 [M][K] (16-byte aligned, finite), for
 * verification: codes [K/32][M][32] E4M3 bytes (8-byte aligned), scales
 * [K/32][M] E8M0 bytes -- the layout w4a8_mx_linear stages in library scratch.
 */
W4A8_API int w4a8_mx_quantize_act(const uint16_t* x, int64_t M, int64_t K, uint8_t* codes,
                                  uint8_t* scales, hipStream_t stream);

/*
 * out fp32 [M][N] = MXFP8(x) . MXFP4(W)^T with both block scales:
 *   out[m][n] = sum_b 2^(ca[m][b] + cw[n][b] - 254) * sum_{j<32} a[m][32b+j] w[n][32b+j],
 * accumulated in fp32 by the matrix instruction.  x fp16 [M][K]; packed and
 * scales from w4a8_mx_pack_weights.  The activations are converted into
 * library scratch first (one pre-pass launch), then one GEMM launch.
 */
W4A8_API int w4a8_mx_linear(const uint16_t* x, const uint8_t* packed, const uint8_t* scales,
                            int64_t M, int64_t K, int64_t N, float* out, hipStream_t stream);

/*
 * Decode attention of one new token over an fp16 KV cache: the step between
 * a decoder layer's QKV and O projections.  The pages decode with an fp16 KV
 * cache at context 640, kept in a layout chosen for the GPU (ML Drift
 * explainer on tech.dede.sh, section "Stage-aware optimization for large
 * language models"); the operation is scaled dot-product attention with
 * grouped query heads (query head h reads KV head h / (n_heads / n_kv_heads)):
 *
 *   K_t, V_t = cache position t for t < length - 1; position length - 1 is the
 *              new token, fp16(k_new), fp16(v_new), which this call writes into
 *              both caches before attending to it
 *   out[h]   = fp16( sum_t softmax_t(q[h] . K_t / sqrt(head_dim)) V_t ),
 *              t = 0 .. length - 1, accumulated in fp32.
 *
 * q fp32 [n_heads][head_dim]; k_new, v_new fp32 [n_kv_heads][head_dim] (a QKV
 * projection's output row, sliced, fits as is); out fp16 [n_heads][head_dim].
 * Cache storage (fp16, caller-owned, positions 0 .. length - 2 written by
 * earlier calls or by the caller):
 *   k_cache [n_kv_heads][capacity][head_dim]  one contiguous vector per position
 *   v_cache [n_kv_heads][head_dim][capacity]  one contiguous run of positions per
 *                                             dimension (the order the output
 *                                             product reads)
 * Slots past length - 1 are read but never used, whatever they hold.
 * Limits: head_dim 64, 128 or 256; 1 <= n_kv_heads <= 4096; n_heads a multiple
 * of n_kv_heads, at most 8 times it; capacity a multiple of 64 in [64, 2^24];
 * 1 <= length <= capacity; every pointer 16-byte aligned; |q|, |k_new|, |v_new|
 * within fp16 range.  Uses library scratch (about n_kv_heads * (length / 64 +
 * 32) * n_heads / n_kv_heads * (head_dim + 2) * 4 bytes).  Errors: W4A8_EINVAL for
 * arguments outside these limits, W4A8_ENOINIT, W4A8_EHIP.
 */
W4A8_API int w4a8_decode_attention(const float* q, const float* k_new, const float* v_new,
                                   uint16_t* k_cache, uint16_t* v_cache, int64_t n_heads,
                                   int64_t n_kv_heads, int64_t head_dim, int64_t length,
                                   int64_t capacity, uint16_t* out, hipStream_t stream);

/* Message of the last failure on the calling thread ("" if none). */
W4A8_API const char* w4a8_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* W4A8_H */
