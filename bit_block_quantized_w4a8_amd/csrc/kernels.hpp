// Launchers of the W4A8 kernels (host side, C++ linkage, library-internal).
#pragma once

#include "common.hpp"

namespace w4a8 {

int launch_pack(const int8_t* q, const uint16_t* s, int K, int N, uint8_t* packed,
                uint16_t* w_scales, hipStream_t stream);

int launch_quantize_export(const uint16_t* x, int M, int K, int8_t* qx, float* sx,
                           hipStream_t stream);

int launch_quantize_stage(const uint16_t* x, int M, int M_pad, int K, uint8_t* qxs, float* sxs,
                          hipStream_t stream);

// Decode GEMV (int8 dot products, activations quantised in the kernel).
enum GemvMode {
  kGemvOut = 0,     // out[m][n] = y (fp32)
  kGemvSums = 1,    // integer block sums
  kGemvArgmax = 2,  // fused argmax over the row (+ optional logits)
  kGemvCast = 3,    // out (nullable) and y16[m][n] = fp16(y) for n < n16
  kGemvResid = 4,   // resid[m][n] = fma(alpha, y, resid[m][n])
  kGemvGated = 5,   // y16[m][f] = fp16(y[f] * y[N/2 + f]) for f < N/2
};
struct GemvArgs {
  const uint16_t* x;     // fp16 [M][K]; unused when xf is set
  const uint8_t* packed_w;
  const uint16_t* w_scales;
  int M, K, N;
  float* out;            // kGemvOut, kGemvCast (nullable)
  int32_t* sums;         // kGemvSums
  float* logits;         // kGemvArgmax, may be null
  int32_t* argmax;       // kGemvArgmax
  // Decoder-layer fusion (one token row):
  const float* xf = nullptr;  // fp32 [M][K] residual stream, normalised in the prologue:
                              // x_in = fp16(xf / sqrt(mean(xf^2) + eps))
  float eps = 0.0f;
  float* resid = nullptr;     // kGemvResid
  float alpha = 0.0f;
  uint16_t* y16 = nullptr;    // kGemvCast: [M][n16]; kGemvGated: [M][N/2]
  int n16 = 0;
};
int launch_gemv(const GemvArgs& a, int mode, Scratch* sc, hipStream_t stream);
// Whether a fused (one-row) GEMV launch supports the shape: the normalising
// prologue needs the whole row of K in one chunk.
bool gemv_fused_supported(int mode, bool norm, int K, int N);
size_t gemv_scratch_bytes(int M, int K, int N);

// Prefill GEMM (int8 MFMA on pre-quantised activations).
// mode: 0 = scaled output, 1 = integer block sums.
struct GemmArgs {
  const uint16_t* x;
  const uint8_t* packed_w;
  const uint16_t* w_scales;
  int M, K, N;
  float* out;            // mode 0
  int32_t* sums;         // mode 1
  float* resid = nullptr;  // residual epilogue: resid[m][n] = fma(alpha, y[m][n], resid[m][n])
  float alpha = 0.0f;
  uint8_t* q_out = nullptr;  // gated epilogue: staging of the next GEMM (codes, scales, rows)
  float* s_out = nullptr;
  int m_pad_out = 0;
  int n_cast = 0;  // cast epilogue: leading columns quantised into the staging
};
int launch_gemm(const GemmArgs& a, int mode, Scratch* sc, hipStream_t stream);
size_t gemm_scratch_bytes(int M, int K, int N);
// Staging of one GEMM launch in library scratch (the pre-pass's output):
// codes and scales of M_pad rows (rows M .. M_pad-1 zero) for an M x K by K x N
// product.  gemm_staging checks that sc holds it (with room for split-K
// partials after it).
struct GemmStaging {
  uint8_t* qxs;
  float* sxs;
  int m_pad;
};
int gemm_staging(int M, int K, int N, Scratch* sc, GemmStaging* s);
// The GEMM (scaled output) on activations already quantised into `s`.
int launch_gemm_staged(const GemmArgs& a, const GemmStaging& s, Scratch* sc, hipStream_t stream);
// The same, adding alpha times the result into a.resid (fp32 [M][N]) instead
// of writing a.out: one fma per element, as a separate residual add would.
int launch_gemm_staged_resid(const GemmArgs& a, const GemmStaging& s, Scratch* sc, hipStream_t stream);
// Staging in caller memory (gemm_staging_bytes(M, K, N) bytes, 256-byte
// aligned) for a GEMM of that shape.
size_t gemm_staging_bytes(int M, int K, int N);
GemmStaging gemm_staging_at(void* base, int M, int K, int N);
// A gate/up GEMM (columns [gate F | up F], N = 2F) whose epilogue forms
// fp16(gate * up) and quantises it into `out`, the staging of a GEMM with
// K = F, instead of writing a.out; the codes and scales equal those that the
// gated glue kernel and the activation pre-pass write.  Only for shapes that
// run 128 x 128 tiles without a K split, and a staging of at most as many
// rows as the tiles cover.
bool gemm_gated_supported(int M, int K, int N, int m_pad_out);
// A GEMM whose epilogue quantises fp16(y) of its leading n_cast columns
// (a multiple of 32) into `out`, the staging of a GEMM with K = n_cast, and
// writes the other columns to a.out; the codes and scales equal those that
// the cast glue kernel writes.  `out` holds at least M and at most the
// GEMM's tile rows (its m_pad).
bool gemm_cast_supported(int M, int K, int N, int n_cast, int m_pad_out);
int launch_gemm_staged_cast(const GemmArgs& a, int n_cast, const GemmStaging& s, const GemmStaging& out,
                            Scratch* sc, hipStream_t stream);
int launch_gemm_staged_gated(const GemmArgs& a, const GemmStaging& s, const GemmStaging& out, Scratch* sc,
                             hipStream_t stream);

// MX variant (mx.hip): MXFP4 weights x MXFP8 activations on the block-scaled
// matrix instruction.
int mx_m_pad(int M);
size_t mx_scratch_bytes(int M, int K);
int launch_mx_quantize_act(const uint16_t* x, int M, int M_pad, int K, uint8_t* codes, uint8_t* scales,
                           hipStream_t stream);
int launch_mx_pack(const uint16_t* w, int K, int N, uint8_t* packed, uint8_t* scales, hipStream_t stream);
int launch_mx_linear(const uint16_t* x, const uint8_t* packed, const uint8_t* wscales, int M, int K, int N,
                     float* out, Scratch* sc, hipStream_t stream);

// Decode attention over an fp16 KV cache (attention.hip).
int attention_chunks(int length);
size_t attention_scratch_bytes(int n_kv_heads, int group, int head_dim, int length);
// The library's exchange area of the flagged-word merge (device memory,
// zeroed once): for each of `heads` KV heads a fixed region of
// kAttnHeadWords 64-bit words of partials and an epoch word, and the device
// error word.  A KV head's words always sit in its own region, whatever the
// call's shape, so every word only ever carries flags of that head's epoch,
// which rises with every call: a word left by an earlier call never shows the
// current flag.
struct AttnExchange {
  uint64_t* ll = nullptr;
  uint32_t* epochs = nullptr;
  int heads = 0;
  uint32_t* error = nullptr;
};
constexpr int kAttnHeads = 16;                     // KV heads the flagged-word merge serves
constexpr size_t kAttnHeadWords = 32 * 8 * 258;     // 32 chunks x 8 query heads x (256 dims + 2)
// Whether a call of this shape merges through the exchange area.
bool attention_ll_fits(int n_kv_heads, int group, int head_dim, int length, const AttnExchange* ex);
int launch_decode_attention(const float* q, const float* k_new, const float* v_new, uint16_t* k_cache,
                            uint16_t* v_cache, int n_heads, int n_kv_heads, int head_dim, int length, int capacity,
                            uint16_t* out, Scratch* sc, const AttnExchange* ex, hipStream_t stream);

// Small-batch decode kernel (skinny.hip): M = 1 .. 16 rows on the int8 matrix
// instruction, every weight read once; K a multiple of 256, N of 64.  `sums`
// (int32 [M][N][K/32]) selects the block-sum export instead of `out`.
bool skinny_supported(int M, int K, int N);
int launch_skinny(const uint16_t* x, const uint8_t* packed_w, const uint16_t* w_scales, int M, int K, int N,
                  float* out, int32_t* sums, hipStream_t stream);

int gemv_max_m();
// Kernel W4A8_PATH_AUTO picks for an M x K by K x N linear.
int auto_path(int64_t M, int64_t K, int64_t N);

// Glue of the synthetic decoder layer (layer.hip).
int launch_residual_norm_cast(float* x, const float* d, int64_t ld_d, float alpha, float eps, int M, int H,
                              uint16_t* y, hipStream_t stream);
int launch_cast_rows(const float* src, int64_t ld, int M, int H, uint16_t* dst, hipStream_t stream);
// The same glue with the fp16 result quantised straight into GEMM staging.
int launch_residual_norm_quant(float* x, const float* d, int64_t ld_d, float alpha, float eps, int M, int H,
                               const GemmStaging& s, hipStream_t stream);
int launch_cast_quant(const float* src, int64_t ld, int M, int H, const GemmStaging& s, hipStream_t stream);
int launch_gated_quant(const float* g, int M, int F, const GemmStaging& s, hipStream_t stream);
int launch_gated_cast(const float* g, int M, int F, uint16_t* u, hipStream_t stream);

// Byte offsets of a decoder layer's temporaries inside the caller's workspace.
struct LayerWorkspace {
  size_t q, a, o, n, g, u, d, bytes;
};
LayerWorkspace layer_workspace(int M, int H, int n_qkv, int n_gu);

}  // namespace w4a8
