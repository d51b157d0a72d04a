// Synthetic decoder layer around the W4A8 linear: glue kernels and the
// stream-ordered layer chain.
//
// The pages' LLM benchmark runs prefill 512 / decode 128 with argmax sampling
// and a sync every token (ML Drift explainer on tech.dede.sh, section
// "Stage-aware optimization for large language models"), and they fuse
// residual and element-wise work into a normalisation operator (sciencestack
// summary of the ML Drift paper, Figure 4).  The layer wiring here is this
// library's stand-in for a transformer layer without attention:
//
//   n1 = fp16(x / rms(x));  q = L(n1; Wqkv);  a = fp16(q[:, :H])
//   o  = L(a; Wo);          x = x + s*o;      n2 = fp16(x / rms(x))
//   g  = L(n2; Wgu);        u = fp16(g[:, :F] * g[:, F:])
//   d  = L(u; Wdown);       x = x + s*d
//
// with rms(x) = sqrt(mean(x^2) + eps) per row, x an fp32 residual stream and s
// the residual scale.  The query slice stands in for the attention output.
#include "kernels.hpp"

namespace w4a8 {

namespace {

constexpr int kGlueThreads = 256;
// Rows of up to kRegGroups * kGlueThreads 8-element groups stay in registers
// between the sum of squares and the quantisation.
constexpr int kRegGroups = 2;

// Fixed-order workgroup sum of fp64 partial sums of squares: wave shuffles,
// then the 4 wave totals in order.
__device__ __forceinline__ double block_sum(double v, double* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  const double t = ((red[0] + red[1]) + red[2]) + red[3];
  __syncthreads();
  return t;
}

// One workgroup per row: optionally x += alpha * d (one fma per element, so
// x' = RN(x + alpha*d)), then y = fp16(x' * (1 / sqrt(mean(x'^2) + eps))).
__global__ __launch_bounds__(kGlueThreads) void residual_norm_cast_kernel(
    float* __restrict__ x, const float* __restrict__ d, int64_t ld_d, float alpha, float eps, int H,
    uint16_t* __restrict__ y) {
  __shared__ double red[4];
  const int64_t m = blockIdx.x;
  float* xr = x + m * H;
  double ss = 0.0;
  for (int h = threadIdx.x; h < H; h += kGlueThreads) {
    float v = xr[h];
    if (d) {
      v = fmaf(alpha, d[m * ld_d + h], v);
      xr[h] = v;
    }
    ss = add_square(ss, v);
  }
  const float inv = rms_inverse(block_sum(ss, red), H, eps);
  if (y)
    for (int h = threadIdx.x; h < H; h += kGlueThreads) y[m * H + h] = half_of_product(xr[h], inv);
}

// x += alpha * d with no normalised output: elementwise, four floats per
// thread (H and ld_d multiples of 4, 16-byte aligned rows), the grid's y
// dimension walking the rows; the same one fma per element as the kernel above.
__global__ __launch_bounds__(kGlueThreads) void residual_add_kernel(float* __restrict__ x, const float* __restrict__ d,
                                                                    int64_t ld_d, float alpha, int M, int H) {
  const int h = 4 * (blockIdx.x * kGlueThreads + threadIdx.x);
  if (h >= H) return;
  for (int64_t m = blockIdx.y; m < M; m += gridDim.y) {  // grid y: rows
    float4 v = *reinterpret_cast<const float4*>(x + m * H + h);
    const float4 dv = *reinterpret_cast<const float4*>(d + m * ld_d + h);
    v.x = fmaf(alpha, dv.x, v.x);
    v.y = fmaf(alpha, dv.y, v.y);
    v.z = fmaf(alpha, dv.z, v.z);
    v.w = fmaf(alpha, dv.w, v.w);
    *reinterpret_cast<float4*>(x + m * H + h) = v;
  }
}

// dst[m][h] = fp16(src[m * ld + h]) for h < H.
__global__ __launch_bounds__(kGlueThreads) void cast_rows_kernel(const float* __restrict__ src, int64_t ld,
                                                                 int M, int H, uint16_t* __restrict__ dst) {
  const int h = blockIdx.x * kGlueThreads + threadIdx.x;
  if (h >= H) return;
  for (int64_t m = blockIdx.y; m < M; m += gridDim.y) dst[m * H + h] = float_to_half_bits(src[m * ld + h]);
}

// u[m][f] = fp16(fp32(g[m][f] * g[m][F + f])) for f < F (rows of g hold 2F values).
__global__ __launch_bounds__(kGlueThreads) void gated_cast_kernel(const float* __restrict__ g, int M, int F,
                                                                  uint16_t* __restrict__ u) {
  const int f = blockIdx.x * kGlueThreads + threadIdx.x;
  if (f >= F) return;
  for (int64_t m = blockIdx.y; m < M; m += gridDim.y) {
    const float* row = g + m * 2 * static_cast<int64_t>(F);
    u[m * F + f] = half_of_product(row[f], row[F + f]);
  }
}

// The glue kernels below write the next linear's input straight into GEMM
// staging, the bytes the quantise pre-pass would write from the fp16 result of
// the kernels above (each fp16 value is formed the same way and quantised by
// the same device function).  One workgroup per staging row; rows M .. M_pad-1
// get zero codes and scales.  Thread t owns the 8-element groups
// e = t, t + 256, ... of its row, so every aligned quad of lanes holds one
// 32-element block (H is a multiple of 32 and 256 of 4).

// Optionally x += alpha * d, then fp16(x / rms(x)) quantised into staging.
__global__ __launch_bounds__(kGlueThreads) void residual_norm_quant_kernel(
    float* __restrict__ x, const float* __restrict__ d, int64_t ld_d, float alpha, float eps, int M, int H,
    int m_pad, uint8_t* __restrict__ qxs, float* __restrict__ sxs) {
  __shared__ double red[4];
  const int64_t m = blockIdx.x;
  const int groups = H / 8;
  if (m >= M) {  // padding row (uniform)
    const float zero[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int e = threadIdx.x; e < groups; e += kGlueThreads) quantize_to_staging(zero, m, e, m_pad, qxs, sxs);
    return;
  }
  float* xr = x + m * H;
  double ss = 0.0;
  if (groups <= kRegGroups * kGlueThreads) {  // uniform: the row stays in registers
    float4 lo[kRegGroups], hi[kRegGroups];
#pragma unroll
    for (int i = 0; i < kRegGroups; ++i) {
      const int e = threadIdx.x + i * kGlueThreads;
      if (e < groups) {
        lo[i] = *reinterpret_cast<const float4*>(xr + 8 * e);
        hi[i] = *reinterpret_cast<const float4*>(xr + 8 * e + 4);
        if (d) {
          const float4 d0 = *reinterpret_cast<const float4*>(d + m * ld_d + 8 * e);
          const float4 d1 = *reinterpret_cast<const float4*>(d + m * ld_d + 8 * e + 4);
          lo[i].x = fmaf(alpha, d0.x, lo[i].x); lo[i].y = fmaf(alpha, d0.y, lo[i].y);
          lo[i].z = fmaf(alpha, d0.z, lo[i].z); lo[i].w = fmaf(alpha, d0.w, lo[i].w);
          hi[i].x = fmaf(alpha, d1.x, hi[i].x); hi[i].y = fmaf(alpha, d1.y, hi[i].y);
          hi[i].z = fmaf(alpha, d1.z, hi[i].z); hi[i].w = fmaf(alpha, d1.w, hi[i].w);
          *reinterpret_cast<float4*>(xr + 8 * e) = lo[i];
          *reinterpret_cast<float4*>(xr + 8 * e + 4) = hi[i];
        }
        ss = add_square(ss, lo[i].x); ss = add_square(ss, lo[i].y);
        ss = add_square(ss, lo[i].z); ss = add_square(ss, lo[i].w);
        ss = add_square(ss, hi[i].x); ss = add_square(ss, hi[i].y);
        ss = add_square(ss, hi[i].z); ss = add_square(ss, hi[i].w);
      }
    }
    const float inv = rms_inverse(block_sum(ss, red), H, eps);
#pragma unroll
    for (int i = 0; i < kRegGroups; ++i) {
      const int e = threadIdx.x + i * kGlueThreads;
      if (e < groups) {
        const float raw[8] = {lo[i].x, lo[i].y, lo[i].z, lo[i].w, hi[i].x, hi[i].y, hi[i].z, hi[i].w};
        float v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = half_bits_to_float(half_of_product(raw[k], inv));
        quantize_to_staging(v, m, e, m_pad, qxs, sxs);
      }
    }
    return;
  }
  for (int e = threadIdx.x; e < groups; e += kGlueThreads) {
    float4 lo = *reinterpret_cast<const float4*>(xr + 8 * e);
    float4 hi = *reinterpret_cast<const float4*>(xr + 8 * e + 4);
    if (d) {
      const float* dr = d + m * ld_d + 8 * e;
      lo.x = fmaf(alpha, dr[0], lo.x); lo.y = fmaf(alpha, dr[1], lo.y);
      lo.z = fmaf(alpha, dr[2], lo.z); lo.w = fmaf(alpha, dr[3], lo.w);
      hi.x = fmaf(alpha, dr[4], hi.x); hi.y = fmaf(alpha, dr[5], hi.y);
      hi.z = fmaf(alpha, dr[6], hi.z); hi.w = fmaf(alpha, dr[7], hi.w);
      *reinterpret_cast<float4*>(xr + 8 * e) = lo;
      *reinterpret_cast<float4*>(xr + 8 * e + 4) = hi;
    }
    ss = add_square(ss, lo.x); ss = add_square(ss, lo.y); ss = add_square(ss, lo.z); ss = add_square(ss, lo.w);
    ss = add_square(ss, hi.x); ss = add_square(ss, hi.y); ss = add_square(ss, hi.z); ss = add_square(ss, hi.w);
  }
  const float inv = rms_inverse(block_sum(ss, red), H, eps);
  // Each thread re-reads only the elements it wrote above.
  for (int e = threadIdx.x; e < groups; e += kGlueThreads) {
    const float4 lo = *reinterpret_cast<const float4*>(xr + 8 * e);
    const float4 hi = *reinterpret_cast<const float4*>(xr + 8 * e + 4);
    const float raw[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = half_bits_to_float(half_of_product(raw[k], inv));
    quantize_to_staging(v, m, e, m_pad, qxs, sxs);
  }
}

// fp16(src[m * ld + h]) for h < H, quantised into staging.
__global__ __launch_bounds__(kGlueThreads) void cast_quant_kernel(const float* __restrict__ src, int64_t ld,
                                                                  int M, int H, int m_pad,
                                                                  uint8_t* __restrict__ qxs,
                                                                  float* __restrict__ sxs) {
  const int64_t m = blockIdx.x;
  for (int e = threadIdx.x; e < H / 8; e += kGlueThreads) {
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (m < M) {  // uniform
      const float4 lo = *reinterpret_cast<const float4*>(src + m * ld + 8 * e);
      const float4 hi = *reinterpret_cast<const float4*>(src + m * ld + 8 * e + 4);
      const float raw[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = half_bits_to_float(float_to_half_bits(raw[k]));
    }
    quantize_to_staging(v, m, e, m_pad, qxs, sxs);
  }
}

// fp16(g[m][f] * g[m][F + f]) for f < F, quantised into staging.
// Rows are split over gridDim.x workgroups, one 8-element group per thread
// (F / 8 is a multiple of 4, so quads of lanes are whole blocks, in range or not).
__global__ __launch_bounds__(kGlueThreads) void gated_quant_kernel(const float* __restrict__ g, int M, int F,
                                                                   int m_pad, uint8_t* __restrict__ qxs,
                                                                   float* __restrict__ sxs) {
  const int e = blockIdx.x * kGlueThreads + threadIdx.x;
  if (e >= F / 8) return;
  for (int64_t m = blockIdx.y; m < m_pad; m += gridDim.y) {  // grid y: staging rows
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (m < M) {  // uniform
      const float* row = g + m * 2 * static_cast<int64_t>(F) + 8 * e;
      const float4 g0 = *reinterpret_cast<const float4*>(row);
      const float4 g1 = *reinterpret_cast<const float4*>(row + 4);
      const float4 u0 = *reinterpret_cast<const float4*>(row + F);
      const float4 u1 = *reinterpret_cast<const float4*>(row + F + 4);
      const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
      const float uv[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = half_bits_to_float(half_of_product(gv[k], uv[k]));
    }
    quantize_to_staging(v, m, e, m_pad, qxs, sxs);
  }
}

size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

}  // namespace

int launch_residual_norm_cast(float* x, const float* d, int64_t ld_d, float alpha, float eps, int M, int H,
                              uint16_t* y, hipStream_t stream) {
  const bool vec = d && !y && H % 4 == 0 && ld_d % 4 == 0 && reinterpret_cast<uintptr_t>(x) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(d) % 16 == 0;
  if (vec) {
    const dim3 grid((H / 4 + kGlueThreads - 1) / kGlueThreads, M < 65535 ? M : 65535);
    hipLaunchKernelGGL(residual_add_kernel, grid, dim3(kGlueThreads), 0, stream, x, d, ld_d, alpha, M, H);
    W4A8_HIP(hipGetLastError());
    return W4A8_OK;
  }
  hipLaunchKernelGGL(residual_norm_cast_kernel, dim3(M), dim3(kGlueThreads), 0, stream, x, d, ld_d, alpha,
                     eps, H, y);
  W4A8_HIP(hipGetLastError());
  return W4A8_OK;
}

int launch_cast_rows(const float* src, int64_t ld, int M, int H, uint16_t* dst, hipStream_t stream) {
  hipLaunchKernelGGL(cast_rows_kernel, dim3((H + kGlueThreads - 1) / kGlueThreads, M < 65535 ? M : 65535),
                     dim3(kGlueThreads), 0, stream, src, ld, M, H, dst);
  W4A8_HIP(hipGetLastError());
  return W4A8_OK;
}

int launch_gated_cast(const float* g, int M, int F, uint16_t* u, hipStream_t stream) {
  hipLaunchKernelGGL(gated_cast_kernel, dim3((F + kGlueThreads - 1) / kGlueThreads, M < 65535 ? M : 65535),
                     dim3(kGlueThreads), 0, stream, g, M, F, u);
  W4A8_HIP(hipGetLastError());
  return W4A8_OK;
}

int launch_residual_norm_quant(float* x, const float* d, int64_t ld_d, float alpha, float eps, int M, int H,
                               const GemmStaging& s, hipStream_t stream) {
  hipLaunchKernelGGL(residual_norm_quant_kernel, dim3(s.m_pad), dim3(kGlueThreads), 0, stream, x, d, ld_d, alpha,
                     eps, M, H, s.m_pad, s.qxs, s.sxs);
  W4A8_HIP(hipGetLastError());
  return W4A8_OK;
}

int launch_cast_quant(const float* src, int64_t ld, int M, int H, const GemmStaging& s, hipStream_t stream) {
  hipLaunchKernelGGL(cast_quant_kernel, dim3(s.m_pad), dim3(kGlueThreads), 0, stream, src, ld, M, H, s.m_pad,
                     s.qxs, s.sxs);
  W4A8_HIP(hipGetLastError());
  return W4A8_OK;
}

int launch_gated_quant(const float* g, int M, int F, const GemmStaging& s, hipStream_t stream) {
  hipLaunchKernelGGL(gated_quant_kernel,
                     dim3((F / 8 + kGlueThreads - 1) / kGlueThreads, s.m_pad < 65535 ? s.m_pad : 65535),
                     dim3(kGlueThreads), 0, stream, g, M, F, s.m_pad, s.qxs, s.sxs);
  W4A8_HIP(hipGetLastError());
  return W4A8_OK;
}

// Workspace carve-up of one decoder layer: q, a, o, n, g, u, d.
LayerWorkspace layer_workspace(int M, int H, int n_qkv, int n_gu) {
  LayerWorkspace w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  w.q = take(static_cast<size_t>(M) * n_qkv * 4);
  // a: the fp16 query slice, or (when the qkv GEMM quantises it itself) the
  // staging of the o projection.
  const size_t a_bytes = static_cast<size_t>(M) * H * 2;
  const size_t so_bytes = gemm_staging_bytes(M, H, H);
  w.a = take(a_bytes > so_bytes ? a_bytes : so_bytes);
  w.o = take(static_cast<size_t>(M) * H * 4);
  w.n = take(static_cast<size_t>(M) * H * 2);
  // g: the gate/up output, or (when the gate/up GEMM quantises its gated
  // product itself) the staging of the down projection.
  const size_t g_bytes = static_cast<size_t>(M) * n_gu * 4;
  const size_t sd_bytes = gemm_staging_bytes(M, n_gu / 2, H);
  w.g = take(g_bytes > sd_bytes ? g_bytes : sd_bytes);
  w.u = take(static_cast<size_t>(M) * (n_gu / 2) * 2);
  w.d = take(static_cast<size_t>(M) * H * 4);
  w.bytes = off;
  return w;
}

}  // namespace w4a8
