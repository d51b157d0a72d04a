// C ABI of the W4A8 block-32 library: argument validation, per-device scratch,
// stage dispatch (decode GEMV or prefill GEMM) and error reporting.
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "kernels.hpp"

namespace w4a8 {

namespace {

thread_local char g_error[512] = "";

constexpr int kMaxDevices = 64;
constexpr size_t kInitialWork = 32u << 20;

struct DeviceState {
  bool ready = false;
  Scratch sc;
};
DeviceState g_dev[kMaxDevices];
bool g_any_ready = false;
std::mutex g_mutex;

int g_gemv_max_m = -1;
bool g_gemv_max_m_forced = false;

int current_state(DeviceState** out) {
  if (!g_any_ready) {
    set_error("w4a8_init has not been called");
    return W4A8_ENOINIT;
  }
  int dev = -1;
  W4A8_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices || !g_dev[dev].ready) {
    set_error("w4a8_init has not been called for device %d", dev);
    return W4A8_ENOINIT;
  }
  *out = &g_dev[dev];
  return W4A8_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_shape(int64_t M, int64_t K, int64_t N, int64_t max_m) {
  if (M < 1 || M > max_m) {
    set_error("M = %lld out of range [1, %lld]", static_cast<long long>(M), static_cast<long long>(max_m));
    return W4A8_EINVAL;
  }
  if (K < kBlock || K % kBlock != 0 || K >= (int64_t{1} << 31)) {
    set_error("K = %lld must be a positive multiple of 32 below 2^31", static_cast<long long>(K));
    return W4A8_EINVAL;
  }
  if (N < 64 || N % 64 != 0 || N / 64 >= kMaxTickets - 1) {
    set_error("N = %lld must be a positive multiple of 64 below %lld", static_cast<long long>(N),
              static_cast<long long>(int64_t{64} * (kMaxTickets - 1)));
    return W4A8_EINVAL;
  }
  if (K / 2 * N >= (int64_t{1} << 40)) {
    set_error("packed weights of %lld x %lld exceed 2^40 bytes", static_cast<long long>(K),
              static_cast<long long>(N));
    return W4A8_EINVAL;
  }
  return W4A8_OK;
}

#define W4A8_REQUIRE(cond, ...)   \
  do {                            \
    if (!(cond)) {                \
      set_error(__VA_ARGS__);     \
      return W4A8_EINVAL;         \
    }                             \
  } while (0)

int check_linear_args(const uint16_t* x, const uint8_t* pw, const uint16_t* ws, int64_t M, int64_t K,
                      int64_t N, int64_t max_m) {
  W4A8_REQUIRE(x && pw && ws, "null input pointer");
  int rc = check_shape(M, K, N, max_m);
  if (rc != W4A8_OK) return rc;
  W4A8_REQUIRE(aligned(x, 16), "x must be 16-byte aligned");
  W4A8_REQUIRE(aligned(pw, 16), "packed_w must be 16-byte aligned");
  W4A8_REQUIRE(aligned(ws, 16), "w_scales must be 16-byte aligned");
  return W4A8_OK;
}

}  // namespace

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_error, sizeof(g_error), fmt, ap);
  va_end(ap);
}

int hip_fail(hipError_t e, const char* what) {
  set_error("%s failed: %s", what, hipGetErrorString(e));
  return W4A8_EHIP;
}

int scratch_for(size_t work_bytes, Scratch** out) {
  DeviceState* st = nullptr;
  int rc = current_state(&st);
  if (rc != W4A8_OK) return rc;
  Scratch& sc = st->sc;
  if (work_bytes > sc.work_bytes) {
    std::lock_guard<std::mutex> lock(g_mutex);
    if (work_bytes > sc.work_bytes) {
      // Kernels already queued may still read the old buffer.
      W4A8_HIP(hipDeviceSynchronize());
      if (sc.work) W4A8_HIP(hipFree(sc.work));
      sc.work = nullptr;
      sc.work_bytes = 0;
      const size_t bytes = (work_bytes + (1u << 20) - 1) & ~static_cast<size_t>((1u << 20) - 1);
      W4A8_HIP(hipMalloc(&sc.work, bytes));
      sc.work_bytes = bytes;
    }
  }
  *out = &sc;
  return W4A8_OK;
}

int gemv_max_m() {
  if (g_gemv_max_m < 0) {
    int v = 4;
    if (const char* e = std::getenv("W4A8_GEMV_MAX_M")) {
      const int u = std::atoi(e);
      if (u >= 0 && u <= 64) {
        v = u;
        g_gemv_max_m_forced = true;
      }
    }
    g_gemv_max_m = v;
  }
  return g_gemv_max_m;
}

// Stage of W4A8_PATH_AUTO.  The GEMV's time grows with M (every workgroup
// quantises all M rows of x it reads and forms M dot products per weight
// load) while the GEMM's barely moves at small M, so the crossover falls with
// the size of the weight matrix: measured on MI355X with cold weights, the GEMV
// is faster through M = 4 for 2048 x 2560, 2048 x 16384 and 8192 x 2048, but
// only through M = 2 for 4096 x 14336 (2^25.8 values).  W4A8_GEMV_MAX_M in the
// environment replaces the rule by a plain M threshold.
int auto_path(int64_t M, int64_t K, int64_t N) {
  const int lim = gemv_max_m();
  if (g_gemv_max_m_forced) return M <= lim ? W4A8_PATH_GEMV : W4A8_PATH_GEMM;
  const bool big = K * N > (int64_t{1} << 25);
  return M <= (big ? (lim < 2 ? lim : 2) : lim) ? W4A8_PATH_GEMV : W4A8_PATH_GEMM;
}

}  // namespace w4a8

using namespace w4a8;

extern "C" {

int w4a8_init(int device) {
  int count = 0;
  W4A8_HIP(hipGetDeviceCount(&count));
  W4A8_REQUIRE(device >= 0 && device < count && device < kMaxDevices, "device %d not present", device);
  W4A8_HIP(hipSetDevice(device));
  std::lock_guard<std::mutex> lock(g_mutex);
  DeviceState& st = g_dev[device];
  if (st.ready) return W4A8_OK;
  hipDeviceProp_t prop;
  W4A8_HIP(hipGetDeviceProperties(&prop, device));
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
    set_error("device %d is %s; this library is built for gfx950 only", device, prop.gcnArchName);
    return W4A8_EUNSUPPORTED;
  }
  Scratch& sc = st.sc;
  sc.bytes = kMaxTickets * sizeof(uint32_t) + kMaxArgmaxRows * kArgmaxSpread * sizeof(unsigned long long);
  W4A8_HIP(hipMalloc(&sc.base, sc.bytes));
  W4A8_HIP(hipMemset(sc.base, 0, sc.bytes));
  sc.slots = static_cast<unsigned long long*>(sc.base);
  sc.tickets = reinterpret_cast<uint32_t*>(static_cast<char*>(sc.base) +
                                           kMaxArgmaxRows * kArgmaxSpread * sizeof(unsigned long long));
  W4A8_HIP(hipMalloc(&sc.work, kInitialWork));
  sc.work_bytes = kInitialWork;
  W4A8_HIP(hipDeviceSynchronize());
  st.ready = true;
  g_any_ready = true;
  return W4A8_OK;
}

int w4a8_pack_weights(const int8_t* q, const uint16_t* s, int64_t K, int64_t N, uint8_t* packed_w,
                      uint16_t* w_scales, hipStream_t stream) {
  W4A8_REQUIRE(q && s && packed_w && w_scales, "null pointer");
  int rc = check_shape(1, K, N, 1);
  if (rc != W4A8_OK) return rc;
  W4A8_REQUIRE(aligned(packed_w, 16), "packed_w must be 16-byte aligned");
  W4A8_REQUIRE(aligned(s, 2) && aligned(w_scales, 2), "scales must be 2-byte aligned");
  DeviceState* st = nullptr;
  rc = current_state(&st);
  if (rc != W4A8_OK) return rc;
  return launch_pack(q, s, static_cast<int>(K), static_cast<int>(N), packed_w, w_scales, stream);
}

int w4a8_linear_path(const uint16_t* x, const uint8_t* packed_w, const uint16_t* w_scales, int64_t M,
                     int64_t K, int64_t N, float* out, int path, hipStream_t stream) {
  int rc = check_linear_args(x, packed_w, w_scales, M, K, N, int64_t{1} << 20);
  if (rc != W4A8_OK) return rc;
  W4A8_REQUIRE(out, "null output pointer");
  W4A8_REQUIRE(aligned(out, 16), "out must be 16-byte aligned");
  W4A8_REQUIRE(path == W4A8_PATH_AUTO || path == W4A8_PATH_GEMV || path == W4A8_PATH_GEMM,
               "unknown path %d", path);
  DeviceState* st = nullptr;
  rc = current_state(&st);
  if (rc != W4A8_OK) return rc;
  if (path == W4A8_PATH_AUTO) path = auto_path(M, K, N);
  if (path == W4A8_PATH_GEMV) {
    GemvArgs a{x, packed_w, w_scales, static_cast<int>(M), static_cast<int>(K), static_cast<int>(N),
               out, nullptr, nullptr, nullptr};
    return launch_gemv(a, 0, stream);
  }
  GemmArgs a{x, packed_w, w_scales, static_cast<int>(M), static_cast<int>(K), static_cast<int>(N), out,
             nullptr};
  return launch_gemm(a, 0, stream);
}

int w4a8_linear(const uint16_t* x, const uint8_t* packed_w, const uint16_t* w_scales, int64_t M,
                int64_t K, int64_t N, float* out, hipStream_t stream) {
  return w4a8_linear_path(x, packed_w, w_scales, M, K, N, out, W4A8_PATH_AUTO, stream);
}

int w4a8_linear_argmax(const uint16_t* x, const uint8_t* packed_w, const uint16_t* w_scales, int64_t M,
                       int64_t K, int64_t N, float* logits, int32_t* argmax, hipStream_t stream) {
  int rc = check_linear_args(x, packed_w, w_scales, M, K, N, kMaxArgmaxRows);
  if (rc != W4A8_OK) return rc;
  W4A8_REQUIRE(argmax, "null argmax pointer");
  W4A8_REQUIRE(aligned(argmax, 4), "argmax must be 4-byte aligned");
  W4A8_REQUIRE(!logits || aligned(logits, 16), "logits must be 16-byte aligned");
  DeviceState* st = nullptr;
  rc = current_state(&st);
  if (rc != W4A8_OK) return rc;
  GemvArgs a{x, packed_w, w_scales, static_cast<int>(M), static_cast<int>(K), static_cast<int>(N),
             nullptr, nullptr, logits, argmax};
  return launch_gemv(a, 2, stream);
}

int w4a8_quantize_act(const uint16_t* x, int64_t M, int64_t K, int8_t* qx, float* sx,
                      hipStream_t stream) {
  W4A8_REQUIRE(x && qx && sx, "null pointer");
  int rc = check_shape(M, K, 64, int64_t{1} << 24);
  if (rc != W4A8_OK) return rc;
  W4A8_REQUIRE(M * K < (int64_t{1} << 34), "M * K too large");
  W4A8_REQUIRE(aligned(x, 16) && aligned(qx, 8) && aligned(sx, 4), "misaligned pointer");
  DeviceState* st = nullptr;
  rc = current_state(&st);
  if (rc != W4A8_OK) return rc;
  return launch_quantize_export(x, static_cast<int>(M), static_cast<int>(K), qx, sx, stream);
}

int w4a8_block_sums(const uint16_t* x, const uint8_t* packed_w, int64_t M, int64_t K, int64_t N,
                    int32_t* sums, int path, hipStream_t stream) {
  // The block-sum kernels read no scales; the packed weights stand in for them here.
  int rc = check_linear_args(x, packed_w, reinterpret_cast<const uint16_t*>(packed_w), M, K, N,
                             int64_t{1} << 16);
  if (rc != W4A8_OK) return rc;
  W4A8_REQUIRE(sums && aligned(sums, 16), "sums must be a 16-byte aligned pointer");
  W4A8_REQUIRE(path == W4A8_PATH_AUTO || path == W4A8_PATH_GEMV || path == W4A8_PATH_GEMM,
               "unknown path %d", path);
  DeviceState* st = nullptr;
  rc = current_state(&st);
  if (rc != W4A8_OK) return rc;
  if (path == W4A8_PATH_AUTO) path = auto_path(M, K, N);
  if (path == W4A8_PATH_GEMV) {
    GemvArgs a{x, packed_w, nullptr, static_cast<int>(M), static_cast<int>(K), static_cast<int>(N),
               nullptr, sums, nullptr, nullptr};
    return launch_gemv(a, 1, stream);
  }
  GemmArgs a{x, packed_w, nullptr, static_cast<int>(M), static_cast<int>(K), static_cast<int>(N),
             nullptr, sums};
  return launch_gemm(a, 1, stream);
}

int w4a8_residual_norm_cast(float* x, const float* d, int64_t ld_d, float alpha, float eps, int64_t M,
                            int64_t H, uint16_t* y, hipStream_t stream) {
  W4A8_REQUIRE(x, "null x");
  W4A8_REQUIRE(M >= 1 && M <= (int64_t{1} << 20) && H >= 1 && H < (int64_t{1} << 24), "bad shape M=%lld H=%lld",
               static_cast<long long>(M), static_cast<long long>(H));
  W4A8_REQUIRE(!d || ld_d >= H, "ld_d must be at least H");
  W4A8_REQUIRE(eps >= 0.0f, "eps must be non-negative");
  DeviceState* st = nullptr;
  int rc = current_state(&st);
  if (rc != W4A8_OK) return rc;
  return launch_residual_norm_cast(x, d, ld_d, alpha, eps, static_cast<int>(M), static_cast<int>(H), y, stream);
}

namespace {
int check_weights(const w4a8_weights* w, const char* name) {
  W4A8_REQUIRE(w && w->packed_w && w->w_scales, "%s: null weights", name);
  W4A8_REQUIRE(aligned(w->packed_w, 16) && aligned(w->w_scales, 16), "%s: weights must be 16-byte aligned", name);
  return check_shape(1, w->K, w->N, 1);
}
}  // namespace

int w4a8_decoder_layer_workspace(int64_t M, int64_t H, const w4a8_weights* qkv, const w4a8_weights* gate_up,
                                 size_t* bytes) {
  W4A8_REQUIRE(bytes && qkv && gate_up, "null pointer");
  W4A8_REQUIRE(M >= 1 && M <= 65536 && H >= 64 && H % 64 == 0 && H < (int64_t{1} << 24), "bad shape");
  W4A8_REQUIRE(qkv->N >= H && qkv->N < (int64_t{1} << 30) && gate_up->N >= 128 && gate_up->N < (int64_t{1} << 30),
               "bad weight shapes");
  *bytes = layer_workspace(static_cast<int>(M), static_cast<int>(H), static_cast<int>(qkv->N),
                           static_cast<int>(gate_up->N)).bytes;
  return W4A8_OK;
}

int w4a8_decoder_layer(float* x, int64_t M, int64_t H, const w4a8_weights* qkv, const w4a8_weights* o,
                       const w4a8_weights* gate_up, const w4a8_weights* down, float residual_scale, float eps,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  W4A8_REQUIRE(x && aligned(x, 16), "x must be a 16-byte aligned pointer");
  W4A8_REQUIRE(M >= 1 && M <= 65536 && H >= 64 && H % 64 == 0 && H < (int64_t{1} << 24), "bad shape M=%lld H=%lld",
               static_cast<long long>(M), static_cast<long long>(H));
  int rc;
  if ((rc = check_weights(qkv, "qkv")) != W4A8_OK || (rc = check_weights(o, "o")) != W4A8_OK ||
      (rc = check_weights(gate_up, "gate_up")) != W4A8_OK || (rc = check_weights(down, "down")) != W4A8_OK)
    return rc;
  W4A8_REQUIRE(qkv->K == H && qkv->N >= H, "qkv must be H x N with N >= H");
  W4A8_REQUIRE(o->K == H && o->N == H, "o must be H x H");
  W4A8_REQUIRE(gate_up->K == H && gate_up->N % 128 == 0 && down->K == gate_up->N / 2 && down->N == H,
               "gate_up must be H x 2F and down F x H");
  W4A8_REQUIRE(gate_up->N < (int64_t{1} << 30) && qkv->N < (int64_t{1} << 30), "weights too wide");
  const LayerWorkspace w = layer_workspace(static_cast<int>(M), static_cast<int>(H), static_cast<int>(qkv->N),
                                           static_cast<int>(gate_up->N));
  W4A8_REQUIRE(workspace && aligned(workspace, 256) && workspace_bytes >= w.bytes,
               "workspace must be 256-byte aligned and hold %zu bytes", w.bytes);
  DeviceState* st = nullptr;
  rc = current_state(&st);
  if (rc != W4A8_OK) return rc;

  char* base = static_cast<char*>(workspace);
  float* q = reinterpret_cast<float*>(base + w.q);
  uint16_t* a = reinterpret_cast<uint16_t*>(base + w.a);
  float* ob = reinterpret_cast<float*>(base + w.o);
  uint16_t* n = reinterpret_cast<uint16_t*>(base + w.n);
  float* g = reinterpret_cast<float*>(base + w.g);
  uint16_t* u = reinterpret_cast<uint16_t*>(base + w.u);
  float* d = reinterpret_cast<float*>(base + w.d);
  const int Mi = static_cast<int>(M), Hi = static_cast<int>(H);
  const int F = static_cast<int>(gate_up->N / 2);
#define W4A8_STEP(call)              \
  do {                              \
    if ((rc = (call)) != W4A8_OK) return rc; \
  } while (0)
  if (M == 1 && gemv_fused_supported(kGemvCast, true, Hi, static_cast<int>(qkv->N)) &&
      gemv_fused_supported(kGemvGated, true, Hi, 2 * F)) {
    // One token: four GEMV launches, with the normalisation in the prologue
    // of qkv and gate/up and the cast, residual and gated product in the
    // epilogues (the same values as the launches below, up to the summation
    // order of the norm).
    GemvArgs qa{nullptr, qkv->packed_w, qkv->w_scales, 1, Hi, static_cast<int>(qkv->N), q, nullptr, nullptr, nullptr};
    qa.xf = x;
    qa.eps = eps;
    qa.y16 = a;
    qa.n16 = Hi;
    W4A8_STEP(launch_gemv(qa, kGemvCast, stream));
    GemvArgs oa{a, o->packed_w, o->w_scales, 1, Hi, Hi, nullptr, nullptr, nullptr, nullptr};
    oa.resid = x;
    oa.alpha = residual_scale;
    W4A8_STEP(launch_gemv(oa, kGemvResid, stream));
    GemvArgs ga{nullptr, gate_up->packed_w, gate_up->w_scales, 1, Hi, 2 * F, nullptr, nullptr, nullptr, nullptr};
    ga.xf = x;
    ga.eps = eps;
    ga.y16 = u;
    W4A8_STEP(launch_gemv(ga, kGemvGated, stream));
    GemvArgs da{u, down->packed_w, down->w_scales, 1, F, Hi, nullptr, nullptr, nullptr, nullptr};
    da.resid = x;
    da.alpha = residual_scale;
    W4A8_STEP(launch_gemv(da, kGemvResid, stream));
    return W4A8_OK;
  }
  const int Nq = static_cast<int>(qkv->N);
  if (auto_path(M, H, qkv->N) == W4A8_PATH_GEMM && auto_path(M, H, H) == W4A8_PATH_GEMM &&
      auto_path(M, H, gate_up->N) == W4A8_PATH_GEMM && auto_path(M, F, H) == W4A8_PATH_GEMM) {
    // Many rows: every projection is a prefill GEMM, and the glue kernels
    // write their fp16 results straight into the next GEMM's quantised
    // staging, so no separate quantise pre-pass runs (four launches fewer).
    GemmStaging sg{};
    W4A8_STEP(gemm_staging(Mi, Hi, Nq, &sg));
    W4A8_STEP(launch_residual_norm_quant(x, nullptr, 0, 0.0f, eps, Mi, Hi, sg, stream));
    const GemmArgs qa{nullptr, qkv->packed_w, qkv->w_scales, Mi, Hi, Nq, q, nullptr};
    GemmStaging so = gemm_staging_at(a, Mi, Hi, Hi);
    if (gemm_cast_supported(Mi, Hi, Nq, Hi, so.m_pad)) {
      // The qkv GEMM quantises fp16 of its query slice into the o
      // projection's staging (in the workspace, in place of a) itself.
      W4A8_STEP(launch_gemm_staged_cast(qa, Hi, sg, so, stream));
    } else {
      W4A8_STEP(launch_gemm_staged(qa, sg, stream));
      W4A8_STEP(gemm_staging(Mi, Hi, Hi, &so));
      W4A8_STEP(launch_cast_quant(q, qkv->N, Mi, Hi, so, stream));
    }
    // The o projection adds 0.01 * o into the residual stream in its
    // epilogue; the normalisation then reads x alone.
    GemmArgs oa{nullptr, o->packed_w, o->w_scales, Mi, Hi, Hi, nullptr, nullptr};
    oa.resid = x;
    oa.alpha = residual_scale;
    W4A8_STEP(launch_gemm_staged_resid(oa, so, stream));
    W4A8_STEP(gemm_staging(Mi, Hi, 2 * F, &sg));
    W4A8_STEP(launch_residual_norm_quant(x, nullptr, 0, 0.0f, eps, Mi, Hi, sg, stream));
    const GemmArgs gua{nullptr, gate_up->packed_w, gate_up->w_scales, Mi, Hi, 2 * F, g, nullptr};
    GemmStaging sd = gemm_staging_at(g, Mi, F, Hi);
    if (gemm_gated_supported(Mi, Hi, 2 * F, sd.m_pad)) {
      // The gate/up GEMM forms fp16(gate * up) and quantises it into the down
      // projection's staging (in the workspace, in place of g) itself.
      W4A8_STEP(launch_gemm_staged_gated(gua, sg, sd, stream));
    } else {
      W4A8_STEP(launch_gemm_staged(gua, sg, stream));
      W4A8_STEP(gemm_staging(Mi, F, Hi, &sd));
      W4A8_STEP(launch_gated_quant(g, Mi, F, sd, stream));
    }
    // The down projection adds 0.01 * d straight into the residual stream in
    // its epilogue (the same fma per element as a separate residual add).
    GemmArgs da{nullptr, down->packed_w, down->w_scales, Mi, F, Hi, nullptr, nullptr};
    da.resid = x;
    da.alpha = residual_scale;
    W4A8_STEP(launch_gemm_staged_resid(da, sd, stream));
    return W4A8_OK;
  }
  W4A8_STEP(launch_residual_norm_cast(x, nullptr, 0, 0.0f, eps, Mi, Hi, n, stream));
  W4A8_STEP(w4a8_linear(n, qkv->packed_w, qkv->w_scales, M, H, qkv->N, q, stream));
  W4A8_STEP(launch_cast_rows(q, qkv->N, Mi, Hi, a, stream));
  W4A8_STEP(w4a8_linear(a, o->packed_w, o->w_scales, M, H, H, ob, stream));
  W4A8_STEP(launch_residual_norm_cast(x, ob, H, residual_scale, eps, Mi, Hi, n, stream));
  W4A8_STEP(w4a8_linear(n, gate_up->packed_w, gate_up->w_scales, M, H, gate_up->N, g, stream));
  W4A8_STEP(launch_gated_cast(g, Mi, F, u, stream));
  W4A8_STEP(w4a8_linear(u, down->packed_w, down->w_scales, M, F, H, d, stream));
  W4A8_STEP(launch_residual_norm_cast(x, d, H, residual_scale, eps, Mi, Hi, nullptr, stream));
#undef W4A8_STEP
  return W4A8_OK;
}

int w4a8_norm_linear_argmax(const float* x, float eps, const uint8_t* packed_w, const uint16_t* w_scales,
                            int64_t M, int64_t K, int64_t N, float* logits, int32_t* argmax, hipStream_t stream) {
  W4A8_REQUIRE(x && aligned(x, 16), "x must be a 16-byte aligned pointer");
  W4A8_REQUIRE(eps >= 0.0f, "eps must be non-negative");
  // The weights and sizes are checked as for the fp16 entry point (x stands in for the fp16 input).
  int rc = check_linear_args(reinterpret_cast<const uint16_t*>(x), packed_w, w_scales, M, K, N, kMaxArgmaxRows);
  if (rc != W4A8_OK) return rc;
  W4A8_REQUIRE(argmax && aligned(argmax, 4), "argmax must be a 4-byte aligned pointer");
  W4A8_REQUIRE(!logits || aligned(logits, 16), "logits must be 16-byte aligned");
  DeviceState* st = nullptr;
  rc = current_state(&st);
  if (rc != W4A8_OK) return rc;
  const int Mi = static_cast<int>(M), Ki = static_cast<int>(K), Ni = static_cast<int>(N);
  if (M == 1 && gemv_fused_supported(kGemvArgmax, true, Ki, Ni)) {
    GemvArgs a{nullptr, packed_w, w_scales, 1, Ki, Ni, nullptr, nullptr, logits, argmax};
    a.xf = x;
    a.eps = eps;
    return launch_gemv(a, kGemvArgmax, stream);
  }
  // Otherwise normalise into library scratch, then the fused-argmax GEMV.
  Scratch* sc = nullptr;
  rc = scratch_for(static_cast<size_t>(M) * K * 2, &sc);
  if (rc != W4A8_OK) return rc;
  uint16_t* y = static_cast<uint16_t*>(sc->work);
  rc = launch_residual_norm_cast(const_cast<float*>(x), nullptr, 0, 0.0f, eps, Mi, Ki, y, stream);
  if (rc != W4A8_OK) return rc;
  GemvArgs a{y, packed_w, w_scales, Mi, Ki, Ni, nullptr, nullptr, logits, argmax};
  return launch_gemv(a, kGemvArgmax, stream);
}

int w4a8_mx_pack_weights(const uint16_t* w, int64_t K, int64_t N, uint8_t* packed, uint8_t* scales,
                         hipStream_t stream) {
  W4A8_REQUIRE(w && packed && scales, "null pointer");
  int rc = check_shape(1, K, N, 1);
  if (rc != W4A8_OK) return rc;
  W4A8_REQUIRE(K % 64 == 0, "K = %lld must be a multiple of 64", static_cast<long long>(K));
  W4A8_REQUIRE(aligned(w, 16) && aligned(packed, 16), "w and packed must be 16-byte aligned");
  DeviceState* st = nullptr;
  rc = current_state(&st);
  if (rc != W4A8_OK) return rc;
  return launch_mx_pack(w, static_cast<int>(K), static_cast<int>(N), packed, scales, stream);
}

int w4a8_mx_quantize_act(const uint16_t* x, int64_t M, int64_t K, uint8_t* codes, uint8_t* scales,
                         hipStream_t stream) {
  W4A8_REQUIRE(x && codes && scales, "null pointer");
  int rc = check_shape(M, K, 64, int64_t{1} << 24);
  if (rc != W4A8_OK) return rc;
  W4A8_REQUIRE(K % 64 == 0, "K = %lld must be a multiple of 64", static_cast<long long>(K));
  W4A8_REQUIRE(M * K < (int64_t{1} << 34), "M * K too large");
  W4A8_REQUIRE(aligned(x, 16) && aligned(codes, 8), "misaligned pointer");
  DeviceState* st = nullptr;
  rc = current_state(&st);
  if (rc != W4A8_OK) return rc;
  return launch_mx_quantize_act(x, static_cast<int>(M), static_cast<int>(M), static_cast<int>(K), codes, scales,
                                stream);
}

int w4a8_mx_linear(const uint16_t* x, const uint8_t* packed, const uint8_t* scales, int64_t M, int64_t K,
                   int64_t N, float* out, hipStream_t stream) {
  W4A8_REQUIRE(x && packed && scales && out, "null pointer");
  int rc = check_shape(M, K, N, int64_t{1} << 20);
  if (rc != W4A8_OK) return rc;
  W4A8_REQUIRE(K % 64 == 0, "K = %lld must be a multiple of 64", static_cast<long long>(K));
  W4A8_REQUIRE(aligned(x, 16) && aligned(packed, 16) && aligned(out, 4), "misaligned pointer");
  DeviceState* st = nullptr;
  rc = current_state(&st);
  if (rc != W4A8_OK) return rc;
  return launch_mx_linear(x, packed, scales, static_cast<int>(M), static_cast<int>(K), static_cast<int>(N), out,
                          stream);
}

int w4a8_decode_attention(const float* q, const float* k_new, const float* v_new, uint16_t* k_cache,
                          uint16_t* v_cache, int64_t n_heads, int64_t n_kv_heads, int64_t head_dim, int64_t length,
                          int64_t capacity, uint16_t* out, hipStream_t stream) {
  W4A8_REQUIRE(q && k_new && v_new && k_cache && v_cache && out, "null pointer");
  W4A8_REQUIRE(head_dim == 64 || head_dim == 128 || head_dim == 256, "head_dim = %lld must be 64, 128 or 256",
               static_cast<long long>(head_dim));
  W4A8_REQUIRE(n_kv_heads >= 1 && n_kv_heads <= 4096, "n_kv_heads = %lld out of range [1, 4096]",
               static_cast<long long>(n_kv_heads));
  W4A8_REQUIRE(n_heads >= n_kv_heads && n_heads % n_kv_heads == 0 && n_heads / n_kv_heads <= 8,
               "n_heads = %lld must be 1 to 8 times n_kv_heads = %lld", static_cast<long long>(n_heads),
               static_cast<long long>(n_kv_heads));
  W4A8_REQUIRE(capacity >= 64 && capacity % 64 == 0 && capacity <= (int64_t{1} << 24),
               "capacity = %lld must be a multiple of 64 in [64, 2^24]", static_cast<long long>(capacity));
  W4A8_REQUIRE(length >= 1 && length <= capacity, "length = %lld out of range [1, capacity = %lld]",
               static_cast<long long>(length), static_cast<long long>(capacity));
  W4A8_REQUIRE(n_kv_heads * capacity * head_dim < (int64_t{1} << 38), "KV cache too large");
  W4A8_REQUIRE(aligned(q, 16) && aligned(k_new, 16) && aligned(v_new, 16) && aligned(out, 16) &&
                   aligned(k_cache, 16) && aligned(v_cache, 16),
               "every pointer must be 16-byte aligned");
  const int Hq = static_cast<int>(n_heads), Hkv = static_cast<int>(n_kv_heads), D = static_cast<int>(head_dim);
  const int Li = static_cast<int>(length), cap = static_cast<int>(capacity);
  Scratch* sc = nullptr;
  int rc = scratch_for(attention_scratch_bytes(Hkv, Hq / Hkv, D, Li), &sc);
  if (rc != W4A8_OK) return rc;
  return launch_decode_attention(q, k_new, v_new, k_cache, v_cache, Hq, Hkv, D, Li, cap, out, sc, stream);
}

int w4a8_gemv_max_m(void) { return gemv_max_m(); }

int w4a8_auto_path(int64_t M, int64_t K, int64_t N) { return auto_path(M, K, N); }

const char* w4a8_last_error(void) { return g_error; }

}  // extern "C"
