// C ABI of the W4A8 block-32 library: argument validation, per-device scratch,
// stage dispatch (decode GEMV or prefill GEMM) and error reporting.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "kernels.hpp"
#include "resident.hpp"

namespace w4a8 {

namespace {

thread_local char g_error[512] = "";

constexpr int kMaxDevices = 64;
// Work area reserved by w4a8_init: enough for every shape of the pages'
// workloads (prefill staging of 512 x 8192 is 4.7 MB, decode attention over
// 32768 positions of one KV head ~2 MB); w4a8_reserve_scratch adds more.
constexpr size_t kInitialWork = 64u << 20;

// Scratch of w4a8_linear_noalloc, for callers that cannot allocate: a
// file-scope device array, so the library never allocates it; every GPU the
// library runs on holds its own copy until the process ends.  Host code never
// uses the array's name as an address (on the host it is only a stand-in):
// w4a8_init looks up the device address once per device and keeps it in
// DeviceState::noalloc.  Layout: tickets, argmax slots, then the work area.
constexpr size_t kNoallocBytes = 32u << 20;
constexpr int kNoallocTickets = 1024;
constexpr size_t kNoallocTicketBytes = kNoallocTickets * sizeof(uint32_t);
constexpr size_t kNoallocSlotBytes = kMaxArgmaxRows * kArgmaxSpread * sizeof(unsigned long long);
constexpr size_t kNoallocWorkOffset = (kNoallocTicketBytes + kNoallocSlotBytes + 255) & ~size_t{255};
static __device__ __align__(256) unsigned char scratch[kNoallocBytes];

struct DeviceState {
  bool ready = false;
  Scratch sc;
  Scratch noalloc;  // a view of this device's copy of `scratch`
  // Exchange area of the one-launch decoder layer (epoch, done and error
  // words, hand-over buffers), zeroed at init; and whether the device holds
  // all of that kernel's workgroups at once.
  uint32_t* exchange = nullptr;
  bool resident_ok = false;
  // Exchange area of decode attention's flagged-word merge (zeroed at init).
  AttnExchange attn;
  // Work areas replaced by w4a8_reserve_scratch.  They are never freed: a HIP
  // graph captured while one was current still reads and writes it.
  std::vector<void*> retired;
};
DeviceState g_dev[kMaxDevices];
bool g_any_ready = false;
std::mutex g_mutex;

int g_gemv_max_m = -1;
bool g_gemv_max_m_forced = false;
// W4A8_OPTION_RESIDENT_LAYER: the one-token decoder layer in one launch when
// the shape and the device allow it (1, the default) or as four launches (0).
int g_resident_layer = 1;

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

int library_scratch(Scratch** out) {
  DeviceState* st = nullptr;
  const int rc = current_state(&st);
  if (rc != W4A8_OK) return rc;
  *out = &st->sc;
  return W4A8_OK;
}

int require_scratch(const Scratch* sc, size_t work_bytes) {
  if (work_bytes > sc->work_bytes) {
    set_error("this call needs %zu bytes of scratch and %zu are reserved: call w4a8_reserve_scratch(%zu) first",
              work_bytes, sc->work_bytes, work_bytes);
    return W4A8_EINVAL;
  }
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
// is the fastest through M = 4 for 2048 x 2560, 2048 x 16384 and 8192 x 2048,
// but only through M = 2 for 4096 x 14336 (2^25.8 values).  From M = 2 on
// such large matrices, and above the GEMV's rows elsewhere, up to 16 rows the
// small-batch kernel beats both (4096 x 14336: 11.7 us at M = 2, against the
// GEMV's 12.8; 11.7 - 11.9 us at M = 3 - 8 and 14.8 us at M = 16, against the
// GEMM's 16.6 - 17.6 us), except where few 64-column workgroups each stream a
// long K (8192 x 2048: 32 workgroups, two rounds), which stays on the GEMM.
// W4A8_GEMV_MAX_M in the environment replaces the rule by a plain M threshold
// between GEMV and GEMM.
int auto_path(int64_t M, int64_t K, int64_t N) {
  const int lim = gemv_max_m();
  if (g_gemv_max_m_forced) return M <= lim ? W4A8_PATH_GEMV : W4A8_PATH_GEMM;
  const bool big = K * N > (int64_t{1} << 25);
  const bool batch = M <= 16 && skinny_supported(static_cast<int>(M), static_cast<int>(K), static_cast<int>(N)) &&
                     (N >= 8192 || K <= 4096);
  if (big && M >= 2 && batch) return W4A8_PATH_BATCH;
  if (M <= (big ? (lim < 2 ? lim : 2) : lim)) return W4A8_PATH_GEMV;
  return batch ? W4A8_PATH_BATCH : W4A8_PATH_GEMM;
}

namespace {

int check_weights(const w4a8_weights* w, const char* name) {
  W4A8_REQUIRE(w && w->packed_w && w->w_scales, "%s: null weights", name);
  W4A8_REQUIRE(aligned(w->packed_w, 16) && aligned(w->w_scales, 16), "%s: weights must be 16-byte aligned", name);
  return check_shape(1, w->K, w->N, 1);
}

int check_layer_shapes(int64_t M, int64_t H, const w4a8_weights* qkv, const w4a8_weights* gate_up) {
  W4A8_REQUIRE(qkv && gate_up, "null weights");
  W4A8_REQUIRE(M >= 1 && M <= 65536 && H >= 64 && H % 64 == 0 && H < (int64_t{1} << 24), "bad shape M=%lld H=%lld",
               static_cast<long long>(M), static_cast<long long>(H));
  W4A8_REQUIRE(qkv->K == H && qkv->N >= H && qkv->N < (int64_t{1} << 30) && qkv->N % 64 == 0,
               "qkv must be H x N with N >= H");
  W4A8_REQUIRE(gate_up->K == H && gate_up->N % 128 == 0 && gate_up->N >= 128 && gate_up->N < (int64_t{1} << 30),
               "gate_up must be H x 2F with 2F a multiple of 128");
  return W4A8_OK;
}

// Whether the one-token layer runs as the four fused GEMV launches.
bool layer_fused(int64_t M, int64_t H, int64_t n_qkv, int64_t n_gu) {
  return M == 1 && gemv_fused_supported(kGemvCast, true, static_cast<int>(H), static_cast<int>(n_qkv)) &&
         gemv_fused_supported(kGemvGated, true, static_cast<int>(H), static_cast<int>(n_gu));
}

// Whether every projection of the layer runs the prefill GEMM.
bool layer_all_gemm(int64_t M, int64_t H, int64_t n_qkv, int64_t n_gu) {
  return auto_path(M, H, n_qkv) == W4A8_PATH_GEMM && auto_path(M, H, H) == W4A8_PATH_GEMM &&
         auto_path(M, H, n_gu) == W4A8_PATH_GEMM && auto_path(M, n_gu / 2, H) == W4A8_PATH_GEMM;
}

// How a decoder layer of this shape runs on the device (W4A8_LAYER_*).
int layer_kernel(const DeviceState* st, int64_t M, int64_t H, int64_t n_qkv, int64_t n_gu) {
  if (layer_fused(M, H, n_qkv, n_gu)) {
    if (g_resident_layer && st->resident_ok &&
        resident::layer_supported(static_cast<int>(H), static_cast<int>(n_qkv), static_cast<int>(n_gu)))
      return W4A8_LAYER_RESIDENT;
    return W4A8_LAYER_GEMV4;
  }
  return layer_all_gemm(M, H, n_qkv, n_gu) ? W4A8_LAYER_GEMM : W4A8_LAYER_CHAIN;
}

size_t linear_scratch(int64_t M, int64_t K, int64_t N, int path) {
  if (path == W4A8_PATH_AUTO) path = auto_path(M, K, N);
  if (path == W4A8_PATH_GEMV || path == W4A8_PATH_BATCH) return 0;
  return gemm_scratch_bytes(static_cast<int>(M), static_cast<int>(K), static_cast<int>(N));
}

// Scratch of one decoder layer: every linear of it runs with the library's
// staging and split-K partials (the fused one-token launches need none).
size_t layer_scratch(int64_t M, int64_t H, int64_t n_qkv, int64_t n_gu) {
  if (layer_fused(M, H, n_qkv, n_gu)) return 0;
  const size_t a = linear_scratch(M, H, n_qkv, W4A8_PATH_AUTO), b = linear_scratch(M, H, H, W4A8_PATH_AUTO);
  const size_t c = linear_scratch(M, H, n_gu, W4A8_PATH_AUTO), d = linear_scratch(M, n_gu / 2, H, W4A8_PATH_AUTO);
  return std::max(std::max(a, b), std::max(c, d));
}

size_t norm_argmax_scratch(int64_t M, int64_t K, int64_t N) {
  if (M == 1 && gemv_fused_supported(kGemvArgmax, true, static_cast<int>(K), static_cast<int>(N))) return 0;
  return static_cast<size_t>(M) * K * 2;
}

int check_attention(int64_t n_heads, int64_t n_kv_heads, int64_t head_dim, int64_t length) {
  W4A8_REQUIRE(head_dim == 64 || head_dim == 128 || head_dim == 256, "head_dim = %lld must be 64, 128 or 256",
               static_cast<long long>(head_dim));
  W4A8_REQUIRE(n_kv_heads >= 1 && n_kv_heads <= 4096, "n_kv_heads = %lld out of range [1, 4096]",
               static_cast<long long>(n_kv_heads));
  W4A8_REQUIRE(n_heads >= n_kv_heads && n_heads % n_kv_heads == 0 && n_heads / n_kv_heads <= 8,
               "n_heads = %lld must be 1 to 8 times n_kv_heads = %lld", static_cast<long long>(n_heads),
               static_cast<long long>(n_kv_heads));
  W4A8_REQUIRE(length >= 1 && length <= (int64_t{1} << 24), "length = %lld out of range [1, 2^24]",
               static_cast<long long>(length));
  return W4A8_OK;
}

}  // namespace

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
  sc.n_tickets = kMaxTickets;
  W4A8_HIP(hipMalloc(&sc.work, kInitialWork));
  sc.work_bytes = kInitialWork;
  // This device's copy of the static scratch: its address, then its tickets
  // cleared (every launch leaves them at zero again).
  void* ptr = nullptr;
  W4A8_HIP(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
  W4A8_HIP(hipMemset(ptr, 0, kNoallocWorkOffset));
  Scratch& na = st.noalloc;
  na.base = ptr;
  na.bytes = kNoallocBytes;
  na.tickets = static_cast<uint32_t*>(ptr);
  na.n_tickets = kNoallocTickets;
  na.slots = reinterpret_cast<unsigned long long*>(static_cast<char*>(ptr) + kNoallocTicketBytes);
  na.work = static_cast<char*>(ptr) + kNoallocWorkOffset;
  na.work_bytes = kNoallocBytes - kNoallocWorkOffset;
  W4A8_HIP(hipMalloc(&st.exchange, resident::kExchangeBytes));
  W4A8_HIP(hipMemset(st.exchange, 0, resident::kExchangeBytes));
  {
    const size_t bytes = kAttnHeads * kAttnHeadWords * sizeof(uint64_t) + kAttnHeads * sizeof(uint32_t);
    void* p = nullptr;
    W4A8_HIP(hipMalloc(&p, bytes));
    W4A8_HIP(hipMemset(p, 0, bytes));
    st.attn.ll = static_cast<uint64_t*>(p);
    st.attn.epochs = reinterpret_cast<uint32_t*>(st.attn.ll + kAttnHeads * kAttnHeadWords);
    st.attn.heads = kAttnHeads;
    st.attn.error = st.exchange + resident::kErrorWord;
  }
  int blocks = 0;
  W4A8_HIP(resident::co_resident_blocks(&blocks) == W4A8_OK ? hipSuccess : hipErrorUnknown);
  st.resident_ok = blocks >= resident::kG;
  W4A8_HIP(hipDeviceSynchronize());
  st.ready = true;
  g_any_ready = true;
  return W4A8_OK;
}

int w4a8_set_option(int option, int value) {
  W4A8_REQUIRE(option == W4A8_OPTION_RESIDENT_LAYER, "unknown option %d", option);
  W4A8_REQUIRE(value == 0 || value == 1, "option %d takes 0 or 1, not %d", option, value);
  std::lock_guard<std::mutex> lock(g_mutex);
  g_resident_layer = value;
  return W4A8_OK;
}

int w4a8_get_option(int option, int* value) {
  W4A8_REQUIRE(value, "null pointer");
  W4A8_REQUIRE(option == W4A8_OPTION_RESIDENT_LAYER, "unknown option %d", option);
  *value = g_resident_layer;
  return W4A8_OK;
}

int w4a8_take_device_errors(uint32_t* errors) {
  W4A8_REQUIRE(errors, "null pointer");
  DeviceState* st = nullptr;
  const int rc = current_state(&st);
  if (rc != W4A8_OK) return rc;
  uint32_t* word = st->exchange + resident::kErrorWord;
  W4A8_HIP(hipDeviceSynchronize());
  W4A8_HIP(hipMemcpy(errors, word, sizeof(uint32_t), hipMemcpyDeviceToHost));
  W4A8_HIP(hipMemset(word, 0, sizeof(uint32_t)));
  W4A8_HIP(hipDeviceSynchronize());
  return W4A8_OK;
}

int w4a8_layer_kernel(int64_t M, int64_t H, const w4a8_weights* qkv, const w4a8_weights* gate_up, int* kernel) {
  W4A8_REQUIRE(kernel, "null pointer");
  int rc = check_layer_shapes(M, H, qkv, gate_up);
  if (rc != W4A8_OK) return rc;
  DeviceState* st = nullptr;
  rc = current_state(&st);
  if (rc != W4A8_OK) return rc;
  *kernel = layer_kernel(st, M, H, qkv->N, gate_up->N);
  return W4A8_OK;
}

int w4a8_reserve_scratch(size_t bytes) {
  W4A8_REQUIRE(bytes <= (size_t{1} << 40), "scratch of %zu bytes is beyond 2^40", bytes);
  DeviceState* st = nullptr;
  int rc = current_state(&st);
  if (rc != W4A8_OK) return rc;
  std::lock_guard<std::mutex> lock(g_mutex);
  Scratch& sc = st->sc;
  if (bytes <= sc.work_bytes) return W4A8_OK;
  const size_t rounded = (bytes + (size_t{1} << 20) - 1) & ~((size_t{1} << 20) - 1);
  void* p = nullptr;
  W4A8_HIP(hipMalloc(&p, rounded));
  st->retired.push_back(sc.work);
  sc.work = p;
  sc.work_bytes = rounded;
  return W4A8_OK;
}

int w4a8_scratch_capacity(size_t* bytes) {
  W4A8_REQUIRE(bytes, "null pointer");
  Scratch* sc = nullptr;
  const int rc = library_scratch(&sc);
  if (rc != W4A8_OK) return rc;
  *bytes = sc->work_bytes;
  return W4A8_OK;
}

namespace {
// W4A8_EINVAL unless `path` names a kernel that can run an M x K by K x N product.
int check_path(int path, int64_t M, int64_t K, int64_t N) {
  W4A8_REQUIRE(path == W4A8_PATH_AUTO || path == W4A8_PATH_GEMV || path == W4A8_PATH_GEMM ||
                   path == W4A8_PATH_BATCH,
               "unknown path %d", path);
  W4A8_REQUIRE(path != W4A8_PATH_BATCH || (M <= 16 && K % 256 == 0 && skinny_supported(static_cast<int>(M),
                                                                                       static_cast<int>(K),
                                                                                       static_cast<int>(N))),
               "W4A8_PATH_BATCH takes M <= 16 and K a multiple of 256 (M = %lld, K = %lld)",
               static_cast<long long>(M), static_cast<long long>(K));
  return W4A8_OK;
}
}  // namespace

int w4a8_linear_scratch_bytes(int64_t M, int64_t K, int64_t N, int path, size_t* bytes) {
  W4A8_REQUIRE(bytes, "null pointer");
  int rc = check_shape(M, K, N, int64_t{1} << 20);
  if (rc != W4A8_OK) return rc;
  if ((rc = check_path(path, M, K, N)) != W4A8_OK) return rc;
  *bytes = linear_scratch(M, K, N, path);
  return W4A8_OK;
}

int w4a8_decoder_layer_scratch_bytes(int64_t M, int64_t H, const w4a8_weights* qkv, const w4a8_weights* gate_up,
                                     size_t* bytes) {
  W4A8_REQUIRE(bytes, "null pointer");
  const int rc = check_layer_shapes(M, H, qkv, gate_up);
  if (rc != W4A8_OK) return rc;
  *bytes = layer_scratch(M, H, qkv->N, gate_up->N);
  return W4A8_OK;
}

int w4a8_norm_linear_argmax_scratch_bytes(int64_t M, int64_t K, int64_t N, size_t* bytes) {
  W4A8_REQUIRE(bytes, "null pointer");
  const int rc = check_shape(M, K, N, kMaxArgmaxRows);
  if (rc != W4A8_OK) return rc;
  *bytes = norm_argmax_scratch(M, K, N);
  return W4A8_OK;
}

int w4a8_mx_linear_scratch_bytes(int64_t M, int64_t K, int64_t N, size_t* bytes) {
  W4A8_REQUIRE(bytes, "null pointer");
  const int rc = check_shape(M, K, N, int64_t{1} << 20);
  if (rc != W4A8_OK) return rc;
  W4A8_REQUIRE(K % 64 == 0, "K = %lld must be a multiple of 64", static_cast<long long>(K));
  *bytes = mx_scratch_bytes(static_cast<int>(M), static_cast<int>(K));
  return W4A8_OK;
}

int w4a8_decode_attention_scratch_bytes(int64_t n_heads, int64_t n_kv_heads, int64_t head_dim, int64_t length,
                                        size_t* bytes) {
  W4A8_REQUIRE(bytes, "null pointer");
  const int rc = check_attention(n_heads, n_kv_heads, head_dim, length);
  if (rc != W4A8_OK) return rc;
  *bytes = attention_scratch_bytes(static_cast<int>(n_kv_heads), static_cast<int>(n_heads / n_kv_heads),
                                   static_cast<int>(head_dim), static_cast<int>(length));
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

namespace {
// w4a8_linear_path on the scratch `sc`, arguments already checked.
int linear_on(const uint16_t* x, const uint8_t* packed_w, const uint16_t* w_scales, int64_t M, int64_t K, int64_t N,
              float* out, int path, Scratch* sc, hipStream_t stream) {
  if (path == W4A8_PATH_AUTO) path = auto_path(M, K, N);
  const int rc = require_scratch(sc, linear_scratch(M, K, N, path));
  if (rc != W4A8_OK) return rc;
  if (path == W4A8_PATH_GEMV) {
    GemvArgs a{x, packed_w, w_scales, static_cast<int>(M), static_cast<int>(K), static_cast<int>(N),
               out, nullptr, nullptr, nullptr};
    return launch_gemv(a, 0, sc, stream);
  }
  if (path == W4A8_PATH_BATCH)
    return launch_skinny(x, packed_w, w_scales, static_cast<int>(M), static_cast<int>(K), static_cast<int>(N), out,
                         nullptr, stream);
  GemmArgs a{x, packed_w, w_scales, static_cast<int>(M), static_cast<int>(K), static_cast<int>(N), out,
             nullptr};
  return launch_gemm(a, 0, sc, stream);
}

}  // namespace

int w4a8_linear_path(const uint16_t* x, const uint8_t* packed_w, const uint16_t* w_scales, int64_t M,
                     int64_t K, int64_t N, float* out, int path, hipStream_t stream) {
  int rc = check_linear_args(x, packed_w, w_scales, M, K, N, int64_t{1} << 20);
  if (rc != W4A8_OK) return rc;
  W4A8_REQUIRE(out, "null output pointer");
  W4A8_REQUIRE(aligned(out, 16), "out must be 16-byte aligned");
  if ((rc = check_path(path, M, K, N)) != W4A8_OK) return rc;
  Scratch* sc = nullptr;
  rc = library_scratch(&sc);
  if (rc != W4A8_OK) return rc;
  return linear_on(x, packed_w, w_scales, M, K, N, out, path, sc, stream);
}

int w4a8_linear(const uint16_t* x, const uint8_t* packed_w, const uint16_t* w_scales, int64_t M,
                int64_t K, int64_t N, float* out, hipStream_t stream) {
  return w4a8_linear_path(x, packed_w, w_scales, M, K, N, out, W4A8_PATH_AUTO, stream);
}

int w4a8_linear_noalloc(const uint16_t* x, const uint8_t* packed_w, const uint16_t* w_scales, int64_t M,
                        int64_t K, int64_t N, float* out, hipStream_t stream) {
  int rc = check_linear_args(x, packed_w, w_scales, M, K, N, int64_t{1} << 20);
  if (rc != W4A8_OK) return rc;
  W4A8_REQUIRE(out, "null output pointer");
  W4A8_REQUIRE(aligned(out, 16), "out must be 16-byte aligned");
  DeviceState* st = nullptr;
  rc = current_state(&st);
  if (rc != W4A8_OK) return rc;
  const size_t need = linear_scratch(M, K, N, W4A8_PATH_AUTO);
  W4A8_REQUIRE(need <= st->noalloc.work_bytes,
               "w4a8_linear_noalloc: this call needs %zu bytes of scratch and the static scratch holds %zu", need,
               st->noalloc.work_bytes);
  return linear_on(x, packed_w, w_scales, M, K, N, out, W4A8_PATH_AUTO, &st->noalloc, stream);
}

int w4a8_noalloc_scratch_bytes(size_t* bytes) {
  W4A8_REQUIRE(bytes, "null pointer");
  *bytes = kNoallocBytes - kNoallocWorkOffset;
  return W4A8_OK;
}

int w4a8_linear_argmax(const uint16_t* x, const uint8_t* packed_w, const uint16_t* w_scales, int64_t M,
                       int64_t K, int64_t N, float* logits, int32_t* argmax, hipStream_t stream) {
  int rc = check_linear_args(x, packed_w, w_scales, M, K, N, kMaxArgmaxRows);
  if (rc != W4A8_OK) return rc;
  W4A8_REQUIRE(argmax, "null argmax pointer");
  W4A8_REQUIRE(aligned(argmax, 4), "argmax must be 4-byte aligned");
  W4A8_REQUIRE(!logits || aligned(logits, 16), "logits must be 16-byte aligned");
  Scratch* sc = nullptr;
  rc = library_scratch(&sc);
  if (rc != W4A8_OK) return rc;
  GemvArgs a{x, packed_w, w_scales, static_cast<int>(M), static_cast<int>(K), static_cast<int>(N),
             nullptr, nullptr, logits, argmax};
  return launch_gemv(a, 2, sc, stream);
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
  if ((rc = check_path(path, M, K, N)) != W4A8_OK) return rc;
  Scratch* sc = nullptr;
  rc = library_scratch(&sc);
  if (rc != W4A8_OK) return rc;
  if (path == W4A8_PATH_AUTO) path = auto_path(M, K, N);
  rc = require_scratch(sc, linear_scratch(M, K, N, path));
  if (rc != W4A8_OK) return rc;
  if (path == W4A8_PATH_BATCH)
    return launch_skinny(x, packed_w, nullptr, static_cast<int>(M), static_cast<int>(K), static_cast<int>(N),
                         nullptr, sums, stream);
  if (path == W4A8_PATH_GEMV) {
    GemvArgs a{x, packed_w, nullptr, static_cast<int>(M), static_cast<int>(K), static_cast<int>(N),
               nullptr, sums, nullptr, nullptr};
    return launch_gemv(a, 1, sc, stream);
  }
  GemmArgs a{x, packed_w, nullptr, static_cast<int>(M), static_cast<int>(K), static_cast<int>(N),
             nullptr, sums};
  return launch_gemm(a, 1, sc, stream);
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

int w4a8_decoder_layer_workspace(int64_t M, int64_t H, const w4a8_weights* qkv, const w4a8_weights* gate_up,
                                 size_t* bytes) {
  W4A8_REQUIRE(bytes, "null pointer");
  const int rc = check_layer_shapes(M, H, qkv, gate_up);
  if (rc != W4A8_OK) return rc;
  *bytes = layer_workspace(static_cast<int>(M), static_cast<int>(H), static_cast<int>(qkv->N),
                           static_cast<int>(gate_up->N)).bytes;
  return W4A8_OK;
}

int w4a8_decoder_layer_workspace_offsets(int64_t M, int64_t H, const w4a8_weights* qkv, const w4a8_weights* gate_up,
                                         size_t offsets[7]) {
  W4A8_REQUIRE(offsets, "null pointer");
  const int rc = check_layer_shapes(M, H, qkv, gate_up);
  if (rc != W4A8_OK) return rc;
  const LayerWorkspace w = layer_workspace(static_cast<int>(M), static_cast<int>(H), static_cast<int>(qkv->N),
                                           static_cast<int>(gate_up->N));
  const size_t o[7] = {w.q, w.a, w.o, w.n, w.g, w.u, w.d};
  for (int i = 0; i < 7; ++i) offsets[i] = o[i];
  return W4A8_OK;
}

namespace {
// One decoder layer on the launches other than the resident kernel (shapes
// and workspace already checked).
int run_layer(DeviceState* st, Scratch* sc, float* x, int64_t M, int64_t H, const w4a8_weights* qkv,
              const w4a8_weights* o, const w4a8_weights* gate_up, const w4a8_weights* down, float residual_scale,
              float eps, char* base, const LayerWorkspace& w, hipStream_t stream) {
  int rc = W4A8_OK;
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
  const int kernel = layer_kernel(st, M, H, qkv->N, gate_up->N);
  if (kernel == W4A8_LAYER_GEMV4) {
    // One token: four GEMV launches, with the normalisation in the prologue
    // of qkv and gate/up and the cast, residual and gated product in the
    // epilogues (the same values as the launches below, up to the summation
    // order of the norm).
    GemvArgs qa{nullptr, qkv->packed_w, qkv->w_scales, 1, Hi, static_cast<int>(qkv->N), q, nullptr, nullptr, nullptr};
    qa.xf = x;
    qa.eps = eps;
    qa.y16 = a;
    qa.n16 = Hi;
    W4A8_STEP(launch_gemv(qa, kGemvCast, sc, stream));
    // Each projection's own output also goes to the workspace (o, g and d, as
    // the nine-launch chain leaves them).
    GemvArgs oa{a, o->packed_w, o->w_scales, 1, Hi, Hi, ob, nullptr, nullptr, nullptr};
    oa.resid = x;
    oa.alpha = residual_scale;
    W4A8_STEP(launch_gemv(oa, kGemvResid, sc, stream));
    GemvArgs ga{nullptr, gate_up->packed_w, gate_up->w_scales, 1, Hi, 2 * F, g, nullptr, nullptr, nullptr};
    ga.xf = x;
    ga.eps = eps;
    ga.y16 = u;
    W4A8_STEP(launch_gemv(ga, kGemvGated, sc, stream));
    GemvArgs da{u, down->packed_w, down->w_scales, 1, F, Hi, d, nullptr, nullptr, nullptr};
    da.resid = x;
    da.alpha = residual_scale;
    W4A8_STEP(launch_gemv(da, kGemvResid, sc, stream));
    return W4A8_OK;
  }
  const int Nq = static_cast<int>(qkv->N);
  if (kernel == W4A8_LAYER_GEMM) {
    // Many rows: every projection is a prefill GEMM, and the glue kernels
    // write their fp16 results straight into the next GEMM's quantised
    // staging, so no separate quantise pre-pass runs (four launches fewer).
    GemmStaging sg{};
    W4A8_STEP(gemm_staging(Mi, Hi, Nq, sc, &sg));
    W4A8_STEP(launch_residual_norm_quant(x, nullptr, 0, 0.0f, eps, Mi, Hi, sg, stream));
    const GemmArgs qa{nullptr, qkv->packed_w, qkv->w_scales, Mi, Hi, Nq, q, nullptr};
    GemmStaging so = gemm_staging_at(a, Mi, Hi, Hi);
    if (gemm_cast_supported(Mi, Hi, Nq, Hi, so.m_pad)) {
      // The qkv GEMM quantises fp16 of its query slice into the o
      // projection's staging (in the workspace, in place of a) itself.
      W4A8_STEP(launch_gemm_staged_cast(qa, Hi, sg, so, sc, stream));
    } else {
      W4A8_STEP(launch_gemm_staged(qa, sg, sc, stream));
      W4A8_STEP(gemm_staging(Mi, Hi, Hi, sc, &so));
      W4A8_STEP(launch_cast_quant(q, qkv->N, Mi, Hi, so, stream));
    }
    // The o projection adds 0.01 * o into the residual stream in its
    // epilogue; the normalisation then reads x alone.
    GemmArgs oa{nullptr, o->packed_w, o->w_scales, Mi, Hi, Hi, nullptr, nullptr};
    oa.resid = x;
    oa.alpha = residual_scale;
    W4A8_STEP(launch_gemm_staged_resid(oa, so, sc, stream));
    W4A8_STEP(gemm_staging(Mi, Hi, 2 * F, sc, &sg));
    W4A8_STEP(launch_residual_norm_quant(x, nullptr, 0, 0.0f, eps, Mi, Hi, sg, stream));
    const GemmArgs gua{nullptr, gate_up->packed_w, gate_up->w_scales, Mi, Hi, 2 * F, g, nullptr};
    GemmStaging sd = gemm_staging_at(g, Mi, F, Hi);
    if (gemm_gated_supported(Mi, Hi, 2 * F, sd.m_pad)) {
      // The gate/up GEMM forms fp16(gate * up) and quantises it into the down
      // projection's staging (in the workspace, in place of g) itself.
      W4A8_STEP(launch_gemm_staged_gated(gua, sg, sd, sc, stream));
    } else {
      W4A8_STEP(launch_gemm_staged(gua, sg, sc, stream));
      W4A8_STEP(gemm_staging(Mi, F, Hi, sc, &sd));
      W4A8_STEP(launch_gated_quant(g, Mi, F, sd, stream));
    }
    // The down projection adds 0.01 * d straight into the residual stream in
    // its epilogue (the same fma per element as a separate residual add).
    GemmArgs da{nullptr, down->packed_w, down->w_scales, Mi, F, Hi, nullptr, nullptr};
    da.resid = x;
    da.alpha = residual_scale;
    W4A8_STEP(launch_gemm_staged_resid(da, sd, sc, stream));
    return W4A8_OK;
  }
  W4A8_STEP(launch_residual_norm_cast(x, nullptr, 0, 0.0f, eps, Mi, Hi, n, stream));
  W4A8_STEP(linear_on(n, qkv->packed_w, qkv->w_scales, M, H, qkv->N, q, W4A8_PATH_AUTO, sc, stream));
  W4A8_STEP(launch_cast_rows(q, qkv->N, Mi, Hi, a, stream));
  W4A8_STEP(linear_on(a, o->packed_w, o->w_scales, M, H, H, ob, W4A8_PATH_AUTO, sc, stream));
  W4A8_STEP(launch_residual_norm_cast(x, ob, H, residual_scale, eps, Mi, Hi, n, stream));
  W4A8_STEP(linear_on(n, gate_up->packed_w, gate_up->w_scales, M, H, gate_up->N, g, W4A8_PATH_AUTO, sc, stream));
  W4A8_STEP(launch_gated_cast(g, Mi, F, u, stream));
  W4A8_STEP(linear_on(u, down->packed_w, down->w_scales, M, F, H, d, W4A8_PATH_AUTO, sc, stream));
  W4A8_STEP(launch_residual_norm_cast(x, d, H, residual_scale, eps, Mi, Hi, nullptr, stream));
#undef W4A8_STEP
  return W4A8_OK;
}

}  // namespace

int w4a8_decoder_layer(float* x, int64_t M, int64_t H, const w4a8_weights* qkv, const w4a8_weights* o,
                       const w4a8_weights* gate_up, const w4a8_weights* down, float residual_scale, float eps,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const w4a8_weights layer[4] = {qkv ? *qkv : w4a8_weights{}, o ? *o : w4a8_weights{},
                                 gate_up ? *gate_up : w4a8_weights{}, down ? *down : w4a8_weights{}};
  W4A8_REQUIRE(qkv && o && gate_up && down, "null weights");
  return w4a8_decoder_stack(x, M, H, layer, 1, residual_scale, eps, workspace, workspace_bytes, stream);
}

int w4a8_decoder_stack(float* x, int64_t M, int64_t H, const w4a8_weights* layers, int64_t n_layers,
                       float residual_scale, float eps, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  W4A8_REQUIRE(x && aligned(x, 16), "x must be a 16-byte aligned pointer");
  W4A8_REQUIRE(layers, "null layers");
  W4A8_REQUIRE(n_layers >= 1 && n_layers <= (int64_t{1} << 20), "n_layers = %lld out of range [1, 2^20]",
               static_cast<long long>(n_layers));
  const w4a8_weights* qkv0 = &layers[0];
  const w4a8_weights* gu0 = &layers[2];
  int rc = check_layer_shapes(M, H, qkv0, gu0);
  if (rc != W4A8_OK) return rc;
  // Every layer is checked before the first launch, so a rejected call leaves x untouched.
  for (int64_t l = 0; l < n_layers; ++l) {
    const w4a8_weights* qkv = &layers[4 * l];
    const w4a8_weights* o = &layers[4 * l + 1];
    const w4a8_weights* gate_up = &layers[4 * l + 2];
    const w4a8_weights* down = &layers[4 * l + 3];
    if ((rc = check_weights(qkv, "qkv")) != W4A8_OK || (rc = check_weights(o, "o")) != W4A8_OK ||
        (rc = check_weights(gate_up, "gate_up")) != W4A8_OK || (rc = check_weights(down, "down")) != W4A8_OK)
      return rc;
    W4A8_REQUIRE(qkv->K == H && qkv->N == qkv0->N && gate_up->K == H && gate_up->N == gu0->N,
                 "layer %lld: every layer must have the shapes of layer 0", static_cast<long long>(l));
    W4A8_REQUIRE(o->K == H && o->N == H, "layer %lld: o must be H x H", static_cast<long long>(l));
    W4A8_REQUIRE(down->K == gate_up->N / 2 && down->N == H, "layer %lld: gate_up must be H x 2F and down F x H",
                 static_cast<long long>(l));
  }
  const LayerWorkspace w = layer_workspace(static_cast<int>(M), static_cast<int>(H), static_cast<int>(qkv0->N),
                                           static_cast<int>(gu0->N));
  W4A8_REQUIRE(workspace && aligned(workspace, 256) && workspace_bytes >= w.bytes,
               "workspace must be 256-byte aligned and hold %zu bytes", w.bytes);
  Scratch* sc = nullptr;
  rc = library_scratch(&sc);
  if (rc != W4A8_OK) return rc;
  rc = require_scratch(sc, layer_scratch(M, H, qkv0->N, gu0->N));
  if (rc != W4A8_OK) return rc;
  DeviceState* st = nullptr;
  rc = current_state(&st);
  if (rc != W4A8_OK) return rc;
  char* base = static_cast<char*>(workspace);
  if (layer_kernel(st, M, H, qkv0->N, gu0->N) == W4A8_LAYER_RESIDENT) {
    // One token through up to resident::kMaxStack layers per launch of
    // resident workgroups (the same values as the four GEMV launches per
    // layer, bit for bit).
    resident::StackArgs ra{};
    ra.x = x;
    ra.n_qkv = static_cast<int>(qkv0->N);
    ra.alpha = residual_scale;
    ra.eps = eps;
    ra.q = reinterpret_cast<float*>(base + w.q);
    ra.a = reinterpret_cast<uint16_t*>(base + w.a);
    ra.o = reinterpret_cast<float*>(base + w.o);
    ra.g = reinterpret_cast<float*>(base + w.g);
    ra.u = reinterpret_cast<uint16_t*>(base + w.u);
    ra.d = reinterpret_cast<float*>(base + w.d);
    ra.exchange = st->exchange;
    for (int64_t l0 = 0; l0 < n_layers; l0 += resident::kMaxStack) {
      ra.n_layers = static_cast<int>(std::min<int64_t>(resident::kMaxStack, n_layers - l0));
      for (int i = 0; i < ra.n_layers; ++i) {
        const w4a8_weights* lw = &layers[4 * (l0 + i)];
        ra.w[i] = {lw[0].packed_w, lw[0].w_scales, lw[1].packed_w, lw[1].w_scales,
                   lw[2].packed_w, lw[2].w_scales, lw[3].packed_w, lw[3].w_scales};
      }
      rc = resident::launch_stack(ra, stream);
      if (rc != W4A8_OK) return rc;
    }
    return W4A8_OK;
  }
  for (int64_t l = 0; l < n_layers; ++l) {
    rc = run_layer(st, sc, x, M, H, &layers[4 * l], &layers[4 * l + 1], &layers[4 * l + 2], &layers[4 * l + 3],
                   residual_scale, eps, base, w, stream);
    if (rc != W4A8_OK) return rc;
  }
  return W4A8_OK;
}


int w4a8_decoder_layer_attention(float* x, int64_t H, const w4a8_weights* qkv, const w4a8_weights* o,
                                 const w4a8_weights* gate_up, const w4a8_weights* down, float residual_scale,
                                 float eps, uint16_t* k_cache, uint16_t* v_cache, int64_t n_heads, int64_t n_kv_heads,
                                 int64_t head_dim, int64_t length, int64_t capacity, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  W4A8_REQUIRE(x && aligned(x, 16), "x must be a 16-byte aligned pointer");
  int rc = check_layer_shapes(1, H, qkv, gate_up);
  if (rc != W4A8_OK) return rc;
  if ((rc = check_weights(qkv, "qkv")) != W4A8_OK || (rc = check_weights(o, "o")) != W4A8_OK ||
      (rc = check_weights(gate_up, "gate_up")) != W4A8_OK || (rc = check_weights(down, "down")) != W4A8_OK)
    return rc;
  W4A8_REQUIRE(o->K == H && o->N == H, "o must be H x H");
  W4A8_REQUIRE(down->K == gate_up->N / 2 && down->N == H, "gate_up must be H x 2F and down F x H");
  rc = check_attention(n_heads, n_kv_heads, head_dim, length);
  if (rc != W4A8_OK) return rc;
  W4A8_REQUIRE(k_cache && v_cache && aligned(k_cache, 16) && aligned(v_cache, 16), "caches must be 16-byte aligned");
  W4A8_REQUIRE(capacity >= 64 && capacity % 64 == 0 && capacity <= (int64_t{1} << 24) && length <= capacity,
               "capacity = %lld must be a multiple of 64 in [64, 2^24] and at least length = %lld",
               static_cast<long long>(capacity), static_cast<long long>(length));
  W4A8_REQUIRE(n_kv_heads * capacity * head_dim < (int64_t{1} << 38), "KV cache too large");
  W4A8_REQUIRE(n_heads * head_dim == H, "n_heads * head_dim = %lld must equal H = %lld",
               static_cast<long long>(n_heads * head_dim), static_cast<long long>(H));
  W4A8_REQUIRE(qkv->N == (n_heads + 2 * n_kv_heads) * head_dim,
               "qkv.N = %lld must hold the queries, one key and one value per KV head ((n_heads + 2 n_kv_heads) * "
               "head_dim = %lld)",
               static_cast<long long>(qkv->N), static_cast<long long>((n_heads + 2 * n_kv_heads) * head_dim));
  W4A8_REQUIRE(layer_fused(1, H, qkv->N, gate_up->N), "the one-token GEMV launches do not support this shape");
  const LayerWorkspace w = layer_workspace(1, static_cast<int>(H), static_cast<int>(qkv->N),
                                           static_cast<int>(gate_up->N));
  W4A8_REQUIRE(workspace && aligned(workspace, 256) && workspace_bytes >= w.bytes,
               "workspace must be 256-byte aligned and hold %zu bytes", w.bytes);
  Scratch* sc = nullptr;
  rc = library_scratch(&sc);
  if (rc != W4A8_OK) return rc;
  const int Hq = static_cast<int>(n_heads), Hkv = static_cast<int>(n_kv_heads), D = static_cast<int>(head_dim);
  rc = require_scratch(sc, attention_scratch_bytes(Hkv, Hq / Hkv, D, static_cast<int>(length)));
  if (rc != W4A8_OK) return rc;
  DeviceState* st = nullptr;
  rc = current_state(&st);
  if (rc != W4A8_OK) return rc;
  char* base = static_cast<char*>(workspace);
  float* q = reinterpret_cast<float*>(base + w.q);
  uint16_t* a = reinterpret_cast<uint16_t*>(base + w.a);
  float* ob = reinterpret_cast<float*>(base + w.o);
  float* g = reinterpret_cast<float*>(base + w.g);
  uint16_t* u = reinterpret_cast<uint16_t*>(base + w.u);
  float* d = reinterpret_cast<float*>(base + w.d);
  const int Hi = static_cast<int>(H), F = static_cast<int>(gate_up->N / 2);
  // qkv with the normalisation in its prologue: the queries, keys and values in fp32.
  GemvArgs qa{nullptr, qkv->packed_w, qkv->w_scales, 1, Hi, static_cast<int>(qkv->N), q, nullptr, nullptr, nullptr};
  qa.xf = x;
  qa.eps = eps;
  qa.n16 = 0;
  if ((rc = launch_gemv(qa, kGemvCast, sc, stream)) != W4A8_OK) return rc;
  // Attention of the new token over the cache; its fp16 output is the o projection's input.
  if ((rc = launch_decode_attention(q, q + Hq * D, q + (Hq + Hkv) * D, k_cache, v_cache, Hq, Hkv, D,
                                    static_cast<int>(length), static_cast<int>(capacity), a, sc, &st->attn,
                                    stream)) != W4A8_OK)
    return rc;
  if (layer_kernel(st, 1, H, qkv->N, gate_up->N) == W4A8_LAYER_RESIDENT) {
    // o, gate/up and down in one launch of resident workgroups, from the
    // attention output on (the same values as the three GEMV launches below,
    // bit for bit).
    resident::StackArgs ra{};
    ra.x = x;
    ra.n_qkv = static_cast<int>(qkv->N);
    ra.n_layers = 1;
    ra.alpha = residual_scale;
    ra.eps = eps;
    ra.q = q;
    ra.a = a;
    ra.o = ob;
    ra.g = g;
    ra.u = u;
    ra.d = d;
    ra.exchange = st->exchange;
    ra.o_in = a;
    ra.w[0] = {qkv->packed_w, qkv->w_scales, o->packed_w, o->w_scales,
               gate_up->packed_w, gate_up->w_scales, down->packed_w, down->w_scales};
    return resident::launch_stack(ra, stream);
  }
  GemvArgs oa{a, o->packed_w, o->w_scales, 1, Hi, Hi, ob, nullptr, nullptr, nullptr};
  oa.resid = x;
  oa.alpha = residual_scale;
  if ((rc = launch_gemv(oa, kGemvResid, sc, stream)) != W4A8_OK) return rc;
  GemvArgs ga{nullptr, gate_up->packed_w, gate_up->w_scales, 1, Hi, 2 * F, g, nullptr, nullptr, nullptr};
  ga.xf = x;
  ga.eps = eps;
  ga.y16 = u;
  if ((rc = launch_gemv(ga, kGemvGated, sc, stream)) != W4A8_OK) return rc;
  GemvArgs da{u, down->packed_w, down->w_scales, 1, F, Hi, d, nullptr, nullptr, nullptr};
  da.resid = x;
  da.alpha = residual_scale;
  return launch_gemv(da, kGemvResid, sc, stream);
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
  Scratch* sc = nullptr;
  rc = library_scratch(&sc);
  if (rc != W4A8_OK) return rc;
  rc = require_scratch(sc, norm_argmax_scratch(M, K, N));
  if (rc != W4A8_OK) return rc;
  const int Mi = static_cast<int>(M), Ki = static_cast<int>(K), Ni = static_cast<int>(N);
  if (norm_argmax_scratch(M, K, N) == 0) {
    GemvArgs a{nullptr, packed_w, w_scales, 1, Ki, Ni, nullptr, nullptr, logits, argmax};
    a.xf = x;
    a.eps = eps;
    return launch_gemv(a, kGemvArgmax, sc, stream);
  }
  // Otherwise normalise into library scratch, then the fused-argmax GEMV.
  uint16_t* y = static_cast<uint16_t*>(sc->work);
  rc = launch_residual_norm_cast(const_cast<float*>(x), nullptr, 0, 0.0f, eps, Mi, Ki, y, stream);
  if (rc != W4A8_OK) return rc;
  GemvArgs a{y, packed_w, w_scales, Mi, Ki, Ni, nullptr, nullptr, logits, argmax};
  return launch_gemv(a, kGemvArgmax, sc, stream);
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
  Scratch* sc = nullptr;
  rc = library_scratch(&sc);
  if (rc != W4A8_OK) return rc;
  return launch_mx_linear(x, packed, scales, static_cast<int>(M), static_cast<int>(K), static_cast<int>(N), out,
                          sc, stream);
}

int w4a8_decode_attention(const float* q, const float* k_new, const float* v_new, uint16_t* k_cache,
                          uint16_t* v_cache, int64_t n_heads, int64_t n_kv_heads, int64_t head_dim, int64_t length,
                          int64_t capacity, uint16_t* out, hipStream_t stream) {
  W4A8_REQUIRE(q && k_new && v_new && k_cache && v_cache && out, "null pointer");
  int rc = check_attention(n_heads, n_kv_heads, head_dim, length);
  if (rc != W4A8_OK) return rc;
  W4A8_REQUIRE(capacity >= 64 && capacity % 64 == 0 && capacity <= (int64_t{1} << 24),
               "capacity = %lld must be a multiple of 64 in [64, 2^24]", static_cast<long long>(capacity));
  W4A8_REQUIRE(length <= capacity, "length = %lld out of range [1, capacity = %lld]",
               static_cast<long long>(length), static_cast<long long>(capacity));
  W4A8_REQUIRE(n_kv_heads * capacity * head_dim < (int64_t{1} << 38), "KV cache too large");
  W4A8_REQUIRE(aligned(q, 16) && aligned(k_new, 16) && aligned(v_new, 16) && aligned(out, 16) &&
                   aligned(k_cache, 16) && aligned(v_cache, 16),
               "every pointer must be 16-byte aligned");
  const int Hq = static_cast<int>(n_heads), Hkv = static_cast<int>(n_kv_heads), D = static_cast<int>(head_dim);
  const int Li = static_cast<int>(length), cap = static_cast<int>(capacity);
  Scratch* sc = nullptr;
  rc = library_scratch(&sc);
  if (rc != W4A8_OK) return rc;
  DeviceState* st = nullptr;
  rc = current_state(&st);
  if (rc != W4A8_OK) return rc;
  return launch_decode_attention(q, k_new, v_new, k_cache, v_cache, Hq, Hkv, D, Li, cap, out, sc, &st->attn, stream);
}

int w4a8_gemv_max_m(void) { return gemv_max_m(); }

int w4a8_auto_path(int64_t M, int64_t K, int64_t N) { return auto_path(M, K, N); }

const char* w4a8_last_error(void) { return g_error; }

}  // extern "C"
