// Prefill-stage GEMM: many token rows, int8 matrix cores.
//
// The pages run a different kernel for the compute-bound prefill stage than
// for decode (ML Drift explainer on tech.dede.sh, section "Stage-aware
// optimization for large language models"; x-techcon article, section on
// moving less data).  Here a pre-pass quantises the activations once into a
// staging layout (quant.hip), and this kernel runs one
// v_mfma_i32_32x32x32_i8 per 32x32 output tile per 32-element block: K = 32 is
// exactly one quantisation block, so every MFMA yields the integer block sums
// I[n][m] of one block, which the fp32 epilogue scales by sx[m][b] and sw[n][b].
//
// Operand roles: the weights are the MFMA's A operand (rows n) and the tokens
// its B operand (columns m).  In the 32x32 result, lane l holds token column
// m = l % 32 and weight rows n = 8(r/4) + 4(l/32) + r%4 in register r, so the
// token scale is one value per lane and the 16 weight scales of a lane are
// fp16 values that v_fma_mix_f32 consumes without conversion.
//
// Operand fragments: lane half h = l / 32 of an A operand loads bytes 8h .. 8h+7
// of the 16-byte weight group of its column; their low nibbles are elements
// 8h .. 8h+7 and their high nibbles elements 16+8h .. 16+8h+7 of the block.
// The B operand of lane half h loads 16 staged bytes with the same elements in
// the same order.  The MFMA pairs byte slot s of lane half h of A with byte
// slot s of lane half h of B (checked on gfx950), so the product is the block's
// full 32-element dot product.
//
// Epilogue per element and block, with the accumulator started at the bits of
// 1.5 * 2^23 so that D = 1.5 * 2^23 + 16 * I as an fp32 number:
//   t   = fma(D, sxq, -1.5 * 2^23 * sxq) = RN(I * sxq * 16),  sxq = sx' / 16
//   acc = fma(t, sw, acc)                  (v_fma_mix_f32, sw read as fp16)
// where sx' is sx with its two lowest significand bits cleared, which makes
// 1.5 * 2^23 * sxq exact (relative change of sx below 2^-22).
#include "kernels.hpp"

namespace w4a8 {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// Per-block operands of one wave, loaded one block ahead of their use.
template <int TN, int TM>
struct Operands {
  uint2 a[TN];      // 8 packed weight bytes of this lane's column and half
  uint2 s[TN][4];   // 16 fp16 weight scales of this lane's 16 result rows
  v4i b[TM];        // 16 staged activation codes
  float sx[TM];     // activation block scale of this lane's token
};

// Loads are unconditional, with column indices clamped into range (results of
// out-of-range columns are never stored): the compiler can then count the
// loads in flight and wait only for the current block, not for the prefetch.
template <int TN, int TM, int MODE>
__device__ __forceinline__ void load_operands(Operands<TN, TM>& o, const uint8_t* __restrict__ pw,
                                              const uint16_t* __restrict__ ws,
                                              const uint8_t* __restrict__ qxs,
                                              const float* __restrict__ sxs, int b, int N, int M_pad,
                                              int n_base, int m_base, int h, int l32) {
#pragma unroll
  for (int i = 0; i < TN; ++i) {
    const int n = min(n_base + 32 * i + l32, N - 1);
    o.a[i] = *reinterpret_cast<const uint2*>(pw + (static_cast<int64_t>(b) * N + n) * kPackedBytes + 8 * h);
    if (MODE != 1) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int nq = min(n_base + 32 * i + 8 * q + 4 * h, N - 4);
        o.s[i][q] = *reinterpret_cast<const uint2*>(ws + static_cast<int64_t>(b) * N + nq);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    const int64_t row = static_cast<int64_t>(b) * M_pad + m_base + 32 * j + l32;
    o.b[j] = *reinterpret_cast<const v4i*>(qxs + row * kBlock + 16 * h);
    o.sx[j] = sxs[row];
  }
}

__device__ __forceinline__ void store_agent(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float* p) {
  return __uint_as_float(__hip_atomic_load(reinterpret_cast<uint32_t*>(const_cast<float*>(p)),
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

template <int TN, int TM, int WAVES_M, int MODE>
__global__ __launch_bounds__(256) void gemm_kernel(
    const uint8_t* __restrict__ pw, const uint16_t* __restrict__ ws, const uint8_t* __restrict__ qxs,
    const float* __restrict__ sxs, int M, int M_pad, int K, int N, int tiles_n, int tiles_m, int bps,
    float* __restrict__ out, int32_t* __restrict__ sums, float* __restrict__ partials,
    uint32_t* __restrict__ tickets) {
  constexpr int WAVES_N = 4 / WAVES_M;
  constexpr int WG_N = 32 * TN * WAVES_N;
  constexpr int WG_M = 32 * TM * WAVES_M;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wn = wave % WAVES_N;
  const int wm = wave / WAVES_N;
  const int h = lane >> 5;
  const int l32 = lane & 31;

  // Tiles sharing a weight tile (consecutive m tiles) go to the same XCD: the
  // hardware deals workgroups round-robin over the 8 XCDs.
  const int ntiles = tiles_n * tiles_m;
  int id = blockIdx.x;
  if ((ntiles & 7) == 0) id = (id & 7) * (ntiles >> 3) + (id >> 3);
  const int tn = id / tiles_m;
  const int tm = id % tiles_m;
  const int split = blockIdx.y;
  const int ksplit = gridDim.y;
  const int nb = K / kBlock;
  const int b_begin = split * bps;
  const int b_end = min(nb, b_begin + bps);
  const int n_base = tn * WG_N + wn * 32 * TN;
  const int m_base = tm * WG_M + wm * 32 * TM;

  v16i magic;
#pragma unroll
  for (int r = 0; r < 16; ++r) magic[r] = kMagicBits;

  float acc[TN][TM][16];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Two operand buffers in ping-pong: while one block is multiplied and
  // scaled, the loads of the next block are in flight.
  auto step = [&](const Operands<TN, TM>& cur, int b) {
    v4i afrag[TN];
#pragma unroll
    for (int i = 0; i < TN; ++i) {
      afrag[i][0] = static_cast<int>(low_nibbles_x16(cur.a[i].x));
      afrag[i][1] = static_cast<int>(low_nibbles_x16(cur.a[i].y));
      afrag[i][2] = static_cast<int>(high_nibbles_x16(cur.a[i].x));
      afrag[i][3] = static_cast<int>(high_nibbles_x16(cur.a[i].y));
    }
    v16i d[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j)
        d[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(afrag[i], cur.b[j], magic, 0, 0, 0);
    if (MODE == 1) {
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) {
          const int m = m_base + 32 * j + l32;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int n = n_base + 32 * i + 8 * (r / 4) + 4 * h + (r % 4);
            if (m < M && n < N)
              sums[(static_cast<int64_t>(m) * N + n) * nb + b] = (d[i][j][r] - kMagicBits) >> 4;
          }
        }
      return;
    }
    float sxq[TM], cx[TM];
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      sxq[j] = __uint_as_float(__float_as_uint(cur.sx[j]) & 0xFFFFFFFCu) * 0.0625f;
      cx[j] = sxq[j] * -kMagic;
    }
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t word = (r & 2) ? cur.s[i][r / 4].y : cur.s[i][r / 4].x;
          const float sw = half_bits_to_float((r & 1) ? (word >> 16) : (word & 0xFFFFu));
          const float t = fmaf(__int_as_float(d[i][j][r]), sxq[j], cx[j]);
          acc[i][j][r] = fmaf(t, sw, acc[i][j][r]);
        }
  };

  if (b_begin < b_end) {
    const int last = b_end - 1;
    Operands<TN, TM> buf0, buf1;
    load_operands<TN, TM, MODE>(buf0, pw, ws, qxs, sxs, b_begin, N, M_pad, n_base, m_base, h, l32);
    // sched_barrier keeps each prefetch issued before the step that hides it
    // (left alone, the scheduler sinks the loads below the arithmetic).
    for (int b = b_begin; b < b_end; b += 2) {
      load_operands<TN, TM, MODE>(buf1, pw, ws, qxs, sxs, min(b + 1, last), N, M_pad, n_base, m_base, h, l32);
      __builtin_amdgcn_sched_barrier(0);
      step(buf0, b);
      __builtin_amdgcn_sched_barrier(0);
      load_operands<TN, TM, MODE>(buf0, pw, ws, qxs, sxs, min(b + 2, last), N, M_pad, n_base, m_base, h, l32);
      __builtin_amdgcn_sched_barrier(0);
      if (b + 1 < b_end) step(buf1, b + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  if (MODE == 1) return;

  if (ksplit > 1) {
    // Partial tiles meet in library scratch.  Every access to it and to the
    // ticket is a device-scope atomic, so no cache-wide fence is needed; the
    // explicit wait makes each lane's partial stores complete before the
    // workgroup takes its ticket.
    __shared__ int last_flag;
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        const int m = m_base + 32 * j + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int n = n_base + 32 * i + 8 * (r / 4) + 4 * h + (r % 4);
          if (m < M && n < N) store_agent(partials + (static_cast<int64_t>(split) * M + m) * N + n, acc[i][j][r]);
        }
      }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0)
      last_flag = __hip_atomic_fetch_add(&tickets[1 + id], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                  static_cast<uint32_t>(ksplit - 1);
    __syncthreads();
    if (!last_flag) return;
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        const int m = m_base + 32 * j + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int n = n_base + 32 * i + 8 * (r / 4) + 4 * h + (r % 4);
          float t = 0.0f;
          if (m < M && n < N)
            for (int sp = 0; sp < ksplit; ++sp) t += load_agent(partials + (static_cast<int64_t>(sp) * M + m) * N + n);
          acc[i][j][r] = t;
        }
      }
    if (threadIdx.x == 0) __hip_atomic_store(&tickets[1 + id], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int m = m_base + 32 * j + l32;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n_base + 32 * i + 8 * q + 4 * h;
        if (m < M && n < N)
          *reinterpret_cast<float4*>(out + static_cast<int64_t>(m) * N + n) =
              make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
      }
    }
}

struct Plan {
  int tn, tm, waves_m;   // MFMA tiles per wave (n, m), waves along m
  int wg_n, wg_m;
  int tiles_n, tiles_m, m_pad;
  int ksplit, bps;
};

Plan make_plan(int tn, int tm, int waves_m, int M, int N) {
  Plan p{};
  p.tn = tn;
  p.tm = tm;
  p.waves_m = waves_m;
  p.wg_n = 32 * tn * (4 / waves_m);
  p.wg_m = 32 * tm * waves_m;
  p.tiles_n = (N + p.wg_n - 1) / p.wg_n;
  p.tiles_m = (M + p.wg_m - 1) / p.wg_m;
  p.m_pad = p.tiles_m * p.wg_m;
  return p;
}

// Largest tile that still yields a full wave of workgroups; split K only when
// even the smallest tile leaves CUs idle (split partials cost HBM traffic).
Plan plan_gemm(int M, int K, int N) {
  constexpr int kFull = 256;
  Plan p;
  if (M <= 32) {
    p = make_plan(1, 1, 1, M, N);
  } else if (M <= 64) {
    p = make_plan(2, 1, 2, M, N);
    if (p.tiles_n * p.tiles_m < kFull) p = make_plan(1, 1, 2, M, N);
  } else {
    p = make_plan(2, 2, 2, M, N);
    if (p.tiles_n * p.tiles_m < kFull) p = make_plan(1, 2, 2, M, N);
    if (p.tiles_n * p.tiles_m < kFull) p = make_plan(1, 1, 2, M, N);
  }
  const int nb = K / kBlock;
  const int tiles = p.tiles_n * p.tiles_m;
  constexpr int kMinBlocksPerSplit = 8;
  int ks = (kFull + tiles - 1) / tiles;
  const int ks_max = nb / kMinBlocksPerSplit;
  if (ks > ks_max) ks = ks_max;
  if (ks < 1) ks = 1;
  p.bps = (nb + ks - 1) / ks;
  p.ksplit = (nb + p.bps - 1) / p.bps;
  return p;
}

size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

}  // namespace

size_t gemm_scratch_bytes(int M, int K, int N) {
  const Plan p = plan_gemm(M, K, N);
  const size_t nb = K / kBlock;
  size_t bytes = align256(nb * p.m_pad * kBlock) + align256(nb * p.m_pad * sizeof(float));
  if (p.ksplit > 1) bytes += static_cast<size_t>(p.ksplit) * M * N * sizeof(float);
  return bytes;
}

int launch_gemm(const GemmArgs& a, int mode, hipStream_t stream) {
  const Plan p = plan_gemm(a.M, a.K, a.N);
  if (p.tiles_n * p.tiles_m >= kMaxTickets - 1) return hip_fail(hipErrorInvalidValue, "gemm: too many tiles");
  Scratch* sc = nullptr;
  int rc = scratch_for(gemm_scratch_bytes(a.M, a.K, a.N), &sc);
  if (rc != W4A8_OK) return rc;
  const size_t nb = a.K / kBlock;
  uint8_t* base = static_cast<uint8_t*>(sc->work);
  uint8_t* qxs = base;
  float* sxs = reinterpret_cast<float*>(base + align256(nb * p.m_pad * kBlock));
  float* partials = reinterpret_cast<float*>(base + align256(nb * p.m_pad * kBlock) +
                                             align256(nb * p.m_pad * sizeof(float)));
  rc = launch_quantize_stage(a.x, a.M, p.m_pad, a.K, qxs, sxs, stream);
  if (rc != W4A8_OK) return rc;
  const dim3 grid(p.tiles_n * p.tiles_m, p.ksplit);
#define W4A8_GEMM_LAUNCH(TN, TM, WM, MODE)                                                             \
  hipLaunchKernelGGL((gemm_kernel<TN, TM, WM, MODE>), grid, dim3(256), 0, stream, a.packed_w, a.w_scales, \
                     qxs, sxs, a.M, p.m_pad, a.K, a.N, p.tiles_n, p.tiles_m, p.bps, a.out, a.sums,       \
                     partials, sc->tickets)
  if (mode == 1) {
    if (p.waves_m == 1) W4A8_GEMM_LAUNCH(1, 1, 1, 1);
    else if (p.tn == 2 && p.tm == 2) W4A8_GEMM_LAUNCH(2, 2, 2, 1);
    else if (p.tn == 2) W4A8_GEMM_LAUNCH(2, 1, 2, 1);
    else if (p.tm == 2) W4A8_GEMM_LAUNCH(1, 2, 2, 1);
    else W4A8_GEMM_LAUNCH(1, 1, 2, 1);
  } else {
    if (p.waves_m == 1) W4A8_GEMM_LAUNCH(1, 1, 1, 0);
    else if (p.tn == 2 && p.tm == 2) W4A8_GEMM_LAUNCH(2, 2, 2, 0);
    else if (p.tn == 2) W4A8_GEMM_LAUNCH(2, 1, 2, 0);
    else if (p.tm == 2) W4A8_GEMM_LAUNCH(1, 2, 2, 0);
    else W4A8_GEMM_LAUNCH(1, 1, 2, 0);
  }
#undef W4A8_GEMM_LAUNCH
  W4A8_HIP(hipGetLastError());
  return W4A8_OK;
}

}  // namespace w4a8
