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
// Data movement: a workgroup stages each K block's operands through LDS (two
// stages): its packed weights [BN][16 B], weight scales [BN] fp16, activation
// scales [BM] fp32 and staged activation codes [BM][32 B], contiguous in
// global memory per block, are fetched by every thread as exactly two 16-byte
// loads, kDepth blocks ahead through a register ring, and written to LDS one
// step before use.  Waves read their MFMA fragments and scales from LDS, so no
// operand is fetched from global memory twice by one workgroup.
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

constexpr int kThreads = 256;
constexpr int kDepth = 4;  // K blocks in flight per thread (the ring below has four slots)

// Byte layout of one LDS stage (one K block of one workgroup tile).
template <int BN, int BM>
struct Stage {
  static constexpr int kA = 0;              // packed weights [BN][16]
  static constexpr int kSW = BN * 16;       // weight scales fp16 [BN]
  static constexpr int kSX = kSW + BN * 2;  // activation scales fp32 [BM]
  static constexpr int kB = kSX + BM * 4;   // staged activation codes [BM][32]
  static constexpr int kBytes = kB + BM * 32;
  static constexpr int kChunks = kBytes / 16;
  static_assert(kChunks <= 2 * kThreads, "at most two 16-byte chunks per thread");
};

// Global address of 16-byte chunk c of the stage for block 0, and its stride
// per block.  Column indices are clamped into range (the data of columns past
// N is loaded but never stored), so every thread issues its loads
// unconditionally and the compiler can count them.
template <int BN, int BM>
__device__ __forceinline__ void chunk_address(int c, const uint8_t* pw, const uint16_t* ws,
                                              const uint8_t* qxs, const float* sxs, int N, int M_pad,
                                              int n0, int m0, const uint8_t** base, int64_t* stride) {
  const uint8_t* pa = pw + static_cast<int64_t>(min(n0 + c, N - 1)) * kPackedBytes;
  const int cs = c - BN;
  const uint8_t* psw = reinterpret_cast<const uint8_t*>(ws + min(n0 + 8 * cs, N - 8));
  const int cx = cs - BN / 8;
  const uint8_t* psx = reinterpret_cast<const uint8_t*>(sxs + m0 + 4 * cx);
  const int cb = min(cx - BM / 4, 2 * BM - 1);
  const uint8_t* pb = qxs + static_cast<int64_t>(m0 + (cb >> 1)) * kBlock + 16 * (cb & 1);
  if (c < BN) {
    *base = pa;
    *stride = static_cast<int64_t>(N) * kPackedBytes;
  } else if (cs < BN / 8) {
    *base = psw;
    *stride = static_cast<int64_t>(N) * 2;
  } else if (cx < BM / 4) {
    *base = psx;
    *stride = static_cast<int64_t>(M_pad) * 4;
  } else {
    *base = pb;
    *stride = static_cast<int64_t>(M_pad) * kBlock;
  }
}

// Workgroup barrier that orders LDS accesses only.  __syncthreads() also
// orders global memory, which makes every wave wait for all of its loads in
// flight, draining the operand prefetch at each K block.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
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
__global__ __launch_bounds__(kThreads) void gemm_kernel(
    const uint8_t* __restrict__ pw, const uint16_t* __restrict__ ws, const uint8_t* __restrict__ qxs,
    const float* __restrict__ sxs, int M, int M_pad, int K, int N, int tiles_n, int tiles_m, int bps,
    float* __restrict__ out, int32_t* __restrict__ sums, float* __restrict__ partials,
    uint32_t* __restrict__ tickets) {
  constexpr int WAVES_N = 4 / WAVES_M;
  constexpr int BN = 32 * TN * WAVES_N;
  constexpr int BM = 32 * TM * WAVES_M;
  using St = Stage<BN, BM>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][St::kBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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
  const int n0 = tn * BN;
  const int m0 = tm * BM;
  const int n_base = n0 + wn * 32 * TN;
  const int m_base = m0 + wm * 32 * TM;

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

  // One block: fragments and scales from LDS, TN x TM MFMAs, fp32 epilogue.
  auto compute = [&](const uint8_t* st, int b) __attribute__((always_inline)) {
    v4i afrag[TN];
    uint2 sraw[TN][4];
#pragma unroll
    for (int i = 0; i < TN; ++i) {
      const int col = (wn * TN + i) * 32;
      const uint2 araw = *reinterpret_cast<const uint2*>(st + St::kA + (col + l32) * 16 + 8 * h);
      afrag[i][0] = static_cast<int>(low_nibbles_x16(araw.x));
      afrag[i][1] = static_cast<int>(low_nibbles_x16(araw.y));
      afrag[i][2] = static_cast<int>(high_nibbles_x16(araw.x));
      afrag[i][3] = static_cast<int>(high_nibbles_x16(araw.y));
#pragma unroll
      for (int q = 0; q < 4; ++q)
        sraw[i][q] = *reinterpret_cast<const uint2*>(st + St::kSW + (col + 8 * q + 4 * h) * 2);
    }
    v4i bfrag[TM];
    float sxv[TM];
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int row = (wm * TM + j) * 32 + l32;
      bfrag[j] = *reinterpret_cast<const v4i*>(st + St::kB + row * kBlock + 16 * h);
      sxv[j] = *reinterpret_cast<const float*>(st + St::kSX + row * 4);
    }
    v16i d[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j)
        d[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(afrag[i], bfrag[j], magic, 0, 0, 0);
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
      sxq[j] = __uint_as_float(__float_as_uint(sxv[j]) & 0xFFFFFFFCu) * 0.0625f;
      cx[j] = sxq[j] * -kMagic;
    }
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t word = (r & 2) ? sraw[i][r / 4].y : sraw[i][r / 4].x;
          const float sw = half_bits_to_float((r & 1) ? (word >> 16) : (word & 0xFFFFu));
          const float t = fmaf(__int_as_float(d[i][j][r]), sxq[j], cx[j]);
          acc[i][j][r] = fmaf(t, sw, acc[i][j][r]);
        }
  };

  if (b_begin < b_end) {
    const int last = b_end - 1;
    const int c0 = tid;
    const int c1 = tid + kThreads;
    const uint8_t* base0;
    const uint8_t* base1;
    int64_t stride0, stride1;
    chunk_address<BN, BM>(min(c0, St::kChunks - 1), pw, ws, qxs, sxs, N, M_pad, n0, m0, &base0, &stride0);
    chunk_address<BN, BM>(min(c1, St::kChunks - 1), pw, ws, qxs, sxs, N, M_pad, n0, m0, &base1, &stride1);

    // Register ring of kDepth = 4 blocks held in eight named variables: an
    // array (or references to one) would be placed in scratch memory.
    uint4 r0a, r0b, r1a, r1b, r2a, r2b, r3a, r3b;
#define W4A8_FETCH(A, B, BLK)                                                  \
  do {                                                                         \
    const int blk_ = (BLK);                                                    \
    A = *reinterpret_cast<const uint4*>(base0 + blk_ * stride0);               \
    B = *reinterpret_cast<const uint4*>(base1 + blk_ * stride1);               \
  } while (0)
#define W4A8_PIPE_STEP(A, B, ST, BLK)                                           \
  do {                                                                         \
    const int b_ = (BLK);                                                      \
    if (c0 < St::kChunks) *reinterpret_cast<uint4*>((ST) + c0 * 16) = A;       \
    if (c1 < St::kChunks) *reinterpret_cast<uint4*>((ST) + c1 * 16) = B;       \
    W4A8_FETCH(A, B, min(b_ + kDepth, last));                                  \
    lds_barrier();                                                             \
    if (b_ < b_end) compute((ST), b_);                                         \
  } while (0)
    W4A8_FETCH(r0a, r0b, min(b_begin + 0, last));
    W4A8_FETCH(r1a, r1b, min(b_begin + 1, last));
    W4A8_FETCH(r2a, r2b, min(b_begin + 2, last));
    W4A8_FETCH(r3a, r3b, min(b_begin + 3, last));
    for (int bb = b_begin; bb < b_end; bb += kDepth) {
      W4A8_PIPE_STEP(r0a, r0b, lds[0], bb + 0);
      W4A8_PIPE_STEP(r1a, r1b, lds[1], bb + 1);
      W4A8_PIPE_STEP(r2a, r2b, lds[0], bb + 2);
      W4A8_PIPE_STEP(r3a, r3b, lds[1], bb + 3);
    }
#undef W4A8_PIPE_STEP
#undef W4A8_FETCH
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
    p = make_plan(2, 1, 1, M, N);      // 256 x 32
  } else if (M <= 64) {
    p = make_plan(2, 1, 2, M, N);      // 128 x 64
  } else {
    p = make_plan(2, 2, 2, M, N);      // 128 x 128
    if (p.tiles_n * p.tiles_m < kFull) p = make_plan(1, 2, 2, M, N);  // 64 x 128
    if (p.tiles_n * p.tiles_m < kFull) p = make_plan(1, 1, 2, M, N);  // 64 x 64
  }
  // Fewer than two tiles per CU leave too few waves to hide latency: split K
  // towards four workgroups per CU, keeping at least 64 blocks per split (the
  // partial tiles cost HBM traffic that short splits do not amortise).
  const int nb = K / kBlock;
  const int tiles = p.tiles_n * p.tiles_m;
  constexpr int kMinBlocksPerSplit = 64;
  constexpr int kTargetGroups = 1024;
  int ks = tiles < 2 * kFull ? (kTargetGroups + tiles - 1) / tiles : 1;
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
  // Every thread stages scale chunks unconditionally; the block-sum export has
  // no scales (w_scales may be null), so it stages bytes of the packed weights
  // instead (at least as large as the scales would be) and never reads them.
  const uint16_t* ws = mode == 1 ? reinterpret_cast<const uint16_t*>(a.packed_w) : a.w_scales;
#define W4A8_GEMM_LAUNCH(TN, TM, WM, MODE)                                                             \
  hipLaunchKernelGGL((gemm_kernel<TN, TM, WM, MODE>), grid, dim3(256), 0, stream, a.packed_w, ws,        \
                     qxs, sxs, a.M, p.m_pad, a.K, a.N, p.tiles_n, p.tiles_m, p.bps, a.out, a.sums,       \
                     partials, sc->tickets)
  if (mode == 1) {
    if (p.waves_m == 1) W4A8_GEMM_LAUNCH(2, 1, 1, 1);
    else if (p.tn == 2 && p.tm == 2) W4A8_GEMM_LAUNCH(2, 2, 2, 1);
    else if (p.tn == 2) W4A8_GEMM_LAUNCH(2, 1, 2, 1);
    else if (p.tm == 2) W4A8_GEMM_LAUNCH(1, 2, 2, 1);
    else W4A8_GEMM_LAUNCH(1, 1, 2, 1);
  } else {
    if (p.waves_m == 1) W4A8_GEMM_LAUNCH(2, 1, 1, 0);
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
