// Decode-stage GEMV: few token rows, weights streamed once from HBM.
//
// The pages' decode kernel quantises activations inside the kernel so that no
// int8 copy of the activations travels through memory (ML Drift explainer on
// tech.dede.sh, section "Stage-aware optimization for large language models";
// x-techcon article, section on moving less data).  Here every wave quantises
// the activation blocks it consumes, in registers, and broadcasts the codes to
// its lanes with v_readlane; weights arrive as one 16-byte load per lane per
// block, so a wave reads 1 KiB of contiguous packed weights per block.
//
// Grid: x = column tile of 64 (one column per lane), y = split of the K
// blocks.  Each of the 4 waves of a workgroup takes `bpw` consecutive blocks of
// its split.  Waves are reduced through LDS in a fixed order; splits are
// reduced by the last workgroup to finish its tile (a completion ticket), in
// split order, so results are identical from run to run.
#include "kernels.hpp"

namespace w4a8 {

namespace {

constexpr int kWaves = 4;
constexpr int kRowsMax = 8;   // token rows per launch
constexpr int kChunk = 8;     // blocks quantised per wave per pass: 8 lanes per block

__device__ __forceinline__ int bcast(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }

template <int MR, int MODE>
__global__ __launch_bounds__(256) void gemv_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ pw, const uint16_t* __restrict__ ws,
    int M, int K, int N, int bpw, float* __restrict__ out, int32_t* __restrict__ sums,
    float* __restrict__ logits, int32_t* __restrict__ argmax_out, float* __restrict__ partials,
    uint32_t* __restrict__ tickets, unsigned long long* __restrict__ slots) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int tile = blockIdx.x;
  const int split = blockIdx.y;
  const int ksplit = gridDim.y;
  const int n = tile * 64 + lane;
  const int nb = K / kBlock;
  const int b_begin = (split * kWaves + wave) * bpw;
  const int b_end = min(b_begin + bpw, nb);

  float acc[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) acc[m] = 0.0f;

  for (int cb = b_begin; cb < b_end; cb += kChunk) {
    const int cnt = min(kChunk, b_end - cb);

    // Weights and scales of up to 8 blocks, all loads issued before any use.
    uint4 w[kChunk];
    uint32_t s[kChunk];
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      if (i < cnt) {
        const int64_t g = static_cast<int64_t>(cb + i) * N + n;
        w[i] = *reinterpret_cast<const uint4*>(pw + g * kPackedBytes);
        s[i] = MODE == 1 ? 0u : ws[g];  // the block-sum export reads no scales
      } else {
        w[i] = make_uint4(0u, 0u, 0u, 0u);
        s[i] = 0u;
      }
    }

    // Quantise the activation blocks of this pass: lanes 8i .. 8i+7 hold block cb+i.
    uint32_t qd[MR];
    int sq[MR];  // sx / 16 as fp32 bits
    const int qb = cb + (lane >> 3);
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      float v[4] = {0.f, 0.f, 0.f, 0.f};
      if (m < M && qb < b_end)
        unpack_half4(*reinterpret_cast<const uint2*>(x + static_cast<int64_t>(m) * K +
                                                     static_cast<int64_t>(qb) * kBlock + 4 * (lane & 7)),
                     v);
      float scale;
      qd[m] = quantize4_group8(v[0], v[1], v[2], v[3], &scale);
      sq[m] = __float_as_int(scale * 0.0625f);
    }

#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      if (i < cnt) {
        const uint32_t l0 = low_nibbles_x16(w[i].x), l1 = low_nibbles_x16(w[i].y);
        const uint32_t l2 = low_nibbles_x16(w[i].z), l3 = low_nibbles_x16(w[i].w);
        const uint32_t h0 = high_nibbles_x16(w[i].x), h1 = high_nibbles_x16(w[i].y);
        const uint32_t h2 = high_nibbles_x16(w[i].z), h3 = high_nibbles_x16(w[i].w);
        const float swf = half_bits_to_float(s[i]);
        const float c = swf * -kMagic;  // exact: sw has 11 significant bits
#pragma unroll
        for (int m = 0; m < MR; ++m) {
          // a = bits(1.5 * 2^23) + 16 * I  (bytes of l*, h* are 16 * weight)
          int a = kMagicBits;
          const int qm = static_cast<int>(qd[m]);
          a = __builtin_amdgcn_sdot4(static_cast<int>(l0), bcast(qm, 8 * i + 0), a, false);
          a = __builtin_amdgcn_sdot4(static_cast<int>(l1), bcast(qm, 8 * i + 1), a, false);
          a = __builtin_amdgcn_sdot4(static_cast<int>(l2), bcast(qm, 8 * i + 2), a, false);
          a = __builtin_amdgcn_sdot4(static_cast<int>(l3), bcast(qm, 8 * i + 3), a, false);
          a = __builtin_amdgcn_sdot4(static_cast<int>(h0), bcast(qm, 8 * i + 4), a, false);
          a = __builtin_amdgcn_sdot4(static_cast<int>(h1), bcast(qm, 8 * i + 5), a, false);
          a = __builtin_amdgcn_sdot4(static_cast<int>(h2), bcast(qm, 8 * i + 6), a, false);
          a = __builtin_amdgcn_sdot4(static_cast<int>(h3), bcast(qm, 8 * i + 7), a, false);
          if (MODE == 1) {
            if (m < M)
              sums[(static_cast<int64_t>(m) * N + n) * nb + cb + i] = (a - kMagicBits) >> 4;
          } else {
            // t = RN(16 * I * sw); acc += t * (sx / 16)
            const float t = fmaf(__int_as_float(a), swf, c);
            acc[m] = fmaf(t, __int_as_float(bcast(sq[m], 8 * i)), acc[m]);
          }
        }
      }
    }
  }

  if (MODE == 1) return;

  __shared__ float red[kWaves][MR][64];
  __shared__ int last_flag;
#pragma unroll
  for (int m = 0; m < MR; ++m) red[wave][m][lane] = acc[m];
  __syncthreads();
  float v[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) v[m] = ((red[0][m][lane] + red[1][m][lane]) + red[2][m][lane]) + red[3][m][lane];

  if (ksplit > 1) {
    if (wave == 0) {
#pragma unroll
      for (int m = 0; m < MR; ++m)
        if (m < M) partials[(static_cast<int64_t>(split) * M + m) * N + n] = v[m];
      __threadfence();
    }
    __syncthreads();
    if (threadIdx.x == 0) last_flag = (atomicAdd(&tickets[1 + tile], 1u) == static_cast<uint32_t>(ksplit - 1));
    __syncthreads();
    if (!last_flag) return;
    __threadfence();
    if (wave == 0) {
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        float t = 0.0f;
        if (m < M)
          for (int sp = 0; sp < ksplit; ++sp) t += partials[(static_cast<int64_t>(sp) * M + m) * N + n];
        v[m] = t;
      }
    }
    if (threadIdx.x == 0) atomicExch(&tickets[1 + tile], 0u);
  }
  if (wave != 0) return;

  if (MODE == 0) {
#pragma unroll
    for (int m = 0; m < MR; ++m)
      if (m < M) out[static_cast<int64_t>(m) * N + n] = v[m];
    return;
  }

  // MODE 2: argmax over all columns, per row.
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    if (m >= M) break;
    if (logits) logits[static_cast<int64_t>(m) * N + n] = v[m];
    unsigned long long key = argmax_key(v[m], static_cast<uint32_t>(n));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const unsigned long long o = __shfl_xor(key, off);
      key = o > key ? o : key;
    }
    if (lane == 0) atomicMax(&slots[m], key);
  }
  __threadfence();
  if (lane == 0) {
    const uint32_t done = atomicAdd(&tickets[0], 1u);
    if (done == gridDim.x - 1) {
      __threadfence();
      for (int m = 0; m < M; ++m) {
        const unsigned long long k = atomicExch(&slots[m], 0ull);
        argmax_out[m] = static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(k & 0xFFFFFFFFull));
      }
      atomicExch(&tickets[0], 0u);
    }
  }
}

struct Plan {
  int ksplit;
  int bpw;
};

Plan plan_gemv(int K, int N) {
  const int nb = K / kBlock;
  const int tiles = N / 64;
  constexpr int kTargetGroups = 1024;
  constexpr int kMinBlocksPerWave = 4;
  int ks = (kTargetGroups + tiles - 1) / tiles;
  const int ks_max = nb / (kWaves * kMinBlocksPerWave);
  if (ks > ks_max) ks = ks_max;
  if (ks < 1) ks = 1;
  int bpw = (nb + ks * kWaves - 1) / (ks * kWaves);
  ks = (nb + kWaves * bpw - 1) / (kWaves * bpw);
  return {ks, bpw};
}

template <int MODE>
int launch_rows(const GemvArgs& a, int r0, int rows, const Plan& p, Scratch* sc,
                hipStream_t stream) {
  const dim3 grid(a.N / 64, p.ksplit);
  const uint16_t* x = a.x + static_cast<int64_t>(r0) * a.K;
  float* out = a.out ? a.out + static_cast<int64_t>(r0) * a.N : nullptr;
  int32_t* sums = a.sums ? a.sums + static_cast<int64_t>(r0) * a.N * (a.K / kBlock) : nullptr;
  float* logits = a.logits ? a.logits + static_cast<int64_t>(r0) * a.N : nullptr;
  int32_t* am = a.argmax ? a.argmax + r0 : nullptr;
  float* partials = static_cast<float*>(sc->work);
  unsigned long long* slots = sc->slots + r0;
#define W4A8_GEMV_LAUNCH(MR)                                                                        \
  hipLaunchKernelGGL((gemv_kernel<MR, MODE>), grid, dim3(256), 0, stream, x, a.packed_w, a.w_scales, \
                     rows, a.K, a.N, p.bpw, out, sums, logits, am, partials, sc->tickets, slots)
  if (rows == 1) W4A8_GEMV_LAUNCH(1);
  else if (rows == 2) W4A8_GEMV_LAUNCH(2);
  else if (rows <= 4) W4A8_GEMV_LAUNCH(4);
  else W4A8_GEMV_LAUNCH(8);
#undef W4A8_GEMV_LAUNCH
  W4A8_HIP(hipGetLastError());
  return W4A8_OK;
}

}  // namespace

size_t gemv_scratch_bytes(int M, int K, int N) {
  (void)M;
  const Plan p = plan_gemv(K, N);
  return p.ksplit > 1 ? static_cast<size_t>(p.ksplit) * kRowsMax * N * sizeof(float) : 0;
}

int launch_gemv(const GemvArgs& a, int mode, hipStream_t stream) {
  const Plan p = plan_gemv(a.K, a.N);
  Scratch* sc = nullptr;
  int rc = scratch_for(gemv_scratch_bytes(a.M, a.K, a.N), &sc);
  if (rc != W4A8_OK) return rc;
  for (int r0 = 0; r0 < a.M; r0 += kRowsMax) {
    const int rows = a.M - r0 < kRowsMax ? a.M - r0 : kRowsMax;
    if (mode == 0) rc = launch_rows<0>(a, r0, rows, p, sc, stream);
    else if (mode == 1) rc = launch_rows<1>(a, r0, rows, p, sc, stream);
    else rc = launch_rows<2>(a, r0, rows, p, sc, stream);
    if (rc != W4A8_OK) return rc;
  }
  return W4A8_OK;
}

}  // namespace w4a8
