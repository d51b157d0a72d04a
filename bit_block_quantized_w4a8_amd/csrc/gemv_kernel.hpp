// Decode-stage GEMV kernel template (instantiated by gemv*.hip).
//
// Decode-stage GEMV: few token rows, weights streamed once from HBM.
//
// The pages' decode kernel quantises activations inside the kernel so that no
// int8 copy of the activations travels through memory (ML Drift explainer on
// tech.dede.sh, section "Stage-aware optimization for large language models";
// x-techcon article, section on moving less data).  Here every workgroup
// quantises the activations it needs into LDS, then streams its weights.
//
// Work split: a workgroup owns C consecutive output columns (C = 8 .. 64) over
// all of K, so no result crosses workgroups.  Its 256 lanes form C columns x
// S = 256 / C block slots; one load instruction of a wave reads 64 / C blocks
// of C columns, i.e. 64/C runs of 16*C contiguous bytes of the K-block-major
// weights.  K is walked in chunks of 64 blocks: the weight loads of a chunk
// are issued first, the chunk's activations are quantised into LDS while they
// are in flight, and then every lane forms its blocks' int8 dot products.
// Slots are reduced with cross-lane shuffles and waves through LDS, in a fixed
// order, so results are identical from run to run.
#pragma once

#include "kernels.hpp"


namespace w4a8 {
namespace gemv_detail {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kRowsMax = 8;        // token rows per launch
constexpr int kMaxLoadsPerLane = 16;
constexpr int kMaxChunkBlocks = 256;

// 16 bytes (8 fp16) of activations for quantisation task g of a chunk:
// task g = (row m, block e / 4, quarter e % 4) with m = g / (4 nbc), e = g % (4 nbc).
__device__ __forceinline__ uint4 load_x16(const uint16_t* __restrict__ x, int K, int kb0, int nbc, int g) {
  const int m = g / (nbc * 4);
  const int e = g % (nbc * 4);
  return *reinterpret_cast<const uint4*>(x + static_cast<int64_t>(m) * K +
                                         static_cast<int64_t>(kb0) * kBlock + 8 * e);
}

__device__ __forceinline__ uint32_t atomic_add_agent(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// C: output columns per workgroup; R: weight loads per lane per chunk, so a
// chunk holds R * 256 / C blocks.  The host picks R to cover K in one chunk
// when it can (every weight load of the workgroup then in flight at once).
template <int MR, int MODE, int C, int R>
__global__ __launch_bounds__(kThreads) void gemv_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ pw, const uint16_t* __restrict__ ws,
    int M, int K, int N, float* __restrict__ out, int32_t* __restrict__ sums,
    float* __restrict__ logits, int32_t* __restrict__ argmax_out, uint32_t* __restrict__ tickets,
    unsigned long long* __restrict__ slots, int never_set) {
  constexpr int S = kThreads / C;           // block slots per round
  constexpr int kChunkBlocks = S * R;
  static_assert(kChunkBlocks <= kMaxChunkBlocks && R <= kMaxLoadsPerLane, "chunk too large");
  // Activation loads per lane per batch: every task of a full chunk, at most 8.
  constexpr int XQ = (MR * kChunkBlocks * 4 + kThreads - 1) / kThreads < 8
                         ? (MR * kChunkBlocks * 4 + kThreads - 1) / kThreads : 8;

  __shared__ uint32_t q_lds[MR][kChunkBlocks][8];  // int8 codes, 8 dwords per block
  __shared__ float s_lds[MR][kChunkBlocks];         // sx / 16 per block

  const int tid = threadIdx.x;
  const int c = tid % C;
  const int slot = tid / C;
  // Neighbouring column tiles share 128-byte lines of the weight scales (a
  // tile reads 2C bytes of them per block).  Workgroups are dealt round-robin
  // over the 8 XCDs, each with its own L2, so consecutive tiles are mapped to
  // the same XCD: otherwise every XCD would fetch the shared lines again.
  const int tiles = gridDim.x;
  const int tile = (tiles & 7) == 0 ? (blockIdx.x & 7) * (tiles >> 3) + (blockIdx.x >> 3) : blockIdx.x;
  const int n = tile * C + c;
  const int nb = K / kBlock;

  float acc[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) acc[m] = 0.0f;
  uint32_t keep = 0;

  for (int kb0 = 0; kb0 < nb; kb0 += kChunkBlocks) {
    const int nbc = min(kChunkBlocks, nb - kb0);
    // Quantisation tasks of the chunk: (row, block, quarter), 8 elements each,
    // an aligned quad of lanes per block.
    const int tasks = M * nbc * 4;

    // 1. All loads are unconditional (addresses clamped into range, surplus
    //    results discarded) so the compiler can wait for exactly the loads a
    //    step needs: the first batch of activations is issued first, then every
    //    weight load of the chunk, and quantisation starts as soon as the
    //    activations arrive while the weights are still in flight.
    uint4 xv[XQ];
#pragma unroll
    for (int j = 0; j < XQ; ++j) xv[j] = load_x16(x, K, kb0, nbc, min(j * kThreads + tid, tasks - 1));
    __builtin_amdgcn_sched_barrier(0);  // keep the activation loads ahead of the weights
    uint4 w[R];
    uint32_t s[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int bl = min(slot + r * S, nbc - 1);
      const int64_t g = static_cast<int64_t>(kb0 + bl) * N + n;
      w[r] = *reinterpret_cast<const uint4*>(pw + g * kPackedBytes);
      s[r] = MODE == 1 ? 0u : ws[g];  // the block-sum export reads no scales
    }
    __builtin_amdgcn_sched_barrier(0);

    // 2. Quantise into LDS.  The first batch is straight-line code after the
    //    loads; further batches (many rows or a long chunk) loop behind it.
    auto quantize_batch = [&](int t0) {
#pragma unroll
      for (int j = 0; j < XQ; ++j) {
        if (t0 + j * kThreads < tasks) {  // uniform: skips batches with no task
          const int g = t0 + j * kThreads + tid;
          float v[8];
          unpack_half8(xv[j], v);
          float scale;
          const uint2 codes = quantize8_group4(v, &scale);
          if (g < tasks) {
            const int m = g / (nbc * 4);
            const int e = g % (nbc * 4);
            *reinterpret_cast<uint2*>(&q_lds[m][e >> 2][2 * (e & 3)]) = codes;
            if ((e & 3) == 0) s_lds[m][e >> 2] = scale * 0.0625f;
          }
        }
      }
    };
    quantize_batch(0);
    // A use of every first-batch load outside the branches above: without it
    // the compiler sinks the loads of later batches into their branch, behind
    // the weight loads, where they would wait for every weight to arrive.
#pragma unroll
    for (int j = 0; j < XQ; ++j) keep ^= xv[j].x;
    for (int t0 = XQ * kThreads; t0 < tasks; t0 += XQ * kThreads) {
#pragma unroll
      for (int j = 0; j < XQ; ++j) xv[j] = load_x16(x, K, kb0, nbc, min(t0 + j * kThreads + tid, tasks - 1));
      quantize_batch(t0);
    }
    __syncthreads();

    // 3. Integer block dots and the fp32 epilogue.
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int bl = slot + r * S;
      if (bl < nbc) {
        const uint32_t l0 = low_nibbles_x16(w[r].x), l1 = low_nibbles_x16(w[r].y);
        const uint32_t l2 = low_nibbles_x16(w[r].z), l3 = low_nibbles_x16(w[r].w);
        const uint32_t h0 = high_nibbles_x16(w[r].x), h1 = high_nibbles_x16(w[r].y);
        const uint32_t h2 = high_nibbles_x16(w[r].z), h3 = high_nibbles_x16(w[r].w);
        const float swf = half_bits_to_float(s[r]);
        const float cst = swf * -kMagic;  // exact: sw has 11 significant bits
#pragma unroll
        for (int m = 0; m < MR; ++m) {
          if (m < M) {
            const uint4 qa = *reinterpret_cast<const uint4*>(&q_lds[m][bl][0]);
            const uint4 qb = *reinterpret_cast<const uint4*>(&q_lds[m][bl][4]);
            // a = bits(1.5 * 2^23) + 16 * I   (bytes of l*, h* hold 16 * weight)
            int a = kMagicBits;
            a = __builtin_amdgcn_sdot4(static_cast<int>(l0), static_cast<int>(qa.x), a, false);
            a = __builtin_amdgcn_sdot4(static_cast<int>(l1), static_cast<int>(qa.y), a, false);
            a = __builtin_amdgcn_sdot4(static_cast<int>(l2), static_cast<int>(qa.z), a, false);
            a = __builtin_amdgcn_sdot4(static_cast<int>(l3), static_cast<int>(qa.w), a, false);
            a = __builtin_amdgcn_sdot4(static_cast<int>(h0), static_cast<int>(qb.x), a, false);
            a = __builtin_amdgcn_sdot4(static_cast<int>(h1), static_cast<int>(qb.y), a, false);
            a = __builtin_amdgcn_sdot4(static_cast<int>(h2), static_cast<int>(qb.z), a, false);
            a = __builtin_amdgcn_sdot4(static_cast<int>(h3), static_cast<int>(qb.w), a, false);
            if (MODE == 1) {
              sums[(static_cast<int64_t>(m) * N + n) * nb + kb0 + bl] = (a - kMagicBits) >> 4;
            } else {
              // t = RN(16 * I * sw); acc += t * (sx / 16)
              const float t = fmaf(__int_as_float(a), swf, cst);
              acc[m] = fmaf(t, s_lds[m][bl], acc[m]);
            }
          }
        }
      }
    }
    __syncthreads();  // the next chunk overwrites the LDS codes
  }

  if (never_set) tickets[0] = keep;  // `never_set` is 0: the store only keeps `keep` alive
  if (MODE == 1) return;

  // Slots of one wave: lanes c, c + C, c + 2C, ... hold the same column.
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int off = C; off < 64; off <<= 1) acc[m] += __shfl_xor(acc[m], off);

  __shared__ float red[kWaves][MR][C];
  const int lane = tid & 63;
  const int wave = tid >> 6;
  if (lane < C) {
#pragma unroll
    for (int m = 0; m < MR; ++m) red[wave][m][lane] = acc[m];
  }
  __syncthreads();
  if (wave != 0) return;

  float v[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    float t = red[0][m][lane % C];
#pragma unroll
    for (int wv = 1; wv < kWaves; ++wv) t += red[wv][m][lane % C];
    v[m] = t;
  }

  if (MODE == 0) {
    if (lane < C) {
#pragma unroll
      for (int m = 0; m < MR; ++m)
        if (m < M) out[static_cast<int64_t>(m) * N + n] = v[m];
    }
    return;
  }

  // MODE 2: argmax over all columns of each row.  Keys meet in one 64-bit
  // atomic max per row; the workgroup that finishes last publishes the index
  // and clears the slots.  Every cross-workgroup access is a device-scope
  // atomic, and each atomic waits for the previous one's result.
  bool never = false;  // stays false: depends on every returned key, see below
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    if (m >= M) break;
    if (logits && lane < C) logits[static_cast<int64_t>(m) * N + n] = v[m];
    unsigned long long key = lane < C ? argmax_key(v[m], static_cast<uint32_t>(n)) : 0ull;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const unsigned long long o = __shfl_xor(key, off);
      key = o > key ? o : key;
    }
    if (lane == 0)
      never |= __hip_atomic_fetch_max(&slots[m], key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == ~0ull;
  }
  if (lane == 0) {
    // A key of a finite value is below 2^64 - 1, so `never` is false and `inc`
    // is 1; the data dependency on every returned key orders the ticket after
    // all the maxima.
    const uint32_t inc = never ? 2u : 1u;
    const uint32_t done = atomic_add_agent(&tickets[0], inc);
    if (done == gridDim.x - 1) {
      for (int m = 0; m < M; ++m) {
        const unsigned long long k =
            __hip_atomic_exchange(&slots[m], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        argmax_out[m] = static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(k & 0xFFFFFFFFull));
      }
      __hip_atomic_store(&tickets[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Column tile: the widest tile that still gives at least 512 workgroups.
// Wider tiles repeat the in-kernel quantisation of x in fewer workgroups;
// 8 columns is the narrowest that keeps every load on whole 128-byte lines.
inline int pick_columns(int N) {
  if (N / 64 >= 512) return 64;
  if (N / 32 >= 512) return 32;
  if (N / 16 >= 512) return 16;
  return 8;
}

// Weight loads per lane: enough for all K blocks in one chunk, capped by
// registers (16) and LDS (256 blocks of codes per row).
inline int pick_loads(int nb, int cols) {
  const int slots = kThreads / cols;
  int r = 2;
  while (r < kMaxLoadsPerLane && r * slots < nb && 2 * r * slots <= kMaxChunkBlocks) r *= 2;
  return r;
}

template <int MODE, int MR, int C>
int launch_rows_c(const GemvArgs& a, int rows, int loads, const uint16_t* x, float* out, int32_t* sums,
                  float* logits, int32_t* am, Scratch* sc, unsigned long long* slots, hipStream_t stream) {
  const dim3 grid(a.N / C);
  // The block-sum export, the argmax and 8-row launches use one load count per
  // tile width (surplus loads are clamped duplicates); only the decode GEMV of
  // 1, 2 and 4 rows is specialised on K, to keep the build small.
  constexpr bool kSpecialise = MODE == 0 && MR <= 4;
#define W4A8_GEMV_LAUNCH(R)                                                                                  \
  hipLaunchKernelGGL((gemv_kernel<MR, MODE, C, R>), grid, dim3(kThreads), 0, stream, x, a.packed_w, a.w_scales, \
                     rows, a.K, a.N, out, sums, logits, am, sc->tickets, slots, 0)
  if constexpr (!kSpecialise) {
    if constexpr (C == 8) W4A8_GEMV_LAUNCH(8);
    else W4A8_GEMV_LAUNCH(16);
  } else if (loads <= 2) {
    W4A8_GEMV_LAUNCH(2);
  } else if (loads <= 4) {
    W4A8_GEMV_LAUNCH(4);
  } else if constexpr (C == 8) {
    W4A8_GEMV_LAUNCH(8);  // 8 columns: 8 loads per lane already cover 256 blocks
  } else {
    if (loads <= 8) W4A8_GEMV_LAUNCH(8);
    else W4A8_GEMV_LAUNCH(16);
  }
#undef W4A8_GEMV_LAUNCH
  W4A8_HIP(hipGetLastError());
  return W4A8_OK;
}

template <int MODE, int MR>
int launch_rows_mr(const GemvArgs& a, int rows, int cols, const uint16_t* x, float* out,
                   int32_t* sums, float* logits, int32_t* am, Scratch* sc, unsigned long long* slots,
                   hipStream_t stream) {
  const int loads = pick_loads(a.K / kBlock, cols);
  if (cols == 64) return launch_rows_c<MODE, MR, 64>(a, rows, loads, x, out, sums, logits, am, sc, slots, stream);
  if (cols == 32) return launch_rows_c<MODE, MR, 32>(a, rows, loads, x, out, sums, logits, am, sc, slots, stream);
  if (cols == 16) return launch_rows_c<MODE, MR, 16>(a, rows, loads, x, out, sums, logits, am, sc, slots, stream);
  return launch_rows_c<MODE, MR, 8>(a, rows, loads, x, out, sums, logits, am, sc, slots, stream);
}

// launch_rows_mr is instantiated in gemv.hip (MODE 0, 1 row), gemv_rows.hip
// (MODE 0, 2, 4 and 8 rows) and gemv_aux.hip (block-sum export and argmax).

#define W4A8_GEMV_INSTANTIATE(MODE, MR)                                                                \
  template int launch_rows_mr<MODE, MR>(const GemvArgs&, int, int, const uint16_t*, float*, int32_t*, \
                                        float*, int32_t*, Scratch*, unsigned long long*, hipStream_t);

}  // namespace gemv_detail
}  // namespace w4a8
