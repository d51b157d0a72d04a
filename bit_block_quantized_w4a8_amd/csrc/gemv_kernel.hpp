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
// Work split: a workgroup owns C output columns (C = 8 .. 64) over all of K,
// so no result crosses workgroups.  Its T lanes (256, or 512 for some one-row
// shapes) form C columns x S = T / C block slots; one load instruction of a wave reads 64 / C blocks
// of C columns, i.e. runs of 16*C contiguous bytes of the K-block-major
// weights.  K is walked in chunks: the weight loads of a chunk are issued
// first, the chunk's activations are quantised into LDS while they are in
// flight, and then every lane forms its blocks' int8 dot products.  Slots are
// summed within 16-lane rows by DPP moves and across rows and waves through
// LDS, in a fixed order, so results are identical from run to run.
//
// Decoder-layer fusion (the pages fold residual and element-wise work into
// neighbouring operators: sciencestack summary of the ML Drift paper,
// Figure 4): with NORM the input is the fp32 residual stream x, and the
// prologue forms fp16(x / sqrt(mean(x^2) + eps)) before quantising it; the
// epilogue can also write an fp16 copy of the leading columns (kGemvCast),
// add the result into the residual stream (kGemvResid), or multiply paired
// gate and up columns (kGemvGated: a workgroup owns C/2 columns f and their
// partners N/2 + f).
#pragma once

#include "kernels.hpp"


namespace w4a8 {
namespace gemv_detail {

constexpr int kThreads = 256;      // default workgroup size
constexpr int kWideThreads = 512;  // some one-row shapes (see pick_plan)
constexpr int kRowsMax = 8;        // token rows per launch
constexpr int kMaxLoadsPerLane = 16;
constexpr int kMaxChunkBlocks = 256;

// Task g of a chunk (8 activations) -> row m and 8-element group e of the
// chunk: m = g / (4 nbc), e = g % (4 nbc).  Tasks never reach row MR, so m is
// counted with MR - 1 comparisons instead of an integer division by a runtime
// size (about 40 instructions ahead of the first load); one-row kernels
// (MR = 1) use g directly.
template <int MR>
__device__ __forceinline__ int task_row(int g, int nbc) {
  int m = 0;
#pragma unroll
  for (int i = 1; i < MR; ++i) m += g >= i * (nbc * 4) ? 1 : 0;
  return m;
}
template <int MR>
__device__ __forceinline__ int task_group(int g, int nbc) { return g - task_row<MR>(g, nbc) * (nbc * 4); }

// 16 bytes (8 fp16) of activations for quantisation task g of a chunk:
// task g = (row m, block e / 4, quarter e % 4).
template <int MR>
__device__ __forceinline__ uint4 load_x16(const uint16_t* __restrict__ x, int K, int kb0, int nbc, int g) {
  const int m = task_row<MR>(g, nbc);
  const int e = task_group<MR>(g, nbc);
  return *reinterpret_cast<const uint4*>(x + static_cast<int64_t>(m) * K +
                                         static_cast<int64_t>(kb0) * kBlock + 8 * e);
}

__device__ __forceinline__ uint32_t atomic_add_agent(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// DPP move within 16-lane rows (no LDS traffic); out-of-row sources read 0.
template <int kCtrl>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), kCtrl, 0xF, 0xF, true));
}

// Sum over the lanes of each 16-lane row that share lane % P (P = 1, 2, 4, 8 or
// 16): afterwards every lane holds its row's sum for its residue.  The same
// additions run in every row, so the lanes a caller reads give fixed results.
template <int P>
__device__ __forceinline__ float row_sum(float v) {
  if constexpr (P < 2) v += dpp_move<0xB1>(v);   // quad_perm [1,0,3,2]: lane ^ 1
  if constexpr (P < 4) v += dpp_move<0x4E>(v);   // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (P < 8) v += dpp_move<0x124>(v);  // row_ror 4
  if constexpr (P < 16) v += dpp_move<0x128>(v); // row_ror 8
  return v;
}

// row_sum<1> on fp64 values: the same DPP pattern on both halves.
template <int kCtrl>
__device__ __forceinline__ double dpp_move_f64(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = __builtin_amdgcn_mov_dpp(static_cast<int>(static_cast<uint32_t>(b)), kCtrl, 0xF, 0xF, true);
  const uint32_t hi = __builtin_amdgcn_mov_dpp(static_cast<int>(static_cast<uint32_t>(b >> 32)), kCtrl, 0xF, 0xF, true);
  return __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
}
__device__ __forceinline__ double row_sum_f64(double v) {
  v += dpp_move_f64<0xB1>(v);
  v += dpp_move_f64<0x4E>(v);
  v += dpp_move_f64<0x124>(v);
  v += dpp_move_f64<0x128>(v);
  return v;
}

// Output column of lane column c in tile `tile`.
template <int MODE, int C>
__device__ __forceinline__ int column_of(int tile, int c, int N) {
  if constexpr (MODE == kGemvGated) {
    constexpr int kHalf = C / 2;
    return c < kHalf ? tile * kHalf + c : N / 2 + tile * kHalf + (c - kHalf);
  } else {
    return tile * C + c;
  }
}

// C: output columns per workgroup; R: weight loads per lane per chunk, so a
// chunk holds R * 256 / C blocks.  The host picks R to cover K in one chunk
// when it can (every weight load of the workgroup then in flight at once).
// NORM: the input is the fp32 residual stream, normalised in the prologue
// (the host guarantees one chunk and one batch of quantisation tasks).
template <int MR, int MODE, int C, int R, bool NORM, int T>
__global__ __launch_bounds__(T) void gemv_kernel(GemvArgs a, uint32_t* __restrict__ tickets,
                                                 unsigned long long* __restrict__ slots, int never_set) {
  constexpr int kWaves = T / 64;
  constexpr int S = T / C;                  // block slots per round
  // Partial sums per column per wave once each 16-lane row is reduced.
  constexpr int kParts = C <= 16 ? 4 : 64 / C;
  constexpr int kChunkBlocks = S * R;
  static_assert(kChunkBlocks <= kMaxChunkBlocks && R <= kMaxLoadsPerLane, "chunk too large");
  static_assert(MODE != kGemvGated || C >= 2, "gated tiles pair columns");
  // Activation loads per lane per batch: every task of a full chunk, at most 8.
  constexpr int XQ = (MR * kChunkBlocks * 4 + T - 1) / T < 8 ? (MR * kChunkBlocks * 4 + T - 1) / T : 8;
  // The residual kernels of the one-token layer (o and down, whose fp16
  // input the previous projection has just written) quantise per wave: each
  // wave quantises exactly the blocks its own lanes multiply (its 64 / C
  // slots over the R loads), writes their codes to LDS and reads them back
  // itself, so no workgroup barrier separates the quantisation from the dot
  // products and every wave starts as soon as its own activations arrive.
  // (Measured on MI355X: the end-to-end decode gains about 2%; for the plain
  // decode GEMVs, whose input stays cached between launches, it lost.)
  constexpr bool kWaveQuant = MR == 1 && !NORM && MODE == kGemvResid;
  constexpr int kSpw = C <= 64 ? 64 / C : 1;       // block slots per wave
  constexpr int kWaveTasks = kSpw * R * 4;          // quantisation tasks per wave
  constexpr int XQW = (kWaveTasks + 63) / 64;       // per lane
  static_assert(!kWaveQuant || (C <= 64 && XQW <= 8), "per-wave quantisation");

  __shared__ uint32_t q_lds[MR][kChunkBlocks][8];  // int8 codes, 8 dwords per block
  __shared__ float s_lds[MR][kChunkBlocks];         // sx / 16 per block
  __shared__ float red[kWaves][MR][kParts][C];
  __shared__ double red_ss[NORM ? kWaves : 1][MR][4];

  const uint16_t* __restrict__ x = a.x;
  const uint8_t* __restrict__ pw = a.packed_w;
  const uint16_t* __restrict__ ws = a.w_scales;
  const int M = a.M, K = a.K, N = a.N;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c = tid % C;
  const int slot = tid / C;
  // Neighbouring column tiles share 128-byte lines of the weight scales (a
  // tile reads 2C bytes of them per block).  Workgroups are dealt round-robin
  // over the 8 XCDs, each with its own L2, so consecutive tiles are mapped to
  // the same XCD: otherwise every XCD would fetch the shared lines again.
  const int tiles = gridDim.x;
  const int tile = (tiles & 7) == 0 ? (blockIdx.x & 7) * (tiles >> 3) + (blockIdx.x >> 3) : blockIdx.x;
  const int n = column_of<MODE, C>(tile, c, N);
  const int nb = K / kBlock;

  float acc[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) acc[m] = 0.0f;
  uint32_t keep = 0;
  // The residual entries this workgroup updates, fetched before the weights
  // so that the epilogue does not wait on a memory round trip.
  float resid_in[MR];
  if constexpr (MODE == kGemvResid) {
#pragma unroll
    for (int m = 0; m < MR; ++m) resid_in[m] = a.resid[static_cast<int64_t>(min(m, M - 1)) * N + n];
  }

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
    uint4 xv[kWaveQuant && XQW > XQ ? XQW : XQ];
    // Chunk block that wave-local quantisation task t (quad t / 4) covers:
    // slot kSpw * wave + i of load r, with (i, r) = (q % kSpw, q / kSpw).
    auto wave_block = [&](int t) __attribute__((always_inline)) {
      const int q = t >> 2;
      return kSpw * wave + (q % kSpw) + (q / kSpw) * S;
    };
    float4 xa[NORM ? XQ : 1], xb[NORM ? XQ : 1];
    if constexpr (NORM) {
#pragma unroll
      for (int j = 0; j < XQ; ++j) {
        const int g = min(j * T + tid, tasks - 1);
        const int m = task_row<MR>(g, nbc);
        const int e = task_group<MR>(g, nbc);
        const float* p = a.xf + static_cast<int64_t>(m) * K + static_cast<int64_t>(kb0) * kBlock + 8 * e;
        xa[j] = *reinterpret_cast<const float4*>(p);
        xb[j] = *reinterpret_cast<const float4*>(p + 4);
      }
    } else if constexpr (kWaveQuant) {
#pragma unroll
      for (int j = 0; j < XQW; ++j) {
        const int bl = min(wave_block(j * 64 + lane), nbc - 1);
        xv[j] = *reinterpret_cast<const uint4*>(x + static_cast<int64_t>(kb0 + bl) * kBlock + 8 * (lane & 3));
      }
    } else {
#pragma unroll
      for (int j = 0; j < XQ; ++j) xv[j] = load_x16<MR>(x, K, kb0, nbc, min(j * T + tid, tasks - 1));
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the activation loads ahead of the weights
    // With 8 or more loads per lane, the weight loads go in two halves: the
    // first before the quantisation, the second after the barrier that
    // publishes the codes.  A CU accepts loads only as fast as the memory
    // system drains them, so a wave that issued all of its loads first would
    // reach the barrier late and hold every other wave's dot products back
    // until then; with the split, the dot products of the first half run while
    // the second half streams in (gate_up 2048 x 16384: 5.81 -> 5.42 us).  With
    // 2 or 4 loads per lane the split lost (qkv 3.33 -> 3.47 us, o 2.99 ->
    // 3.23 us).
    constexpr int RH = R >= 8 ? R / 2 : R;
    uint4 w[R];
    uint32_t s[R];
    auto load_weights = [&](int r) __attribute__((always_inline)) {
      const int bl = min(slot + r * S, nbc - 1);
      const int64_t g = static_cast<int64_t>(kb0 + bl) * N + n;
      w[r] = *reinterpret_cast<const uint4*>(pw + g * kPackedBytes);
      s[r] = MODE == kGemvSums ? 0u : ws[g];  // the block-sum export reads no scales
    };
#pragma unroll
    for (int r = 0; r < RH; ++r) load_weights(r);
    __builtin_amdgcn_sched_barrier(0);

    // 2. Quantise into LDS.
    auto store_codes = [&](int g, const float* v) __attribute__((always_inline)) {
      float scale;
      const uint2 codes = quantize8_group4(v, &scale);
      if (g < tasks) {
        const int m = task_row<MR>(g, nbc);
        const int e = task_group<MR>(g, nbc);
        *reinterpret_cast<uint2*>(&q_lds[m][e >> 2][2 * (e & 3)]) = codes;
        if ((e & 3) == 0) s_lds[m][e >> 2] = scale * 0.0625f;
      }
    };
    if constexpr (NORM) {
      // Sum of squares of each row (one chunk holds the whole row) in fp64:
      // per lane, then across the wave, then the waves (rms_inverse).
      double ss[MR];
#pragma unroll
      for (int m = 0; m < MR; ++m) ss[m] = 0.0;
#pragma unroll
      for (int j = 0; j < XQ; ++j) {
        const int g = j * T + tid;
        if (g < tasks) {
          const int m = task_row<MR>(g, nbc);
          double q = add_square(0.0, xa[j].x);
          q = add_square(q, xa[j].y);
          q = add_square(q, xa[j].z);
          q = add_square(q, xa[j].w);
          q = add_square(q, xb[j].x);
          q = add_square(q, xb[j].y);
          q = add_square(q, xb[j].z);
          q = add_square(q, xb[j].w);
#pragma unroll
          for (int mm = 0; mm < MR; ++mm)
            if (m == mm) ss[mm] += q;
        }
      }
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        const double rs = row_sum_f64(ss[m]);
        if ((lane & 15) == 0) red_ss[wave][m][lane >> 4] = rs;
      }
      __syncthreads();
      float inv[MR];
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        double t = 0.0;
#pragma unroll
        for (int wv = 0; wv < kWaves; ++wv)
#pragma unroll
          for (int r = 0; r < 4; ++r) t += red_ss[wv][m][r];
        inv[m] = rms_inverse(t, K, a.eps);
      }
#pragma unroll
      for (int j = 0; j < XQ; ++j) {
        if (j * T < tasks) {  // uniform
          const int g = j * T + tid;
          const int m = task_row<MR>(min(g, tasks - 1), nbc);
          float im = inv[0];
#pragma unroll
          for (int mm = 1; mm < MR; ++mm)
            if (m == mm) im = inv[mm];
          const float raw[8] = {xa[j].x, xa[j].y, xa[j].z, xa[j].w, xb[j].x, xb[j].y, xb[j].z, xb[j].w};
          float v[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) v[k] = half_bits_to_float(half_of_product(raw[k], im));
          store_codes(g, v);
        }
      }
    } else if constexpr (kWaveQuant) {
#pragma unroll
      for (int j = 0; j < XQW; ++j) {
        const int t = j * 64 + lane;
        float v[8];
        unpack_half8(xv[j], v);
        float scale;
        const uint2 codes = quantize8_group4(v, &scale);   // the whole quad takes part
        const int bl = wave_block(t);
        if (t < kWaveTasks && bl < nbc) {
          *reinterpret_cast<uint2*>(&q_lds[0][bl][2 * (lane & 3)]) = codes;
          if ((lane & 3) == 0) s_lds[0][bl] = scale * 0.0625f;
        }
      }
    } else {
      // The first batch is straight-line code after the loads; further
      // batches (many rows or a long chunk) loop behind it.
      auto quantize_batch = [&](int t0) {
#pragma unroll
        for (int j = 0; j < XQ; ++j) {
          if (t0 + j * T < tasks) {  // uniform: skips batches with no task
            float v[8];
            unpack_half8(xv[j], v);
            store_codes(t0 + j * T + tid, v);
          }
        }
      };
      quantize_batch(0);
      // A use of every first-batch load outside the branches above: without it
      // the compiler sinks the loads of later batches into their branch, behind
      // the weight loads, where they would wait for every weight to arrive.
#pragma unroll
      for (int j = 0; j < XQ; ++j) keep ^= xv[j].x;
      for (int t0 = XQ * T; t0 < tasks; t0 += XQ * T) {
#pragma unroll
        for (int j = 0; j < XQ; ++j) xv[j] = load_x16<MR>(x, K, kb0, nbc, min(t0 + j * T + tid, tasks - 1));
        quantize_batch(t0);
      }
    }
    // A wave's LDS accesses run in order, so with per-wave quantisation the
    // wave reads its own codes back without a workgroup barrier.
    if constexpr (kWaveQuant) __builtin_amdgcn_wave_barrier();
    else __syncthreads();
    // 3. Integer block dots and the fp32 epilogue, block slot r at a time
    // (the accumulation order is r = 0, 1, ..).
    auto dot_block = [&](int r) __attribute__((always_inline)) {
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
            int acc_i = kMagicBits;
            acc_i = __builtin_amdgcn_sdot4(static_cast<int>(l0), static_cast<int>(qa.x), acc_i, false);
            acc_i = __builtin_amdgcn_sdot4(static_cast<int>(l1), static_cast<int>(qa.y), acc_i, false);
            acc_i = __builtin_amdgcn_sdot4(static_cast<int>(l2), static_cast<int>(qa.z), acc_i, false);
            acc_i = __builtin_amdgcn_sdot4(static_cast<int>(l3), static_cast<int>(qa.w), acc_i, false);
            acc_i = __builtin_amdgcn_sdot4(static_cast<int>(h0), static_cast<int>(qb.x), acc_i, false);
            acc_i = __builtin_amdgcn_sdot4(static_cast<int>(h1), static_cast<int>(qb.y), acc_i, false);
            acc_i = __builtin_amdgcn_sdot4(static_cast<int>(h2), static_cast<int>(qb.z), acc_i, false);
            acc_i = __builtin_amdgcn_sdot4(static_cast<int>(h3), static_cast<int>(qb.w), acc_i, false);
            if (MODE == kGemvSums) {
              a.sums[(static_cast<int64_t>(m) * N + n) * nb + kb0 + bl] = (acc_i - kMagicBits) >> 4;
            } else {
              // t = RN(16 * I * sw); acc += t * (sx / 16)
              const float t = fmaf(__int_as_float(acc_i), swf, cst);
              acc[m] = fmaf(t, s_lds[m][bl], acc[m]);
            }
          }
        }
      }
    };
    if constexpr (RH < R) {
      // Each second-half load is followed by the dot products of a
      // first-half block, whose data has long arrived: a wave held at a load
      // (the CU accepts loads only as fast as the memory system drains them)
      // does the first half's arithmetic between its issues instead of after
      // its last one, and only the second half is left once the last data
      // arrives.
#pragma unroll
      for (int r = RH; r < R; ++r) {
        load_weights(r);
        __builtin_amdgcn_sched_barrier(0);
        dot_block(r - RH);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int r = R - RH; r < R; ++r) dot_block(r);
    } else {
#pragma unroll
      for (int r = 0; r < R; ++r) dot_block(r);
    }
    // The next chunk overwrites the LDS codes (with per-wave quantisation each
    // wave rewrites only the blocks it reads itself).
    if constexpr (kWaveQuant) __builtin_amdgcn_wave_barrier();
    else __syncthreads();
  }

  if (never_set) tickets[0] = keep;  // `never_set` is 0: the store only keeps `keep` alive
  if (MODE == kGemvSums) return;

  // Slots of one wave: lanes c, c + C, c + 2C, ... hold the same column.  They
  // are summed within each 16-lane row, and the kParts row sums of every wave
  // through LDS, in a fixed order.
#pragma unroll
  for (int m = 0; m < MR; ++m) acc[m] = row_sum<C < 16 ? C : 16>(acc[m]);
  if (C >= 16 || (lane & 15) < C) {
    const int part = C <= 16 ? lane >> 4 : lane / C;
#pragma unroll
    for (int m = 0; m < MR; ++m) red[wave][m][part][lane % C] = acc[m];
  }
  __syncthreads();
  if (wave != 0) return;

  float v[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    float t = 0.0f;
#pragma unroll
    for (int wv = 0; wv < kWaves; ++wv)
#pragma unroll
      for (int p = 0; p < kParts; ++p) t += red[wv][m][p][lane % C];
    v[m] = t;
  }

  if constexpr (MODE == kGemvOut || MODE == kGemvCast) {
    if (lane < C) {
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        if (m < M) {
          if (MODE == kGemvOut || a.out) a.out[static_cast<int64_t>(m) * N + n] = v[m];
          if (MODE == kGemvCast && n < a.n16) a.y16[static_cast<int64_t>(m) * a.n16 + n] = float_to_half_bits(v[m]);
        }
      }
    }
    return;
  }
  if constexpr (MODE == kGemvResid) {
    if (lane < C) {
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        if (m < M) {
          a.resid[static_cast<int64_t>(m) * N + n] = fmaf(a.alpha, v[m], resid_in[m]);
          if (a.out) a.out[static_cast<int64_t>(m) * N + n] = v[m];  // the projection's own output
        }
      }
    }
    return;
  }
  if constexpr (MODE == kGemvGated) {
    constexpr int kHalf = C / 2;
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      const float up = __shfl(v[m], (lane + kHalf) & 63);  // lane < C/2: its up column
      if (a.out && lane < C && m < M) a.out[static_cast<int64_t>(m) * N + n] = v[m];  // gate and up values
      if (lane < kHalf && m < M)
        a.y16[static_cast<int64_t>(m) * (N / 2) + n] = half_of_product(v[m], up);
    }
    return;
  }

  // kGemvArgmax: argmax over all columns of each row.  Each workgroup folds
  // its best key into one of kArgmaxSpread slots of the row with an atomic
  // max whose result it does not wait for; argmax_finalize_kernel, launched
  // next on the stream, reduces the slots, publishes the index and clears them.
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    if (m >= M) break;
    if (a.logits && lane < C) a.logits[static_cast<int64_t>(m) * N + n] = v[m];
    unsigned long long key = lane < C ? argmax_key(v[m], static_cast<uint32_t>(n)) : 0ull;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const unsigned long long o = __shfl_xor(key, off);
      key = o > key ? o : key;
    }
    if (lane == 0)
      __hip_atomic_fetch_max(&slots[m * kArgmaxSpread + (tile & (kArgmaxSpread - 1))], key, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Launch shape: C columns per workgroup, T threads, R weight loads per lane.
struct Plan {
  int cols, threads, loads;
};

// Weight loads per lane: enough for all K blocks in one chunk, capped by
// registers (16, or 8 in 512-thread workgroups, where 16 ran slower than two
// chunks) and LDS (256 blocks of codes per row).
inline int pick_loads(int nb, int cols, int threads) {
  const int slots = threads / cols;
  const int cap = threads == kWideThreads ? 8 : kMaxLoadsPerLane;
  int r = 2;
  while (r < cap && r * slots < nb && 2 * r * slots <= kMaxChunkBlocks) r *= 2;
  return r;
}

// Column tile: the widest that still gives at least 512 workgroups.  Wider
// tiles repeat the in-kernel quantisation of x in fewer workgroups; 8 columns
// is the narrowest that keeps every load on whole 128-byte lines.  One-row
// kernels (`wide`) also take 512-thread workgroups: of 64 columns when that
// gives 256..511 workgroups (half as many quantisations of x as 32-column
// tiles, the same lanes per column), and of 8 columns over more than 4096 K
// (every lane then quantises and multiplies half as many blocks).
inline Plan pick_plan(int K, int N, bool wide) {
  int cols = 8, threads = kThreads;
  if (N / 64 >= 512) cols = 64;
  else if (wide && N / 64 >= 256) cols = 64, threads = kWideThreads;
  else if (N / 32 >= 512) cols = 32;
  else if (N / 16 >= 512) cols = 16;
  else if (wide && K > 4096) threads = kWideThreads;
  return {cols, threads, pick_loads(K / kBlock, cols, threads)};
}

// Kernels specialised on K (one chunk when it fits): the decode GEMV of 1, 2
// and 4 rows and the fused one-row kernels.  The block-sum export, the argmax
// of fp16 rows and 8-row launches use one load count per tile width (surplus
// loads are clamped duplicates).
template <int MODE, int MR, bool NORM>
constexpr bool kSpecialised = (MODE == kGemvOut && MR <= 4) || NORM || MODE >= kGemvCast;
// 512-thread workgroups: one-row kernels specialised on K.
template <int MODE, int MR, bool NORM>
constexpr bool kWideOk = MR == 1 && kSpecialised<MODE, MR, NORM>;

// `a` already points at the launch's first row.
template <int MODE, int MR, int C, bool NORM, int T>
int launch_rows_ct(const GemvArgs& a, int loads, Scratch* sc, unsigned long long* slots, hipStream_t stream) {
  const dim3 grid(a.N / C);
#define W4A8_GEMV_LAUNCH(R) \
  hipLaunchKernelGGL((gemv_kernel<MR, MODE, C, R, NORM, T>), grid, dim3(T), 0, stream, a, sc->tickets, slots, 0)
  if constexpr (!kSpecialised<MODE, MR, NORM>) {
    if constexpr (C == 8) W4A8_GEMV_LAUNCH(8);
    else W4A8_GEMV_LAUNCH(16);
  } else if (loads <= 2) {
    W4A8_GEMV_LAUNCH(2);
  } else if (loads <= 4) {
    W4A8_GEMV_LAUNCH(4);
  } else if constexpr (C == 8 && T == kThreads) {
    W4A8_GEMV_LAUNCH(8);  // 8 columns: 8 loads per lane already cover 256 blocks
  } else if constexpr (T == kThreads) {
    if (loads <= 8) W4A8_GEMV_LAUNCH(8);
    else W4A8_GEMV_LAUNCH(16);
  } else if constexpr (C > 8) {
    W4A8_GEMV_LAUNCH(8);  // pick_loads caps 512-thread workgroups at 8
  } else {
    return hip_fail(hipErrorInvalidValue, "gemv: no wide-workgroup kernel for this K");
  }
#undef W4A8_GEMV_LAUNCH
  W4A8_HIP(hipGetLastError());
  return W4A8_OK;
}

// Blocks one launch of the plan covers per chunk (the R it launches above).
inline int chunk_blocks(const Plan& p) {
  const int r = p.loads <= 2 ? 2 : p.loads <= 4 ? 4 : p.cols == 8 || p.threads == kWideThreads ? 8 : p.loads;
  return p.threads / p.cols * r;
}

template <int MODE, int MR, int C, bool NORM>
int launch_rows_c(const GemvArgs& a, const Plan& p, Scratch* sc, unsigned long long* slots, hipStream_t stream) {
  if constexpr (kWideOk<MODE, MR, NORM> && (C == 8 || C == 64)) {
    if (p.threads == kWideThreads) return launch_rows_ct<MODE, MR, C, NORM, kWideThreads>(a, p.loads, sc, slots, stream);
  }
  return launch_rows_ct<MODE, MR, C, NORM, kThreads>(a, p.loads, sc, slots, stream);
}

template <int MODE, int MR, bool NORM>
int launch_rows_mr(const GemvArgs& a, Scratch* sc, unsigned long long* slots, hipStream_t stream) {
  const Plan p = pick_plan(a.K, a.N, kWideOk<MODE, MR, NORM>);
  if (p.cols == 64) return launch_rows_c<MODE, MR, 64, NORM>(a, p, sc, slots, stream);
  if (p.cols == 32) return launch_rows_c<MODE, MR, 32, NORM>(a, p, sc, slots, stream);
  if (p.cols == 16) return launch_rows_c<MODE, MR, 16, NORM>(a, p, sc, slots, stream);
  return launch_rows_c<MODE, MR, 8, NORM>(a, p, sc, slots, stream);
}

// launch_rows_mr is instantiated in gemv.hip (decode GEMV, 1 row), gemv_rows.hip
// (2, 4 and 8 rows), gemv_aux.hip (block-sum export and argmax) and
// gemv_fused.hip (the one-row decoder-layer kernels).

#define W4A8_GEMV_INSTANTIATE(MODE, MR, NORM)                                                      \
  template int launch_rows_mr<MODE, MR, NORM>(const GemvArgs&, Scratch*, unsigned long long*, \
                                              hipStream_t);

}  // namespace gemv_detail
}  // namespace w4a8
