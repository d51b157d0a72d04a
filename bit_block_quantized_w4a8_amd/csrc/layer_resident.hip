// One-token decoder layers in one launch: the four projections of the decode
// stage (qkv with the normalising prologue and the fp16 cast of the query
// slice, o with the residual add, gate/up with the normalising prologue and the
// gated product, down with the residual add), for one layer or a stack of up
// to 32 layers, run in one grid of workgroups that stay resident on the chip
// and hand each projection's output to the next inside the launch.
//
// Why: decode is memory-bound (ML Drift explainer on tech.dede.sh, section
// "Stage-aware optimization for large language models"), and a launch per
// projection leaves the memory idle between kernels: each launch costs a few
// microseconds of dispatch, ramp-up and drain.  The pages overlap transfers
// with compute (aigridhq article on the WebGPU kernel studio); here each
// projection's weights are requested as soon as the previous projection's
// output has been handed over, and the next layer's qkv weights while the
// current layer's down projection waits for its input.
//
// Work split: workgroup w owns the same tiles as in the four GEMV launches of
// the layer (8 columns of o and down, 32 paired gate/up columns, one or two
// 8-column qkv tiles), with the same lanes, block slots and reduction order,
// so every output equals the four-launch layer's bit for bit.  Its 768 threads
// are 8 compute waves, which hold the weights in registers and form the dot
// products, and 4 loader waves, which wait for a projection's inputs,
// normalise and quantise them into LDS and hand them over at a workgroup
// barrier.  The split keeps the compute waves' weight loads out of the way of
// the input loads: a wave's vector loads retire in issue order.
//
// Hand-over between workgroups: every word of a projection's output that the
// next projection reads is written as one 64-bit atomic store holding 32 bits
// of data and a flag, and read with 64-bit atomic loads (agent scope: coherent
// across the chip's L2 caches), so a reader that sees the flag also sees the
// data and no barrier or fence is needed.  Layer l of a launch uses the flag
// epoch + 1 + l, with the epoch word of the exchange area, which workgroup 0
// advances once every workgroup has read it.  Every wait is bounded: after
// one wait of a workgroup gives up (raising the error word), its later waits
// do not wait, so every launch ends.
#include "gemv_kernel.hpp"
#include "resident.hpp"

namespace w4a8 {
namespace resident {
namespace {

using gemv_detail::row_sum;
using gemv_detail::row_sum_f64;

constexpr int kComputeThreads = 512;
constexpr int kLoaderThreads = 256;
constexpr int kThreads = kComputeThreads + kLoaderThreads;
constexpr int kSpinLimit = 1 << 20;

// Tile of launch block `b` in a GEMV launch of `tiles` workgroups: consecutive
// tiles on one XCD (the mapping of gemv_kernel).
__device__ __forceinline__ int tile_of(int b, int tiles) {
  return (tiles & 7) == 0 ? (b & 7) * (tiles >> 3) + (b >> 3) : b;
}

__device__ __forceinline__ void ll_store(uint64_t* p, uint32_t data, uint32_t flag) {
  __hip_atomic_store(p, (static_cast<uint64_t>(flag) << 32) | data, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ll_load(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The NW words at p once all carry `flag`.  Lane 0 of the wave polls its
// first word alone (one load per round, with a short sleep) until it is
// there; then every lane polls its first word and reads its other words,
// repeating for any that is not there yet.  A wave's producers finish at
// about the same time, and polling with one lane instead of 64 keeps the
// 256 workgroups' polls from crowding the memory system that the last
// producers' stores must cross (measured on MI355X: about 4 us less per
// launch than every lane polling).  Returns false, with whatever the words
// hold, after `limit` rounds of each kind.
template <int NW>
__device__ __forceinline__ bool ll_wait(const uint64_t* p, uint32_t flag, int limit, uint32_t (&data)[NW]) {
  uint64_t v[NW] = {};
  bool ready = false;
  for (int spin = 0; spin < limit; ++spin) {
    int lead = 1;
    if ((threadIdx.x & 63) == 0) lead = static_cast<uint32_t>(ll_load(p) >> 32) == flag;
    if (__builtin_amdgcn_readfirstlane(lead)) break;
    __builtin_amdgcn_s_sleep(2);
  }
  for (int spin = 0; spin < limit; ++spin) {
    v[0] = ll_load(p);
    if (static_cast<uint32_t>(v[0] >> 32) != flag) {
      __builtin_amdgcn_s_sleep(2);
      continue;
    }
#pragma unroll
    for (int i = 1; i < NW; ++i) v[i] = ll_load(p + i);
    ready = true;
#pragma unroll
    for (int i = 1; i < NW; ++i) ready &= static_cast<uint32_t>(v[i] >> 32) == flag;
    if (ready) break;
  }
#pragma unroll
  for (int i = 0; i < NW; ++i) data[i] = static_cast<uint32_t>(v[i]);
  return ready;
}

// acc + RN(16 I sw) * (sx / 16) for one (block, column): the GEMV's block step.
// s32 is the aligned 32-bit word holding the column's fp16 scale and its
// neighbour's; `shift` (0 or 16) selects the column's half.  Loading whole
// words leaves the compiler no 16-bit value to widen next to the load (it
// would wait for the load there, long before the weights are needed), and
// the empty asm statement keeps the selection at the use.
__device__ __forceinline__ float block_step(uint4 w, uint32_t s32, int shift, const uint32_t* q, float sx16,
                                            float acc) {
  asm volatile("" : "+v"(s32));
  const uint32_t s16 = s32 >> shift;
  const uint4 qa = *reinterpret_cast<const uint4*>(q);
  const uint4 qb = *reinterpret_cast<const uint4*>(q + 4);
  int acc_i = kMagicBits;
  acc_i = __builtin_amdgcn_sdot4(static_cast<int>(low_nibbles_x16(w.x)), static_cast<int>(qa.x), acc_i, false);
  acc_i = __builtin_amdgcn_sdot4(static_cast<int>(low_nibbles_x16(w.y)), static_cast<int>(qa.y), acc_i, false);
  acc_i = __builtin_amdgcn_sdot4(static_cast<int>(low_nibbles_x16(w.z)), static_cast<int>(qa.z), acc_i, false);
  acc_i = __builtin_amdgcn_sdot4(static_cast<int>(low_nibbles_x16(w.w)), static_cast<int>(qa.w), acc_i, false);
  acc_i = __builtin_amdgcn_sdot4(static_cast<int>(high_nibbles_x16(w.x)), static_cast<int>(qb.x), acc_i, false);
  acc_i = __builtin_amdgcn_sdot4(static_cast<int>(high_nibbles_x16(w.y)), static_cast<int>(qb.y), acc_i, false);
  acc_i = __builtin_amdgcn_sdot4(static_cast<int>(high_nibbles_x16(w.z)), static_cast<int>(qb.z), acc_i, false);
  acc_i = __builtin_amdgcn_sdot4(static_cast<int>(high_nibbles_x16(w.w)), static_cast<int>(qb.w), acc_i, false);
  const float swf = half_bits_to_float(s16);
  const float t = fmaf(__int_as_float(acc_i), swf, swf * -kMagic);
  return fmaf(t, sx16, acc);
}

// The aligned 32-bit word of fp16 scales that holds scale g (and g ^ 1).
__device__ __forceinline__ uint32_t scale_word(const uint16_t* s, uint32_t g) {
  return *reinterpret_cast<const uint32_t*>(s + (g & ~1u));
}

// Sum of squares of eight fp32 values in fp64, in the GEMV prologue's order.
__device__ __forceinline__ double square_sum8(const float (&v)[8]) {
  double q = 0.0;
#pragma unroll
  for (int k = 0; k < 8; ++k) q = add_square(q, v[k]);
  return q;
}

// Quantise eight elements (task g: block g / 4, quarter g % 4) into LDS codes
// and scales; called by all 64 lanes of a wave (aligned quads per block).
__device__ __forceinline__ void quantize_task(const float (&v)[8], int g, uint32_t (*q)[8], float* s) {
  float scale;
  const uint2 codes = quantize8_group4(v, &scale);
  *reinterpret_cast<uint2*>(&q[g >> 2][2 * (g & 3)]) = codes;
  if ((g & 3) == 0) s[g >> 2] = scale * 0.0625f;
}

// LDS of one workgroup.
struct Lds {
  uint32_t q_a[kNbH][8], q_b[kNbH][8], q_c[kNbH][8], q_d[kNbF][8];  // int8 codes per block
  float s_a[kNbH], s_b[kNbH], s_c[kNbH], s_d[kNbF];                  // sx / 16 per block
  float red[512];        // per-wave partial sums of a projection
  double red_ss[4][4];   // loader partial sums of squares
  float x_res[8];        // residual entries of this workgroup's o and down columns
  float x_mid[8];        // the same after the o projection
  uint32_t flag;
};

__device__ __forceinline__ const uint64_t* exchange_words(const StackArgs& a, size_t offset) {
  return reinterpret_cast<const uint64_t*>(reinterpret_cast<const char*>(a.exchange) + offset);
}
__device__ __forceinline__ uint64_t* exchange_words_rw(const StackArgs& a, size_t offset) {
  return reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(a.exchange) + offset);
}

// Loader waves (waves 8..11): thread lt quantises task lt (block lt / 4,
// quarter lt % 4) of each 64-block input and takes block lt of the down
// projection's input.  Ten workgroup barriers per layer, matching the compute
// waves'.
__device__ __forceinline__ void loader_role(const StackArgs& a, Lds& s, int lt, int lane, int lwave, int tile) {
  uint32_t* const state = a.exchange;
  const uint64_t* const ll_a = exchange_words(a, kLlAOffset);
  const uint64_t* const ll_x = exchange_words(a, kLlXOffset);
  const uint64_t* const ll_u = exchange_words(a, kLlUOffset);
  const uint64_t* const ll_y = exchange_words(a, kLlYOffset);
  // The first layer's input: the residual stream x in memory.
  float xv[8];
  {
    const float4 x0 = *reinterpret_cast<const float4*>(a.x + 8 * lt);
    const float4 x1 = *reinterpret_cast<const float4*>(a.x + 8 * lt + 4);
    xv[0] = x0.x, xv[1] = x0.y, xv[2] = x0.z, xv[3] = x0.w;
    xv[4] = x1.x, xv[5] = x1.y, xv[6] = x1.z, xv[7] = x1.w;
  }
  if (lt == 0) s.flag = __hip_atomic_load(state + kEpochWord, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
  // fp64 sum of squares: per lane, across each 16-lane row, then the 4 x 4
  // row sums in order (the GEMV prologue's order).
  auto partial_squares = [&]() __attribute__((always_inline)) {
    const double rs = row_sum_f64(square_sum8(xv));
    if ((lane & 15) == 0) s.red_ss[lwave][lane >> 4] = rs;
  };
  auto normalise_into = [&](uint32_t (*q)[8], float* sc) __attribute__((always_inline)) {
    double t = 0.0;
#pragma unroll
    for (int wv = 0; wv < 4; ++wv)
#pragma unroll
      for (int r = 0; r < 4; ++r) t += s.red_ss[wv][r];
    const float inv = rms_inverse(t, kH, a.eps);
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = half_bits_to_float(half_of_product(xv[k], inv));
    quantize_task(v, lt, q, sc);
  };
  bool ok = true;
  uint32_t flag = 0;
  const bool tail = a.o_in != nullptr;  // one layer from o on: no qkv input to form
  for (int l = 0; l < a.n_layers; ++l) {
    if (l > 0) {  // this layer's input: the previous layer's output stream
      uint32_t d[8];
      ok &= ll_wait<8>(ll_y + 8 * lt, flag, ok ? kSpinLimit : 1, d);
#pragma unroll
      for (int k = 0; k < 8; ++k) xv[k] = __uint_as_float(d[k]);
    }
    if (!tail) partial_squares();
    if (lt == tile) {
#pragma unroll
      for (int k = 0; k < 8; ++k) s.x_res[k] = xv[k];
    }
    __syncthreads();  // 1
    flag = s.flag + static_cast<uint32_t>(l);
    if (!tail) normalise_into(s.q_a, s.s_a);
    __syncthreads();  // 2
    __syncthreads();  // 3: qkv partial sums
    // o input: the query slice from every qkv tile, or the given fp16 row.
    {
      uint32_t d[4];
      if (tail) {
        const uint4 t4 = *reinterpret_cast<const uint4*>(a.o_in + 8 * lt);
        d[0] = t4.x, d[1] = t4.y, d[2] = t4.z, d[3] = t4.w;
      } else {
        ok &= ll_wait<4>(ll_a + 4 * lt, flag, ok ? kSpinLimit : 1, d);
      }
      float v[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[2 * k] = half_bits_to_float(d[k] & 0xFFFFu);
        v[2 * k + 1] = half_bits_to_float(d[k] >> 16);
      }
      quantize_task(v, lt, s.q_b, s.s_b);
    }
    __syncthreads();  // 4
    __syncthreads();  // 5: o partial sums
    // gate/up input: the residual stream after o, normalised.
    {
      uint32_t d[8];
      ok &= ll_wait<8>(ll_x + 8 * lt, flag, ok ? kSpinLimit : 1, d);
#pragma unroll
      for (int k = 0; k < 8; ++k) xv[k] = __uint_as_float(d[k]);
      partial_squares();
    }
    __syncthreads();  // 6
    normalise_into(s.q_c, s.s_c);
    __syncthreads();  // 7
    __syncthreads();  // 8: gate/up partial sums
    // down input: the quantised blocks of u, one per gate/up tile.
    {
      uint32_t d[9];
      ok &= ll_wait<9>(ll_u + 9 * lt, flag, ok ? kSpinLimit : 1, d);
      *reinterpret_cast<uint4*>(&s.q_d[lt][0]) = make_uint4(d[0], d[1], d[2], d[3]);
      *reinterpret_cast<uint4*>(&s.q_d[lt][4]) = make_uint4(d[4], d[5], d[6], d[7]);
      s.s_d[lt] = __uint_as_float(d[8]) * 0.0625f;
    }
    // Every workgroup writes one block of u of the last layer, after it has
    // read the epoch, so once workgroup 0 holds all 256 of them no workgroup
    // of this launch reads the epoch again: it is advanced for the next launch.
    if (l == a.n_layers - 1 && blockIdx.x == 0 && lt == 0)
      __hip_atomic_store(state + kEpochWord, flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();  // 9
    __syncthreads();  // 10: down partial sums
  }
  if (!ok) __hip_atomic_store(state + kErrorWord, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Compute waves (waves 0..7, thread ct): hold the weights in registers and
// form the dot products.  HAS_O: waves 0..3, which also hold the o tile.
// HAS_Q: the thread's qkv tile exists (launch block w for waves 0..3,
// 256 + w for waves 4..7).  Each projection's weights are requested right
// after the previous projection's output has been handed over (the
// hand-over stores then do not queue behind them), and the next layer's qkv
// weights after the gate/up hand-over.  (Measured on MI355X, one layer per
// launch: requesting every projection's weights at the start, or one
// projection ahead, was 0.7 us slower per layer, the input waits queueing
// behind the weights in flight.)
template <bool HAS_O, bool HAS_Q>
__device__ __forceinline__ void compute_role(const StackArgs& a, Lds& s, int ct, int lane, int wave, int w, int tile) {
  uint64_t* const ll_a = exchange_words_rw(a, kLlAOffset);
  uint64_t* const ll_x = exchange_words_rw(a, kLlXOffset);
  uint64_t* const ll_u = exchange_words_rw(a, kLlUOffset);
  uint64_t* const ll_y = exchange_words_rw(a, kLlYOffset);
  const int half = wave >> 2;
  const int tiles_q = a.n_qkv / 8;
  // Per-lane indices and weight offsets are formed from `ct` anew in every
  // layer (an empty asm statement hides that it does not change), so the
  // compiler does not keep 32 offsets alive across the layer loop.
  int n_q = 0, n_g = 0;
  auto lane_indices = [&]() __attribute__((always_inline)) {
    asm volatile("" : "+v"(ct));
    n_q = HAS_Q ? tile_of(half ? kG + w : w, tiles_q) * 8 + (ct & 7) : 0;
    const int c64 = ct & 63;
    n_g = c64 < 32 ? tile * 32 + c64 : kF + tile * 32 + (c64 - 32);
  };
  lane_indices();
  // Every tile starts at an even column, so a lane's column parity is ct & 1.
  const int shift = 16 * (ct & 1);

  uint4 wq[2], wo[2], wg[8], wd[4];
  uint32_t sq[2], so[2], sg[8], sd[4];
  auto issue_qkv = [&](int l) __attribute__((always_inline)) {
    if constexpr (HAS_Q) {
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const uint32_t g = static_cast<uint32_t>((((ct & 255) >> 3) + 32 * r) * a.n_qkv + n_q);
        wq[r] = *reinterpret_cast<const uint4*>(a.w[l].qkv_w + g * kPackedBytes);
        sq[r] = scale_word(a.w[l].qkv_s, g);
      }
    }
  };
  auto issue_o = [&](int l) __attribute__((always_inline)) {
    if constexpr (HAS_O) {
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const uint32_t g = static_cast<uint32_t>(((ct >> 3) + 32 * r) * kH + tile * 8 + (ct & 7));
        wo[r] = *reinterpret_cast<const uint4*>(a.w[l].o_w + g * kPackedBytes);
        so[r] = scale_word(a.w[l].o_s, g);
      }
    }
  };
  auto issue_gate_up = [&](int l) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const uint32_t g = static_cast<uint32_t>(((ct >> 6) + 8 * r) * (2 * kF) + n_g);
      wg[r] = *reinterpret_cast<const uint4*>(a.w[l].gate_up_w + g * kPackedBytes);
      sg[r] = scale_word(a.w[l].gate_up_s, g);
    }
  };
  auto issue_down = [&](int l) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t g = static_cast<uint32_t>(((ct >> 3) + 64 * r) * kH + tile * 8 + (ct & 7));
      wd[r] = *reinterpret_cast<const uint4*>(a.w[l].down_w + g * kPackedBytes);
      sd[r] = scale_word(a.w[l].down_s, g);
    }
  };
  issue_qkv(0);
  __builtin_amdgcn_sched_barrier(0);

  for (int l = 0; l < a.n_layers; ++l) {
    const bool last = l == a.n_layers - 1;
    if (l > 0) lane_indices();
    __syncthreads();  // 1
    const uint32_t flag = s.flag + static_cast<uint32_t>(l);
    __syncthreads();  // 2: qkv input in LDS

    // qkv: tiles of 8 columns, 256 lanes each (32 slots x 2 blocks).
    if constexpr (HAS_Q) {
      float acc = 0.0f;
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int bl = ((ct & 255) >> 3) + 32 * r;
        acc = block_step(wq[r], sq[r], shift, s.q_a[bl], s.s_a[bl], acc);
      }
      acc = row_sum<8>(acc);
      if ((lane & 15) < 8) s.red[((half * 4 + (wave & 3)) * 4 + (lane >> 4)) * 8 + (lane & 7)] = acc;
    }
    __syncthreads();  // 3
    if (HAS_Q && (wave & 3) == 0 && lane < 8) {
      float v = 0.0f;
#pragma unroll
      for (int wv = 0; wv < 4; ++wv)
#pragma unroll
        for (int p = 0; p < 4; ++p) v += s.red[((half * 4 + wv) * 4 + p) * 8 + lane];
      if (n_q < kH) {  // the query slice: fp16 copy for o, two columns per exchange word
        const uint32_t h = float_to_half_bits(v);
        const uint32_t hn = __shfl_xor(h, 1);
        if ((lane & 1) == 0) ll_store(ll_a + n_q / 2, h | (hn << 16), flag);
        if (last) a.a[n_q] = static_cast<uint16_t>(h);
      }
      if (last) a.q[n_q] = v;
    }
    __builtin_amdgcn_sched_barrier(0);
    issue_o(l);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();  // 4: o input in LDS

    // o: 8 columns, 256 lanes; residual add in the epilogue.
    if constexpr (HAS_O) {
      float acc = 0.0f;
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int bl = (ct >> 3) + 32 * r;
        acc = block_step(wo[r], so[r], shift, s.q_b[bl], s.s_b[bl], acc);
      }
      acc = row_sum<8>(acc);
      if ((lane & 15) < 8) s.red[(wave * 4 + (lane >> 4)) * 8 + (lane & 7)] = acc;
    }
    __syncthreads();  // 5
    if (HAS_O && wave == 0 && lane < 8) {
      float v = 0.0f;
#pragma unroll
      for (int wv = 0; wv < 4; ++wv)
#pragma unroll
        for (int p = 0; p < 4; ++p) v += s.red[(wv * 4 + p) * 8 + lane];
      const int n = tile * 8 + lane;
      const float xm = fmaf(a.alpha, v, s.x_res[lane]);
      ll_store(ll_x + n, __float_as_uint(xm), flag);
      s.x_mid[lane] = xm;
      if (last) a.o[n] = v;
    }
    __builtin_amdgcn_sched_barrier(0);
    issue_gate_up(l);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();  // 6
    __syncthreads();  // 7: gate/up input in LDS

    // gate/up: 64 columns (32 gate, their 32 up partners), 512 lanes (8 slots x 8 blocks).
    {
      float acc = 0.0f;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int bl = (ct >> 6) + 8 * r;
        acc = block_step(wg[r], sg[r], shift, s.q_c[bl], s.s_c[bl], acc);
      }
      s.red[wave * 64 + lane] = acc;
    }
    __syncthreads();  // 8
    if (wave == 0) {
      float v = 0.0f;
#pragma unroll
      for (int wv = 0; wv < 8; ++wv) v += s.red[wv * 64 + lane];
      const float up = __shfl(v, (lane + 32) & 63);
      const uint32_t uh = half_of_product(v, up);  // lanes < 32: u of column tile * 32 + lane
      // The block of u this tile forms (32 consecutive columns) is quantised
      // here, lanes 0..3 holding elements 8 l .. 8 l + 7, and handed over as
      // eight words of codes and one of its scale.
      float uv[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) uv[k] = half_bits_to_float(__shfl(uh, 8 * (lane & 3) + k));
      float scale;
      const uint2 codes = quantize8_group4(uv, &scale);
      if (lane < 4) {
        ll_store(ll_u + 9 * tile + 2 * lane, codes.x, flag);
        ll_store(ll_u + 9 * tile + 2 * lane + 1, codes.y, flag);
      }
      if (lane == 0) ll_store(ll_u + 9 * tile + 8, __float_as_uint(scale), flag);
      if (last) {
        a.g[n_g] = v;
        if (lane < 32) a.u[n_g] = static_cast<uint16_t>(uh);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    issue_down(l);
    if (!last) issue_qkv(l + 1);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();  // 9: down input in LDS

    // down: 8 columns, 512 lanes (64 slots x 4 blocks); residual add.
    {
      float acc = 0.0f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int bl = (ct >> 3) + 64 * r;
        acc = block_step(wd[r], sd[r], shift, s.q_d[bl], s.s_d[bl], acc);
      }
      acc = row_sum<8>(acc);
      if ((lane & 15) < 8) s.red[(wave * 4 + (lane >> 4)) * 8 + (lane & 7)] = acc;
    }
    __syncthreads();  // 10
    if (wave == 0 && lane < 8) {
      float v = 0.0f;
#pragma unroll
      for (int wv = 0; wv < 8; ++wv)
#pragma unroll
        for (int p = 0; p < 4; ++p) v += s.red[(wv * 4 + p) * 8 + lane];
      const int n = tile * 8 + lane;
      const float xo = fmaf(a.alpha, v, s.x_mid[lane]);
      if (last) {
        a.d[n] = v;
        a.x[n] = xo;
      } else {
        ll_store(ll_y + n, __float_as_uint(xo), flag);  // the next layer's input
      }
    }
  }
}

__global__ __launch_bounds__(kThreads) void decode_stack_kernel(StackArgs a) {
  __shared__ __align__(16) Lds s;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // The wave index as a scalar: every branch below is uniform per wave.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int w = blockIdx.x;
  const int tile = tile_of(w, kG);  // tile of o, gate/up and down (256 tiles each)
  // A launch that starts at o (a.o_in) holds no qkv tiles.
  const bool tail = a.o_in != nullptr;
  if (wave >= 8) loader_role(a, s, tid - kComputeThreads, lane, wave - 8, tile);
  else if (wave < 4 && tail) compute_role<true, false>(a, s, tid, lane, wave, w, tile);
  else if (wave < 4) compute_role<true, true>(a, s, tid, lane, wave, w, tile);
  else if (!tail && kG + w < a.n_qkv / 8) compute_role<false, true>(a, s, tid, lane, wave, w, tile);
  else compute_role<false, false>(a, s, tid, lane, wave, w, tile);
}

}  // namespace

bool layer_supported(int H, int n_qkv, int n_gu) {
  return H == kH && n_gu == 2 * kF && n_qkv >= kH && n_qkv <= 2 * kG * 8 && n_qkv % 64 == 0;
}

int co_resident_blocks(int* blocks) {
  int per_cu = 0, dev = 0, cus = 0;
  W4A8_HIP(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_stack_kernel, kThreads, 0));
  W4A8_HIP(hipGetDevice(&dev));
  W4A8_HIP(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
  *blocks = per_cu * cus;
  return W4A8_OK;
}

int launch_stack(const StackArgs& a, hipStream_t stream) {
  if (a.n_layers < 1 || a.n_layers > kMaxStack) return hip_fail(hipErrorInvalidValue, "resident stack: layer count");
  if (a.o_in && a.n_layers != 1) return hip_fail(hipErrorInvalidValue, "resident stack: a launch from o runs one layer");
  hipLaunchKernelGGL(decode_stack_kernel, dim3(kG), dim3(kThreads), 0, stream, a);
  W4A8_HIP(hipGetLastError());
  return W4A8_OK;
}

}  // namespace resident
}  // namespace w4a8
