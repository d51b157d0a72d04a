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
// four runs of four consecutive columns.
//
// Operand fragments: lane half h = l / 32 of an A operand loads bytes 8h .. 8h+7
// of the 16-byte weight group of its column; their low nibbles are elements
// 8h .. 8h+7 and their high nibbles elements 16+8h .. 16+8h+7 of the block.
// The B operand of lane half h loads 16 staged bytes with the same elements in
// the same order.  The MFMA pairs byte slot s of lane half h of A with byte
// slot s of lane half h of B (checked on gfx950), so the product is the block's
// full 32-element dot product.
//
// Data movement: per K block, a workgroup needs its packed weights [BN][16 B],
// weight scales [BN] fp16, activation scales [BM] fp32 and staged activation
// codes [BM][32 B]; each is one contiguous run in global memory per block.
// They are copied straight into LDS with global_load_lds_dwordx4 (no register
// round trip): chunk c of a stage is 16 bytes, and 64-chunk group g is one
// DMA instruction of wave g % NW (NW waves), whose lane i lands at chunk
// 64g + i.  A ring of four LDS stages is filled three steps ahead (deeper
// rings cost LDS that is worth more as occupancy); each wave waits on its own
// DMA count (s_waitcnt vmcnt) and a workgroup barrier then publishes the stage.  The staged activation codes are laid out so that a
// wave's 64 B-fragment reads hit 64 consecutive 16-byte slots (no LDS bank
// conflicts).
//
// K split inside the workgroup: the waves form a WN x WM x WK grid; the
// WK waves of one (n, m) position take interleaved K blocks (a step stages WK
// consecutive blocks) and add their accumulators through LDS at the end, in
// a fixed order.  Shapes with few output tiles thus still give every SIMD
// several waves to switch between.
//
// Epilogue per element and block, with the accumulator started at the bits of
// 1.5 * 2^23 so that D = 1.5 * 2^23 + 16 * I as an fp32 number:
//   t   = fma(D, sxq, -1.5 * 2^23 * sxq) = RN(I * sxq * 16),  sxq = sx' / 16
//   acc = fma(t, sw, acc)                  (sw widened to fp32 once per stage)
// where sx' is sx with its two lowest significand bits cleared, which makes
// 1.5 * 2^23 * sxq exact (relative change of sx below 2^-22).
#include "kernels.hpp"
#include "lds_dma.hpp"

namespace w4a8 {

namespace {

using lds::dma16;
using lds::stage_barrier;
using lds::wait_vmcnt;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
// Plain vector types for LDS reads: every read then keeps the alias
// information that lets the compiler tell it apart from DMA into another stage.
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));


// Byte layout of one LDS stage: WK K blocks of one workgroup tile.
template <int BN, int BM, int WK, int NW>
struct Stage {
  static constexpr int kA = 0;              // packed weights [BN][16]
  static constexpr int kSW = BN * 16;       // weight scales fp16 [BN]
  static constexpr int kSX = kSW + BN * 2;  // activation scales fp32 [BM]
  static constexpr int kB = kSX + BM * 4;   // staged codes [BM/32][2][32][16]
  static constexpr int kBlockBytes = kB + BM * 32;
  static constexpr int kBlockChunks = kBlockBytes / 16;
  static constexpr int kChunks = WK * kBlockChunks;
  static constexpr int kGroups = (kChunks + 63) / 64;   // DMA instructions per stage
  static constexpr int kMaxLoads = (kGroups + NW - 1) / NW;  // per wave
  static constexpr int kSWF = kGroups * 64 * 16;       // weight scales widened to fp32 [WK][BN]
  static constexpr int kBytes = kSWF + WK * BN * 4;
  static_assert(kBlockBytes % 16 == 0, "16-byte chunks");
  static_assert(2 * kMaxLoads <= 63, "vmcnt range");
};

// Source of one lane's DMA chunk: global address of its bytes in K block 0
// of the region, the region's stride per K block, and which of the step's
// WK blocks it belongs to.  Columns are clamped into range, so every lane of
// every DMA instruction reads valid memory.  With GATED the tile's columns
// are BN/2 gate columns and their partners N/2 further on (tile t covers
// gate columns t*BN/2 .. t*BN/2 + BN/2 - 1).
template <int BN, int BM, int WK, int NW, bool GATED>
__device__ __forceinline__ void chunk_source(int c, const uint8_t* pw, const uint16_t* ws, const uint8_t* qxs,
                                             const float* sxs, int N, int M_pad, int n0, int m0,
                                             const uint8_t** base, uint32_t* stride, int* kk) {
  using St = Stage<BN, BM, WK, NW>;
  c = min(c, St::kChunks - 1);  // padding lanes repeat the last chunk into the pad
  *kk = c / St::kBlockChunks;
  const int cc = c - *kk * St::kBlockChunks;
  auto column = [&](int lc) { return !GATED ? n0 + lc : lc < BN / 2 ? n0 / 2 + lc : N / 2 + n0 / 2 + lc - BN / 2; };
  if (cc < BN) {
    *base = pw + static_cast<int64_t>(min(column(cc), N - 1)) * kPackedBytes;
    *stride = static_cast<uint32_t>(N) * kPackedBytes;
  } else if (cc < BN + BN / 8) {
    *base = reinterpret_cast<const uint8_t*>(ws + min(column(8 * (cc - BN)), N - 8));
    *stride = static_cast<uint32_t>(N) * 2;
  } else if (cc < BN + BN / 8 + BM / 4) {
    *base = reinterpret_cast<const uint8_t*>(sxs + m0 + 4 * (cc - BN - BN / 8));
    *stride = static_cast<uint32_t>(M_pad) * 4;
  } else {
    *base = qxs + static_cast<int64_t>(m0) * kBlock + 16 * (cc - BN - BN / 8 - BM / 4);
    *stride = static_cast<uint32_t>(M_pad) * kBlock;
  }
}

// One activation block of the next GEMM from a 32 x 32 result tile: lane l
// holds row m's values at block positions 8q + 4h + i in v[4q + i] (h = l / 32)
// and lane l ^ 32 the other 16.  Quantised as the activation pre-pass does
// (same max-abs, scale and code routine) into the staging layout: codes of
// block bo at qout + bo * m_pad_out * 32, 16-byte slot ((m / 32) * 2 + q % 2)
// * 32 + m % 32, byte 8 * (q / 2) + 4h; scale at sout[bo * m_pad_out + m].
// Rows at or past m_pad_out are not stored.  Every lane of the wave calls it.
__device__ __forceinline__ void quantize_pair_to_staging(const float* v, int m, int h, int bo, int m_pad_out,
                                                         uint8_t* __restrict__ qout, float* __restrict__ sout) {
  float a = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) a = fmaxf(a, fabsf(v[r]));
  a = fmaxf(a, __shfl_xor(a, 32));
  const float sx = a / 127.0f;
  const uint2 c0 = quantize8_codes(v, a, sx);
  const uint2 c1 = quantize8_codes(v + 8, a, sx);
  if (m < m_pad_out) {
    uint8_t* row = qout + static_cast<int64_t>(bo) * m_pad_out * kBlock + (m & 31) * 16 + 4 * h;
    const int64_t s0 = static_cast<int64_t>((m >> 5) * 2) * 32 * 16;
    *reinterpret_cast<uint32_t*>(row + s0) = c0.x;                // q = 0
    *reinterpret_cast<uint32_t*>(row + s0 + 32 * 16) = c0.y;      // q = 1
    *reinterpret_cast<uint32_t*>(row + s0 + 8) = c1.x;            // q = 2
    *reinterpret_cast<uint32_t*>(row + s0 + 32 * 16 + 8) = c1.y;  // q = 3
    if (h == 0) sout[static_cast<int64_t>(bo) * m_pad_out + m] = sx;
  }
}

template <int TN, int TM, int WN, int WM, int WK, int MODE>
__global__ __launch_bounds__(64 * WN * WM * WK) __attribute__((amdgpu_waves_per_eu(MODE != 1 && WK == 1 ? 4 : 1)))
void gemm_kernel(
    const uint8_t* __restrict__ pw, const uint16_t* __restrict__ ws, const uint8_t* __restrict__ qxs,
    const float* __restrict__ sxs, int M, int M_pad, int K, int N, int tiles_n, int tiles_m, int bps,
    float* __restrict__ out, int32_t* __restrict__ sums, float* __restrict__ partials,
    uint32_t* __restrict__ tickets, float alpha, uint8_t* __restrict__ qout, float* __restrict__ sout,
    int m_pad_out, int n_cast) {
  constexpr int NW = WN * WM * WK;  // waves per workgroup
  static_assert(NW == 4 || NW == 8, "four or eight waves");
  static_assert(WK == 1 || (WK == 4 && WN * WM == 1), "K split only over four waves of one position");
  constexpr int BN = 32 * TN * WN;
  constexpr int BM = 32 * TM * WM;
  using St = Stage<BN, BM, WK, NW>;
  constexpr int kL = St::kMaxLoads;
  static_assert(WK == 1 || TN * TM * 64 * 16 * 4 <= St::kBytes, "K-split partials fit in one stage");
  static_assert(2 * kL <= 63, "vmcnt range");
  // Wave 0 widens a stage's weight scales to fp32 (two per lane) one step
  // ahead of use, which turns every half-rate v_fma_mix_f32 of the epilogue
  // into a full-rate v_fma_f32 but leaves each stage one step less time to
  // arrive.  The K-split tiles are short on latency hiding, so they keep the
  // fp16 scales and the three-step lead.
  // MODE 0 writes the scaled output; MODE 2 adds alpha times it into `out`
  // (the residual stream); MODE 1 exports the integer block sums; MODE 3
  // (gated) forms fp16(gate * up) of the tile's column pairs and quantises it
  // into the staging of the next GEMM (qout, sout) instead of writing out;
  // MODE 4 does the same with fp16(y) of the leading n_cast columns and
  // writes the others out as MODE 0.
  constexpr bool kGated = MODE == 3;
  static_assert(!kGated || (TN == 1 && WN == 4 && WK == 1), "gated tiles: four 32-column waves along n");
  constexpr bool kWiden = MODE != 1 && WK == 1;
  static_assert(!kWiden || BN == 128, "one wave widens the scales of a stage, two per lane");
  // Ring of four stages: blocks are fetched three steps ahead.
  __shared__ __attribute__((aligned(16))) uint8_t st0[St::kBytes];
  __shared__ __attribute__((aligned(16))) uint8_t st1[St::kBytes];
  __shared__ __attribute__((aligned(16))) uint8_t st2[St::kBytes];
  __shared__ __attribute__((aligned(16))) uint8_t st3[St::kBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave % WN;
  const int wm = (wave / WN) % WM;
  const int wk = wave / (WN * WM);
  const int h = lane >> 5;
  const int l32 = lane & 31;
  const int my_loads = (St::kGroups - wave + NW - 1) / NW;  // kL or kL - 1

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
  // Opaque to the optimiser: the splat then lives in one register tuple that
  // every MFMA reads as its C operand, instead of being rebuilt (16 moves)
  // in each MFMA's destination registers before every block.
  asm volatile("" : "+v"(magic));

  float acc[TN][TM][16];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // One K block of this wave: fragments and scales from LDS, TN x TM MFMAs,
  // then the fp32 epilogue (or, for the block-sum export, the integer sums).
  auto compute = [&](const uint8_t* st, int b) __attribute__((always_inline)) {
    const uint8_t* sb = st + wk * St::kBlockBytes;
    v4i afrag[TN];
    v4f swf[TN][4];
    v2u sraw[TN][4];
#pragma unroll
    for (int i = 0; i < TN; ++i) {
      const int col = (wn * TN + i) * 32;
      const v2u araw = *reinterpret_cast<const v2u*>(sb + St::kA + (col + l32) * 16 + 8 * h);
      afrag[i][0] = static_cast<int>(low_nibbles_x16(araw.x));
      afrag[i][1] = static_cast<int>(low_nibbles_x16(araw.y));
      afrag[i][2] = static_cast<int>(high_nibbles_x16(araw.x));
      afrag[i][3] = static_cast<int>(high_nibbles_x16(araw.y));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (kWiden) swf[i][q] = *reinterpret_cast<const v4f*>(st + St::kSWF + (wk * BN + col + 8 * q + 4 * h) * 4);
        else sraw[i][q] = *reinterpret_cast<const v2u*>(sb + St::kSW + (col + 8 * q + 4 * h) * 2);
      }
    }
    v4i bfrag[TM];
    float sxv[TM];
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int rg = wm * TM + j;
      bfrag[j] = *reinterpret_cast<const v4i*>(sb + St::kB + ((rg * 2 + h) * 32 + l32) * 16);
      sxv[j] = *reinterpret_cast<const float*>(sb + St::kSX + (rg * 32 + l32) * 4);
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
          float sw;
          if (kWiden) {
            sw = swf[i][r / 4][r % 4];
          } else {
            const uint32_t word = (r & 2) ? sraw[i][r / 4].y : sraw[i][r / 4].x;
            sw = half_bits_to_float((r & 1) ? (word >> 16) : (word & 0xFFFFu));  // folds into v_fma_mix_f32
          }
          const float t = fmaf(__int_as_float(d[i][j][r]), sxq[j], cx[j]);
          acc[i][j][r] = fmaf(t, sw, acc[i][j][r]);
        }
  };

  if (b_begin < b_end) {
    const int last = b_end - 1;
    const int nsteps = (b_end - b_begin + WK - 1) / WK;
    // DMA sources of this lane, one per instruction; a wave with fewer
    // groups than kL leaves its last slot unused.
    const uint8_t* src0;
    const uint8_t* src1;
    const uint8_t* src2;
    uint32_t str0, str1, str2;
    int kk0, kk1, kk2;
    static_assert(kL <= 3, "three DMA instructions per wave and stage at most");
    chunk_source<BN, BM, WK, NW, kGated>((wave + 0 * NW) * 64 + lane, pw, ws, qxs, sxs, N, M_pad, n0, m0, &src0, &str0, &kk0);
    chunk_source<BN, BM, WK, NW, kGated>((wave + 1 * NW) * 64 + lane, pw, ws, qxs, sxs, N, M_pad, n0, m0, &src1, &str1, &kk1);
    chunk_source<BN, BM, WK, NW, kGated>((wave + 2 * NW) * 64 + lane, pw, ws, qxs, sxs, N, M_pad, n0, m0, &src2, &str2, &kk2);

    // Stage `st` <- the WK blocks of step s (clamped to the last block, so
    // the steps past the end re-read it and every wave issues the same
    // number of DMAs per step).
#define W4A8_DMA(ST, S)                                                                          \
  do {                                                                                           \
    const int sd_ = (S);                                                                          \
    const int bsd_ = b_begin + sd_ * WK;                                                           \
    if (kL > 0 && my_loads > 0)                                                                  \
      dma16(src0 + static_cast<uint64_t>(static_cast<uint32_t>(min(bsd_ + kk0, last))) * str0,        \
            (ST) + (wave + 0 * NW) * 1024);                                                         \
    if (kL > 1 && my_loads > 1)                                                                  \
      dma16(src1 + static_cast<uint64_t>(static_cast<uint32_t>(min(bsd_ + kk1, last))) * str1,        \
            (ST) + (wave + 1 * NW) * 1024);                                                         \
    if (kL > 2 && my_loads > 2)                                                                  \
      dma16(src2 + static_cast<uint64_t>(static_cast<uint32_t>(min(bsd_ + kk2, last))) * str2,        \
            (ST) + (wave + 2 * NW) * 1024);                                                         \
  } while (0)
    // Widening runs one step ahead: stage s + 1 is converted while the waves
    // compute stage s, and the next barrier publishes it.
    auto convert_scales = [&](uint8_t* st) __attribute__((always_inline)) {
      if (kWiden && wave == 0) {
        const int kk = lane / (BN / 2);
        const int p = lane % (BN / 2);
        const uint32_t two = *reinterpret_cast<const uint32_t*>(st + kk * St::kBlockBytes + St::kSW + 4 * p);
        v2f f;
        f.x = half_bits_to_float(two & 0xFFFFu);
        f.y = half_bits_to_float(two >> 16);
        *reinterpret_cast<v2f*>(st + St::kSWF + (kk * BN + 2 * p) * 4) = f;
      }
    };
    // Step s: wait for this wave's DMAs into the stage of step s + 1 when
    // widening (else of step s), publish it, refill the stage drained last
    // step with step s + 3, widen the scales of step s + 1, compute step s.
    // vmcnt counts loads and stores together, and a store may complete ahead
    // of older loads, so the block-sum export (which stores inside the loop)
    // drains the counter instead.
#define W4A8_STEP(CUR, NXT, REFILL, S)                                                           \
  do {                                                                                           \
    const int s_ = (S);                                                                          \
    if (MODE == 1) wait_vmcnt<0>();                                                              \
    else if (kWiden && my_loads == kL) wait_vmcnt<kL>();                                         \
    else if (kWiden) wait_vmcnt<kL - 1>();                                                       \
    else if (my_loads == kL) wait_vmcnt<2 * kL>();                                               \
    else wait_vmcnt<2 * (kL - 1)>();                                                             \
    stage_barrier();                                                                             \
    W4A8_DMA(REFILL, s_ + 3);                                                                    \
    convert_scales(NXT);                                                                         \
    const int b_ = b_begin + s_ * WK + wk;                                                       \
    if (s_ < nsteps && b_ < b_end) compute((CUR), b_);                                           \
  } while (0)
    W4A8_DMA(st0, 0);
    W4A8_DMA(st1, 1);
    W4A8_DMA(st2, 2);
    if (kWiden) {
      if (my_loads == kL) wait_vmcnt<2 * kL>();
      else wait_vmcnt<2 * (kL - 1)>();
      stage_barrier();
      convert_scales(st0);
    }
    for (int s = 0; s < nsteps; s += 4) {
      W4A8_STEP(st0, st1, st3, s + 0);
      W4A8_STEP(st1, st2, st0, s + 1);
      W4A8_STEP(st2, st3, st1, s + 2);
      W4A8_STEP(st3, st0, st2, s + 3);
    }
#undef W4A8_STEP
#undef W4A8_DMA
    // The refills past the end are still in flight: drain them before the
    // stages are reused or the workgroup ends.
    wait_vmcnt<0>();
  }

  if (MODE == 1) return;

  if (kGated) {
    // Waves wn = 2, 3 hold the partners of the gate columns of waves wn - 2.
    // Each hands its accumulators to its gate wave through one LDS stage, one
    // 32-row tile j at a time; the gate wave forms v = fp16(g * u) and
    // quantises each row's 32 values (one block of the next GEMM's K: lane l
    // holds 16 of them, lane l ^ 32 the other 16) exactly as the activation
    // pre-pass does, into the staging layout.  Rows from M up to m_pad_out
    // get zero codes and scales, as the pre-pass writes for padding rows.
    const int pair = (wn & 1) + 2 * wm;
    float* xch = reinterpret_cast<float*>(pair == 0 ? st0 : pair == 1 ? st1 : pair == 2 ? st2 : st3);
    const int bo = (n0 >> 6) + wn;  // output block: gate columns 32 * bo .. 32 * bo + 31
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      __syncthreads();
      if (wn >= 2) {
#pragma unroll
        for (int r = 0; r < 16; ++r) xch[r * 64 + lane] = acc[0][j][r];
      }
      __syncthreads();
      if (wn < 2) {
        const int m = m_base + 32 * j + l32;
        float v[16];
#pragma unroll
        for (int r = 0; r < 16; ++r)
          v[r] = m < M ? half_bits_to_float(half_of_product(acc[0][j][r], xch[r * 64 + lane])) : 0.0f;
        quantize_pair_to_staging(v, m, h, bo, m_pad_out, qout, sout);
      }
    }
    return;
  }

  // Waves wk > 0 hand their accumulators to wave wk = 0 of their (n, m)
  // position through LDS; that wave adds them in wk order.
  if (WK > 1) {
    stage_barrier();
    const int pos = wave % (WN * WM);
    if (wk > 0) {
      const int slot = pos * (WK - 1) + wk - 1;
      float* dst = reinterpret_cast<float*>(slot == 0 ? st0 : slot == 1 ? st1 : st2);
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) dst[((i * TM + j) * 16 + r) * 64 + lane] = acc[i][j][r];
    }
    stage_barrier();
    if (wk == 0) {
#pragma unroll
      for (int k = 1; k < WK; ++k) {
        const int slot = pos * (WK - 1) + k - 1;
        const float* src = reinterpret_cast<const float*>(slot == 0 ? st0 : slot == 1 ? st1 : st2);
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
          for (int j = 0; j < TM; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] += src[((i * TM + j) * 16 + r) * 64 + lane];
      }
    }
  }
  const bool owner = wk == 0;  // wave that holds the workgroup's result for its (n, m) position

  if (ksplit > 1) {
    // Partial tiles meet in library scratch.  Every access to it and to the
    // ticket is a device-scope atomic, so no cache-wide fence is needed; the
    // explicit wait makes each lane's partial stores complete before the
    // workgroup takes its ticket.
    __shared__ int last_flag;
    if (owner) {
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
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0)
      last_flag = __hip_atomic_fetch_add(&tickets[1 + id], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                  static_cast<uint32_t>(ksplit - 1);
    __syncthreads();
    if (!last_flag) return;
    if (owner) {
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
    }
    if (threadIdx.x == 0) __hip_atomic_store(&tickets[1 + id], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  if (!owner) return;
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int m = m_base + 32 * j + l32;
      if (MODE == 4 && n_base + 32 * i < n_cast) {
        // A block of the leading n_cast columns: fp16(y) quantised into the
        // next GEMM's staging instead of written out.
        float v[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] = m < M ? half_bits_to_float(float_to_half_bits(acc[i][j][r])) : 0.0f;
        quantize_pair_to_staging(v, m, h, (n_base + 32 * i) >> 5, m_pad_out, qout, sout);
        continue;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n_base + 32 * i + 8 * q + 4 * h;
        if (m < M && n < N) {
          float4* dst = reinterpret_cast<float4*>(out + static_cast<int64_t>(m) * N + n);
          float4 y = make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
          if (MODE == 2) {
            const float4 r = *dst;
            y = make_float4(fmaf(alpha, y.x, r.x), fmaf(alpha, y.y, r.y), fmaf(alpha, y.z, r.z), fmaf(alpha, y.w, r.w));
          }
          *dst = y;
        }
      }
    }
}

struct Plan {
  int tn, tm, wn, wm, wk;  // MFMA tiles per wave (n, m); waves along n, m and K
  int wg_n, wg_m;
  int tiles_n, tiles_m, m_pad;
  int ksplit, bps;
};

Plan make_plan(int tn, int tm, int wn, int wm, int wk, int M, int N) {
  Plan p{};
  p.tn = tn;
  p.tm = tm;
  p.wn = wn;
  p.wm = wm;
  p.wk = wk;
  p.wg_n = 32 * tn * wn;
  p.wg_m = 32 * tm * wm;
  p.tiles_n = (N + p.wg_n - 1) / p.wg_n;
  p.tiles_m = (M + p.wg_m - 1) / p.wg_m;
  p.m_pad = p.tiles_m * p.wg_m;
  return p;
}

// Each wave owns 32 x 64 outputs (32 x 32 for at most 32 tokens).  Large
// problems take the widest workgroup tile that still fills the chip twice
// over: the bytes staged per MFMA fall as the tile grows (the activation
// codes of a block are shared by all BN weight columns).  Otherwise the four
// waves of a workgroup split K over one 32 x 32 tile (measured on MI355X at
// M = 512: 32 x 32 tiles beat 32 x 64 ones by 0.7-2 us on 2048 x 2560,
// 2048 x 2048 and 8192 x 2048, fewer registers and more waves per SIMD
// outweighing the extra staging).  Split K across workgroups only when even
// that leaves CUs idle.
Plan plan_gemm(int M, int K, int N) {
  constexpr int kCUs = 256;
  const int tm = M <= 32 ? 1 : 2;
  Plan p;
  if (M > 64) p = make_plan(1, 2, 4, 2, 1, M, N);       // 128 x 128, eight waves
  else p = make_plan(1, tm, 4, 1, 1, M, N);             // 128 x 32 or 128 x 64
  if (p.tiles_n * p.tiles_m < 2 * kCUs) p = make_plan(1, 1, 1, 1, 4, M, N);
  const int nb = K / kBlock;
  const int tiles = p.tiles_n * p.tiles_m;
  constexpr int kMinBlocksPerSplit = 64;
  int ks = tiles < kCUs ? (2 * kCUs + tiles - 1) / tiles : 1;
  const int ks_max = nb / kMinBlocksPerSplit;
  if (ks > ks_max) ks = ks_max;
  if (ks < 1) ks = 1;
  p.bps = (nb + ks - 1) / ks;
  p.ksplit = (nb + p.bps - 1) / p.bps;
  return p;
}

size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

}  // namespace

bool gemm_gated_supported(int M, int K, int N, int m_pad_out) {
  const Plan p = plan_gemm(M, K, N);
  return p.wm == 2 && p.wk == 1 && p.ksplit == 1 && N % 128 == 0 && m_pad_out >= M && m_pad_out <= p.m_pad &&
         m_pad_out % 32 == 0;
}

bool gemm_cast_supported(int M, int K, int N, int n_cast, int m_pad_out) {
  const Plan p = plan_gemm(M, K, N);
  return n_cast >= 32 && n_cast % 32 == 0 && n_cast <= N && m_pad_out >= M && m_pad_out <= p.m_pad &&
         m_pad_out % 32 == 0;
}

size_t gemm_staging_bytes(int M, int K, int N) {
  const Plan p = plan_gemm(M, K, N);
  const size_t nb = K / kBlock;
  return align256(nb * p.m_pad * kBlock) + align256(nb * p.m_pad * sizeof(float));
}

GemmStaging gemm_staging_at(void* base, int M, int K, int N) {
  const Plan p = plan_gemm(M, K, N);
  const size_t nb = K / kBlock;
  GemmStaging s{};
  s.qxs = static_cast<uint8_t*>(base);
  s.sxs = reinterpret_cast<float*>(static_cast<uint8_t*>(base) + align256(nb * p.m_pad * kBlock));
  s.m_pad = p.m_pad;
  return s;
}

size_t gemm_scratch_bytes(int M, int K, int N) {
  const Plan p = plan_gemm(M, K, N);
  const size_t nb = K / kBlock;
  size_t bytes = align256(nb * p.m_pad * kBlock) + align256(nb * p.m_pad * sizeof(float));
  if (p.ksplit > 1) bytes += static_cast<size_t>(p.ksplit) * M * N * sizeof(float);
  return bytes;
}

namespace {

// Partial tiles of a split-K launch follow the room for a staging in library
// scratch (whether or not the staging in use lies there).
float* gemm_partials(void* work, const GemmStaging& s, int K) {
  const size_t nb = K / kBlock;
  return reinterpret_cast<float*>(static_cast<uint8_t*>(work) + align256(nb * s.m_pad * kBlock) +
                                  align256(nb * s.m_pad * sizeof(float)));
}

int launch_gemm_kernel(const GemmArgs& a, int mode, const GemmStaging& s, Scratch* sc, hipStream_t stream) {
  const Plan p = plan_gemm(a.M, a.K, a.N);
  if (p.tiles_n * p.tiles_m >= kMaxTickets - 1) return hip_fail(hipErrorInvalidValue, "gemm: too many tiles");
  if (s.m_pad != p.m_pad) return hip_fail(hipErrorInvalidValue, "gemm: staging of another shape");
  int rc = require_scratch(sc, gemm_scratch_bytes(a.M, a.K, a.N));
  if (rc != W4A8_OK) return rc;
  if (p.ksplit > 1 && p.tiles_n * p.tiles_m + 1 > sc->n_tickets)
    return hip_fail(hipErrorInvalidValue, "gemm: more split tiles than tickets");
  const uint8_t* qxs = s.qxs;
  const float* sxs = s.sxs;
  float* partials = gemm_partials(sc->work, s, a.K);
  const dim3 grid(p.tiles_n * p.tiles_m, p.ksplit);
  // Every thread stages scale chunks unconditionally; the block-sum export has
  // no scales (w_scales may be null), so it stages bytes of the packed weights
  // instead (at least as large as the scales would be) and never reads them.
  const uint16_t* ws = mode == 1 ? reinterpret_cast<const uint16_t*>(a.packed_w) : a.w_scales;
#define W4A8_GEMM_LAUNCH(TN, TM, WN, WM, WK, MODE)                                                     \
  hipLaunchKernelGGL((gemm_kernel<TN, TM, WN, WM, WK, MODE>), grid, dim3(64 * WN * WM * WK), 0,     \
                     stream, a.packed_w, ws, qxs, sxs, a.M, p.m_pad, a.K, a.N, p.tiles_n, p.tiles_m,       \
                     p.bps, mode == 2 ? a.resid : a.out, a.sums, partials, sc->tickets, a.alpha, a.q_out,        \
                     a.s_out, a.m_pad_out, a.n_cast)
#define W4A8_GEMM_MODE(MODE)                                                                           \
  do {                                                                                                 \
    if (p.wk == 4) {                                                                                   \
      W4A8_GEMM_LAUNCH(1, 1, 1, 1, 4, MODE);                                                           \
    } else if (p.wm == 2) {                                                                            \
      W4A8_GEMM_LAUNCH(1, 2, 4, 2, 1, MODE);                                                           \
    } else if (p.tm == 2) {                                                                            \
      W4A8_GEMM_LAUNCH(1, 2, 4, 1, 1, MODE);                                                           \
    } else {                                                                                           \
      W4A8_GEMM_LAUNCH(1, 1, 4, 1, 1, MODE);                                                           \
    }                                                                                                  \
  } while (0)
  if (mode == 3) {
    if (!gemm_gated_supported(a.M, a.K, a.N, a.m_pad_out) || !a.q_out || !a.s_out)
      return hip_fail(hipErrorInvalidValue, "gemm: gated epilogue needs 128 x 128 tiles, N % 128 == 0 and a staging within the tile rows");
    W4A8_GEMM_LAUNCH(1, 2, 4, 2, 1, 3);
  } else if (mode == 4) {
    if (!gemm_cast_supported(a.M, a.K, a.N, a.n_cast, a.m_pad_out) || !a.q_out || !a.s_out)
      return hip_fail(hipErrorInvalidValue, "gemm: cast epilogue needs whole blocks and a staging within the tile rows");
    W4A8_GEMM_MODE(4);
  } else if (mode == 1) W4A8_GEMM_MODE(1);
  else if (mode == 2) W4A8_GEMM_MODE(2);
  else W4A8_GEMM_MODE(0);
#undef W4A8_GEMM_MODE
#undef W4A8_GEMM_LAUNCH
  W4A8_HIP(hipGetLastError());
  return W4A8_OK;
}

}  // namespace

int gemm_staging(int M, int K, int N, Scratch* sc, GemmStaging* s) {
  const Plan p = plan_gemm(M, K, N);
  const int rc = require_scratch(sc, gemm_scratch_bytes(M, K, N));
  if (rc != W4A8_OK) return rc;
  const size_t nb = K / kBlock;
  uint8_t* base = static_cast<uint8_t*>(sc->work);
  s->qxs = base;
  s->sxs = reinterpret_cast<float*>(base + align256(nb * p.m_pad * kBlock));
  s->m_pad = p.m_pad;
  return W4A8_OK;
}

int launch_gemm(const GemmArgs& a, int mode, Scratch* sc, hipStream_t stream) {
  GemmStaging s{};
  int rc = gemm_staging(a.M, a.K, a.N, sc, &s);
  if (rc != W4A8_OK) return rc;
  rc = launch_quantize_stage(a.x, a.M, s.m_pad, a.K, s.qxs, s.sxs, stream);
  if (rc != W4A8_OK) return rc;
  return launch_gemm_kernel(a, mode, s, sc, stream);
}

int launch_gemm_staged(const GemmArgs& a, const GemmStaging& s, Scratch* sc, hipStream_t stream) {
  return launch_gemm_kernel(a, 0, s, sc, stream);
}

int launch_gemm_staged_resid(const GemmArgs& a, const GemmStaging& s, Scratch* sc, hipStream_t stream) {
  return launch_gemm_kernel(a, 2, s, sc, stream);
}

int launch_gemm_staged_cast(const GemmArgs& a, int n_cast, const GemmStaging& s, const GemmStaging& out,
                            Scratch* sc, hipStream_t stream) {
  GemmArgs g = a;
  g.q_out = out.qxs;
  g.s_out = out.sxs;
  g.m_pad_out = out.m_pad;
  g.n_cast = n_cast;
  return launch_gemm_kernel(g, 4, s, sc, stream);
}

int launch_gemm_staged_gated(const GemmArgs& a, const GemmStaging& s, const GemmStaging& out, Scratch* sc,
                             hipStream_t stream) {
  GemmArgs g = a;
  g.q_out = out.qxs;
  g.s_out = out.sxs;
  g.m_pad_out = out.m_pad;
  return launch_gemm_kernel(g, 3, s, sc, stream);
}

}  // namespace w4a8
