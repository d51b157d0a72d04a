// Decode attention: the newest token's query heads over an fp16 KV cache, the
// step between a decoder layer's QKV and O projections.  The pages decode
// with an fp16 KV cache at context 640 and store that cache in a layout
// chosen for the GPU (ML Drift explainer on tech.dede.sh, section
// "Stage-aware optimization for large language models").
//
// Computed: scaled dot-product attention with grouped query heads (query head
// h reads KV head h / G, G = Hq / Hkv), softmax over the L cached positions,
// the newest (position L - 1) included after its key and value are rounded to
// fp16 and written into the cache by this same launch.
//
// Cache storage, chosen so that both products run on the fp16 matrix
// instruction with operands read as contiguous runs:
//   k_cache [Hkv][capacity][D]  -- scores S = Q K^T: a lane's B operand is a
//                                  run of one position's dimensions
//   v_cache [Hkv][D][capacity]  -- output O = P V: a lane's B operand is a run
//                                  of one dimension's positions
//
// One workgroup (four waves) per 64-position chunk and KV head:
//   1. loads its chunk of K and V and the group's fp32 queries in one round;
//   2. S = [Q_hi; Q_lo] K^T on v_mfma_f32_16x16x16_f16, the 16 matrix rows
//      holding the fp16 high parts of up to 8 query heads and, scaled by 2^12,
//      their low parts (q = hi + lo / 2^12 to about 22 bits), so the fp32
//      queries keep their precision on fp16 inputs at no extra instruction;
//   3. a chunk-local softmax in base 2 (running max m, weight sum l);
//   4. O = [P_hi; P_lo] V, the weights split the same way;
//   5. writes (m, l, O) as a partial.  Chunks form at most kMaxGroups merge
//      groups of consecutive chunks; the last workgroup of a group to finish
//      (an atomic ticket) merges the group's partials in chunk order, and with
//      more than one group the last group merger merges the group results in
//      group order, so the result does not depend on which workgroup finishes
//      when.  The final merge writes the fp16 output.  A merge keeps a running
//      maximum (online softmax) and fetches eight partials per round, so its
//      memory round trips grow with chunks / 8, not with chunks.
//   5'. Up to kMaxLlChunks chunks (context 2048 at most), when the partials fit
//      the library's attention exchange area: every chunk writes its partials
//      as 64-bit words of 32 bits of data and a flag (agent-scope atomics, no
//      store to wait for, no ticket), and every workgroup merges a run of
//      consecutive outputs (head * D + dimension), one output per thread
//      (a few for short contexts), in chunk order.  A wave's polls read
//      consecutive words, so a poll round costs a few cache lines per
//      instruction.  With many chunks the workgroup's threads split the
//      chunks into two or four ranges merged side by side and combined in
//      order through LDS.  Each KV head has its own
//      fixed region of words and epoch word; the flag is 1 + that epoch,
//      which workgroup 0 of the head advances once it has read every chunk's
//      words.  Every wait is bounded and raises the device error word.
#include <algorithm>
#include <cmath>

#include "kernels.hpp"

namespace w4a8 {

namespace {

constexpr int kChunk = 64;          // positions per workgroup
constexpr int kThreads = 256;       // four waves
constexpr int kRows = 16;           // matrix rows: hi parts of 8 heads, then lo parts
constexpr int kMaxGroup = 8;        // query heads per KV head
constexpr float kLo = 4096.0f;      // lo parts are stored times 2^12
constexpr float kInvLo = 1.0f / 4096.0f;
constexpr int kMaxGroups = 32;      // merge groups per KV head
constexpr int kGroupChunks = 16;    // chunks per merge group, at least
constexpr int kMergeUnroll = 8;     // partials fetched per merge round
constexpr int kMaxLlChunks = 32;    // chunks the flagged-word merge serves
constexpr int kLlSpin = 1 << 20;    // polls before a wait gives up
constexpr int kLlSlots = 16;        // (output, chunk) pairs a thread of the flagged-word merge holds

// The flagged-word merge's split of a KV head's `outputs` (G * D, a multiple
// of 64) over its chunks' workgroups: the first `workers` workgroups (the
// largest divisor of outputs / 64 not above the chunk count) merge `per`
// consecutive outputs each, `per` a multiple of 64.  A workgroup's threads
// form `split` ranges of `cs` consecutive chunks (4 with per <= 64, 2 with
// per <= 128), each range's kThreads / split threads covering the
// workgroup's outputs, `reps` outputs per thread (kThreads / split apart).
// Whether a thread has its r-th output is uniform over its wave.  A thread
// holds at most reps * cs words.
struct LlPlan {
  int workers, per, split, reps, cs;
  int tlog;  // log2(kThreads / split)
};
LlPlan ll_plan(int outputs, int chunks) {
  LlPlan p;
  const int blocks = outputs / 64;
  p.workers = 1;
  for (int d = 1; d <= std::min(blocks, chunks); ++d)
    if (blocks % d == 0) p.workers = d;
  p.per = outputs / p.workers;
  p.split = p.per <= 64 ? 4 : p.per <= 128 ? 2 : 1;
  p.tlog = p.split == 4 ? 6 : p.split == 2 ? 7 : 8;
  p.reps = (p.per + (1 << p.tlog) - 1) >> p.tlog;
  p.cs = (chunks + p.split - 1) / p.split;
  return p;
}

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

struct AttnArgs {
  const float* q;        // fp32 [Hkv * G][D]
  const float* k_new;    // fp32 [Hkv][D]
  const float* v_new;    // fp32 [Hkv][D]
  uint16_t* k_cache;     // fp16 [Hkv][capacity][D]
  uint16_t* v_cache;     // fp16 [Hkv][D][capacity]
  uint16_t* out;         // fp16 [Hkv * G][D]
  float* part;           // [Hkv][chunks][G][D] unnormalised chunk outputs
  float* stats;          // [Hkv][chunks][G][2]: chunk max (base-2 units), weight sum
  float* part2;          // [Hkv][kMaxGroups][G][D] unnormalised merge-group outputs
  float* stats2;         // [Hkv][kMaxGroups][G][2]
  uint32_t* tickets;     // [Hkv][max_groups + 1], zero between launches
  int group, length, capacity;
  int group_chunks;      // chunks per merge group
  int max_groups;        // merge groups per KV head at most (<= kMaxGroups): the ticket stride
  float scale2;          // log2(e) / sqrt(D)
  // Flagged-word merge (nullable: the ticket merge above).
  uint64_t* ll;          // [kAttnHeads][kAttnHeadWords] words; head g: [chunks][G][D + 2] (output dims, then max
                         // and weight sum)
  uint32_t* epochs;      // [Hkv]
  uint32_t* error;       // device error word
  LlPlan llp;            // the flagged-word merge's split (ll_plan)
};

// A KV head's flagged words are reached through a buffer resource: a
// uniform base and size in scalar registers, a 32-bit byte offset per lane
// and one per access (a scalar or a constant), so an access costs one
// instruction and no 64-bit address arithmetic.  Offsets at or past the
// region's end drop a store (the way lanes with nothing to write skip it).
// Every access is one aligned 64-bit load or store with the device-coherent
// cache policy (sc1), what a relaxed agent-scope atomic compiles to here.
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
constexpr int kCoherent = 16;               // cache policy bits: sc1
constexpr uint32_t kDropOffset = 0x80000000u;  // past every region's end
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_words(uint64_t* ll, int g) {
  // The base is uniform; readfirstlane keeps it (and the resource) in
  // scalar registers wherever it is used.
  const uint64_t p = reinterpret_cast<uint64_t>(ll + static_cast<int64_t>(g) * kAttnHeadWords);
  // (readfirstlane returns int: go through uint32_t, or the low half would be
  // sign-extended into the high one.)
  const uint64_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p)));
  const uint64_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p >> 32)));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(hi << 32 | lo), 0,
                                           static_cast<int>(kAttnHeadWords * sizeof(uint64_t)), 0x00020000);
}
__device__ __forceinline__ void ll_put(__amdgpu_buffer_rsrc_t r, uint32_t lane_off, uint32_t off, float v,
                                       uint32_t flag) {
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(v), flag}, r, lane_off, off, kCoherent);
}
__device__ __forceinline__ u32x2 ll_get(__amdgpu_buffer_rsrc_t r, uint32_t lane_off, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, lane_off, off, kCoherent);
}

// Max or sum over each 32-lane half of a wave, the result in all its lanes:
// DPP within quads (lane ^ 1, lane ^ 2), within 8-lane and 16-lane rows
// (mirrors), then the two 16-lane rows of the half (v_permlane16_swap).  The
// pairing is that of a lane ^ 1, 2, 4, 8, 16 butterfly, so every lane forms the
// same sums in the same order; no LDS traffic.
template <bool kMax>
__device__ __forceinline__ float half_wave_reduce(float v) {
  auto op = [](float x, float y) { return kMax ? fmaxf(x, y) : x + y; };
  v = op(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true)));   // quad_perm [1,0,3,2]
  v = op(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true)));   // quad_perm [2,3,0,1]
  v = op(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true)));  // row_half_mirror
  v = op(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, true)));  // row_mirror
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Lanes 0 .. 31 receive lanes 32 .. 63 of v (one v_permlane32_swap).
__device__ __forceinline__ float upper_half(float v) {
  return __uint_as_float(__builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false)[1]);
}

__device__ __forceinline__ uint32_t pack2(_Float16 a, _Float16 b) {
  return static_cast<uint32_t>(__builtin_bit_cast(unsigned short, a)) |
         (static_cast<uint32_t>(__builtin_bit_cast(unsigned short, b)) << 16);
}

// The four fp16 values at half offset 4 * i of a run held as 16-byte words.
__device__ __forceinline__ h4 half4_at(const uint4* run, int i) {
  const uint4 w = run[i >> 1];
  const uint2 v = (i & 1) ? make_uint2(w.z, w.w) : make_uint2(w.x, w.y);
  return __builtin_bit_cast(h4, v);
}

// Sixteen positions of one dimension (two 16-byte words): positions at or past
// `valid` become 0 (cache slots not yet written may hold any bits, and 0 * NaN
// would reach the sum), and position `at` (if in 0 .. 15) becomes `fresh`.
__device__ __forceinline__ void fix_run(uint4* run, int valid, int at, uint32_t fresh) {
  uint32_t w[8] = {run[0].x, run[0].y, run[0].z, run[0].w, run[1].x, run[1].y, run[1].z, run[1].w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {  // word i holds positions 2 i (low half) and 2 i + 1
    uint32_t v = w[i] & ((2 * i < valid ? 0x0000FFFFu : 0u) | (2 * i + 1 < valid ? 0xFFFF0000u : 0u));
    v = 2 * i == at ? (v & 0xFFFF0000u) | fresh : v;
    v = 2 * i + 1 == at ? (v & 0x0000FFFFu) | (fresh << 16) : v;
    w[i] = v;
  }
  run[0] = make_uint4(w[0], w[1], w[2], w[3]);
  run[1] = make_uint4(w[4], w[5], w[6], w[7]);
}

__device__ __forceinline__ float2 load_agent2(const float* p) {
  const uint64_t v = __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<float*>(p)), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float(static_cast<uint32_t>(v)), __uint_as_float(static_cast<uint32_t>(v >> 32)));
}

// Online-softmax merge of partials [cb, ce) of one query head h, dimensions
// d0 .. d0 + 7: stats (max in base-2 units, weight sum) at st[(c * G + h) * 2],
// unnormalised outputs at pp[(c * G + h) * D + d0 ..].  Returns the merged max
// m, weight sum l and unnormalised output acc, taking the partials in index
// order.  Each round fetches kMergeUnroll partials before using any.
__device__ __forceinline__ void merge_range(const float* st, const float* pp, int G, int D, int h, int d0, int cb,
                                            int ce, float& m, float& l, float acc[8]) {
  m = -INFINITY;
  l = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.f;
  for (int c0 = cb; c0 < ce; c0 += kMergeUnroll) {
    float2 sv[kMergeUnroll], pv[kMergeUnroll][4];
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      const int cc = min(c0 + u, ce - 1);
      sv[u] = load_agent2(st + (static_cast<int64_t>(cc) * G + h) * 2);
      const float* src = pp + (static_cast<int64_t>(cc) * G + h) * D + d0;
#pragma unroll
      for (int k = 0; k < 4; ++k) pv[u][k] = load_agent2(src + 2 * k);
    }
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      if (c0 + u < ce) {
        const float mn = fmaxf(m, sv[u].x);   // every partial's max is finite
        const float sc = exp2f(m - mn);       // 0 on the first partial (m = -inf)
        const float w = exp2f(sv[u].x - mn);
        l = l * sc + w * sv[u].y;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          acc[2 * k] = acc[2 * k] * sc + w * pv[u][k].x;
          acc[2 * k + 1] = acc[2 * k + 1] * sc + w * pv[u][k].y;
        }
        m = mn;
      }
    }
  }
}

// kLlReps = 0: the ticket merge; 1, 2, 4 or 8: the flagged-word merge with up
// to that many outputs per thread (the power of two at or above the plan's
// reps) and up to kLlSlots / kLlReps chunks per range.
template <int D, int kLlReps>
__global__ __launch_bounds__(kThreads) void decode_attention_kernel(AttnArgs a) {
  constexpr bool LL = kLlReps > 0;
  constexpr int kReps = LL ? kLlReps : 1;
  constexpr int kRange = kLlSlots / kReps;  // chunk slots per output
  constexpr int kSeg = D / 4;        // dimensions of a lane group's share of one key
  constexpr int kSteps = D / 16;     // score MFMAs per wave
  constexpr int kTiles = D / 64;     // 16-dimension output tiles per wave
  constexpr int kQS = D + 8;         // LDS row strides (padded against bank conflicts)
  constexpr int kSS = kChunk + 4;
  constexpr int kPS = kChunk + 8;
  __shared__ __align__(16) _Float16 q_hl[kRows * kQS];
  __shared__ __align__(16) float s_raw[kRows * kSS];
  __shared__ __align__(16) _Float16 p_hl[kRows * kPS];
  __shared__ int last;
  __shared__ uint32_t flag_s;
  __shared__ __align__(16) uint16_t new_k[D], new_v[D];  // the newest token's key and value, fp16
  // Flagged-word merge: (max, weight sum, output) of each chunk range's merge.
  __shared__ float comb[LL ? 3 * kThreads : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, lg = lane >> 4;
  const int c = blockIdx.x, g = blockIdx.y, chunks = gridDim.x;
  const int G = a.group, L = a.length, cap = a.capacity;
  const int t0 = c * kChunk;
  const int newest = L - 1;
  // The loads below are unconditional (addresses clamped in range, unused
  // values dropped later) and all issued before any is waited for: a load
  // inside a branch gets its use (and the wait for it) pulled into the
  // branch, which would hold the wave's later loads back.
  const uint32_t epoch = LL ? __hip_atomic_load(a.epochs + g, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;

  // The group's queries (item tid: head h, dimensions d0 .. d0 + 7) first,
  // then the newest token's key and value (fp32): a wave's loads complete in
  // order, so the queries' conversion runs while the cache tiles are in
  // flight, and the chunk that holds position L - 1 has its new key and value
  // before its scores (behind the cache loads they would hold that chunk,
  // and every merge waiting for it, back).
  static_assert(kMaxGroup * (D / 8) <= kThreads, "one query item per thread");
  const int qh = tid / (D / 8), qd0 = (tid % (D / 8)) * 8;
  const bool q_item = tid < kMaxGroup * (D / 8);
  float4 qx0, qx1;
  {
    const float4* src =
        reinterpret_cast<const float4*>(a.q + (static_cast<int64_t>(g) * G + min(qh, G - 1)) * D + (q_item ? qd0 : 0));
    qx0 = src[0];
    qx1 = src[1];
  }
  const bool holds_newest = newest >= t0 && newest < t0 + kChunk;  // uniform per workgroup
  const float4 kx = reinterpret_cast<const float4*>(a.k_new + static_cast<int64_t>(g) * D)[tid % (D / 4)];
  const float4 vx = reinterpret_cast<const float4*>(a.v_new + static_cast<int64_t>(g) * D)[tid % (D / 4)];
  __builtin_amdgcn_sched_barrier(0);  // these ahead of the cache tiles

  // 1. Loads.  Key: this lane's position (column `col` of the wave's 16) and
  // its lane group's quarter of the dimensions.  Value: sixteen positions of
  // each of the wave's output dimensions.  Every address lies below the
  // capacity, which is a multiple of the chunk.
  const int tk = t0 + 16 * wave + col;
  uint16_t* krow = a.k_cache + (static_cast<int64_t>(g) * cap + tk) * D + lg * kSeg;
  uint4 kr[kSeg / 8];
#pragma unroll
  for (int i = 0; i < kSeg / 8; ++i) kr[i] = reinterpret_cast<const uint4*>(krow)[i];
  uint4 vr[kTiles][2];
#pragma unroll
  for (int nt = 0; nt < kTiles; ++nt) {
    const int d = wave * (D / 4) + 16 * nt + col;
    const uint4* vrow =
        reinterpret_cast<const uint4*>(a.v_cache + (static_cast<int64_t>(g) * D + d) * cap + t0 + 16 * lg);
    vr[nt][0] = vrow[0];
    vr[nt][1] = vrow[1];
  }
  // Every load is issued before any of them is waited for.
  __builtin_amdgcn_sched_barrier(0);
  if (LL && tid == 0) flag_s = epoch + 1u;
  // Queries of the group -> hi / lo rows of the A operand.
  if (q_item) {
    const int h = qh, d0 = qd0;
    const bool live = h < G;  // heads past the group get zero rows
    const float v[8] = {live ? qx0.x : 0.f, live ? qx0.y : 0.f, live ? qx0.z : 0.f, live ? qx0.w : 0.f,
                        live ? qx1.x : 0.f, live ? qx1.y : 0.f, live ? qx1.z : 0.f, live ? qx1.w : 0.f};
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const _Float16 h0 = static_cast<_Float16>(v[2 * i]), h1 = static_cast<_Float16>(v[2 * i + 1]);
      hi[i] = pack2(h0, h1);
      lo[i] = pack2(static_cast<_Float16>((v[2 * i] - static_cast<float>(h0)) * kLo),
                    static_cast<_Float16>((v[2 * i + 1] - static_cast<float>(h1)) * kLo));
    }
    *reinterpret_cast<uint4*>(q_hl + h * kQS + d0) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    *reinterpret_cast<uint4*>(q_hl + (h + kMaxGroup) * kQS + d0) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
  }
  // The newest token: its key and value enter the cache as fp16 and are used
  // in that form; no other workgroup reads position L - 1.  The chunk's
  // workgroup rounds them into LDS (four values per thread of its first wave)
  // and writes them to the cache; after the barrier the lanes that hold
  // position L - 1 take them from LDS.
  // The cache stores themselves wait until the chunk's outputs are out
  // (write_newest): every workgroup barrier before then would wait for them.
  uint2 kp = {0u, 0u}, vp = {0u, 0u};
  if (holds_newest && tid < D / 4) {
    const _Float16 k4[4] = {static_cast<_Float16>(kx.x), static_cast<_Float16>(kx.y), static_cast<_Float16>(kx.z),
                            static_cast<_Float16>(kx.w)};
    const _Float16 v4[4] = {static_cast<_Float16>(vx.x), static_cast<_Float16>(vx.y), static_cast<_Float16>(vx.z),
                            static_cast<_Float16>(vx.w)};
    kp = make_uint2(pack2(k4[0], k4[1]), pack2(k4[2], k4[3]));
    vp = make_uint2(pack2(v4[0], v4[1]), pack2(v4[2], v4[3]));
    *reinterpret_cast<uint2*>(new_k + 4 * tid) = kp;
    *reinterpret_cast<uint2*>(new_v + 4 * tid) = vp;
  }
  auto write_newest = [&]() __attribute__((always_inline)) {
    if (holds_newest && tid < D / 4) {
      *reinterpret_cast<uint2*>(a.k_cache + (static_cast<int64_t>(g) * cap + newest) * D + 4 * tid) = kp;
      const uint32_t vh[4] = {vp.x & 0xFFFFu, vp.x >> 16, vp.y & 0xFFFFu, vp.y >> 16};
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a.v_cache[(static_cast<int64_t>(g) * D + 4 * tid + i) * cap + newest] = static_cast<uint16_t>(vh[i]);
    }
  };
  __syncthreads();
  if (holds_newest && tk == newest) {
#pragma unroll
    for (int i = 0; i < kSeg / 8; ++i) kr[i] = *reinterpret_cast<const uint4*>(new_k + lg * kSeg + 8 * i);
  }

  // 2. Scores of the wave's 16 positions: row r of the result is head r's hi
  // part (r < 8) or head r - 8's lo part; lane l holds rows 4 * (l / 16) + j
  // of column l % 16.  The contraction index k = 4 * lg + j of step `ks` is
  // dimension lg * D / 4 + 4 * ks + j, for the A and the B operand alike.
  {
    f4 acc = {0.f, 0.f, 0.f, 0.f};
    const _Float16* qa = q_hl + col * kQS + lg * kSeg;
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks) {
      const h4 av = *reinterpret_cast<const h4*>(qa + 4 * ks);
      acc = __builtin_amdgcn_mfma_f32_16x16x16f16(av, half4_at(kr, ks), acc, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) s_raw[(4 * lg + j) * kSS + 16 * wave + col] = acc[j];
  }
  __syncthreads();

  // 3. Chunk softmax: thread -> head tid / 32, positions 2 * (tid % 32) + {0, 1};
  // the 32 threads of a head are one half of a wave.
  {
    const int h = tid >> 5, tt = 2 * (tid & 31);
    float s[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float v = (s_raw[h * kSS + tt + e] + s_raw[(h + kMaxGroup) * kSS + tt + e] * kInvLo) * a.scale2;
      s[e] = t0 + tt + e < L ? v : -INFINITY;
    }
    const float m = half_wave_reduce<true>(fmaxf(s[0], s[1]));
    const float p0 = exp2f(s[0] - m), p1 = exp2f(s[1] - m);
    const float l = half_wave_reduce<false>(p0 + p1);
    uint32_t hi = 0u, lo = 0u;
    if (h < G) {
      const _Float16 h0 = static_cast<_Float16>(p0), h1 = static_cast<_Float16>(p1);
      hi = pack2(h0, h1);
      lo = pack2(static_cast<_Float16>((p0 - static_cast<float>(h0)) * kLo),
                 static_cast<_Float16>((p1 - static_cast<float>(h1)) * kLo));
      if ((tid & 31) == 0) {
        if constexpr (LL) {
          // the max and weight sum words follow the head's D output words
          const __amdgpu_buffer_rsrc_t rw = head_words(a.ll, g);
          const uint32_t wo = static_cast<uint32_t>(((c * G + h) * (D + 2) + D) * 8);
          ll_put(rw, wo, 0, m, flag_s);
          ll_put(rw, wo, 8, l, flag_s);
        } else {
          float* st = a.stats + ((static_cast<int64_t>(g) * chunks + c) * G + h) * 2;
          store_agent(st, m);
          store_agent(st + 1, l);
        }
      }
    }
    *reinterpret_cast<uint32_t*>(p_hl + h * kPS + tt) = hi;
    *reinterpret_cast<uint32_t*>(p_hl + (h + kMaxGroup) * kPS + tt) = lo;
  }
  __syncthreads();

  // The value runs change only here, where they are first used, so the
  // scores never wait for the value loads.  Only a run holding the newest
  // position or reaching past it changes (valid length L - first of at most
  // 16; 16 when the newest is its last).
  if (holds_newest) {
    const int first = t0 + 16 * lg;  // position of element 0 of this lane's value runs
    const int at = newest - first;
    if (L - first <= 16) {
#pragma unroll
      for (int nt = 0; nt < kTiles; ++nt) {
        const int d = wave * (D / 4) + 16 * nt + col;
        fix_run(vr[nt], L - first, at, (at >= 0 && at < 16) ? new_v[d] : 0u);
      }
    }
  }

  // 4. Chunk output of the wave's D / 4 dimensions: the contraction index of
  // step `ks` is position 16 * lg + 4 * ks + j, matching the value runs.  Rows
  // 0 .. 7 of the result sit in lanes 0 .. 31 and their lo rows 32 lanes up.
  // Every tile's MFMAs come before the first store: stores count in the
  // same wait counter as loads, so a tile's wait for its value loads would
  // otherwise also wait for the previous tiles' stores to be acknowledged.
  {
    h4 pa[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) pa[ks] = *reinterpret_cast<const h4*>(p_hl + col * kPS + 16 * lg + 4 * ks);
    f4 acc[kTiles];
#pragma unroll
    for (int nt = 0; nt < kTiles; ++nt) {
      acc[nt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa[ks], half4_at(vr[nt], ks), acc[nt], 0, 0, 0);
    }
    if constexpr (LL) {
      // Word (head 4 lg + j, dimension wave * D / 4 + 16 nt + col) of this
      // chunk's block: a lane offset plus a constant per (nt, j); lanes of
      // the lo rows and of heads past G get an offset that drops the store.
      const uint32_t flag = flag_s;
      const __amdgpu_buffer_rsrc_t rw = head_words(a.ll, g);
      const uint32_t base = static_cast<uint32_t>(((c * G + 4 * lg) * (D + 2) + wave * (D / 4) + col) * 8);
      uint32_t lo[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) lo[j] = lane < 32 && 4 * lg + j < G ? base : kDropOffset;
#pragma unroll
      for (int nt = 0; nt < kTiles; ++nt) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          ll_put(rw, lo[j], (j * (D + 2) + 16 * nt) * 8, acc[nt][j] + upper_half(acc[nt][j]) * kInvLo, flag);
      }
    } else {
#pragma unroll
      for (int nt = 0; nt < kTiles; ++nt) {
        const int d = wave * (D / 4) + 16 * nt + col;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float up = upper_half(acc[nt][j]);
          const int h = 4 * lg + j;
          if (lane < 32 && h < G)
            store_agent(a.part + ((static_cast<int64_t>(g) * chunks + c) * G + h) * D + d, acc[nt][j] + up * kInvLo);
        }
      }
    }
  }

  write_newest();
  if constexpr (LL) {
    // 5'. Flagged-word merge (no barrier before it: a workgroup barrier's
    // fence would wait for this workgroup's word stores to be acknowledged,
    // and a reader checks every word's flag anyway).  Thread (range sub,
    // index st) merges outputs f0, f0 + T, ... over the range's chunks.
    const uint32_t flag = flag_s;
    const LlPlan pl = a.llp;
    if (c >= pl.workers) return;  // no outputs here (uniform)
    // This workgroup's own word stores acknowledged first: a poll issued
    // behind them would wait for them anyway, and one issued a little later
    // finds the other chunks' words in one round more often (measured with
    // per-phase timestamps: 0.5 us less per call at 640 positions).
    __builtin_amdgcn_s_waitcnt(0);
    const int T = 1 << pl.tlog;   // threads per chunk range
    const int sub = __builtin_amdgcn_readfirstlane(tid >> pl.tlog);  // uniform per wave (T >= 64)
    const int st = tid & (T - 1);
    const int cb = sub * pl.cs;
    const int nc = max(0, min(chunks - cb, pl.cs));  // the range's chunks
    // Outputs c * per + st + T * r for r < nr; per and T are multiples of 64,
    // so nr is the same for the whole wave.
    const int st0 = __builtin_amdgcn_readfirstlane(st & ~63);
    const int nr = st0 < pl.per ? min(pl.reps, (pl.per - st0 + T - 1) >> pl.tlog) : 0;  // at most kReps
    const int f0 = c * pl.per + st;
    // Word offsets in a chunk's block of G * (D + 2): output f0, and its
    // head's max (the weight sum follows).  With several outputs per thread
    // T is a multiple of D, so output f0 + T * r lies r * r_words further.
    const uint32_t o_b = static_cast<uint32_t>((f0 / D * (D + 2) + f0 % D) * 8);
    const uint32_t s_b = static_cast<uint32_t>((f0 / D * (D + 2) + D) * 8);
    const int r_bytes = T >= D ? T / D * (D + 2) * 8 : 0;
    const int c_bytes = G * (D + 2) * 8;
    const int b0 = cb * c_bytes;
    const __amdgpu_buffer_rsrc_t rw = head_words(a.ll, g);
    // Each (output r, chunk k) pair's output word and its chunk's max and
    // weight-sum words, every load of a round issued before any is tested:
    // lanes of a wave read consecutive output words, and the max and sum
    // words of a head.  Slot (r, k) is compile-time; r < nr and k < nc are
    // uniform, and so is each load's block offset.
    u32x2 w[kReps][kRange][3];
    bool ok = true;
    for (int spin = 0;; ++spin) {
      asm volatile("" ::: "memory");  // every round loads afresh
#pragma unroll
      for (int r = 0; r < kReps; ++r) {
#pragma unroll
        for (int k = 0; k < kRange; ++k) {
          if (r < nr && k < nc) {
            const uint32_t blk = __builtin_amdgcn_readfirstlane(b0 + k * c_bytes + r * r_bytes);
            w[r][k][0] = ll_get(rw, o_b, blk);
            w[r][k][1] = ll_get(rw, s_b, blk);
            w[r][k][2] = ll_get(rw, s_b, blk + 8);
          }
        }
      }
      uint32_t stale = 0u;
#pragma unroll
      for (int r = 0; r < kReps; ++r) {
#pragma unroll
        for (int k = 0; k < kRange; ++k) {
          if (r < nr && k < nc) stale |= (w[r][k][0].y ^ flag) | (w[r][k][1].y ^ flag) | (w[r][k][2].y ^ flag);
        }
      }
      if (stale == 0u) break;
      if (spin >= kLlSpin) {
        ok = false;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (!ok) __hip_atomic_store(a.error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // Online-softmax merge of the range's chunks in chunk order, one output
    // at a time.
    float m = -INFINITY, l = 0.f, acc = 0.f;
#pragma unroll
    for (int r = 0; r < kReps; ++r) {
      if (r < nr) {
        m = -INFINITY;
        l = 0.f;
        acc = 0.f;
#pragma unroll
        for (int k = 0; k < kRange; ++k) {
          if (k < nc) {
            const float pm = __uint_as_float(w[r][k][1].x);
            const float mn = fmaxf(m, pm);  // every chunk's max is finite
            // 2^x on the hardware's exponential: results below 2^-126 become
            // 0, a change far below the fp16 output's rounding (the largest
            // chunk weight is 1).  0 on the first chunk (m = -inf).
            const float sc = __builtin_amdgcn_exp2f(m - mn);
            const float wt = __builtin_amdgcn_exp2f(pm - mn);
            l = l * sc + wt * __uint_as_float(w[r][k][2].x);
            acc = acc * sc + wt * __uint_as_float(w[r][k][0].x);
            m = mn;
          }
        }
        if (pl.split == 1)
          a.out[static_cast<int64_t>(g) * G * D + f0 + T * r] =
              __builtin_bit_cast(unsigned short, static_cast<_Float16>(acc / l));
      }
    }
    if (pl.split > 1 && nr > 0) {  // one output per thread (reps = 1)
      comb[tid] = m;
      comb[kThreads + tid] = l;
      comb[2 * kThreads + tid] = acc;
    }
    if (pl.split > 1) {
      // Combine the ranges' results in range (chunk) order.
      __syncthreads();
      if (sub == 0 && nr > 0) {
        float m = comb[st], l = comb[kThreads + st], acc = comb[2 * kThreads + st];
        for (int s2 = 1; s2 < pl.split && s2 * pl.cs < chunks; ++s2) {
          const int t = s2 * T + st;
          const float mn = fmaxf(m, comb[t]);
          const float sc = exp2f(m - mn);
          const float wt = exp2f(comb[t] - mn);
          l = l * sc + wt * comb[kThreads + t];
          acc = acc * sc + wt * comb[2 * kThreads + t];
          m = mn;
        }
        a.out[static_cast<int64_t>(g) * G * D + f0] = __builtin_bit_cast(unsigned short, static_cast<_Float16>(acc / l));
      }
    }
    // Workgroup 0 of the head has now read every chunk's words (thread 0 alone
    // with one chunk range; every range before the barrier above otherwise),
    // so every workgroup of the head has read the epoch: advance it for the
    // next call.
    if (c == 0 && tid == 0) __hip_atomic_store(a.epochs + g, flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }

  // 5. Merge.  The last workgroup of this chunk's merge group to finish
  // merges the group; with several groups, the last group merger merges the
  // group results.  Tickets reset themselves once every member has arrived.
  const int gsz = a.group_chunks;
  const int ngroups = (chunks + gsz - 1) / gsz;
  const int grp = c / gsz;
  const int cb = grp * gsz, ce = min(chunks, cb + gsz);
  uint32_t* tix = a.tickets + g * (a.max_groups + 1);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0)
    last = __hip_atomic_fetch_add(&tix[grp], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
           static_cast<uint32_t>(ce - cb - 1);
  __syncthreads();
  if (!last) return;
  if (tid == 0) __hip_atomic_store(&tix[grp], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const float* st = a.stats + static_cast<int64_t>(g) * chunks * G * 2;
  const float* pp = a.part + static_cast<int64_t>(g) * chunks * G * D;
  float* st2 = a.stats2 + static_cast<int64_t>(g) * kMaxGroups * G * 2;
  float* pp2 = a.part2 + static_cast<int64_t>(g) * kMaxGroups * G * D;
  if (ngroups > 1) {
    for (int it = tid; it < G * (D / 8); it += kThreads) {
      const int h = it / (D / 8), d0 = (it % (D / 8)) * 8;
      float m, l, acc[8];
      merge_range(st, pp, G, D, h, d0, cb, ce, m, l, acc);
      if (d0 == 0) {
        store_agent(st2 + (grp * G + h) * 2, m);
        store_agent(st2 + (grp * G + h) * 2 + 1, l);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) store_agent(pp2 + (static_cast<int64_t>(grp) * G + h) * D + d0 + k, acc[k]);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0)
      last = __hip_atomic_fetch_add(&tix[a.max_groups], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             static_cast<uint32_t>(ngroups - 1);
    __syncthreads();
    if (!last) return;
    if (tid == 0) __hip_atomic_store(&tix[a.max_groups], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  for (int it = tid; it < G * (D / 8); it += kThreads) {
    const int h = it / (D / 8), d0 = (it % (D / 8)) * 8;
    float m, l, acc[8];
    if (ngroups > 1) merge_range(st2, pp2, G, D, h, d0, 0, ngroups, m, l, acc);
    else merge_range(st, pp, G, D, h, d0, cb, ce, m, l, acc);
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = pack2(static_cast<_Float16>(acc[2 * i] / l), static_cast<_Float16>(acc[2 * i + 1] / l));
    *reinterpret_cast<uint4*>(a.out + (static_cast<int64_t>(g) * G + h) * D + d0) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

}  // namespace

int attention_chunks(int length) { return (length + kChunk - 1) / kChunk; }

size_t attention_scratch_bytes(int n_kv_heads, int group, int head_dim, int length) {
  return static_cast<size_t>(n_kv_heads) * (attention_chunks(length) + kMaxGroups) * group * (head_dim + 2) *
         sizeof(float);
}

bool attention_ll_fits(int n_kv_heads, int group, int head_dim, int length, const AttnExchange* ex) {
  const int chunks = attention_chunks(length);
  static_assert(kAttnHeadWords >= size_t{kMaxLlChunks} * kMaxGroup * (256 + 2), "attention exchange region");
  if (!(ex && ex->ll && chunks <= kMaxLlChunks && n_kv_heads <= ex->heads && group <= kMaxGroup && head_dim <= 256))
    return false;
  const LlPlan p = ll_plan(group * head_dim, chunks);
  const int reps = p.reps <= 1 ? 1 : p.reps <= 2 ? 2 : p.reps <= 4 ? 4 : 8;
  return p.reps <= 8 && p.cs <= kLlSlots / reps;
}

template <int D>
void launch_ll(int reps, dim3 grid, const AttnArgs& a, hipStream_t stream) {
  switch (reps) {
    case 1: hipLaunchKernelGGL((decode_attention_kernel<D, 1>), grid, dim3(kThreads), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((decode_attention_kernel<D, 2>), grid, dim3(kThreads), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((decode_attention_kernel<D, 4>), grid, dim3(kThreads), 0, stream, a); break;
    default: hipLaunchKernelGGL((decode_attention_kernel<D, 8>), grid, dim3(kThreads), 0, stream, a); break;
  }
}

int launch_decode_attention(const float* q, const float* k_new, const float* v_new, uint16_t* k_cache,
                            uint16_t* v_cache, int n_heads, int n_kv_heads, int head_dim, int length, int capacity,
                            uint16_t* out, Scratch* sc, const AttnExchange* ex, hipStream_t stream) {
  if (n_heads % n_kv_heads != 0 || n_heads / n_kv_heads > kMaxGroup || capacity % kChunk != 0 ||
      length < 1 || length > capacity || n_kv_heads < 1 || n_kv_heads >= (kMaxTickets - 2) / 2 ||
      sc->n_tickets < kMaxTickets)
    return hip_fail(hipErrorInvalidValue, "decode attention: shape outside the kernel's limits");
  const int rc = require_scratch(sc, attention_scratch_bytes(n_kv_heads, n_heads / n_kv_heads, head_dim, length));
  if (rc != W4A8_OK) return rc;
  const int chunks = attention_chunks(length);
  const int group = n_heads / n_kv_heads;
  AttnArgs a{};
  a.q = q;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.out = out;
  a.part = static_cast<float*>(sc->work);
  a.stats = a.part + static_cast<size_t>(n_kv_heads) * chunks * group * head_dim;
  a.part2 = a.stats + static_cast<size_t>(n_kv_heads) * chunks * group * 2;
  a.stats2 = a.part2 + static_cast<size_t>(n_kv_heads) * kMaxGroups * group * head_dim;
  // The tickets (one per merge group and one for the group results, per KV
  // head) must fit the library's ticket array: many KV heads get fewer groups.
  a.max_groups = std::min(kMaxGroups, (kMaxTickets - 2) / n_kv_heads - 1);
  a.tickets = sc->tickets + 1;
  a.group_chunks = std::max(kGroupChunks, (chunks + a.max_groups - 1) / a.max_groups);
  a.group = group;
  a.length = length;
  a.capacity = capacity;
  a.scale2 = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(head_dim)));
  const dim3 grid(chunks, n_kv_heads);
  if (attention_ll_fits(n_kv_heads, group, head_dim, length, ex)) {
    a.ll = ex->ll;
    a.llp = ll_plan(group * head_dim, chunks);
    const int reps = a.llp.reps <= 1 ? 1 : a.llp.reps <= 2 ? 2 : a.llp.reps <= 4 ? 4 : 8;
    a.epochs = ex->epochs;
    a.error = ex->error;
    switch (head_dim) {
      case 64: launch_ll<64>(reps, grid, a, stream); break;
      case 128: launch_ll<128>(reps, grid, a, stream); break;
      case 256: launch_ll<256>(reps, grid, a, stream); break;
      default: return hip_fail(hipErrorInvalidValue, "decode attention: head_dim must be 64, 128 or 256");
    }
  } else {
    switch (head_dim) {
      case 64: hipLaunchKernelGGL((decode_attention_kernel<64, 0>), grid, dim3(kThreads), 0, stream, a); break;
      case 128: hipLaunchKernelGGL((decode_attention_kernel<128, 0>), grid, dim3(kThreads), 0, stream, a); break;
      case 256: hipLaunchKernelGGL((decode_attention_kernel<256, 0>), grid, dim3(kThreads), 0, stream, a); break;
      default: return hip_fail(hipErrorInvalidValue, "decode attention: head_dim must be 64, 128 or 256");
    }
  }
  W4A8_HIP(hipGetLastError());
  return W4A8_OK;
}

}  // namespace w4a8
