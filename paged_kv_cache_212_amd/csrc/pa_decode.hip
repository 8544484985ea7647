// PagedAttention decode on gfx950.
//
// For every sequence b and KV head g, waves walk the block table from
// logical to physical blocks and read the 16-token K and V tiles they need,
// in logical order (page 3, abeam.tech review, sections 「用語解説」 (block
// table) and 「モデル構造ではなくサービング基盤の変更」: the kernel follows the
// table to read the KV it needs).  They compute softmax(scale * q.K^T) V for
// the G query heads that share KV head g with an online (running max,
// running sum) softmax.  A context cut into pieces leaves per-piece (max,
// sum, weighted V) partials that merge_kernel combines with a log-sum-exp
// reduction; paging changes where K/V live, not the result (page 3, section
// 「よくある質問」; page 4, FAQ).
//
// Work distribution:
//   * decode_split_kernel: the batch's (sequence, KV head, run of blocks)
//     units cut into equal chunks, one per wave (4 waves per workgroup, one
//     workgroup per compute unit);
//   * decode_fixed_kernel: one wave per (KV head, fixed partition, sequence).
// Engines (one wave attends one (b, g) range of blocks):
//   * attend4 (fp16/bf16 and 8-bit codes, G <= 16): 4 blocks per step on the
//     4x4x4 16-block MFMA with broadcast operands, ceil(G / 4) groups of 4
//     query heads per K/V load.  P.V takes P split into a high and a low
//     half-precision part, so the weights keep ~16 (bf16) / ~22 (fp16)
//     significant bits.
//   * decode_generic_kernel (any dtype, fp32 pools): plain fp32 FMAs.
// Scores are kept in the log2 domain (scale * log2(e) folded in) and
// exponentiated with exp2.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <cmath>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>

#include "pa_device.h"
#include "pa_mfma.h"

namespace pa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxGroup = 16;  // query heads per KV head supported

struct Params {
  float* out;          // [B][Hq][D]
  float* part_m;       // [B][Hq][maxP]   running max (log2 domain) per partition
  float* part_l;       // [B][Hq][maxP]   sum of exp2(s - m)
  float* part_acc;     // [B][Hq][maxP][D] sum of exp2(s - m) * v
  int* counters;       // [B][Hkv] slots written for a (sequence, KV head) (even split)
  const void* k_new;   // [B][Hkv][D] new token of each sequence (fused append), or null
  const void* v_new;
  const int64_t* slots;  // [B] slot of each new token (fused append)
  void* kpool_w;       // writable pools (fused append)
  void* vpool_w;
  int write_new_in_merge;  // fused append: the merge kernel writes the new tokens
                           // to their slots (the attention kernel only uses them)
  const void* q;       // [B][Hq][D]
  const void* kpool;
  const void* vpool;
  const int32_t* tables;
  const int32_t* lens;
  int B, Hq, Hkv, G, D;
  int num_blocks, max_blocks, max_ctx;
  int P, maxP;
  float scale_log2;
  float out_scale;     // factor of the final rows (V scale of a quantized cache, else 1)
  float enc_k, enc_v;  // quantized cache, fused append: fp32 reciprocals of the K/V scales
  int window;          // sliding window: attend the last `window` positions (0: all)
  int range_ticks;     // even split: cost of starting a (sequence, KV head) range, in
                       // kUnitTicks per unit
  // Shared prefixes (pa_decode_step_shared): prefix[b] positions of sequence
  // b were attended by the prefix pass in pre_pieces key ranges, whose
  // partials are in slot p of pre_out (unnormalised weighted sums of V) and
  // pre_ml (log2-domain max and sum of 2^(s - max)), each slot it wrote
  // stamped with the call's epoch; the even split attends the rest and the
  // merge folds them all (null: no prefix pass).
  const int32_t* prefix;       // [B]
  const float* pre_out;        // [pre_pieces][B][Hq][D]
  const float2* pre_ml;        // [pre_pieces][B][Hq]
  uint32_t* pre_stamp;         // [pre_pieces][B][Hq] (the merge clears what it reads)
  uint32_t epoch;
  int pre_pieces;
};

__device__ inline bool len_valid(int L, const Params& pr) {
  return L >= 0 && L <= pr.max_ctx && L <= pr.max_blocks * kBlockSize;
}

// Whether `pre` is a usable shared prefix of a sequence of length L: a
// whole number of blocks, leaving at least the sequence's last position.
__device__ inline bool prefix_ok(int pre, int L) {
  return pre > 0 && pre < L && pre % kBlockSize == 0;
}

// First position a sequence of length L attends: the end of its shared
// prefix when a prefix pass attended that (pre; an unusable one counts as
// none here, and the merge turns the row into NaN), else L - window with a
// sliding window, else 0.  Table entries of blocks wholly before it are never
// read (they may have been released).
__device__ inline int first_pos(int L, const Params& pr, int pre = 0) {
  if (prefix_ok(pre, L)) return pre;
  return pr.window > 0 ? max(0, L - pr.window) : 0;
}
__device__ inline int prefix_of(const Params& pr, int b) { return pr.prefix ? pr.prefix[b] : 0; }

// Zero rows for empty sequences, NaN rows for sequences whose length is out of
// the declared bounds.  Done by partition 0's workgroup only.
__device__ inline void write_trivial_rows(const Params& pr, int b, int g, int L) {
  const float v = (L == 0) ? 0.f : __builtin_nanf("");
  const int n = pr.G * pr.D;
  float* o = pr.out + (static_cast<int64_t>(b) * pr.Hq + g * pr.G) * pr.D;
  for (int i = threadIdx.x; i < n; i += blockDim.x) o[i] = v;
}

// ---------------------------------------------------------------------------
// Generic partition kernel: 256 threads; tokens in chunks of 128.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_generic_kernel(Params pr) {
  using bits = typename T::bits;
  constexpr int NT = 256, CH = 128;
  constexpr int ACC = kMaxGroup * D / NT;
  __shared__ float sq[kMaxGroup][D];
  __shared__ float ss[kMaxGroup][CH];
  __shared__ float s_m[kMaxGroup], s_l[kMaxGroup], s_alpha[kMaxGroup];
  __shared__ int s_bad;

  const int p = blockIdx.x, g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int G = pr.G;
  const int L = pr.lens[b];
  if (!len_valid(L, pr) || L == 0) {
    if (p == 0) write_trivial_rows(pr, b, g, L);
    return;
  }
  // partitions count from the one holding the first attended position
  const int f = first_pos(L, pr), p0 = f / pr.P;
  const int np = (L + pr.P - 1) / pr.P - p0;
  if (p >= np) return;
  const int tok0 = max((p + p0) * pr.P, f), tok1 = min(L, (p + p0 + 1) * pr.P);

  const bits* q = static_cast<const bits*>(pr.q) +
                  (static_cast<int64_t>(b) * pr.Hq + g * G) * D;
  for (int i = tid; i < G * D; i += NT) sq[i / D][i % D] = T::to_float(q[i]);
  if (tid < G) {
    s_m[tid] = -INFINITY;
    s_l[tid] = 0.f;
  }
  if (tid == 0) s_bad = 0;
  float acc[ACC];
#pragma unroll
  for (int k = 0; k < ACC; ++k) acc[k] = 0.f;
  __syncthreads();

  const bits* kp = static_cast<const bits*>(pr.kpool);
  const bits* vp = static_cast<const bits*>(pr.vpool);
  const int32_t* trow = pr.tables + static_cast<int64_t>(b) * pr.max_blocks;

  for (int c0 = tok0; c0 < tok1; c0 += CH) {
    const int nv = min(CH, tok1 - c0);
    for (int idx = tid; idx < G * CH; idx += NT) {
      const int h = idx / CH, t = idx % CH;
      float s = -INFINITY;
      if (t < nv) {
        const int pos = c0 + t;
        const int phys = trow[pos / kBlockSize];
        if (phys < 0 || phys >= pr.num_blocks) {
          s_bad = 1;
        } else {
          const bits* kt = kp + tile_base(phys, g, pr.Hkv, D);
          const int tt = pos % kBlockSize;
          float dot = 0.f;
          for (int d = 0; d < D; ++d) dot = fmaf(sq[h][d], T::to_float(kt[k_elem<T>(tt, d)]), dot);
          s = dot * pr.scale_log2;
        }
      }
      ss[h][t] = s;
    }
    __syncthreads();
    if (tid < G) {
      const int h = tid;
      float cm = -INFINITY;
      for (int t = 0; t < nv; ++t) cm = fmaxf(cm, ss[h][t]);
      const float mo = s_m[h], mn = fmaxf(mo, cm);
      const float alpha = exp2f(mo - mn);
      float sum = 0.f;
      for (int t = 0; t < nv; ++t) {
        const float e = exp2f(ss[h][t] - mn);
        ss[h][t] = e;
        sum += e;
      }
      s_l[h] = s_l[h] * alpha + sum;
      s_m[h] = mn;
      s_alpha[h] = alpha;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < ACC; ++k) {
      const int idx = tid + k * NT;
      if (idx < G * D) {
        const int h = idx / D, d = idx % D;
        float a = acc[k] * s_alpha[h];
        for (int t = 0; t < nv; ++t) {
          const int pos = c0 + t;
          const int phys = trow[pos / kBlockSize];
          if (phys < 0 || phys >= pr.num_blocks) continue;
          const bits* vt = vp + tile_base(phys, g, pr.Hkv, D);
          a = fmaf(ss[h][t], T::to_float(vt[v_elem<T>(pos % kBlockSize, d, D)]), a);
        }
        acc[k] = a;
      }
    }
    __syncthreads();
  }

  const bool bad = s_bad != 0;
#pragma unroll
  for (int k = 0; k < ACC; ++k) {
    const int idx = tid + k * NT;
    if (idx >= G * D) continue;
    const int h = idx / D, d = idx % D;
    const int64_t row = static_cast<int64_t>(b) * pr.Hq + g * G + h;
    const float a = bad ? __builtin_nanf("") : acc[k];
    const float l = bad ? __builtin_nanf("") : s_l[h];
    if (np == 1) {
      pr.out[row * D + d] = a / l;
    } else {
      pr.part_acc[(row * pr.maxP + p) * D + d] = a;
      if (d == 0) {
        pr.part_m[row * pr.maxP + p] = bad ? 0.f : s_m[h];
        pr.part_l[row * pr.maxP + p] = l;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Matrix-core engine on the 4x4x4 16-block MFMA: NG groups of 4 query heads
// (G <= 4 * NG) per K/V load
// (v_mfma_f32_4x4x4_16b: sixteen independent 4x4x4 products per instruction,
// block k on lanes 4k..4k+3; with CBSZ=4 / ABID=a every block uses the A
// operand of block a).
//
// One step covers a quad of 4 consecutive blocks (64 tokens); lane l owns
// token l of the quad (block l/16, in-block token l%16).
//   QK: S (4 heads x 64 tokens) = Q . K^T over D/4 k-steps of 4 dims.  Step
//     s takes A = Q broadcast from block s%16 (register s/16 holds, at lane
//     4a+i, head i's dims 4*(16*(s/16) + a) .. +3) and B = K (lane l: dims
//     4s..4s+3 of token l).  Result: lane l holds S[head e][token l], e=0..3.
//   A 4x4 transpose inside each lane quad (DPP) turns that into lane 4a+i
//     holding S[head i][token 4a+e]: the softmax runs per lane over 4 tokens
//     of one head, and the probabilities are already the A operand of P.V.
//   PV: O (4 heads x 64 dims) += P (4 heads x 4 tokens) . V (4 tokens x 64
//     dims) for k-step a = tokens 4a..4a+3, A broadcast from block a, B lane
//     l = V[tokens 4a..4a+3][dim 64t + l]: half of one 16-byte load of the
//     V tile (8 consecutive tokens of a dim are contiguous).  O: lane l
//     holds dim 64t + l of heads e = 0..3.
// K loads: lane l reads 16-byte chunks c of token l (D/8 loads; per
// instruction 4 runs of 256 contiguous bytes).  V loads: per (block, half,
// 64-dim tile) one 16-byte load per lane, 1 KiB contiguous per instruction.
// ---------------------------------------------------------------------------
template <typename F, int... I>
__device__ __forceinline__ void unroll_seq(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
// Calls f(integral_constant<int, i>) for i = 0..N-1 (indices usable as
// instruction immediates).
template <int N, typename F>
__device__ __forceinline__ void unroll(F&& f) {
  unroll_seq(f, std::make_integer_sequence<int, N>{});
}

template <typename T>
struct Mfma4;

template <>
struct Mfma4<BF16> {
  template <int ABID>
  __device__ static inline f32x4_t mma(uint2 a, uint2 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(i16x4_t, a),
                                                  __builtin_bit_cast(i16x4_t, b), c, 4, ABID, 0);
  }
  __device__ static inline void split(const float pe[4], uint2& hi, uint2& lo) {
    Mfma<BF16>::split(pe, hi, lo);
  }
};

template <>
struct Mfma4<F16> {
  template <int ABID>
  __device__ static inline f32x4_t mma(uint2 a, uint2 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(f16x4_t, a),
                                              __builtin_bit_cast(f16x4_t, b), c, 4, ABID, 0);
  }
  __device__ static inline void split(const float pe[4], uint2& hi, uint2& lo) {
    Mfma<F16>::split(pe, hi, lo);
  }
};

// Pool formats of the 4x4x4 engine.  Mma: the matrix op (both operands in
// its 16-bit type); kCodes: the pool holds 8-bit codes, widened exactly to
// bf16 before each MFMA (widen: 4 codes of a 32-bit word -> 4 bf16 as the
// uint2 operand, element order kept).
template <typename KV>
struct Kv4 {
  using Mma = Mfma4<KV>;
  static constexpr bool kCodes = false;
};
// bf16 pair from two floats whose values are bf16 values: their high halves.
__device__ __forceinline__ uint32_t bf16_pair(float a, float b) {
  return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}
template <>
struct Kv4<E4M3> {
  using Mma = Mfma4<BF16>;
  static constexpr bool kCodes = true;
  // every E4M3 value (3 mantissa bits, exponents 2^-9 .. 2^8) is a bf16 value:
  // gfx950 converts two codes to a bf16 pair in one instruction (scale 1:
  // exact).  Measured against two codes to fp32 then a byte permute: 34.1
  // against 34.5 us for the Llama-3-8B batch's attention kernel.
  __device__ static inline uint2 widen(uint32_t w) {
    return make_uint2(
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)));
  }
};
template <>
struct Kv4<I8> {
  using Mma = Mfma4<BF16>;
  static constexpr bool kCodes = true;
  // integers in [-128, 127] have at most 8 significant bits: bf16 values
  __device__ static inline uint2 widen(uint32_t w) {
    const int v = static_cast<int>(w);
    const float f0 = static_cast<float>((v << 24) >> 24), f1 = static_cast<float>((v << 16) >> 24);
    const float f2 = static_cast<float>((v << 8) >> 24), f3 = static_cast<float>(v >> 24);
    return make_uint2(bf16_pair(f0, f1), bf16_pair(f2, f3));
  }
};

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
constexpr int kDppQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;

// 4x4 transpose across each lane quad: afterwards lane 4a+i holds in m[e]
// what lane 4a+e held in m[i].  Two 2x2 exchanges (lane bit 1 with element
// bit 1, then lane bit 0 with element bit 0).
__device__ __forceinline__ void quad_transpose(float (&m)[4]) {
  const int lane = threadIdx.x & 63;
  const bool b1 = lane & 2, b0 = lane & 1;
  float s0 = b1 ? m[0] : m[2], s1 = b1 ? m[1] : m[3];
  float r0 = dpp<kDppQuadXor2>(s0), r1 = dpp<kDppQuadXor2>(s1);
  if (b1) {
    m[0] = r0;
    m[1] = r1;
  } else {
    m[2] = r0;
    m[3] = r1;
  }
  s0 = b0 ? m[0] : m[1];
  s1 = b0 ? m[2] : m[3];
  r0 = dpp<kDppQuadXor1>(s0);
  r1 = dpp<kDppQuadXor1>(s1);
  if (b0) {
    m[0] = r0;
    m[2] = r1;
  } else {
    m[1] = r0;
    m[3] = r1;
  }
}

// Max / sum over the 16 lanes that share lane % 4.
__device__ __forceinline__ float max16(float v) {
  v = fmaxf(v, dpp<kDppRowRor4>(v));
  v = fmaxf(v, dpp<kDppRowRor8>(v));
  v = fmaxf(v, __shfl_xor(v, 16));
  return fmaxf(v, __shfl_xor(v, 32));
}
__device__ __forceinline__ float sum16(float v) {
  v += dpp<kDppRowRor4>(v);
  v += dpp<kDppRowRor8>(v);
  v += __shfl_xor(v, 16);
  return v + __shfl_xor(v, 32);
}

// NG groups of 4 query heads share each K/V load (G <= 4 * NG); group n
// holds heads 4n .. 4n+3 of the KV head's G.
template <int D, int NG = 1>
struct WaveState4 {
  float m_run[NG];           // running max (log2 domain) of head 4n + lane%4
  float l_lane[NG];          // this lane's share of that head's running sum
  f32x4_t acc[NG][D / 64];   // O: lane l = dim 64t + l, element e = head 4n + e
  bool bad;                  // a table entry of the range was out of the pool
};

// Loads a range's first dependencies before its length is known: Q (A
// operand of QK: lane 4a+i holds head i, dims 64r + 4a .. +3) and the raw
// table entries blk_begin + lane of sequence b (in bounds of the table row;
// attend4 validates the ones it uses).
template <int D, int NG = 1>
struct Prologue4 {
  uint2 qr[NG][D / 64];
  int tab;
};

template <int D, int NG>
__device__ __forceinline__ void prologue4(const Params& pr, int b, int g, int blk_begin,
                                          Prologue4<D, NG>& pre) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int n = 0; n < NG; ++n) {
    const int i = 4 * n + (lane & 3);   // head of the KV head's group
    const uint16_t* qb = static_cast<const uint16_t*>(pr.q) +
                         (static_cast<int64_t>(b) * pr.Hq + g * pr.G + i) * D + 4 * (lane >> 2);
#pragma unroll
    for (int r = 0; r < D / 64; ++r)
      pre.qr[n][r] = i < pr.G ? *reinterpret_cast<const uint2*>(qb + 64 * r) : make_uint2(0, 0);
  }
  const int k = blk_begin + lane;
  pre.tab = k < pr.max_blocks ? pr.tables[static_cast<int64_t>(b) * pr.max_blocks + k] : 0;
}

// with_new (uniform): the range ends at the sequence's last position, which
// holds the step's new token (fused append).  A run-time flag rather than a
// template parameter, so the kernel carries one copy of the loop.
// Positions before tok_begin (a sliding window's start inside the range's
// first block) are masked like positions past tok_end.
// after_start(): called once the range's first loads are out and its start
// checks are done; the caller issues the next range's prologue there, so
// that no wait at this range's start stands behind those loads (loads
// return in order).
struct NoStartHook {
  __device__ void operator()() const {}
};
template <typename T, int D, int NG, typename StartHook = NoStartHook>
__device__ __forceinline__ void attend4(const Params& pr, int b, int g, int blk_begin, int nblk,
                                        int tok_begin, int tok_end, WaveState4<D, NG>& st,
                                        const Prologue4<D, NG>& pre, bool with_new,
                                        StartHook after_start = StartHook{}) {
  using Fmt = Kv4<T>;
  using Mma = typename Fmt::Mma;
  constexpr bool kCodes = Fmt::kCodes;
  constexpr int NC = D * T::kBytes / 16;   // 16-byte K chunks per token
  constexpr int NT = D / 64;               // 64-dim output tiles
  constexpr int NH = 16 / T::kVecElems;    // V chunks per (block, dim): 2 (16-bit), 1 (codes)
  constexpr int64_t kTileBytes = static_cast<int64_t>(D) * kBlockSize * T::kBytes;
  const int lane = threadIdx.x & 63;
  const int nquad = (nblk + 3) >> 2;

  const char* kbase = static_cast<const char*>(pr.kpool) + g * kTileBytes;
  const char* vbase = static_cast<const char*>(pr.vpool) + g * kTileBytes;
  const int64_t block_stride = static_cast<int64_t>(pr.Hkv) * kTileBytes;
  const int32_t* trow = pr.tables + static_cast<int64_t>(b) * pr.max_blocks + blk_begin;

  // Table entries, 64 per register (lane i holds entry 64*c + i of chunk c).
  auto load_chunk = [&](int c) -> int {
    const int k = c * 64 + lane;
    return k < nblk ? trow[k] : 0;
  };
  // A chunk is loaded one chunk ahead and checked when it becomes the
  // current one: checking it at once would make the wave wait for it, and
  // (loads return in order) for every load issued before it.
  auto check_chunk = [&](int c, int e) -> int {
    const bool lane_bad = c * 64 + lane < nblk && (e < 0 || e >= pr.num_blocks);
    if (__any(lane_bad)) st.bad = true;
    return lane_bad ? 0 : e;
  };
  int chunk = 0;
  int tcur = check_chunk(0, pre.tab);
  int tnext = 0;   // loaded once the first quad's loads are out
  // Physical blocks of quad qd (qd increases across calls; the 4 entries of a
  // quad never straddle a 64-entry chunk); blocks past the range map to its
  // last block.
  auto quad_phys = [&](int qd, int (&ph)[4]) {
    const int c = qd >> 4;
    if (c != chunk) {
      chunk = c;
      tcur = check_chunk(c, tnext);
      tnext = (c + 1) * 64 < nblk ? load_chunk(c + 1) : 0;
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      ph[kb] = __builtin_amdgcn_readlane(tcur, min(4 * qd + kb, nblk - 1) & 63);
  };

  uint4 kr[NC];
  uint4 vr[4][NH][NT];
  int ph[4];
  auto issue_k = [&]() {
    const int kb = lane >> 4;
    const int p = kb == 0 ? ph[0] : kb == 1 ? ph[1] : kb == 2 ? ph[2] : ph[3];
    const char* kt = kbase + p * block_stride + (lane & 15) * 16;
#pragma unroll
    for (int c = 0; c < NC; ++c) kr[c] = load_stream(kt + c * 256);
  };
  auto issue_v_block = [&](int kb) {
    const char* vt = vbase + ph[kb] * block_stride + lane * 16;
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int t = 0; t < NT; ++t)
        vr[kb][h][t] = load_stream(vt + (h * D + 64 * t) * 16);
  };
  auto issue_v = [&]() {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const char* vt = vbase + ph[kb] * block_stride + lane * 16;
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int t = 0; t < NT; ++t)
          vr[kb][h][t] = load_stream(vt + (h * D + 64 * t) * 16);
    }
  };

  // New token of the step (fused append): its rows are loaded once the
  // first quad's loads are out, staged in LDS before the last quad, put into
  // the last quad's registers and written to its pool slot.  8-bit pools
  // stage its codes (encoded from the bf16 rows as the quantizing append
  // encodes them), D/4 words of 4 codes per pool.  The slot is read with a
  // scalar load, which no vector load waits for.
  constexpr int kStageWords = D * T::kBytes / 4;
  // one staging area per wave of the workgroup (the even split runs 4 waves
  // per workgroup)
  __shared__ uint32_t s_new_waves[4][2][D / 2];
  auto& s_new = s_new_waves[(threadIdx.x >> 6) & 3];
  // 16-bit pools: one word (2 values) per lane; 8-bit pools: 4 bf16 values
  using StageT = std::conditional_t<kCodes, uint2, uint32_t>;
  StageT stage_k{}, stage_v{};
  int64_t new_slot = -1;
  auto load_new = [&]() {
    if (with_new)
      new_slot = ((const __attribute__((address_space(4))) int64_t*)
                      pr.slots)[__builtin_amdgcn_readfirstlane(b)];
    if (with_new && lane < kStageWords) {
      const int64_t nrow = (static_cast<int64_t>(b) * pr.Hkv + g) * D;
      stage_k = reinterpret_cast<const StageT*>(static_cast<const uint16_t*>(pr.k_new) + nrow)[lane];
      stage_v = reinterpret_cast<const StageT*>(static_cast<const uint16_t*>(pr.v_new) + nrow)[lane];
    }
  };
  auto stage_new = [&]() {
    if (lane < kStageWords) {
      if constexpr (kCodes) {
        s_new[0][lane] = encode4_bf16<T>(stage_k, pr.enc_k);
        s_new[1][lane] = encode4_bf16<T>(stage_v, pr.enc_v);
      } else {
        s_new[0][lane] = stage_k;
        s_new[1][lane] = stage_v;
      }
    }
    __builtin_amdgcn_wave_barrier();
  };
  // Puts the new token into the last quad's registers (its pool slot may
  // still hold an older value for this wave's loads).
  // The new token sits at position tok_end - 1, in the last quad: lane qt
  // of the quad (block qt / 16), V half h = (qt / 8) % 2, element qt % 8.
  // It enters the attention only when its slot is the table's slot of that
  // position (the caller's contract), so that pa_decode_step has the effect
  // of pa_cache_append then the attention over the pool for every slot.
  const int qt = tok_end - 1 - (blk_begin + 4 * (nquad - 1)) * kBlockSize;  // 0..63
  // (the token is in the range's last block, nblk - 1, whose table entry is
  // in the current chunk once the last quad is issued)
  auto new_phys = [&]() { return __builtin_amdgcn_readlane(tcur, (nblk - 1) & 63); };
  auto new_at_table = [&]() {
    const int phys = new_phys();
    return new_slot >= 0 && new_slot < static_cast<int64_t>(pr.num_blocks) * kBlockSize &&
           new_slot == static_cast<int64_t>(phys) * kBlockSize + (qt & 15);
  };
  // K before the last quad's QK, V before its P.V (so QK does not wait for V).
  auto substitute_k = [&]() {
    if (lane == qt) {
#pragma unroll
      for (int c = 0; c < NC; ++c) kr[c] = reinterpret_cast<const uint4*>(s_new[0])[c];
    }
  };
  auto substitute_v = [&]() {
    if constexpr (kCodes) {
      // byte qt % 16 of the block's chunk of each dim 64t + lane.  Masks
      // applied to every block's registers (not a branch per block, which
      // the compiler turns into an indexed access through scratch memory).
      const uint8_t* vn = reinterpret_cast<const uint8_t*>(s_new[1]);
      const int kb = qt >> 4, e = qt & 15;
      const uint32_t byte = 0xFFu << ((e & 3) * 8);
      const int dw = e >> 2;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint32_t val = static_cast<uint32_t>(vn[64 * t + lane]) * 0x01010101u;
#pragma unroll
        for (int KB = 0; KB < 4; ++KB) {
          const uint32_t m = KB == kb ? byte : 0u;
          const uint32_t mx = dw == 0 ? m : 0u, my = dw == 1 ? m : 0u;
          const uint32_t mz = dw == 2 ? m : 0u, mw = dw == 3 ? m : 0u;
          uint4& vv = vr[KB][0][t];
          vv.x = (vv.x & ~mx) | (val & mx);
          vv.y = (vv.y & ~my) | (val & my);
          vv.z = (vv.z & ~mz) | (val & mz);
          vv.w = (vv.w & ~mw) | (val & mw);
        }
      }
      return;
    }
    const uint16_t* vn = reinterpret_cast<const uint16_t*>(s_new[1]);
    const int kb = qt >> 4, h = (qt >> 3) & 1, e = qt & 7;
    const uint32_t keep = (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
    const int sh = (e & 1) * 16, dw = e >> 1;
#pragma unroll
    for (int KB = 0; KB < 4; ++KB)
#pragma unroll
      for (int H = 0; H < NH; ++H)
        if (KB == kb && H == h) {
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const uint32_t val = static_cast<uint32_t>(vn[64 * t + lane]) << sh;
            uint4& vv = vr[KB][H][t];
            vv.x = dw == 0 ? ((vv.x & keep) | val) : vv.x;
            vv.y = dw == 1 ? ((vv.y & keep) | val) : vv.y;
            vv.z = dw == 2 ? ((vv.z & keep) | val) : vv.z;
            vv.w = dw == 3 ? ((vv.w & keep) | val) : vv.w;
          }
        }
  };
  // Pool write of the new token, unless the merge kernel does it:
  //   * at the table's slot: the wave holds the token's whole half block (8
  //     tokens, all dims: as loaded, with the token put in); writing that
  //     back as whole 128-byte lines stores the token and rewrites the other
  //     tokens' current bytes unchanged (2-byte V stores would leave 16
  //     partly written lines per head);
  //   * any other slot in the pool: the token alone, element by element;
  //   * slot out of the pool (-1): nothing.
  auto write_new = [&](bool at_table) {
    if constexpr (kCodes) return;   // 8-bit pools: the merge kernel writes the codes
    const int64_t slot = new_slot;
    if (pr.write_new_in_merge || slot < 0 ||
        slot >= static_cast<int64_t>(pr.num_blocks) * kBlockSize)
      return;
    const int kb = qt >> 4, h = NH == 2 ? (qt >> 3) & 1 : 0;
    const int phys = new_phys();
    if (at_table) {
      const int64_t tile = (static_cast<int64_t>(phys) * pr.Hkv + g) * kTileBytes;
      char* kt = static_cast<char*>(pr.kpool_w) + tile + (lane & 15) * 16;
      if ((lane >> 3) == (qt >> 3)) {
#pragma unroll
        for (int c = 0; c < NC; ++c) *reinterpret_cast<uint4*>(kt + c * 256) = kr[c];
      }
      char* vt = static_cast<char*>(pr.vpool_w) + tile + lane * 16;
#pragma unroll
      for (int KB = 0; KB < 4; ++KB)
#pragma unroll
        for (int H = 0; H < NH; ++H)
          if (KB == kb && H == h) {
#pragma unroll
            for (int t = 0; t < NT; ++t)
              *reinterpret_cast<uint4*>(vt + (H * D + 64 * t) * 16) = vr[KB][H][t];
          }
    } else {
      const uint16_t* kn = reinterpret_cast<const uint16_t*>(s_new[0]);
      const uint16_t* vn = reinterpret_cast<const uint16_t*>(s_new[1]);
      const int64_t blk = slot / kBlockSize;
      const int ts = static_cast<int>(slot % kBlockSize);
      uint16_t* kt = static_cast<uint16_t*>(pr.kpool_w) + tile_base(blk, g, pr.Hkv, D);
      uint16_t* vt = static_cast<uint16_t*>(pr.vpool_w) + tile_base(blk, g, pr.Hkv, D);
      if (lane < NC)
        *reinterpret_cast<uint4*>(kt + (lane * kBlockSize + ts) * 8) =
            *reinterpret_cast<const uint4*>(kn + lane * 8);
#pragma unroll
      for (int d = lane; d < D; d += 64) vt[((ts >> 3) * D + d) * 8 + (ts & 7)] = vn[d];
    }
  };

  auto qk_softmax = [&](int qd, uint2 (&phi)[NG], uint2 (&plo)[NG]) {
    f32x4_t s0[NG], s1[NG];
#pragma unroll
    for (int n = 0; n < NG; ++n) s0[n] = s1[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    unroll<D / 4>([&](auto ic) {
      constexpr int s = decltype(ic)::value;   // dims 4s .. 4s+3
      uint2 kv;
      if constexpr (kCodes) {
        const uint4& kc = kr[s / 4];
        kv = Fmt::widen((s & 3) == 0 ? kc.x : (s & 3) == 1 ? kc.y : (s & 3) == 2 ? kc.z : kc.w);
      } else {
        const uint4& kc = kr[s / 2];
        kv = (s & 1) ? make_uint2(kc.z, kc.w) : make_uint2(kc.x, kc.y);
      }
#pragma unroll
      for (int n = 0; n < NG; ++n) {
        if constexpr (s & 1)
          s1[n] = Mma::template mma<s % 16>(pre.qr[n][s / 16], kv, s1[n]);
        else
          s0[n] = Mma::template mma<s % 16>(pre.qr[n][s / 16], kv, s0[n]);
      }
    });
    const int qpos = (blk_begin + 4 * qd) * kBlockSize;   // position of the quad's token 0
    const bool valid = qpos + lane < tok_end && qpos + lane >= tok_begin;
#pragma unroll
    for (int n = 0; n < NG; ++n) {
      float sv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        sv[e] = valid ? (s0[n][e] + s1[n][e]) * pr.scale_log2 : -INFINITY;
      quad_transpose(sv);   // lane 4a+i: head 4n+i, tokens 4a+e
      const float lm = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
      if (__any(lm > st.m_run[n])) {
        // the running max moved for some head: rescale by 2^(m_old - m_new)
        const float mn = fmaxf(st.m_run[n], max16(lm));
        const float alpha = __builtin_amdgcn_exp2f(st.m_run[n] - mn);
        st.l_lane[n] *= alpha;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float ah = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), e));
#pragma unroll
          for (int t = 0; t < NT; ++t) st.acc[n][t][e] *= ah;
        }
        st.m_run[n] = mn;
      }
      float pe[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) pe[e] = __builtin_amdgcn_exp2f(sv[e] - st.m_run[n]);
      st.l_lane[n] += (pe[0] + pe[1]) + (pe[2] + pe[3]);
      Mma::split(pe, phi[n], plo[n]);
    }
  };

  // last: the quad may reach past the end of the range (only the range's last
  // quad can)
  // refill: V of the next quad (blocks in ph) is loaded block by block as
  // soon as P.V has consumed the block's registers.
  auto pv = [&](int qd, const uint2 (&phi)[NG], const uint2 (&plo)[NG], auto last,
                auto refill) {
    const int qpos = (blk_begin + 4 * qd) * kBlockSize;
    if (decltype(last)::value && qpos + 4 * kBlockSize > tok_end && kCodes) {
      // as below, for 16 one-byte tokens per chunk: byte e of word w is
      // token 4w + e of the block
      auto keep = [](int n) -> uint32_t {   // bytes 0 .. n-1 of a word
        return n >= 4 ? 0xFFFFFFFFu : n <= 0 ? 0u : (1u << (8 * n)) - 1u;
      };
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int nv = tok_end - (qpos + 16 * kb);   // valid tokens of the block
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          vr[kb][0][t].x &= keep(nv);
          vr[kb][0][t].y &= keep(nv - 4);
          vr[kb][0][t].z &= keep(nv - 8);
          vr[kb][0][t].w &= keep(nv - 12);
        }
      }
    } else if (decltype(last)::value && qpos + 4 * kBlockSize > tok_end) {
      // the quad reaches past the end of the range: zero V of masked
      // positions so unused slots (even NaN) cannot reach the output via 0*v
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int nv = tok_end - (qpos + 16 * kb + 8 * h);   // valid tokens of the 8
          const uint32_t m0 = (nv > 0 ? 0x0000FFFFu : 0u) | (nv > 1 ? 0xFFFF0000u : 0u);
          const uint32_t m1 = (nv > 2 ? 0x0000FFFFu : 0u) | (nv > 3 ? 0xFFFF0000u : 0u);
          const uint32_t m2 = (nv > 4 ? 0x0000FFFFu : 0u) | (nv > 5 ? 0xFFFF0000u : 0u);
          const uint32_t m3 = (nv > 6 ? 0x0000FFFFu : 0u) | (nv > 7 ? 0xFFFF0000u : 0u);
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            if constexpr (kCodes) continue;
            vr[kb][h][t].x &= m0;
            vr[kb][h][t].y &= m1;
            vr[kb][h][t].z &= m2;
            vr[kb][h][t].w &= m3;
          }
        }
    }
    unroll<16>([&](auto ic) {
      constexpr int a = decltype(ic)::value;   // tokens 4a..4a+3
      constexpr int kb = a >> 2;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        uint2 vv;
        if constexpr (kCodes) {
          const uint4& v = vr[kb][0][t];
          vv = Fmt::widen((a & 3) == 0 ? v.x : (a & 3) == 1 ? v.y : (a & 3) == 2 ? v.z : v.w);
        } else {
          const uint4& v = vr[kb][(a >> 1) & 1][t];
          vv = (a & 1) ? make_uint2(v.z, v.w) : make_uint2(v.x, v.y);
        }
#pragma unroll
        for (int n = 0; n < NG; ++n) {
          st.acc[n][t] = Mma::template mma<a>(phi[n], vv, st.acc[n][t]);
          st.acc[n][t] = Mma::template mma<a>(plo[n], vv, st.acc[n][t]);
        }
      }
      if constexpr (decltype(refill)::value && (a & 3) == 3) {
        __builtin_amdgcn_sched_barrier(0);
        issue_v_block(kb);
        __builtin_amdgcn_sched_barrier(0);
      }
    });
  };

  quad_phys(0, ph);
  issue_k();
  issue_v();
  __builtin_amdgcn_sched_barrier(0);
  load_new();
  if (nblk > 64) tnext = load_chunk(1);
  after_start();
  __builtin_amdgcn_sched_barrier(0);
  // steady state: K of the next quad is issued once QK has consumed the
  // current one, V of the next quad once P.V has.  The scheduling barriers
  // keep the compiler from hoisting the loads above the matrix ops that still
  // read their destination registers (which would cost register copies).
  for (int qd = 0; qd + 1 < nquad; ++qd) {
    uint2 phi[NG], plo[NG];
    qk_softmax(qd, phi, plo);
    __builtin_amdgcn_sched_barrier(0);
    quad_phys(qd + 1, ph);
    issue_k();
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NG >= 2 || !kCodes) {
      // loading the next quad's V block by block as P.V frees each block
      // shortens the wait for it (measured: 16-bit pools, and 8-bit pools
      // with several head groups; 8-bit pools with one group lost time)
      pv(qd, phi, plo, std::false_type{}, std::true_type{});
    } else {
      pv(qd, phi, plo, std::false_type{}, std::false_type{});
      __builtin_amdgcn_sched_barrier(0);
      issue_v();
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if (with_new) stage_new();
  const bool at_table = with_new && new_at_table();
  if (at_table) substitute_k();
  uint2 phi[NG], plo[NG];
  qk_softmax(nquad - 1, phi, plo);
  if (with_new) {
    if (at_table) substitute_v();
    write_new(at_table);
  }
  pv(nquad - 1, phi, plo, std::true_type{}, std::false_type{});
}

template <int D, int NG>
__device__ __forceinline__ void reset_state4(WaveState4<D, NG>& st) {
#pragma unroll
  for (int n = 0; n < NG; ++n) {
    st.m_run[n] = -INFINITY;
    st.l_lane[n] = 0.f;
  }
  st.bad = false;
#pragma unroll
  for (int n = 0; n < NG; ++n)
#pragma unroll
    for (int t = 0; t < D / 64; ++t) st.acc[n][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
}

template <int D, int NG>
__device__ __forceinline__ void emit_state4(const Params& pr, int b, int g, int slot,
                                            WaveState4<D, NG>& st) {
  constexpr int NT = D / 64;
  const int lane = threadIdx.x & 63;
  const int G = pr.G;
#pragma unroll
  for (int n = 0; n < NG; ++n) {
    float l = sum16(st.l_lane[n]);
    float m = st.m_run[n];
    if (st.bad) {
      m = 0.f;
      l = __builtin_nanf("");
#pragma unroll
      for (int t = 0; t < NT; ++t) st.acc[n][t] = f32x4_t{l, l, l, l};
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (4 * n + e < G) {
        const float mh = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), e));
        const float lh = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(l), e));
        const int64_t row = static_cast<int64_t>(b) * pr.Hq + g * G + 4 * n + e;
        const float inv = pr.out_scale / lh;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int d = 64 * t + lane;
          if (slot < 0)
            pr.out[row * D + d] = st.acc[n][t][e] * inv;
          else
            pr.part_acc[(row * pr.maxP + slot) * D + d] = st.acc[n][t][e];
        }
        if (slot >= 0 && lane == 0) {
          pr.part_m[row * pr.maxP + slot] = mh;
          pr.part_l[row * pr.maxP + slot] = lh;
        }
      }
    }
  }
}

// NG head groups per K/V load: G <= 4 * NG.
template <typename T, int D, int NG = 1>
struct Engine4 {
  using State = WaveState4<D, NG>;
  using Pre = Prologue4<D, NG>;
  static constexpr int kUnitBlocks = 4;  // blocks per step (one quad)
  __device__ static void prologue(const Params& pr, int b, int g, int blk_begin, Pre& pre) {
    prologue4<D, NG>(pr, b, g, blk_begin, pre);
  }
  template <typename StartHook = NoStartHook>
  __device__ static void attend_rt(const Params& pr, int b, int g, int blk_begin, int nblk,
                                   int tok_begin, int tok_end, State& st, const Pre& pre,
                                   bool with_new, StartHook after_start = StartHook{}) {
    attend4<T, D, NG>(pr, b, g, blk_begin, nblk, tok_begin, tok_end, st, pre, with_new,
                      after_start);
  }
  // waits for the prologue's table entries here (an empty asm that reads
  // the register)
  __device__ static void settle(const Pre& pre) { asm volatile("" ::"v"(pre.tab)); }
  __device__ static void reset(State& st) { reset_state4(st); }
  __device__ static void emit(const Params& pr, int b, int g, int slot, State& st) {
    emit_state4(pr, b, g, slot, st);
  }
};

// Fixed partitions: one wave per (KV head, partition, sequence); grid
// x = head + Hkv * partition (the heads of a partition are dispatched
// together), z = sequence.  kFused: the partition holding the sequence's
// last position also appends the step's new token.
template <typename Eng, bool kFused, int kWaves>
__global__ __launch_bounds__(64, kWaves) void decode_fixed_kernel(Params pr) {
  const int g = blockIdx.x % pr.Hkv, p = blockIdx.x / pr.Hkv, b = blockIdx.z;
  // Q and the partition's table entries are fetched together with the
  // length, not after it (each dependent round trip costs a full memory
  // latency under load).
  typename Eng::Pre pre;
  Eng::prologue(pr, b, g, p * (pr.P / kBlockSize), pre);
  const int L = pr.lens[b];
  if (!len_valid(L, pr) || L == 0) {
    if (p == 0) write_trivial_rows(pr, b, g, L);
    return;
  }
  // partitions count from the one holding the first attended position (a
  // sliding window's start; 0 without a window)
  const int f = first_pos(L, pr), p0 = f / pr.P;
  const int np = (L + pr.P - 1) / pr.P - p0;
  if (p >= np) return;
  const int tok0 = max((p + p0) * pr.P, f), tok1 = min(L, (p + p0 + 1) * pr.P);
  const int blk0 = tok0 / kBlockSize;
  const int nblk = (tok1 - blk0 * kBlockSize + kBlockSize - 1) / kBlockSize;
  if (blk0 != p * (pr.P / kBlockSize)) Eng::prologue(pr, b, g, blk0, pre);   // window only
  typename Eng::State st;
  Eng::reset(st);
  Eng::attend_rt(pr, b, g, blk0, nblk, tok0, tok1, st, pre, kFused && p == np - 1);
  Eng::emit(pr, b, g, np == 1 ? -1 : p, st);
}

// ---------------------------------------------------------------------------
// Balanced split.  The work of a step is the list of units (sequence b, KV
// head g, run of U consecutive blocks, U = the engine's step), ordered by b,
// then g, then unit.  The cut balances cost, counted in ticks: a unit costs
// kUnitTicks, and each (b, g) range costs pr.range_ticks more at its start
// (a wave that moves to another range mid-chunk pays about that: the row it
// leaves, the new token at the range's end, the next range's first loads).
// Range (b, g) occupies ticks [S, S + range_ticks + kUnitTicks * units(b)),
// its unit k starting at tick S + range_ticks + kUnitTicks * k.  With W waves
// the ticks are cut into chunks of C (C >= kMinChunkBlocks blocks' worth of
// units plus one range start); wave w attends the units whose start tick lies
// in [w * C, (w + 1) * C), which may cover the end of one (b, g) range and
// the start of the next.  A (b, g) range cut into several chunks leaves one
// partial per chunk, merged by merge_kernel; a range inside one chunk is
// written final.  When every range has the same number of units (decode
// steps of beams or samples of equal length), the cut instead gives each
// range k chunks exactly (chunk and range boundaries then coincide: no wave
// changes range), by choosing the start charge and C for it.
// ---------------------------------------------------------------------------
constexpr int kMinChunkBlocks = 8;
constexpr int kUnitTicks = 8;
// Cost of a range start.  Per-wave clocks of the Llama-3-8B batch: a wave
// with one more range took 0.4 of a unit's time longer on 16-bit pools and
// about one unit's time on 8-bit pools.  The values are the best of a sweep
// of the kernel time (16-bit: Llama-3-8B, OPT-13B and copy-on-write batches;
// 8-bit: E4M3 and INT8 pools of the Llama-3-8B batch).
constexpr int kRangeTicks16 = 9;
constexpr int kRangeTicksCodes = 12;

// Units of U blocks of a sequence: from the block holding its first attended
// position to its last block.
template <int U>
__device__ __forceinline__ int units_of(int L, const Params& pr, int pre = 0) {
  return (len_valid(L, pr) && L > 0)
             ? ((L + kBlockSize - 1) / kBlockSize - first_pos(L, pr, pre) / kBlockSize + U - 1) /
                   U
             : 0;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

// Ticks of one (b, g) range of a sequence of length L (none without units),
// rt ticks charged at its start.
template <int U>
__device__ __forceinline__ int range_cost(int L, int rt, const Params& pr, int pre = 0) {
  const int nub = units_of<U>(L, pr, pre);
  return nub > 0 ? rt + kUnitTicks * nub : 0;
}

__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}

struct SplitPlan {
  int total;  // ticks
  int C;      // ticks per chunk
  int chunks; // chunks with work (chunk w holds a unit start iff w * C <= total - kUnitTicks)
  int rt;     // ticks charged at each range's start
};

// The batch's units: sequences with work, all their units, and the least and
// most units of one of their ranges.
struct UnitStats {
  int nseq = 0, units = 0, umin = 0x7fffffff, umax = 0;
  __device__ void add(int nub) {   // one lane's sequence (wave-uniform result)
    nseq += wave_sum(nub > 0 ? 1 : 0);
    units += wave_sum(nub);
    umin = min(umin, wave_min(nub > 0 ? nub : 0x7fffffff));
    umax = max(umax, wave_max(nub));
  }
};

template <int U>
__device__ __forceinline__ SplitPlan make_split(const UnitStats& us, const Params& pr, int W) {
  constexpr int kMinUnits = (kMinChunkBlocks + U - 1) / U;
  SplitPlan sp;
  const int nranges = us.nseq * pr.Hkv;
  if (nranges > 0 && us.umin == us.umax) {
    // every range has nub units: k chunks of u units per range, the first
    // u*k - nub of them charged at the range's start, so that a range is
    // exactly k chunks; taken when it keeps 7/8 of the waves busy
    const int nub = us.umax;
    for (int k = min(W / nranges, nub / kMinUnits); k >= 2; --k) {
      const int u = (nub + k - 1) / k;
      if (u * k - nub < u && 8 * nranges * k >= 7 * W &&
          static_cast<int64_t>(nranges) * kUnitTicks * u * k < (int64_t{1} << 30)) {
        sp.rt = kUnitTicks * (u * k - nub);
        sp.C = kUnitTicks * u;
        sp.total = nranges * kUnitTicks * u * k;
        sp.chunks = (sp.total - kUnitTicks) / sp.C + 1;   // nranges * k
        return sp;
      }
    }
  }
  sp.rt = pr.range_ticks;
  sp.total = (kUnitTicks * us.units + sp.rt * us.nseq) * pr.Hkv;
  sp.C = max(kUnitTicks * kMinUnits + sp.rt, (sp.total + W - 1) / W);
  sp.chunks = sp.total > 0 ? (sp.total - kUnitTicks) / sp.C + 1 : 0;
  return sp;
}

template <int U>
__device__ __forceinline__ SplitPlan split_plan(const Params& pr, int W) {
  const int lane = threadIdx.x & 63;
  UnitStats us;
  for (int c = 0; c < pr.B; c += 64) {
    const int b = c + lane;
    us.add(b < pr.B ? units_of<U>(pr.lens[b], pr, prefix_of(pr, b)) : 0);
  }
  return make_split<U>(us, pr, W);
}

// The sequence whose ticks contain tick t, and the first tick of that
// sequence (t < total).
template <int U>
__device__ __forceinline__ void locate(const Params& pr, int rt, int t, int& b_out,
                                       int& base_out) {
  const int lane = threadIdx.x & 63;
  int carried = 0;
  for (int c = 0; c < pr.B; c += 64) {
    const int b = c + lane;
    const int cost =
        (b < pr.B ? range_cost<U>(pr.lens[b], rt, pr, prefix_of(pr, b)) : 0) * pr.Hkv;
    const int incl = carried + wave_incl_scan(cost);
    const uint64_t hit = __ballot(b < pr.B && incl > t);
    if (hit) {
      const int k = __builtin_ctzll(hit);
      b_out = c + k;
      base_out = __builtin_amdgcn_readlane(incl, k) - __builtin_amdgcn_readlane(cost, k);
      return;
    }
    carried = __builtin_amdgcn_readlane(incl, 63);
  }
  b_out = pr.B;
  base_out = carried;
}

// Context length of sequence b: from the register copy (lane b) when the
// batch fits one wave, else from memory.
__device__ __forceinline__ int len_of(const Params& pr, int lens_reg, int b) {
  return pr.B <= 64 ? __builtin_amdgcn_readlane(lens_reg, b) : pr.lens[b];
}

// Workgroups of kSplitWavesPerGroup waves (one per SIMD of a compute unit:
// 4x as few workgroups to dispatch as one-wave workgroups, measured 1.5 us
// faster on the Llama-3-8B step); wave w of W takes chunk w.
template <typename Eng, int kWaves>
__global__ __launch_bounds__(256, kWaves) void decode_split_kernel(Params pr) {
  constexpr int U = Eng::kUnitBlocks;
  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int W = gridDim.x * (blockDim.x >> 6);
  SplitPlan sp;
  int b, base;
  int lens_reg = 0, pre_reg = 0;
  if (pr.B <= 64) {
    // one pass: the batch's lengths (and shared prefixes) stay in registers
    // for the whole kernel
    lens_reg = lane < pr.B ? pr.lens[lane] : 0;
    pre_reg = (lane < pr.B && pr.prefix) ? pr.prefix[lane] : 0;
    const int nub = lane < pr.B ? units_of<U>(lens_reg, pr, pre_reg) : 0;
    UnitStats us;
    us.add(nub);
    sp = make_split<U>(us, pr, W);
    const int cost = (nub > 0 ? sp.rt + kUnitTicks * nub : 0) * pr.Hkv;
    if (w >= sp.chunks) return;
    const int incl = wave_incl_scan(cost);
    const uint64_t hit = __ballot(lane < pr.B && incl > w * sp.C);
    const int k = __builtin_ctzll(hit);   // hit != 0: w * C < total
    b = k;
    base = __builtin_amdgcn_readlane(incl, k) - __builtin_amdgcn_readlane(cost, k);
  } else {
    sp = split_plan<U>(pr, W);
    if (w >= sp.chunks) return;
    locate<U>(pr, sp.rt, w * sp.C, b, base);
  }
  const int t_begin = w * sp.C, t_end = min(sp.total, t_begin + sp.C);
  // A segment is the part of the chunk inside one (b, g) range: its units
  // k0 .. k1 - 1.
  struct Seg {
    int b, g, base, L, pre, nub, rc, rstart, k0, k1, blk_begin, nblk, tok_begin, tok_end;
  };
  auto pre_of = [&](int b) {
    return pr.B <= 64 ? __builtin_amdgcn_readlane(pre_reg, b) : prefix_of(pr, b);
  };
  // units of a range from its tick offset: those starting before tick x
  auto units_before = [](int x) { return x > 0 ? (x + kUnitTicks - 1) / kUnitTicks : 0; };
  auto make_seg = [&](int b, int base, int g) {
    Seg sg;
    sg.b = b;
    sg.base = base;
    sg.L = len_of(pr, lens_reg, b);
    sg.pre = pre_of(b);
    sg.nub = units_of<U>(sg.L, pr, sg.pre);
    sg.rc = sp.rt + kUnitTicks * sg.nub;
    sg.g = g;
    sg.rstart = base + g * sg.rc;
    const int u0 = sg.rstart + sp.rt;                          // start tick of unit 0
    sg.k0 = min(sg.nub, units_before(t_begin - u0));
    sg.k1 = min(sg.nub, units_before(t_end - u0));
    const int nblk_seq = (sg.L + kBlockSize - 1) / kBlockSize;
    sg.tok_begin = first_pos(sg.L, pr, sg.pre);
    const int fb = sg.tok_begin / kBlockSize;                  // the range's first block
    sg.blk_begin = fb + U * sg.k0;
    sg.nblk = min(fb + U * sg.k1, nblk_seq) - sg.blk_begin;
    sg.tok_end = min(sg.L, (sg.blk_begin + sg.nblk) * kBlockSize);
    return sg;
  };
  // The range after cur's, from its first unit (it starts at tick
  // cur.rstart + cur.rc: sequences without units own no ticks).
  auto next_seg = [&](const Seg& cur) {
    if (cur.g + 1 < pr.Hkv) return make_seg(cur.b, cur.base, cur.g + 1);
    int b2 = cur.b;
    do {
      ++b2;
    } while (b2 < pr.B && units_of<U>(len_of(pr, lens_reg, b2), pr, pre_of(b2)) == 0);
    return make_seg(b2, cur.base + pr.Hkv * cur.rc, 0);
  };
  Seg cur = make_seg(b, base, (t_begin - base) / range_cost<U>(len_of(pr, lens_reg, b), sp.rt,
                                                               pr, pre_of(b)));
  // t_begin may lie past the last unit start of its range (in the range's
  // tail or the next one's start ticks): then the chunk starts with the next
  // range's unit 0 (every chunk holds a unit start: C exceeds the largest gap
  // between two, kUnitTicks + range_ticks)
  if (cur.k0 == cur.nub) cur = next_seg(cur);
  typename Eng::Pre pre;
  Eng::prologue(pr, cur.b, cur.g, cur.blk_begin, pre);
  // The table entries a segment checks first are made resident before the
  // loop and, for the next segment, at the end of each segment (when they
  // are long in): the wait then never falls at a segment's start, where it
  // would also wait for the previous segment's partial stores.
  Eng::settle(pre);
  typename Eng::State st;
  while (true) {
    // the next segment's Q and table entries are fetched while this one
    // streams, so the switch costs no dependent round trip; they go out
    // once this segment's first loads are out and its start checks done
    // (a start check issued after them would wait for them too)
    const bool more = cur.k1 == cur.nub && cur.rstart + cur.rc + sp.rt < t_end;
    Seg nxt = cur;
    typename Eng::Pre pre_next;
    if (more) nxt = next_seg(cur);
    Eng::reset(st);
    Eng::attend_rt(pr, cur.b, cur.g, cur.blk_begin, cur.nblk, cur.tok_begin, cur.tok_end, st,
                   pre, pr.k_new != nullptr && cur.tok_end == cur.L, [&]() {
                     if (more) Eng::prologue(pr, nxt.b, nxt.g, nxt.blk_begin, pre_next);
                   });
    if (more) Eng::settle(pre_next);
    const int u0 = cur.rstart + sp.rt;
    const int first_chunk = u0 / sp.C;
    const int nslots = (u0 + kUnitTicks * (cur.nub - 1)) / sp.C - first_chunk + 1;
    // a sequence with a shared prefix always leaves a partial: the merge
    // folds it with the prefix pass's row
    Eng::emit(pr, cur.b, cur.g, (nslots == 1 && cur.pre == 0) ? -1 : w - first_chunk, st);
    // the wave holding the range's first unit records how many slots the
    // merge has to combine
    if (cur.k0 == 0 && lane == 0)
      pr.counters[static_cast<int64_t>(cur.b) * pr.Hkv + cur.g] = nslots;
    if (!more) break;
    cur = nxt;
    pre = pre_next;
  }
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of a row's partials: one wave per (sequence b, query
// head h), four heads per workgroup, grid (ceil(Hq / 4), B); lane i owns
// output dims E*i .. E*i + E - 1 (E = D / 64).
//   out = sum_k 2^(m_k - M) acc_k / sum_k 2^(m_k - M) l_k,  M = max_k m_k
// The values every lane of the wave needs (the length, the slot count, the
// slots' maxima and sums, the prefix partials' pairs) are scalar loads.  The
// first kMergeSpec slots' weighted sums are loaded with them, before the slot
// count is known (slots are in bounds of the row's maxP workspace slots;
// values beyond the row's count are never used); the rest of a batch of
// kMergeBatch, only those the row holds, once the count is in.  Later slots
// are folded in batches with the running maximum rescaled.
//   kSplit: slot counts come from the balanced-split kernel's counters, and
//   the rows of empty (zeros) and out-of-bounds (NaN) sequences, which own
//   no work there, are written here; otherwise a sequence of length L has
//   ceil(L / P) partitions.
// ---------------------------------------------------------------------------
constexpr int kMergeBatch = 8;
constexpr int kMergeSpec = 2;
constexpr int kMergeRowsPerGroup = 4;
constexpr int kMergeFold = 16;   // weighted sums loaded together on the many-slot path

// A value read at the same address by every lane of the wave, through the
// scalar data cache (the address must be wave-uniform).
template <typename V>
__device__ __forceinline__ V uniform_load(const V* p) {
  return *(const __attribute__((address_space(4))) V*)p;
}

// E consecutive floats of a row (E = 1 or 2).
template <int E>
__device__ __forceinline__ void load_row(float (&v)[E], const float* p) {
  if constexpr (E == 2) {
    const float2 t = *reinterpret_cast<const float2*>(p);
    v[0] = t.x;
    v[1] = t.y;
  } else {
    v[0] = *p;
  }
}
template <int E>
__device__ __forceinline__ void store_row(float* p, const float (&v)[E]) {
  if constexpr (E == 2)
    *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
  else
    *p = v[0];
}

// C: void when the pools hold 16-bit values (new tokens moved as bits), else
// the 8-bit code format the new tokens are encoded into.
template <int D, bool kSplit, typename C = void>
__global__ __launch_bounds__(64 * kMergeRowsPerGroup) void merge_kernel(Params pr) {
  constexpr bool kCodes = !std::is_void_v<C>;
  constexpr int E = D / 64;
  const int lane = threadIdx.x & 63;
  const int h = blockIdx.x * kMergeRowsPerGroup + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = blockIdx.y;
  if (h >= pr.Hq) return;
  const int d0 = lane * E;
  const int64_t row = static_cast<int64_t>(b) * pr.Hq + h;
  const int g = h / pr.G;
  const int L = uniform_load(pr.lens + b);
  // maxP == 1: no workspace (every row is written final or trivial)
  const bool have_ws = pr.maxP > 1;
  const int ns_split =
      (kSplit && have_ws) ? uniform_load(pr.counters + static_cast<int64_t>(b) * pr.Hkv + g) : 0;
  const int kfirst = have_ws ? min(kMergeBatch, pr.maxP) : 0;
  const float* pm = pr.part_m + row * pr.maxP;
  const float* pl = pr.part_l + row * pr.maxP;
  const float* pa = pr.part_acc + row * pr.maxP * D + d0;
  float m[kMergeBatch], l[kMergeBatch], a[kMergeBatch][E];
#pragma unroll
  for (int k = 0; k < kMergeBatch; ++k) {
    if (k < kfirst) {
      m[k] = uniform_load(pm + k);
      l[k] = uniform_load(pl + k);
    }
  }
#pragma unroll
  for (int k = 0; k < kMergeSpec; ++k)
    if (k < kfirst) load_row<E>(a[k], pa + static_cast<int64_t>(k) * D);
  // shared prefix: the prefix pass's partials (loaded with the others; rows
  // without a prefix do not use them)
  const int pre = (kSplit && pr.prefix) ? uniform_load(pr.prefix + b) : 0;
  float2 pre_ml[kMaxPrefixPieces];
  float pre_o[kMaxPrefixPieces][E];
  bool stamped = true;
  if (kSplit && pr.prefix) {
    const int64_t plane = static_cast<int64_t>(pr.B) * pr.Hq;   // rows per piece
#pragma unroll
    for (int p = 0; p < kMaxPrefixPieces; ++p) {
      if (p < pr.pre_pieces) {
        const float* ml = reinterpret_cast<const float*>(pr.pre_ml + p * plane + row);
        pre_ml[p] = make_float2(uniform_load(ml), uniform_load(ml + 1));
        load_row<E>(pre_o[p], pr.pre_out + (p * plane + row) * D + d0);
        stamped = stamped && uniform_load(pr.pre_stamp + p * plane + row) == pr.epoch;
      }
    }
  }
  // Fused append of pa_decode_step: the wave of the first query head of each
  // (sequence, KV head) writes the new token into its slot; its loads go out
  // with the partials'.  16-bit pools: lanes below D/8 move one 16-byte K
  // chunk each, every lane its E V values.  8-bit pools: the bf16 rows are
  // encoded as the quantizing append encodes them (lanes below D/16 read 16 K
  // values for one 16-byte chunk of codes).
  const bool appends = pr.write_new_in_merge && h % pr.G == 0;
  int64_t slot = -1;
  uint4 kchunk = make_uint4(0, 0, 0, 0), kchunk2 = make_uint4(0, 0, 0, 0);
  uint16_t vval[E];
  if (appends) {
    slot = uniform_load(pr.slots + b);
    const int64_t nrow = (static_cast<int64_t>(b) * pr.Hkv + g) * D;
    const uint16_t* kn = static_cast<const uint16_t*>(pr.k_new) + nrow;
    if constexpr (kCodes) {
      if (lane < D / 16) {
        kchunk = *reinterpret_cast<const uint4*>(kn + lane * 16);
        kchunk2 = *reinterpret_cast<const uint4*>(kn + lane * 16 + 8);
      }
    } else if (lane < D / 8) {
      kchunk = *reinterpret_cast<const uint4*>(kn + lane * 8);
    }
    const uint16_t* vn = static_cast<const uint16_t*>(pr.v_new) + nrow + d0;
    if constexpr (E == 2) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(vn);
      vval[0] = static_cast<uint16_t>(w & 0xFFFFu);
      vval[1] = static_cast<uint16_t>(w >> 16);
    } else {
      vval[0] = vn[0];
    }
  }
  float* orow = pr.out + row * D + d0;
  if (!len_valid(L, pr) || L == 0) {
    // (an empty sequence given a shared prefix has no usable one: NaN)
    if (kSplit) {
      const float v = (L == 0 && pre == 0) ? 0.f : __builtin_nanf("");
      float r[E];
#pragma unroll
      for (int e = 0; e < E; ++e) r[e] = v;
      store_row<E>(orow, r);
    }
    return;
  }
  if (appends && slot >= 0 && slot < static_cast<int64_t>(pr.num_blocks) * kBlockSize) {
    const int64_t blk = slot / kBlockSize;
    const int ts = static_cast<int>(slot % kBlockSize);
    if constexpr (kCodes) {
      uint8_t* kt = static_cast<uint8_t*>(pr.kpool_w) + tile_base(blk, g, pr.Hkv, D);
      uint8_t* vt = static_cast<uint8_t*>(pr.vpool_w) + tile_base(blk, g, pr.Hkv, D);
      if (lane < D / 16)
        *reinterpret_cast<uint4*>(kt + (lane * kBlockSize + ts) * 16) =
            make_uint4(encode4_bf16<C>(make_uint2(kchunk.x, kchunk.y), pr.enc_k),
                       encode4_bf16<C>(make_uint2(kchunk.z, kchunk.w), pr.enc_k),
                       encode4_bf16<C>(make_uint2(kchunk2.x, kchunk2.y), pr.enc_k),
                       encode4_bf16<C>(make_uint2(kchunk2.z, kchunk2.w), pr.enc_k));
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float vf = __uint_as_float(static_cast<uint32_t>(vval[e]) << 16);
        vt[(d0 + e) * kBlockSize + ts] = static_cast<uint8_t>(Encode<C>::pair(vf, 0.f, pr.enc_v));
      }
    } else {
      uint16_t* kt = static_cast<uint16_t*>(pr.kpool_w) + tile_base(blk, g, pr.Hkv, D);
      uint16_t* vt = static_cast<uint16_t*>(pr.vpool_w) + tile_base(blk, g, pr.Hkv, D);
      if (lane < D / 8) *reinterpret_cast<uint4*>(kt + (lane * kBlockSize + ts) * 8) = kchunk;
#pragma unroll
      for (int e = 0; e < E; ++e) vt[((ts >> 3) * D + d0 + e) * 8 + (ts & 7)] = vval[e];
    }
  }
  const int ns = kSplit ? ns_split : (L + pr.P - 1) / pr.P - first_pos(L, pr) / pr.P;
  const bool has_pre = pre != 0;
  // an unusable prefix length, or a prefix the prefix pass did not attend
  // in this call (the sequence in no group, or its prefix not its group's)
  if (has_pre && lane == 0) {
    // the stamps are consumed: a later call (or a later replay of a captured
    // one, whose epoch is the same) that does not write this row sees 0
    const int64_t plane = static_cast<int64_t>(pr.B) * pr.Hq;
#pragma unroll
    for (int p = 0; p < kMaxPrefixPieces; ++p)
      if (p < pr.pre_pieces) pr.pre_stamp[p * plane + row] = 0;
  }
  if (has_pre && (!prefix_ok(pre, L) || !stamped)) {
    float r[E];
#pragma unroll
    for (int e = 0; e < E; ++e) r[e] = __builtin_nanf("");
    store_row<E>(orow, r);
    return;
  }
  if (!has_pre && (ns <= 1 || !have_ws)) return;             // written final
  float M = -INFINITY;
  if (has_pre) {
#pragma unroll
    for (int p = 0; p < kMaxPrefixPieces; ++p)
      if (p < pr.pre_pieces) M = fmaxf(M, pre_ml[p].x);
  }
  float num[E], den = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) num[e] = 0.f;
  if (ns <= kMergeBatch) {
    // the rest of the first batch: only the slots the row holds
#pragma unroll
    for (int k = kMergeSpec; k < kMergeBatch; ++k)
      if (k < kfirst && k < ns) load_row<E>(a[k], pa + static_cast<int64_t>(k) * D);
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k)
      if (k < ns) M = fmaxf(M, m[k]);
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {
      if (k < ns) {
        const float wgt = exp2f(m[k] - M);
        den = fmaf(wgt, l[k], den);
#pragma unroll
        for (int e = 0; e < E; ++e) num[e] = fmaf(wgt, a[k][e], num[e]);
      }
    }
  } else {
    // Many slots (long contexts in fixed partitions, or cut into many
    // chunks).  Slots go in groups of 256, four per lane: their maxima (and
    // sums) are loaded four at a time per lane, all in flight together; M is
    // the maximum over every group (a first sweep when there are more than
    // 256 slots); the weighted sums are then folded 16 slots at a time, their
    // loads issued together, with nothing to rescale.
    constexpr int kGroup = 256;
    auto group_ml = [&](int c0, float (&mv)[4], float (&lv)[4], bool sums) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int k = c0 + 64 * u + lane;
        mv[u] = k < ns ? pm[k] : -INFINITY;
        if (sums) lv[u] = k < ns ? pl[k] : 0.f;
      }
    };
    float mv[4], lv[4];
    if (ns > kGroup) {
      float mloc = -INFINITY;
      for (int c0 = 0; c0 < ns; c0 += kGroup) {
        group_ml(c0, mv, lv, false);
        mloc = fmaxf(mloc, fmaxf(fmaxf(mv[0], mv[1]), fmaxf(mv[2], mv[3])));
      }
      M = fmaxf(M, wave_max(mloc));
    }
    float dloc = 0.f;
    for (int c0 = 0; c0 < ns; c0 += kGroup) {
      group_ml(c0, mv, lv, true);
      if (ns <= kGroup) M = fmaxf(M, wave_max(fmaxf(fmaxf(mv[0], mv[1]), fmaxf(mv[2], mv[3]))));
      float w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        w[u] = exp2f(mv[u] - M);            // 0 for slots past the row's count
        dloc = fmaf(w[u], lv[u], dloc);
      }
      const int cnt = min(kGroup, ns - c0);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        for (int j0 = 0; j0 < 64 && 64 * u + j0 < cnt; j0 += kMergeFold) {
          const int base = c0 + 64 * u + j0;
          float av[kMergeFold][E];
          if (base + kMergeFold <= ns) {
#pragma unroll
            for (int f = 0; f < kMergeFold; ++f)
              load_row<E>(av[f], pa + static_cast<int64_t>(base + f) * D);
          } else {
#pragma unroll
            for (int f = 0; f < kMergeFold; ++f) {
              if (base + f < ns) {
                load_row<E>(av[f], pa + static_cast<int64_t>(base + f) * D);
              } else {
#pragma unroll
                for (int e = 0; e < E; ++e) av[f][e] = 0.f;
              }
            }
          }
#pragma unroll
          for (int f = 0; f < kMergeFold; ++f) {
            const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w[u]), j0 + f));
#pragma unroll
            for (int e = 0; e < E; ++e) num[e] = fmaf(wk, av[f][e], num[e]);
          }
        }
      }
    }
    den = wave_sum(dloc);
  }
  // each prefix piece counts as one more partial (an empty piece has max
  // -inf and sum 0: weight 0)
  if (has_pre) {
#pragma unroll
    for (int p = 0; p < kMaxPrefixPieces; ++p) {
      if (p < pr.pre_pieces) {
        const float wgt = exp2f(pre_ml[p].x - M);
        den = fmaf(wgt, pre_ml[p].y, den);
#pragma unroll
        for (int e = 0; e < E; ++e) num[e] = fmaf(wgt, pre_o[p][e], num[e]);
      }
    }
  }
  float r[E];
#pragma unroll
  for (int e = 0; e < E; ++e) r[e] = (num[e] / den) * pr.out_scale;
  store_row<E>(orow, r);
}

// Merge launch: one wave per (sequence, query head).
template <int D, bool kSplit, typename C = void>
void launch_merge(const Params& pr, hipStream_t s) {
  const dim3 grid((pr.Hq + kMergeRowsPerGroup - 1) / kMergeRowsPerGroup, pr.B);
  merge_kernel<D, kSplit, C><<<grid, 64 * kMergeRowsPerGroup, 0, s>>>(pr);
}

// Kernel family of the decode calls, set by pa_set_decode_kernel (process
// wide; PA_KERNEL_GENERIC makes fp16/bf16 take the plain-FMA kernel too, so
// both kernels can be checked).  Read once per call, never from the
// environment.
std::atomic<int> g_decode_kernel{PA_KERNEL_AUTO};
bool generic_selected() { return g_decode_kernel.load(std::memory_order_relaxed) == PA_KERNEL_GENERIC; }

constexpr int kDefaultPartition = 256;  // fixed-partition size of the plain-FMA kernel
constexpr int kFixedWaves4 = 3;         // waves per SIMD the 4x4x4 fixed kernel is built for
constexpr int kSplitWavesPerCU = 4;     // balanced split: grid = CUs * this (one wave per SIMD)
constexpr int kSplitWavesPerGroup = 4;  // waves per workgroup of the 4x4x4 split kernel

constexpr int kEvenSplit = -1;          // partition_size value selecting the even split

bool partition_ok(int P) { return P == kEvenSplit || (P >= 0 && P % kBlockSize == 0); }

bool decode_args_ok(int B, int Hq, int Hkv, int D, int max_ctx, int P, pa_dtype dt) {
  return B >= 0 && B <= 65535 && Hkv > 0 && Hkv <= 65535 && Hq > 0 && Hq % Hkv == 0 &&
         Hq / Hkv <= kMaxGroup && (D == 64 || D == 128) &&
         max_ctx >= 0 && partition_ok(P) && pool_dtype_ok(dt);
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Workspace: part_m, part_l, part_acc rows (maxP slots per (sequence, query
// head)), then one int per (sequence, KV head) (slots written, even split),
// each region 256-byte aligned.
size_t workspace_bytes(int B, int Hq, int Hkv, int D, int maxP) {
  if (maxP <= 1) return 0;
  const size_t rows = static_cast<size_t>(B) * Hq * maxP;
  return 2 * align256(rows * sizeof(float)) + align256(rows * D * sizeof(float)) +
         align256(static_cast<size_t>(B) * Hkv * sizeof(int));
}

// Waves of the balanced-split grid for the current device.
int split_waves() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  return cus * kSplitWavesPerCU;
}

// How a call is executed: the balanced split (matrix-core path, no partition
// size given) or fixed partitions of P tokens; maxP = workspace slots per
// (sequence, query head) row.
struct LaunchPlan {
  bool split;
  bool generic;
  bool unfit;   // the even split was asked for and cannot count this batch's work
  int P;
  int maxP;
  int W;
};

// The even split counts the batch's work in 32-bit ticks; it is used only
// while the largest count these sizes allow (every sequence at max_ctx)
// stays below 2^30 (chunk ends reach up to twice the count).
bool split_fits(int num_seqs, int num_kv_heads, int max_ctx) {
  const int64_t max_blk = (static_cast<int64_t>(max_ctx) + kBlockSize - 1) / kBlockSize;
  const int64_t range = std::max(kRangeTicks16, kRangeTicksCodes) + kUnitTicks * ((max_blk + 3) / 4);
  return static_cast<int64_t>(num_seqs) * num_kv_heads * range < (int64_t{1} << 30);
}

LaunchPlan make_plan(int num_seqs, int num_kv_heads, int max_ctx, int partition_size,
                     pa_dtype dt, bool generic_env) {
  LaunchPlan lp{};
  lp.generic = dt == PA_F32 || (generic_env && !code_dtype(dt));
  // default (0) on the matrix-core path: the even split, unless the batch is
  // too large for its count (then fixed partitions; asked for explicitly
  // (-1), the call is refused)
  lp.split = (partition_size == kEvenSplit || partition_size == 0) && !lp.generic;
  if (lp.split && !split_fits(num_seqs, num_kv_heads, max_ctx)) {
    lp.split = false;
    lp.unfit = partition_size == kEvenSplit;
  }
  if (lp.split) {
    lp.W = split_waves();
    // a range of nblk blocks is cut into at most ceil(nblk / kMinChunkBlocks) + 1
    // chunks (chunks hold at least kMinChunkBlocks blocks' worth of units)
    const int64_t max_blk = (static_cast<int64_t>(max_ctx) + kBlockSize - 1) / kBlockSize;
    lp.P = 0;
    lp.maxP = max_blk == 0 ? 1
                           : static_cast<int>(std::min<int64_t>(
                                 (max_blk + kMinChunkBlocks - 1) / kMinChunkBlocks + 1, lp.W));
  } else {
    lp.P = partition_size > 0 ? partition_size : kDefaultPartition;  // 0 or -1 on fp32
    lp.maxP = max_ctx <= 0 ? 1
                           : static_cast<int>((static_cast<int64_t>(max_ctx) + lp.P - 1) / lp.P);
  }
  return lp;
}

// Events armed by pa_time_next_attention for the next attention kernel of
// this host thread; consumed (and cleared) by the next decode call.
struct TimingEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
thread_local TimingEvents t_armed;
thread_local TimingEvents t_call;   // the events of the call in progress

// Launches an attention kernel; with events armed for the call, they are
// recorded by the kernel's own dispatch (start and end of its execution).
template <typename K>
void launch_attention(K kernel, dim3 grid, dim3 block, hipStream_t s, const Params& pr) {
  if (t_call.start != nullptr) {
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, t_call.start, t_call.stop, 0, pr);
    t_call = TimingEvents{};
  } else {
    kernel<<<grid, block, 0, s>>>(pr);
  }
}

// Fixed partitions on the 4x4x4 engine with NG head groups.
// (two head groups: 2 waves per SIMD, whose 256 registers hold both
// groups' state without spilling at D = 128; three or four: 1 wave per SIMD)
template <typename T, int D, int NG>
void launch_fixed4(const Params& pr, bool fused, hipStream_t s) {
  constexpr int kWaves = NG == 1 ? kFixedWaves4 : NG == 2 ? 2 : 1;
  // x = KV head + Hkv * partition (the heads of one partition are dispatched
  // together), z = sequence
  const dim3 grid(pr.Hkv * pr.maxP, 1, pr.B);
  if (fused)
    launch_attention(decode_fixed_kernel<Engine4<T, D, NG>, true, kWaves>, grid, 64, s, pr);
  else
    launch_attention(decode_fixed_kernel<Engine4<T, D, NG>, false, kWaves>, grid, 64, s, pr);
}

// The even split over W waves on the 4x4x4 engine with NG head groups.
template <typename T, int D, int NG>
void launch_split4(const Params& pr, int W, hipStream_t s) {
  launch_attention(decode_split_kernel<Engine4<T, D, NG>, 1>, W / kSplitWavesPerGroup,
                   64 * kSplitWavesPerGroup, s, pr);
}

// The matrix-core attention kernel for G = Hq / Hkv <= kMaxGroup: ceil(G / 4)
// head groups, on the even split (split) or fixed partitions (fused: the
// kernel appends the step's new tokens).
template <typename T, int D, int NG>
void launch_matrix_ng(const Params& pr, bool split, int W, bool fused, hipStream_t s) {
  if (split)
    launch_split4<T, D, NG>(pr, W, s);
  else
    launch_fixed4<T, D, NG>(pr, fused, s);
}
template <typename T, int D>
void launch_matrix(const Params& pr, bool split, int W, bool fused, hipStream_t s) {
  static_assert(kMaxGroup == 16, "head groups 1..4 cover G <= 16");
  switch ((pr.G + 3) / 4) {
    case 1: launch_matrix_ng<T, D, 1>(pr, split, W, fused, s); break;
    case 2: launch_matrix_ng<T, D, 2>(pr, split, W, fused, s); break;
    case 3: launch_matrix_ng<T, D, 3>(pr, split, W, fused, s); break;
    default: launch_matrix_ng<T, D, 4>(pr, split, W, fused, s); break;
  }
}

template <typename T, int D>
void launch_partitions(const Params& pr, bool generic, bool fused, hipStream_t s) {
  if (generic)
    launch_attention(decode_generic_kernel<T, D>, dim3(pr.maxP, pr.Hkv, pr.B), 256, s, pr);
  else
    launch_matrix<T, D>(pr, false, 0, fused, s);
}

template <>
void launch_partitions<F32, 64>(const Params& pr, bool, bool, hipStream_t s) {
  launch_attention(decode_generic_kernel<F32, 64>, dim3(pr.maxP, pr.Hkv, pr.B), 256, s, pr);
}
template <>
void launch_partitions<F32, 128>(const Params& pr, bool, bool, hipStream_t s) {
  launch_attention(decode_generic_kernel<F32, 128>, dim3(pr.maxP, pr.Hkv, pr.B), 256, s, pr);
}

enum class Phase { kPartitions = 1, kMerge = 2, kBoth = 3 };

// 8-bit pools (C = E4M3 or I8): the 4x4x4 engine.
template <typename C, int D>
void launch_code_phases(const Params& pr, const LaunchPlan& lp, bool first, bool second,
                        hipStream_t s) {
  if (first) launch_matrix<C, D>(pr, lp.split, lp.W, pr.k_new != nullptr, s);
  if (lp.split) {
    if (second) launch_merge<D, true, C>(pr, s);
    return;
  }
  // with the step's new tokens the merge kernel always runs: it writes them
  if (second && (pr.maxP > 1 || pr.write_new_in_merge))
    launch_merge<D, false, C>(pr, s);
}

template <int D>
void launch_phases(const Params& pr, pa_dtype dt, const LaunchPlan& lp, Phase ph,
                   hipStream_t s) {
  const bool first = static_cast<int>(ph) & static_cast<int>(Phase::kPartitions);
  const bool second = static_cast<int>(ph) & static_cast<int>(Phase::kMerge);
  if (dt == PA_FP8_E4M3) return launch_code_phases<E4M3, D>(pr, lp, first, second, s);
  if (dt == PA_INT8) return launch_code_phases<I8, D>(pr, lp, first, second, s);
  if (lp.split) {
    if (first) {
      if (dt == PA_F16)
        launch_matrix<F16, D>(pr, true, lp.W, false, s);
      else
        launch_matrix<BF16, D>(pr, true, lp.W, false, s);
    }
    if (second) launch_merge<D, true>(pr, s);
    return;
  }
  if (first) {
    switch (dt) {
      case PA_F32: launch_partitions<F32, D>(pr, true, false, s); break;
      case PA_F16: launch_partitions<F16, D>(pr, lp.generic, pr.k_new != nullptr, s); break;
      case PA_BF16: launch_partitions<BF16, D>(pr, lp.generic, pr.k_new != nullptr, s); break;
    }
  }
  if (second && pr.maxP > 1) launch_merge<D, false>(pr, s);
}

// Whether the partition kernel of this plan appends the step's new tokens
// itself (pa_decode_step); otherwise pa_cache_append runs first.
bool fuses_append(const LaunchPlan& lp) { return !lp.generic; }

// Validates the arguments shared by pa_decode / pa_decode_partial /
// pa_decode_merge and launches the requested phases.
struct NewTokens {
  const void* k_new;
  const void* v_new;
  const int64_t* slots;
};
// Scales of a quantized cache (pa_decode_quant / pa_decode_step_quant).
struct CodeScales {
  float k_scale;
  float v_scale;
};

// Shared prefixes of pa_decode_step_shared: the prefix pass's outputs.
struct SharedPrefix {
  const int32_t* prefix;
  const float* pre_out;
  const float2* pre_ml;
  uint32_t* pre_stamp;
  uint32_t epoch;
  int pieces;
  hipEvent_t join;   // recorded after the prefix pass on another stream: the merge waits
};

pa_status run_decode(const char* fn, Phase ph, const NewTokens* nt, const CodeScales* cs,
                     int32_t window, const SharedPrefix* shp, float* out, const void* q,
                     const void* k_pool, const void* v_pool, const int32_t* block_tables,
                     const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                     int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                     float scale, int32_t partition_size, pa_dtype dtype, void* workspace,
                     size_t workspace_bytes_given, void* stream) {
  t_call = t_armed;   // armed events apply to this call only
  t_armed = TimingEvents{};
  if (block_size != kBlockSize)
    return fail(PA_ERR_UNSUPPORTED, "%s: block_size %d (only 16 is supported)", fn, block_size);
  if (cs == nullptr && code_dtype(dtype))
    return fail(PA_ERR_INVALID_ARG, "%s: 8-bit pools are attended by pa_decode_quant", fn);
  if (cs != nullptr && !code_dtype(dtype))
    return fail(PA_ERR_INVALID_ARG, "%s: cache dtype %d is not an 8-bit code dtype", fn,
                (int)dtype);
  if (!pool_dtype_ok(dtype))
    return fail(PA_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dtype);
  if (cs != nullptr && (!(cs->k_scale > 0.f) || !(cs->v_scale > 0.f) ||
                        !std::isfinite(cs->k_scale) || !std::isfinite(cs->v_scale)))
    return fail(PA_ERR_INVALID_ARG, "%s: scales must be positive and finite", fn);
  if (head_dim != 64 && head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "%s: head_dim %d (64 or 128 supported)", fn, head_dim);
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARG, "%s: num_q_heads %d not a multiple of num_kv_heads %d", fn,
                num_q_heads, num_kv_heads);
  if (num_q_heads / num_kv_heads > kMaxGroup)
    return fail(PA_ERR_UNSUPPORTED, "%s: %d query heads per KV head (max %d)", fn,
                num_q_heads / num_kv_heads, kMaxGroup);
  if (num_seqs < 0 || num_seqs > 65535 || num_kv_heads > 65535)
    return fail(PA_ERR_INVALID_ARG, "%s: num_seqs/num_kv_heads out of range", fn);
  if (num_blocks <= 0 || max_blocks_per_seq < 0 || max_context_len < 0)
    return fail(PA_ERR_INVALID_ARG, "%s: negative or zero size", fn);
  if (!partition_ok(partition_size))
    return fail(PA_ERR_INVALID_ARG, "%s: partition_size %d (a multiple of 16, 0 or -1)", fn,
                partition_size);
  if (!(scale > 0.f) || !std::isfinite(scale))
    return fail(PA_ERR_INVALID_ARG, "%s: scale must be positive and finite", fn);
  if (window < 0) return fail(PA_ERR_INVALID_ARG, "%s: window %d < 0", fn, window);
  if (num_seqs == 0) return ok();
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens)
    return fail(PA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_pool) |
       reinterpret_cast<uintptr_t>(v_pool)) & 15)
    return fail(PA_ERR_INVALID_ARG, "%s: q and pools must be 16-byte aligned", fn);

  if (nt && (!nt->k_new || !nt->v_new || !nt->slots))
    return fail(PA_ERR_INVALID_ARG, "%s: NULL new-token pointer", fn);
  if (nt && ((reinterpret_cast<uintptr_t>(nt->k_new) | reinterpret_cast<uintptr_t>(nt->v_new)) & 15))
    return fail(PA_ERR_INVALID_ARG, "%s: k_new and v_new must be 16-byte aligned", fn);
  const LaunchPlan lp = make_plan(num_seqs, num_kv_heads, max_context_len, partition_size, dtype,
                                  generic_selected());
  if (lp.unfit)
    return fail(PA_ERR_UNSUPPORTED,
                "%s: %d sequences x %d KV heads up to %d positions exceed the even split's "
                "32-bit work count; give a partition size",
                fn, num_seqs, num_kv_heads, max_context_len);
  if (shp && !lp.split)
    return fail(PA_ERR_UNSUPPORTED, "%s: shared prefixes need the even split on the matrix cores",
                fn);
  const size_t need = workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, lp.maxP);
  if (need > 0 && (!workspace || workspace_bytes_given < need))
    return fail(PA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                workspace ? workspace_bytes_given : size_t(0));
  if (need > 0 && (reinterpret_cast<uintptr_t>(workspace) & 255))
    return fail(PA_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", fn);

  Params pr{};
  pr.out = out;
  pr.q = q;
  pr.kpool = k_pool;
  pr.vpool = v_pool;
  pr.tables = block_tables;
  pr.lens = context_lens;
  pr.B = num_seqs;
  pr.Hq = num_q_heads;
  pr.Hkv = num_kv_heads;
  pr.G = num_q_heads / num_kv_heads;
  pr.D = head_dim;
  pr.num_blocks = num_blocks;
  pr.max_blocks = max_blocks_per_seq;
  pr.max_ctx = max_context_len;
  pr.P = lp.P;
  pr.maxP = lp.maxP;
  // a quantized cache: K = k_scale * code (folded into the softmax scale),
  // V = v_scale * code (applied to the final rows)
  pr.scale_log2 = (cs ? scale * cs->k_scale : scale) * kLog2e;
  pr.out_scale = cs ? cs->v_scale : 1.0f;
  pr.window = window;
  pr.range_ticks = code_dtype(dtype) ? kRangeTicksCodes : kRangeTicks16;
  if (shp) {
    pr.prefix = shp->prefix;
    pr.pre_out = shp->pre_out;
    pr.pre_ml = shp->pre_ml;
    pr.pre_stamp = shp->pre_stamp;
    pr.epoch = shp->epoch;
    pr.pre_pieces = shp->pieces;
  }
  if (need > 0) {
    const size_t rows = static_cast<size_t>(num_seqs) * num_q_heads * lp.maxP;
    char* ws = static_cast<char*>(workspace);
    pr.part_m = reinterpret_cast<float*>(ws);
    pr.part_l = reinterpret_cast<float*>(ws + align256(rows * sizeof(float)));
    pr.part_acc = reinterpret_cast<float*>(ws + 2 * align256(rows * sizeof(float)));
    pr.counters = reinterpret_cast<int*>(ws + 2 * align256(rows * sizeof(float)) +
                                         align256(rows * head_dim * sizeof(float)));
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (nt) {
    if (fuses_append(lp)) {
      // append fused: the attention kernel uses the new tokens; the merge
      // kernel writes them to the pool when a merge kernel runs, else the
      // attention kernel does
      pr.k_new = nt->k_new;
      pr.v_new = nt->v_new;
      pr.slots = nt->slots;
      pr.kpool_w = const_cast<void*>(k_pool);
      pr.vpool_w = const_cast<void*>(v_pool);
      // 8-bit pools: always the merge kernel (the attention kernel only
      // attends the encoded tokens)
      pr.write_new_in_merge = lp.split || lp.maxP > 1 || cs != nullptr;
      if (cs) {   // the same fp32 reciprocals as pa_cache_append_quant's
        pr.enc_k = 1.0f / cs->k_scale;
        pr.enc_v = 1.0f / cs->v_scale;
      }
    } else if (static_cast<int>(ph) & static_cast<int>(Phase::kPartitions)) {
      const pa_status st =
          cs ? pa_cache_append_quant(const_cast<void*>(k_pool), const_cast<void*>(v_pool),
                                     nt->k_new, nt->v_new, nt->slots, num_seqs, num_blocks,
                                     num_kv_heads, head_dim, block_size, dtype, PA_BF16,
                                     cs->k_scale, cs->v_scale, stream)
             : pa_cache_append(const_cast<void*>(k_pool), const_cast<void*>(v_pool), nt->k_new,
                               nt->v_new, nt->slots, num_seqs, num_blocks, num_kv_heads,
                               head_dim, block_size, dtype, stream);
      if (st != PA_OK) return st;
    }
  }
  auto phases = [&](Phase p) {
    if (head_dim == 64)
      launch_phases<64>(pr, dtype, lp, p, s);
    else
      launch_phases<128>(pr, dtype, lp, p, s);
  };
  if (shp && shp->join && ph == Phase::kBoth) {
    // the prefix pass runs beside the attention kernel; the merge needs both
    phases(Phase::kPartitions);
    const hipError_t e = hipStreamWaitEvent(s, shp->join, 0);
    if (e != hipSuccess)
      return fail(PA_ERR_HIP, "%s: hipStreamWaitEvent: %s", fn, hipGetErrorString(e));
    phases(Phase::kMerge);
  } else {
    phases(ph);
  }
  return launch_status(fn);
}

// ---------------------------------------------------------------------------
// Fixed device scratch of pa_decode_step_noalloc, for callers that cannot
// allocate device memory.  Each device holds its own copy of the array from
// the library's load until the process ends.  In host code `scratch` names a
// host-side stand-in, never the device memory: its device address is looked
// up once per device (hipGetSymbolAddress, with that device current) and only
// that address is passed to kernels.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of the current device's scratch array (looked up on the
// first call on each device).
pa_status scratch_of_current_device(const char* fn, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess)
    return fail(PA_ERR_HIP, "%s: hipGetDevice failed", fn);
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(PA_ERR_UNSUPPORTED, "%s: device %d beyond the %d with a scratch address slot", fn,
                dev, kMaxScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return fail(PA_ERR_HIP, "%s: hipGetSymbolAddress(scratch) on device %d: %s", fn, dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return ok();
}

}  // namespace
}  // namespace pa

using namespace pa;

extern "C" pa_decode_kernel pa_set_decode_kernel(pa_decode_kernel kernel) {
  if (kernel != PA_KERNEL_AUTO && kernel != PA_KERNEL_GENERIC) {
    fail(PA_ERR_INVALID_ARG, "pa_set_decode_kernel: unknown kernel %d", (int)kernel);
    return static_cast<pa_decode_kernel>(g_decode_kernel.load());
  }
  return static_cast<pa_decode_kernel>(g_decode_kernel.exchange(kernel));
}

extern "C" pa_status pa_time_next_attention(void* start_event, void* stop_event) {
  if ((start_event == nullptr) != (stop_event == nullptr))
    return fail(PA_ERR_INVALID_ARG, "pa_time_next_attention: give both events or neither");
  t_armed = TimingEvents{static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event)};
  return ok();
}

extern "C" int32_t pa_decode_partition_size(int32_t num_seqs, int32_t num_q_heads,
                                            int32_t num_kv_heads, int32_t head_dim,
                                            int32_t max_context_len, int32_t partition_size,
                                            pa_dtype dtype) {
  if (!decode_args_ok(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                      partition_size, dtype))
    return -1;
  const LaunchPlan lp =
      make_plan(num_seqs, num_kv_heads, max_context_len, partition_size, dtype,
                generic_selected());
  return lp.unfit ? -1 : lp.P;
}

extern "C" size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                            int32_t num_kv_heads, int32_t head_dim,
                                            int32_t max_context_len, int32_t partition_size,
                                            pa_dtype dtype) {
  if (!decode_args_ok(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                      partition_size, dtype))
    return 0;
  const LaunchPlan lp = make_plan(num_seqs, num_kv_heads, max_context_len, partition_size,
                                  dtype, generic_selected());
  if (lp.unfit) return 0;
  return workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, lp.maxP);
}

#define PA_DECODE_ARGS                                                                      \
  float *out, const void *q, const void *k_pool, const void *v_pool,                          \
      const int32_t *block_tables, const int32_t *context_lens, int32_t num_seqs,             \
      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,        \
      int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len, float scale,   \
      int32_t partition_size, pa_dtype dtype, void *workspace, size_t workspace_bytes_given,  \
      void *stream
#define PA_DECODE_FWD                                                                        \
  out, q, k_pool, v_pool, block_tables, context_lens, num_seqs, num_q_heads, num_kv_heads,    \
      head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len, scale,           \
      partition_size, dtype, workspace, workspace_bytes_given, stream

extern "C" pa_status pa_decode(PA_DECODE_ARGS) {
  return run_decode("pa_decode", Phase::kBoth, nullptr, nullptr, 0, nullptr, PA_DECODE_FWD);
}

extern "C" pa_status pa_decode_partial(PA_DECODE_ARGS) {
  return run_decode("pa_decode_partial", Phase::kPartitions, nullptr, nullptr, 0, nullptr, PA_DECODE_FWD);
}

extern "C" pa_status pa_decode_merge(PA_DECODE_ARGS) {
  return run_decode("pa_decode_merge", Phase::kMerge, nullptr, nullptr, 0, nullptr, PA_DECODE_FWD);
}

#define PA_STEP_ARGS                                                                        \
  float *out, const void *q, void *k_pool, void *v_pool, const void *k_new, const void *v_new, \
      const int64_t *slot_mapping, const int32_t *block_tables, const int32_t *context_lens,  \
      int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,          \
      int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,                     \
      int32_t max_context_len, float scale, int32_t partition_size, pa_dtype dtype,           \
      void *workspace, size_t workspace_bytes_given, void *stream
#define PA_STEP_FWD                                                                         \
  out, q, k_pool, v_pool, block_tables, context_lens, num_seqs, num_q_heads, num_kv_heads,    \
      head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len, scale,           \
      partition_size, dtype, workspace, workspace_bytes_given, stream

extern "C" pa_status pa_decode_step(PA_STEP_ARGS) {
  const NewTokens nt{k_new, v_new, slot_mapping};
  return run_decode("pa_decode_step", Phase::kBoth, &nt, nullptr, 0, nullptr, PA_STEP_FWD);
}

extern "C" pa_status pa_decode_step_noalloc(
    float* out, const void* q, void* k_pool, void* v_pool, const void* k_new, const void* v_new,
    const int64_t* slot_mapping, const int32_t* block_tables, const int32_t* context_lens,
    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
    int32_t max_context_len, float scale, int32_t partition_size, pa_dtype dtype,
    void* stream) {
  const char* fn = "pa_decode_step_noalloc";
  // the partials this call needs, checked against the array before any
  // device call (0 for invalid arguments: run_decode reports those)
  const size_t need = pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                max_context_len, partition_size, dtype);
  if (need > kScratchBytes)
    return fail(PA_ERR_WORKSPACE,
                "%s: these sizes need %zu bytes of partials; the static scratch holds %zu "
                "(use pa_decode_step with a workspace)", fn, need, kScratchBytes);
  void* workspace = nullptr;
  if (need > 0 && num_seqs > 0) {
    const pa_status st = scratch_of_current_device(fn, &workspace);
    if (st != PA_OK) return st;
  }
  const NewTokens nt{k_new, v_new, slot_mapping};
  const size_t workspace_bytes_given = workspace ? kScratchBytes : 0;
  return run_decode(fn, Phase::kBoth, &nt, nullptr, 0, nullptr, PA_STEP_FWD);
}

// Side stream of pa_decode_step_shared, per device: the prefix pass runs on it
// beside the attention kernel on the caller's stream (both are bound by
// memory latency at these sizes, so running together they overlap their
// waits).  `fork` is recorded on the caller's stream and waited by the side
// stream; `join` is recorded after the prefix pass and waited by the
// caller's stream before the merge.  Created on the first call on each device
// (default priority, non-blocking), kept until the process ends.  The events
// are shared by every call on the device, so one call's fork-to-wait sequence
// is enqueued under g_side_mu.
struct SideStream {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_side_mu;
SideStream g_side[kMaxScratchDevices];

// The current device's side stream (g_side_mu held by the caller).
pa_status side_stream_of_current_device(const char* fn, SideStream** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(PA_ERR_UNSUPPORTED, "%s: device %d beyond the %d supported", fn, dev,
                kMaxScratchDevices);
  SideStream& ss = g_side[dev];
  if (ss.stream == nullptr) {
    SideStream n;
    e = hipStreamCreateWithFlags(&n.stream, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&n.fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&n.join, hipEventDisableTiming);
    if (e != hipSuccess) {
      if (n.join) (void)hipEventDestroy(n.join);
      if (n.fork) (void)hipEventDestroy(n.fork);
      if (n.stream) (void)hipStreamDestroy(n.stream);
      return fail(PA_ERR_HIP, "%s: side stream set-up: %s", fn, hipGetErrorString(e));
    }
    ss = n;
  }
  *out = &ss;
  return ok();
}

// Workspace of pa_decode_step_shared: the even split's partials, then the
// prefix pass's rows, their (max, sum) pairs and per-sequence stamps.
struct SharedWorkspace {
  size_t split, pre_out, pre_ml, stamp, total;   // byte offsets of the parts; total size
};
SharedWorkspace shared_workspace_parts(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                       int32_t max_ctx, pa_dtype dtype) {
  SharedWorkspace w{};
  w.split = 0;
  w.pre_out = align256(pa_decode_workspace_bytes(B, Hq, Hkv, D, max_ctx, kEvenSplit, dtype));
  const size_t P = kMaxPrefixPieces;
  w.pre_ml = w.pre_out + align256(P * B * Hq * D * sizeof(float));
  w.stamp = w.pre_ml + align256(P * B * Hq * sizeof(float2));
  w.total = w.stamp + align256(P * B * Hq * sizeof(uint32_t));
  return w;
}

// Epoch of each pa_decode_step_shared call (never 0: a fresh workspace may
// hold zeros).
std::atomic<uint32_t> g_shared_epoch{0};
uint32_t next_epoch() {
  uint32_t e = g_shared_epoch.fetch_add(1, std::memory_order_relaxed) + 1;
  while (e == 0) e = g_shared_epoch.fetch_add(1, std::memory_order_relaxed) + 1;
  return e;
}

extern "C" size_t pa_decode_shared_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                                   int32_t num_kv_heads, int32_t head_dim,
                                                   int32_t max_context_len, pa_dtype dtype) {
  if (!decode_args_ok(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                      kEvenSplit, dtype))
    return 0;
  return shared_workspace_parts(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                                dtype)
      .total;
}

extern "C" pa_status pa_decode_step_shared(
    float* out, const void* q, void* k_pool, void* v_pool, const void* k_new, const void* v_new,
    const int64_t* slot_mapping, const int32_t* block_tables, const int32_t* context_lens,
    const int32_t* prefix_len, const int32_t* group_rows, const int32_t* group_start,
    int32_t num_groups, int32_t num_rows, int32_t max_group_size, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
    pa_dtype dtype, void* workspace, size_t workspace_bytes_given, void* stream) {
  const char* fn = "pa_decode_step_shared";
  if (dtype != PA_BF16 && dtype != PA_F16)
    return fail(PA_ERR_UNSUPPORTED, "%s: dtype %d (fp16/bf16 pools only)", fn, (int)dtype);
  if (generic_selected())
    return fail(PA_ERR_UNSUPPORTED, "%s: needs the matrix-core kernels", fn);
  if (!(scale > 0.f) || !std::isfinite(scale))
    return fail(PA_ERR_INVALID_ARG, "%s: scale must be positive and finite", fn);
  if (num_groups < 0 || num_rows < 0 || max_group_size < 0 || num_rows > num_seqs ||
      (num_groups > 0 && (num_rows < 2 * num_groups || max_group_size < 2 ||
                          max_group_size > num_rows)))
    return fail(PA_ERR_INVALID_ARG, "%s: bad group counts", fn);
  if (num_seqs > 0 && !decode_args_ok(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                      max_context_len, kEvenSplit, dtype))
    return fail(PA_ERR_INVALID_ARG, "%s: bad sizes", fn);
  if (num_seqs > 0 && (!prefix_len || (num_groups > 0 && (!group_rows || !group_start))))
    return fail(PA_ERR_INVALID_ARG, "%s: NULL prefix or group pointer", fn);
  const SharedWorkspace wp =
      num_seqs > 0 ? shared_workspace_parts(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                            max_context_len, dtype)
                   : SharedWorkspace{};
  const size_t need = wp.total;
  if (need > 0 && (!workspace || workspace_bytes_given < need))
    return fail(PA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                workspace ? workspace_bytes_given : size_t(0));
  if (need > 0 && (reinterpret_cast<uintptr_t>(workspace) & 255))
    return fail(PA_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", fn);
  if (num_seqs == 0) return ok();
  char* ws = static_cast<char*>(workspace);
  float* pre_out = reinterpret_cast<float*>(ws + wp.pre_out);
  float2* pre_ml = reinterpret_cast<float2*>(ws + wp.pre_ml);
  uint32_t* pre_stamp = reinterpret_cast<uint32_t*>(ws + wp.stamp);
  const uint32_t epoch = next_epoch();
  // The step's new tokens are never in a shared prefix (every member keeps
  // its last position, and its last block is its own), so the prefix pass
  // reads nothing the step writes; it runs on the side stream, after the
  // caller's earlier work (copy-on-write copies) and beside the attention
  // kernel, and the merge waits for it.
  std::unique_lock<std::mutex> lock(g_side_mu, std::defer_lock);
  hipEvent_t join = nullptr;
  const int pieces = num_groups > 0 ? shared_prefix_pieces(num_groups, max_group_size, num_q_heads,
                                                           num_kv_heads, max_context_len)
                                    : 1;
  if (num_groups > 0) {
    if (block_size != kBlockSize)
      return fail(PA_ERR_UNSUPPORTED, "%s: block_size %d (only 16 is supported)", fn, block_size);
    if (!q || !k_pool || !v_pool || !block_tables)
      return fail(PA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    lock.lock();
    SideStream* ss = nullptr;
    pa_status st = side_stream_of_current_device(fn, &ss);
    if (st != PA_OK) return st;
    hipStream_t cs = static_cast<hipStream_t>(stream);
    hipError_t e = hipEventRecord(ss->fork, cs);
    if (e == hipSuccess) e = hipStreamWaitEvent(ss->stream, ss->fork, 0);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: fork: %s", fn, hipGetErrorString(e));
    st = launch_shared_prefix(pre_out, reinterpret_cast<float*>(pre_ml), pre_stamp, epoch, pieces, q,
                              k_pool, v_pool, block_tables, prefix_len, group_rows, group_start,
                              num_groups, num_rows, max_group_size, num_seqs, num_q_heads,
                              num_kv_heads, head_dim, num_blocks, max_blocks_per_seq,
                              max_context_len, scale, dtype, ss->stream);
    if (st != PA_OK) return st;
    e = hipEventRecord(ss->join, ss->stream);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: join: %s", fn, hipGetErrorString(e));
    join = ss->join;
  }
  const NewTokens nt{k_new, v_new, slot_mapping};
  const SharedPrefix shp{prefix_len, pre_out, pre_ml, pre_stamp, epoch, pieces, join};
  const int32_t partition_size = kEvenSplit;
  const pa_status st =
      run_decode(fn, Phase::kBoth, &nt, nullptr, 0, &shp, out, q, k_pool, v_pool, block_tables,
                 context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                 num_blocks, max_blocks_per_seq, max_context_len, scale, partition_size, dtype,
                 workspace, wp.pre_out, stream);
  // on an error the caller's stream still waits for the prefix pass, so
  // nothing it frees afterwards is still being written
  if (st != PA_OK && join) (void)hipStreamWaitEvent(static_cast<hipStream_t>(stream), join, 0);
  return st;
}

extern "C" pa_status pa_decode_step_partial(PA_STEP_ARGS) {
  const NewTokens nt{k_new, v_new, slot_mapping};
  return run_decode("pa_decode_step_partial", Phase::kPartitions, &nt, nullptr, 0, nullptr, PA_STEP_FWD);
}

extern "C" pa_status pa_decode_step_merge(PA_STEP_ARGS) {
  const NewTokens nt{k_new, v_new, slot_mapping};
  return run_decode("pa_decode_step_merge", Phase::kMerge, &nt, nullptr, 0, nullptr, PA_STEP_FWD);
}

extern "C" pa_status pa_decode_quant(float* out, const void* q, const void* k_pool,
                                     const void* v_pool, const int32_t* block_tables,
                                     const int32_t* context_lens, int32_t num_seqs,
                                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                     int32_t block_size, int32_t num_blocks,
                                     int32_t max_blocks_per_seq, int32_t max_context_len,
                                     float scale, int32_t partition_size, pa_dtype dtype,
                                     float k_scale, float v_scale, void* workspace,
                                     size_t workspace_bytes_given, void* stream) {
  const CodeScales cs{k_scale, v_scale};
  return run_decode("pa_decode_quant", Phase::kBoth, nullptr, &cs, 0, nullptr, PA_DECODE_FWD);
}

extern "C" pa_status pa_decode_step_quant(float* out, const void* q, void* k_pool, void* v_pool,
                                          const void* k_new, const void* v_new,
                                          const int64_t* slot_mapping,
                                          const int32_t* block_tables,
                                          const int32_t* context_lens, int32_t num_seqs,
                                          int32_t num_q_heads, int32_t num_kv_heads,
                                          int32_t head_dim, int32_t block_size,
                                          int32_t num_blocks, int32_t max_blocks_per_seq,
                                          int32_t max_context_len, float scale,
                                          int32_t partition_size, pa_dtype dtype, float k_scale,
                                          float v_scale, void* workspace,
                                          size_t workspace_bytes_given, void* stream) {
  const NewTokens nt{k_new, v_new, slot_mapping};
  const CodeScales cs{k_scale, v_scale};
  return run_decode("pa_decode_step_quant", Phase::kBoth, &nt, &cs, 0, nullptr, PA_STEP_FWD);
}

extern "C" pa_status pa_decode_window(float* out, const void* q, const void* k_pool,
                                      const void* v_pool, const int32_t* block_tables,
                                      const int32_t* context_lens, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                      int32_t max_blocks_per_seq, int32_t max_context_len,
                                      float scale, int32_t window, int32_t partition_size,
                                      pa_dtype dtype, void* workspace,
                                      size_t workspace_bytes_given, void* stream) {
  return run_decode("pa_decode_window", Phase::kBoth, nullptr, nullptr, window, nullptr, PA_DECODE_FWD);
}

extern "C" pa_status pa_decode_step_window(float* out, const void* q, void* k_pool,
                                           void* v_pool, const void* k_new, const void* v_new,
                                           const int64_t* slot_mapping,
                                           const int32_t* block_tables,
                                           const int32_t* context_lens, int32_t num_seqs,
                                           int32_t num_q_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t block_size,
                                           int32_t num_blocks, int32_t max_blocks_per_seq,
                                           int32_t max_context_len, float scale, int32_t window,
                                           int32_t partition_size, pa_dtype dtype,
                                           void* workspace, size_t workspace_bytes_given,
                                           void* stream) {
  const NewTokens nt{k_new, v_new, slot_mapping};
  return run_decode("pa_decode_step_window", Phase::kBoth, &nt, nullptr, window, nullptr, PA_STEP_FWD);
}
