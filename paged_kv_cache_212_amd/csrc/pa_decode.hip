// PagedAttention decode on gfx950.
//
// For every sequence b, KV head g and partition p (a run of P tokens), one
// workgroup walks the block table from logical to physical blocks and reads
// the 16-token K and V tiles it needs, in logical order (page 3, abeam.tech
// review, sections 「用語解説」 (block table) and
// 「モデル構造ではなくサービング基盤の変更」: the kernel follows the table to read
// the KV it needs).  It computes softmax(scale * q.K^T) V for the G query
// heads that share KV head g with an online (running max, running sum)
// softmax.  A sequence longer than one partition leaves per-partition
// (max, sum, weighted V) partials that merge_kernel combines with a
// log-sum-exp reduction; paging changes where K/V live, not the result (page 3,
// section 「よくある質問」; page 4, FAQ).
//
// Two partition kernels:
//   * decode_mfma_kernel (fp16/bf16, G <= 16): one 64-lane wave per block at a
//     time; S^T = K.Q^T on a 16x16x32 MFMA (tokens x heads), P.V on 16x16x16
//     MFMAs (heads x dims) with P split into a high and a low half-precision
//     part so the weights keep ~16 (bf16) / ~22 (fp16) significant bits.
//   * decode_generic_kernel (any dtype): plain fp32 FMAs, one thread per
//     (head, token) score and per (head, dim) output.
// Scores are kept in the log2 domain (scale * log2(e) folded in) and
// exponentiated with exp2.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <cstring>

#include "pa_device.h"

namespace pa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxGroup = 16;  // query heads per KV head supported

struct Params {
  float* out;          // [B][Hq][D]
  float* part_m;       // [B][Hq][maxP]   running max (log2 domain) per partition
  float* part_l;       // [B][Hq][maxP]   sum of exp2(s - m)
  float* part_acc;     // [B][Hq][maxP][D] sum of exp2(s - m) * v
  const void* q;       // [B][Hq][D]
  const void* kpool;
  const void* vpool;
  const int32_t* tables;
  const int32_t* lens;
  int B, Hq, Hkv, G, D;
  int num_blocks, max_blocks, max_ctx;
  int P, maxP;
  float scale_log2;
};

__device__ inline bool len_valid(int L, const Params& pr) {
  return L >= 0 && L <= pr.max_ctx && L <= pr.max_blocks * kBlockSize;
}

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
  const int np = (L + pr.P - 1) / pr.P;
  if (p >= np) return;
  const int tok0 = p * pr.P, tok1 = min(L, tok0 + pr.P);

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
          a = fmaf(ss[h][t], T::to_float(vt[v_elem(pos % kBlockSize, d)]), a);
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
// Matrix-core partition kernel.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <typename T>
struct Mfma;

template <>
struct Mfma<BF16> {
  // S^T tile (16 tokens x 16 heads) += K (16 tokens x 32 dims) . Q^T (32 dims x 16 heads)
  __device__ static inline f32x4_t qk(uint4 k, uint4 q, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, k),
                                                   __builtin_bit_cast(bf16x8_t, q), c, 0, 0, 0);
  }
  // O tile (16 heads x 16 dims) += P (16 heads x 16 tokens) . V (16 tokens x 16 dims)
  __device__ static inline f32x4_t pv(uint2 p, uint2 v, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, p),
                                                     __builtin_bit_cast(i16x4_t, v), c, 0, 0, 0);
  }
  // O tile (16 heads x 16 dims) += P (16 heads x 32 tokens) . V (32 tokens x 16 dims)
  __device__ static inline f32x4_t pv8(uint4 p, uint4 v, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, p),
                                                   __builtin_bit_cast(bf16x8_t, v), c, 0, 0, 0);
  }
  __device__ static inline void split8(const float pe[8], uint4& hi, uint4& lo) {
    uint32_t h[8], l[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t u = __float_as_uint(pe[e]);
      h[e] = u >> 16;
      const float r = pe[e] - __uint_as_float(u & 0xFFFF0000u);
      l[e] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(r));
    }
    hi = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                    h[6] | (h[7] << 16));
    lo = make_uint4(l[0] | (l[1] << 16), l[2] | (l[3] << 16), l[4] | (l[5] << 16),
                    l[6] | (l[7] << 16));
  }
  // p (>= 0) = hi + lo with hi = p truncated to bf16 (exact remainder) and
  // lo = remainder rounded to bf16.
  __device__ static inline void split(const float pe[4], uint2& hi, uint2& lo) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t u = __float_as_uint(pe[e]);
      h[e] = u >> 16;
      const float r = pe[e] - __uint_as_float(u & 0xFFFF0000u);
      l[e] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(r));
    }
    hi = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
    lo = make_uint2(l[0] | (l[1] << 16), l[2] | (l[3] << 16));
  }
};

template <>
struct Mfma<F16> {
  __device__ static inline f32x4_t pv8(uint4 p, uint4 v, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, p),
                                                  __builtin_bit_cast(f16x8_t, v), c, 0, 0, 0);
  }
  __device__ static inline void split8(const float pe[8], uint4& hi, uint4& lo) {
    uint32_t h[8], l[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const _Float16 hh = static_cast<_Float16>(pe[e]);
      const float r = pe[e] - static_cast<float>(hh);
      h[e] = __builtin_bit_cast(uint16_t, hh);
      l[e] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(r));
    }
    hi = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                    h[6] | (h[7] << 16));
    lo = make_uint4(l[0] | (l[1] << 16), l[2] | (l[3] << 16), l[4] | (l[5] << 16),
                    l[6] | (l[7] << 16));
  }
  __device__ static inline f32x4_t qk(uint4 k, uint4 q, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, k),
                                                  __builtin_bit_cast(f16x8_t, q), c, 0, 0, 0);
  }
  __device__ static inline f32x4_t pv(uint2 p, uint2 v, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, p),
                                                 __builtin_bit_cast(f16x4_t, v), c, 0, 0, 0);
  }
  __device__ static inline void split(const float pe[4], uint2& hi, uint2& lo) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const _Float16 hh = static_cast<_Float16>(pe[e]);
      const float r = pe[e] - static_cast<float>(hh);
      h[e] = __builtin_bit_cast(uint16_t, hh);
      l[e] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(r));
    }
    hi = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
    lo = make_uint2(l[0] | (l[1] << 16), l[2] | (l[3] << 16));
  }
};

// Two blocks (A = logical block 2q, B = 2q+1 of the partition) per iteration.
// Lane = 16*j + n (n = lane % 16, j = lane / 16).
//   QK, half hh in {0,1}: S^T (16 rows x 16 heads) = K rows . Q^T where row
//     i < 8 is token i + 8*hh of A and row i >= 8 token i - 8 + 8*hh of B.
//     A operand (K): lane reads row n, dims kk*32 + 8j .. +8 (16 bytes).
//     B operand (Q): head n, dims kk*32 + 8j .. +8.
//     Result: lane (head n, j) holds rows 4j+e, i.e. block j/2, tokens
//     4*(j%2) + e + 8*hh (e = 0..3).
//   PV: O (16 heads x 16 dims) += P (heads x 32 tokens) . V (32 tokens x dims)
//     with lane (n, j) holding k-slots {S_hh0[e], S_hh1[e]}: 8 tokens of block
//     j/2, namely 4*(j%2) + {0..3} and 8 + 4*(j%2) + {0..3}.  In the V tile
//     the 16 token slots of each dim row are stored in the order 0-3, 8-11,
//     4-7, 12-15, so those 8 tokens are 16 contiguous bytes at
//     dim*32 + 16*(j%2): one 16-byte load per lane and tile.
//   O result: lane (dim t*16 + n, j) holds heads 4j + e.
// K tile (block, head) bytes: [D/8 chunks][16 tokens][8 dims] -> chunk
// kk*4 + j, token r at (kk*4 + j)*256 + 16*r.
//
// One wave per (KV head, partition, sequence).  NPAIR block pairs are in
// flight in a register ring; the loop is peeled so the steady state issues
// its loads unconditionally (static wait counts) and the tail issues none.
template <typename T, int D, int NPAIR, bool kSmallGroup>
__global__ __launch_bounds__(64) void decode_mfma_kernel(Params pr) {
  constexpr int NKK = D / 32;
  constexpr int NTL = D / 16;
  constexpr int64_t kTileBytes = static_cast<int64_t>(D) * kBlockSize * 2;

  const int g = blockIdx.x % pr.Hkv, p = blockIdx.x / pr.Hkv, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int n = lane & 15, j = lane >> 4;
  const int G = pr.G;
  const int L = pr.lens[b];
  if (!len_valid(L, pr) || L == 0) {
    if (p == 0) write_trivial_rows(pr, b, g, L);
    return;
  }
  const int np = (L + pr.P - 1) / pr.P;
  if (p >= np) return;
  const int tok0 = p * pr.P, tok1 = min(L, tok0 + pr.P);
  const int blk0 = tok0 / kBlockSize;
  const int nblk = (tok1 - tok0 + kBlockSize - 1) / kBlockSize;
  const int npair = (nblk + 1) >> 1;

  uint4 qv[NKK];
  {
    const uint16_t* qb = static_cast<const uint16_t*>(pr.q) +
                         (static_cast<int64_t>(b) * pr.Hq + g * G + n) * D;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      qv[kk] = n < G ? *reinterpret_cast<const uint4*>(qb + kk * 32 + j * 8)
                     : make_uint4(0, 0, 0, 0);
  }

  const char* kbase = static_cast<const char*>(pr.kpool) + g * kTileBytes;
  const char* vbase = static_cast<const char*>(pr.vpool) + g * kTileBytes;
  const int64_t block_stride = static_cast<int64_t>(pr.Hkv) * kTileBytes;
  const int32_t* trow = pr.tables + static_cast<int64_t>(b) * pr.max_blocks + blk0;

  // Table entries, 64 per register (lane i holds entry 64*c + i of chunk c).
  bool bad = false;
  auto load_chunk = [&](int c) -> int {
    const int k = c * 64 + lane;
    const int e = k < nblk ? trow[k] : 0;
    const bool lane_bad = k < nblk && (e < 0 || e >= pr.num_blocks);
    if (__any(lane_bad)) bad = true;
    return lane_bad ? 0 : e;
  };
  int chunk = 0;
  int tcur = load_chunk(0);
  int tnext = nblk > 64 ? load_chunk(1) : 0;
  // Physical block of partition block k (k increases across calls); k >= nblk
  // (the missing half of a last, odd pair) maps to block nblk-1, whose lines
  // are being fetched by the same instruction anyway.
  auto phys_of = [&](int k) -> int {
    if (k >= nblk) k = nblk - 1;
    const int c = k >> 6;
    if (c != chunk) {
      chunk = c;
      tcur = tnext;
      tnext = (c + 1) * 64 < nblk ? load_chunk(c + 1) : 0;
    }
    return __builtin_amdgcn_readlane(tcur, k & 63);
  };

  uint4 kb[NPAIR][2][NKK];
  uint4 vb[NPAIR][NTL];
  auto issue = [&](int u, int q) {
    const int pa = phys_of(2 * q), pb = phys_of(2 * q + 1);
    const int mine = (n < 8) ? pa : pb;             // K row block of this lane
    const char* kt = kbase + mine * block_stride + (n & 7) * 16 + j * 256;
    const char* vt = vbase + ((j >> 1) ? pb : pa) * block_stride + n * 32 + (j & 1) * 16;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
        kb[u][hh][kk] = *reinterpret_cast<const uint4*>(kt + kk * 1024 + hh * 128);
#pragma unroll
    for (int t = 0; t < NTL; ++t) vb[u][t] = *reinterpret_cast<const uint4*>(vt + t * 512);
  };

  float m_run = -INFINITY, l_lane = 0.f;
  f32x4_t acc[NTL];
#pragma unroll
  for (int t = 0; t < NTL; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int u, int q) {
    f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      s0 = Mfma<T>::qk(kb[u][0][kk], qv[kk], s0);
      s1 = Mfma<T>::qk(kb[u][1][kk], qv[kk], s1);
    }
    // position of S_hh[e] in the sequence
    const int base = (blk0 + 2 * q + (j >> 1)) * kBlockSize + 4 * (j & 1);
    float sv[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sv[e] = (base + e < tok1) ? s0[e] * pr.scale_log2 : -INFINITY;
      sv[4 + e] = (base + 8 + e < tok1) ? s1[e] * pr.scale_log2 : -INFINITY;
    }
    float bm = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                     fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
    bm = fmaxf(bm, __shfl_xor(bm, 16));
    bm = fmaxf(bm, __shfl_xor(bm, 32));
    const float mn = fmaxf(m_run, bm);
    if (__any(mn != m_run)) {
      // running max moved for some head: rescale rows 4j+e by 2^(m_old - m_new)
      const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
      l_lane *= alpha;
      if constexpr (kSmallGroup) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float ah = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), e));
#pragma unroll
          for (int t = 0; t < NTL; ++t) acc[t][e] *= ah;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float ah = __shfl(alpha, 4 * j + e);
#pragma unroll
          for (int t = 0; t < NTL; ++t) acc[t][e] *= ah;
        }
      }
      m_run = mn;
    }
    float pe[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pe[e] = __builtin_amdgcn_exp2f(sv[e] - mn);
    l_lane += ((pe[0] + pe[1]) + (pe[2] + pe[3])) + ((pe[4] + pe[5]) + (pe[6] + pe[7]));
    uint4 phi, plo;
    Mfma<T>::split8(pe, phi, plo);
    uint4 vmask = make_uint4(~0u, ~0u, ~0u, ~0u);
    if ((blk0 + 2 * q + 2) * kBlockSize > tok1) {
      // the pair reaches past the end of the sequence: zero V of positions
      // >= L so unused slots (even NaN) cannot reach the output through 0*v
      vmask.x = (base + 0 < tok1 ? 0x0000FFFFu : 0u) | (base + 1 < tok1 ? 0xFFFF0000u : 0u);
      vmask.y = (base + 2 < tok1 ? 0x0000FFFFu : 0u) | (base + 3 < tok1 ? 0xFFFF0000u : 0u);
      vmask.z = (base + 8 < tok1 ? 0x0000FFFFu : 0u) | (base + 9 < tok1 ? 0xFFFF0000u : 0u);
      vmask.w = (base + 10 < tok1 ? 0x0000FFFFu : 0u) | (base + 11 < tok1 ? 0xFFFF0000u : 0u);
    }
#pragma unroll
    for (int t = 0; t < NTL; ++t) {
      const uint4 vv = make_uint4(vb[u][t].x & vmask.x, vb[u][t].y & vmask.y,
                                  vb[u][t].z & vmask.z, vb[u][t].w & vmask.w);
      acc[t] = Mfma<T>::pv8(phi, vv, acc[t]);
      acc[t] = Mfma<T>::pv8(plo, vv, acc[t]);
    }
  };

  // prologue: first min(NPAIR, npair) pairs in flight
#pragma unroll
  for (int u = 0; u < NPAIR; ++u)
    if (u < npair) issue(u, u);
  int q0 = 0;
  for (; q0 + 2 * NPAIR <= npair; q0 += NPAIR) {
#pragma unroll
    for (int u = 0; u < NPAIR; ++u) {
      compute(u, q0 + u);
      issue(u, q0 + u + NPAIR);
    }
  }
  // tail: at most 2*NPAIR - 1 pairs left, the first min(NPAIR, left) in flight
#pragma unroll
  for (int u = 0; u < NPAIR; ++u) {
    if (q0 + u < npair) {
      compute(u, q0 + u);
      if (q0 + u + NPAIR < npair) issue(u, q0 + u + NPAIR);
    }
  }
#pragma unroll
  for (int u = 0; u < NPAIR; ++u)
    if (q0 + NPAIR + u < npair) compute(u, q0 + NPAIR + u);

  l_lane += __shfl_xor(l_lane, 16);
  l_lane += __shfl_xor(l_lane, 32);
  if (bad) {
    m_run = 0.f;
    l_lane = __builtin_nanf("");
#pragma unroll
    for (int t = 0; t < NTL; ++t) acc[t] = f32x4_t{l_lane, l_lane, l_lane, l_lane};
  }

#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int h = 4 * j + e;
    const float mh = __shfl(m_run, h);
    const float lh = __shfl(l_lane, h);
    if (h < G) {
      const int64_t row = static_cast<int64_t>(b) * pr.Hq + g * G + h;
      const float inv = 1.0f / lh;
#pragma unroll
      for (int t = 0; t < NTL; ++t) {
        const int d = t * 16 + n;
        if (np == 1)
          pr.out[row * D + d] = acc[t][e] * inv;
        else
          pr.part_acc[(row * pr.maxP + p) * D + d] = acc[t][e];
      }
      if (np > 1 && n == 0) {
        pr.part_m[row * pr.maxP + p] = mh;
        pr.part_l[row * pr.maxP + p] = lh;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of partition partials: grid (Hq, B), 256 threads.
//   out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p,  M = max_p m_p
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(Params pr) {
  constexpr int NT = 256, SPLIT = NT / D;
  __shared__ float red[NT / 64];
  __shared__ float part[SPLIT][D];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int L = pr.lens[b];
  if (!len_valid(L, pr) || L == 0) return;
  const int np = (L + pr.P - 1) / pr.P;
  if (np <= 1) return;
  const int64_t row = static_cast<int64_t>(b) * pr.Hq + h;
  const float* pm = pr.part_m + row * pr.maxP;
  const float* pl = pr.part_l + row * pr.maxP;
  const float* pa = pr.part_acc + row * pr.maxP * D;

  float M = -INFINITY;
  for (int i = tid; i < np; i += NT) M = fmaxf(M, pm[i]);
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  if ((tid & 63) == 0) red[tid >> 6] = M;
  __syncthreads();
  M = red[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) M = fmaxf(M, red[w]);
  __syncthreads();

  float den = 0.f;
  for (int i = tid; i < np; i += NT) den = fmaf(exp2f(pm[i] - M), pl[i], den);
  for (int o = 32; o > 0; o >>= 1) den += __shfl_xor(den, o);
  if ((tid & 63) == 0) red[tid >> 6] = den;
  __syncthreads();
  den = 0.f;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) den += red[w];

  const int d = tid % D, s = tid / D;
  float a = 0.f;
  for (int i = s; i < np; i += SPLIT) a = fmaf(exp2f(pm[i] - M), pa[static_cast<int64_t>(i) * D + d], a);
  part[s][d] = a;
  __syncthreads();
  if (s == 0) {
    float tot = 0.f;
#pragma unroll
    for (int k = 0; k < SPLIT; ++k) tot += part[k][d];
    pr.out[row * D + d] = tot / den;
  }
}

// Kernel selection: PA_DECODE_KERNEL=generic forces the plain-FMA kernel for
// every dtype (used by tests to check both kernels); default picks the
// matrix-core kernel for fp16/bf16.
enum class Path { kAuto, kGeneric };
Path path_from_env() {
  const char* v = std::getenv("PA_DECODE_KERNEL");
  return (v && std::strcmp(v, "generic") == 0) ? Path::kGeneric : Path::kAuto;
}

constexpr int kDefaultPartition = 256;
constexpr int kPairsInFlight = 2;

bool decode_args_ok(int B, int Hq, int Hkv, int D, int max_ctx, int P, pa_dtype dt) {
  return B >= 0 && B <= 65535 && Hkv > 0 && Hkv <= 65535 && Hq > 0 && Hq % Hkv == 0 &&
         Hq / Hkv <= kMaxGroup && (D == 64 || D == 128) && max_ctx >= 0 && P >= 0 &&
         P % kBlockSize == 0 && dtype_ok(dt);
}

int resolve_partition(int P) { return P > 0 ? P : kDefaultPartition; }

int num_partitions(int max_ctx, int P) { return max_ctx <= 0 ? 1 : (max_ctx + P - 1) / P; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

size_t workspace_bytes(int B, int Hq, int D, int maxP) {
  if (maxP <= 1) return 0;
  const size_t rows = static_cast<size_t>(B) * Hq * maxP;
  return 2 * align256(rows * sizeof(float)) + align256(rows * D * sizeof(float));
}

template <typename T, int D>
void launch_partitions(const Params& pr, bool generic, hipStream_t s) {
  // matrix-core kernel: x = KV head + Hkv * partition (the heads of one
  // partition are dispatched together), z = sequence
  dim3 grid_m(pr.Hkv * pr.maxP, 1, pr.B);
  if (generic)
    decode_generic_kernel<T, D><<<dim3(pr.maxP, pr.Hkv, pr.B), 256, 0, s>>>(pr);
  else if (pr.G <= 4)
    decode_mfma_kernel<T, D, kPairsInFlight, true><<<grid_m, 64, 0, s>>>(pr);
  else
    decode_mfma_kernel<T, D, kPairsInFlight, false><<<grid_m, 64, 0, s>>>(pr);
}

template <>
void launch_partitions<F32, 64>(const Params& pr, bool, hipStream_t s) {
  decode_generic_kernel<F32, 64><<<dim3(pr.maxP, pr.Hkv, pr.B), 256, 0, s>>>(pr);
}
template <>
void launch_partitions<F32, 128>(const Params& pr, bool, hipStream_t s) {
  decode_generic_kernel<F32, 128><<<dim3(pr.maxP, pr.Hkv, pr.B), 256, 0, s>>>(pr);
}

enum class Phase { kPartitions = 1, kMerge = 2, kBoth = 3 };

template <int D>
void launch_phases(const Params& pr, pa_dtype dt, bool generic, Phase ph, hipStream_t s) {
  if (static_cast<int>(ph) & static_cast<int>(Phase::kPartitions)) {
    switch (dt) {
      case PA_F32: launch_partitions<F32, D>(pr, true, s); break;
      case PA_F16: launch_partitions<F16, D>(pr, generic, s); break;
      case PA_BF16: launch_partitions<BF16, D>(pr, generic, s); break;
    }
  }
  if ((static_cast<int>(ph) & static_cast<int>(Phase::kMerge)) && pr.maxP > 1)
    merge_kernel<D><<<dim3(pr.Hq, pr.B), 256, 0, s>>>(pr);
}

// Validates the arguments shared by pa_decode / pa_decode_partial /
// pa_decode_merge and launches the requested phases.
pa_status run_decode(const char* fn, Phase ph, float* out, const void* q, const void* k_pool,
                     const void* v_pool, const int32_t* block_tables,
                     const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                     int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                     float scale, int32_t partition_size, pa_dtype dtype, void* workspace,
                     size_t workspace_bytes_given, void* stream) {
  if (block_size != kBlockSize)
    return fail(PA_ERR_UNSUPPORTED, "%s: block_size %d (only 16 is supported)", fn, block_size);
  if (!dtype_ok(dtype)) return fail(PA_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dtype);
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
  if (partition_size < 0 || partition_size % kBlockSize != 0)
    return fail(PA_ERR_INVALID_ARG, "%s: partition_size %d not a multiple of 16", fn,
                partition_size);
  if (!(scale > 0.f) || !std::isfinite(scale))
    return fail(PA_ERR_INVALID_ARG, "%s: scale must be positive and finite", fn);
  if (num_seqs == 0) return ok();
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens)
    return fail(PA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_pool) |
       reinterpret_cast<uintptr_t>(v_pool)) & 15)
    return fail(PA_ERR_INVALID_ARG, "%s: q and pools must be 16-byte aligned", fn);

  const int P = resolve_partition(partition_size);
  const int maxP = num_partitions(max_context_len, P);
  const size_t need = workspace_bytes(num_seqs, num_q_heads, head_dim, maxP);
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
  pr.P = P;
  pr.maxP = maxP;
  pr.scale_log2 = scale * kLog2e;
  if (need > 0) {
    const size_t rows = static_cast<size_t>(num_seqs) * num_q_heads * maxP;
    char* ws = static_cast<char*>(workspace);
    pr.part_m = reinterpret_cast<float*>(ws);
    pr.part_l = reinterpret_cast<float*>(ws + align256(rows * sizeof(float)));
    pr.part_acc = reinterpret_cast<float*>(ws + 2 * align256(rows * sizeof(float)));
  }
  const bool generic = path_from_env() == Path::kGeneric;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (head_dim == 64)
    launch_phases<64>(pr, dtype, generic, ph, s);
  else
    launch_phases<128>(pr, dtype, generic, ph, s);
  return launch_status(fn);
}

}  // namespace
}  // namespace pa

using namespace pa;

extern "C" int32_t pa_decode_partition_size(int32_t num_seqs, int32_t num_q_heads,
                                            int32_t num_kv_heads, int32_t head_dim,
                                            int32_t max_context_len, int32_t partition_size,
                                            pa_dtype dtype) {
  if (!decode_args_ok(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                      partition_size, dtype))
    return 0;
  return resolve_partition(partition_size);
}

extern "C" size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                            int32_t num_kv_heads, int32_t head_dim,
                                            int32_t max_context_len, int32_t partition_size,
                                            pa_dtype dtype) {
  if (!decode_args_ok(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                      partition_size, dtype))
    return 0;
  const int P = resolve_partition(partition_size);
  return workspace_bytes(num_seqs, num_q_heads, head_dim, num_partitions(max_context_len, P));
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
  return run_decode("pa_decode", Phase::kBoth, PA_DECODE_FWD);
}

extern "C" pa_status pa_decode_partial(PA_DECODE_ARGS) {
  return run_decode("pa_decode_partial", Phase::kPartitions, PA_DECODE_FWD);
}

extern "C" pa_status pa_decode_merge(PA_DECODE_ARGS) {
  return run_decode("pa_decode_merge", Phase::kMerge, PA_DECODE_FWD);
}
