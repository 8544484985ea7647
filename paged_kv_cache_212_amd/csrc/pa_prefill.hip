// Attention of a chunk of query tokens per sequence over the paged cache
// (prefill, chunked prefill) on gfx950.
//
// Sequence b holds L = context_lens[b] tokens, the last n_b of which are the
// chunk; query row query_start[b] + i is the token at position L - n_b + i and
// attends causally to positions 0 .. its own, read through the block table
// in logical order (page 3, abeam.tech review, sections 「KV キャッシュマネージャ」
// and 「モデル構造ではなくサービング基盤の変更」; the review names the prompt
// phase as a stage of its own in 「今後注目すべき方向性」).  With n_b = 1 it is
// the decode step.
//
// One 64-lane wave per (query head h, tile of 16 query tokens, sequence);
// lane = 16*j + n; four such waves (four query heads of one KV head) share a
// workgroup and their K/V through LDS when the group size is a multiple of 4.  K/V of a block are re-read by every tile and query head of
// its KV head, so they use plain (cached) loads.  Per 16-token block of keys:
//   S^T (16 keys x 16 queries) = K . Q^T on v_mfma_f32_16x16x32: A = K (lane
//     reads key n, dims kk*32 + 8j .. +8), B = Q (query n, same dims).  Result:
//     lane (n, j) holds query n against keys 4j + e (e = 0..3).
//   That is the A operand of O (16 queries x 16 dims) += P (16 queries x 16
//     keys) . V (16 keys x 16 dims) on v_mfma_f32_16x16x16 (lane: row n,
//     k = keys 4j + e), so the probabilities need no transpose.  B = V: lane
//     (n, j) holds dim t*16 + n of keys 4j .. 4j+3, 8 contiguous bytes of the
//     V tile (8 consecutive tokens of a dim are stored together).  P is split
//     into a high and a low half-precision part (two MFMAs).
//   O: lane (n, j) holds dim t*16 + n of queries 4j + e.
// Online softmax per query in the log2 domain (max and sum across the 4 lane
// groups with two xor shuffles); the causal mask selects scores to -inf, and
// V rows at positions >= L are zeroed so unwritten slots never reach O.
// Blocks are double-buffered: the loads of block kb + 2 are issued once block
// kb has been consumed.
#include <hip/hip_runtime.h>

#include <cmath>
#include <type_traits>

#include "pa_device.h"
#include "pa_mfma.h"

namespace pa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kQTile = 16;  // query tokens per wave

struct PrefillParams {
  float* out;               // [T][Hq][D]
  const void* q;            // [T][Hq][D]
  const void* kpool;
  const void* vpool;
  const int32_t* tables;    // [B][max_blocks]
  const int32_t* lens;      // [B]
  const int32_t* qstart;    // [B + 1]
  int B, T, Hq, Hkv, G;
  int num_blocks, max_blocks, max_ctx, max_qlen;
  int ntiles;               // query tiles per sequence
  float scale_log2;
};

// WPG: waves per workgroup.  1: one query head per workgroup, K/V read by
// each wave from global memory (L2).  4 (G a multiple of 4): four query heads
// of one KV head and the same tile per workgroup; each pair of K/V blocks is
// loaded once, a quarter by each wave, into LDS and read from there by all
// four (a quarter of the L2 traffic).
template <typename T, int D, int WPG>
__global__ __launch_bounds__(64 * WPG, WPG > 1 ? 3 : 1) void prefill_kernel(PrefillParams pr) {
  constexpr int NKK = D / 32;     // 32-dim steps of Q.K^T
  constexpr int NTL = D / 16;     // 16-dim output tiles
  constexpr int64_t kTileBytes = static_cast<int64_t>(D) * kBlockSize * 2;
  constexpr int kTileU4 = static_cast<int>(kTileBytes / 16);   // 16-byte words per tile
  // Workgroup order: KV head fastest, then the group of WPG query heads, then
  // the tile, then the sequence.  Workgroups are dealt round-robin to the
  // XCDs, so with Hkv a multiple of their number every query head and tile of
  // one KV head runs on one XCD and re-reads its K/V from that XCD's L2.
  int lin = blockIdx.x;
  const int g = lin % pr.Hkv;
  lin /= pr.Hkv;
  const int e_head = (lin % (pr.G / WPG)) * WPG + (threadIdx.x >> 6);
  lin /= pr.G / WPG;
  const int tile = lin % pr.ntiles, b = lin / pr.ntiles;
  const int h = g * pr.G + e_head;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, j = lane >> 4;

  const int L = pr.lens[b];
  const int q0 = pr.qstart[b], q1 = pr.qstart[b + 1];
  const bool rows_ok = q0 >= 0 && q0 <= q1 && q1 <= pr.T;
  if (!rows_ok) return;                                   // no row can be trusted
  const int nq = q1 - q0;
  const int i0 = tile * kQTile;                           // first query of the tile
  if (i0 >= nq) return;
  float* orow = pr.out + (static_cast<int64_t>(q0) + i0) * pr.Hq * D + static_cast<int64_t>(h) * D;
  const bool seq_ok = L >= 0 && L <= pr.max_ctx && L <= pr.max_blocks * kBlockSize &&
                      nq <= L && nq <= pr.max_qlen;
  if (!seq_ok) {
    // length out of the declared bounds: NaN rows
    for (int idx = lane; idx < kQTile * D; idx += 64) {
      const int r = idx / D;
      if (i0 + r < nq) orow[static_cast<int64_t>(r) * pr.Hq * D + idx % D] = __builtin_nanf("");
    }
    return;
  }

  // Q (B operand): query n of the tile, dims kk*32 + 8j .. +8
  uint4 qr[NKK];
  {
    const bool real = i0 + n < nq;
    const uint16_t* qb = static_cast<const uint16_t*>(pr.q) +
                         ((static_cast<int64_t>(q0) + i0 + n) * pr.Hq + h) * D + j * 8;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      qr[kk] = real ? *reinterpret_cast<const uint4*>(qb + kk * 32) : make_uint4(0, 0, 0, 0);
  }
  const int first_pos = L - nq;                           // position of query 0
  const int qpos = first_pos + i0 + n;                    // this lane's query position
  const int last_pos = first_pos + min(nq, i0 + kQTile) - 1;
  const int nblk = last_pos / kBlockSize + 1;             // key blocks the tile needs

  const char* kbase = static_cast<const char*>(pr.kpool) + g * kTileBytes;
  const char* vbase = static_cast<const char*>(pr.vpool) + g * kTileBytes;
  const int64_t block_stride = static_cast<int64_t>(pr.Hkv) * kTileBytes;
  const int32_t* trow = pr.tables + static_cast<int64_t>(b) * pr.max_blocks;
  // Every table entry the tile reads is checked once, up front; an entry out
  // of the pool turns the tile's rows into NaN.  (Sequence and tile are the
  // same for every wave of a workgroup, so the early return is uniform.)
  bool bad = false;
  for (int k = lane; k - lane < nblk; k += 64) {
    const int e = k < nblk ? trow[k] : 0;
    if (__any(e < 0 || e >= pr.num_blocks)) bad = true;
  }
  if (bad) {
    for (int idx = lane; idx < kQTile * D; idx += 64) {
      const int r = idx / D;
      if (i0 + r < nq) orow[static_cast<int64_t>(r) * pr.Hq * D + idx % D] = __builtin_nanf("");
    }
    return;
  }
  // The entries are then read one at a time with scalar loads (the index is
  // the same in every lane): these wait on their own counter, so taking an
  // entry does not drain the K/V loads still in flight.
  const auto* trow_s = (const __attribute__((address_space(4))) int32_t*)trow;
  auto phys_of = [&](int k) -> int { return trow_s[k]; };

  // Keys are taken 32 at a time, a pair of blocks (2pp, 2pp + 1).  Lane (n,
  // j) scores query n against keys 4j .. 4j+3 of each block of the pair; as
  // the A operand of the 16x16x32 P.V its k index 8j + e stands for key
  // 4j + e of the first block (e < 4) or of the second (e >= 4), and its V
  // operand is those keys' two 8-byte runs side by side.  A pair past the
  // tile's last block re-reads that block (its keys are masked).
  const int npair = (nblk + 1) / 2;
  uint4 kreg[2][NKK];      // K of the pair's two blocks
  uint2 vreg[2][NTL];      // V of the pair's two blocks
  int ph[2];
  // LDS staging (WPG > 1): kBufs buffers of a pair's [K0 | K1 | V0 | V1] tiles.
  // Word c of a buffer (16 bytes) is moved by thread c % (64 * WPG) straight
  // from global memory into LDS (global_load_lds: lane i of a wave writes the
  // wave's LDS base + 16 i), so no registers hold the staged data.
  constexpr int kStage = WPG > 1 ? 4 * kTileU4 / (64 * WPG) : 1;   // loads per thread per pair
  constexpr int kBufs = 3;      // pairs in LDS: the one computed and two in flight
  // three separate arrays, so the compiler can tell a buffer being filled
  // from the one being read and need not wait for the fill before the reads
  __shared__ uint4 lds0[4][WPG > 1 ? kTileU4 : 1];
  __shared__ uint4 lds1[4][WPG > 1 ? kTileU4 : 1];
  __shared__ uint4 lds2[4][WPG > 1 ? kTileU4 : 1];
  auto buf_of = [&](auto bc) -> uint4(*)[WPG > 1 ? kTileU4 : 1] {
    constexpr int bi = decltype(bc)::value;
    if constexpr (bi == 0) return lds0;
    else if constexpr (bi == 1) return lds1;
    else return lds2;
  };
  auto gload_lds = [&](int pp, auto bc) {
    const int p0 = phys_of(min(2 * pp, nblk - 1)), p1 = phys_of(min(2 * pp + 1, nblk - 1));
#pragma unroll
    for (int r = 0; r < kStage; ++r) {
      const int c = static_cast<int>(threadIdx.x) + r * 64 * WPG;
      const int part = c / kTileU4, idx = c % kTileU4;
      const char* src = (part < 2 ? kbase : vbase) + ((part & 1) ? p1 : p0) * block_stride +
                        idx * 16;
      uint4* dst = &buf_of(bc)[0][0] + (c - lane);      // the wave's first word
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                       (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
    }
  };
  auto lread_k = [&](auto bc) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) kreg[u][kk] = buf_of(bc)[u][(j * 16 + n) + kk * 64];
  };
  auto lread_v = [&](auto bc) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint2* vt = reinterpret_cast<const uint2*>(buf_of(bc)[2 + u]) +
                        (((j >> 1) * D + n) * 16 + (j & 1) * 8) / 8;
#pragma unroll
      for (int t = 0; t < NTL; ++t) vreg[u][t] = vt[t * 16 * 16 / 8];
    }
  };
  auto issue_k = [&](int pp) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      ph[u] = phys_of(min(2 * pp + u, nblk - 1));
      const char* kt = kbase + ph[u] * block_stride + ((j * 16) + n) * 16;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
        kreg[u][kk] = *reinterpret_cast<const uint4*>(kt + kk * 64 * 16);
    }
  };
  auto issue_v = [&]() {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const char* vt = vbase + ph[u] * block_stride + ((j >> 1) * D + n) * 16 + (j & 1) * 8;
#pragma unroll
      for (int t = 0; t < NTL; ++t)
        vreg[u][t] = *reinterpret_cast<const uint2*>(vt + t * 16 * 16);
    }
  };

  float m_run = -INFINITY, l_lane = 0.f;
  f32x4_t acc[NTL];
#pragma unroll
  for (int t = 0; t < NTL; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto qk_softmax = [&](int pp, uint4& phi, uint4& plo) {
    f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      s0 = Mfma<T>::qk(kreg[0][kk], qr[kk], s0);
      s1 = Mfma<T>::qk(kreg[1][kk], qr[kk], s1);
    }
    const int kpos0 = 2 * pp * kBlockSize + 4 * j;        // key position of s0[0]
    float sv[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sv[e] = (kpos0 + e <= qpos) ? s0[e] * pr.scale_log2 : -INFINITY;
      sv[4 + e] = (kpos0 + kBlockSize + e <= qpos) ? s1[e] * pr.scale_log2 : -INFINITY;
    }
    float bm = sv[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) bm = fmaxf(bm, sv[e]);
    bm = fmaxf(bm, __shfl_xor(bm, 16));
    bm = fmaxf(bm, __shfl_xor(bm, 32));
    const float mn = fmaxf(m_run, bm);
    if (__any(mn != m_run)) {
      // a query's running max moved: rescale its O row by 2^(m_old - m_new)
      const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
      l_lane *= alpha;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float ar = __shfl(alpha, 4 * j + e);        // alpha of O row 4j + e
#pragma unroll
        for (int t = 0; t < NTL; ++t) acc[t][e] *= ar;
      }
      m_run = mn;
    }
    float pe[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pe[e] = __builtin_amdgcn_exp2f(sv[e] - m_run);
    l_lane += ((pe[0] + pe[1]) + (pe[2] + pe[3])) + ((pe[4] + pe[5]) + (pe[6] + pe[7]));
    Mfma<T>::split8(pe, phi, plo);
  };

  auto pv = [&](int pp, uint4 phi, uint4 plo) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int kb = 2 * pp + u;
      if ((kb + 1) * kBlockSize > L) {
        // the block reaches past the sequence: zero V of unwritten positions
        const int kp = kb * kBlockSize + 4 * j;
        const uint32_t mx = (kp + 0 < L ? 0x0000FFFFu : 0u) | (kp + 1 < L ? 0xFFFF0000u : 0u);
        const uint32_t my = (kp + 2 < L ? 0x0000FFFFu : 0u) | (kp + 3 < L ? 0xFFFF0000u : 0u);
#pragma unroll
        for (int t = 0; t < NTL; ++t) {
          vreg[u][t].x &= mx;
          vreg[u][t].y &= my;
        }
      }
    }
#pragma unroll
    for (int t = 0; t < NTL; ++t) {
      const uint4 v = make_uint4(vreg[0][t].x, vreg[0][t].y, vreg[1][t].x, vreg[1][t].y);
      acc[t] = Mfma<T>::pv8(phi, v, acc[t]);
      acc[t] = Mfma<T>::pv8(plo, v, acc[t]);
    }
  };

  if constexpr (WPG == 1) {
    // K of the next pair is issued once QK has consumed the current one, V of
    // the next pair once P.V has (scheduling barriers keep the compiler from
    // hoisting the loads above the matrix ops that still read the registers)
    issue_k(0);
    issue_v();
    for (int pp = 0; pp < npair; ++pp) {
      uint4 phi, plo;
      qk_softmax(pp, phi, plo);
      __builtin_amdgcn_sched_barrier(0);
      if (pp + 1 < npair) issue_k(pp + 1);
      __builtin_amdgcn_sched_barrier(0);
      pv(pp, phi, plo);
      __builtin_amdgcn_sched_barrier(0);
      if (pp + 1 < npair) issue_v();
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    // pairs pp + 1 and pp + 2 travel global -> LDS while pair pp is computed
    // from LDS; one barrier per pair orders both a buffer's writes before its
    // reads and its reads before the rewrite three pairs later (every wave of
    // the workgroup runs the same npair).  The only vector-memory operations
    // in the loop are these loads, so "at most kStage outstanding" means the
    // next pair's have landed.
    // s_waitcnt immediates: vmcnt in bits 3:0 and 15:14, expcnt left at its
    // no-wait maximum 7, lgkmcnt 0 so that this wave's LDS reads of the pair
    // have returned before the barrier lets a refill of that buffer start
    constexpr int kWaitNext = (kStage & 0xF) | (7 << 4) | ((kStage >> 4) << 14);
    constexpr int kWaitAll = 7 << 4;
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    using B2 = std::integral_constant<int, 2>;
    gload_lds(0, B0{});
    if (npair > 1) {
      gload_lds(1, B1{});
      __builtin_amdgcn_s_waitcnt(kWaitNext);
    } else {
      __builtin_amdgcn_s_waitcnt(kWaitAll);
    }
    __syncthreads();
    // pair pp in buffer pp % 3; the loop is unrolled by three so that every
    // buffer index is a constant
    auto step = [&](int pp, auto cur, auto fill) {
      // the buffer filled here was last read in pair pp - 1, before the barrier
      if (pp + 2 < npair) gload_lds(pp + 2, fill);
      lread_k(cur);
      uint4 phi, plo;
      qk_softmax(pp, phi, plo);
      lread_v(cur);
      pv(pp, phi, plo);
      if (pp + 2 < npair)
        __builtin_amdgcn_s_waitcnt(kWaitNext);    // this wave's pair pp + 1 has landed
      else
        __builtin_amdgcn_s_waitcnt(kWaitAll);
      // ... and every wave's.  A bare barrier: the fence of __syncthreads
      // would also drain the loads of pair pp + 2.  The clobber keeps the
      // compiler from moving LDS reads across it.
      asm volatile("s_barrier" ::: "memory");
    };
    for (int pp = 0; pp < npair; pp += 3) {
      step(pp, B0{}, B2{});
      if (pp + 1 < npair) step(pp + 1, B1{}, B0{});
      if (pp + 2 < npair) step(pp + 2, B2{}, B1{});
    }
  }

  // l of query n, then of O row 4j + e
  float l = l_lane;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int r = 4 * j + e;
    const float lr = __shfl(l, r);
    if (i0 + r < nq) {
      const float inv = 1.0f / lr;
#pragma unroll
      for (int t = 0; t < NTL; ++t)
        orow[static_cast<int64_t>(r) * pr.Hq * D + t * 16 + n] = acc[t][e] * inv;
    }
  }
}

}  // namespace
}  // namespace pa

using namespace pa;

extern "C" pa_status pa_prefill(float* out, const void* q, const void* k_pool,
                                const void* v_pool, const int32_t* block_tables,
                                const int32_t* context_lens, const int32_t* query_start,
                                int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                int32_t num_blocks, int32_t max_blocks_per_seq,
                                int32_t max_context_len, int32_t max_query_len, float scale,
                                pa_dtype dtype, void* stream) {
  const char* fn = "pa_prefill";
  if (block_size != kBlockSize)
    return fail(PA_ERR_UNSUPPORTED, "%s: block_size %d (only 16 is supported)", fn, block_size);
  if (!dtype_ok(dtype)) return fail(PA_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dtype);
  if (dtype == PA_F32)
    return fail(PA_ERR_UNSUPPORTED, "%s: fp32 KV (matrix-core path: fp16/bf16 only)", fn);
  if (head_dim != 64 && head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "%s: head_dim %d (64 or 128 supported)", fn, head_dim);
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 ||
      num_q_heads > 65535)
    return fail(PA_ERR_INVALID_ARG, "%s: num_q_heads %d / num_kv_heads %d", fn, num_q_heads,
                num_kv_heads);
  if (num_seqs < 0 || num_seqs > 65535 || num_tokens < 0 || num_blocks <= 0 ||
      max_blocks_per_seq < 0 || max_context_len < 0 || max_query_len < 0 ||
      max_query_len > 65535 * kQTile)
    return fail(PA_ERR_INVALID_ARG, "%s: size out of range", fn);
  if (!(scale > 0.f) || !std::isfinite(scale))
    return fail(PA_ERR_INVALID_ARG, "%s: scale must be positive and finite", fn);
  if (num_seqs == 0 || num_tokens == 0 || max_query_len == 0) return ok();
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens || !query_start)
    return fail(PA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_pool) |
       reinterpret_cast<uintptr_t>(v_pool)) & 15)
    return fail(PA_ERR_INVALID_ARG, "%s: q and pools must be 16-byte aligned", fn);
  PrefillParams pr{};
  pr.out = out;
  pr.q = q;
  pr.kpool = k_pool;
  pr.vpool = v_pool;
  pr.tables = block_tables;
  pr.lens = context_lens;
  pr.qstart = query_start;
  pr.B = num_seqs;
  pr.T = num_tokens;
  pr.Hq = num_q_heads;
  pr.Hkv = num_kv_heads;
  pr.G = num_q_heads / num_kv_heads;
  pr.num_blocks = num_blocks;
  pr.max_blocks = max_blocks_per_seq;
  pr.max_ctx = max_context_len;
  pr.max_qlen = max_query_len;
  pr.scale_log2 = scale * kLog2e;
  pr.ntiles = (max_query_len + kQTile - 1) / kQTile;
  // four query heads per workgroup when the group size allows it
  const int wpg = pr.G % 4 == 0 ? 4 : 1;
  const uint64_t nwg = static_cast<uint64_t>(num_q_heads / wpg) * pr.ntiles * num_seqs;
  if (nwg > 0x7fffffffull)
    return fail(PA_ERR_INVALID_ARG, "%s: %llu workgroups exceed the launch limit", fn,
                static_cast<unsigned long long>(nwg));
  const dim3 grid(static_cast<uint32_t>(nwg));
  hipStream_t s = static_cast<hipStream_t>(stream);
#define PA_PREFILL(TAG, DIM)                                               \
  (wpg == 4 ? (prefill_kernel<TAG, DIM, 4><<<grid, 256, 0, s>>>(pr), 0)    \
            : (prefill_kernel<TAG, DIM, 1><<<grid, 64, 0, s>>>(pr), 0))
  if (dtype == PA_BF16)
    head_dim == 64 ? PA_PREFILL(BF16, 64) : PA_PREFILL(BF16, 128);
  else
    head_dim == 64 ? PA_PREFILL(F16, 64) : PA_PREFILL(F16, 128);
#undef PA_PREFILL
  return launch_status(fn);
}
