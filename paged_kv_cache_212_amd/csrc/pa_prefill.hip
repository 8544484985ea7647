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
// One 64-lane wave per (query head h, tiles of 16 query tokens, sequence);
// lane = 16*j + n.  When the group size is a multiple of 4, four such waves
// (four query heads of one KV head) share a workgroup and their K/V through
// LDS, and each wave takes two consecutive tiles; otherwise one wave, one
// tile.  K/V of a block are re-read by every tile and query head of its KV
// head, so they use plain (cached) loads.  Keys go in pairs of 16-token blocks
// (32 keys); per pair and tile:
//   S^T (16 keys x 16 queries) = K . Q^T on v_mfma_f32_16x16x32, one chain
//     per block: A = K (lane reads key n, dims kk*32 + 8j .. +8), B = Q (query
//     n, same dims).  Result: lane (n, j) holds query n against keys 4j + e
//     (e = 0..3) of the block.
//   That is the A operand of O (16 queries x 16 dims) += P (16 queries x 32
//     keys) . V (32 keys x 16 dims) on v_mfma_f32_16x16x32 (lane: row n; k
//     index 8j + e is key 4j + e of the first block for e < 4, of the second
//     for e >= 4), so the probabilities need no transpose.  B = V: lane (n, j)
//     holds dim t*16 + n of keys 4j .. 4j+3 of both blocks, 8 contiguous bytes
//     of each V tile (8 consecutive tokens of a dim are stored together).  P is
//     split into a high and a low half-precision part (two MFMAs).
//   O: lane (n, j) holds dim t*16 + n of queries 4j + e.
// Online softmax per query in the log2 domain (max across the 4 lane groups
// with lane swaps, lazy rescaling); the causal mask selects scores to -inf,
// and V rows at positions >= L are zeroed so unwritten slots never reach O.
// With four query heads per workgroup the pairs travel global -> LDS two
// pairs ahead (four LDS buffers, one barrier per two pairs); a one-wave
// workgroup double-buffers them in registers.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <type_traits>

#include "pa_device.h"
#include "pa_mfma.h"

namespace pa {

// The arguments of both prefill kernels (also handed to the ping-pong
// kernel's launcher, which lives in pa_prefill_pp.hip).
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
  // Shared-prefix mode (decode over prefixes shared by several sequences):
  // "sequence" b is piece b % pieces of group b / pieces, whose query rows
  // qstart[g] .. qstart[g+1]-1 are batch sequences rows[r].  The group's
  // prefix is the first prefix_len[rows[qstart[g]]] positions of that
  // member's table; piece p takes its key blocks from p * nb / pieces to
  // (p + 1) * nb / pieces (rounded down to even; nb blocks in all), with no
  // causal mask (every row sees the whole piece).  Each row's partial goes
  // to slot p at the member's batch row: the unnormalised weighted sum of V
  // to pre_out, the log2-domain (max, sum of 2^(s - max)) to pre_ml, and the
  // call's epoch to pre_stamp (per row; the merge clears it once read).  A
  // row whose member is out of the batch, or whose prefix length or prefix
  // blocks differ from the group's, is not written (nor is any row of a
  // group whose length or table is unusable).
  const int32_t* rows;      // [T] batch index of each row
  const int32_t* prefix_len;  // [num_seqs] prefix tokens per batch sequence
  float* pre_out;           // [pieces][num_seqs][Hq][D]
  float2* pre_ml;           // [pieces][num_seqs][Hq]
  uint32_t* pre_stamp;      // [pieces][num_seqs][Hq]
  uint32_t epoch;
  int num_seqs;
  int pieces;
};

// Launches prefill_pp_kernel<T, D> (defined below; instantiated in
// pa_prefill_pp.hip, which the build compiles with its own scheduling
// strategy).
template <typename T, int D>
void launch_prefill_pp(dim3 grid, hipStream_t s, const PrefillParams& pr);

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kQTile = 16;     // query tokens per tile
constexpr int kPairTiles = 2;  // tiles per wave with four query heads per workgroup
constexpr float kRescaleSlack = 8.f;  // log2-domain headroom before the running max moves

// LDS slot of V chunk c: the low three bits XORed with bits 4..6 (an
// involution that permutes each group of 16 chunks).
__device__ __forceinline__ int vswz(int c) { return c ^ ((c >> 4) & 7); }

// max(v of lane l, v of lane l ^ 16) and of lane l ^ 32.  v_permlane16_swap /
// v_permlane32_swap of a register with itself give every lane both values of
// its pair (lanes with bit 4, resp. bit 5, clear then set): a VALU exchange,
// no LDS round trip.
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// WPG: waves per workgroup.  1: one query head per workgroup, K/V read by
// each wave from global memory (L2).  4 (G a multiple of 4): four query heads
// of one KV head and the same tiles per workgroup; each pair of K/V blocks is
// loaded once, a quarter by each wave, into LDS and read from there by all
// four (a quarter of the L2 traffic).
// TQ: consecutive 16-query tiles per wave.  The K/V operands read for a pair
// of blocks serve all TQ tiles (TQ times the matrix work per LDS read), and
// the tiles' softmax and matrix chains are independent, so one hides the
// other's latency.
template <typename T, int D, int WPG, int TQ, bool kShared = false>
__global__ __launch_bounds__(64 * WPG, WPG > 1 ? (TQ > 1 ? 2 : 3) : 1) void prefill_kernel(
    PrefillParams pr) {
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
  const int ngroups = (pr.ntiles + TQ - 1) / TQ;           // groups of TQ tiles
  const int tgroup = lin % ngroups, b = lin / ngroups;
  // shared mode: piece and group
  const int piece = kShared ? b % pr.pieces : 0;
  const int grp = kShared ? b / pr.pieces : b;
  const int h = g * pr.G + e_head;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, j = lane >> 4;

  const int q0 = pr.qstart[grp], q1 = pr.qstart[grp + 1];
  const bool rows_ok = q0 >= 0 && q0 <= q1 && q1 <= pr.T;
  if (!rows_ok) return;                                   // no row can be trusted
  const int nq = q1 - q0;
  const int i0 = tgroup * TQ * kQTile;                    // first query of the wave
  if (i0 >= nq) return;
  // batch row of query i of the sequence (shared mode: the member), and the
  // table row the keys come from
  auto in_batch = [&](int64_t r) { return r >= 0 && r < pr.num_seqs; };
  const int64_t tb = kShared ? pr.rows[q0] : b;
  if (kShared && !in_batch(tb)) return;
  const int L = kShared ? pr.prefix_len[tb] : pr.lens[b];
  float* orow = pr.out + (static_cast<int64_t>(q0) + i0) * pr.Hq * D + static_cast<int64_t>(h) * D;
  const bool seq_ok = L >= 0 && L <= pr.max_ctx && L <= pr.max_blocks * kBlockSize &&
                      (kShared ? L >= kBlockSize && L % kBlockSize == 0 : nq <= L) &&
                      nq <= pr.max_qlen;
  // shared mode: an unusable group writes nothing (its rows' stamps stay old)
  if (kShared && !seq_ok) return;
  // Keys of the wave: positions [kb0 * 16, kb0 * 16 + Lk) (Lk = L but for a
  // piece of a shared prefix, which is attended like a sequence of Lk
  // positions with every query after them; a piece may be empty).
  int kb0 = 0, Lk = L;
  if constexpr (kShared) {
    const int nbp = L / kBlockSize;
    kb0 = (piece * nbp / pr.pieces) & ~1;
    const int kb1 = piece + 1 == pr.pieces ? nbp : ((piece + 1) * nbp / pr.pieces) & ~1;
    Lk = (kb1 - kb0) * kBlockSize;
  }
  if (!seq_ok) {
    // length out of the declared bounds: NaN rows
    for (int idx = lane; idx < TQ * kQTile * D; idx += 64) {
      const int r = idx / D;
      if (i0 + r < nq) orow[static_cast<int64_t>(r) * pr.Hq * D + idx % D] = __builtin_nanf("");
    }
    return;
  }

  // Shared mode: the member of query 16t + n of the wave (mrow; -1 past the
  // group or out of the batch) and whether its prefix is the group's: the
  // same length and the same blocks (lanes j, j + 4, ... compare entries;
  // the four lanes of a query OR their findings).
  int mrow[TQ];
  bool row_ok[TQ];
#pragma unroll
  for (int t = 0; t < TQ; ++t) {
    mrow[t] = -1;
    row_ok[t] = true;
    if constexpr (kShared) {
      const int i = i0 + kQTile * t + n;
      const int r = i < nq ? pr.rows[q0 + i] : -1;
      mrow[t] = in_batch(r) ? r : -1;
      bool diff = mrow[t] < 0 || pr.prefix_len[max(mrow[t], 0)] != L;
      if (!diff) {
        const int32_t* mt = pr.tables + static_cast<int64_t>(mrow[t]) * pr.max_blocks;
        const int32_t* gt = pr.tables + tb * pr.max_blocks;
        for (int p = j; p < L / kBlockSize; p += 4) diff |= mt[p] != gt[p];
      }
      int dv = diff;
      dv |= __shfl_xor(dv, 16);
      dv |= __shfl_xor(dv, 32);
      row_ok[t] = dv == 0;
    }
  }

  // Q (B operand) of tile t: query 16t + n of the wave, dims kk*32 + 8j .. +8
  // (queries past the chunk read as zero; their rows are not written)
  uint4 qr[TQ][NKK];
#pragma unroll
  for (int t = 0; t < TQ; ++t) {
    const bool real = i0 + kQTile * t + n < nq;
    const int64_t qrow = kShared ? max(mrow[t], 0) : static_cast<int64_t>(q0) + i0 + kQTile * t + n;
    const uint16_t* qb = static_cast<const uint16_t*>(pr.q) + ((real ? qrow : 0) * pr.Hq + h) * D +
                         j * 8;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      qr[t][kk] = real ? *reinterpret_cast<const uint4*>(qb + kk * 32) : make_uint4(0, 0, 0, 0);
  }
  // position of query 0; shared mode: every query sits after the piece
  const int first_pos = kShared ? Lk - 1 : L - nq;
  int qpos[TQ];                                           // this lane's query positions
#pragma unroll
  for (int t = 0; t < TQ; ++t) qpos[t] = kShared ? Lk - 1 : first_pos + i0 + kQTile * t + n;
  const int last_pos = kShared ? Lk - 1 : first_pos + min(nq, i0 + TQ * kQTile) - 1;
  const int nblk = Lk > 0 ? last_pos / kBlockSize + 1 : 0;   // key blocks the wave needs

  const char* kbase = static_cast<const char*>(pr.kpool) + g * kTileBytes;
  const char* vbase = static_cast<const char*>(pr.vpool) + g * kTileBytes;
  const int64_t block_stride = static_cast<int64_t>(pr.Hkv) * kTileBytes;
  const int32_t* trow = pr.tables + tb * pr.max_blocks + kb0;
  // Every table entry the tile reads is checked once, up front; an entry out
  // of the pool turns the tile's rows into NaN.  (Sequence and tile are the
  // same for every wave of a workgroup, so the early return is uniform.)
  bool bad = false;
  for (int k = lane; k - lane < nblk; k += 64) {
    const int e = k < nblk ? trow[k] : 0;
    if (__any(e < 0 || e >= pr.num_blocks)) bad = true;
  }
  if (bad) {
    if (kShared) return;                                  // rows not written
    for (int idx = lane; idx < TQ * kQTile * D; idx += 64) {
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
  // kBufs pairs in LDS: the two computed and the two in flight.  Separate
  // arrays, so the compiler can tell a buffer being filled from the one being
  // read and need not wait for the fill before the reads.
  constexpr int kBufs = 4;
  __shared__ uint4 lds0[4][WPG > 1 ? kTileU4 : 1];
  __shared__ uint4 lds1[4][WPG > 1 ? kTileU4 : 1];
  __shared__ uint4 lds2[4][WPG > 1 ? kTileU4 : 1];
  __shared__ uint4 lds3[4][WPG > 1 ? kTileU4 : 1];
  auto buf_of = [&](auto bc) -> uint4(*)[WPG > 1 ? kTileU4 : 1] {
    constexpr int bi = decltype(bc)::value;
    if constexpr (bi == 0) return lds0;
    else if constexpr (bi == 1) return lds1;
    else if constexpr (bi == 2) return lds2;
    else return lds3;
  };
  // The 64 words a wave moves per load lie in one tile (kTileU4 is a
  // multiple of 64), so the tile's global base and the LDS destination are
  // the same for the whole wave (scalar registers); only the 32-bit offset
  // inside the tile is per lane.
  const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  auto gload_lds = [&](int pp, auto bc) {
    const int p0 = phys_of(min(2 * pp, nblk - 1)), p1 = phys_of(min(2 * pp + 1, nblk - 1));
#pragma unroll
    for (int r = 0; r < kStage; ++r) {
      const int c0 = wv * 64 + r * 64 * WPG;            // the wave's first word
      const int part = c0 / kTileU4, idx = c0 % kTileU4 + lane;
      // V tiles: LDS slot idx holds chunk vswz(idx) (see lread_v)
      const int sidx = part < 2 ? idx : vswz(idx);
      const char* base = (part < 2 ? kbase : vbase) +
                         static_cast<int64_t>((part & 1) ? p1 : p0) * block_stride;
      const char* src = base + static_cast<uint32_t>(sidx * 16);
      uint4* dst = &buf_of(bc)[0][0] + c0;
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
  // V chunk c (16 bytes: 8 tokens of one dim) sits in LDS slot vswz(c).  A
  // lane reads dim n of the 8 tiles t (chunks 16t + n, 256 bytes apart: one
  // bank); swizzled, tile t's chunk moves by (n ^ t) - n slots, so the 8 reads
  // of a lane fall in 8 different banks, while one read of a tile still covers
  // 16 distinct slots.
  auto lread_v = [&](auto bc) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint2* vt = reinterpret_cast<const uint2*>(buf_of(bc)[2 + u]);
#pragma unroll
      for (int t = 0; t < NTL; ++t)
        vreg[u][t] = vt[vswz((j >> 1) * D + t * 16 + n) * 2 + (j & 1)];
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

  float m_run[TQ], l_lane[TQ];
  float thr[TQ];   // raw score above which the row's max moves m_run
  f32x4_t acc[TQ][NTL];
#pragma unroll
  for (int t = 0; t < TQ; ++t) {
    m_run[t] = -INFINITY;
    thr[t] = -INFINITY;
    l_lane[t] = 0.f;
#pragma unroll
    for (int d = 0; d < NTL; ++d) acc[t][d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // Scores of the TQ tiles against the pair's 32 keys: 2 * TQ independent
  // chains of matrix ops issued together.  The causal mask is applied only
  // to pairs that reach past the first tile's first query position (earlier
  // pairs hold no later key for any tile; the mask itself is exact per key
  // and query, so applying it to every tile of such a pair is correct).
  auto qk_scores = [&](int pp, float (&sv)[TQ][8]) {
    f32x4_t s0[TQ], s1[TQ];
#pragma unroll
    for (int t = 0; t < TQ; ++t) s0[t] = s1[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
      for (int t = 0; t < TQ; ++t) {
        s0[t] = Mfma<T>::qk(kreg[0][kk], qr[t][kk], s0[t]);
        s1[t] = Mfma<T>::qk(kreg[1][kk], qr[t][kk], s1[t]);
      }
    }
#pragma unroll
    for (int t = 0; t < TQ; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sv[t][e] = s0[t][e];
        sv[t][4 + e] = s1[t][e];
      }
    // the first tile's first query position: first_pos + i0 (uniform); in
    // shared mode every query is at Lk - 1, so only keys past the piece (a
    // re-read last block) are masked
    if ((2 * pp + 2) * kBlockSize - 1 > (kShared ? Lk - 1 : first_pos + i0)) {
      const int kpos0 = 2 * pp * kBlockSize + 4 * j;      // key position of s0[0]
#pragma unroll
      for (int t = 0; t < TQ; ++t) {
        // key kpos0 + k is visible to the lane's query iff k <= dq (compares
        // with constants, all inside this branch)
        const int dq = qpos[t] - kpos0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sv[t][e] = e <= dq ? sv[t][e] : -INFINITY;
          sv[t][4 + e] = kBlockSize + e <= dq ? sv[t][4 + e] : -INFINITY;
        }
      }
    }
  };
  // Online softmax update of the TQ tiles from their scores, and P split into
  // the two half-precision parts of P.V's A operand.  The running max is kept
  // in the log2 domain (scale * log2(e) applied) and each weight is
  // exp2(s * scale - m) with one fused multiply-add.
  // Lazy rescaling: m_run is only a reference (numerator and denominator
  // share it), so it moves only when some row's max exceeds it by more than
  // kRescaleSlack; weights then stay below 2^kRescaleSlack, far inside fp32
  // and with the same relative precision in the hi/lo split.  Whether a row
  // passes that bound is a compare of each raw score with the row's
  // threshold (m_run + slack) / scale (the scale is positive), kept beside
  // m_run; the tiles share one test, and the row max itself (a reduction
  // across lanes) is taken only when some row passes.  A tile whose queries
  // all precede the pair keeps m = -inf rows only while no key was valid; the
  // first pair holds key 0, valid for every query, so m_run is finite from
  // there on.
  auto rescale_test = [&](float (&sv)[TQ][8]) {
    bool over = false;   // (bitwise: no short-circuit branches)
#pragma unroll
    for (int t = 0; t < TQ; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e) over |= sv[t][e] > thr[t];
    if (__any(over)) {
#pragma unroll
      for (int t = 0; t < TQ; ++t) {
        float bm = sv[t][0];
#pragma unroll
        for (int e = 1; e < 8; ++e) bm = fmaxf(bm, sv[t][e]);
        bm = max_xor16(bm);
        bm = max_xor32(bm);
        const float mn = fmaxf(m_run[t], bm * pr.scale_log2);
        // a query's running max moved: rescale its O row by 2^(m_old - m_new)
        const float alpha = __builtin_amdgcn_exp2f(m_run[t] - mn);
        l_lane[t] *= alpha;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float ar = __shfl(alpha, 4 * j + e);        // alpha of O row 4j + e
#pragma unroll
          for (int d = 0; d < NTL; ++d) acc[t][d][e] *= ar;
        }
        m_run[t] = mn;
        thr[t] = (mn + kRescaleSlack) / pr.scale_log2;
      }
    }
  };
  // Weights 2k, 2k + 1 of tile t: their sum, and their parts in word k of
  // the P.V operands.
  auto weight_pair = [&](int t, int k, const float (&sv)[TQ][8], uint32_t& hi, uint32_t& lo) {
    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[t][2 * k], pr.scale_log2, -m_run[t]));
    const float p1 =
        __builtin_amdgcn_exp2f(__builtin_fmaf(sv[t][2 * k + 1], pr.scale_log2, -m_run[t]));
    Mfma<T>::split2(p0, p1, hi, lo);
    return p0 + p1;
  };
  auto weights = [&](int t, const float (&sv)[TQ][8], uint4& phi, uint4& plo) {
    const float s0 = weight_pair(t, 0, sv, phi.x, plo.x);
    const float s1 = weight_pair(t, 1, sv, phi.y, plo.y);
    const float s2 = weight_pair(t, 2, sv, phi.z, plo.z);
    const float s3 = weight_pair(t, 3, sv, phi.w, plo.w);
    l_lane[t] += (s0 + s1) + (s2 + s3);
  };
  auto softmax = [&](float (&sv)[TQ][8], uint4 (&phi)[TQ], uint4 (&plo)[TQ]) {
    rescale_test(sv);
#pragma unroll
    for (int t = 0; t < TQ; ++t) weights(t, sv, phi[t], plo[t]);
  };

  // V rows at positions >= L are zeroed, so unwritten slots never reach O
  auto mask_v = [&](int pp) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int kb = 2 * pp + u;
      if ((kb + 1) * kBlockSize > Lk) {
        // the block reaches past the sequence: zero V of unwritten positions
        const int nv = Lk - (kb * kBlockSize + 4 * j);     // the lane's keys k < nv are written
        const uint32_t mx = (0 < nv ? 0x0000FFFFu : 0u) | (1 < nv ? 0xFFFF0000u : 0u);
        const uint32_t my = (2 < nv ? 0x0000FFFFu : 0u) | (3 < nv ? 0xFFFF0000u : 0u);
#pragma unroll
        for (int d = 0; d < NTL; ++d) {
          vreg[u][d].x &= mx;
          vreg[u][d].y &= my;
        }
      }
    }
  };
  auto pv_tile = [&](int t, int d, uint4 phi, uint4 plo) {
    const uint4 v = make_uint4(vreg[0][d].x, vreg[0][d].y, vreg[1][d].x, vreg[1][d].y);
    acc[t][d] = Mfma<T>::pv8(phi, v, acc[t][d]);
    acc[t][d] = Mfma<T>::pv8(plo, v, acc[t][d]);
  };
  auto pv = [&](int t, uint4 phi, uint4 plo) {
#pragma unroll
    for (int d = 0; d < NTL; ++d) pv_tile(t, d, phi, plo);
  };
  // P.V of tile t - 1 with the weights of tile t (independent work for the
  // matrix and the vector units): per weight pair k of tile t, the P.V of
  // output tiles NTL/4 * k ..; scheduling barriers keep each group together.
  auto pv_with_weights = [&](int t, const float (&sv)[TQ][8], uint4 (&phi)[TQ],
                             uint4 (&plo)[TQ]) {
    constexpr int kPer = NTL / 4;
    float s[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int d = kPer * k; d < kPer * (k + 1); ++d) pv_tile(t - 1, d, phi[t - 1], plo[t - 1]);
      uint32_t h, l;
      s[k] = weight_pair(t, k, sv, h, l);
      (k == 0 ? phi[t].x : k == 1 ? phi[t].y : k == 2 ? phi[t].z : phi[t].w) = h;
      (k == 0 ? plo[t].x : k == 1 ? plo[t].y : k == 2 ? plo[t].z : plo[t].w) = l;
    }
    __builtin_amdgcn_sched_barrier(0);
    l_lane[t] += (s[0] + s[1]) + (s[2] + s[3]);
  };

  if constexpr (WPG == 1) {
    static_assert(TQ == 1, "one-wave workgroups take one tile");
    // K of the next pair is issued once QK has consumed the current one, V of
    // the next pair once P.V has (scheduling barriers keep the compiler from
    // hoisting the loads above the matrix ops that still read the registers)
    if (npair > 0) {
      issue_k(0);
      issue_v();
    }
    for (int pp = 0; pp < npair; ++pp) {
      uint4 phi[1], plo[1];
      float sv[1][8];
      qk_scores(pp, sv);
      softmax(sv, phi, plo);
      __builtin_amdgcn_sched_barrier(0);
      if (pp + 1 < npair) issue_k(pp + 1);
      __builtin_amdgcn_sched_barrier(0);
      mask_v(pp);
      pv(0, phi[0], plo[0]);
      __builtin_amdgcn_sched_barrier(0);
      if (pp + 1 < npair) issue_v();
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    // Pairs are taken two at a time: while pairs pp and pp + 1 are computed
    // from LDS, pairs pp + 2 and pp + 3 travel global -> LDS into the two
    // buffers read in the previous double step.  One wait and one barrier
    // per double step order both the buffers' writes before their reads and
    // their reads before the rewrite (every wave of the workgroup runs the
    // same npair).  The only vector-memory operations in the loop are these
    // loads.
    // s_waitcnt immediate: vmcnt 0, expcnt left at its no-wait maximum 7,
    // lgkmcnt 0 so that this wave's LDS reads have returned before the
    // barrier lets a refill of those buffers start
    constexpr int kWaitAll = 7 << 4;
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    using B2 = std::integral_constant<int, 2>;
    using B3 = std::integral_constant<int, 3>;
    static_assert(kBufs == 4, "the pair loop below is written for four buffers");
    auto compute = [&](int pp, auto cur) {
      lread_k(cur);
      uint4 phi[TQ], plo[TQ];
      float sv[TQ][8];
      qk_scores(pp, sv);
      rescale_test(sv);
      lread_v(cur);
      mask_v(pp);
      weights(0, sv, phi[0], plo[0]);
#pragma unroll
      for (int t = 1; t < TQ; ++t) pv_with_weights(t, sv, phi, plo);
      pv(TQ - 1, phi[TQ - 1], plo[TQ - 1]);
    };
    auto dstep = [&](int pp, auto ca, auto cb, auto fa, auto fb) {
      if (pp + 2 < npair) gload_lds(pp + 2, fa);
      if (pp + 3 < npair) gload_lds(pp + 3, fb);
      compute(pp, ca);
      if (pp + 1 < npair) compute(pp + 1, cb);
      __builtin_amdgcn_s_waitcnt(kWaitAll);
      // a bare barrier: the clobber keeps the compiler from moving LDS reads
      // across it
      asm volatile("s_barrier" ::: "memory");
    };
    if (npair > 0) gload_lds(0, B0{});
    if (npair > 1) gload_lds(1, B1{});
    __builtin_amdgcn_s_waitcnt(kWaitAll);
    __syncthreads();
    // pair pp in buffer pp % 4; unrolled by four pairs so that every buffer
    // index is a constant
    for (int pp = 0; pp < npair; pp += 4) {
      dstep(pp, B0{}, B1{}, B2{}, B3{});
      if (pp + 2 < npair) dstep(pp + 2, B2{}, B3{}, B0{}, B1{});
    }
  }

  // l of query n, then of O row 4j + e, for each tile
#pragma unroll
  for (int t = 0; t < TQ; ++t) {
    float l = l_lane[t];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = kQTile * t + 4 * j + e;               // row of the wave's queries
      const float lr = __shfl(l, 4 * j + e);
      if constexpr (kShared) {
        // (lane swaps in uniform control flow: a swap inside the n == 0
        // branch below would read inactive lanes)
        const int mr = __shfl(mrow[t], 4 * j + e);
        const bool ok = __shfl(static_cast<int>(row_ok[t]), 4 * j + e) != 0;
        const float mq = __shfl(m_run[t], 4 * j + e);
        if (i0 + r < nq && ok) {
          // the piece's partial, unnormalised (an empty piece leaves max
          // -inf, sum 0 and a zero row, which the merge weighs as nothing)
          const int64_t slot = static_cast<int64_t>(piece) * pr.num_seqs + mr;
          float* po = pr.pre_out + (slot * pr.Hq + h) * D;
#pragma unroll
          for (int d = 0; d < NTL; ++d) po[d * 16 + n] = acc[t][d][e];
          // the row's running max and sum (log2 domain; every lane of the
          // row's quad holds the same max)
          if (n == 0) {
            pr.pre_ml[slot * pr.Hq + h] = make_float2(mq, lr);
            pr.pre_stamp[slot * pr.Hq + h] = pr.epoch;
          }
        }
      } else if (i0 + r < nq) {
        const float inv = 1.0f / lr;
#pragma unroll
        for (int d = 0; d < NTL; ++d)
          orow[static_cast<int64_t>(r) * pr.Hq * D + d * 16 + n] = acc[t][d][e] * inv;
      }
    }
  }
}


// ---------------------------------------------------------------------------
// Ping-pong prefill (G a multiple of 4): eight waves per workgroup, two per
// SIMD, in two groups of four (the four query heads of one KV head).  Group
// 0 takes queries 0 .. 31 of the workgroup's 64-query block, group 1 queries
// 32 .. 63; both read the same key pairs from LDS.  The work of a key pair is
// cut into a matrix phase (P.V of the previous pair, then Q.K^T of this one)
// and a vector phase (causal mask, rescale test, weights and their split),
// and the groups run them one phase apart with a workgroup barrier between
// phases: while one wave of a SIMD issues matrix ops, the other issues the
// vector work, so the matrix pipe and the vector ALU run side by side.
// Pair m is staged in LDS buffer m % 4 from phase 2m - 4 on; the wait at the
// end of phase 2m - 1 leaves only pair m + 1's loads in flight.  Every wave
// runs the same phases and barriers; a wave skips the work of pairs past its
// own queries (and all of it when its group has no queries).
// ---------------------------------------------------------------------------
constexpr int kPPWaves = 8;
constexpr int kPPQueries = 64;   // query tokens per workgroup

template <typename T, int D>
__global__ __launch_bounds__(64 * kPPWaves, 1) void prefill_pp_kernel(PrefillParams pr) {
  constexpr int TQ = 2;
  constexpr int NKK = D / 32, NTL = D / 16;
  constexpr int64_t kTileBytes = static_cast<int64_t>(D) * kBlockSize * 2;
  constexpr int kTileU4 = static_cast<int>(kTileBytes / 16);
  constexpr int kStage = 4 * kTileU4 / (64 * kPPWaves);     // loads per thread per pair
  static_assert(kStage >= 1 && kStage * 64 * kPPWaves == 4 * kTileU4, "pair staging");
  static_assert(kTileU4 % 64 == 0, "a wave's 64 words lie in one tile");

  int lin = blockIdx.x;
  const int g = lin % pr.Hkv;
  lin /= pr.Hkv;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int grp = wave >> 2;
  const int e_head = (lin % (pr.G / 4)) * 4 + (wave & 3);
  lin /= pr.G / 4;
  const int nqb = (pr.ntiles * kQTile + kPPQueries - 1) / kPPQueries;
  const int qb = lin % nqb, b = lin / nqb;
  const int h = g * pr.G + e_head;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, j = lane >> 4;

  // (every early return below is uniform over the workgroup)
  const int q0 = pr.qstart[b], q1 = pr.qstart[b + 1];
  if (!(q0 >= 0 && q0 <= q1 && q1 <= pr.T)) return;     // no row can be trusted
  const int nq = q1 - q0;
  const int iwg = qb * kPPQueries;
  if (iwg >= nq) return;
  const int i0 = iwg + TQ * kQTile * grp;                 // the wave's first query
  const bool active = i0 < nq;                            // (uniform over the group)
  const int L = pr.lens[b];
  float* orow = pr.out + (static_cast<int64_t>(q0) + i0) * pr.Hq * D + static_cast<int64_t>(h) * D;
  auto nan_rows = [&]() {
    if (!active) return;
    for (int idx = lane; idx < TQ * kQTile * D; idx += 64) {
      const int r = idx / D;
      if (i0 + r < nq) orow[static_cast<int64_t>(r) * pr.Hq * D + idx % D] = __builtin_nanf("");
    }
  };
  const bool seq_ok = L >= 0 && L <= pr.max_ctx && L <= pr.max_blocks * kBlockSize && nq <= L &&
                      nq <= pr.max_qlen;
  if (!seq_ok) {
    nan_rows();   // length out of the declared bounds
    return;
  }

  // Q (B operand) of tile t: query 16t + n of the wave, dims kk*32 + 8j .. +8
  uint4 qr[TQ][NKK];
#pragma unroll
  for (int t = 0; t < TQ; ++t) {
    const int i = i0 + kQTile * t + n;
    const bool real = i < nq;
    const uint16_t* qb_ = static_cast<const uint16_t*>(pr.q) +
                          ((real ? static_cast<int64_t>(q0) + i : 0) * pr.Hq + h) * D + j * 8;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      qr[t][kk] = real ? *reinterpret_cast<const uint4*>(qb_ + kk * 32) : make_uint4(0, 0, 0, 0);
  }
  const int first_pos = L - nq;                           // position of query 0
  // key blocks of the workgroup, pairs of the workgroup and of the wave
  const int nblk = (first_pos + min(nq, iwg + kPPQueries) - 1) / kBlockSize + 1;
  const int npair = (nblk + 1) / 2;
  const int npw = active ? ((first_pos + min(nq, i0 + TQ * kQTile) - 1) / kBlockSize + 2) / 2 : 0;

  const char* kbase = static_cast<const char*>(pr.kpool) + g * kTileBytes;
  const char* vbase = static_cast<const char*>(pr.vpool) + g * kTileBytes;
  const int64_t block_stride = static_cast<int64_t>(pr.Hkv) * kTileBytes;
  const int32_t* trow = pr.tables + static_cast<int64_t>(b) * pr.max_blocks;
  // every table entry the workgroup reads is checked up front (each wave
  // checks them all, so the outcome is the same in every wave)
  bool bad = false;
  for (int k = lane; k - lane < nblk; k += 64) {
    const int e = k < nblk ? trow[k] : 0;
    if (__any(e < 0 || e >= pr.num_blocks)) bad = true;
  }
  if (bad) {
    nan_rows();
    return;
  }
  const auto* trow_s = (const __attribute__((address_space(4))) int32_t*)trow;
  auto phys_of = [&](int k) -> int { return trow_s[k]; };

  // Four pair buffers of [K0 | K1 | V0 | V1] tiles, read at a per-lane
  // offset plus a constant.  Separate arrays, so the compiler's wait
  // insertion can tell the buffer being filled from the ones being read (in
  // one array it waits for every load into LDS before any LDS read).
  __shared__ uint4 lds0[4 * kTileU4];
  __shared__ uint4 lds1[4 * kTileU4];
  __shared__ uint4 lds2[4 * kTileU4];
  __shared__ uint4 lds3[4 * kTileU4];
  auto buf_of = [&](auto bc) -> uint4* {
    constexpr int bi = decltype(bc)::value;
    if constexpr (bi == 0) return lds0;
    else if constexpr (bi == 1) return lds1;
    else if constexpr (bi == 2) return lds2;
    else return lds3;
  };
  // K: lane reads word (j*16 + n) + 64 kk of each K tile
  const int k_lane = (j * 16 + n) * 16;
  // V: chunk c sits in slot vswz(c); for the lane's chunks c = A + 16t + n
  // (A = (j >> 1) * D, t < NTL), slot = (A + n) ^ s ^ t with s = (A / 16) & 7,
  // so the byte address of tile t is v_lane ^ (t << 4) ^ (t << 8) (bits 8..10
  // of v_lane are clear).
  const int v_lane = ((((j >> 1) * D + n) ^ (((j >> 1) * D / 16) & 7)) * 16) + (j & 1) * 8;
  // Pair pp's [K0 | K1 | V0 | V1] tiles, global -> LDS (V chunks swizzled)
  auto gload_lds = [&](int pp, auto bc) {
    if (pp >= npair) return;
    const int p0 = phys_of(min(2 * pp, nblk - 1)), p1 = phys_of(min(2 * pp + 1, nblk - 1));
#pragma unroll
    for (int r = 0; r < kStage; ++r) {
      const int c0 = wave * 64 + r * 64 * kPPWaves;     // the wave's first word
      const int part = c0 / kTileU4, idx = c0 % kTileU4 + lane;
      const int sidx = part < 2 ? idx : vswz(idx);
      const char* base = (part < 2 ? kbase : vbase) +
                         static_cast<int64_t>((part & 1) ? p1 : p0) * block_stride;
      // Issued as written (scalar base, 32-bit lane offset, the wave's LDS
      // destination in m0; each lane's 16 bytes land at m0 + 16 * lane).
      // The compiler does not see these loads, so it adds no waits for them
      // before LDS reads (it cannot tell which buffer they fill): the waits
      // at the end of each step below are the ones that order them.
      const uint32_t off = static_cast<uint32_t>(sidx * 16);
      const uint32_t dst = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(buf_of(bc) + c0));
      asm volatile(
          "s_mov_b32 m0, %0\n\t"
          "s_nop 0\n\t"
          "global_load_lds_dwordx4 %1, %2"
          :
          : "s"(dst), "v"(off), "s"(base)
          : "memory", "m0");
    }
  };

  float m_run[TQ], l_lane[TQ], thr[TQ];
  f32x4_t acc[TQ][NTL];
#pragma unroll
  for (int t = 0; t < TQ; ++t) {
    m_run[t] = -INFINITY;
    thr[t] = -INFINITY;
    l_lane[t] = 0.f;
#pragma unroll
    for (int d = 0; d < NTL; ++d) acc[t][d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  float sv[TQ][8];          // scores of the pair: matrix phase -> vector phase
  uint4 phi[TQ], plo[TQ];   // its split weights: vector phase -> next matrix phase
  // (defined from the start: a value left undefined on the paths that skip
  // a pair costs registers across the phase branches)
#pragma unroll
  for (int t = 0; t < TQ; ++t) {
    phi[t] = plo[t] = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int e = 0; e < 8; ++e) sv[t][e] = 0.f;
  }

  // (The phases are forced inline: each is used at eight places, and an
  // outlined phase would take its arrays through scratch memory.)
  // Matrix phase of pair m: P.V of pair m - 1 (weights from the previous
  // vector phase), then the scores of pair m.
  auto mfma_phase = [&](int m, auto bk, auto bv) __attribute__((always_inline)) {
    const bool do_pv = m >= 1 && m - 1 < npw;
    const bool do_qk = m < npw;
    if (do_pv) {
      uint2 vreg[2][NTL];
      const char* vb = reinterpret_cast<const char*>(buf_of(bv)) + 2 * kTileBytes;
      // (opaque: the NTL addresses are formed here, one XOR each, rather
      // than hoisted out of the loop into as many registers)
      int vl = v_lane;
      asm volatile("" : "+v"(vl));
#pragma unroll
      for (int t = 0; t < NTL; ++t) {
        const char* vt = vb + (vl ^ ((t << 4) | (t << 8)));
#pragma unroll
        for (int u = 0; u < 2; ++u)
          vreg[u][t] = *reinterpret_cast<const uint2*>(vt + u * static_cast<int>(kTileBytes));
      }
      // V rows at positions >= L are zeroed, so unwritten slots never reach O
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int kb = 2 * (m - 1) + u;
        if ((kb + 1) * kBlockSize > L) {
          const int nv = (L - kb * kBlockSize) - 4 * j;
          const uint32_t mx = (0 < nv ? 0x0000FFFFu : 0u) | (1 < nv ? 0xFFFF0000u : 0u);
          const uint32_t my = (2 < nv ? 0x0000FFFFu : 0u) | (3 < nv ? 0xFFFF0000u : 0u);
#pragma unroll
          for (int d = 0; d < NTL; ++d) {
            vreg[u][d].x &= mx;
            vreg[u][d].y &= my;
          }
        }
      }
      // output tile by output tile, so V registers free up as P.V goes
#pragma unroll
      for (int d = 0; d < NTL; ++d) {
        const uint4 v = make_uint4(vreg[0][d].x, vreg[0][d].y, vreg[1][d].x, vreg[1][d].y);
#pragma unroll
        for (int t = 0; t < TQ; ++t) {
          acc[t][d] = Mfma<T>::pv8(phi[t], v, acc[t][d]);
          acc[t][d] = Mfma<T>::pv8(plo[t], v, acc[t][d]);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (do_qk) {
      uint4 kreg[2][NKK];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
          kreg[u][kk] = *reinterpret_cast<const uint4*>(
              reinterpret_cast<const char*>(buf_of(bk)) + u * kTileBytes + k_lane + kk * 1024);
      f32x4_t s0[TQ], s1[TQ];
#pragma unroll
      for (int t = 0; t < TQ; ++t) s0[t] = s1[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
        for (int t = 0; t < TQ; ++t) {
          s0[t] = Mfma<T>::qk(kreg[0][kk], qr[t][kk], s0[t]);
          s1[t] = Mfma<T>::qk(kreg[1][kk], qr[t][kk], s1[t]);
        }
#pragma unroll
      for (int t = 0; t < TQ; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sv[t][e] = s0[t][e];
          sv[t][4 + e] = s1[t][e];
        }
    }
  };

  // Vector phase of pair m: causal mask, lazy rescale (as in prefill_kernel),
  // weights and their hi/lo split.
  auto valu_phase = [&](int m) __attribute__((always_inline)) {
    if (m < 0 || m >= npw) return;
    if ((2 * m + 2) * kBlockSize - 1 > first_pos + i0) {
      // lane part of (query position - key position) for query n of a tile
      // and keys 4j .. of a block (recomputed here: this branch is rare)
      const int ln = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
      const int nj = (ln & 15) - 4 * (ln >> 4);
#pragma unroll
      for (int t = 0; t < TQ; ++t) {
        // key 2m*16 + 4j + k is visible to query 16t + n iff k <= dq
        const int dq = (first_pos + i0 + kQTile * t - 2 * m * kBlockSize) + nj;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sv[t][e] = e <= dq ? sv[t][e] : -INFINITY;
          sv[t][4 + e] = kBlockSize + e <= dq ? sv[t][4 + e] : -INFINITY;
        }
      }
    }
    bool over = false;
#pragma unroll
    for (int t = 0; t < TQ; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e) over |= sv[t][e] > thr[t];
    if (__any(over)) {
#pragma unroll
      for (int t = 0; t < TQ; ++t) {
        float bm = sv[t][0];
#pragma unroll
        for (int e = 1; e < 8; ++e) bm = fmaxf(bm, sv[t][e]);
        bm = max_xor16(bm);
        bm = max_xor32(bm);
        const float mn = fmaxf(m_run[t], bm * pr.scale_log2);
        const float alpha = __builtin_amdgcn_exp2f(m_run[t] - mn);
        l_lane[t] *= alpha;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float ar = __shfl(alpha, 4 * j + e);
#pragma unroll
          for (int d = 0; d < NTL; ++d) acc[t][d][e] *= ar;
        }
        m_run[t] = mn;
        thr[t] = (mn + kRescaleSlack) / pr.scale_log2;
      }
    }
#pragma unroll
    for (int t = 0; t < TQ; ++t) {
      float pe[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        pe[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[t][e], pr.scale_log2, -m_run[t]));
      l_lane[t] += ((pe[0] + pe[1]) + (pe[2] + pe[3])) + ((pe[4] + pe[5]) + (pe[6] + pe[7]));
      Mfma<T>::split8(pe, phi[t], plo[t]);
    }
  };

  // s_waitcnt immediates (expcnt left at 7): vmcnt 0 and lgkmcnt 0; vmcnt
  // kStage with lgkmcnt not waited for (15)
  constexpr int kWaitAll = 7 << 4;
  constexpr int kWaitStage = kStage | (7 << 4) | (15 << 8);
  constexpr int kWaitVm0 = (7 << 4) | (15 << 8);
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  using B2 = std::integral_constant<int, 2>;
  using B3 = std::integral_constant<int, 3>;
  gload_lds(0, B0{});
  gload_lds(1, B1{});
  __builtin_amdgcn_s_waitcnt(kWaitAll);
  __syncthreads();
  // Step m: phase 2m (group 0: matrix phase of pair m; group 1: vector
  // phase of pair m - 1), then phase 2m + 1 (group 0: vector phase of pair
  // m; group 1: matrix phase of pair m), a barrier between them.  Pair m + 2
  // goes into the buffer of pair m - 2, whose last reader ran in phase
  // 2m - 1.  Each group runs its own copy of the loop (the same barriers in
  // the same order), so neither carries the other's branches and register
  // moves.
  auto end_step = [&](int m) {
    if (m + 2 < npair)
      __builtin_amdgcn_s_waitcnt(kWaitStage);
    else
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
    asm volatile("s_barrier" ::: "memory");
  };
  auto step0 = [&](int m, auto bc) {
    constexpr int c = decltype(bc)::value;
    gload_lds(m + 2, std::integral_constant<int, (c + 2) % 4>{});
    mfma_phase(m, std::integral_constant<int, c>{}, std::integral_constant<int, (c + 3) % 4>{});
    asm volatile("s_barrier" ::: "memory");
    valu_phase(m);
    end_step(m);
  };
  auto step1 = [&](int m, auto bc) {
    constexpr int c = decltype(bc)::value;
    gload_lds(m + 2, std::integral_constant<int, (c + 2) % 4>{});
    valu_phase(m - 1);
    asm volatile("s_barrier" ::: "memory");
    mfma_phase(m, std::integral_constant<int, c>{}, std::integral_constant<int, (c + 3) % 4>{});
    end_step(m);
  };
  if (grp == 0) {
    for (int m = 0; m <= npair; m += 4) {
      step0(m, B0{});
      if (m + 1 <= npair) step0(m + 1, B1{});
      if (m + 2 <= npair) step0(m + 2, B2{});
      if (m + 3 <= npair) step0(m + 3, B3{});
    }
  } else {
    for (int m = 0; m <= npair; m += 4) {
      step1(m, B0{});
      if (m + 1 <= npair) step1(m + 1, B1{});
      if (m + 2 <= npair) step1(m + 2, B2{});
      if (m + 3 <= npair) step1(m + 3, B3{});
    }
  }

  if (!active) return;
#pragma unroll
  for (int t = 0; t < TQ; ++t) {
    float l = l_lane[t];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = kQTile * t + 4 * j + e;
      const float lr = __shfl(l, 4 * j + e);
      if (i0 + r < nq) {
        const float inv = 1.0f / lr;
#pragma unroll
        for (int d = 0; d < NTL; ++d)
          orow[static_cast<int64_t>(r) * pr.Hq * D + d * 16 + n] = acc[t][d][e] * inv;
      }
    }
  }
}

}  // namespace
}  // namespace pa

#ifdef PA_PREFILL_PP_TU
// Second translation unit (pa_prefill_pp.hip): the ping-pong kernel's
// launcher and its instances only.
namespace pa {
template <typename T, int D>
void launch_prefill_pp(dim3 grid, hipStream_t s, const PrefillParams& pr) {
  prefill_pp_kernel<T, D><<<grid, 64 * kPPWaves, 0, s>>>(pr);
}
template void launch_prefill_pp<BF16, 64>(dim3, hipStream_t, const PrefillParams&);
template void launch_prefill_pp<BF16, 128>(dim3, hipStream_t, const PrefillParams&);
template void launch_prefill_pp<F16, 64>(dim3, hipStream_t, const PrefillParams&);
template void launch_prefill_pp<F16, 128>(dim3, hipStream_t, const PrefillParams&);
}  // namespace pa
#else

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
  // four query heads per workgroup when the group size allows it, each wave
  // then taking kPairTiles consecutive query tiles
  const int wpg = pr.G % 4 == 0 ? 4 : 1;
  const int tq = wpg == 4 ? kPairTiles : 1;
  const uint64_t nwg = static_cast<uint64_t>(num_q_heads / wpg) *
                       ((pr.ntiles + tq - 1) / tq) * num_seqs;
  if (nwg > 0x7fffffffull)
    return fail(PA_ERR_INVALID_ARG, "%s: %llu workgroups exceed the launch limit", fn,
                static_cast<unsigned long long>(nwg));
  const dim3 grid(static_cast<uint32_t>(nwg));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint64_t nwg_pp = static_cast<uint64_t>(num_q_heads / 4) *
                          ((pr.ntiles * kQTile + kPPQueries - 1) / kPPQueries) * num_seqs;
  const dim3 grid_pp(static_cast<uint32_t>(nwg_pp));
#define PA_PREFILL(TAG, DIM)                                                             \
  (wpg == 4 ? (launch_prefill_pp<TAG, DIM>(grid_pp, s, pr), 0)                       \
            : (prefill_kernel<TAG, DIM, 1, 1><<<grid, 64, 0, s>>>(pr), 0))
  if (dtype == PA_BF16)
    head_dim == 64 ? PA_PREFILL(BF16, 64) : PA_PREFILL(BF16, 128);
  else
    head_dim == 64 ? PA_PREFILL(F16, 64) : PA_PREFILL(F16, 128);
#undef PA_PREFILL
  return launch_status(fn);
}

namespace pa {

// Workgroups of the prefix pass without pieces, and the number of key-range
// pieces it is cut into: enough for about kPrefixWorkgroups workgroups (one
// per compute unit: measured on 32 groups of 8 with 64-block prefixes, four
// pieces were 15% slower than one, their extra partials costing more in the
// merge than the shorter pieces saved), at most kMaxPrefixPieces, and pieces
// of at least 16 blocks on prefixes as long as the longest context.
constexpr int kPrefixWorkgroups = 256;

int prefix_layout(int num_groups, int max_group, int Hq, int Hkv, int* wpg, int* tq) {
  const int G = Hq / Hkv;
  *wpg = G % 4 == 0 ? 4 : 1;
  const int ntiles = (max_group + kQTile - 1) / kQTile;
  *tq = (*wpg == 4 && ntiles > 1) ? kPairTiles : 1;
  return ntiles;
}

int shared_prefix_pieces(int num_groups, int max_group, int Hq, int Hkv, int max_ctx) {
  int wpg = 1, tq = 1;
  const int ntiles = prefix_layout(num_groups, max_group, Hq, Hkv, &wpg, &tq);
  const int64_t base = static_cast<int64_t>(Hq / wpg) * ((ntiles + tq - 1) / tq) * num_groups;
  if (base <= 0) return 1;
  int64_t p = (kPrefixWorkgroups + base - 1) / base;
  p = std::min<int64_t>(p, kMaxPrefixPieces);
  p = std::min<int64_t>(p, std::max(1, max_ctx / (16 * kBlockSize)));
  return static_cast<int>(std::max<int64_t>(p, 1));
}

pa_status launch_shared_prefix(float* pre_out, float* pre_ml, uint32_t* pre_stamp, uint32_t epoch,
                               int pieces, const void* q, const void* k_pool, const void* v_pool,
                               const int32_t* tables, const int32_t* prefix_len,
                               const int32_t* group_rows, const int32_t* group_start,
                               int num_groups, int num_rows, int max_group, int num_seqs, int Hq,
                               int Hkv, int D, int num_blocks, int max_blocks, int max_ctx,
                               float scale, pa_dtype dtype, void* stream) {
  PrefillParams pr{};
  pr.q = q;
  pr.kpool = k_pool;
  pr.vpool = v_pool;
  pr.tables = tables;
  pr.qstart = group_start;
  pr.B = num_groups * pieces;
  pr.T = num_rows;
  pr.Hq = Hq;
  pr.Hkv = Hkv;
  pr.G = Hq / Hkv;
  pr.num_blocks = num_blocks;
  pr.max_blocks = max_blocks;
  pr.max_ctx = max_ctx;
  pr.max_qlen = max_group;
  pr.scale_log2 = scale * kLog2e;
  pr.rows = group_rows;
  pr.prefix_len = prefix_len;
  pr.pre_out = pre_out;
  pr.pre_ml = reinterpret_cast<float2*>(pre_ml);
  pr.pre_stamp = pre_stamp;
  pr.epoch = epoch;
  pr.num_seqs = num_seqs;
  pr.pieces = pieces;
  int wpg = 1, tq = 1;
  pr.ntiles = prefix_layout(num_groups, max_group, Hq, Hkv, &wpg, &tq);
  const uint64_t nwg =
      static_cast<uint64_t>(Hq / wpg) * ((pr.ntiles + tq - 1) / tq) * num_groups * pieces;
  if (nwg == 0) return ok();
  if (nwg > 0x7fffffffull)
    return fail(PA_ERR_INVALID_ARG, "shared prefix pass: %llu workgroups exceed the launch limit",
                static_cast<unsigned long long>(nwg));
  const dim3 grid(static_cast<uint32_t>(nwg));
  hipStream_t s = static_cast<hipStream_t>(stream);
#define PA_PREFIX(TAG, DIM)                                                                   \
  (wpg == 1     ? (prefill_kernel<TAG, DIM, 1, 1, true><<<grid, 64, 0, s>>>(pr), 0)          \
   : tq == 1    ? (prefill_kernel<TAG, DIM, 4, 1, true><<<grid, 256, 0, s>>>(pr), 0)         \
                : (prefill_kernel<TAG, DIM, 4, kPairTiles, true><<<grid, 256, 0, s>>>(pr), 0))
  if (dtype == PA_BF16)
    D == 64 ? PA_PREFIX(BF16, 64) : PA_PREFIX(BF16, 128);
  else
    D == 64 ? PA_PREFIX(F16, 64) : PA_PREFIX(F16, 128);
#undef PA_PREFIX
  return launch_status("pa_decode_step_shared (prefix pass)");
}

}  // namespace pa

#endif  // PA_PREFILL_PP_TU
