// Paged-cache data movement on gfx950: token append (the write into a
// sequence's last block), copy-on-write block copy, and the table-walk gather.
//
// All three are pure bit moves (no dtype conversion), so their results are
// exact; the quantizing append encodes 16-bit/fp32 values into the 8-bit
// codes of a quantized cache (page 1, jisaku.com glossary, section
// 「他のKVキャッシュ最適化との組み合わせ」).  Append follows page 3 (abeam.tech review), section
// 「KV キャッシュマネージャ」: new tokens fill the sequence's last block; copy
// follows the same page, section 「用語解説」 (Copy-on-Write): a shared block is
// duplicated before it is written; the gather follows the block table in
// logical order (page 1, jisaku.com glossary, section 「PagedAttentionの解決策」).
#include <hip/hip_runtime.h>

#include <cmath>

#include "pa_device.h"

namespace pa {
namespace {

// Whether the x-token group holding `slot` (x = tokens per 16-byte chunk) is
// appended whole by this call, in order, by consecutive rows: row i holds
// token slot % x of the group, so rows i - slot % x ... i - slot % x + x - 1
// must hold the group's slots one after the other.  Such a group is written
// by its first row in whole 16-byte chunks (x tokens of one dim of V, and x
// consecutive K chunks: whole lines), the other rows skip it; any other
// token is written alone, V element by element.  (A run of appended tokens
// that fills whole groups, as a prompt or a prefill chunk does, thus writes
// every line of its tiles once and whole.)
template <int X>
__device__ inline bool whole_group(const int64_t* __restrict__ slots, int64_t i, int64_t n,
                                   int64_t slot) {
  const int k = static_cast<int>(slot % X);
  const int64_t first = i - k;
  if (first < 0 || first + X > n) return false;
  bool ok = true;
#pragma unroll
  for (int m = 0; m < X; ++m) ok = ok && slots[first + m] == slot - k + m;
  return ok;
}

// 16 bytes from x elements (x * sizeof(element) = 16).
template <typename B, int X>
__device__ inline uint4 pack16(const B (&v)[X]) {
  static_assert(sizeof(B) * X == 16, "a chunk is 16 bytes");
  uint4 r;
  __builtin_memcpy(&r, v, 16);
  return r;
}

// One workgroup per new token.  K moves in 16-byte chunks (a chunk is x
// consecutive dims of one head, contiguous in both source and pool); V goes
// in whole 16-byte chunks for whole groups (see whole_group), otherwise
// element by element.  vchunks: the V pool is 16-byte aligned.
template <typename T>
__global__ __launch_bounds__(256) void append_kernel(typename T::bits* __restrict__ kpool,
                                                     typename T::bits* __restrict__ vpool,
                                                     const typename T::bits* __restrict__ knew,
                                                     const typename T::bits* __restrict__ vnew,
                                                     const int64_t* __restrict__ slots,
                                                     int64_t num_slots_total, int Hkv, int D,
                                                     bool vchunks) {
  using bits = typename T::bits;
  constexpr int X = T::kVecElems;
  const int64_t i = blockIdx.x;
  const int64_t slot = slots[i];
  if (slot < 0 || slot >= num_slots_total) return;  // skipped or out of range
  const int64_t blk = slot / kBlockSize;
  const int t = static_cast<int>(slot % kBlockSize);
  const int chunks_per_head = D / X;
  const int nchunks = Hkv * chunks_per_head;
  const int64_t row = static_cast<int64_t>(Hkv) * D;   // elements per token row
  if (vchunks && whole_group<X>(slots, i, gridDim.x, slot)) {
    if (t % X != 0) return;                          // the group's first row writes it
    // K: thread c takes chunk c / X of head h for token t + c % X (X
    // consecutive threads fill X consecutive 16-byte pieces of the tile)
    for (int c = threadIdx.x; c < nchunks * X; c += blockDim.x) {
      const int m = c % X, hc = c / X;
      const int h = hc / chunks_per_head, ch = hc % chunks_per_head;
      const uint4 val = *reinterpret_cast<const uint4*>(knew + (i + m) * row +
                                                        static_cast<int64_t>(h) * D + ch * X);
      bits* dst = kpool + tile_base(blk, h, Hkv, D) + (ch * kBlockSize + t + m) * X;
      *reinterpret_cast<uint4*>(dst) = val;
    }
    // V: one chunk per (head, dim): the dim's X tokens
    for (int e = threadIdx.x; e < Hkv * D; e += blockDim.x) {
      const int h = e / D, d = e % D;
      bits v[X];
#pragma unroll
      for (int m = 0; m < X; ++m) v[m] = vnew[(i + m) * row + e];
      *reinterpret_cast<uint4*>(vpool + tile_base(blk, h, Hkv, D) + v_elem<T>(t, d, D)) =
          pack16<bits, X>(v);
    }
    return;
  }
  const bits* ksrc = knew + i * row;
  const bits* vsrc = vnew + i * row;
  for (int c = threadIdx.x; c < nchunks; c += blockDim.x) {
    const int h = c / chunks_per_head, ch = c % chunks_per_head;
    const uint4 val = *reinterpret_cast<const uint4*>(ksrc + static_cast<int64_t>(h) * D +
                                                      ch * X);
    bits* dst = kpool + tile_base(blk, h, Hkv, D) + (ch * kBlockSize + t) * X;
    *reinterpret_cast<uint4*>(dst) = val;
  }
  const int nelem = Hkv * D;
  for (int e = threadIdx.x; e < nelem; e += blockDim.x) {
    const int h = e / D, d = e % D;
    vpool[tile_base(blk, h, Hkv, D) + v_elem<T>(t, d, D)] = vsrc[e];
  }
}

// Quantizing append: one workgroup per new token.  K: each thread encodes 16
// consecutive dims of one head (one 16-byte chunk of the pool); V: one byte
// per element (a V chunk holds 16 tokens of one dim), or whole chunks when
// the call appends the block's 16 tokens in order (see whole_group).
template <typename Src, typename Code>
__global__ __launch_bounds__(256) void append_quant_kernel(uint8_t* __restrict__ kpool,
                                                           uint8_t* __restrict__ vpool,
                                                           const typename Src::bits* __restrict__ knew,
                                                           const typename Src::bits* __restrict__ vnew,
                                                           const int64_t* __restrict__ slots,
                                                           int64_t num_slots_total, int Hkv, int D,
                                                           float rk, float rv, bool vchunks) {
  using bits = typename Src::bits;
  constexpr int X = 16;                               // codes per 16-byte chunk
  const int64_t i = blockIdx.x;
  const int64_t slot = slots[i];
  if (slot < 0 || slot >= num_slots_total) return;
  const int64_t blk = slot / kBlockSize;
  const int t = static_cast<int>(slot % kBlockSize);
  const int chunks_per_head = D / 16;
  const int64_t row = static_cast<int64_t>(Hkv) * D;
  // the codes of 16 consecutive dims of one head of token row r
  auto k_chunk = [&](int64_t r, int h, int ch) {
    const bits* x = knew + r * row + static_cast<int64_t>(h) * D + ch * 16;
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = Encode<Code>::pair(Src::to_float(x[4 * j]), Src::to_float(x[4 * j + 1]), rk);
      const uint32_t hi = Encode<Code>::pair(Src::to_float(x[4 * j + 2]), Src::to_float(x[4 * j + 3]), rk);
      w[j] = lo | (hi << 16);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
  };
  if (vchunks && whole_group<X>(slots, i, gridDim.x, slot)) {
    if (t % X != 0) return;                          // the block's first row writes it
    for (int c = threadIdx.x; c < Hkv * chunks_per_head * X; c += blockDim.x) {
      const int m = c % X, hc = c / X;
      const int h = hc / chunks_per_head, ch = hc % chunks_per_head;
      *reinterpret_cast<uint4*>(kpool + tile_base(blk, h, Hkv, D) + (ch * kBlockSize + t + m) * 16) =
          k_chunk(i + m, h, ch);
    }
    for (int e = threadIdx.x; e < Hkv * D; e += blockDim.x) {
      const int h = e / D, d = e % D;
      uint8_t v[X];
#pragma unroll
      for (int m = 0; m < X; ++m)
        v[m] = static_cast<uint8_t>(Encode<Code>::pair(Src::to_float(vnew[(i + m) * row + e]),
                                                       0.f, rv) & 0xFFu);
      *reinterpret_cast<uint4*>(vpool + tile_base(blk, h, Hkv, D) + v_elem<U8>(t, d, D)) =
          pack16<uint8_t, X>(v);
    }
    return;
  }
  const bits* vsrc = vnew + i * row;
  for (int c = threadIdx.x; c < Hkv * chunks_per_head; c += blockDim.x) {
    const int h = c / chunks_per_head, ch = c % chunks_per_head;
    *reinterpret_cast<uint4*>(kpool + tile_base(blk, h, Hkv, D) + (ch * kBlockSize + t) * 16) =
        k_chunk(i, h, ch);
  }
  for (int e = threadIdx.x; e < Hkv * D; e += blockDim.x) {
    const int h = e / D, d = e % D;
    const uint32_t code = Encode<Code>::pair(Src::to_float(vsrc[e]), 0.f, rv) & 0xFFu;
    vpool[tile_base(blk, h, Hkv, D) + v_elem<U8>(t, d, D)] = static_cast<uint8_t>(code);
  }
}

// grid = (num_pairs, 2, slices): y selects the K or the V pool, z a 4 KiB
// slice of the block (each workgroup moves 256 x 16 bytes, so a pair's copy
// is spread over many workgroups instead of one streaming the whole block).
constexpr int kCopySliceChunks = 256;

__global__ __launch_bounds__(256) void copy_blocks_kernel(uint4* __restrict__ kpool,
                                                          uint4* __restrict__ vpool,
                                                          const int32_t* __restrict__ pairs,
                                                          int num_blocks,
                                                          int64_t chunks_per_block) {
  const int src = pairs[2 * blockIdx.x], dst = pairs[2 * blockIdx.x + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks || src == dst) return;
  uint4* pool = blockIdx.y == 0 ? kpool : vpool;
  const uint4* s = pool + static_cast<int64_t>(src) * chunks_per_block;
  uint4* d = pool + static_cast<int64_t>(dst) * chunks_per_block;
  for (int64_t c = static_cast<int64_t>(blockIdx.z) * kCopySliceChunks + threadIdx.x;
       c < chunks_per_block; c += static_cast<int64_t>(gridDim.z) * kCopySliceChunks)
    d[c] = s[c];
}

// grid = (num_pairs, 2 * num_layers, slices): y = 2 * layer + (0: K pool,
// 1: V pool), z a 4 KiB slice of the block.
__global__ __launch_bounds__(256) void copy_blocks_layers_kernel(
    uint4* const* __restrict__ kpools, uint4* const* __restrict__ vpools,
    const int32_t* __restrict__ pairs, int num_blocks, int64_t chunks_per_block) {
  const int src = pairs[2 * blockIdx.x], dst = pairs[2 * blockIdx.x + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks || src == dst) return;
  const int layer = blockIdx.y >> 1;
  uint4* pool = (blockIdx.y & 1) ? vpools[layer] : kpools[layer];
  const uint4* s = pool + static_cast<int64_t>(src) * chunks_per_block;
  uint4* d = pool + static_cast<int64_t>(dst) * chunks_per_block;
  for (int64_t c = static_cast<int64_t>(blockIdx.z) * kCopySliceChunks + threadIdx.x;
       c < chunks_per_block; c += static_cast<int64_t>(gridDim.z) * kCopySliceChunks)
    d[c] = s[c];
}

// Slices per block copy (gridDim.z), at most 64 (a block's copy still covers
// every chunk through the grid-stride loop).
unsigned copy_slices(int64_t chunks_per_block) {
  const int64_t n = (chunks_per_block + kCopySliceChunks - 1) / kCopySliceChunks;
  return static_cast<unsigned>(n < 1 ? 1 : n > 64 ? 64 : n);
}

// grid = (ceil(max_len/16), Hkv, B): one logical block of one head per
// workgroup, written to [B][Hkv][max_len][D] in logical order.
template <typename T>
__global__ __launch_bounds__(256) void gather_kernel(typename T::bits* __restrict__ kout,
                                                     typename T::bits* __restrict__ vout,
                                                     const typename T::bits* __restrict__ kpool,
                                                     const typename T::bits* __restrict__ vpool,
                                                     const int32_t* __restrict__ tables,
                                                     const int32_t* __restrict__ lens, int Hkv,
                                                     int D, int num_blocks, int max_blocks,
                                                     int max_len) {
  using bits = typename T::bits;
  const int lb = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int L = lens[b];
  const bool len_ok = L >= 0 && L <= max_len && L <= max_blocks * kBlockSize;
  const int phys = (len_ok && lb * kBlockSize < L) ? tables[static_cast<int64_t>(b) * max_blocks + lb]
                                                   : -1;
  const bool blk_ok = phys >= 0 && phys < num_blocks;
  const int64_t row = (static_cast<int64_t>(b) * Hkv + g) * max_len;
  for (int idx = threadIdx.x; idx < kBlockSize * D; idx += blockDim.x) {
    const int t = idx / D, d = idx % D;
    const int pos = lb * kBlockSize + t;
    if (pos >= max_len) continue;
    bits kv = 0, vv = 0;
    if (!len_ok) {
      kv = vv = static_cast<bits>(~bits(0));  // all-ones = NaN pattern: bad length
    } else if (pos < L) {
      if (blk_ok) {
        const int64_t base = tile_base(phys, g, Hkv, D);
        kv = kpool[base + k_elem<T>(t, d)];
        vv = vpool[base + v_elem<T>(t, d, D)];
      } else {
        kv = vv = static_cast<bits>(~bits(0));  // bad table entry
      }
    }
    kout[(row + pos) * D + d] = kv;
    vout[(row + pos) * D + d] = vv;
  }
}

// Streaming read of n16 16-byte words (grid-stride, non-temporal loads),
// folded with XOR into one word per thread; the result is stored only if it
// equals a value no buffer of identical words produces, so the loads stay
// live without a write per thread.  A context measure of the chip's read
// bandwidth for the decode kernels.
typedef int i32x4_t __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void stream_read_kernel(const i32x4_t* __restrict__ p,
                                                          int64_t n16, int* __restrict__ sink) {
  i32x4_t acc = {0, 0, 0, 0};
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n16;
       i += stride)
    acc ^= __builtin_nontemporal_load(p + i);
  if (acc.x == 0x5A5A5A5A && acc.y == 0x3C3C3C3C && acc.z == acc.w) sink[0] = acc.x;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

pa_status check_common(const char* fn, int num_blocks, int Hkv, int D, int bs, pa_dtype dt) {
  if (!pool_dtype_ok(dt)) return fail(PA_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dt);
  if (bs != kBlockSize)
    return fail(PA_ERR_UNSUPPORTED, "%s: block_size %d (only 16 is supported)", fn, bs);
  if (num_blocks <= 0 || Hkv <= 0 || D <= 0)
    return fail(PA_ERR_INVALID_ARG, "%s: num_blocks/num_kv_heads/head_dim must be > 0", fn);
  if (D % 16 != 0 || D > 256)
    return fail(PA_ERR_UNSUPPORTED, "%s: head_dim %d (multiple of 16 up to 256)", fn, D);
  return PA_OK;
}

}  // namespace
}  // namespace pa

using namespace pa;

extern "C" pa_status pa_stream_read(const void* buf, size_t bytes, int32_t* sink,
                                    void* stream) {
  if (!buf || !sink) return fail(PA_ERR_INVALID_ARG, "pa_stream_read: NULL pointer");
  if (!aligned16(buf) || bytes % 16 != 0)
    return fail(PA_ERR_INVALID_ARG, "pa_stream_read: buffer must be 16-byte aligned and sized");
  if (bytes == 0) return ok();
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  stream_read_kernel<<<cus * 8, 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const i32x4_t*>(buf), static_cast<int64_t>(bytes / 16), sink);
  return launch_status("pa_stream_read");
}

extern "C" pa_status pa_cache_append(void* k_pool, void* v_pool, const void* k_new,
                                     const void* v_new, const int64_t* slot_mapping,
                                     int32_t num_tokens, int32_t num_blocks,
                                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                     pa_dtype dtype, void* stream) {
  pa_status st = check_common("pa_cache_append", num_blocks, num_kv_heads, head_dim, block_size,
                              dtype);
  if (st != PA_OK) return st;
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "pa_cache_append: num_tokens < 0");
  if (num_tokens == 0) return ok();
  if (!k_pool || !v_pool || !k_new || !v_new || !slot_mapping)
    return fail(PA_ERR_INVALID_ARG, "pa_cache_append: NULL pointer");
  if (!aligned16(k_pool) || !aligned16(k_new))
    return fail(PA_ERR_INVALID_ARG, "pa_cache_append: K pointers must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t total = static_cast<int64_t>(num_blocks) * kBlockSize;
  dim3 grid(num_tokens), block(256);
  const bool vchunks = aligned16(v_pool);
  switch (dtype) {
    case PA_F32:
      append_kernel<F32><<<grid, block, 0, s>>>(
          static_cast<uint32_t*>(k_pool), static_cast<uint32_t*>(v_pool),
          static_cast<const uint32_t*>(k_new), static_cast<const uint32_t*>(v_new), slot_mapping,
          total, num_kv_heads, head_dim, vchunks);
      break;
    case PA_F16:
      append_kernel<F16><<<grid, block, 0, s>>>(
          static_cast<uint16_t*>(k_pool), static_cast<uint16_t*>(v_pool),
          static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new), slot_mapping,
          total, num_kv_heads, head_dim, vchunks);
      break;
    case PA_BF16:
      append_kernel<BF16><<<grid, block, 0, s>>>(
          static_cast<uint16_t*>(k_pool), static_cast<uint16_t*>(v_pool),
          static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new), slot_mapping,
          total, num_kv_heads, head_dim, vchunks);
      break;
    case PA_FP8_E4M3:
    case PA_INT8:
      append_kernel<U8><<<grid, block, 0, s>>>(
          static_cast<uint8_t*>(k_pool), static_cast<uint8_t*>(v_pool),
          static_cast<const uint8_t*>(k_new), static_cast<const uint8_t*>(v_new), slot_mapping,
          total, num_kv_heads, head_dim, vchunks);
      break;
  }
  return launch_status("pa_cache_append");
}

extern "C" pa_status pa_cache_append_quant(void* k_pool, void* v_pool, const void* k_new,
                                           const void* v_new, const int64_t* slot_mapping,
                                           int32_t num_tokens, int32_t num_blocks,
                                           int32_t num_kv_heads, int32_t head_dim,
                                           int32_t block_size, pa_dtype cache_dtype,
                                           pa_dtype src_dtype, float k_scale, float v_scale,
                                           void* stream) {
  const char* fn = "pa_cache_append_quant";
  pa_status st = check_common(fn, num_blocks, num_kv_heads, head_dim, block_size, cache_dtype);
  if (st != PA_OK) return st;
  if (!code_dtype(cache_dtype))
    return fail(PA_ERR_INVALID_ARG, "%s: cache dtype %d is not an 8-bit code dtype", fn,
                (int)cache_dtype);
  if (!dtype_ok(src_dtype))
    return fail(PA_ERR_INVALID_ARG, "%s: source dtype %d (fp32, fp16 or bf16)", fn,
                (int)src_dtype);
  if (!(k_scale > 0.f) || !(v_scale > 0.f) || !std::isfinite(k_scale) || !std::isfinite(v_scale))
    return fail(PA_ERR_INVALID_ARG, "%s: scales must be positive and finite", fn);
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "%s: num_tokens < 0", fn);
  if (num_tokens == 0) return ok();
  if (!k_pool || !v_pool || !k_new || !v_new || !slot_mapping)
    return fail(PA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (!aligned16(k_pool)) return fail(PA_ERR_INVALID_ARG, "%s: k_pool must be 16-byte aligned", fn);
  // the reciprocals, rounded once to fp32 on the host
  const float rk = 1.0f / k_scale, rv = 1.0f / v_scale;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t total = static_cast<int64_t>(num_blocks) * kBlockSize;
  dim3 grid(num_tokens), block(256);
  uint8_t* kp = static_cast<uint8_t*>(k_pool);
  uint8_t* vp = static_cast<uint8_t*>(v_pool);
  const bool vchunks = aligned16(v_pool);
#define PA_APPEND_Q(SRC, CODE)                                                                 \
  append_quant_kernel<SRC, CODE><<<grid, block, 0, s>>>(                                      \
      kp, vp, static_cast<const SRC::bits*>(k_new), static_cast<const SRC::bits*>(v_new),     \
      slot_mapping, total, num_kv_heads, head_dim, rk, rv, vchunks)
  const bool fp8 = cache_dtype == PA_FP8_E4M3;
  switch (src_dtype) {
    case PA_F32: if (fp8) PA_APPEND_Q(F32, E4M3); else PA_APPEND_Q(F32, I8); break;
    case PA_F16: if (fp8) PA_APPEND_Q(F16, E4M3); else PA_APPEND_Q(F16, I8); break;
    default: if (fp8) PA_APPEND_Q(BF16, E4M3); else PA_APPEND_Q(BF16, I8); break;
  }
#undef PA_APPEND_Q
  return launch_status(fn);
}

extern "C" pa_status pa_copy_blocks(void* k_pool, void* v_pool, const int32_t* block_pairs,
                                    int32_t num_pairs, int32_t num_blocks, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t block_size, pa_dtype dtype,
                                    void* stream) {
  pa_status st = check_common("pa_copy_blocks", num_blocks, num_kv_heads, head_dim, block_size,
                              dtype);
  if (st != PA_OK) return st;
  if (num_pairs < 0) return fail(PA_ERR_INVALID_ARG, "pa_copy_blocks: num_pairs < 0");
  if (num_pairs == 0) return ok();
  if (!k_pool || !v_pool || !block_pairs)
    return fail(PA_ERR_INVALID_ARG, "pa_copy_blocks: NULL pointer");
  if (!aligned16(k_pool) || !aligned16(v_pool))
    return fail(PA_ERR_INVALID_ARG, "pa_copy_blocks: pools must be 16-byte aligned");
  const int64_t block_bytes = static_cast<int64_t>(num_kv_heads) * head_dim * kBlockSize *
                              static_cast<int64_t>(dtype_bytes(dtype));
  dim3 grid(num_pairs, 2, copy_slices(block_bytes / 16)), block(256);
  copy_blocks_kernel<<<grid, block, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<uint4*>(k_pool), static_cast<uint4*>(v_pool), block_pairs, num_blocks,
      block_bytes / 16);
  return launch_status("pa_copy_blocks");
}

extern "C" pa_status pa_copy_blocks_layers(void* const* k_pools, void* const* v_pools,
                                           int32_t num_layers, const int32_t* block_pairs,
                                           int32_t num_pairs, int32_t num_blocks,
                                           int32_t num_kv_heads, int32_t head_dim,
                                           int32_t block_size, pa_dtype dtype, void* stream) {
  const char* fn = "pa_copy_blocks_layers";
  pa_status st = check_common(fn, num_blocks, num_kv_heads, head_dim, block_size, dtype);
  if (st != PA_OK) return st;
  if (num_pairs < 0 || num_layers < 0)
    return fail(PA_ERR_INVALID_ARG, "%s: negative count", fn);
  if (num_layers > 32767) return fail(PA_ERR_INVALID_ARG, "%s: too many layers", fn);
  if (num_pairs == 0 || num_layers == 0) return ok();
  if (!k_pools || !v_pools || !block_pairs) return fail(PA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  const int64_t block_bytes = static_cast<int64_t>(num_kv_heads) * head_dim * kBlockSize *
                              static_cast<int64_t>(dtype_bytes(dtype));
  dim3 grid(num_pairs, 2 * num_layers, copy_slices(block_bytes / 16)), block(256);
  copy_blocks_layers_kernel<<<grid, block, 0, static_cast<hipStream_t>(stream)>>>(
      reinterpret_cast<uint4* const*>(k_pools), reinterpret_cast<uint4* const*>(v_pools),
      block_pairs, num_blocks, block_bytes / 16);
  return launch_status(fn);
}

extern "C" pa_status pa_gather_kv(void* k_out, void* v_out, const void* k_pool,
                                  const void* v_pool, const int32_t* block_tables,
                                  const int32_t* context_lens, int32_t num_seqs,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                  int32_t num_blocks, int32_t max_blocks_per_seq,
                                  int32_t max_context_len, pa_dtype dtype, void* stream) {
  pa_status st = check_common("pa_gather_kv", num_blocks, num_kv_heads, head_dim, block_size,
                              dtype);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || max_blocks_per_seq < 0 || max_context_len < 0)
    return fail(PA_ERR_INVALID_ARG, "pa_gather_kv: negative size");
  if (num_seqs == 0 || max_context_len == 0) return ok();
  if (!k_out || !v_out || !k_pool || !v_pool || !block_tables || !context_lens)
    return fail(PA_ERR_INVALID_ARG, "pa_gather_kv: NULL pointer");
  dim3 grid((max_context_len + kBlockSize - 1) / kBlockSize, num_kv_heads, num_seqs), block(256);
  hipStream_t s = static_cast<hipStream_t>(stream);
#define PA_GATHER(TAG, BITS)                                                                  \
  gather_kernel<TAG><<<grid, block, 0, s>>>(                                                  \
      static_cast<BITS*>(k_out), static_cast<BITS*>(v_out), static_cast<const BITS*>(k_pool), \
      static_cast<const BITS*>(v_pool), block_tables, context_lens, num_kv_heads, head_dim,   \
      num_blocks, max_blocks_per_seq, max_context_len)
  switch (dtype) {
    case PA_F32: PA_GATHER(F32, uint32_t); break;
    case PA_F16: PA_GATHER(F16, uint16_t); break;
    case PA_BF16: PA_GATHER(BF16, uint16_t); break;
    case PA_FP8_E4M3:
    case PA_INT8: PA_GATHER(U8, uint8_t); break;
  }
#undef PA_GATHER
  return launch_status("pa_gather_kv");
}
