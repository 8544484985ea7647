// Internal helpers shared by the library's host translation units.
#pragma once

#include <cstdarg>
#include <cstdio>
#include <string>

#include "pa.h"

namespace pa {

// Records a formatted message for pa_last_error() and returns `st`.
pa_status fail(pa_status st, const char* fmt, ...);
// Clears the message and returns PA_OK.
pa_status ok();

// The prefix pass of pa_decode_step_shared (pa_prefill.hip): for each group
// g of sequences sharing a prefix (rows group_rows[group_start[g] ..
// group_start[g+1]-1], batch indices below num_seqs), attention of the
// members' queries over the first prefix_len[first member] positions of the
// first member's table, cut into `pieces` key ranges.  Piece p of each
// member row writes its partial to slot p: the unnormalised weighted sum of V
// to pre_out [pieces][B][Hq][D], the log2-domain (max, sum of 2^(s - max))
// pair to pre_ml [pieces][B][Hq][2] and `epoch` to pre_stamp [pieces][B][Hq].
// Members whose prefix length or prefix blocks differ from the first
// member's, and every member of a group with an unusable length or table,
// are left unwritten.  Sizes validated by the caller.
constexpr int kMaxPrefixPieces = 4;
// Pieces the prefix pass takes for this batch (1 .. kMaxPrefixPieces).
int shared_prefix_pieces(int num_groups, int max_group, int Hq, int Hkv, int max_ctx);
pa_status launch_shared_prefix(float* pre_out, float* pre_ml, uint32_t* pre_stamp, uint32_t epoch,
                               int pieces, const void* q, const void* k_pool, const void* v_pool,
                               const int32_t* tables, const int32_t* prefix_len,
                               const int32_t* group_rows, const int32_t* group_start,
                               int num_groups, int num_rows, int max_group, int num_seqs, int Hq,
                               int Hkv, int D, int num_blocks, int max_blocks, int max_ctx,
                               float scale, pa_dtype dtype, void* stream);

}  // namespace pa
