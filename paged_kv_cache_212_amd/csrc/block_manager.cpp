// Host-side KV block manager: free pool, per-sequence block tables, reference
// counts, fork and copy-on-write planning.
//
// Rules (pages: page 2, hubblespacetelescope blog, section 「OSの知恵をGPUへ…」;
// page 3, abeam.tech review, sections 「KV キャッシュマネージャ」 and
// 「並列サンプリングやビームサーチでの共有」):
//   * a sequence takes one new block whenever a write starts a block
//     (position % block_size == 0), so only its last block can hold slack;
//   * a finished sequence returns its blocks to the pool;
//   * forks share blocks by reference count; a write into a block held more
//     than once first copies it (the writer moves to the copy).
// Choices where the pages are silent: LIFO free stack seeded with free_order,
// blocks released in table order, all-or-nothing batches.
// Sliding window (page 1, jisaku.com glossary, section
// 「他のKVキャッシュ最適化との組み合わせ」: blocks that left the window can be
// freed): pa_bm_release_before drops a sequence's blocks whose slots all lie
// before a position; their table entries become -1 (placeholders, so
// position p keeps mapping to entry p / block_size).
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pa_internal.h"

struct pa_bm {
  struct Seq {
    std::vector<int32_t> table;  // logical block -> physical block (-1: released)
    int32_t len = 0;             // tokens written so far
    uint64_t stamp = 0;          // last pa_bm_step call that named it (repeat check)
  };
  uint64_t step_gen = 0;         // pa_bm_step calls so far
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> free_stack;  // back() is the next block handed out
  std::vector<int32_t> ref;         // reference count per physical block
  std::unordered_map<int64_t, Seq> seqs;

  int32_t take() {
    int32_t b = free_stack.back();
    free_stack.pop_back();
    ref[b] = 1;
    return b;
  }

  // Blocks needed to write positions [len, len + n) of `s`.  `pending` holds
  // count decrements of copies planned earlier in the same batch.
  int64_t blocks_needed(const Seq& s, int32_t n,
                        std::unordered_map<int32_t, int32_t>* pending) const {
    if (n == 0) return 0;
    int64_t need = 0;
    const int32_t L = s.len;
    if (L % block_size != 0) {
      const int32_t tail = s.table[L / block_size];
      int32_t eff = ref[tail];
      if (pending) {
        auto it = pending->find(tail);
        if (it != pending->end()) eff -= it->second;
      }
      if (eff > 1) {
        ++need;
        if (pending) (*pending)[tail] += 1;
      }
    }
    const int64_t have = (static_cast<int64_t>(L) + block_size - 1) / block_size;
    const int64_t after = (static_cast<int64_t>(L) + n + block_size - 1) / block_size;
    return need + (after - have);
  }

  // Performs the write planned by blocks_needed (caller checked capacity).
  void write(Seq& s, int32_t n, int64_t* slots, int32_t* pairs, int32_t* num_pairs) {
    for (int32_t i = 0; i < n; ++i) {
      const int32_t p = s.len + i;
      const int32_t lb = p / block_size;
      if (p % block_size == 0) {
        s.table.push_back(take());
      } else {
        const int32_t old = s.table[lb];
        if (ref[old] > 1) {
          const int32_t fresh = take();
          --ref[old];
          s.table[lb] = fresh;
          if (pairs) {
            pairs[2 * *num_pairs] = old;
            pairs[2 * *num_pairs + 1] = fresh;
          }
          ++*num_pairs;
        }
      }
      if (slots) slots[i] = static_cast<int64_t>(s.table[lb]) * block_size + p % block_size;
    }
    s.len += n;
  }
};

using pa::fail;

extern "C" pa_status pa_bm_create(int32_t num_blocks, int32_t block_size,
                                  const int32_t* free_order, pa_bm** out) {
  if (!out) return fail(PA_ERR_INVALID_ARG, "pa_bm_create: out is NULL");
  *out = nullptr;
  if (num_blocks <= 0 || block_size <= 0)
    return fail(PA_ERR_INVALID_ARG, "pa_bm_create: num_blocks=%d block_size=%d must be > 0",
                num_blocks, block_size);
  pa_bm* bm = new (std::nothrow) pa_bm();
  if (!bm) return fail(PA_ERR_INVALID_ARG, "pa_bm_create: host allocation failed");
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->ref.assign(num_blocks, 0);
  bm->free_stack.resize(num_blocks);
  std::vector<uint8_t> seen(num_blocks, 0);
  for (int32_t i = 0; i < num_blocks; ++i) {
    const int32_t b = free_order ? free_order[i] : i;
    if (b < 0 || b >= num_blocks || seen[b]) {
      delete bm;
      return fail(PA_ERR_INVALID_ARG, "pa_bm_create: free_order is not a permutation of [0,%d)",
                  num_blocks);
    }
    seen[b] = 1;
    bm->free_stack[num_blocks - 1 - i] = b;  // first handed out = free_order[0]
  }
  *out = bm;
  return pa::ok();
}

extern "C" void pa_bm_destroy(pa_bm* bm) { delete bm; }

extern "C" pa_status pa_bm_add_seq(pa_bm* bm, int64_t seq_id, int32_t num_tokens,
                                   int64_t* slots_out) {
  if (!bm) return fail(PA_ERR_INVALID_ARG, "pa_bm_add_seq: bm is NULL");
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "pa_bm_add_seq: num_tokens < 0");
  if (bm->seqs.count(seq_id)) return fail(PA_ERR_SEQ_EXISTS, "sequence %lld exists",
                                          static_cast<long long>(seq_id));
  pa_bm::Seq s;
  const int64_t need = bm->blocks_needed(s, num_tokens, nullptr);
  if (need > static_cast<int64_t>(bm->free_stack.size()))
    return fail(PA_ERR_OUT_OF_BLOCKS, "pa_bm_add_seq: need %lld blocks, %zu free",
                static_cast<long long>(need), bm->free_stack.size());
  int32_t np = 0;
  bm->write(s, num_tokens, slots_out, nullptr, &np);
  bm->seqs.emplace(seq_id, std::move(s));
  return pa::ok();
}

extern "C" pa_status pa_bm_fork(pa_bm* bm, int64_t parent_id, int64_t child_id) {
  if (!bm) return fail(PA_ERR_INVALID_ARG, "pa_bm_fork: bm is NULL");
  auto it = bm->seqs.find(parent_id);
  if (it == bm->seqs.end()) return fail(PA_ERR_UNKNOWN_SEQ, "unknown sequence %lld",
                                        static_cast<long long>(parent_id));
  if (bm->seqs.count(child_id)) return fail(PA_ERR_SEQ_EXISTS, "sequence %lld exists",
                                            static_cast<long long>(child_id));
  pa_bm::Seq child = it->second;
  for (int32_t b : child.table)
    if (b >= 0) ++bm->ref[b];
  bm->seqs.emplace(child_id, std::move(child));
  return pa::ok();
}

extern "C" pa_status pa_bm_extend(pa_bm* bm, int64_t seq_id, int32_t num_tokens,
                                  int64_t* slots_out, int32_t* cow_pairs_out,
                                  int32_t* num_cow_out) {
  if (!bm) return fail(PA_ERR_INVALID_ARG, "pa_bm_extend: bm is NULL");
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "pa_bm_extend: num_tokens < 0");
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return fail(PA_ERR_UNKNOWN_SEQ, "unknown sequence %lld",
                                        static_cast<long long>(seq_id));
  pa_bm::Seq& s = it->second;
  if (static_cast<int64_t>(s.len) + num_tokens > INT32_MAX)
    return fail(PA_ERR_INVALID_ARG, "pa_bm_extend: length overflow");
  std::unordered_map<int32_t, int32_t> pending;
  const int64_t need = bm->blocks_needed(s, num_tokens, &pending);
  if (!pending.empty() && !cow_pairs_out)
    return fail(PA_ERR_INVALID_ARG, "pa_bm_extend: a copy is needed but cow_pairs_out is NULL");
  if (need > static_cast<int64_t>(bm->free_stack.size()))
    return fail(PA_ERR_OUT_OF_BLOCKS, "pa_bm_extend: need %lld blocks, %zu free",
                static_cast<long long>(need), bm->free_stack.size());
  int32_t np = 0;
  bm->write(s, num_tokens, slots_out, cow_pairs_out, &np);
  if (num_cow_out) *num_cow_out = np;
  return pa::ok();
}

extern "C" pa_status pa_bm_append_slots(pa_bm* bm, const int64_t* seq_ids, int32_t n,
                                        int64_t* slots_out, int32_t* cow_pairs_out,
                                        int32_t* num_cow_out) {
  if (!bm) return fail(PA_ERR_INVALID_ARG, "pa_bm_append_slots: bm is NULL");
  if (n < 0 || (n > 0 && (!seq_ids || !slots_out || !cow_pairs_out)))
    return fail(PA_ERR_INVALID_ARG, "pa_bm_append_slots: bad n or NULL buffer");
  std::vector<pa_bm::Seq*> seqs(n);
  std::unordered_set<int64_t> distinct;
  distinct.reserve(n * 2 + 1);
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end()) return fail(PA_ERR_UNKNOWN_SEQ, "unknown sequence %lld",
                                          static_cast<long long>(seq_ids[i]));
    if (!distinct.insert(seq_ids[i]).second)
      return fail(PA_ERR_INVALID_ARG, "pa_bm_append_slots: sequence %lld twice in batch",
                  static_cast<long long>(seq_ids[i]));
    if (it->second.len == INT32_MAX) return fail(PA_ERR_INVALID_ARG, "length overflow");
    seqs[i] = &it->second;
  }
  std::unordered_map<int32_t, int32_t> pending;
  int64_t need = 0;
  for (int32_t i = 0; i < n; ++i) need += bm->blocks_needed(*seqs[i], 1, &pending);
  if (need > static_cast<int64_t>(bm->free_stack.size()))
    return fail(PA_ERR_OUT_OF_BLOCKS, "pa_bm_append_slots: need %lld blocks, %zu free",
                static_cast<long long>(need), bm->free_stack.size());
  int32_t np = 0;
  for (int32_t i = 0; i < n; ++i) bm->write(*seqs[i], 1, slots_out + i, cow_pairs_out, &np);
  if (num_cow_out) *num_cow_out = np;
  return pa::ok();
}

extern "C" pa_status pa_bm_step(pa_bm* bm, const int64_t* seq_ids, int32_t n, int32_t max_blocks,
                                int64_t* slots_out, int32_t* cow_pairs_out, int32_t* num_cow_out,
                                int32_t* tables_out, int32_t* lens_out,
                                int32_t* blocks_needed_out) {
  if (!bm) return fail(PA_ERR_INVALID_ARG, "pa_bm_step: bm is NULL");
  if (n < 0 || max_blocks < 0 || !blocks_needed_out ||
      (n > 0 && (!seq_ids || !slots_out || !cow_pairs_out || !tables_out || !lens_out)))
    return fail(PA_ERR_INVALID_ARG, "pa_bm_step: bad n/max_blocks or NULL buffer");
  // Each sequence looked up once; a repeat is caught by the call's stamp.
  // The checks all come before any change (all-or-nothing).
  const uint64_t gen = ++bm->step_gen;
  std::vector<pa_bm::Seq*> seqs(n);
  int32_t need_rows = 0;
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end()) return fail(PA_ERR_UNKNOWN_SEQ, "unknown sequence %lld",
                                          static_cast<long long>(seq_ids[i]));
    pa_bm::Seq& sq = it->second;
    if (sq.stamp == gen)
      return fail(PA_ERR_INVALID_ARG, "pa_bm_step: sequence %lld twice in batch",
                  static_cast<long long>(seq_ids[i]));
    sq.stamp = gen;
    if (sq.len == INT32_MAX) return fail(PA_ERR_INVALID_ARG, "length overflow");
    const int64_t len = static_cast<int64_t>(sq.len) + 1;
    need_rows = static_cast<int32_t>(
        std::max<int64_t>(need_rows, (len + bm->block_size - 1) / bm->block_size));
    seqs[i] = &sq;
  }
  *blocks_needed_out = need_rows;
  if (need_rows > max_blocks)
    return fail(PA_ERR_INVALID_ARG, "pa_bm_step: tables need %d blocks > max_blocks %d",
                need_rows, max_blocks);
  std::unordered_map<int32_t, int32_t> pending;
  int64_t need = 0;
  for (int32_t i = 0; i < n; ++i) need += bm->blocks_needed(*seqs[i], 1, &pending);
  if (need > static_cast<int64_t>(bm->free_stack.size()))
    return fail(PA_ERR_OUT_OF_BLOCKS, "pa_bm_step: need %lld blocks, %zu free",
                static_cast<long long>(need), bm->free_stack.size());
  int32_t np = 0;
  for (int32_t i = 0; i < n; ++i) {
    pa_bm::Seq& sq = *seqs[i];
    bm->write(sq, 1, slots_out + i, cow_pairs_out, &np);
    int32_t* row = tables_out + static_cast<int64_t>(i) * max_blocks;
    const size_t nb = sq.table.size();
    std::memcpy(row, sq.table.data(), nb * sizeof(int32_t));
    std::fill(row + nb, row + max_blocks, -1);
    lens_out[i] = sq.len;
  }
  if (num_cow_out) *num_cow_out = np;
  return pa::ok();
}

extern "C" pa_status pa_bm_free_seq(pa_bm* bm, int64_t seq_id) {
  if (!bm) return fail(PA_ERR_INVALID_ARG, "pa_bm_free_seq: bm is NULL");
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return fail(PA_ERR_UNKNOWN_SEQ, "unknown sequence %lld",
                                        static_cast<long long>(seq_id));
  for (int32_t b : it->second.table)
    if (b >= 0 && --bm->ref[b] == 0) bm->free_stack.push_back(b);
  bm->seqs.erase(it);
  return pa::ok();
}

extern "C" pa_status pa_bm_reorder(pa_bm* bm, const int64_t* old_ids, int32_t num_old,
                                   const int64_t* new_ids, const int32_t* parents,
                                   int32_t num_new) {
  if (!bm) return fail(PA_ERR_INVALID_ARG, "pa_bm_reorder: bm is NULL");
  if (num_old < 0 || num_new < 0 || (num_old > 0 && !old_ids) ||
      (num_new > 0 && (!new_ids || !parents)))
    return fail(PA_ERR_INVALID_ARG, "pa_bm_reorder: bad count or NULL buffer");
  // validate everything first: the call is all-or-nothing
  std::unordered_set<int64_t> olds, news;
  olds.reserve(2 * num_old + 1);
  news.reserve(2 * num_new + 1);
  for (int32_t i = 0; i < num_old; ++i) {
    if (!bm->seqs.count(old_ids[i]))
      return fail(PA_ERR_UNKNOWN_SEQ, "unknown sequence %lld", static_cast<long long>(old_ids[i]));
    if (!olds.insert(old_ids[i]).second)
      return fail(PA_ERR_INVALID_ARG, "pa_bm_reorder: old id %lld repeated",
                  static_cast<long long>(old_ids[i]));
  }
  for (int32_t j = 0; j < num_new; ++j) {
    if (!news.insert(new_ids[j]).second)
      return fail(PA_ERR_INVALID_ARG, "pa_bm_reorder: new id %lld repeated",
                  static_cast<long long>(new_ids[j]));
    if (parents[j] < 0 || parents[j] >= num_old)
      return fail(PA_ERR_INVALID_ARG, "pa_bm_reorder: parent index %d out of range", parents[j]);
    if (new_ids[j] != old_ids[parents[j]] && bm->seqs.count(new_ids[j]))
      return fail(PA_ERR_SEQ_EXISTS, "sequence %lld exists", static_cast<long long>(new_ids[j]));
  }
  // forks first, so blocks of dropped parents stay alive for their children
  for (int32_t j = 0; j < num_new; ++j) {
    const int64_t parent = old_ids[parents[j]];
    if (new_ids[j] == parent) continue;
    pa_bm::Seq child = bm->seqs.find(parent)->second;
    for (int32_t b : child.table)
      if (b >= 0) ++bm->ref[b];
    bm->seqs.emplace(new_ids[j], std::move(child));
  }
  for (int32_t i = 0; i < num_old; ++i) {
    if (news.count(old_ids[i])) continue;
    auto it = bm->seqs.find(old_ids[i]);
    for (int32_t b : it->second.table)
      if (b >= 0 && --bm->ref[b] == 0) bm->free_stack.push_back(b);
    bm->seqs.erase(it);
  }
  return pa::ok();
}

extern "C" pa_status pa_bm_release_before(pa_bm* bm, int64_t seq_id, int32_t first_pos,
                                          int32_t* released_out) {
  if (!bm) return fail(PA_ERR_INVALID_ARG, "pa_bm_release_before: bm is NULL");
  if (first_pos < 0) return fail(PA_ERR_INVALID_ARG, "pa_bm_release_before: first_pos < 0");
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return fail(PA_ERR_UNKNOWN_SEQ, "unknown sequence %lld",
                                        static_cast<long long>(seq_id));
  pa_bm::Seq& s = it->second;
  // blocks k with (k + 1) * block_size <= min(first_pos, len)
  const int32_t whole = std::min(first_pos, s.len) / bm->block_size;
  int32_t n = 0;
  for (int32_t k = 0; k < whole; ++k) {
    const int32_t b = s.table[k];
    if (b < 0) continue;
    if (--bm->ref[b] == 0) bm->free_stack.push_back(b);
    s.table[k] = -1;
    ++n;
  }
  if (released_out) *released_out = n;
  return pa::ok();
}

extern "C" pa_status pa_bm_block_tables(const pa_bm* bm, const int64_t* seq_ids, int32_t n,
                                        int32_t max_blocks, int32_t* tables_out,
                                        int32_t* lens_out) {
  if (!bm) return fail(PA_ERR_INVALID_ARG, "pa_bm_block_tables: bm is NULL");
  if (n < 0 || max_blocks < 0 || (n > 0 && (!seq_ids || !tables_out)))
    return fail(PA_ERR_INVALID_ARG, "pa_bm_block_tables: bad n/max_blocks or NULL buffer");
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end()) return fail(PA_ERR_UNKNOWN_SEQ, "unknown sequence %lld",
                                          static_cast<long long>(seq_ids[i]));
    if (static_cast<int64_t>(it->second.table.size()) > max_blocks)
      return fail(PA_ERR_INVALID_ARG, "sequence %lld has %zu blocks > max_blocks %d",
                  static_cast<long long>(seq_ids[i]), it->second.table.size(), max_blocks);
  }
  for (int32_t i = 0; i < n; ++i) {
    const pa_bm::Seq& s = bm->seqs.find(seq_ids[i])->second;
    int32_t* row = tables_out + static_cast<int64_t>(i) * max_blocks;
    const size_t nb = s.table.size();
    if (nb) std::memcpy(row, s.table.data(), nb * sizeof(int32_t));
    for (int32_t j = static_cast<int32_t>(nb); j < max_blocks; ++j) row[j] = -1;
    if (lens_out) lens_out[i] = s.len;
  }
  return pa::ok();
}

extern "C" pa_status pa_bm_seq_len(const pa_bm* bm, int64_t seq_id, int32_t* len_out) {
  if (!bm || !len_out) return fail(PA_ERR_INVALID_ARG, "pa_bm_seq_len: NULL argument");
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return fail(PA_ERR_UNKNOWN_SEQ, "unknown sequence %lld",
                                        static_cast<long long>(seq_id));
  *len_out = it->second.len;
  return pa::ok();
}

extern "C" pa_status pa_bm_refcount(const pa_bm* bm, int32_t block_id, int32_t* count_out) {
  if (!bm || !count_out) return fail(PA_ERR_INVALID_ARG, "pa_bm_refcount: NULL argument");
  if (block_id < 0 || block_id >= bm->num_blocks)
    return fail(PA_ERR_INVALID_ARG, "pa_bm_refcount: block %d out of range", block_id);
  *count_out = bm->ref[block_id];
  return pa::ok();
}

extern "C" pa_status pa_bm_stats(const pa_bm* bm, pa_bm_stats_t* out) {
  if (!bm || !out) return fail(PA_ERR_INVALID_ARG, "pa_bm_stats: NULL argument");
  pa_bm_stats_t st{};
  st.num_blocks = bm->num_blocks;
  st.free_blocks = static_cast<int32_t>(bm->free_stack.size());
  for (int32_t r : bm->ref) {
    st.used_blocks += r > 0;
    st.shared_blocks += r > 1;
  }
  st.num_seqs = static_cast<int32_t>(bm->seqs.size());
  for (const auto& kv : bm->seqs) {
    st.tokens += kv.second.len;
    st.slack_slots += static_cast<int64_t>(kv.second.table.size()) * bm->block_size -
                      kv.second.len;
  }
  *out = st;
  return pa::ok();
}

// Shared-prefix plan of a decode batch (host).  Sequences whose block tables
// begin with the same physical blocks hold the same tokens there (a block is
// shared only by forks, which share their parent's positions), so their
// queries can attend those blocks together, each block read once.  Sequences
// are grouped by their first physical block, in batch order; a group's
// shared prefix is the longest run of equal entries common to all its
// members, capped so that every member keeps at least one position of its
// own (the step's new token) after it.  Groups with fewer than two members
// or a prefix under min_shared_blocks are dropped.
extern "C" pa_status pa_shared_prefix_plan(const int32_t* tables, const int32_t* lens, int32_t n,
                                           int32_t max_blocks, int32_t block_size,
                                           int32_t min_shared_blocks, int32_t* prefix_len_out,
                                           int32_t* group_rows_out, int32_t* group_start_out,
                                           int32_t* num_groups_out, int32_t* max_group_out) {
  if (n < 0 || max_blocks < 0 || block_size <= 0 || min_shared_blocks < 1)
    return fail(PA_ERR_INVALID_ARG, "pa_shared_prefix_plan: bad sizes");
  if (n > 0 && (!tables || !lens || !prefix_len_out || !group_rows_out || !group_start_out ||
                !num_groups_out || !max_group_out))
    return fail(PA_ERR_INVALID_ARG, "pa_shared_prefix_plan: NULL pointer");
  if (n == 0) {
    if (num_groups_out) *num_groups_out = 0;
    if (max_group_out) *max_group_out = 0;
    if (group_start_out) group_start_out[0] = 0;
    return pa::ok();
  }
  std::vector<int32_t> order;                       // first blocks, in order of appearance
  std::unordered_map<int32_t, std::vector<int32_t>> by_first;
  for (int32_t i = 0; i < n; ++i) {
    prefix_len_out[i] = 0;
    const int64_t L = lens[i];
    if (max_blocks < 1 || L <= static_cast<int64_t>(block_size) * min_shared_blocks) continue;
    const int32_t first = tables[static_cast<int64_t>(i) * max_blocks];
    if (first < 0) continue;
    auto it = by_first.find(first);
    if (it == by_first.end()) {
      order.push_back(first);
      by_first.emplace(first, std::vector<int32_t>{i});
    } else {
      it->second.push_back(i);
    }
  }
  int32_t ng = 0, nrows = 0, max_group = 0;
  group_start_out[0] = 0;
  for (int32_t first : order) {
    const std::vector<int32_t>& m = by_first[first];
    if (m.size() < 2) continue;
    // every member keeps at least one own position after the prefix
    int64_t cap = max_blocks;
    for (int32_t i : m) cap = std::min<int64_t>(cap, (static_cast<int64_t>(lens[i]) - 1) / block_size);
    int64_t P = 0;
    while (P < cap) {
      const int32_t e = tables[static_cast<int64_t>(m[0]) * max_blocks + P];
      if (e < 0) break;
      bool same = true;
      for (size_t k = 1; k < m.size() && same; ++k)
        same = tables[static_cast<int64_t>(m[k]) * max_blocks + P] == e;
      if (!same) break;
      ++P;
    }
    if (P < min_shared_blocks) continue;
    for (int32_t i : m) {
      prefix_len_out[i] = static_cast<int32_t>(P * block_size);
      group_rows_out[nrows++] = i;
    }
    max_group = std::max<int32_t>(max_group, static_cast<int32_t>(m.size()));
    group_start_out[++ng] = nrows;
  }
  *num_groups_out = ng;
  *max_group_out = max_group;
  return pa::ok();
}
