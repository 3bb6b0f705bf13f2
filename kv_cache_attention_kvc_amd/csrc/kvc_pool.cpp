// Host-side block pool of the paged KV cache: first-fit allocation, reference counts, fork and
// copy-on-write ("KV Cache and PagedAttention", sections 2.1, 2.2, 3.1, 3.3 and 5.1), and the
// rolling window in paged form ("KV Cache Mechanism Explained", section 8, item 2): blocks wholly
// before a sequence's window are dropped from its table (entry -1), a prefix of the table.
//
// Host memory only; no HIP calls. Free blocks are kept in a bitmap indexed by position in the
// pool's search order, so first fit is "lowest set bit at or after a hint". Every mutating call
// either succeeds or restores the pool from an undo journal (strong guarantee).
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <new>
#include <set>
#include <vector>

#include "kvc.h"

namespace {

struct Seq {
  bool live = false;
  int32_t len = 0;
  std::vector<int32_t> table;
};

}  // namespace

struct kvc_pool {
  int32_t num_blocks = 0;
  int32_t max_blocks = 0;
  std::vector<int32_t> order;   // position -> block id (first-fit search order)
  std::vector<int32_t> pos_of;  // block id -> position in order
  std::vector<int32_t> refcount;
  std::vector<uint64_t> free_bits;  // bit p set <=> block order[p] is free
  int32_t hint_word = 0;            // no free bit below this word
  std::vector<Seq> seqs;
  std::set<int32_t> free_ids;  // ids below seqs.size() that are not live
  int32_t live_count = 0;
  int64_t cow_copies = 0;

  void mark_free(int32_t blk) {
    const int32_t p = pos_of[blk];
    free_bits[p >> 6] |= (uint64_t{1} << (p & 63));
    hint_word = std::min(hint_word, p >> 6);
  }
  void mark_used(int32_t blk) {
    const int32_t p = pos_of[blk];
    free_bits[p >> 6] &= ~(uint64_t{1} << (p & 63));
  }
  // First free block in pool order, or -1.
  int32_t first_fit() {
    const int32_t words = static_cast<int32_t>(free_bits.size());
    for (int32_t w = hint_word; w < words; ++w) {
      if (free_bits[w]) {
        hint_word = w;
        const int32_t p = (w << 6) + __builtin_ctzll(free_bits[w]);
        return order[p];
      }
    }
    hint_word = words;
    return -1;
  }
  void set_refcount(int32_t blk, int32_t v) {
    const int32_t old = refcount[blk];
    refcount[blk] = v;
    if (old == 0 && v != 0) mark_used(blk);
    if (old != 0 && v == 0) mark_free(blk);
  }
  bool is_live(int32_t s) const {
    return s >= 0 && s < static_cast<int32_t>(seqs.size()) && seqs[s].live;
  }
  int32_t new_seq_id() {
    if (!free_ids.empty()) {
      const int32_t id = *free_ids.begin();
      free_ids.erase(free_ids.begin());
      return id;
    }
    seqs.emplace_back();
    return static_cast<int32_t>(seqs.size()) - 1;
  }
};

extern "C" {

const char *kvc_status_str(kvc_status s) {
  switch (s) {
    case KVC_OK: return "ok";
    case KVC_E_INVALID: return "invalid argument";
    case KVC_E_OOM: return "out of blocks";
    case KVC_E_NOSEQ: return "no such sequence";
    case KVC_E_CAPACITY: return "block table full";
    case KVC_E_UNSUPPORTED: return "unsupported combination";
    case KVC_E_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

kvc_status kvc_pool_create(int32_t num_blocks, int32_t block_size, int32_t max_blocks_per_seq,
                           const int32_t *order, kvc_pool **out) {
  if (!out || num_blocks < 1 || block_size != KVC_BLOCK_SIZE || max_blocks_per_seq < 1 ||
      num_blocks > (INT32_MAX / KVC_BLOCK_SIZE) || max_blocks_per_seq > (INT32_MAX / KVC_BLOCK_SIZE))
    return KVC_E_INVALID;
  kvc_pool *p = nullptr;
  try {
    p = new kvc_pool();
    p->num_blocks = num_blocks;
    p->max_blocks = max_blocks_per_seq;
    p->order.resize(num_blocks);
    p->pos_of.assign(num_blocks, -1);
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t b = order ? order[i] : i;
      if (b < 0 || b >= num_blocks || p->pos_of[b] != -1) {
        delete p;
        return KVC_E_INVALID;
      }
      p->order[i] = b;
      p->pos_of[b] = i;
    }
    p->refcount.assign(num_blocks, 0);
    p->free_bits.assign((num_blocks + 63) / 64, 0);
    for (int32_t i = 0; i < num_blocks; ++i) p->free_bits[i >> 6] |= uint64_t{1} << (i & 63);
  } catch (const std::bad_alloc &) {
    delete p;
    return KVC_E_OOM;
  }
  *out = p;
  return KVC_OK;
}

void kvc_pool_destroy(kvc_pool *pool) { delete pool; }

kvc_status kvc_alloc(kvc_pool *pool, int32_t *seq_out) {
  if (!pool || !seq_out) return KVC_E_INVALID;
  try {
    const int32_t id = pool->new_seq_id();
    Seq &s = pool->seqs[id];
    s.live = true;
    s.len = 0;
    s.table.clear();
    pool->live_count++;
    *seq_out = id;
  } catch (const std::bad_alloc &) {
    return KVC_E_OOM;
  }
  return KVC_OK;
}

kvc_status kvc_append(kvc_pool *pool, const int32_t *seqs, int32_t n_seqs, int32_t n_tokens,
                      int64_t *slots_out, int32_t *cow_src_out, int32_t *cow_dst_out,
                      int32_t cow_cap, int32_t *n_cow_out) {
  if (!pool || n_seqs < 0 || n_tokens < 0 || !n_cow_out) return KVC_E_INVALID;
  if (n_seqs > 0 && !seqs) return KVC_E_INVALID;
  if (n_seqs > 0 && n_tokens > 0 && !slots_out) return KVC_E_INVALID;
  if (cow_cap < n_seqs) return KVC_E_INVALID;
  if (n_seqs > 0 && (!cow_src_out || !cow_dst_out)) return KVC_E_INVALID;
  for (int32_t i = 0; i < n_seqs; ++i)
    if (!pool->is_live(seqs[i])) return KVC_E_NOSEQ;

  struct SeqSnap {
    int32_t id, len;
    std::vector<int32_t> table;
  };
  std::vector<SeqSnap> seq_log;                      // first-touch snapshot of each sequence
  std::vector<std::pair<int32_t, int32_t>> rc_log;  // (block, refcount before change)
  const int64_t cow_before = pool->cow_copies;
  int32_t n_cow = 0;
  kvc_status st = KVC_OK;
  try {
    std::vector<char> touched(pool->seqs.size(), 0);
    int64_t k = 0;
    for (int32_t i = 0; i < n_seqs && st == KVC_OK; ++i) {
      const int32_t sid = seqs[i];
      Seq &s = pool->seqs[sid];
      if (!touched[sid]) {
        touched[sid] = 1;
        seq_log.push_back({sid, s.len, s.table});
      }
      for (int32_t t = 0; t < n_tokens; ++t) {
        const int32_t L = s.len;
        const int32_t idx = L / KVC_BLOCK_SIZE;
        const int32_t off = L % KVC_BLOCK_SIZE;
        int32_t blk;
        if (off == 0) {
          if (idx >= pool->max_blocks) { st = KVC_E_CAPACITY; break; }
          blk = pool->first_fit();
          if (blk < 0) { st = KVC_E_OOM; break; }
          rc_log.emplace_back(blk, pool->refcount[blk]);
          pool->set_refcount(blk, 1);
          s.table.push_back(blk);
        } else {
          blk = s.table[idx];
          if (pool->refcount[blk] > 1) {
            const int32_t nb = pool->first_fit();
            if (nb < 0) { st = KVC_E_OOM; break; }
            rc_log.emplace_back(nb, pool->refcount[nb]);
            pool->set_refcount(nb, 1);
            rc_log.emplace_back(blk, pool->refcount[blk]);
            pool->set_refcount(blk, pool->refcount[blk] - 1);
            s.table[idx] = nb;
            cow_src_out[n_cow] = blk;
            cow_dst_out[n_cow] = nb;
            ++n_cow;
            pool->cow_copies++;
            blk = nb;
          }
        }
        slots_out[k++] = static_cast<int64_t>(blk) * KVC_BLOCK_SIZE + off;
        s.len = L + 1;
      }
    }
  } catch (const std::bad_alloc &) {
    st = KVC_E_OOM;
  }
  if (st != KVC_OK) {
    for (auto it = rc_log.rbegin(); it != rc_log.rend(); ++it) pool->set_refcount(it->first, it->second);
    for (auto &snap : seq_log) {
      Seq &s = pool->seqs[snap.id];
      s.len = snap.len;
      s.table.swap(snap.table);
    }
    pool->cow_copies = cow_before;
    return st;
  }
  *n_cow_out = n_cow;
  return KVC_OK;
}

kvc_status kvc_fork(kvc_pool *pool, int32_t parent, int32_t *child_out) {
  if (!pool || !child_out) return KVC_E_INVALID;
  if (!pool->is_live(parent)) return KVC_E_NOSEQ;
  for (int32_t b : pool->seqs[parent].table)
    if (b >= 0 && pool->refcount[b] == INT32_MAX) return KVC_E_INVALID;
  try {
    std::vector<int32_t> table = pool->seqs[parent].table;  // copy before any change
    const int32_t len = pool->seqs[parent].len;
    const int32_t id = pool->new_seq_id();
    Seq &c = pool->seqs[id];
    c.live = true;
    c.len = len;
    c.table.swap(table);
    for (int32_t b : c.table)
      if (b >= 0) pool->set_refcount(b, pool->refcount[b] + 1);
    pool->live_count++;
    *child_out = id;
  } catch (const std::bad_alloc &) {
    return KVC_E_OOM;
  }
  return KVC_OK;
}

kvc_status kvc_free(kvc_pool *pool, int32_t seq) {
  if (!pool) return KVC_E_INVALID;
  if (!pool->is_live(seq)) return KVC_E_NOSEQ;
  try {
    pool->free_ids.insert(seq);
  } catch (const std::bad_alloc &) {
    return KVC_E_OOM;
  }
  Seq &s = pool->seqs[seq];
  for (int32_t b : s.table)
    if (b >= 0) pool->set_refcount(b, pool->refcount[b] - 1);
  s.live = false;
  s.len = 0;
  std::vector<int32_t>().swap(s.table);
  pool->live_count--;
  return KVC_OK;
}

kvc_status kvc_slide(kvc_pool *pool, const int32_t *seqs, int32_t n_seqs, int32_t window,
                     int32_t *n_dropped_out) {
  if (!pool || n_seqs < 0 || window < 0) return KVC_E_INVALID;
  if (n_seqs > 0 && !seqs) return KVC_E_INVALID;
  for (int32_t i = 0; i < n_seqs; ++i)
    if (!pool->is_live(seqs[i])) return KVC_E_NOSEQ;
  int32_t dropped = 0;
  if (window > 0) {
    for (int32_t i = 0; i < n_seqs; ++i) {
      Seq &s = pool->seqs[seqs[i]];
      const int32_t start = std::max(0, s.len - window);
      const int32_t n = std::min<int32_t>(start / KVC_BLOCK_SIZE,
                                          static_cast<int32_t>(s.table.size()));
      for (int32_t j = 0; j < n; ++j) {
        const int32_t b = s.table[j];
        if (b < 0) continue;
        pool->set_refcount(b, pool->refcount[b] - 1);
        s.table[j] = -1;
        ++dropped;
      }
    }
  }
  if (n_dropped_out) *n_dropped_out = dropped;
  return KVC_OK;
}

kvc_status kvc_block_table(const kvc_pool *pool, const int32_t *seqs, int32_t n_seqs,
                           int32_t *tables_out, int32_t *lens_out) {
  if (!pool || n_seqs < 0) return KVC_E_INVALID;
  if (n_seqs > 0 && (!seqs || !tables_out)) return KVC_E_INVALID;
  for (int32_t i = 0; i < n_seqs; ++i)
    if (!pool->is_live(seqs[i])) return KVC_E_NOSEQ;
  const int64_t mb = pool->max_blocks;
  for (int32_t i = 0; i < n_seqs; ++i) {
    const Seq &s = pool->seqs[seqs[i]];
    int32_t *row = tables_out + i * mb;
    const int64_t n = static_cast<int64_t>(s.table.size());
    if (n) std::memcpy(row, s.table.data(), n * sizeof(int32_t));
    for (int64_t j = n; j < mb; ++j) row[j] = -1;
    if (lens_out) lens_out[i] = s.len;
  }
  return KVC_OK;
}

kvc_status kvc_stats(const kvc_pool *pool, kvc_pool_stats *out) {
  if (!pool || !out) return KVC_E_INVALID;
  kvc_pool_stats st{};
  st.num_blocks = pool->num_blocks;
  for (int32_t r : pool->refcount) {
    if (r > 0) st.used++;
    if (r > 1) st.shared++;
  }
  st.free_blocks = pool->num_blocks - st.used;
  st.num_seqs = pool->live_count;
  st.cow_copies = pool->cow_copies;
  for (const Seq &s : pool->seqs) {
    if (!s.live) continue;
    st.tokens += s.len;
    for (int32_t b : s.table)
      if (b >= 0) st.slots_logical += KVC_BLOCK_SIZE;
  }
  *out = st;
  return KVC_OK;
}

kvc_status kvc_check(const kvc_pool *pool) {
  if (!pool) return KVC_E_INVALID;
  try {
    std::vector<int32_t> refs(pool->num_blocks, 0);
    std::vector<int32_t> seen(pool->num_blocks, -1);
    int32_t live = 0;
    for (size_t sid = 0; sid < pool->seqs.size(); ++sid) {
      const Seq &s = pool->seqs[sid];
      if (!s.live) {
        if (!pool->free_ids.count(static_cast<int32_t>(sid))) return KVC_E_INVALID;
        continue;
      }
      live++;
      const int64_t need = (static_cast<int64_t>(s.len) + KVC_BLOCK_SIZE - 1) / KVC_BLOCK_SIZE;
      if (s.len < 0 || static_cast<int64_t>(s.table.size()) != need ||
          need > pool->max_blocks)
        return KVC_E_INVALID;
      size_t k = 0;  // entries dropped by a rolling window form a prefix
      while (k < s.table.size() && s.table[k] == -1) ++k;
      for (size_t j = k; j < s.table.size(); ++j) {
        const int32_t b = s.table[j];
        if (b < 0 || b >= pool->num_blocks) return KVC_E_INVALID;
        if (seen[b] == static_cast<int32_t>(sid)) return KVC_E_INVALID;
        seen[b] = static_cast<int32_t>(sid);
        refs[b]++;
      }
    }
    if (live != pool->live_count) return KVC_E_INVALID;
    for (int32_t b = 0; b < pool->num_blocks; ++b) {
      if (refs[b] != pool->refcount[b]) return KVC_E_INVALID;
      const int32_t p = pool->pos_of[b];
      const bool bit = (pool->free_bits[p >> 6] >> (p & 63)) & 1;
      if (bit != (refs[b] == 0)) return KVC_E_INVALID;
    }
  } catch (const std::bad_alloc &) {
    return KVC_E_OOM;
  }
  return KVC_OK;
}

}  // extern "C"
