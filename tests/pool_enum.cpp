// Every sequence of at most DEPTH operations from a fixed alphabet, applied to the library's host
// block pool through its C ABI (4 blocks, tables of 3), visited depth first with children in
// alphabet order. After each operation the outcome (status, the call's results, the statistics,
// every live sequence's length and table) is folded into a 64-bit FNV-1a hash over 64-bit words,
// exactly as tests/golden/make_pool_enum.py does with the oracle's pool model. Prints
// "nodes <n per depth...> failed <n> fnv1a64 <hex>"; exit status 0 unless a call broke the
// pool's invariants (kvc_check).
// Usage: pool_enum <depth>
#include <cinttypes>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "kvc.h"

namespace {

constexpr int32_t kBlocks = 4, kMaxBlocks = 3;
constexpr uint64_t kOffset = 0xCBF29CE484222325ull, kPrime = 0x100000001B3ull;

enum Kind { ALLOC, APPEND, FORK, FREE, SLIDE };
struct Op {
  Kind kind;
  std::vector<int> idx;  // append / slide: indices into the live list
  int n;                 // append: tokens; slide: window; fork / free: live index
};

// the alphabet of tests/golden/make_pool_enum.py, in the same order
const std::vector<Op> kAlphabet = {
    {ALLOC, {}, 0},         {APPEND, {0}, 1},       {APPEND, {0}, 15},   {APPEND, {0}, 17},
    {APPEND, {0, 1}, 1},    {APPEND, {1, 0}, 9},    {FORK, {}, 0},       {FORK, {}, 1},
    {FREE, {}, 0},          {FREE, {}, 1},          {SLIDE, {0}, 3},     {SLIDE, {1, 0}, 17}};

struct State {
  kvc_pool *pool = nullptr;
  std::vector<int32_t> live;
};

uint64_t g_hash = kOffset;
std::vector<long long> g_nodes;
long long g_failed = 0;
bool g_broken = false;

void fold(std::vector<int64_t> &w) {
  for (int64_t v : w) {
    g_hash ^= static_cast<uint64_t>(v);
    g_hash *= kPrime;
  }
}

std::vector<int32_t> pick(const State &s, const std::vector<int> &idx) {
  std::vector<int32_t> seqs;
  if (s.live.empty()) return {0};
  for (int i : idx) seqs.push_back(s.live[i % s.live.size()]);
  return seqs;
}

// Apply one operation; fills the result words (status first).
void apply(State &s, const Op &op, std::vector<int64_t> &res) {
  res.clear();
  kvc_status st = KVC_OK;
  std::vector<int64_t> out;
  if (op.kind == ALLOC) {
    int32_t id = -1;
    st = kvc_alloc(s.pool, &id);
    if (st == KVC_OK) {
      out.push_back(id);
      s.live.push_back(id);
    }
  } else if (op.kind == APPEND) {
    const std::vector<int32_t> seqs = pick(s, op.idx);
    const int32_t n = static_cast<int32_t>(seqs.size());
    std::vector<int64_t> slots(static_cast<size_t>(n) * op.n + 1);
    std::vector<int32_t> src(n), dst(n);
    int32_t ncow = 0;
    st = kvc_append(s.pool, seqs.data(), n, op.n, slots.data(), src.data(), dst.data(), n, &ncow);
    if (st == KVC_OK) {
      out.push_back(static_cast<int64_t>(n) * op.n);
      for (int64_t i = 0; i < static_cast<int64_t>(n) * op.n; ++i) out.push_back(slots[i]);
      out.push_back(ncow);
      for (int32_t i = 0; i < ncow; ++i) {
        out.push_back(src[i]);
        out.push_back(dst[i]);
      }
    }
  } else if (op.kind == FORK) {
    const int32_t p = s.live.empty() ? 7 : s.live[op.n % s.live.size()];
    int32_t c = -1;
    st = kvc_fork(s.pool, p, &c);
    if (st == KVC_OK) {
      out.push_back(c);
      s.live.push_back(c);
    }
  } else if (op.kind == FREE) {
    const int32_t p = s.live.empty() ? 7 : s.live[op.n % s.live.size()];
    st = kvc_free(s.pool, p);
    if (st == KVC_OK) {
      std::vector<int32_t> keep;
      for (int32_t x : s.live)
        if (x != p) keep.push_back(x);
      s.live = keep;
    }
  } else {
    const std::vector<int32_t> seqs = pick(s, op.idx);
    int32_t dropped = 0;
    st = kvc_slide(s.pool, seqs.data(), static_cast<int32_t>(seqs.size()), op.n, &dropped);
    if (st == KVC_OK) out.push_back(dropped);
  }
  res.push_back(st);
  res.insert(res.end(), out.begin(), out.end());
}

void outcome(const State &s, int depth, int op_i, const std::vector<int64_t> &res,
             std::vector<int64_t> &w) {
  w.clear();
  w.push_back(depth);
  w.push_back(op_i);
  w.insert(w.end(), res.begin(), res.end());
  kvc_pool_stats st{};
  if (kvc_stats(s.pool, &st) != KVC_OK) g_broken = true;
  for (int64_t v : {static_cast<int64_t>(st.num_blocks), static_cast<int64_t>(st.used),
                    static_cast<int64_t>(st.free_blocks), static_cast<int64_t>(st.shared),
                    static_cast<int64_t>(st.num_seqs), st.cow_copies, st.tokens,
                    st.slots_logical, static_cast<int64_t>(s.live.size())})
    w.push_back(v);
  if (!s.live.empty()) {
    std::vector<int32_t> tables(s.live.size() * kMaxBlocks), lens(s.live.size());
    if (kvc_block_table(s.pool, s.live.data(), static_cast<int32_t>(s.live.size()),
                        tables.data(), lens.data()) != KVC_OK)
      g_broken = true;
    for (size_t i = 0; i < s.live.size(); ++i) {
      w.push_back(lens[i]);
      for (int k = 0; k < kMaxBlocks; ++k) w.push_back(tables[i * kMaxBlocks + k]);
    }
  }
}

// A fresh pool with the operations of `path` applied.
State replay(const std::vector<int> &path) {
  State s;
  if (kvc_pool_create(kBlocks, KVC_BLOCK_SIZE, kMaxBlocks, nullptr, &s.pool) != KVC_OK) {
    std::fprintf(stderr, "kvc_pool_create failed\n");
    std::exit(2);
  }
  std::vector<int64_t> res;
  for (int i : path) apply(s, kAlphabet[i], res);
  return s;
}

void visit(std::vector<int> &path, int depth, int max_depth) {
  std::vector<int64_t> res, w;
  for (int op_i = 0; op_i < static_cast<int>(kAlphabet.size()); ++op_i) {
    State s = replay(path);
    apply(s, kAlphabet[op_i], res);
    if (kvc_check(s.pool) != KVC_OK) g_broken = true;
    outcome(s, depth, op_i, res, w);
    fold(w);
    ++g_nodes[depth];
    g_failed += res[0] != KVC_OK;
    kvc_pool_destroy(s.pool);
    if (depth < max_depth) {
      path.push_back(op_i);
      visit(path, depth + 1, max_depth);
      path.pop_back();
    }
  }
}

}  // namespace

int main(int argc, char **argv) {
  const int depth = argc > 1 ? std::atoi(argv[1]) : 6;
  if (depth < 1 || depth > 8) return 2;
  g_nodes.assign(depth + 1, 0);
  std::vector<int> path;
  visit(path, 1, depth);
  std::printf("nodes");
  for (int d = 1; d <= depth; ++d) std::printf(" %lld", g_nodes[d]);
  std::printf(" failed %lld fnv1a64 %016" PRIx64 "\n", g_failed, g_hash);
  return g_broken ? 1 : 0;
}
