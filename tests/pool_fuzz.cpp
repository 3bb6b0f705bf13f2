// Randomised operation sequences against the host block pool's C ABI, for sanitizer builds.
// After every call the pool's invariants must hold (kvc_check), statistics must be consistent,
// a call that fails must leave every live sequence's table and length unchanged, and a rolling-
// window slide may only drop blocks that lie wholly before the window.
// Usage: pool_fuzz <seeds> <ops-per-seed>; exit status 0 on success.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "kvc.h"

namespace {

struct Rng {
  uint64_t s;
  explicit Rng(uint64_t seed) : s(seed * 0x9E3779B97F4A7C15ull + 1) {}
  uint32_t next() {
    s ^= s << 13;
    s ^= s >> 7;
    s ^= s << 17;
    return static_cast<uint32_t>(s >> 11);
  }
  int below(int n) { return static_cast<int>(next() % static_cast<uint32_t>(n)); }
};

#define FAIL(...)                     \
  do {                                \
    std::fprintf(stderr, __VA_ARGS__); \
    std::fprintf(stderr, "\n");       \
    return false;                     \
  } while (0)

bool snapshot(kvc_pool *p, const std::vector<int32_t> &live, int32_t mb,
              std::vector<int32_t> &tables, std::vector<int32_t> &lens) {
  tables.assign(live.size() * mb, 0);
  lens.assign(live.size(), 0);
  if (live.empty()) return true;
  return kvc_block_table(p, live.data(), static_cast<int32_t>(live.size()), tables.data(),
                         lens.data()) == KVC_OK;
}

bool run(uint64_t seed, int ops) {
  Rng r(seed);
  const int32_t nblk = 1 + r.below(48);
  const int32_t mb = 1 + r.below(8);
  std::vector<int32_t> order(nblk);
  for (int32_t i = 0; i < nblk; ++i) order[i] = i;
  if (r.below(2))
    for (int32_t i = nblk - 1; i > 0; --i) std::swap(order[i], order[r.below(i + 1)]);
  kvc_pool *p = nullptr;
  if (kvc_pool_create(nblk, KVC_BLOCK_SIZE, mb, order.data(), &p) != KVC_OK) FAIL("create");
  std::vector<int32_t> live;
  std::vector<int64_t> slots;
  std::vector<int32_t> src, dst, t0, l0, t1, l1;
  for (int op = 0; op < ops; ++op) {
    if (!snapshot(p, live, mb, t0, l0)) FAIL("snapshot");
    const int kind = live.empty() ? 0 : r.below(11);
    kvc_status st = KVC_OK;
    if (kind < 2) {
      int32_t s = -1;
      st = kvc_alloc(p, &s);
      if (st == KVC_OK) live.push_back(s);
    } else if (kind < 6) {
      const int32_t n = 1 + r.below(4);
      std::vector<int32_t> seqs(n);
      for (auto &s : seqs) s = r.below(5) ? live[r.below(static_cast<int>(live.size()))] : 1000;
      const int32_t tok = r.below(40);
      slots.assign(static_cast<size_t>(n) * tok + 1, 0);
      src.assign(n, 0);
      dst.assign(n, 0);
      int32_t ncow = -1;
      st = kvc_append(p, seqs.data(), n, tok, slots.data(), src.data(), dst.data(), n, &ncow);
      if (st == KVC_OK) {
        if (ncow < 0 || ncow > n) FAIL("seed %llu op %d: cow count %d", (unsigned long long)seed, op, ncow);
        for (int64_t k = 0; k < static_cast<int64_t>(n) * tok; ++k)
          if (slots[k] < 0 || slots[k] >= static_cast<int64_t>(nblk) * KVC_BLOCK_SIZE)
            FAIL("seed %llu op %d: slot out of range", (unsigned long long)seed, op);
      }
    } else if (kind < 8) {
      int32_t c = -1;
      st = kvc_fork(p, live[r.below(static_cast<int>(live.size()))], &c);
      if (st == KVC_OK) live.push_back(c);
    } else if (kind < 10) {
      const int idx = r.below(static_cast<int>(live.size()));
      st = kvc_free(p, live[idx]);
      if (st == KVC_OK) live.erase(live.begin() + idx);
    } else {
      // rolling window: a slide drops only leading blocks, never a position inside the window
      const int32_t n = 1 + r.below(3);
      std::vector<int32_t> seqs(n);
      for (auto &s : seqs) s = live[r.below(static_cast<int>(live.size()))];
      const int32_t window = r.below(60);
      int32_t dropped = -1;
      st = kvc_slide(p, seqs.data(), n, window, &dropped);
      if (st != KVC_OK || dropped < 0) FAIL("seed %llu op %d: slide", (unsigned long long)seed, op);
      if (!snapshot(p, live, mb, t1, l1)) FAIL("snapshot");
      for (size_t i = 0; i < live.size(); ++i)
        for (int32_t j = 0; j < mb; ++j) {
          const int32_t before = t0[i * mb + j], after = t1[i * mb + j];
          const int32_t start = window ? std::max(0, l1[i] - window) : 0;
          if (after != before && (after != -1 || (j + 1) * KVC_BLOCK_SIZE > start))
            FAIL("seed %llu op %d: slide changed a block inside the window",
                 (unsigned long long)seed, op);
        }
    }
    if (kvc_check(p) != KVC_OK) FAIL("seed %llu op %d: invariants broken", (unsigned long long)seed, op);
    kvc_pool_stats stt{};
    if (kvc_stats(p, &stt) != KVC_OK || stt.used + stt.free_blocks != nblk ||
        stt.num_seqs != static_cast<int32_t>(live.size()))
      FAIL("seed %llu op %d: stats", (unsigned long long)seed, op);
    if (st != KVC_OK) {
      if (st != KVC_E_OOM && st != KVC_E_CAPACITY && st != KVC_E_NOSEQ)
        FAIL("seed %llu op %d: unexpected status %d", (unsigned long long)seed, op, st);
      if (!snapshot(p, live, mb, t1, l1) || t0 != t1 || l0 != l1)
        FAIL("seed %llu op %d: failed call changed the pool", (unsigned long long)seed, op);
    }
  }
  // error paths that never change state
  int32_t dummy = 0;
  if (kvc_free(p, -1) != KVC_E_NOSEQ || kvc_fork(p, 1 << 20, &dummy) != KVC_E_NOSEQ)
    FAIL("seed %llu: bad ids accepted", (unsigned long long)seed);
  for (int32_t s : live)
    if (kvc_free(p, s) != KVC_OK) FAIL("seed %llu: free", (unsigned long long)seed);
  kvc_pool_stats stt{};
  kvc_stats(p, &stt);
  if (stt.used != 0 || kvc_check(p) != KVC_OK) FAIL("seed %llu: leak after freeing all", (unsigned long long)seed);
  kvc_pool_destroy(p);
  return true;
}

}  // namespace

int main(int argc, char **argv) {
  const int seeds = argc > 1 ? std::atoi(argv[1]) : 50;
  const int ops = argc > 2 ? std::atoi(argv[2]) : 400;
  for (int s = 0; s < seeds; ++s)
    if (!run(static_cast<uint64_t>(s), ops)) return 1;
  std::printf("pool_fuzz: %d seeds x %d operations ok\n", seeds, ops);
  return 0;
}
