// Host-only driver for the block pool under AddressSanitizer and
// UndefinedBehaviorSanitizer: random forks, appends (with copy on write) and
// releases against a reference-count model, plus every error path; exits
// non-zero on the first disagreement.  Built with g++ by
// tests/test_sanitize_pool.py (no GPU code is involved).
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "mi_attn.h"

namespace mi_attn {
// the library keeps this buffer in its C-ABI translation unit; the driver
// links the pool alone
char* error_buffer() {
  static thread_local char buf[512];
  return buf;
}
}  // namespace mi_attn

#define CHECK(c)                                                  \
  do {                                                            \
    if (!(c)) {                                                   \
      std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
      std::exit(1);                                               \
    }                                                             \
  } while (0)

int main() {
  const int NB = 96, BS = 16, MAXB = 10;
  attn_pool* p = nullptr;
  CHECK(attn_pool_create(NB, BS, &p) == ATTN_OK && p);
  std::vector<int> ref(NB, 0);
  struct Seq {
    std::vector<int32_t> row;
    int len;
  };
  std::vector<Seq> seqs;
  std::mt19937 g(7);
  auto blocks = [&](int len) { return (len + BS - 1) / BS; };
  for (int step = 0; step < 4000; ++step) {
    const int op = (int)(g() % 4);
    if (op == 0 || seqs.empty()) {
      Seq s{std::vector<int32_t>(MAXB, -1), 1 + (int)(g() % 80)};
      std::vector<int32_t> slots(s.len);
      if (attn_seq_reserve(p, s.row.data(), MAXB, 0, s.len, slots.data()) != ATTN_OK) continue;
      for (int b = 0; b < blocks(s.len); ++b) ref[s.row[b]]++;
      seqs.push_back(s);
    } else if (op == 1) {
      const Seq& par = seqs[g() % seqs.size()];
      Seq c{std::vector<int32_t>(MAXB, -1), (int)(g() % (par.len + 1))};
      CHECK(attn_seq_fork(p, par.row.data(), c.len, c.row.data(), MAXB) == ATTN_OK);
      for (int b = 0; b < blocks(c.len); ++b) ref[c.row[b]]++;
      seqs.push_back(c);
    } else if (op == 2) {
      Seq& s = seqs[g() % seqs.size()];
      const int k = 1 + (int)(g() % 40);
      if (blocks(s.len + k) > MAXB) continue;
      std::vector<int32_t> before = s.row, slots(k);
      int32_t pair[2];
      const int st = attn_seq_reserve_cow(p, s.row.data(), MAXB, s.len, k, slots.data(), pair);
      if (st != ATTN_OK) {
        CHECK(st == ATTN_E_NOMEM && s.row == before);
        continue;
      }
      if (pair[0] >= 0) {
        ref[pair[0]]--;
        ref[pair[1]]++;
      }
      for (int b = blocks(s.len); b < blocks(s.len + k); ++b) ref[s.row[b]]++;
      CHECK(attn_pool_refcount(p, s.row[s.len / BS]) == 1);
      for (int i = 0; i < k; ++i) CHECK(slots[i] == s.row[(s.len + i) / BS] * BS + (s.len + i) % BS);
      s.len += k;
    } else {
      const size_t i = g() % seqs.size();
      CHECK(attn_pool_free(p, seqs[i].row.data(), blocks(seqs[i].len)) == ATTN_OK);
      for (int b = 0; b < blocks(seqs[i].len); ++b) ref[seqs[i].row[b]]--;
      seqs.erase(seqs.begin() + (long)i);
    }
    int nfree = 0;
    for (int id = 0; id < NB; ++id) {
      CHECK(attn_pool_refcount(p, id) == ref[id]);
      nfree += ref[id] == 0;
    }
    CHECK(attn_pool_num_free(p) == nfree);
  }
  // error paths: nothing changes on any of them
  int32_t ids[4] = {0, 1, 2, 3};
  int32_t bad[2] = {NB, -1};
  CHECK(attn_pool_free(p, bad, 2) == ATTN_E_INVALID);
  CHECK(attn_pool_retain(p, bad, 1) == ATTN_E_INVALID);
  CHECK(attn_pool_alloc(p, NB + 1, ids) == ATTN_E_NOMEM);
  CHECK(attn_pool_alloc(nullptr, 1, ids) == ATTN_E_INVALID);
  CHECK(attn_seq_fork(p, nullptr, 4, ids, 4) == ATTN_E_INVALID);
  CHECK(attn_seq_reserve_cow(p, ids, 4, 0, 1, nullptr, nullptr) == ATTN_E_INVALID);
  CHECK(attn_pool_refcount(p, NB) == ATTN_E_INVALID);
  for (const Seq& s : seqs) CHECK(attn_pool_free(p, s.row.data(), blocks(s.len)) == ATTN_OK);
  CHECK(attn_pool_num_free(p) == NB);
  int32_t one = 0;
  CHECK(attn_pool_free(p, &one, 1) == ATTN_E_STATE);   // double free
  attn_pool_destroy(p);
  std::printf("pool driver: ok\n");
  return 0;
}
