// Host-only driver for the block pool under ThreadSanitizer.  The pool is
// documented as not thread-safe: callers serialise access to one pool.  This
// driver keeps that rule and checks that nothing else is shared behind the
// caller's back (no hidden global or static state in the pool, the error
// text per thread):
//   * eight threads, each with pools of its own, fork, grow (with copy on
//     write) and release sequences, and check the free count and reference
//     counts against a model of their own;
//   * the same threads share one more pool, every call on it made under one
//     mutex, and hand blocks to each other through it;
//   * every thread provokes errors and reads its own error text.
// Exits non-zero on the first disagreement; ThreadSanitizer reports (and
// fails the run on) any data race.  Built with g++ by
// tests/test_sanitize_pool.py (no GPU code is involved).
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <random>
#include <thread>
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

extern "C" const char* attn_last_error(void) { return mi_attn::error_buffer(); }

#define CHECK(c)                                                                      \
  do {                                                                                \
    if (!(c)) {                                                                       \
      std::fprintf(stderr, "thread check failed line %d: %s\n", __LINE__, #c);        \
      std::exit(1);                                                                   \
    }                                                                                 \
  } while (0)

namespace {

constexpr int kThreads = 8;
constexpr int kRounds = 300;

std::mutex shared_mu;
attn_pool* shared_pool = nullptr;

// One thread's private work: a pool, sequences that grow, fork and end, and a
// model of the reference counts.
void private_work(int t) {
  const int NB = 64, BS = 16, MAXB = 8;
  attn_pool* p = nullptr;
  CHECK(attn_pool_create(NB, BS, &p) == ATTN_OK);
  std::vector<int> ref(NB, 0);
  struct Seq {
    std::vector<int32_t> row;
    int len;
  };
  std::vector<Seq> seqs;
  std::mt19937 g(1000 + t);
  for (int it = 0; it < kRounds; ++it) {
    const int op = (int)(g() % 4);
    if (op == 0 || seqs.empty()) {  // new sequence
      Seq s{std::vector<int32_t>(MAXB, -1), 0};
      const int n = 1 + (int)(g() % 40);
      if (attn_seq_reserve(p, s.row.data(), MAXB, 0, n, nullptr) == ATTN_OK) {
        for (int b = 0; b < (n + BS - 1) / BS; ++b) ref[s.row[b]]++;
        s.len = n;
        seqs.push_back(s);
      }
    } else if (op == 1) {  // fork
      const Seq& par = seqs[g() % seqs.size()];
      Seq c{std::vector<int32_t>(MAXB, -1), par.len};
      CHECK(attn_seq_fork(p, par.row.data(), par.len, c.row.data(), MAXB) == ATTN_OK);
      for (int b = 0; b < (par.len + BS - 1) / BS; ++b) ref[c.row[b]]++;
      seqs.push_back(c);
    } else if (op == 2) {  // grow with copy on write
      Seq& s = seqs[g() % seqs.size()];
      const int n = 1 + (int)(g() % 20);
      if (s.len + n > MAXB * BS) continue;
      int32_t pair[2];
      const int before = (s.len + BS - 1) / BS;
      std::vector<int32_t> old = s.row;
      const int rc = attn_seq_reserve_cow(p, s.row.data(), MAXB, s.len, n, nullptr, pair);
      if (rc == ATTN_E_NOMEM) {
        CHECK(s.row == old);
        continue;
      }
      CHECK(rc == ATTN_OK);
      if (pair[0] >= 0) {
        ref[pair[0]]--;
        ref[pair[1]]++;
      }
      for (int b = before; b < (s.len + n + BS - 1) / BS; ++b) ref[s.row[b]]++;
      s.len += n;
    } else {  // end a sequence
      const size_t i = g() % seqs.size();
      const int nb = (seqs[i].len + BS - 1) / BS;
      CHECK(attn_pool_free(p, seqs[i].row.data(), nb) == ATTN_OK);
      for (int b = 0; b < nb; ++b) ref[seqs[i].row[b]]--;
      seqs.erase(seqs.begin() + (long)i);
    }
    int used = 0;
    for (int b = 0; b < NB; ++b) {
      CHECK(attn_pool_refcount(p, b) == ref[b]);
      used += ref[b] > 0;
    }
    CHECK(attn_pool_num_free(p) == NB - used);
    // errors are reported on this thread's own text
    if (it % 16 == 0) {
      const int32_t bad = NB + t;
      CHECK(attn_pool_free(p, &bad, 1) == ATTN_E_INVALID);
      CHECK(std::strstr(attn_last_error(), "attn_pool_free") != nullptr);
    }
  }
  for (const Seq& s : seqs) CHECK(attn_pool_free(p, s.row.data(), (s.len + BS - 1) / BS) == ATTN_OK);
  CHECK(attn_pool_num_free(p) == NB);
  attn_pool_destroy(p);
}

// Shared pool: every call under the mutex; blocks taken by one thread may be
// released by another (through a shared list).
std::vector<int32_t> handed;

void shared_work(int t) {
  std::mt19937 g(2000 + t);
  for (int it = 0; it < kRounds; ++it) {
    std::lock_guard<std::mutex> lock(shared_mu);
    if (g() % 2 == 0) {
      int32_t ids[3];
      const int n = 1 + (int)(g() % 3);
      if (attn_pool_alloc(shared_pool, n, ids) == ATTN_OK)
        for (int i = 0; i < n; ++i) {
          CHECK(attn_pool_refcount(shared_pool, ids[i]) == 1);
          handed.push_back(ids[i]);
        }
    } else if (!handed.empty()) {
      const int32_t id = handed.back();
      handed.pop_back();
      CHECK(attn_pool_free(shared_pool, &id, 1) == ATTN_OK);
    }
    CHECK(attn_pool_num_free(shared_pool) + (int)handed.size() == attn_pool_num_blocks(shared_pool));
  }
}

}  // namespace

int main() {
  CHECK(attn_pool_create(48, 16, &shared_pool) == ATTN_OK);
  std::vector<std::thread> th;
  for (int t = 0; t < kThreads; ++t)
    th.emplace_back([t] {
      private_work(t);
      shared_work(t);
    });
  for (auto& x : th) x.join();
  CHECK(attn_pool_free(shared_pool, handed.data(), (int32_t)handed.size()) == ATTN_OK);
  CHECK(attn_pool_num_free(shared_pool) == 48);
  attn_pool_destroy(shared_pool);
  std::printf("pool threads: ok\n");
  return 0;
}
