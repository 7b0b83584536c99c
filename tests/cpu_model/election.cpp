// Host model of the completion protocol ("ep_signal_completion", description:
// rank-level completion with ep_ord_r, and the per-expert form without it),
// for ThreadSanitizer.  E producer threads (the local experts) each write a
// plain payload word per destination rank (the rows they send), store the
// (e, rk) count word, then take part in rank rk's election: a fetch-add on
// rk's counter; the producer that finds E - 1 there resets the counter and
// release-stores rk's flag.  R consumer threads acquire their rank's flag
// once and read every producer's payload and count word for that rank.
//
//   acq_rel     the election RMW is acquire-release: every consumer read is
//               ordered after the write it reads (TSan stays silent)
//   relaxed     the election RMW is relaxed: the elected producer does not
//               synchronise with the others, so a consumer's read of another
//               producer's payload is a data race (TSan must report it)
//   per_expert  no election: each count word is release-stored and the
//               consumer acquires all E of its rank's words (TSan silent)
//
// The device code reaches the acquire-release form with a release fence, a
// relaxed RMW and an acquire fence; TSan does not model standalone fences,
// so the model uses the RMW form the fences are equivalent to.
// Exit status: 0 when every value the consumers read is the one written.
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <thread>
#include <vector>

namespace {

constexpr int E = 8;       // producers (local experts)
constexpr int R = 4;       // consumers (destination ranks)

struct Step {
  int payload[E][R];                       // plain data: the rows
  std::atomic<long> count[E][R];           // count word (e, rk)
  std::atomic<int> counter[R];             // election counters
  std::atomic<long> flag[R];               // rank flags (epoch)
};

long value(int e, int rk, long epoch) { return epoch * 1000 + e * 10 + rk; }

void producer(Step& s, int e, long epoch, std::memory_order rmw, bool per_expert) {
  for (int rk = 0; rk < R; ++rk) {
    s.payload[e][rk] = (int)value(e, rk, epoch);
    if (per_expert) {
      s.count[e][rk].store(value(e, rk, epoch), std::memory_order_release);
      continue;
    }
    s.count[e][rk].store(value(e, rk, epoch), std::memory_order_relaxed);
    if (s.counter[rk].fetch_add(1, rmw) == E - 1) {
      s.counter[rk].store(0, std::memory_order_relaxed);
      s.flag[rk].store(epoch, std::memory_order_release);
    }
  }
}

int consumer(Step& s, int rk, long epoch, bool per_expert) {
  if (per_expert) {
    for (int e = 0; e < E; ++e)
      while (s.count[e][rk].load(std::memory_order_acquire) != value(e, rk, epoch)) {
      }
  } else {
    while (s.flag[rk].load(std::memory_order_acquire) != epoch) {
    }
  }
  int bad = 0;
  for (int e = 0; e < E; ++e) {
    if (s.payload[e][rk] != (int)value(e, rk, epoch)) ++bad;
    if (s.count[e][rk].load(std::memory_order_relaxed) != value(e, rk, epoch)) ++bad;
  }
  return bad;
}

}  // namespace

int main(int argc, char** argv) {
  const char* mode = argc > 1 ? argv[1] : "acq_rel";
  const int rounds = argc > 2 ? std::atoi(argv[2]) : 200;
  const bool per_expert = std::strcmp(mode, "per_expert") == 0;
  const std::memory_order rmw =
      std::strcmp(mode, "relaxed") == 0 ? std::memory_order_relaxed : std::memory_order_acq_rel;
  int bad = 0;
  for (int round = 1; round <= rounds; ++round) {
    Step s;
    for (int e = 0; e < E; ++e)
      for (int rk = 0; rk < R; ++rk) {
        s.payload[e][rk] = 0;
        s.count[e][rk].store(0, std::memory_order_relaxed);
      }
    for (int rk = 0; rk < R; ++rk) {
      s.counter[rk].store(0, std::memory_order_relaxed);
      s.flag[rk].store(0, std::memory_order_relaxed);
    }
    std::vector<int> got(R, 0);
    std::vector<std::thread> threads;
    for (int rk = 0; rk < R; ++rk)
      threads.emplace_back([&, rk] { got[rk] = consumer(s, rk, round, per_expert); });
    for (int e = 0; e < E; ++e)
      threads.emplace_back([&, e] { producer(s, e, round, rmw, per_expert); });
    for (auto& t : threads) t.join();
    for (int rk = 0; rk < R; ++rk) bad += got[rk];
    for (int rk = 0; rk < R && !per_expert; ++rk)
      if (s.counter[rk].load() != 0) ++bad;       // the elected producer re-armed it
  }
  std::printf("%s: %d rounds, %d wrong values\n", mode, rounds, bad);
  return bad == 0 ? 0 : 1;
}
