// Host model of the completion protocol ("ep_signal_completion", description:
// rank-level completion with ep_ord_r, and the per-expert form without it),
// for ThreadSanitizer.
//
// Expert level (modes acq_rel, relaxed, per_expert): E producer threads (the
// local experts) each write a plain payload word per destination rank (the
// rows they send), store the (e, rk) count word, then take part in rank rk's
// election: a fetch-add on rk's counter; the producer that finds E - 1 there
// resets the counter and release-stores rk's flag.  R consumer threads acquire
// their rank's flag once and read every producer's payload and count word for
// that rank.
//
//   acq_rel     the election RMW is acquire-release: every consumer read is
//               ordered after the write it reads (TSan stays silent)
//   relaxed     the election RMW is relaxed: the elected producer does not
//               synchronise with the others, so a consumer's read of another
//               producer's payload is a data race (TSan must report it)
//   per_expert  no election: each count word is release-stored and the
//               consumer acquires all E of its rank's words (TSan silent)
//
// Tile level (modes tiles, tiles_relaxed_counter, tiles_no_wg_fence): every
// expert's output is TPE tiles, each made by its own workgroup of W threads
// (waves).  Every wave writes its rows of the tile (plain payload words for
// each rank), then the workgroup meets at a barrier; its first thread then
// counts the tile with a fetch-add on the expert's tile counter, and the
// thread that finds TPE - 1 there (the expert's last tile) re-arms the
// counter, stores the expert's count words and joins the rank elections as
// above.  This is the device code's hand-off: row stores, a workgroup barrier
// bracketed by workgroup-scope release / acquire fences, then one thread's
// agent-scope release fence + relaxed RMW + acquire fence on the tile counter.
//
//   tiles                   barrier arrive = release, wait = acquire; tile
//                           counter RMW acquire-release (TSan silent)
//   tiles_relaxed_counter   tile counter RMW relaxed: the thread that counts
//                           an expert's last tile does not synchronise with
//                           the other tiles' workgroups (TSan must report it)
//   tiles_no_wg_fence       barrier arrive and wait relaxed: the counting
//                           thread's release does not carry the other waves'
//                           row stores (TSan must report it)
//
// The device code reaches the acquire-release forms with release fences, a
// relaxed RMW and acquire fences; TSan does not model standalone fences, so
// the model uses the RMW and load/store forms the fences are equivalent to.
// Exit status: 0 when every value the consumers read is the one written.
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <thread>
#include <vector>

namespace {

constexpr int E = 8;       // producers (local experts), expert-level modes
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

int run_expert_level(const char* mode, int rounds) {
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
  return bad;
}

// ---------------------------------------------------------------- tile level

constexpr int TE = 3;      // experts
constexpr int TPE = 3;     // tiles per expert, one workgroup each
constexpr int W = 3;       // waves (threads) per workgroup

struct TileStep {
  int rows[TE][TPE][W][R];                 // plain data: wave w's rows of tile p for rank rk
  std::atomic<int> arrive[TE][TPE];        // the tile workgroup's barrier
  std::atomic<int> tile_counter[TE];
  std::atomic<long> count[TE][R];
  std::atomic<int> counter[R];
  std::atomic<long> flag[R];
};

int row_value(int e, int p, int w, int rk, long epoch) {
  return (int)(epoch * 10000 + e * 1000 + p * 100 + w * 10 + rk);
}

void tile_wave(TileStep& s, int e, int p, int w, long epoch, std::memory_order arrive_o,
               std::memory_order wait_o, std::memory_order tile_rmw) {
  for (int rk = 0; rk < R; ++rk) s.rows[e][p][w][rk] = row_value(e, p, w, rk, epoch);
  // workgroup barrier: every wave arrives, then waits for all W
  s.arrive[e][p].fetch_add(1, arrive_o);
  while (s.arrive[e][p].load(wait_o) < W) {
  }
  if (w != 0) return;
  // the first thread counts the tile; the expert's last tile publishes
  if (s.tile_counter[e].fetch_add(1, tile_rmw) != TPE - 1) return;
  s.tile_counter[e].store(0, std::memory_order_relaxed);
  for (int rk = 0; rk < R; ++rk) {
    s.count[e][rk].store(value(e, rk, epoch), std::memory_order_relaxed);
    if (s.counter[rk].fetch_add(1, std::memory_order_acq_rel) == TE - 1) {
      s.counter[rk].store(0, std::memory_order_relaxed);
      s.flag[rk].store(epoch, std::memory_order_release);
    }
  }
}

int tile_consumer(TileStep& s, int rk, long epoch) {
  while (s.flag[rk].load(std::memory_order_acquire) != epoch) {
  }
  int bad = 0;
  for (int e = 0; e < TE; ++e) {
    for (int p = 0; p < TPE; ++p)
      for (int w = 0; w < W; ++w)
        if (s.rows[e][p][w][rk] != row_value(e, p, w, rk, epoch)) ++bad;
    if (s.count[e][rk].load(std::memory_order_relaxed) != value(e, rk, epoch)) ++bad;
  }
  return bad;
}

int run_tile_level(const char* mode, int rounds) {
  std::memory_order arrive_o = std::memory_order_release, wait_o = std::memory_order_acquire;
  std::memory_order tile_rmw = std::memory_order_acq_rel;
  if (std::strcmp(mode, "tiles_relaxed_counter") == 0) tile_rmw = std::memory_order_relaxed;
  if (std::strcmp(mode, "tiles_no_wg_fence") == 0)
    arrive_o = wait_o = std::memory_order_relaxed;
  int bad = 0;
  for (int round = 1; round <= rounds; ++round) {
    TileStep s;
    std::memset(s.rows, 0, sizeof s.rows);
    for (int e = 0; e < TE; ++e) {
      s.tile_counter[e].store(0, std::memory_order_relaxed);
      for (int p = 0; p < TPE; ++p) s.arrive[e][p].store(0, std::memory_order_relaxed);
      for (int rk = 0; rk < R; ++rk) s.count[e][rk].store(0, std::memory_order_relaxed);
    }
    for (int rk = 0; rk < R; ++rk) {
      s.counter[rk].store(0, std::memory_order_relaxed);
      s.flag[rk].store(0, std::memory_order_relaxed);
    }
    std::vector<int> got(R, 0);
    std::vector<std::thread> threads;
    for (int rk = 0; rk < R; ++rk)
      threads.emplace_back([&, rk] { got[rk] = tile_consumer(s, rk, round); });
    for (int e = 0; e < TE; ++e)
      for (int p = 0; p < TPE; ++p)
        for (int w = 0; w < W; ++w)
          threads.emplace_back(
              [&, e, p, w] { tile_wave(s, e, p, w, round, arrive_o, wait_o, tile_rmw); });
    for (auto& t : threads) t.join();
    for (int rk = 0; rk < R; ++rk) bad += got[rk];
    for (int e = 0; e < TE; ++e)
      if (s.tile_counter[e].load() != 0) ++bad;   // the last tile re-armed it
    for (int rk = 0; rk < R; ++rk)
      if (s.counter[rk].load() != 0) ++bad;
  }
  return bad;
}

}  // namespace

int main(int argc, char** argv) {
  const char* mode = argc > 1 ? argv[1] : "acq_rel";
  const int rounds = argc > 2 ? std::atoi(argv[2]) : 200;
  const int bad = std::strncmp(mode, "tiles", 5) == 0 ? run_tile_level(mode, rounds)
                                                      : run_expert_level(mode, rounds);
  std::printf("%s: %d rounds, %d wrong values\n", mode, rounds, bad);
  return bad == 0 ? 0 : 1;
}
