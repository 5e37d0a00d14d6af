// Host model of the split-sequence hand-off of the forward scan (test code).
//
// The forward scan cuts a long sequence into chunks that run concurrently.
// Each chunk scans from a zero state and reduces to an affine map of its
// entering state, h_out = A_k h_in + H_k per state (A_k the product of the
// decays over the chunk, H_k the end state from zero). Chunk k > 0 waits for
// chunk k-1's inclusive end state, forms its own as A_k h_in + H_k and hands
// it on. This program re-implements that protocol with std::thread workers
// standing for workgroups, the same memory orders as the kernel (relaxed
// flag loads and stores, an acquire fence after the wait, a release fence
// before the flag), random delays at every step, and fewer workers than
// chunks (a workgroup only takes new work once it has finished its chunk).
// The chunks are dealt out as the kernel deals them: 8 ticket queues (one
// per XCD), queue q holding the groups [q nbg / 8, (q + 1) nbg / 8) chunk-
// major; a worker takes from the queue of "its" XCD, else from the next ones.
//
//   handoff_model <order> <nbg> <nchunks> <workers> <seed> <spin_limit> <lost>
//     order: "ticket"  the queues, worker w on XCD w mod 8 (the kernel's
//                      protocol)
//            "skew"    the queues, every worker on XCD 0 (an uneven dispatch:
//                      the other queues are only reached by the fallback)
//            "static"  worker w takes blocks w, w + workers, ... in the
//                      XCD-interleaved block order (a fixed assignment; its
//                      predecessor may belong to a worker that is itself
//                      waiting)
//     lost:  a chunk index (>= 0) whose workers never hand their state on
//            (a lost workgroup), or -1
//
// Checks: every chunk is taken exactly once; per channel group, every
// inclusive state equals the sequential
// composition bit for bit (same operations in the same order), or is NaN
// exactly for the chunks after a give-up; a give-up sets the error word.
// Prints one line "ok ..." and exits 0, or prints the failure and exits 1.
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <string>
#include <thread>
#include <vector>

namespace {

constexpr int kStates = 16;

struct Shared {
  int nbg = 0, nchunks = 0;
  unsigned spin_limit = 0;
  int lost = -1;
  std::atomic<unsigned> ticket[8];
  std::vector<std::atomic<int>> taken;  // times each chunk was taken
  std::atomic<unsigned> err{0};
  std::vector<std::atomic<int>> flag;
  std::vector<float> state;     // [slot][kStates], the hand-off buffer
  std::vector<float> A, H;      // chunk aggregates [slot][kStates]
  std::vector<float> incl;      // every chunk's inclusive state (checked afterwards)
  std::atomic<long> waits{0}, gave_up{0};
  explicit Shared(int nslots) : taken(nslots), flag(nslots), state(nslots * kStates), A(nslots * kStates),
                                H(nslots * kStates), incl(nslots * kStates) {
    for (auto& f : flag) f.store(0, std::memory_order_relaxed);
    for (auto& t : taken) t.store(0, std::memory_order_relaxed);
    for (auto& t : ticket) t.store(0u, std::memory_order_relaxed);
  }
};

void jitter(std::mt19937& rng) {
  const unsigned r = rng() % 16;
  if (r < 8) return;
  if (r < 14) {
    std::this_thread::yield();
    return;
  }
  std::this_thread::sleep_for(std::chrono::microseconds(rng() % 200));
}

int queue_start(int q, int nbg) { return q * nbg / 8; }

// a chunk from the queue of XCD xcc, else from the following queues
bool take_chunk(Shared& s, int xcc, int* k, int* bg) {
  for (int d = 0; d < 8; ++d) {
    const int q = (xcc + d) % 8;
    const int g0 = queue_start(q, s.nbg), ng = queue_start(q + 1, s.nbg) - g0;
    if (ng == 0) continue;
    const unsigned j = s.ticket[q].fetch_add(1u, std::memory_order_relaxed);
    if (j < static_cast<unsigned>(ng * s.nchunks)) {
      *k = static_cast<int>(j) / ng;
      *bg = g0 + static_cast<int>(j) % ng;
      return true;
    }
  }
  return false;
}

// one chunk: main pass (a delay), then the hand-off
void run_chunk(Shared& s, int k, int bg, std::mt19937& rng) {
  jitter(rng);  // the chunk's main pass
  const int slot = bg * s.nchunks + k;
  s.taken[slot].fetch_add(1, std::memory_order_relaxed);
  float hin[kStates];
  for (int j = 0; j < kStates; ++j) hin[j] = 0.f;
  if (k > 0) {
    bool ok = false;
    for (unsigned it = 0;; ++it) {
      if (s.flag[slot - 1].load(std::memory_order_relaxed) != 0) {
        ok = true;
        break;
      }
      if (it >= s.spin_limit) {
        s.err.fetch_or(1u, std::memory_order_relaxed);
        break;
      }
      std::this_thread::yield();
    }
    s.waits.fetch_add(1, std::memory_order_relaxed);
    std::atomic_thread_fence(std::memory_order_acquire);
    for (int j = 0; j < kStates; ++j) hin[j] = s.state[(slot - 1) * kStates + j];
    if (!ok) {
      s.gave_up.fetch_add(1, std::memory_order_relaxed);
      for (int j = 0; j < kStates; ++j) hin[j] = std::nanf("");
    }
  }
  jitter(rng);
  float out[kStates];
  for (int j = 0; j < kStates; ++j)
    out[j] = k > 0 ? std::fma(s.A[slot * kStates + j], hin[j], s.H[slot * kStates + j]) : s.H[slot * kStates + j];
  for (int j = 0; j < kStates; ++j) s.incl[slot * kStates + j] = out[j];
  if (k + 1 < s.nchunks && k != s.lost) {
    for (int j = 0; j < kStates; ++j) s.state[slot * kStates + j] = out[j];
    std::atomic_thread_fence(std::memory_order_release);
    s.flag[slot].store(1, std::memory_order_relaxed);
  }
  jitter(rng);  // the chunk's correction pass
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 8) {
    std::fprintf(stderr, "usage: %s ticket|static nbg nchunks workers seed spin_limit lost\n", argv[0]);
    return 2;
  }
  const std::string order = argv[1];
  const int nbg = std::atoi(argv[2]), nchunks = std::atoi(argv[3]), workers = std::atoi(argv[4]);
  const unsigned seed = static_cast<unsigned>(std::strtoul(argv[5], nullptr, 10));
  const unsigned spin = static_cast<unsigned>(std::strtoul(argv[6], nullptr, 10));
  const int lost = std::atoi(argv[7]);
  if (nbg <= 0 || nchunks <= 0 || workers <= 0 || (order != "ticket" && order != "skew" && order != "static"))
    return 2;
  const int nslots = nbg * nchunks;
  Shared s(nslots);
  s.nbg = nbg;
  s.nchunks = nchunks;
  s.spin_limit = spin;
  s.lost = lost;
  std::mt19937 rng(seed);
  std::uniform_real_distribution<float> ua(0.2f, 1.0f), uh(-3.f, 3.f);
  for (int i = 0; i < nslots * kStates; ++i) s.A[i] = ua(rng), s.H[i] = uh(rng);

  std::vector<std::thread> th;
  for (int w = 0; w < workers; ++w) {
    th.emplace_back([&, w] {
      std::mt19937 r(seed * 7919u + static_cast<unsigned>(w));
      if (order != "static") {
        const int xcc = order == "skew" ? 0 : w % 8;
        int k, bg;
        while (take_chunk(s, xcc, &k, &bg)) run_chunk(s, k, bg, r);
      } else {
        // fixed blocks, XCD-interleaved over all blocks, chunk-major after the remap
        for (int blk = w; blk < nslots; blk += workers) {
          const int lb = (nslots % 8 == 0) ? (blk & 7) * (nslots >> 3) + (blk >> 3) : blk;
          run_chunk(s, lb / nbg, lb % nbg, r);
        }
      }
    });
  }
  for (auto& t : th) t.join();

  // reference: the sequential composition, and which chunks must be NaN
  long mismatches = 0, nan_chunks = 0;
  for (int i = 0; i < nslots; ++i)
    if (s.taken[i].load() != 1) {
      std::printf("FAIL chunk %d taken %d times\n", i, s.taken[i].load());
      return 1;
    }
  for (int bg = 0; bg < nbg; ++bg) {
    float ref[kStates];
    bool poisoned = false;
    for (int k = 0; k < nchunks; ++k) {
      const int slot = bg * nchunks + k;
      for (int j = 0; j < kStates; ++j)
        ref[j] = k > 0 ? std::fma(s.A[slot * kStates + j], ref[j], s.H[slot * kStates + j]) : s.H[slot * kStates + j];
      const bool is_nan = std::isnan(s.incl[slot * kStates]);
      if (is_nan) {
        ++nan_chunks;
        poisoned = true;
      }
      for (int j = 0; j < kStates; ++j) {
        const float got = s.incl[slot * kStates + j];
        if (poisoned) {
          if (!std::isnan(got)) ++mismatches;  // once poisoned, every later chunk of the group is NaN
        } else if (std::memcmp(&got, &ref[j], sizeof(float)) != 0) {
          ++mismatches;
        }
      }
    }
  }
  const unsigned err = s.err.load();
  const long gave_up = s.gave_up.load();
  // a give-up must set the error word and leave NaN behind; without one there is no NaN
  if (mismatches || (gave_up > 0) != (err != 0) || (gave_up > 0) != (nan_chunks > 0)) {
    std::printf("FAIL order=%s mismatches=%ld gave_up=%ld err=%u nan_chunks=%ld\n", order.c_str(), mismatches,
                gave_up, err, nan_chunks);
    return 1;
  }
  std::printf("ok order=%s chunks=%d workers=%d waits=%ld gave_up=%ld err=%u nan_chunks=%ld\n", order.c_str(),
              nslots, workers, s.waits.load(), gave_up, err, nan_chunks);
  return 0;
}
