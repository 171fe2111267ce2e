// exchange_model.cpp -- a CPU model of the decode kernel's exchange protocol, run with threads.
//
// The kernel's workgroups exchange values as 64-bit words (value bits << 32 | epoch) through
// buffers that are separate per layer and per hop; a reader accepts a word only when its tag is
// the current step's epoch, and each step ends with an all-gather of one word per workgroup (the
// sampling candidates). Each thread here plays one workgroup: per step, per layer, per hop it
// publishes its words, then gathers every thread's words of that hop and checks their values;
// random delays stand in for the workgroups' uneven progress. The model checks that no reader
// ever accepts a wrong value and that every wait ends.
//
// usage: exchange_model <threads> <layers> <steps> <seed> [shared|nojoin|sametag]
//   shared:  one buffer per hop for all layers;
//   sametag: the same tag in every step;
//   nojoin:  no all-gather at the end of a step.
//   The first two are deliberately broken and must report violations or a stuck wait.
#include <atomic>
#include <chrono>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <thread>
#include <string_view>
#include <vector>

namespace {
constexpr int kHops = 6;   // q/k/v, partials, o, x after O, h, x after down
constexpr int kWords = 3;  // words each thread publishes per hop

uint32_t value_of(int step, int layer, int hop, int w, int k) {
  uint32_t x = (uint32_t)step * 0x9E3779B1u ^ (uint32_t)layer * 0x85EBCA77u ^ (uint32_t)hop * 0xC2B2AE3Du ^
               (uint32_t)w * 0x27D4EB2Fu ^ (uint32_t)k * 0x165667B1u;
  x ^= x >> 15;
  x *= 0x2C1B3C6Du;
  x ^= x >> 12;
  return x;
}
}  // namespace

int main(int argc, char** argv) {
  if (argc < 5) {
    std::fprintf(stderr, "usage: %s threads layers steps seed [shared]\n", argv[0]);
    return 2;
  }
  const int W = std::atoi(argv[1]), L = std::atoi(argv[2]), S = std::atoi(argv[3]);
  const unsigned seed = (unsigned)std::atoi(argv[4]);
  const std::string_view mode = argc > 5 ? argv[5] : "";
  const bool shared = mode == "shared", sametag = mode == "sametag", nojoin = mode == "nojoin";
  const int nbuf = shared ? kHops : L * kHops;
  std::vector<std::atomic<uint64_t>> buf((size_t)nbuf * W * kWords);
  std::vector<std::atomic<uint64_t>> join((size_t)W);
  for (auto& b : buf) b.store(0, std::memory_order_relaxed);
  for (auto& b : join) b.store(0, std::memory_order_relaxed);
  std::atomic<long> violations{0}, stuck{0};
  const auto limit = std::chrono::seconds(5);

  auto run = [&](int w) {
    std::mt19937 rng(seed * 7919u + (unsigned)w);
    std::uniform_int_distribution<int> delay(0, 40);
    auto pause = [&]() {
      const int us = delay(rng);
      if (us > 30) std::this_thread::sleep_for(std::chrono::microseconds(us));
      else for (int i = 0; i < us * 10; ++i) std::this_thread::yield();
    };
    auto wait_for = [&](std::atomic<uint64_t>& word, uint32_t epoch, uint64_t* got) {
      const auto t0 = std::chrono::steady_clock::now();
      for (;;) {
        const uint64_t v = word.load(std::memory_order_relaxed);
        if ((uint32_t)v == epoch) {
          *got = v;
          return true;
        }
        if (std::chrono::steady_clock::now() - t0 > limit) return false;
        std::this_thread::yield();
      }
    };
    for (int s = 0; s < S; ++s) {
      const uint32_t epoch = sametag ? 1u : (uint32_t)s + 1u;
      for (int l = 0; l < L; ++l) {
        for (int h = 0; h < kHops; ++h) {
          const size_t base = (size_t)((shared ? 0 : l) * kHops + h) * W * kWords;
          pause();
          for (int k = 0; k < kWords; ++k)
            buf[base + (size_t)w * kWords + k].store(((uint64_t)value_of(s, l, h, w, k) << 32) | epoch,
                                                     std::memory_order_relaxed);
          for (int w2 = 0; w2 < W; ++w2)
            for (int k = 0; k < kWords; ++k) {
              uint64_t v;
              if (!wait_for(buf[base + (size_t)w2 * kWords + k], epoch, &v)) {
                stuck.fetch_add(1);
                return;
              }
              if ((uint32_t)(v >> 32) != value_of(s, l, h, w2, k)) violations.fetch_add(1);
            }
        }
      }
      if (nojoin) continue;
      // the step's join: one word per thread, gathered by all
      pause();
      join[w].store(((uint64_t)(uint32_t)w << 32) | epoch, std::memory_order_relaxed);
      for (int w2 = 0; w2 < W; ++w2) {
        uint64_t v;
        if (!wait_for(join[w2], epoch, &v)) {
          stuck.fetch_add(1);
          return;
        }
        if ((uint32_t)(v >> 32) != (uint32_t)w2) violations.fetch_add(1);
      }
    }
  };
  std::vector<std::thread> th;
  for (int w = 0; w < W; ++w) th.emplace_back(run, w);
  for (auto& t : th) t.join();
  std::printf("%s violations %ld stuck %ld\n", violations == 0 && stuck == 0 ? "ok" : "FAIL", violations.load(),
              stuck.load());
  return violations == 0 && stuck == 0 ? 0 : 1;
}
