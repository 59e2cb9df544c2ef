// Host simulation of the chain barrier's counters (chain_sync.h), driven
// across the 32-bit wrap of the cumulative counters.
//
//   chain_counters_sim G n_lin gen0 launches [old]
//
// Starts from the counter state after gen0 complete launches, then runs
// `launches` launches of n_lin linears with G workgroups arriving in a
// shuffled order. Checks, per launch and linear: exactly one arrival
// releases, it is the last one, no waiter sees the release before it and
// every waiter sees it after; and exactly one exit advances the generation.
// With "old", the launch count is derived back from the wrapped target
// (target / G) instead of carried, which is expected to fail near the wrap.
// Prints "ok" and returns 0, or prints the first violation and returns 1.

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "chain_sync.h"

using namespace specv;

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32() {  // xorshift64*
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}

int main(int argc, char** argv) {
  if (argc < 5) {
    fprintf(stderr, "usage: %s G n_lin gen0 launches [old]\n", argv[0]);
    return 2;
  }
  const int G = atoi(argv[1]);
  const int n_lin = atoi(argv[2]);
  const unsigned gen0 = (unsigned)strtoul(argv[3], nullptr, 0);
  const int launches = atoi(argv[4]);
  const bool old = argc > 5;
  const int kGroups = 8;
  const int n_groups = G < kGroups ? G : kGroups;

  // state after gen0 complete launches
  unsigned gen = gen0, exit_count = chain_target(gen0, G);
  std::vector<unsigned> counts(n_lin, gen0 * (unsigned)n_groups);
  std::vector<unsigned> flags(n_lin, chain_target(gen0, G));
  std::vector<unsigned> gc((size_t)n_lin * kGroups);
  for (int l = 0; l < n_lin; ++l)
    for (int g = 0; g < kGroups; ++g) gc[(size_t)l * kGroups + g] = gen0 * chain_group_size(G, g, kGroups);

  std::vector<int> order(G);
  for (int launch = 0; launch < launches; ++launch) {
    const unsigned s_gen = gen;
    const unsigned target = chain_target(s_gen + 1u, G);
    const unsigned gen1 = old ? target / (unsigned)G : s_gen + 1u;
    for (int l = 0; l < n_lin; ++l) {
      for (int i = 0; i < G; ++i) order[i] = i;
      for (int i = G - 1; i > 0; --i) {
        const int j = (int)(next_u32() % (unsigned)(i + 1));
        const int t = order[i];
        order[i] = order[j];
        order[j] = t;
      }
      int releases = 0;
      for (int i = 0; i < G; ++i) {
        if (chain_released(flags[l], target)) {
          printf("launch %d (gen %u) linear %d: released before arrival %d of %d\n", launch, s_gen,
                 l, i, G);
          return 1;
        }
        const int bid = order[i];
        const int g = bid % kGroups;
        const unsigned gp = gc[(size_t)l * kGroups + g]++;
        if (chain_group_complete(gp, gen1, chain_group_size(G, g, kGroups))) {
          const unsigned prev = counts[l]++;
          if (chain_linear_complete(prev, gen1, n_groups)) {
            flags[l] = target;
            ++releases;
            if (i != G - 1) {
              printf("launch %d linear %d: released at arrival %d of %d\n", launch, l, i, G);
              return 1;
            }
          }
        }
      }
      if (releases != 1 || !chain_released(flags[l], target)) {
        printf("launch %d (gen %u) linear %d: %d releases, flag %u, target %u\n", launch, s_gen, l,
               releases, flags[l], target);
        return 1;
      }
    }
    int advances = 0;
    for (int i = 0; i < G; ++i) {
      const unsigned prev = exit_count++;
      if (prev + 1u == target) {
        ++gen;
        ++advances;
      }
    }
    if (advances != 1 || gen != s_gen + 1u) {
      printf("launch %d: generation advanced %d times (gen %u)\n", launch, advances, gen);
      return 1;
    }
  }
  printf("ok\n");
  return 0;
}
