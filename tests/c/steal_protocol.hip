// Host test of the steal schedule's share-word protocol (fd_steal.h): one
// owner and several thieves act on one word in random interleavings, with
// the operations the kernel performs -- the owner's fetch_add claims, each
// issued while it still streams its previous chunk, and the thieves'
// compare-exchange takes computed from a word value loaded earlier (stale
// loads included). After every interleaving each chunk of the share must
// belong to exactly one run, the owner's run must be [0, k), every take a
// range below the owner's run, the steal count at most cap, and the steal
// count the owner reads with its last claim must equal the number of takes.
// Built for the host only; no device code runs.
#include <stdio.h>
#include <stdlib.h>
#include <stdint.h>
#include <vector>

#include "fd_steal.h"

using fd::StealTake;

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(uint32_t n) {  // xorshift64*, uniform enough for a test
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (uint32_t)((rng_state * 2685821657736338717ull) >> 33) % n;
}

static int fail(const char* what, int nc, int cap, int thieves, long it) {
  printf("FAIL %s nc=%d cap=%d thieves=%d case=%ld\n", what, nc, cap, thieves, it);
  return 1;
}

int main() {
  long cases = 0, takes_total = 0;
  for (long it = 0; it < 200000; ++it) {
    const int nc = 1 + (int)rnd(40);
    const int cap = 1 + (int)rnd(15);
    const int nthieves = 1 + (int)rnd(8);
    unsigned long long word = 0;  // zeroed before the launch
    std::vector<int> owner_of(nc, -1);  // -1 unclaimed, 0 owner, 1 + t thief t
    owner_of[0] = 0;
    // owner: chunk 0 streamed at once; with nc >= 2 its first claim is in flight
    int owned = 1;
    bool owner_done = nc < 2;
    bool claim_in_flight = !owner_done;
    bool first_claim = true;
    int owner_steals_seen = 0;
    // thieves: each holds a word value it loaded (possibly stale)
    std::vector<unsigned long long> seen(nthieves, 0);
    std::vector<bool> done(nthieves, false);
    int takes = 0;
    for (int step = 0; step < 100000; ++step) {
      bool all_done = owner_done;
      for (int t = 0; t < nthieves; ++t) all_done = all_done && done[t];
      if (all_done) break;
      const int who = (int)rnd((uint32_t)nthieves + 1);
      if (who == 0) {
        if (owner_done || !claim_in_flight) continue;
        // the claim lands: fetch_add
        const unsigned long long old = word;
        word += first_claim ? fd::steal_first_claim(nc) : fd::kStealClaim;
        first_claim = false;
        const int chunk = fd::steal_claimed_chunk(old, nc);
        owner_steals_seen = fd::steal_count(old);
        if (chunk < 0) {
          owner_done = true;
        } else {
          if (chunk != owned) return fail("owner chunk out of order", nc, cap, nthieves, it);
          if (owner_of[chunk] != -1) return fail("owner claimed a taken chunk", nc, cap, nthieves, it);
          owner_of[chunk] = 0;
          ++owned;
          // the next claim is issued only if a next chunk exists
          claim_in_flight = owned < nc;
          if (!claim_in_flight) owner_done = true;
        }
      } else {
        const int t = who - 1;
        if (done[t]) continue;
        if (rnd(3) == 0) {  // load the word now (otherwise act on an older value)
          seen[t] = word;
          continue;
        }
        const StealTake tk = fd::steal_take(seen[t], cap);
        if (tk.m == 0) {
          // nothing to take in the value it holds: a fresh load of a
          // published (or never to be published) word ends the thief
          if (seen[t] == word && (fd::steal_chunks(word) > 0 || owner_done)) done[t] = true;
          seen[t] = word;
          continue;
        }
        if (word != seen[t]) {  // compare-exchange fails, returns the current value
          seen[t] = word;
          continue;
        }
        word = tk.want;
        if (tk.c0 < 1 || tk.c1 > nc || tk.c0 >= tk.c1 || tk.m != tk.c1 - tk.c0)
          return fail("take out of range", nc, cap, nthieves, it);
        for (int c = tk.c0; c < tk.c1; ++c) {
          if (owner_of[c] != -1) return fail("take overlaps a run", nc, cap, nthieves, it);
          owner_of[c] = 1 + t;
        }
        if (tk.slot != takes) return fail("steal slot out of order", nc, cap, nthieves, it);
        ++takes;
        seen[t] = word;
      }
    }
    if (!owner_done) return fail("owner did not finish", nc, cap, nthieves, it);
    for (int t = 0; t < nthieves; ++t)
      if (!done[t]) {
        // a thief may still hold a stale value; a final fresh check must find nothing
        if (fd::steal_take(word, cap).m != 0) return fail("work left behind", nc, cap, nthieves, it);
      }
    for (int c = 0; c < nc; ++c)
      if (owner_of[c] == -1) return fail("chunk never claimed", nc, cap, nthieves, it);
    for (int c = 0; c < owned; ++c)
      if (owner_of[c] != 0) return fail("owner run not contiguous", nc, cap, nthieves, it);
    for (int c = owned; c < nc; ++c)
      if (owner_of[c] == 0) return fail("owner chunk past its run", nc, cap, nthieves, it);
    if (takes > cap) return fail("more steals than slots", nc, cap, nthieves, it);
    if (nc >= 2 && owner_steals_seen != takes)
      return fail("owner's last claim missed a steal", nc, cap, nthieves, it);
    if (nc < 2 && (word != 0 || takes != 0)) return fail("one-chunk share touched", nc, cap, nthieves, it);
    if (fd::steal_unclaimed(word) > 0 && nc >= 2) return fail("unclaimed chunks at the end", nc, cap, nthieves, it);
    ++cases;
    takes_total += takes;
  }
  printf("steal protocol ok %ld cases %ld takes\n", cases, takes_total);
  return 0;
}
