// The share word of the steal schedule and the arithmetic of its two
// operations -- an owner's claim from the front, a thief's take from the
// back -- as pure functions of word values. The matrix-core kernel
// (fd_split.h) applies them with agent-scope atomics; a host program
// (tests/c/steal_protocol.hip) drives them through random interleavings.
//
// Word (64 bits): chunks the owner claimed after its first (bits 0-19),
// chunks taken from the back (20-39), steals (40-43), and the share's chunk
// count (44-63, published with the owner's first claim; 0 until then, which
// makes the share look empty). Chunk 0 belongs to the owner without a
// claim; its run is [0, 1 + front), each take [n - back - m, n - back).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fd {

constexpr int kStealBackShift = 20;
constexpr int kStealCountShift = 40;
constexpr int kStealChunksShift = 44;
constexpr unsigned long long kStealField = (1ull << 20) - 1;
constexpr int kStealMaxChunks = (1 << 20) - 2;  // front and back stay within 20 bits

__host__ __device__ inline int steal_front(unsigned long long w) { return (int)(w & kStealField); }
__host__ __device__ inline int steal_back(unsigned long long w) {
  return (int)((w >> kStealBackShift) & kStealField);
}
__host__ __device__ inline int steal_count(unsigned long long w) {
  return (int)((w >> kStealCountShift) & 15ull);
}
__host__ __device__ inline int steal_chunks(unsigned long long w) {
  return (int)(w >> kStealChunksShift);
}
// Chunks of a share no run has taken yet (negative once it is exhausted).
__host__ __device__ inline int steal_unclaimed(unsigned long long w) {
  return steal_chunks(w) - 1 - steal_front(w) - steal_back(w);
}

// What the owner of a share of nc >= 2 chunks adds with its first claim:
// the claim of chunk 1 and the chunk count.
__host__ __device__ inline unsigned long long steal_first_claim(int nc) {
  return 1ull + ((unsigned long long)nc << kStealChunksShift);
}
// What the owner adds with each later claim.
constexpr unsigned long long kStealClaim = 1ull;

// The chunk an owner's claim gave it, from the word value its fetch_add
// replaced, or -1: the run ends. nc is the owner's own chunk count (the
// word does not hold it before the first claim). A claim succeeds only
// below the back count of the value it replaced.
__host__ __device__ inline int steal_claimed_chunk(unsigned long long old, int nc) {
  const int chunk = 1 + steal_front(old);
  return chunk < nc - steal_back(old) ? chunk : -1;
}

// A thief's take from a share whose word holds w, with at most cap steals
// per share: m chunks (0: nothing to take), the word to swap in with a
// compare-exchange that expects w, and on success the run [c0, c1) and the
// steal slot. It takes the back half of the unclaimed chunks, rounded up:
// the owner keeps the front half plus the chunk it is streaming. The run
// lies above the front count of w, so it never meets a claim that w has
// not seen: such a claim, made later, sees the raised back count.
struct StealTake {
  int m;
  unsigned long long want;
  int c0, c1, slot;
};

__host__ __device__ inline StealTake steal_take(unsigned long long w, int cap) {
  StealTake t{0, w, 0, 0, 0};
  const int u = steal_unclaimed(w);
  if (u < 1 || steal_count(w) >= cap) return t;
  t.m = (u + 1) / 2;
  t.want = w + ((unsigned long long)t.m << kStealBackShift) + (1ull << kStealCountShift);
  const int n = steal_chunks(w), bk = steal_back(w);
  t.c0 = n - bk - t.m;
  t.c1 = n - bk;
  t.slot = steal_count(w);
  return t;
}

}  // namespace fd
