// LoRA dropout of the adapter input: a keep mask drawn from a counter-based
// generator, so the backward regenerates it instead of storing it.
//
// The pages' adapter configurations use lora_dropout = 0.05 ([P1] "A complete
// run on a 12 GB-class GPU"; [P5] "Walking through the tooling").  Element
// (m, k) of the [M x K] adapter input, flat index e = m K + k, is kept iff
// word (e & 3) of Philox4x32-10(counter = (lo32(e >> 2), hi32(e >> 2), 0, 0),
// key = (lo32(seed), hi32(seed))) is >= thr = floor(p 2^32).  The generator
// is the one of Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
// easy as 1, 2, 3" (SC'11): ten rounds of two 32 x 32 -> 64-bit products
// with a Weyl-sequence key schedule.  The 1 / (1 - p) of inverted dropout is
// folded into the adapter scale by the caller; the kernels only zero.
#pragma once

#include "common.h"

namespace qlora {

struct DropMask {
  uint32_t thr;     // floor(p 2^32); 0 keeps every element
  uint32_t k0, k1;  // seed, low and high word
};

__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
  constexpr uint32_t kM0 = 0xD2511F53u, kM1 = 0xCD9E8D57u;  // round multipliers
  constexpr uint32_t kW0 = 0x9E3779B9u, kW1 = 0xBB67AE85u;  // key increments
#pragma unroll
  for (int rnd = 0; rnd < 10; ++rnd) {
    if (rnd) { k0 += kW0; k1 += kW1; }
    const uint32_t hi0 = __umulhi(kM0, c.x), lo0 = kM0 * c.x;
    const uint32_t hi1 = __umulhi(kM1, c.z), lo1 = kM1 * c.z;
    c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
  }
  return c;
}

// Zero the dropped elements of 8 consecutive bf16 of the adapter input whose
// first flat index e is a multiple of 4 (two generator blocks).
__device__ __forceinline__ uint4 drop8(uint4 v, uint64_t e, const DropMask& d) {
  const uint64_t q = e >> 2;
  const uint4 a = philox4x32_10(make_uint4((uint32_t)q, (uint32_t)(q >> 32), 0u, 0u), d.k0, d.k1);
  const uint4 b = philox4x32_10(make_uint4((uint32_t)(q + 1), (uint32_t)((q + 1) >> 32), 0u, 0u), d.k0, d.k1);
  auto keep2 = [&](uint32_t w, uint32_t u_lo, uint32_t u_hi) {
    return (u_lo >= d.thr ? (w & 0x0000FFFFu) : 0u) | (u_hi >= d.thr ? (w & 0xFFFF0000u) : 0u);
  };
  return make_uint4(keep2(v.x, a.x, a.y), keep2(v.y, a.z, a.w), keep2(v.z, b.x, b.y), keep2(v.w, b.z, b.w));
}

}  // namespace qlora
