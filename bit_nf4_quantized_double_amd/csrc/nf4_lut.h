// Register lookup-table decode of packed NF4 codes to 16-bit floats (bf16 or
// fp16; only the table entries are rounded), shared by the fused GEMM and the
// few-token forward kernel.
//
// A 64-weight block has one scale a' = fp32(q8 * s2); its 16 possible
// decoded values bf16(level[c] * a') ([P1] "The mechanism in brief") form a
// per-block table.  Two lanes that decode halves of the same block each
// build half of it (levels 0..7 on the "even" lane, 8..15 on the "odd" one),
// held as byte planes (low bytes, high bytes of the bf16 values) so that
// v_perm_b32 can index them, and exchange halves with one cross-lane VALU
// move per dword.
// A lookup of 4 codes costs about 12 VALU operations; no LDS traffic.
#pragma once

#include "common.h"

namespace qlora {

struct Lut {
  uint32_t alo0, alo1, ahi0, ahi1;  // my 8 entries (byte planes)
  uint32_t blo0, blo1, bhi0, bhi1;  // partner's 8 entries
};

// How the two lanes sharing a block exchange their halves of the table.
enum class LutPartner {
  // partner = lane ^ 1, one DPP move (quad_perm [1,0,3,2]) per dword; the
  // "a" half is the lane's own, the "b" half the partner's.
  kXor1,
  // partner = lane ^ 16 (the two lanes are in adjacent 16-lane rows, the
  // even row owning levels 0..7).  One v_permlane16_swap_b32 per dword gives
  // every lane the even row's dword and the odd row's dword, so afterwards
  // "a" = levels 0..7 and "b" = levels 8..15 on both lanes: use
  // lane_mask(false) for every lane.
  kRows16,
};

// th[] = the 8 levels this lane owns; a = the block scale; E = the 16-bit
// element type the entries are rounded to (round to nearest even).
template <LutPartner P, typename E = Bf16>
__device__ __forceinline__ Lut build_lut(const float th[8], float a) {
  const uint32_t p0 = E::pack2(th[0] * a, th[1] * a);
  const uint32_t p1 = E::pack2(th[2] * a, th[3] * a);
  const uint32_t p2 = E::pack2(th[4] * a, th[5] * a);
  const uint32_t p3 = E::pack2(th[6] * a, th[7] * a);
  const uint32_t lo0 = __builtin_amdgcn_perm(p1, p0, 0x06040200u);
  const uint32_t hi0 = __builtin_amdgcn_perm(p1, p0, 0x07050301u);
  const uint32_t lo1 = __builtin_amdgcn_perm(p3, p2, 0x06040200u);
  const uint32_t hi1 = __builtin_amdgcn_perm(p3, p2, 0x07050301u);
  Lut L;
  if constexpr (P == LutPartner::kXor1) {
    L.alo0 = lo0; L.ahi0 = hi0; L.alo1 = lo1; L.ahi1 = hi1;
    L.blo0 = __builtin_amdgcn_mov_dpp(lo0, 0xB1, 0xF, 0xF, false);
    L.bhi0 = __builtin_amdgcn_mov_dpp(hi0, 0xB1, 0xF, 0xF, false);
    L.blo1 = __builtin_amdgcn_mov_dpp(lo1, 0xB1, 0xF, 0xF, false);
    L.bhi1 = __builtin_amdgcn_mov_dpp(hi1, 0xB1, 0xF, 0xF, false);
  } else {
    // permlane16_swap(v, v): first = rows (0, 0, 2, 2), second = rows (1, 1, 3, 3)
    const auto r0 = __builtin_amdgcn_permlane16_swap(lo0, lo0, false, false);
    const auto r1 = __builtin_amdgcn_permlane16_swap(hi0, hi0, false, false);
    const auto r2 = __builtin_amdgcn_permlane16_swap(lo1, lo1, false, false);
    const auto r3 = __builtin_amdgcn_permlane16_swap(hi1, hi1, false, false);
    L.alo0 = r0[0]; L.blo0 = r0[1];
    L.ahi0 = r1[0]; L.bhi0 = r1[1];
    L.alo1 = r2[0]; L.blo1 = r2[1];
    L.ahi1 = r3[0]; L.bhi1 = r3[1];
  }
  return L;
}

// Per-lane constants of the lookup: the "odd" lane of a pair owns levels 8..15.
struct LaneMask {
  uint32_t s;    // xor for my-half indices: 0 (even) or 0x08080808 (odd)
  uint32_t x;    // xor for partner-half indices: s ^ 0x08080808
  uint32_t sel;  // base byte selector 0x03020100, bit 2 flipped on odd lanes
};

__device__ __forceinline__ LaneMask lane_mask(bool odd) {
  LaneMask lm;
  lm.s = odd ? 0x08080808u : 0u;
  lm.x = lm.s ^ 0x08080808u;
  lm.sel = odd ? 0x07060504u : 0x03020100u;
  return lm;
}

__device__ __forceinline__ void lane_levels(const Nf4Consts& nf4, bool odd, float th[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) th[i] = odd ? nf4.level[8 + i] : nf4.level[i];
}

// t: bytes hold (code_i | code_{i+1} << 4); the low nibble of byte i is the
// code of output element i.  Index < 8 after the xor: my half of the table;
// >= 8: the partner's half.  Returns {w0,w1}, {w2,w3} as bf16 pairs.
__device__ __forceinline__ void lookup4(const Lut& L, uint32_t t, const LaneMask& lm, uint32_t& o01,
                                        uint32_t& o23) {
  const uint32_t s = (t & 0x0F0F0F0Fu) ^ lm.s;
  const uint32_t x = (t & 0x0F0F0F0Fu) ^ lm.x;
  const uint32_t sel = ((t >> 1) & 0x04040404u) ^ lm.sel;
  const uint32_t lo = __builtin_amdgcn_perm(__builtin_amdgcn_perm(L.blo1, L.blo0, x),
                                            __builtin_amdgcn_perm(L.alo1, L.alo0, s), sel);
  const uint32_t hi = __builtin_amdgcn_perm(__builtin_amdgcn_perm(L.bhi1, L.bhi0, x),
                                            __builtin_amdgcn_perm(L.ahi1, L.ahi0, s), sel);
  o01 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
  o23 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
}

// 8 codes (one dword, element 0 in the low nibble) -> 4 dwords of bf16 pairs.
__device__ __forceinline__ uint4 decode8_lut(const Lut& L, uint32_t d, const LaneMask& lm) {
  const uint32_t sh = d >> 4;
  uint4 o;
  lookup4(L, __builtin_amdgcn_perm(sh, d, 0x05010400u), lm, o.x, o.y);
  lookup4(L, __builtin_amdgcn_perm(sh, d, 0x07030602u), lm, o.z, o.w);
  return o;
}

// ---- element-order lookup (no nibble spread) -------------------------------
// With LutPartner::kRows16 tables ("a" = levels 0..7, "b" = levels 8..15 on
// every lane) the 8 codes of a dword are looked up without first spreading
// them into byte order: the low nibbles (elements 0, 2, 4, 6) and the high
// nibbles (1, 3, 5, 7) are indexed separately, which leaves the decoded
// values in the element order 0, 2, 4, 6, 1, 3, 5, 7.  The other MFMA
// operand must carry the same order (x_order_even_odd).

// Constants of the element-order lookup, held in VGPRs so that each
// (x & m) ^ c folds into one VALU operation (one scalar operand at most).
// `base` selects table "a" for codes 0..7: 0x03020100 with kRows16 tables
// (and with kXor1 tables on the lane that built levels 0..7); the kXor1 lane
// that built levels 8..15 holds them in "a" and takes base 0x07060504, which
// swaps the pick.
struct EoConsts {
  uint32_t m7;    // 0x07070707
  uint32_t m4;    // 0x04040404
  uint32_t base;  // 0x03020100, or 0x07060504 (see above)
};

__device__ __forceinline__ EoConsts eo_consts(bool swap_ab = false) {
  EoConsts k{0x07070707u, 0x04040404u, swap_ab ? 0x07060504u : 0x03020100u};
  asm volatile("" : "+v"(k.m7), "+v"(k.m4), "+v"(k.base));
  return k;
}

// 4 codes: entry indices (one per byte, 0..7) and selector (byte i = i, or
// i + 4 to take table "b") -> {w0,w1}, {w2,w3} as bf16 pairs.
__device__ __forceinline__ void lookup4_eo(const Lut& L, uint32_t idx, uint32_t sel, uint32_t& o01,
                                           uint32_t& o23) {
  const uint32_t lo = __builtin_amdgcn_perm(__builtin_amdgcn_perm(L.blo1, L.blo0, idx),
                                            __builtin_amdgcn_perm(L.alo1, L.alo0, idx), sel);
  const uint32_t hi = __builtin_amdgcn_perm(__builtin_amdgcn_perm(L.bhi1, L.bhi0, idx),
                                            __builtin_amdgcn_perm(L.ahi1, L.ahi0, idx), sel);
  o01 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
  o23 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
}

// 8 codes (one dword, element 0 in the low nibble) -> 8 16-bit values in the
// element order 0, 2, 4, 6, 1, 3, 5, 7, from kRows16 tables built with
// lane_levels (or kXor1 tables, see EoConsts): a code c is looked up at
// entry c & 7 of both tables and bit 3 of c picks the result.  7 operations
// per 8 codes besides the 16 permutes.
__device__ __forceinline__ uint4 decode8_lut_hl(const Lut& L, uint32_t d, const EoConsts& k) {
  const uint32_t ie = d & k.m7;                    // low nibbles: c & 7
  const uint32_t io = (d >> 4) & k.m7;             // high nibbles: c & 7
  const uint32_t se = ((d >> 1) & k.m4) ^ k.base;  // bit 3 of the low nibble -> bit 2
  const uint32_t so = ((d >> 5) & k.m4) ^ k.base;  // bit 3 of the high nibble -> bit 2
  uint4 o;
  lookup4_eo(L, ie, se, o.x, o.y);
  lookup4_eo(L, io, so, o.z, o.w);
  return o;
}

// 8 consecutive bf16 (4 dwords) -> the order 0, 2, 4, 6, 1, 3, 5, 7.
__device__ __forceinline__ uint4 x_order_even_odd(uint4 v) {
  uint4 o;
  o.x = __builtin_amdgcn_perm(v.y, v.x, 0x05040100u);
  o.y = __builtin_amdgcn_perm(v.w, v.z, 0x05040100u);
  o.z = __builtin_amdgcn_perm(v.y, v.x, 0x07060302u);
  o.w = __builtin_amdgcn_perm(v.w, v.z, 0x07060302u);
  return o;
}

}  // namespace qlora
