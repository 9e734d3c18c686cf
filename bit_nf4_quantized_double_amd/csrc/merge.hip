// Merge of the trained adapter into the frozen weight, for shipping a single
// weight file ([P1] "Shipping: merge, re-quantize, verify": merge into a
// 16-bit copy, then re-quantize for serving; [P5] "QLoRA", "Walking through
// the tooling": W' = W + scaled B A at inference):
//
//     Wm[n][k] = bf16( Wbf[n][k] + s * sum_j B[n][j] * A[j][k] ),  s = fp32(alpha / r)
//
// Wbf = bf16(level[c] * fp32(q8 * s2)) is decoded from the stored triple
// exactly as in the products; the rank-r sum is accumulated in fp32 and the
// result rounded once to bf16 (round to nearest even).
//
// Workgroup: 4 waves over a 256-column slice of the weight; the slice of A
// (RP x 256, zero-padded to RP = 16, 32 or 64 ranks) is staged once in LDS
// and each wave then walks 16-row blocks on its own, with no workgroup
// barrier.  The rank-r product of a 16 x 256 block runs on
// v_mfma_f32_16x16x32_bf16 (v_mfma_f32_16x16x16_bf16 for up to 16 ranks,
// so that rank 16 neither reads nor multiplies 16 ranks of zeros) with the
// operands arranged so the accumulator lands where the output goes:
// the MFMA's M index runs over columns, permuted so that lane l ends up
// holding t[n][64 g + 0 .. 63] of row n = l & 15, g = l >> 4 -- exactly one
// 64-weight block.  The lane decodes that block's 32 bytes of codes (with
// the block's 16 decoded values as a byte-plane table in registers, looked
// up with v_perm_b32: no LDS reads; the element-order lookup, whose order
// the pairing with t follows), adds s * t and puts the 128 bytes of merged
// weight in a wave-private LDS tile,
// which the wave reads back row by row so every store instruction writes two
// contiguous 512-byte rows (16-byte pieces of 64 separate rows per store ran
// at half the speed).  The M-operand comes from the LDS copy of A through
// the transposing ds_read_b64_tr_b16, the N-operand is B[n][j] (16 bytes of
// a row per lane).
#include <algorithm>

#include "common.h"
#include "nf4_lut.h"

namespace qlora {
namespace {

typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(8))) short i16x8;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kTileK = 256;       // weight columns per workgroup
constexpr int kWaveRows = 16;     // rows per wave block
constexpr int kSubBlocks = 2;     // 16-row blocks per wave (workgroup: 4 x 2 x 16 rows; 4 and 8 were
                                  // 5-7 % and 15 % slower on the 70B shapes: fewer workgroups in flight)
constexpr int kRowsPerWg = 4 * kWaveRows * kSubBlocks;
// bf16 per row of the A copy: 8 words mod 32 banks between rows, so the 16
// lanes of a transposing read (4 rows x 4 eight-byte pieces) hit 32 banks
constexpr int kAPitch = kTileK + 16;
// bf16 per row of a wave's output staging tile: 4 words mod 32 banks between
// rows, so 8 lanes writing 16 bytes each to 8 rows hit 32 banks
constexpr int kOPitch = kTileK + 8;

// 8 consecutive bf16 of a row, elements past `valid` (and everything when
// !ok) read as zero.
__device__ __forceinline__ uint4 load8(const uint16_t* p, int valid, bool ok, bool vec) {
  if (!ok || valid <= 0) return make_uint4(0, 0, 0, 0);
  if (vec && valid >= 8) return *reinterpret_cast<const uint4*>(p);
  uint16_t h[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = i < valid ? p[i] : (uint16_t)0;
  return make_uint4(h[0] | (uint32_t)h[1] << 16, h[2] | (uint32_t)h[3] << 16, h[4] | (uint32_t)h[5] << 16,
                    h[6] | (uint32_t)h[7] << 16);
}

// The lane's block table, all 16 entries bf16(level[c] * a), as the two
// byte-plane halves decode8_lut_hl reads ("a" = levels 0..7, "b" = 8..15):
// a lane here decodes a whole block, so it builds the whole table itself.
__device__ __forceinline__ Lut block_lut(const Nf4Consts& c, float a) {
  uint32_t p[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] = pack_bf16x2(c.level[2 * i] * a, c.level[2 * i + 1] * a);
  Lut L;
  L.alo0 = __builtin_amdgcn_perm(p[1], p[0], 0x06040200u);
  L.ahi0 = __builtin_amdgcn_perm(p[1], p[0], 0x07050301u);
  L.alo1 = __builtin_amdgcn_perm(p[3], p[2], 0x06040200u);
  L.ahi1 = __builtin_amdgcn_perm(p[3], p[2], 0x07050301u);
  L.blo0 = __builtin_amdgcn_perm(p[5], p[4], 0x06040200u);
  L.bhi0 = __builtin_amdgcn_perm(p[5], p[4], 0x07050301u);
  L.blo1 = __builtin_amdgcn_perm(p[7], p[6], 0x06040200u);
  L.bhi1 = __builtin_amdgcn_perm(p[7], p[6], 0x07050301u);
  return L;
}

template <int RP>
__global__ __launch_bounds__(256) void k_merge(const uint4* __restrict__ codes, const uint8_t* __restrict__ q8,
                                               const float* __restrict__ s2, int N, int K,
                                               const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                                               int r, float s, uint16_t* __restrict__ out, Nf4Consts c) {
  __shared__ __attribute__((aligned(16))) uint16_t sa[RP * kAPitch];
  __shared__ __attribute__((aligned(16))) uint16_t so[4 * kWaveRows * kOPitch];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k0 = blockIdx.x * kTileK, n0 = blockIdx.y * kRowsPerWg;
  const bool vec = (r & 7) == 0;

  // A[:, k0 : k0 + 256] -> LDS (rows j >= r and columns >= K are zero).
  // Column k0 + 64 p + 4 m + e (p < 4, m < 16, e < 4) is stored at
  // 16 m + 4 p + e, so MFMA tile m reads a contiguous 16-column window.
  for (int idx = tid; idx < RP * (kTileK / 8); idx += 256) {
    const int j = idx / (kTileK / 8), kl = 8 * (idx % (kTileK / 8)), k = k0 + kl;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (j < r && k < K && in_bounds((int64_t)j * K + k, 8, (int64_t)r * K))
      v = *reinterpret_cast<const uint4*>(A + (int64_t)j * K + k);
    const int p = kl >> 6, m = (kl & 63) >> 2;  // m even: the 8 columns are tiles m, m + 1
    uint16_t* d = sa + j * kAPitch + 16 * m + 4 * p;
    *reinterpret_cast<uint2*>(d) = make_uint2(v.x, v.y);
    *reinterpret_cast<uint2*>(d + 16) = make_uint2(v.z, v.w);
  }
  __syncthreads();

  const int row = lane & 15, g = lane >> 4;
  const int p = row & 3, q = row >> 2;  // transposing-read address of this lane
  const int kl = 64 * g;                // this lane's block of columns in the slice
  const bool kok = k0 + kl < K;

  // operands of one 16-row block held in registers: this lane's 64 codes
  // and block scale, and its B fragments (B[n][32 u + 8 g .. + 7]).  The
  // next block's are requested before the current one is computed.
  // RP = 16: v_mfma_f32_16x16x16_bf16, 4 ranks per lane group (lane group
  // g: ranks 4 g .. 4 g + 3); else the 32-deep MFMA, 8 ranks per group.
  constexpr int KD = RP == 16 ? 16 : 32;  // MFMA depth
  constexpr int NU = RP / KD;             // MFMAs per output tile
  constexpr int RG = KD / 4;              // ranks per lane group
  uint4 cw[2];
  float sc;
  uint4 bf[NU];
  auto fetch = [&](int nb) {
    const int n = nb + row;
    const uint32_t e = (uint32_t)n * (uint32_t)K + (uint32_t)(k0 + kl);  // first weight of the block
    const int64_t nw = (int64_t)N * K, nblk = nw / 64;
    const bool ok = n < N && kok && in_bounds(e >> 5, 2, nw / 32) && in_bounds(e >> 6, 1, nblk) &&
                    in_bounds(e >> 14, 1, (nblk + 255) / 256);
    cw[0] = ok ? codes[e >> 5] : make_uint4(0, 0, 0, 0);
    cw[1] = ok ? codes[(e >> 5) + 1] : make_uint4(0, 0, 0, 0);
    sc = ok ? block_scale(q8, s2, e >> 6) : 0.f;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int j = KD * u + RG * g;
      const int64_t bi = (int64_t)n * r + j, bn = (int64_t)N * r;
      if (RG == 8) {
        bf[u] = load8(B + bi, r - j, n < N && in_bounds(bi, min(8, max(r - j, 0)), bn), vec);
      } else if ((r & 3) == 0) {  // 4 ranks of a row, 8-byte aligned
        const uint2 v = (n < N && j < r && in_bounds(bi, 4, bn)) ? *reinterpret_cast<const uint2*>(B + bi)
                                                                 : make_uint2(0, 0);
        bf[u] = make_uint4(v.x, v.y, 0u, 0u);
      } else {
        uint16_t h[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = (n < N && j + i < r && in_bounds(bi + i, 1, bn)) ? B[bi + i] : (uint16_t)0;
        bf[u] = make_uint4(h[0] | (uint32_t)h[1] << 16, h[2] | (uint32_t)h[3] << 16, 0u, 0u);
      }
    }
  };
  const int nw0 = n0 + kWaveRows * wave;
  fetch(nw0);

  for (int sb = 0; sb < kSubBlocks; ++sb) {
    const int nb = nw0 + 4 * kWaveRows * sb;
    if (nb >= N) break;  // uniform over the wave
    const uint4 cc0 = cw[0], cc1 = cw[1];
    const float scc = sc;
    uint4 bcur[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) bcur[u] = bf[u];
    if (sb + 1 < kSubBlocks) fetch(nb + 4 * kWaveRows);

    // acc[m][v] = t[nb + row][k0 + 64 g + 4 m + v] = sum_j A[j][k] B[n][j]
    f32x4 acc[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int jb = KD * u + RG * g + q;
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        // lane p + 4 q addresses row jb, stored columns 16 m + 4 p .. + 3; it
        // receives stored column 16 m + (lane & 15), rows jb - q .. + 3 (and + 4 .. + 7)
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(sa + jb * kAPitch + 16 * m + 4 * p));
        if (RG == 8) {
          const i16x4 hi =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(sa + (jb + 4) * kAPitch + 16 * m + 4 * p));
          const i16x8 av = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                           __builtin_bit_cast(bf16x8, bcur[u]), acc[m], 0, 0, 0);
        } else {
          const i16x4 bn = __builtin_bit_cast(i16x4, make_uint2(bcur[u].x, bcur[u].y));
          acc[m] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(lo, bn, acc[m], 0, 0, 0);
        }
      }
    }
    // decode the block and form Wm = bf16(Wbf + s * t) into this wave's
    // staging tile (row, columns 64 g .. + 63)
    uint16_t* sw = so + wave * (kWaveRows * kOPitch);
    const uint32_t cwd[8] = {cc0.x, cc0.y, cc0.z, cc0.w, cc1.x, cc1.y, cc1.z, cc1.w};
    const Lut L = block_lut(c, scc);
    const EoConsts ek = eo_consts();
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      // weights 8 d .. 8 d + 7 (tiles 2 d, 2 d + 1), decoded in the element
      // order 0, 2, 4, 6, 1, 3, 5, 7: wb = {w0 w2, w4 w6, w1 w3, w5 w7}
      const uint4 wb = decode8_lut_hl(L, cwd[d], ek);
      float w[8];
      w[0] = bf16_to_f32((uint16_t)(wb.x & 0xFFFFu)); w[2] = bf16_to_f32((uint16_t)(wb.x >> 16));
      w[4] = bf16_to_f32((uint16_t)(wb.y & 0xFFFFu)); w[6] = bf16_to_f32((uint16_t)(wb.y >> 16));
      w[1] = bf16_to_f32((uint16_t)(wb.z & 0xFFFFu)); w[3] = bf16_to_f32((uint16_t)(wb.z >> 16));
      w[5] = bf16_to_f32((uint16_t)(wb.w & 0xFFFFu)); w[7] = bf16_to_f32((uint16_t)(wb.w >> 16));
      uint32_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4& t = acc[2 * d + (i >> 1)];
        // w + s * t with one rounding (fused multiply-add), then bf16 RNE
        o[i] = pack_bf16x2(__builtin_fmaf(s, t[2 * (i & 1)], w[2 * i]), __builtin_fmaf(s, t[2 * (i & 1) + 1], w[2 * i + 1]));
      }
      *reinterpret_cast<uint4*>(sw + row * kOPitch + kl + 8 * d) = make_uint4(o[0], o[1], o[2], o[3]);
    }
    // LDS operations of one wave complete in order: read the tile back row by
    // row (two 512-byte rows per instruction) and write it out coalesced
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < kWaveRows / 2; ++i) {
      const int rr = 2 * i + (lane >> 5), cl = 8 * (lane & 31);
      const uint4 v = *reinterpret_cast<const uint4*>(sw + rr * kOPitch + cl);
      typedef __attribute__((ext_vector_type(4))) unsigned v4u;
      if (nb + rr < N && k0 + cl < K && in_bounds((int64_t)(nb + rr) * K + k0 + cl, 8, (int64_t)N * K))
        __builtin_nontemporal_store(v4u{v.x, v.y, v.z, v.w},
                                    reinterpret_cast<v4u*>(out + (size_t)(nb + rr) * K + k0 + cl));
    }
    __builtin_amdgcn_wave_barrier();
  }
}

}  // namespace

QLORA_OOB_READER(oob_count_merge)

hipError_t launch_merge(const uint8_t* codes, const uint8_t* q8, const float* s2, int N, int K, const uint16_t* A,
                        const uint16_t* B, int r, float s, uint16_t* out, hipStream_t st) {
  const dim3 grid((K + kTileK - 1) / kTileK, (N + kRowsPerWg - 1) / kRowsPerWg);
  const uint4* cw = reinterpret_cast<const uint4*>(codes);
  if (r <= 16)
    hipLaunchKernelGGL(k_merge<16>, grid, dim3(256), 0, st, cw, q8, s2, N, K, A, B, r, s, out, nf4_consts());
  else if (r <= 32)
    hipLaunchKernelGGL(k_merge<32>, grid, dim3(256), 0, st, cw, q8, s2, N, K, A, B, r, s, out, nf4_consts());
  else
    hipLaunchKernelGGL(k_merge<64>, grid, dim3(256), 0, st, cw, q8, s2, N, K, A, B, r, s, out, nf4_consts());
  return hipGetLastError();
}

}  // namespace qlora
