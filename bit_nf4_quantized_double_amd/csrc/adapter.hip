// Adapter passes of the GEMM path (more than 16 tokens) of the QLoRA linear
// ([P1] "The mechanism in brief": the adapter adds (alpha / r) B A x; the
// backward gives gradients for A and B, never for W).
//
// Row pass, one read of the activations act [M x R] (X in the forward, dY in
// the backward):
//   - writes the fragment-tiled copy of act that the fused GEMM reads
//     (gemm_args.h), and
//   - forms the fp32 partial sums of act w^T over S ranges of the reduction:
//     part[z][m][j] (j < rp = r rounded up to 8), w = A [r x R] (U = X A^T)
//     or B^T (V = dY B).  The GEMM that consumes U~ = E(s U) or V~ = E(s V)
//     adds the S partials in order in its prologue (and writes U~ / V~ out).
// Column pass, after the dX GEMM, one read per job over all M tokens:
//   dA = V~^T (mask * X)   [r x K]      dB = dY^T U~   stored [N x r]
// in fixed orders (no atomics), no partial sums.
//
// Both run v_mfma_f32_32x32x16 on 16-bit elements (bf16, or fp16 for the
// fp16 instance) with the rank on a 32-wide side (zero-padded).
#include <algorithm>

#include "common.h"
#include "dropout.h"
#include "gemm_args.h"
#include "nf4_lut.h"

namespace qlora {

// Splits of the row pass: about one workgroup (32 rows x one range of
// 128-wide chunks) per compute unit, at least 8 chunks per split (one per
// wave), at most 8 splits (the GEMM prologue adds them up), none empty.
RowpassPlan rowpass_plan(int64_t M, int64_t R, int cus) {
  RowpassPlan p;
  p.nch = (int)((R + 127) / 128);
  const int64_t mb = std::max<int64_t>(1, (M + 31) / 32);
  int64_t s = (std::max(cus, 1) + mb - 1) / mb;
  s = std::min<int64_t>(s, std::max<int64_t>(1, p.nch / 8));
  s = std::max<int64_t>(1, std::min<int64_t>(s, 8));
  p.cps = p.nch > 0 ? (int)((p.nch + s - 1) / s) : 0;
  p.S = p.nch > 0 ? (p.nch + p.cps - 1) / p.cps : 1;
  return p;
}

int rank_pitch(int r) { return (r + 7) & ~7; }

size_t rowpass_part_bytes(int64_t M, int64_t R, int r, int cus) {
  return (size_t)rowpass_plan(M, R, cus).S * (size_t)M * (size_t)rank_pitch(r) * 4u;
}

namespace {

typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(8))) short i16x8;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

struct RowpassArgs {
  const uint16_t* in;  // [M x R]
  int M, R;
  const uint16_t* w;   // CONTIG: A [r x R]; else B [R x r]
  int r, S, cps;
  float* part;         // [S][M][rp] fp32
  int rp;
  uint16_t* tiled;     // fragment-tiled copy of `in` (null: none)
  int kbp;
  bool eo;             // the copy in the forward's element order
  DropMask drop;       // dropout of `in` in the product (CONTIG only; thr 0: none)
  // Keep-mask bits of the [M x mK] adapter input (mdrop, the backward's
  // dropout) written by the pass over dY for the column pass: word w of row
  // m holds elements 32 w .. 32 w + 31 (bit b = element 32 w + b).  This
  // workgroup writes its rows' words [z wps, (z + 1) wps); null: none.
  uint32_t* mbits;
  int mwords;          // mK / 32
  DropMask mdrop;
};

// 8 consecutive 16-bit elements at element e of a buffer, the first `valid`
// real and the rest zero.  vec (uniform): e is a multiple of 8, so all 8
// real elements come in one 16-byte load.
__device__ __forceinline__ uint4 ld8(__amdgpu_buffer_rsrc_t rs, uint32_t e, bool ok, int valid, bool vec) {
  if (!ok || valid <= 0) return make_uint4(0, 0, 0, 0);
  if (vec && valid >= 8) return buf_load16(rs, 2u * e);
  uint32_t h[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = i < valid ? __builtin_amdgcn_raw_buffer_load_b16(rs, 2u * (e + i), 0, 0) : 0u;
  return make_uint4(h[0] | h[1] << 16, h[2] | h[3] << 16, h[4] | h[5] << 16, h[6] | h[7] << 16);
}

// The 32x32x16 MFMA operand with k along the rows of a row-major LDS tile
// (pitch in elements): lane l gets column col0 + (l & 31), rows k0 + 8 (l >> 5)
// .. + 7, through two transposing ds_read_b64_tr_b16.
__device__ __forceinline__ uint4 tr_operand(const uint16_t* s, int pitch, int k0, int col0, int lane) {
  const int g = lane >> 4, i = lane & 15;
  const int cb = col0 + (g & 1) * 16 + 4 * (i & 3);
  const int nb = k0 + 8 * (g >> 1) + (i >> 2);
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(s + nb * pitch + cb));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(s + (nb + 4) * pitch + cb));
  return __builtin_bit_cast(uint4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Waves per row-pass workgroup: 8, or 4 for ranks above 32 (LDS).
template <int RT2>
struct RowpassWaves {
  static constexpr int n = RT2 == 1 ? 8 : 4;
};

// Workgroup (32-row block, split z): its waves take the split's 128-wide
// chunks in turn.  Per chunk a wave loads the 32 x 128 activation tile with
// 16 lanes per 256-byte row segment (the fast pattern for global loads),
// passes it through its LDS region to get the 8 MFMA A-operand fragments,
// stores those to the tiled copy (1 KB contiguous each), stages the chunk of
// w in LDS and runs 8 MFMAs per 32 ranks.  The waves' sums are added in wave
// order at the end.
template <bool CONTIG, int RT2, typename E, bool MK = false>
__global__ __launch_bounds__(64 * RowpassWaves<RT2>::n) void k_rowpass(RowpassArgs a) {
  constexpr int NW = RowpassWaves<RT2>::n;
  constexpr int kRanks = 32 * RT2;
  constexpr int kAP = 128 + 8;                            // activation tile [32][kAP]
  constexpr int kAct = 32 * kAP;
  constexpr int kWP = CONTIG ? 128 + 8 : kRanks + 8;      // staged w: [rank][k] or [k][rank]
  constexpr int kW = CONTIG ? kRanks * kWP : 128 * kWP;
  constexpr int kWave = kAct + kW;                        // elements per wave
  constexpr int kRP = kRanks + 1;                         // reduction pitch (odd: no bank conflicts)
  constexpr int kRed = NW * 32 * kRP;                     // fp32 sums of the waves
  constexpr int kLds = NW * kWave * 2 > kRed * 4 ? NW * kWave * 2 : kRed * 4;
  __shared__ __attribute__((aligned(16))) uint8_t s_raw[kLds];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int mb = blockIdx.x, z = blockIdx.y;
  const int m0 = 32 * mb;
  const int nch = (a.R + 127) >> 7;
  const int c_lo = z * a.cps, c_hi = min(nch, c_lo + a.cps);
  uint16_t* sa = reinterpret_cast<uint16_t*>(s_raw) + wave * kWave;
  uint16_t* sw = sa + kAct;
  const __amdgpu_buffer_rsrc_t rin = make_rsrc(a.in, (uint32_t)((uint64_t)a.M * a.R * 2));
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w, (uint32_t)((uint64_t)a.r * a.R * 2));
  const int lrow = lane >> 4, lcol = 8 * (lane & 15);  // load pattern: 4 rows x 16 lanes

  f32x16 acc[RT2];
#pragma unroll
  for (int t = 0; t < RT2; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[t][v] = 0.f;

  // the chunk of w: CONTIG A[j][k0 .. k0 + 127] -> sw[j][k]; else
  // B[k0 .. k0 + 127][j] -> sw[k][j]; ranks past r are zero
  constexpr int kLoads = (CONTIG ? kRanks * 16 : 128 * (kRanks / 8)) / 64;
  auto load = [&](int c, uint4 (&xv)[8], uint4 (&wv)[kLoads]) {
    const int k0 = 128 * c;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int m = m0 + 4 * u + lrow, k = k0 + lcol;
      xv[u] = buf_load16(rin, m < a.M && k < a.R ? ((uint32_t)m * (uint32_t)a.R + (uint32_t)k) * 2u : kOOB);
    }
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      const int idx = lane + 64 * u;
      if (CONTIG) {
        const int j = idx >> 4, cc = idx & 15, k = k0 + 8 * cc;
        wv[u] = ld8(rw, (uint32_t)j * (uint32_t)a.R + (uint32_t)k, j < a.r && k < a.R, 8, true);
      } else {
        const int kk = idx / (kRanks / 8), jc = idx % (kRanks / 8), k = k0 + kk;
        wv[u] = ld8(rw, (uint32_t)k * (uint32_t)a.r + 8u * jc, k < a.R, a.r - 8 * jc, (a.r & 7) == 0);
      }
    }
  };

  // The wave's chunks c_lo + wave, + NW, ...: once a chunk is in LDS the
  // next one's loads are issued into the same registers, so they are in
  // flight while the chunk is stored and multiplied.
  uint4 xv[8], wv[kLoads];
  if (c_lo + wave < c_hi) load(c_lo + wave, xv, wv);
  if (MK) {
    // the keep-mask words, while the first chunk's loads are in flight: 32
    // bits from 8 generator blocks per word (dropout.h)
    const int wps = (a.mwords + a.S - 1) / a.S, w0 = z * wps, nw = max(0, min(wps, a.mwords - w0));
    for (int it = tid; it < 32 * nw; it += 64 * NW) {
      const int rl = it / nw, w = w0 + (it - rl * nw), m = m0 + rl;
      if (m >= a.M) continue;
      const uint64_t q0 = ((uint64_t)m * (uint64_t)a.mwords * 32u + 32u * (uint64_t)w) >> 2;
      uint32_t bits = 0;
#pragma unroll 2
      for (int i = 0; i < 8; ++i) {
        const uint64_t q = q0 + (uint64_t)i;
        const uint4 u = philox4x32_10(make_uint4((uint32_t)q, (uint32_t)(q >> 32), 0u, 0u), a.mdrop.k0, a.mdrop.k1);
        bits |= ((u.x >= a.mdrop.thr ? 1u : 0u) | (u.y >= a.mdrop.thr ? 2u : 0u) | (u.z >= a.mdrop.thr ? 4u : 0u) |
                 (u.w >= a.mdrop.thr ? 8u : 0u)) << (4 * i);
      }
      if (in_bounds((int64_t)m * a.mwords + w, 1, (int64_t)a.M * a.mwords)) a.mbits[(size_t)m * a.mwords + w] = bits;
    }
  }
  for (int c = c_lo + wave; c < c_hi; c += NW) {
    const int k0 = 128 * c;
#pragma unroll
    for (int u = 0; u < 8; ++u) *reinterpret_cast<uint4*>(sa + (4 * u + lrow) * kAP + lcol) = xv[u];
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      const int idx = lane + 64 * u;
      if (CONTIG) *reinterpret_cast<uint4*>(sw + (idx >> 4) * kWP + 8 * (idx & 15)) = wv[u];
      else *reinterpret_cast<uint4*>(sw + (idx / (kRanks / 8)) * kWP + 8 * (idx % (kRanks / 8))) = wv[u];
    }
    if (c + NW < c_hi) load(c + NW, xv, wv);
    // LDS operations of one wave complete in order: the reads below see the
    // stores above, and the next chunk's stores come after these reads
    __builtin_amdgcn_wave_barrier();
    // fragment f: lane l holds row l & 31, columns 16 f + 8 (l >> 5) .. + 7
    uint4 xf[8];
#pragma unroll
    for (int f = 0; f < 8; ++f)
      xf[f] = *reinterpret_cast<const uint4*>(sa + (lane & 31) * kAP + 16 * f + 8 * (lane >> 5));
    if (a.tiled) {
#pragma unroll
      for (int f = 0; f < 8; ++f) {
        const int kb = 8 * c + f;
        if (kb < a.kbp && in_bounds(((int64_t)mb * a.kbp + kb) * 512 + 8 * lane, 8,
                                    (int64_t)tiled_mbp(a.M) * a.kbp * 512))
          *reinterpret_cast<uint4*>(a.tiled + ((size_t)mb * a.kbp + kb) * 512 + 8 * lane) =
              a.eo ? x_order_even_odd(xf[f]) : xf[f];
      }
    }
    if (CONTIG && a.drop.thr) {
      const uint64_t row = (uint64_t)(m0 + (lane & 31));
#pragma unroll
      for (int f = 0; f < 8; ++f)
        xf[f] = drop8(xf[f], row * (uint64_t)a.R + (uint64_t)(k0 + 16 * f + 8 * (lane >> 5)), a.drop);
    }
#pragma unroll
    for (int f = 0; f < 8; ++f)
#pragma unroll
      for (int t = 0; t < RT2; ++t) {
        uint4 bf;
        if (CONTIG)
          bf = *reinterpret_cast<const uint4*>(sw + (32 * t + (lane & 31)) * kWP + 16 * f + 8 * (lane >> 5));
        else
          bf = tr_operand(sw, kWP, 16 * f, 32 * t, lane);
        acc[t] = E::mfma32(E::vec(xf[f]), E::vec(bf), acc[t]);
      }
    __builtin_amdgcn_wave_barrier();
  }

  // the waves' sums, added in wave order
  __syncthreads();
  float* red = reinterpret_cast<float*>(s_raw);
#pragma unroll
  for (int t = 0; t < RT2; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int rl = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3), j = 32 * t + (lane & 31);
      red[(wave * 32 + rl) * kRP + j] = acc[t][v];
    }
  __syncthreads();
  for (int idx = tid; idx < 32 * a.rp; idx += 64 * NW) {
    const int rl = idx / a.rp, j = idx - rl * a.rp;
    if (m0 + rl >= a.M) continue;
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) s += red[(w * 32 + rl) * kRP + j];
    if (in_bounds(((int64_t)z * a.M + m0 + rl) * a.rp + j, 1, (int64_t)a.S * a.M * a.rp))
      a.part[((size_t)z * a.M + m0 + rl) * a.rp + j] = s;
  }
}

struct ColpassJob {
  const uint16_t* in;  // [M x C]: X (dA) or dY (dB)
  int C;
  const uint16_t* v;   // [M x r]: V~ (dA) or U~ (dB)
  float* out;          // dA [r x C] (trans false) or dB [C x r] (trans true)
  bool trans;
  DropMask drop;       // dropout of `in` (dA only)
  int nblk;            // 64-column blocks
  const uint32_t* mbits;  // the keep mask of `in` as bits (see RowpassArgs), or null: from drop
};

// Workgroup = one 64-column block of one job, all M rows: 8 waves take
// 64-row chunks in turn; a chunk of `in` and of `v` is staged in the wave's
// LDS region and read back transposed as the two MFMA operands (k along the
// rows).  out^T[c][j] = sum_m in[m][c] v[m][j]; the 8 waves' sums are added
// in wave order at the end.  Once a chunk is in LDS the next one's loads are
// issued into the same registers, so they are in flight while the chunk is
// multiplied.
template <int RT2, typename E, bool MB = false>
__global__ __launch_bounds__(512) void k_colpass(ColpassJob j0, ColpassJob j1, int M, int r) {
  constexpr int kRanks = 32 * RT2;
  constexpr int kXP = 64 + 8, kVP = kRanks + 8;                 // LDS pitches
  constexpr int kWave = 64 * kXP + 64 * kVP;                    // elements per wave
  constexpr int kRP = kRanks + 1;                               // reduction pitch (odd: no bank conflicts)
  constexpr int kRed = 8 * 64 * kRP;                            // fp32 sums of the 8 waves
  constexpr int kLds = 8 * kWave * 2 > kRed * 4 ? 8 * kWave * 2 : kRed * 4;
  __shared__ __attribute__((aligned(16))) uint8_t s_raw[kLds];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool second = (int)blockIdx.x >= j0.nblk;
  const ColpassJob& jb = second ? j1 : j0;
  const int c0 = 64 * ((int)blockIdx.x - (second ? j0.nblk : 0));
  uint16_t* sx = reinterpret_cast<uint16_t*>(s_raw) + wave * kWave;
  uint16_t* sv = sx + 64 * kXP;
  const __amdgpu_buffer_rsrc_t rin = make_rsrc(jb.in, (uint32_t)((uint64_t)M * jb.C * 2));
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(jb.v, (uint32_t)((uint64_t)M * r * 2));

  f32x16 acc[2][RT2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int t = 0; t < RT2; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[ct][t][v] = 0.f;

  constexpr int kVL = kRanks / 8;  // 16-byte loads per lane of a 64-row chunk of v
  // in[m0 .. m0 + 63][c0 .. c0 + 63] (8 lanes per 128-byte row) and
  // v[m0 .. m0 + 63][0 .. r) (ranks past r zero)
  // MB: the dA job's mask from the row pass's bits (a separate instantiation)
  const bool mb = MB && jb.drop.thr != 0 && jb.mbits != nullptr;
  const __amdgpu_buffer_rsrc_t rmb = make_rsrc(jb.mbits, mb ? (uint32_t)((uint64_t)M * (jb.C >> 5) * 4) : 0u);
  auto load = [&](int ck, uint4 (&xv)[8], uint4 (&vv)[kVL], uint32_t (&mv)[8]) {
    const int m0 = 64 * ck;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int idx = lane + 64 * u, rr = idx >> 3, cc = idx & 7;
      const int m = m0 + rr, c = c0 + 8 * cc;
      xv[u] = buf_load16(rin, m < M && c < jb.C ? ((uint32_t)m * (uint32_t)jb.C + (uint32_t)c) * 2u : kOOB);
      if (mb) mv[u] = buf_load4(rmb, m < M && c < jb.C ? ((uint32_t)m * (uint32_t)(jb.C >> 5) + (uint32_t)(c >> 5)) * 4u : kOOB);
    }
#pragma unroll
    for (int u = 0; u < kVL; ++u) {
      const int idx = lane + 64 * u, rr = idx / (kRanks / 8), jc = idx % (kRanks / 8), m = m0 + rr;
      vv[u] = ld8(rv, (uint32_t)m * (uint32_t)r + 8u * jc, m < M, r - 8 * jc, (r & 7) == 0);
    }
  };

  // The wave's chunks wave, wave + 8, ...: once a chunk is in LDS the next
  // one's loads are issued into the same registers, so they are in flight
  // while the chunk is multiplied.
  const int nck = (M + 63) >> 6;
  uint4 xv[8], vv[kVL];
  uint32_t mv[8];
  if (wave < nck) load(wave, xv, vv, mv);
  for (int ck = wave; ck < nck; ck += 8) {
    const int m0 = 64 * ck;
    if (mb) {
      // 8 bits of the row's mask word per 8 elements (c is a multiple of 8)
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int cc = (lane + 64 * u) & 7;
        const uint32_t k8 = mv[u] >> ((8 * cc + c0) & 31);
        auto keep2 = [&](uint32_t w, int b) {
          return ((k8 >> b) & 1u ? (w & 0x0000FFFFu) : 0u) | ((k8 >> (b + 1)) & 1u ? (w & 0xFFFF0000u) : 0u);
        };
        xv[u] = make_uint4(keep2(xv[u].x, 0), keep2(xv[u].y, 2), keep2(xv[u].z, 4), keep2(xv[u].w, 6));
      }
    } else if (jb.drop.thr) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int idx = lane + 64 * u, rr = idx >> 3, cc = idx & 7;
        xv[u] = drop8(xv[u], (uint64_t)(m0 + rr) * (uint64_t)jb.C + (uint64_t)(c0 + 8 * cc), jb.drop);
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int idx = lane + 64 * u;
      *reinterpret_cast<uint4*>(sx + (idx >> 3) * kXP + 8 * (idx & 7)) = xv[u];
    }
#pragma unroll
    for (int u = 0; u < kVL; ++u) {
      const int idx = lane + 64 * u;
      *reinterpret_cast<uint4*>(sv + (idx / (kRanks / 8)) * kVP + 8 * (idx % (kRanks / 8))) = vv[u];
    }
    if (ck + 8 < nck) load(ck + 8, xv, vv, mv);
    // LDS operations of one wave complete in order: the reads below see the
    // stores above, and the next chunk's stores come after these reads
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      uint4 bv[RT2];
#pragma unroll
      for (int t = 0; t < RT2; ++t) bv[t] = tr_operand(sv, kVP, 16 * ks, 32 * t, lane);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const uint4 ax = tr_operand(sx, kXP, 16 * ks, 32 * ct, lane);
#pragma unroll
        for (int t = 0; t < RT2; ++t) acc[ct][t] = E::mfma32(E::vec(ax), E::vec(bv[t]), acc[ct][t]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  __syncthreads();
  float* red = reinterpret_cast<float*>(s_raw);
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int t = 0; t < RT2; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int cl = 32 * ct + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3), j = 32 * t + (lane & 31);
        red[(wave * 64 + cl) * kRP + j] = acc[ct][t][v];
      }
  __syncthreads();
  for (int idx = tid; idx < 64 * r; idx += 512) {
    // dB (trans): consecutive threads walk ranks of one column; dA: columns of one rank
    const int cl = jb.trans ? idx / r : idx % 64, j = jb.trans ? idx % r : idx / 64;
    if (c0 + cl >= jb.C) continue;
    float s = 0.f;
#pragma unroll
    for (int w8 = 0; w8 < 8; ++w8) s += red[(w8 * 64 + cl) * kRP + j];
    const int64_t oi = jb.trans ? (int64_t)(c0 + cl) * r + j : (int64_t)j * jb.C + c0 + cl;
    if (in_bounds(oi, 1, (int64_t)jb.C * r)) jb.out[oi] = s;
  }
}

// out[m][j] = E(scale * sum over z, in order, of part[z][m][j]): the same
// sum, in the same order, as the fused GEMM's prologue forms from the row
// pass's partials, for a U~ that must be bit-identical to the forward's.
template <typename E>
__global__ __launch_bounds__(256) void k_rowpass_finalize(const float* __restrict__ part, int S, int M, int r,
                                                          int rp, float scale, uint16_t* __restrict__ out) {
  const int64_t n = (int64_t)M * r;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int m = (int)(i / r), j = (int)(i - (int64_t)m * r);
    if (!in_bounds(((int64_t)(S - 1) * M + m) * rp + j, 1, (int64_t)S * M * rp)) continue;
    float s = 0.f;
    for (int z = 0; z < S; ++z) s += part[((int64_t)z * M + m) * rp + j];
    out[i] = (uint16_t)(E::pack2(scale * s, 0.f) & 0xFFFFu);
  }
}

template <bool CONTIG, typename E>
hipError_t rowpass_dispatch(const RowpassArgs& ra, dim3 grid, hipStream_t st) {
  // the keep-mask bits only from the pass over dY (a separate instantiation)
  if (!CONTIG && ra.mbits) {
    if (ra.r <= 32) hipLaunchKernelGGL((k_rowpass<false, 1, E, true>), grid, dim3(64 * RowpassWaves<1>::n), 0, st, ra);
    else hipLaunchKernelGGL((k_rowpass<false, 2, E, true>), grid, dim3(64 * RowpassWaves<2>::n), 0, st, ra);
    return hipGetLastError();
  }
  if (ra.r <= 32) hipLaunchKernelGGL((k_rowpass<CONTIG, 1, E>), grid, dim3(64 * RowpassWaves<1>::n), 0, st, ra);
  else hipLaunchKernelGGL((k_rowpass<CONTIG, 2, E>), grid, dim3(64 * RowpassWaves<2>::n), 0, st, ra);
  return hipGetLastError();
}

}  // namespace

// Row pass over act [M x R] (see above); CONTIG: w = A [r x R] (the forward's
// X A^T, with the dropout mask applied to the product operand and the tiled
// copy in the forward's element order); else w = B [R x r] (dY B, natural
// order).  part: fp32 [S][M][rank_pitch(r)], S = rowpass_plan(M, R, cus).S.
hipError_t launch_rowpass(const uint16_t* act, int M, int R, const uint16_t* w, int r, bool contig, DropMask drop,
                          float* part, uint16_t* tiled, bool f16, int cus, hipStream_t st, uint32_t* mbits,
                          int mK, DropMask mdrop) {
  if (M <= 0 || r <= 0) return hipSuccess;
  const RowpassPlan p = rowpass_plan(M, R, cus);
  RowpassArgs ra{act, M, R, w, r, p.S, p.cps, part, rank_pitch(r), tiled, tiled_kbp(R), contig, drop,
                 mdrop.thr ? mbits : nullptr, mK / 32, mdrop};
  const dim3 grid(tiled_mbp(M), p.S);
  if (contig) return f16 ? rowpass_dispatch<true, F16>(ra, grid, st) : rowpass_dispatch<true, Bf16>(ra, grid, st);
  ra.drop = DropMask{};
  return f16 ? rowpass_dispatch<false, F16>(ra, grid, st) : rowpass_dispatch<false, Bf16>(ra, grid, st);
}

// U = E(scale * sum of the row pass's partials) [M x r], S = rowpass_plan(M, R, cus).S.
hipError_t launch_rowpass_finalize(const float* part, int S, int M, int r, float scale, uint16_t* U, bool f16,
                                   hipStream_t st) {
  const int64_t n = (int64_t)M * r;
  if (n <= 0) return hipSuccess;
  const int blocks = (int)std::min<int64_t>((n + 255) / 256, 2048);
  if (f16) hipLaunchKernelGGL(k_rowpass_finalize<F16>, dim3(blocks), dim3(256), 0, st, part, S, M, r, rank_pitch(r), scale, U);
  else hipLaunchKernelGGL(k_rowpass_finalize<Bf16>, dim3(blocks), dim3(256), 0, st, part, S, M, r, rank_pitch(r), scale, U);
  return hipGetLastError();
}

// Column pass: dA = V~^T (mask * X) [r x K] and dB = dY^T U~ [N x r], all M
// tokens, one dispatch.
hipError_t launch_colpass(const uint16_t* X, int K, const uint16_t* Vt, const uint16_t* dY, int N,
                          const uint16_t* Ut, int M, int r, DropMask drop, float* dA, float* dB, bool f16,
                          hipStream_t st, const uint32_t* mbits) {
  const ColpassJob ja{X, K, Vt, dA, false, drop, (K + 63) / 64, drop.thr ? mbits : nullptr};
  const ColpassJob jb{dY, N, Ut, dB, true, DropMask{}, (N + 63) / 64, nullptr};
  const dim3 grid(ja.nblk + jb.nblk);
  if (grid.x == 0) return hipSuccess;
  if (ja.mbits) {
    if (r <= 32) {
      if (f16) hipLaunchKernelGGL((k_colpass<1, F16, true>), grid, dim3(512), 0, st, ja, jb, M, r);
      else hipLaunchKernelGGL((k_colpass<1, Bf16, true>), grid, dim3(512), 0, st, ja, jb, M, r);
    } else {
      if (f16) hipLaunchKernelGGL((k_colpass<2, F16, true>), grid, dim3(512), 0, st, ja, jb, M, r);
      else hipLaunchKernelGGL((k_colpass<2, Bf16, true>), grid, dim3(512), 0, st, ja, jb, M, r);
    }
  } else if (r <= 32) {
    if (f16) hipLaunchKernelGGL((k_colpass<1, F16>), grid, dim3(512), 0, st, ja, jb, M, r);
    else hipLaunchKernelGGL((k_colpass<1, Bf16>), grid, dim3(512), 0, st, ja, jb, M, r);
  } else {
    if (f16) hipLaunchKernelGGL((k_colpass<2, F16>), grid, dim3(512), 0, st, ja, jb, M, r);
    else hipLaunchKernelGGL((k_colpass<2, Bf16>), grid, dim3(512), 0, st, ja, jb, M, r);
  }
  return hipGetLastError();
}

QLORA_OOB_READER(oob_count_adapter)

}  // namespace qlora
