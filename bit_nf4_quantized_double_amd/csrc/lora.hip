// Skinny rank-r products of the adapter path ([P1] "The mechanism in brief":
// the adapter adds (alpha / r) B A x; backward gives gradients for A and B).
//
//   rowdot:   out[m][j] = bf16(scale * sum_k in[m][k] * w(j, k))       (M x r)
//             U~ = bf16(s X A^T)   and   V~ = bf16(s dY B)
//   coldot:   part[mc][j][c] = sum_{m in chunk mc} v[m][j] * in[m][c]  (fp32)
//   finalize: out = sum over chunks, in a fixed order (deterministic)
//             dA = V~^T X  [r x K]      dB = dY^T U~  -> stored [N x r]
//
// All use v_mfma_f32_16x16x32 on 16-bit elements (bf16, or fp16 for the fp16
// instance) with the rank on the 16-wide side.
#include <algorithm>

#include "common.h"
#include "dropout.h"

namespace qlora {

// K split of the rowdot kernel: enough (row block, split) workgroups to fill
// the GPU (>= 512), splits of whole 256-wide sub-chunks.
void rowdot_split(int M, int Kd, int* nsplit, int* kchunk) {
  const int rb = (M + 63) / 64;
  const int nsub = std::max(1, (Kd + 255) / 256);
  int ns = std::min(nsub, std::max(1, (512 + rb - 1) / rb));
  const int per = (nsub + ns - 1) / ns;
  ns = (nsub + per - 1) / per;
  *nsplit = ns;
  *kchunk = per * 256;
}

// fp32 partial bytes the rowdot kernel needs for these sizes (0 if unsplit).
size_t rowdot_part_bytes(int64_t M, int64_t Kd, int r) {
  int ns, kc;
  rowdot_split((int)M, (int)Kd, &ns, &kc);
  return ns > 1 ? (size_t)ns * (size_t)M * (size_t)r * 4u : 0;
}

namespace {

typedef __attribute__((ext_vector_type(8))) short i16x8;


// ---------------------------------------------------------------- rowdot ----
// out[m][j] = bf16(scale * sum_k in[m][k] * w(j, k)), j < r.
// w(j, k) = wt[j * Kd + k] when CONTIG (A is [r x K]), else wt[k * r + j]
// (B is [N x r]).
//
// Grid (row blocks of 64, K splits).  Each 256-thread workgroup covers 64
// rows (16 per wave) and one K range, walked in 256-wide sub-chunks: the
// sub-chunk of w is staged in LDS (A as [j][k], read with ds_read_b128; B as
// [k][j] -- its rows are contiguous in memory -- read with the transposing
// ds_read_b64_tr_b16), the activations go straight from global memory into
// MFMA A-operand registers, eight 16-byte loads in flight per lane.  With
// one K split the result is rounded and stored directly; otherwise fp32
// partials [split][m][j] are summed in a fixed order by k_rowdot_finalize.
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kRowdotSub = 256;  // reduction columns per LDS sub-chunk

template <bool CONTIG, int RT>
struct RowdotLds {
  // CONTIG: [RT*16][kRowdotSub + 8]; else [kRowdotSub][RT*16 + 8]
  static constexpr int kPitch = CONTIG ? kRowdotSub + 8 : RT * 16 + 8;
  static constexpr int kElems = CONTIG ? RT * 16 * kPitch : kRowdotSub * kPitch;
};

struct RowdotArgs {
  const uint16_t* in;  // [M x Kd]
  int M, Kd;
  const uint16_t* wt;  // A [r x Kd] (CONTIG) or B [Kd x r]
  int r, kchunk, nsplit;
  float scale;
  uint16_t* out;       // [M x r] bf16
  float* part;         // [nsplit][M][r] fp32, or null when nsplit == 1
  DropMask drop;       // dropout of `in` (thr 0: none)
};

// Workgroup (bx, by) = (64-row block, K split) of the rowdot grid.
template <bool CONTIG, int RT, typename E>
__device__ __forceinline__ void rowdot_body(const RowdotArgs& ra, int bx, int by, uint16_t* sw) {
  using Ly = RowdotLds<CONTIG, RT>;
  const uint16_t* __restrict__ in = ra.in;
  const uint16_t* __restrict__ wt = ra.wt;
  const int M = ra.M, Kd = ra.Kd, r = ra.r, kchunk = ra.kchunk;
  const float scale = ra.scale;
  uint16_t* __restrict__ out = ra.out;
  float* __restrict__ part = ra.part;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m0 = bx * 64 + 16 * wave;
  const int split = by;
  const int k_lo = split * kchunk, k_hi = min(Kd, k_lo + kchunk);
  const int row = lane & 15, kg = lane >> 4;
  const __amdgpu_buffer_rsrc_t rin = make_rsrc(in, (uint32_t)((uint64_t)M * Kd * 2));
  const uint32_t row_off = (m0 + row < M) ? (uint32_t)(m0 + row) * (uint32_t)Kd * 2u : kOOB;

  f32x4 acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = k_lo; k0 < k_hi; k0 += kRowdotSub) {
    // activations of this sub-chunk: 8 MFMA steps of 32, lane k-group kg
    uint4 av[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int k = k0 + 32 * u + 8 * kg;
      av[u] = buf_load16(rin, k < k_hi ? row_off + 2u * (uint32_t)k : kOOB);
    }
    if (ra.drop.thr) {
#pragma unroll
      for (int u = 0; u < 8; ++u)
        av[u] = drop8(av[u], (uint64_t)(m0 + row) * (uint64_t)Kd + (uint64_t)(k0 + 32 * u + 8 * kg), ra.drop);
    }
    // stage w for k0 .. k0 + 255 (zero past r / k_hi)
    __syncthreads();  // previous sub-chunk's reads of sw are done
    if (CONTIG) {
      for (int idx = tid; idx < RT * 16 * (kRowdotSub / 8); idx += 256) {
        const int j = idx / (kRowdotSub / 8), ch = idx % (kRowdotSub / 8);
        const int k = k0 + 8 * ch;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (j < r && k < k_hi) v = *reinterpret_cast<const uint4*>(wt + (int64_t)j * Kd + k);
        *reinterpret_cast<uint4*>(sw + j * Ly::kPitch + 8 * ch) = v;
      }
    } else if ((r & 7) == 0) {
      // rows of B are r * 2 bytes, 16-byte aligned: copy 8 ranks at a time
      for (int idx = tid; idx < kRowdotSub * RT * 2; idx += 256) {
        const int kk = idx / (RT * 2), c = idx % (RT * 2);
        const int k = k0 + kk;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (8 * c < r && k < k_hi) v = *reinterpret_cast<const uint4*>(wt + (int64_t)k * r + 8 * c);
        *reinterpret_cast<uint4*>(sw + kk * Ly::kPitch + 8 * c) = v;
      }
    } else {
      for (int idx = tid; idx < kRowdotSub * RT * 16; idx += 256) {
        const int kk = idx / (RT * 16), j = idx % (RT * 16);
        const int k = k0 + kk;
        sw[kk * Ly::kPitch + j] = (j < r && k < k_hi) ? wt[(int64_t)k * r + j] : (uint16_t)0;
      }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const typename E::v8 a = E::vec(av[u]);
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        typename E::v8 b;
        if (CONTIG) {
          const uint4 v = *reinterpret_cast<const uint4*>(sw + (16 * t + row) * Ly::kPitch + 32 * u + 8 * kg);
          b = E::vec(v);
        } else {
          // lane p + 4q of k-group kg addresses row kb + q, columns 4p..4p+3
          // and receives column (lane & 15), rows kb .. kb + 3
          const int p = row & 3, q = row >> 2;
          const int kb = 32 * u + 8 * kg + q;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)(sw + kb * Ly::kPitch + 16 * t + 4 * p));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)(sw + (kb + 4) * Ly::kPitch + 16 * t + 4 * p));
          const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          b = E::vec(__builtin_bit_cast(uint4, v));
        }
        acc[t] = E::mfma16(a, b, acc[t]);
      }
    }
  }
  // D[m][j]: m = m0 + 4 * (lane >> 4) + v, j = 16 t + (lane & 15)
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int j = 16 * t + (lane & 15);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = m0 + 4 * (lane >> 4) + v;
      if (m < M && j < r) {
        if (part) {
          part[((int64_t)split * M + m) * r + j] = acc[t][v];
        } else {
          const uint32_t pk = E::pack2(scale * acc[t][v], 0.f);
          out[(int64_t)m * r + j] = (uint16_t)(pk & 0xFFFFu);
        }
      }
    }
  }
}

template <bool CONTIG, int RT, typename E>
__global__ __launch_bounds__(256) void k_rowdot(RowdotArgs ra) {
  __shared__ __attribute__((aligned(16))) uint16_t sw[RowdotLds<CONTIG, RT>::kElems];
  rowdot_body<CONTIG, RT, E>(ra, blockIdx.x, blockIdx.y, sw);
}

// out[m][j] = bf16(scale * sum_{split} part[split][m][j]), fixed order.
template <typename E>
__device__ __forceinline__ void rowdot_finalize_body(const float* __restrict__ part, int nsplit, int64_t n,
                                                     float scale, uint16_t* __restrict__ out, int b, int nb) {
  for (int64_t i = (int64_t)b * 256 + threadIdx.x; i < n; i += (int64_t)nb * 256) {
    float s = 0.f;
    int k = 0;
    for (; k + 8 <= nsplit; k += 8) {  // 8 loads in flight, added in split order
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = part[(int64_t)(k + j) * n + i];
#pragma unroll
      for (int j = 0; j < 8; ++j) s += v[j];
    }
    for (; k < nsplit; ++k) s += part[(int64_t)k * n + i];
    const uint32_t pk = E::pack2(scale * s, 0.f);
    out[i] = (uint16_t)(pk & 0xFFFFu);
  }
}

template <typename E>
__global__ __launch_bounds__(256) void k_rowdot_finalize(const float* __restrict__ part, int nsplit, int64_t n,
                                                         float scale, uint16_t* __restrict__ out) {
  rowdot_finalize_body<E>(part, nsplit, n, scale, out, blockIdx.x, gridDim.x);
}

// The same sum for few outputs and many splits: 8 lanes per output, lane t
// adding splits t, t + 8, t + 16, ... in order, then the 8 sums combined in a
// fixed butterfly; lane t == 0 stores.  A handful of memory latencies
// instead of nsplit / 8 of them.
template <typename E>
__global__ __launch_bounds__(256) void k_rowdot_finalize8(const float* __restrict__ part, int nsplit, int64_t n,
                                                          float scale, uint16_t* __restrict__ out) {
  const int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t i = gi >> 3;
  const int t = (int)(gi & 7);
  const bool ok = i < n;
  float s = 0.f;
  int k = t;
  for (; k + 56 < nsplit; k += 64) {  // 8 loads in flight
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = ok ? part[(int64_t)(k + 8 * j) * n + i] : 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += v[j];
  }
  for (; k < nsplit; k += 8) s += ok ? part[(int64_t)k * n + i] : 0.f;
  s += __shfl_xor(s, 1);
  s += __shfl_xor(s, 2);
  s += __shfl_xor(s, 4);
  if (ok && t == 0) {
    const uint32_t pk = E::pack2(scale * s, 0.f);
    out[i] = (uint16_t)(pk & 0xFFFFu);
  }
}

// ---------------------------------------------------------------- coldot ----
// Workgroup: 128 columns x one chunk of rows; the 4 waves take interleaved
// 32-row steps and are summed in LDS in a fixed order.  Each lane loads an
// 8 x 8 patch (8 rows x 16 bytes) and transposes it in registers, so column
// c0 + 8q + jj becomes the B operand of MFMA number jj.
struct ColdotArgs {
  const uint16_t* v;   // [M x r] bf16 (U~ or V~)
  int r;
  const uint16_t* in;  // [M x C] bf16 (dY or X)
  int M, C, mchunk;
  float* part;         // [nmc][r][C] fp32
  DropMask drop;       // dropout of `in` (thr 0: none)
};

// Workgroup (bx, by) = (128-column tile, row chunk) of the coldot grid.
template <int RT, typename E>
__device__ __forceinline__ void coldot_body(const ColdotArgs& ca, int bx, int by, f32x4 (*red)[8][64]) {
  const uint16_t* __restrict__ v = ca.v;
  const uint16_t* __restrict__ in = ca.in;
  const int r = ca.r, M = ca.M, C = ca.C, mchunk = ca.mchunk;
  float* __restrict__ part = ca.part;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c0 = bx * 128, mc = by;
  const int mbeg = mc * mchunk, mend = min(M, mbeg + mchunk);
  const int g = lane >> 4, q = lane & 15;
  const bool col_ok = c0 + 8 * q < C;
  f32x4 acc[RT][8];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) acc[t][jj] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int m0 = mbeg + wave * 32; m0 < mend; m0 += 128) {
    uint4 rows[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int m = m0 + 8 * g + i;
      rows[i] = (m < mend && col_ok) ? *reinterpret_cast<const uint4*>(in + (int64_t)m * C + c0 + 8 * q)
                                     : make_uint4(0, 0, 0, 0);
    }
    if (ca.drop.thr) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        rows[i] = drop8(rows[i], (uint64_t)(m0 + 8 * g + i) * (uint64_t)C + (uint64_t)(c0 + 8 * q), ca.drop);
    }
    uint4 colv[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const uint32_t sel = (jj & 1) ? 0x07060302u : 0x05040100u;
      uint32_t d[4];
#pragma unroll
      for (int mm = 0; mm < 4; ++mm) {
        const uint32_t* r0 = reinterpret_cast<const uint32_t*>(&rows[2 * mm]);
        const uint32_t* r1 = reinterpret_cast<const uint32_t*>(&rows[2 * mm + 1]);
        d[mm] = __builtin_amdgcn_perm(r1[jj >> 1], r0[jj >> 1], sel);
      }
      colv[jj] = make_uint4(d[0], d[1], d[2], d[3]);
    }
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const int j = 16 * t + q;
      uint16_t e[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int m = m0 + 8 * g + i;
        e[i] = (j < r && m < mend) ? v[(int64_t)m * r + j] : (uint16_t)0;
      }
      uint4 av = make_uint4(e[0] | ((uint32_t)e[1] << 16), e[2] | ((uint32_t)e[3] << 16),
                            e[4] | ((uint32_t)e[5] << 16), e[6] | ((uint32_t)e[7] << 16));
#pragma unroll
      for (int jj = 0; jj < 8; ++jj)
        acc[t][jj] = E::mfma16(E::vec(av), E::vec(colv[jj]), acc[t][jj]);
    }
  }
  // D[j][col]: j = 16t + 4*(lane>>4) + v, column index lane&15 -> c0 + 8*(lane&15) + jj
#pragma unroll
  for (int t = 0; t < RT; ++t) {
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) red[wave][jj][lane] = acc[t][jj];
    __syncthreads();
    for (int idx = threadIdx.x; idx < 8 * 64; idx += 256) {
      const int jj = idx >> 6, ln = idx & 63;
      f32x4 s = red[0][jj][ln];
#pragma unroll
      for (int w = 1; w < 4; ++w) s += red[w][jj][ln];
      const int c = c0 + 8 * (ln & 15) + jj;
#pragma unroll
      for (int vv = 0; vv < 4; ++vv) {
        const int j = 16 * t + 4 * (ln >> 4) + vv;
        if (j < r && c < C) part[((int64_t)mc * r + j) * C + c] = s[vv];
      }
    }
    __syncthreads();
  }
}

template <int RT, typename E>
__global__ __launch_bounds__(256) void k_coldot(ColdotArgs ca) {
  __shared__ f32x4 red[4][8][64];
  coldot_body<RT, E>(ca, blockIdx.x, blockIdx.y, red);
}

// out[j][c] (or out[c][j] when TRANS) = sum_{mc} part[mc][j][c], fixed order.
template <bool TRANS>
__device__ __forceinline__ void finalize_body(const float* __restrict__ part, int nmc, int r, int C,
                                              float* __restrict__ out, int b, int nb) {
  const int64_t total = (int64_t)r * C;
  for (int64_t idx = (int64_t)b * 256 + threadIdx.x; idx < total; idx += (int64_t)nb * 256) {
    const int j = (int)(idx / C), c = (int)(idx % C);
    float s = 0.f;
    int mc = 0;
    for (; mc + 8 <= nmc; mc += 8) {  // 8 loads in flight, added in chunk order
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = part[((int64_t)(mc + u) * r + j) * C + c];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; mc < nmc; ++mc) s += part[((int64_t)mc * r + j) * C + c];
    if (TRANS) out[(int64_t)c * r + j] = s; else out[idx] = s;
  }
}

template <bool TRANS>
__global__ __launch_bounds__(256) void k_finalize(const float* __restrict__ part, int nmc, int r, int C,
                                                  float* __restrict__ out) {
  finalize_body<TRANS>(part, nmc, r, C, out, blockIdx.x, gridDim.x);
}

// ---- merged launches of the backward (independent work, one dispatch) ----
// Blocks [0, nr) run the V~ rowdot grid (nr = row blocks x splits), blocks
// [nr, nr + nc) the dB coldot grid: both read dY, neither needs the other.
template <int RT, typename E>
__global__ __launch_bounds__(256) void k_vt_and_db(RowdotArgs ra, int rb, ColdotArgs ca, int ctiles) {
  __shared__ __attribute__((aligned(16))) uint16_t sw[RowdotLds<false, RT>::kElems];
  __shared__ f32x4 red[4][8][64];
  const int nr = rb * ra.nsplit;
  const int b = blockIdx.x;
  if (b < nr) rowdot_body<false, RT, E>(ra, b % rb, b / rb, sw);
  else coldot_body<RT, E>(ca, (b - nr) % ctiles, (b - nr) / ctiles, red);
}

// Blocks [0, n1) finalize V~ (when it was split), blocks [n1, n1 + n2)
// finalize dB (stored [N x r]).
template <typename E>
__global__ __launch_bounds__(256) void k_fin_vt_and_db(const float* __restrict__ vpart, int nsplit, int64_t nv,
                                                       float scale, uint16_t* __restrict__ vout, int n1,
                                                       const float* __restrict__ cpart, int nmc, int r, int C,
                                                       float* __restrict__ dB, int n2) {
  const int b = blockIdx.x;
  if (b < n1) rowdot_finalize_body<E>(vpart, nsplit, nv, scale, vout, b, n1);
  else finalize_body<true>(cpart, nmc, r, C, dB, b - n1, n2);
}

__global__ __launch_bounds__(256) void k_fill_zero(float* __restrict__ p, int64_t n) {
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0.f;
}

__global__ __launch_bounds__(256) void k_zero_u16(uint16_t* __restrict__ p, int64_t n) {
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0;
}

template <bool CONTIG, int RT, typename E>
void rowdot_launch(dim3 grid, hipStream_t st, const uint16_t* in, int M, int Kd, const uint16_t* wt, int r,
                   int kchunk, float scale, uint16_t* out, float* part, DropMask drop) {
  const RowdotArgs ra{in, M, Kd, wt, r, kchunk, (int)grid.y, scale, out, part, drop};
  hipLaunchKernelGGL((k_rowdot<CONTIG, RT, E>), grid, dim3(256), 0, st, ra);
}

template <bool CONTIG, typename E>
hipError_t rowdot_dispatch(const uint16_t* in, int M, int Kd, const uint16_t* wt, int r, float scale,
                           uint16_t* out, float* part, DropMask drop, hipStream_t st) {
  int nsplit, kchunk;
  rowdot_split(M, Kd, &nsplit, &kchunk);
  dim3 grid((M + 63) / 64, nsplit);
  float* p = nsplit > 1 ? part : nullptr;
  switch ((r + 15) / 16) {
    case 1: rowdot_launch<CONTIG, 1, E>(grid, st, in, M, Kd, wt, r, kchunk, scale, out, p, drop); break;
    case 2: rowdot_launch<CONTIG, 2, E>(grid, st, in, M, Kd, wt, r, kchunk, scale, out, p, drop); break;
    case 3: rowdot_launch<CONTIG, 3, E>(grid, st, in, M, Kd, wt, r, kchunk, scale, out, p, drop); break;
    default: rowdot_launch<CONTIG, 4, E>(grid, st, in, M, Kd, wt, r, kchunk, scale, out, p, drop); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsplit == 1) return e;
  const int64_t n = (int64_t)M * r;
  if (n <= 4096 && nsplit >= 16) {
    hipLaunchKernelGGL(k_rowdot_finalize8<E>, dim3((int)((8 * n + 255) / 256)), dim3(256), 0, st, part, nsplit, n,
                       scale, out);
    return hipGetLastError();
  }
  const int blocks = (int)std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 2048));
  hipLaunchKernelGGL(k_rowdot_finalize<E>, dim3(blocks), dim3(256), 0, st, part, nsplit, n, scale, out);
  return hipGetLastError();
}

}  // namespace

// U~ = E(s (mask * X) A^T): in = X [M x K], A [r x K]; E = fp16 when f16, else bf16
hipError_t launch_lora_down(const uint16_t* X, int M, int K, const uint16_t* A, int r, float s, uint16_t* U,
                            float* part, DropMask drop, bool f16, hipStream_t st) {
  return f16 ? rowdot_dispatch<true, F16>(X, M, K, A, r, s, U, part, drop, st)
             : rowdot_dispatch<true, Bf16>(X, M, K, A, r, s, U, part, drop, st);
}

int coldot_chunk_rows() { return 256; }

namespace {

template <typename E>
void coldot_launch(dim3 grid, const ColdotArgs& ca, int rt, hipStream_t st) {
  switch (rt) {
    case 1: hipLaunchKernelGGL((k_coldot<1, E>), grid, dim3(256), 0, st, ca); break;
    case 2: hipLaunchKernelGGL((k_coldot<2, E>), grid, dim3(256), 0, st, ca); break;
    case 3: hipLaunchKernelGGL((k_coldot<3, E>), grid, dim3(256), 0, st, ca); break;
    default: hipLaunchKernelGGL((k_coldot<4, E>), grid, dim3(256), 0, st, ca); break;
  }
}

template <typename E>
void vt_and_db_launch(dim3 grid, const RowdotArgs& ra, int rb, const ColdotArgs& ca, int ctiles, int rt,
                      hipStream_t st) {
  switch (rt) {
    case 1: hipLaunchKernelGGL((k_vt_and_db<1, E>), grid, dim3(256), 0, st, ra, rb, ca, ctiles); break;
    case 2: hipLaunchKernelGGL((k_vt_and_db<2, E>), grid, dim3(256), 0, st, ra, rb, ca, ctiles); break;
    case 3: hipLaunchKernelGGL((k_vt_and_db<3, E>), grid, dim3(256), 0, st, ra, rb, ca, ctiles); break;
    default: hipLaunchKernelGGL((k_vt_and_db<4, E>), grid, dim3(256), 0, st, ra, rb, ca, ctiles); break;
  }
}

}  // namespace

// part[mc][j][c] = sum over the mc-th chunk of rows of v[m][j] * (mask * in)[m][c]
hipError_t launch_coldot(const uint16_t* v, int r, const uint16_t* in, int M, int C, float* part, DropMask drop,
                         bool f16, hipStream_t st) {
  const int mchunk = coldot_chunk_rows();
  dim3 grid((C + 127) / 128, (M + mchunk - 1) / mchunk);
  const ColdotArgs ca{v, r, in, M, C, mchunk, part, drop};
  if (f16) coldot_launch<F16>(grid, ca, (r + 15) / 16, st);
  else coldot_launch<Bf16>(grid, ca, (r + 15) / 16, st);
  return hipGetLastError();
}

// Backward adapter reductions over dY in two dispatches:
//   1. V~ split partials (or V~ itself when unsplit) and dB row-chunk partials;
//   2. V~ finalize (when split) and dB finalize.
hipError_t launch_vt_and_db(const uint16_t* dY, int M, int N, const uint16_t* B, const uint16_t* U, int r,
                            float s, uint16_t* V, float* vpart, float* cpart, float* dB, bool f16, hipStream_t st) {
  int nsplit, kchunk;
  rowdot_split(M, N, &nsplit, &kchunk);
  const int rb = (M + 63) / 64;
  const RowdotArgs ra{dY, M, N, B, r, kchunk, nsplit, s, V, nsplit > 1 ? vpart : nullptr, DropMask{}};
  const int mchunk = coldot_chunk_rows();
  const int ctiles = (N + 127) / 128, nmc = (M + mchunk - 1) / mchunk;
  const ColdotArgs ca{U, r, dY, M, N, mchunk, cpart, DropMask{}};
  const dim3 grid(rb * nsplit + ctiles * nmc);
  if (f16) vt_and_db_launch<F16>(grid, ra, rb, ca, ctiles, (r + 15) / 16, st);
  else vt_and_db_launch<Bf16>(grid, ra, rb, ca, ctiles, (r + 15) / 16, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nv = (int64_t)M * r;
  const int n1 = nsplit > 1 ? (int)std::max<int64_t>(1, std::min<int64_t>((nv + 255) / 256, 2048)) : 0;
  const int64_t nc = (int64_t)r * N;
  const int n2 = (int)std::max<int64_t>(1, std::min<int64_t>((nc + 255) / 256, 4096));
  if (f16)
    hipLaunchKernelGGL(k_fin_vt_and_db<F16>, dim3(n1 + n2), dim3(256), 0, st, vpart, nsplit, nv, s, V, n1, cpart,
                       nmc, r, N, dB, n2);
  else
    hipLaunchKernelGGL(k_fin_vt_and_db<Bf16>, dim3(n1 + n2), dim3(256), 0, st, vpart, nsplit, nv, s, V, n1, cpart,
                       nmc, r, N, dB, n2);
  return hipGetLastError();
}

hipError_t launch_finalize(const float* part, int nmc, int r, int C, float* out, bool trans, hipStream_t st) {
  const int64_t total = (int64_t)r * C;
  int blocks = (int)std::min<int64_t>((total + 255) / 256, 4096);
  if (blocks < 1) blocks = 1;
  if (trans) hipLaunchKernelGGL((k_finalize<true>), dim3(blocks), dim3(256), 0, st, part, nmc, r, C, out);
  else hipLaunchKernelGGL((k_finalize<false>), dim3(blocks), dim3(256), 0, st, part, nmc, r, C, out);
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  int blocks = (int)std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(k_fill_zero, dim3(blocks), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

hipError_t launch_zero_u16(uint16_t* p, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  int blocks = (int)std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(k_zero_u16, dim3(blocks), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

}  // namespace qlora
