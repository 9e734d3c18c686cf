// Skinny rank-r products of the adapter path ([P1] "The mechanism in brief":
// the adapter adds (alpha / r) B A x; backward gives gradients for A and B).
//
//   rowdot:   out[m][j] = bf16(scale * sum_k in[m][k] * w(j, k))       (M x r)
//             U~ = bf16(s X A^T)   and   V~ = bf16(s dY B)
//   coldot:   part[mc][j][c] = sum_{m in chunk mc} v[m][j] * in[m][c]  (fp32)
//   finalize: out = sum over chunks, in a fixed order (deterministic)
//             dA = V~^T X  [r x K]      dB = dY^T U~  -> stored [N x r]
//
// All use v_mfma_f32_16x16x32_bf16 with the rank on the 16-wide side.
#include <algorithm>

#include "common.h"

namespace qlora {
namespace {

typedef __attribute__((ext_vector_type(8))) short i16x8;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// ---------------------------------------------------------------- rowdot ----
// One 256-thread workgroup per 16 rows; the 4 waves split the reduction in
// 32-wide chunks and are summed in LDS in a fixed order.
// w(j, k) = wt[j * ldw + k] if CONTIG (A is [r x K]), else wt[k * ldw + j]
// (B is [N x r], read down its columns).
template <bool CONTIG, int RT>
__global__ __launch_bounds__(256) void k_rowdot(const uint16_t* __restrict__ in, int M, int Kd,
                                                const uint16_t* __restrict__ wt, int ldw, int r,
                                                float scale, uint16_t* __restrict__ out) {
  __shared__ f32x4 red[4][RT][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m0 = blockIdx.x * 16;
  const int row = lane & 15, kg = lane >> 4;
  f32x4 acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nchunks = (Kd + 31) / 32;
  const bool row_ok = m0 + row < M;
  for (int ch = wave; ch < nchunks; ch += 4) {
    const int k = ch * 32 + kg * 8;
    uint4 av = make_uint4(0, 0, 0, 0);
    if (row_ok && k < Kd) av = *reinterpret_cast<const uint4*>(in + (int64_t)(m0 + row) * Kd + k);
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const int j = 16 * t + row;
      uint4 bv = make_uint4(0, 0, 0, 0);
      if (j < r && k < Kd) {
        if (CONTIG) {
          bv = *reinterpret_cast<const uint4*>(wt + (int64_t)j * ldw + k);
        } else {
          uint16_t e[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) e[i] = wt[(int64_t)(k + i) * ldw + j];
          bv.x = e[0] | ((uint32_t)e[1] << 16);
          bv.y = e[2] | ((uint32_t)e[3] << 16);
          bv.z = e[4] | ((uint32_t)e[5] << 16);
          bv.w = e[6] | ((uint32_t)e[7] << 16);
        }
      }
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), as_bf16x8(bv), acc[t], 0, 0, 0);
    }
  }
#pragma unroll
  for (int t = 0; t < RT; ++t) red[wave][t][lane] = acc[t];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      f32x4 s = red[0][t][lane];
#pragma unroll
      for (int w = 1; w < 4; ++w) s += red[w][t][lane];
      const int j = 16 * t + (lane & 15);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + 4 * (lane >> 4) + v;
        if (m < M && j < r) {
          uint32_t pk = pack_bf16x2(scale * s[v], 0.f);
          out[(int64_t)m * r + j] = (uint16_t)(pk & 0xFFFFu);
        }
      }
    }
  }
}

// ---------------------------------------------------------------- coldot ----
// Workgroup: 128 columns x one chunk of rows; the 4 waves take interleaved
// 32-row steps and are summed in LDS in a fixed order.  Each lane loads an
// 8 x 8 patch (8 rows x 16 bytes) and transposes it in registers, so column
// c0 + 8q + jj becomes the B operand of MFMA number jj.
template <int RT>
__global__ __launch_bounds__(256) void k_coldot(const uint16_t* __restrict__ v, int r,
                                                const uint16_t* __restrict__ in, int M, int C,
                                                int mchunk, float* __restrict__ part) {
  __shared__ f32x4 red[4][8][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c0 = blockIdx.x * 128, mc = blockIdx.y;
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
    bf16x8 colv[8];
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
      colv[jj] = as_bf16x8(make_uint4(d[0], d[1], d[2], d[3]));
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
        acc[t][jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), colv[jj], acc[t][jj], 0, 0, 0);
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

// out[j][c] (or out[c][j] when TRANS) = sum_{mc} part[mc][j][c], fixed order.
template <bool TRANS>
__global__ __launch_bounds__(256) void k_finalize(const float* __restrict__ part, int nmc, int r, int C,
                                                  float* __restrict__ out) {
  const int64_t total = (int64_t)r * C;
  for (int64_t idx = blockIdx.x * 256 + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * 256) {
    const int j = (int)(idx / C), c = (int)(idx % C);
    float s = 0.f;
    for (int mc = 0; mc < nmc; ++mc) s += part[((int64_t)mc * r + j) * C + c];
    if (TRANS) out[(int64_t)c * r + j] = s; else out[idx] = s;
  }
}

__global__ __launch_bounds__(256) void k_fill_zero(float* __restrict__ p, int64_t n) {
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0.f;
}

__global__ __launch_bounds__(256) void k_zero_u16(uint16_t* __restrict__ p, int64_t n) {
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0;
}

template <bool CONTIG>
hipError_t rowdot_dispatch(const uint16_t* in, int M, int Kd, const uint16_t* wt, int ldw, int r, float scale,
                           uint16_t* out, hipStream_t st) {
  dim3 grid((M + 15) / 16);
  const int rt = (r + 15) / 16;
  switch (rt) {
    case 1: hipLaunchKernelGGL((k_rowdot<CONTIG, 1>), grid, dim3(256), 0, st, in, M, Kd, wt, ldw, r, scale, out); break;
    case 2: hipLaunchKernelGGL((k_rowdot<CONTIG, 2>), grid, dim3(256), 0, st, in, M, Kd, wt, ldw, r, scale, out); break;
    case 3: hipLaunchKernelGGL((k_rowdot<CONTIG, 3>), grid, dim3(256), 0, st, in, M, Kd, wt, ldw, r, scale, out); break;
    default: hipLaunchKernelGGL((k_rowdot<CONTIG, 4>), grid, dim3(256), 0, st, in, M, Kd, wt, ldw, r, scale, out); break;
  }
  return hipGetLastError();
}

}  // namespace

// U~ = bf16(s X A^T): in = X [M x K], A [r x K]
hipError_t launch_lora_down(const uint16_t* X, int M, int K, const uint16_t* A, int r, float s, uint16_t* U,
                            hipStream_t st) {
  return rowdot_dispatch<true>(X, M, K, A, K, r, s, U, st);
}

// V~ = bf16(s dY B): in = dY [M x N], B [N x r]
hipError_t launch_lora_vt(const uint16_t* dY, int M, int N, const uint16_t* B, int r, float s, uint16_t* V,
                          hipStream_t st) {
  return rowdot_dispatch<false>(dY, M, N, B, r, r, s, V, st);
}

int coldot_chunk_rows() { return 256; }

// part[mc][j][c] = sum over the mc-th chunk of rows of v[m][j] * in[m][c]
hipError_t launch_coldot(const uint16_t* v, int r, const uint16_t* in, int M, int C, float* part, hipStream_t st) {
  const int mchunk = coldot_chunk_rows();
  dim3 grid((C + 127) / 128, (M + mchunk - 1) / mchunk);
  const int rt = (r + 15) / 16;
  switch (rt) {
    case 1: hipLaunchKernelGGL((k_coldot<1>), grid, dim3(256), 0, st, v, r, in, M, C, mchunk, part); break;
    case 2: hipLaunchKernelGGL((k_coldot<2>), grid, dim3(256), 0, st, v, r, in, M, C, mchunk, part); break;
    case 3: hipLaunchKernelGGL((k_coldot<3>), grid, dim3(256), 0, st, v, r, in, M, C, mchunk, part); break;
    default: hipLaunchKernelGGL((k_coldot<4>), grid, dim3(256), 0, st, v, r, in, M, C, mchunk, part); break;
  }
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
