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
// Workgroup: 64 rows x 128 columns, 4 waves of 16 rows.  The rank-r product
// runs on v_mfma_f32_16x16x32_bf16 with r zero-padded to RP (32 or 64): the
// A operand is B[n][j] (16 bytes of a row per lane), the B operand is
// A[j][k], read column-wise from an LDS copy of A[:, k0 : k0 + 128] with the
// transposing ds_read_b64_tr_b16.  The 64 x 128 fp32 product goes through LDS
// to a row-major pass in which each thread decodes 8 weights, adds s * t and
// writes 16 bytes of the merged bf16 weight.
#include <algorithm>

#include "common.h"

namespace qlora {
namespace {

typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(8))) short i16x8;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kMTileN = 64, kMTileK = 128;
constexpr int kAPitch = kMTileK + 8;   // bf16 per row of the A copy
constexpr int kTPitch = kMTileK + 4;   // fp32 per row of the product tile

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

template <int RP>
__global__ __launch_bounds__(256) void k_merge(const uint32_t* __restrict__ codes, const uint8_t* __restrict__ q8,
                                               const float* __restrict__ s2, int N, int K,
                                               const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                                               int r, float s, uint16_t* __restrict__ out, Nf4Consts c) {
  __shared__ __attribute__((aligned(16))) uint16_t sa[RP * kAPitch];
  __shared__ __attribute__((aligned(16))) float st[kMTileN * kTPitch];
  __shared__ float lv[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k0 = blockIdx.x * kMTileK, n0 = blockIdx.y * kMTileN;
  const bool vec = (r & 7) == 0;
  if (tid < 16) lv[tid] = c.level[tid];

  // A[:, k0 : k0 + 128] -> LDS (rows j >= r and columns >= K are zero)
  for (int idx = tid; idx < RP * (kMTileK / 8); idx += 256) {
    const int j = idx / (kMTileK / 8), cc = idx % (kMTileK / 8), k = k0 + 8 * cc;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (j < r && k < K) v = *reinterpret_cast<const uint4*>(A + (int64_t)j * K + k);
    *reinterpret_cast<uint4*>(sa + j * kAPitch + 8 * cc) = v;
  }
  __syncthreads();

  // t[n][k] = sum_j B[n][j] A[j][k] for this wave's 16 rows x 128 columns
  const int row = lane & 15, g = lane >> 4;
  const int n = n0 + 16 * wave + row;
  f32x4 acc[kMTileK / 16];
#pragma unroll
  for (int ct = 0; ct < kMTileK / 16; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s32 = 0; s32 < RP / 32; ++s32) {
    const int j = 32 * s32 + 8 * g;
    const bf16x8 af = __builtin_bit_cast(bf16x8, load8(B + (int64_t)n * r + j, r - j, n < N, vec));
    const int p = row & 3, q = row >> 2;
    const int jb = 32 * s32 + 8 * g + q;
#pragma unroll
    for (int ct = 0; ct < kMTileK / 16; ++ct) {
      // lane p + 4q of each 16-lane group addresses row jb, columns 16 ct + 4p;
      // it receives column 16 ct + (lane & 15), rows jb - q .. + 3 (and + 4 .. + 7)
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(sa + jb * kAPitch + 16 * ct + 4 * p));
      const i16x4 hi =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(sa + (jb + 4) * kAPitch + 16 * ct + 4 * p));
      const i16x8 bv = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, __builtin_bit_cast(bf16x8, bv), acc[ct], 0, 0, 0);
    }
  }
  // D layout: lane l, element v -> row 4 (l >> 4) + v of the wave, column l & 15 of the tile
#pragma unroll
  for (int ct = 0; ct < kMTileK / 16; ++ct)
#pragma unroll
    for (int v = 0; v < 4; ++v) st[(16 * wave + 4 * g + v) * kTPitch + 16 * ct + row] = acc[ct][v];
  __syncthreads();

  // row-major pass: thread -> (row, 8 columns); Wm = bf16(Wbf + s * t)
  for (int idx = tid; idx < kMTileN * (kMTileK / 8); idx += 256) {
    const int rl = idx / (kMTileK / 8), cc = idx % (kMTileK / 8);
    const int nn = n0 + rl, k = k0 + 8 * cc;
    if (nn >= N || k >= K) continue;
    const uint32_t e = (uint32_t)nn * (uint32_t)K + (uint32_t)k;  // weight index
    const uint4 wb = decode8(codes[e >> 3], block_scale(q8, s2, e >> 6), lv);
    const float* tp = st + rl * kTPitch + 8 * cc;
    const uint32_t wv[4] = {wb.x, wb.y, wb.z, wb.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float w0 = bf16_to_f32((uint16_t)(wv[i] & 0xFFFFu)), w1 = bf16_to_f32((uint16_t)(wv[i] >> 16));
      o[i] = pack_bf16x2(w0 + s * tp[2 * i], w1 + s * tp[2 * i + 1]);
    }
    *reinterpret_cast<uint4*>(out + e) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

}  // namespace

hipError_t launch_merge(const uint8_t* codes, const uint8_t* q8, const float* s2, int N, int K, const uint16_t* A,
                        const uint16_t* B, int r, float s, uint16_t* out, hipStream_t st) {
  const dim3 grid((K + kMTileK - 1) / kMTileK, (N + kMTileN - 1) / kMTileN);
  const uint32_t* cw = reinterpret_cast<const uint32_t*>(codes);
  if (r <= 32)
    hipLaunchKernelGGL(k_merge<32>, grid, dim3(256), 0, st, cw, q8, s2, N, K, A, B, r, s, out, nf4_consts());
  else
    hipLaunchKernelGGL(k_merge<64>, grid, dim3(256), 0, st, cw, q8, s2, N, K, A, B, r, s, out, nf4_consts());
  return hipGetLastError();
}

}  // namespace qlora
