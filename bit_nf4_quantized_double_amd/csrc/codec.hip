// NF4 + double-quantization codec kernels ([P1] "The mechanism in brief";
// [P4] "NF4 and double quantisation").
//
// Quantize: one 256-thread workgroup per group of 256 blocks, one thread per
// 64-weight block: absmax, x = w / absmax (IEEE fp32 division), code = number
// of decision thresholds below x (the nearest level, exact ties to the lower
// level; found with a table-guided search on a reciprocal product, the IEEE
// quotient formed only for blocks with a weight next to a threshold), two
// codes per byte.  The block absmaxes stay in registers; the group max gives
// the fp32 step s2 = max / 255 and each block's 8-bit code
// q8 = round-half-even(absmax / s2).  No workspace.  The input is fp32 or
// bf16 (widened exactly; used to re-quantize a merged bf16 weight).
//
// Dequant: a streaming decode, 8 weights (one code dword -> 16 bytes of bf16)
// per thread per iteration; HBM-bound (2.516 bytes moved per weight).
//
// Both kernels also serve the storage-format variants the pages compare NF4
// with double quantization against ([P1] "The mechanism in brief": one fp32
// absmax per block costs 4.5 bits per weight; [P2] "Follow-up questions to
// expect": evenly spaced int4 levels): the level table and its code search
// are arguments, and without double quantization the fp32 block absmax is
// stored and read directly.
#include <algorithm>

#include "common.h"

namespace qlora {
namespace {

// Element of the input as fp32: fp32 as is, bf16 widened exactly.
__device__ __forceinline__ void widen4(const uint4& v, const float*, float* w) {
  w[0] = __uint_as_float(v.x); w[1] = __uint_as_float(v.y);
  w[2] = __uint_as_float(v.z); w[3] = __uint_as_float(v.w);
}
__device__ __forceinline__ void widen4(const uint4& v, const uint16_t*, float* w) {
  const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    w[2 * j] = __uint_as_float(d[j] << 16);
    w[2 * j + 1] = __uint_as_float(d[j] & 0xFFFF0000u);
  }
}

// One 256-thread workgroup per group of 256 blocks, one thread per block:
// the group is staged through LDS, the thread takes its 64 weights and the absmax,
// codes each weight with the table-guided search and writes 32 bytes of
// packed codes; the group max then gives s2 and every thread's q8.
// DQ: block absmaxes double-quantized into q8 codes and one s2 per group;
// otherwise each block's fp32 absmax is written to `absmax` (q8, s2 unused).
template <typename T, bool DQ>
__global__ __launch_bounds__(256) void k_quantize(const T* __restrict__ W, uint32_t nb,
                                                  uint8_t* __restrict__ codes, uint8_t* __restrict__ q8,
                                                  float* __restrict__ s2, float* __restrict__ absmax,
                                                  QuantSearch qs) {
  constexpr int kWords = kBlock * (int)sizeof(T) / 4;  // 32-bit words per block
  constexpr int kChunks = kWords / 4;                  // 16-byte chunks per block
  constexpr int kPitch = kWords + 4;                   // 4 words mod 32 banks between blocks
  __shared__ __attribute__((aligned(16))) uint32_t s_w[kGroup * kPitch];
  // per table cell: the candidate threshold t and the candidate count c0
  // (t = 2 past the last threshold: never exceeded, never close)
  __shared__ uint2 s_ct[256];
  __shared__ float s_red[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  {
    const uint32_t c0 = qs.cand[tid];
    s_ct[tid] = make_uint2(__float_as_uint(c0 < 15 ? qs.thr16[c0] : 2.0f), c0);
  }
  const uint32_t g = blockIdx.x, b0 = g * kGroup;
  const uint32_t nblk = min((uint32_t)kGroup, nb - b0);
  const bool valid = (uint32_t)tid < nblk;
  const uint32_t b = b0 + tid;

  // the group's weights -> LDS with coalesced loads (each wave instruction
  // reads 1 KB contiguous), then every thread takes its own block
  {
    const uint4* src = reinterpret_cast<const uint4*>(W) + (size_t)b0 * kChunks;
    uint4 v[kChunks];
#pragma unroll
    for (int j = 0; j < kChunks; ++j) {
      const int c = tid + 256 * j;
      v[j] = (uint32_t)(c / kChunks) < nblk && in_bounds((int64_t)b0 * kChunks + c, 1, (int64_t)nb * kChunks)
                 ? src[c]
                 : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < kChunks; ++j) {
      const int c = tid + 256 * j;
      *reinterpret_cast<uint4*>(s_w + (c / kChunks) * kPitch + 4 * (c % kChunks)) = v[j];
    }
  }
  __syncthreads();  // staged weights and search tables ready
  float w[kBlock];
#pragma unroll
  for (int i = 0; i < kChunks; ++i)
    widen4(*reinterpret_cast<const uint4*>(s_w + tid * kPitch + 4 * i), W, w + (kBlock / kChunks) * i);

  float am = 0.f;
#pragma unroll
  for (int i = 0; i < kBlock; ++i) am = fmaxf(am, fabsf(w[i]));

  if (valid) {
    // x = w / am (IEEE division) decides each code.  The fast pass takes x
    // as w * fp32(1 / am), within 2^-22 relative of the quotient while the
    // quotient is a normal number: that picks the table cell (a neighbouring
    // cell gives the same answer) and decides the comparison with the
    // candidate threshold t unless x lies within max(2^-20 |t|, 2^-100) of t.
    // The absolute floor matters only for a threshold at exactly 0 (the
    // evenly spaced table): there the quotient may underflow to +-0 while
    // the product rounds to the smallest subnormal (w = 3 * 2^-149, am = 6),
    // so any x' within 2^-100 of 0 is decided by the quotient.  A block with
    // any weight that close is coded again with the quotient itself (about
    // one block in 3000 for normal data).  A block whose absmax is so small
    // that 1 / am would overflow is scaled by 2^64 first (exact: every
    // quotient is unchanged).
    float amq = am;
    if (am < 0x1p-100f) {
#pragma unroll
      for (int i = 0; i < kBlock; ++i) w[i] *= 0x1p64f;
      amq = am * 0x1p64f;
    }
    const float rcp = amq > 0.f ? 1.0f / amq : 0.f;
    uint32_t packed[8];
    float nd = 1.f;  // min over the block of |x - t| - max(2^-20 |t|, 2^-100); <= 0: some x is close to its t
#pragma unroll
    for (int h = 0; h < 4; ++h) {  // 16 weights per batch: all 16 table reads in flight
      float x[16];
      uint2 ct[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        x[i] = w[16 * h + i] * rcp;
        const int cell = min(max((int)__builtin_fmaf(x[i], 128.f, 128.f), 0), 255);  // x * 128 is exact
        ct[i] = s_ct[cell];
      }
#pragma unroll
      for (int dd = 0; dd < 2; ++dd) {
        uint32_t word = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int i = 8 * dd + e;
          const float t = __uint_as_float(ct[i].x);
          nd = fminf(nd, fabsf(x[i] - t) - fmaxf(fabsf(t) * 0x1p-20f, 0x1p-100f));
          word |= (ct[i].y + (x[i] > t ? 1u : 0u)) << (4 * e);
        }
        packed[2 * h + dd] = word;
      }
    }
    const bool near = nd <= 0.f;
    if (near) {
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        uint32_t word = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = amq > 0.f ? w[8 * d + e] / amq : 0.f;  // IEEE division
          const int cell = min(max((int)__builtin_fmaf(x, 128.f, 128.f), 0), 255);
          const uint2 ct = s_ct[cell];
          word |= (ct.y + (x > __uint_as_float(ct.x) ? 1u : 0u)) << (4 * e);
        }
        packed[d] = word;
      }
    }
    uint4* out = reinterpret_cast<uint4*>(codes + (size_t)b * (kBlock / 2));
    if (in_bounds(2 * (int64_t)b, 2, 2 * (int64_t)nb)) {
      out[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
      out[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
    }
  }

  if (!DQ) {
    if (valid && in_bounds(b, 1, nb)) absmax[b] = am;
    return;
  }
  // group max -> s2 = max / 255, q8 = round-half-even(absmax / s2)
  float m = am;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if (lane == 0) s_red[wave] = m;
  __syncthreads();
  const float gmax = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  const float step = gmax / 255.0f;
  if (valid) {
    uint32_t q = 0;
    if (step > 0.f) {
      const float t = rintf(am / step);  // round half to even
      q = (uint32_t)fminf(fmaxf(t, 0.f), 255.f);
    }
    if (in_bounds(b, 1, nb)) q8[b] = (uint8_t)q;
  }
  if (tid == 0 && in_bounds(g, 1, ((int64_t)nb + kGroup - 1) / kGroup)) s2[g] = step;
}

template <bool DQ, typename E>
__global__ __launch_bounds__(256) void k_dequant(const uint32_t* __restrict__ codes, const uint8_t* __restrict__ q8,
                                                 const float* __restrict__ s2, const float* __restrict__ absmax,
                                                 uint32_t ndw, uint4* __restrict__ out, Nf4Consts c) {
  __shared__ float lv[16];
  if (threadIdx.x < 16) lv[threadIdx.x] = c.level[threadIdx.x];
  __syncthreads();
  // Grid-stride over code dwords: each wave reads 256 contiguous bytes of
  // codes and writes 1 KB of bf16 per iteration.  The output is written with
  // non-temporal stores (streamed out, not re-read here), which measured
  // ~4 % faster on the 70B shapes than plain stores.
  typedef __attribute__((ext_vector_type(4))) unsigned v4u;
  const uint32_t stride = gridDim.x * blockDim.x;
  const int64_t nblk = ndw / 8, ngrp = (nblk + kGroup - 1) / kGroup;
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < ndw; i += stride) {
    const uint32_t b = i >> 3;
    const bool ok = in_bounds(i, 1, ndw) && in_bounds(b, 1, nblk) && (!DQ || in_bounds(b >> 8, 1, ngrp));
    const float sc = !ok ? 0.f : DQ ? block_scale(q8, s2, b) : absmax[b];
    const uint4 o = decode8<E>(ok ? codes[i] : 0u, sc, lv);
    if (ok) __builtin_nontemporal_store(v4u{o.x, o.y, o.z, o.w}, reinterpret_cast<v4u*>(out + i));
  }
}

}  // namespace

hipError_t launch_quantize_fmt(const float* W, int64_t nweights, bool uniform, bool dq, uint8_t* codes,
                               uint8_t* q8, float* s2, float* absmax, hipStream_t st) {
  const uint32_t nb = (uint32_t)(nweights / kBlock);
  const uint32_t ng = (nb + kGroup - 1) / kGroup;
  if (ng == 0) return hipSuccess;
  const QuantSearch& qs = uniform ? quant_search_int4() : quant_search();
  if (dq) hipLaunchKernelGGL((k_quantize<float, true>), dim3(ng), dim3(256), 0, st, W, nb, codes, q8, s2, absmax, qs);
  else hipLaunchKernelGGL((k_quantize<float, false>), dim3(ng), dim3(256), 0, st, W, nb, codes, q8, s2, absmax, qs);
  return hipGetLastError();
}

hipError_t launch_quantize(const float* W, int64_t nweights, uint8_t* codes, uint8_t* q8, float* s2,
                           hipStream_t st) {
  return launch_quantize_fmt(W, nweights, false, true, codes, q8, s2, nullptr, st);
}

hipError_t launch_quantize_bf16(const uint16_t* W, int64_t nweights, uint8_t* codes, uint8_t* q8, float* s2,
                                hipStream_t st) {
  const uint32_t nb = (uint32_t)(nweights / kBlock);
  const uint32_t ng = (nb + kGroup - 1) / kGroup;
  if (ng == 0) return hipSuccess;
  hipLaunchKernelGGL((k_quantize<uint16_t, true>), dim3(ng), dim3(256), 0, st, W, nb, codes, q8, s2,
                     (float*)nullptr, quant_search());
  return hipGetLastError();
}

hipError_t launch_dequant_fmt(const uint8_t* codes, const uint8_t* q8, const float* s2, const float* absmax,
                              int64_t nweights, bool uniform, bool dq, bool f16, uint16_t* out, hipStream_t st) {
  const uint32_t ndw = (uint32_t)(nweights / 8);
  if (ndw == 0) return hipSuccess;
  const uint32_t blocks = std::min<uint32_t>((ndw + 255) / 256, 4096u);
  const uint32_t* cw = reinterpret_cast<const uint32_t*>(codes);
  uint4* o = reinterpret_cast<uint4*>(out);
  const Nf4Consts& c = uniform ? int4_consts() : nf4_consts();
  if (f16) {
    if (dq) hipLaunchKernelGGL((k_dequant<true, F16>), dim3(blocks), dim3(256), 0, st, cw, q8, s2, absmax, ndw, o, c);
    else hipLaunchKernelGGL((k_dequant<false, F16>), dim3(blocks), dim3(256), 0, st, cw, q8, s2, absmax, ndw, o, c);
  } else {
    if (dq) hipLaunchKernelGGL((k_dequant<true, Bf16>), dim3(blocks), dim3(256), 0, st, cw, q8, s2, absmax, ndw, o, c);
    else hipLaunchKernelGGL((k_dequant<false, Bf16>), dim3(blocks), dim3(256), 0, st, cw, q8, s2, absmax, ndw, o, c);
  }
  return hipGetLastError();
}

QLORA_OOB_READER(oob_count_codec)

hipError_t launch_dequant(const uint8_t* codes, const uint8_t* q8, const float* s2, int64_t nweights,
                          uint16_t* out, bool f16, hipStream_t st) {
  return launch_dequant_fmt(codes, q8, s2, nullptr, nweights, false, true, f16, out, st);
}

}  // namespace qlora
