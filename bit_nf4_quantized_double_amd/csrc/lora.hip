// The adapter's down projection on its own ([P1] "The mechanism in brief":
// the adapter adds (alpha / r) B A x), for the paths that need U~ before
// anything else runs: the few-token forward and the backward when the
// forward's U~ was not kept.
//
//   rowdot:   U~[m][j] = E(s sum_k (mask * X)[m][k] A[j][k])        (M x r)
//
// v_mfma_f32_16x16x32 on 16-bit elements (bf16, or fp16 for the fp16
// instance) with the rank on the 16-wide side; split partial sums over k are
// added in a fixed order (deterministic) by a second pass, or by the
// few-token kernel, which stages them in LDS and adds them the same way.
#include <algorithm>

#include "common.h"
#include "dropout.h"

namespace qlora {

// K split of the rowdot kernel: enough (row block, split) workgroups to fill
// the GPU (>= 512), splits of whole 256-wide sub-chunks -- but no more
// partial sums than fit in 32 KB at a rank pitch of 8 (the few-token kernel
// stages them in LDS and adds them itself).
void rowdot_split(int M, int Kd, int r, int* nsplit, int* kchunk) {
  const int rb = (M + 63) / 64;
  const int nsub = std::max(1, (Kd + 255) / 256);
  const int cap = std::max(1, (32 << 10) / (std::max(M, 1) * std::max((r + 7) & ~7, 8) * 4));
  int ns = std::min({nsub, std::max(1, (512 + rb - 1) / rb), cap});
  const int per = (nsub + ns - 1) / ns;
  ns = (nsub + per - 1) / per;
  *nsplit = ns;
  *kchunk = per * 256;
}

int rowdot_nsplit(int64_t M, int64_t Kd, int r) {
  int ns, kc;
  rowdot_split((int)M, (int)Kd, r, &ns, &kc);
  return ns;
}

// fp32 partial bytes of the rowdot kernel for these sizes (one [M x r] sum
// per split, also when there is one split).
size_t rowdot_part_bytes(int64_t M, int64_t Kd, int r) {
  return (size_t)rowdot_nsplit(M, Kd, r) * (size_t)M * (size_t)r * 4u;
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

// out[m][j] = bf16(scale * sum_{split} part[split][m][j]): split 0's value,
// then the others added in split order (the few-token kernel adds its staged
// copy of the partials the same way).
template <typename E>
__device__ __forceinline__ void rowdot_finalize_body(const float* __restrict__ part, int nsplit, int64_t n,
                                                     float scale, uint16_t* __restrict__ out, int b, int nb) {
  for (int64_t i = (int64_t)b * 256 + threadIdx.x; i < n; i += (int64_t)nb * 256) {
    float s = part[i];
    int k = 1;
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

// keep_part: write the fp32 partial sums (also for one split) and stop
// there; otherwise round them into out (a finalize pass when split).
template <bool CONTIG, typename E>
hipError_t rowdot_dispatch(const uint16_t* in, int M, int Kd, const uint16_t* wt, int r, float scale,
                           uint16_t* out, float* part, DropMask drop, bool keep_part, hipStream_t st) {
  int nsplit, kchunk;
  rowdot_split(M, Kd, r, &nsplit, &kchunk);
  dim3 grid((M + 63) / 64, nsplit);
  float* p = nsplit > 1 || keep_part ? part : nullptr;
  switch ((r + 15) / 16) {
    case 1: rowdot_launch<CONTIG, 1, E>(grid, st, in, M, Kd, wt, r, kchunk, scale, out, p, drop); break;
    case 2: rowdot_launch<CONTIG, 2, E>(grid, st, in, M, Kd, wt, r, kchunk, scale, out, p, drop); break;
    case 3: rowdot_launch<CONTIG, 3, E>(grid, st, in, M, Kd, wt, r, kchunk, scale, out, p, drop); break;
    default: rowdot_launch<CONTIG, 4, E>(grid, st, in, M, Kd, wt, r, kchunk, scale, out, p, drop); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || keep_part || nsplit == 1) return e;
  const int64_t n = (int64_t)M * r;
  const int blocks = (int)std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 2048));
  hipLaunchKernelGGL(k_rowdot_finalize<E>, dim3(blocks), dim3(256), 0, st, part, nsplit, n, scale, out);
  return hipGetLastError();
}

}  // namespace

// U~ = E(s sum over splits of part) for rowdot's nsplit partials [nsplit][M][r].
hipError_t launch_rowdot_finalize(const float* part, int nsplit, int M, int r, float s, uint16_t* U, bool f16,
                                  hipStream_t st) {
  const int64_t n = (int64_t)M * r;
  if (n <= 0) return hipSuccess;
  const int blocks = (int)std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 2048));
  if (f16) hipLaunchKernelGGL(k_rowdot_finalize<F16>, dim3(blocks), dim3(256), 0, st, part, nsplit, n, s, U);
  else hipLaunchKernelGGL(k_rowdot_finalize<Bf16>, dim3(blocks), dim3(256), 0, st, part, nsplit, n, s, U);
  return hipGetLastError();
}

// The split partial sums of (mask * X) A^T alone, [rowdot_nsplit][M][r] fp32,
// for a consumer that adds them itself.
hipError_t launch_lora_down_partials(const uint16_t* X, int M, int K, const uint16_t* A, int r, float* part,
                                     DropMask drop, bool f16, hipStream_t st) {
  return f16 ? rowdot_dispatch<true, F16>(X, M, K, A, r, 1.f, nullptr, part, drop, true, st)
             : rowdot_dispatch<true, Bf16>(X, M, K, A, r, 1.f, nullptr, part, drop, true, st);
}

// U~ = E(s (mask * X) A^T): in = X [M x K], A [r x K]; E = fp16 when f16,
// else bf16.  part: fp32 split partials (rowdot_part_bytes).
hipError_t launch_lora_down(const uint16_t* X, int M, int K, const uint16_t* A, int r, float s, uint16_t* U,
                            float* part, DropMask drop, bool f16, hipStream_t st) {
  return f16 ? rowdot_dispatch<true, F16>(X, M, K, A, r, s, U, part, drop, false, st)
             : rowdot_dispatch<true, Bf16>(X, M, K, A, r, s, U, part, drop, false, st);
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
