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

// K split of the rowdot kernel (M <= 16 rows: one workgroup per split, its
// 4 waves taking the split's 256-wide sub-chunks in turn): about one
// sub-chunk per wave, but no more partial sums than fit in 32 KB at a rank
// pitch of 8 (the few-token kernel stages them in LDS and adds them itself).
void rowdot_split(int M, int Kd, int r, int* nsplit, int* kchunk) {
  const int nsub = std::max(1, (Kd + 255) / 256);
  const int cap = std::max(1, (32 << 10) / (std::max(M, 1) * std::max((r + 7) & ~7, 8) * 4));
  int ns = std::min((nsub + 3) / 4, cap);
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



// ---------------------------------------------------------------- rowdot ----
// out[m][j] = E(scale * sum_k (mask * in)[m][k] * A[j][k]), m < M <= 16, j < r.
//
// Grid (1, K splits) of 256-thread workgroups.  A workgroup covers all M
// rows and one K range; its 4 waves take the range's 256-wide sub-chunks in
// turn (wave w: sub-chunks w, w + 4, ...).  Both MFMA operands come straight
// from global memory into registers -- the activations (lane: row l & 15,
// 8 columns at 8 (l >> 4)) and A (lane: rank 16 t + (l & 15), the same
// columns) are both row-major along k -- so a sub-chunk costs one memory
// round trip and no LDS.  The 4 waves' sums are added in wave order in LDS;
// with one split the result is rounded and stored, otherwise the fp32
// partial [split][m][j] is stored (added up by k_rowdot_finalize, or by the
// few-token kernel, in split order).
constexpr int kRowdotSub = 256;  // reduction columns per sub-chunk

struct RowdotArgs {
  const uint16_t* in;  // [M x Kd], M <= 16
  int M, Kd;
  const uint16_t* wt;  // A [r x Kd]
  int r, kchunk, nsplit;
  float scale;
  uint16_t* out;       // [M x r] bf16
  float* part;         // [nsplit][M][r] fp32, or null (then rounded into out)
  DropMask drop;       // dropout of `in` (thr 0: none)
};

template <int RT, typename E>
__global__ __launch_bounds__(256) void k_rowdot(RowdotArgs ra) {
  constexpr int kRP = 16 * RT + 1;  // LDS pitch of the wave sums (odd: no bank conflicts)
  __shared__ float red[4 * 16 * kRP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int M = ra.M, Kd = ra.Kd, r = ra.r;
  const int split = blockIdx.y;
  const int k_lo = split * ra.kchunk, k_hi = min(Kd, k_lo + ra.kchunk);
  const int row = lane & 15, kg = lane >> 4;
  const __amdgpu_buffer_rsrc_t rin = make_rsrc(ra.in, (uint32_t)((uint64_t)M * Kd * 2));
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(ra.wt, (uint32_t)((uint64_t)r * Kd * 2));
  const uint32_t xrow = row < M ? (uint32_t)row * (uint32_t)Kd * 2u : kOOB;
  uint32_t wrow[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) wrow[t] = 16 * t + row < r ? (uint32_t)(16 * t + row) * (uint32_t)Kd * 2u : kOOB;

  f32x4 acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = k_lo + kRowdotSub * wave; k0 < k_hi; k0 += 4 * kRowdotSub) {
    uint4 av[8], bv[RT][8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int k = k0 + 32 * u + 8 * kg;
      const bool ok = k < k_hi;  // Kd % 8 == 0: the 8 columns are all in range
      av[u] = buf_load16(rin, ok && xrow != kOOB ? xrow + 2u * (uint32_t)k : kOOB);
#pragma unroll
      for (int t = 0; t < RT; ++t) bv[t][u] = buf_load16(rw, ok && wrow[t] != kOOB ? wrow[t] + 2u * (uint32_t)k : kOOB);
    }
    if (ra.drop.thr) {
#pragma unroll
      for (int u = 0; u < 8; ++u)
        av[u] = drop8(av[u], (uint64_t)row * (uint64_t)Kd + (uint64_t)(k0 + 32 * u + 8 * kg), ra.drop);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int t = 0; t < RT; ++t) acc[t] = E::mfma16(E::vec(av[u]), E::vec(bv[t][u]), acc[t]);
  }
  // D[m][j]: m = 4 (lane >> 4) + v, j = 16 t + (lane & 15); waves added in order
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[(wave * 16 + 4 * kg + v) * kRP + 16 * t + row] = acc[t][v];
  __syncthreads();
  for (int idx = tid; idx < 16 * 16 * RT; idx += 256) {
    const int m = idx / (16 * RT), j = idx - m * (16 * RT);
    if (m >= M || j >= r) continue;
    float s = red[m * kRP + j];
#pragma unroll
    for (int w = 1; w < 4; ++w) s += red[(w * 16 + m) * kRP + j];
    if (ra.part) {
      if (in_bounds(((int64_t)split * M + m) * r + j, 1, (int64_t)ra.nsplit * M * r))
        ra.part[((int64_t)split * M + m) * r + j] = s;
    } else {
      const uint32_t pk = E::pack2(ra.scale * s, 0.f);
      if (in_bounds((int64_t)m * r + j, 1, (int64_t)M * r)) ra.out[(int64_t)m * r + j] = (uint16_t)(pk & 0xFFFFu);
    }
  }
}

// out[m][j] = bf16(scale * sum_{split} part[split][m][j]): split 0's value,
// then the others added in split order (the few-token kernel adds its staged
// copy of the partials the same way).
template <typename E>
__device__ __forceinline__ void rowdot_finalize_body(const float* __restrict__ part, int nsplit, int64_t n,
                                                     float scale, uint16_t* __restrict__ out, int b, int nb) {
  for (int64_t i = (int64_t)b * 256 + threadIdx.x; i < n; i += (int64_t)nb * 256) {
    if (!in_bounds((int64_t)(nsplit - 1) * n + i, 1, (int64_t)nsplit * n)) continue;
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
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    if (in_bounds(i, 1, n)) p[i] = 0.f;
}

__global__ __launch_bounds__(256) void k_zero_u16(uint16_t* __restrict__ p, int64_t n) {
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    if (in_bounds(i, 1, n)) p[i] = 0;
}

template <int RT, typename E>
void rowdot_launch(dim3 grid, hipStream_t st, const uint16_t* in, int M, int Kd, const uint16_t* wt, int r,
                   int kchunk, float scale, uint16_t* out, float* part, DropMask drop) {
  const RowdotArgs ra{in, M, Kd, wt, r, kchunk, (int)grid.y, scale, out, part, drop};
  hipLaunchKernelGGL((k_rowdot<RT, E>), grid, dim3(256), 0, st, ra);
}

// keep_part: write the fp32 partial sums (also for one split) and stop
// there; otherwise round them into out (a finalize pass when split).
template <typename E>
hipError_t rowdot_dispatch(const uint16_t* in, int M, int Kd, const uint16_t* wt, int r, float scale,
                           uint16_t* out, float* part, DropMask drop, bool keep_part, hipStream_t st) {
  if (M > 16) return hipErrorInvalidValue;
  int nsplit, kchunk;
  rowdot_split(M, Kd, r, &nsplit, &kchunk);
  dim3 grid(1, nsplit);
  float* p = nsplit > 1 || keep_part ? part : nullptr;
  switch ((r + 15) / 16) {
    case 1: rowdot_launch<1, E>(grid, st, in, M, Kd, wt, r, kchunk, scale, out, p, drop); break;
    case 2: rowdot_launch<2, E>(grid, st, in, M, Kd, wt, r, kchunk, scale, out, p, drop); break;
    case 3: rowdot_launch<3, E>(grid, st, in, M, Kd, wt, r, kchunk, scale, out, p, drop); break;
    default: rowdot_launch<4, E>(grid, st, in, M, Kd, wt, r, kchunk, scale, out, p, drop); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || keep_part || nsplit == 1) return e;
  const int64_t n = (int64_t)M * r;
  const int blocks = (int)std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 2048));
  hipLaunchKernelGGL(k_rowdot_finalize<E>, dim3(blocks), dim3(256), 0, st, part, nsplit, n, scale, out);
  return hipGetLastError();
}

}  // namespace

QLORA_OOB_READER(oob_count_lora)

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
  return f16 ? rowdot_dispatch<F16>(X, M, K, A, r, 1.f, nullptr, part, drop, true, st)
             : rowdot_dispatch<Bf16>(X, M, K, A, r, 1.f, nullptr, part, drop, true, st);
}

// U~ = E(s (mask * X) A^T): in = X [M x K], A [r x K]; E = fp16 when f16,
// else bf16.  part: fp32 split partials (rowdot_part_bytes).
hipError_t launch_lora_down(const uint16_t* X, int M, int K, const uint16_t* A, int r, float s, uint16_t* U,
                            float* part, DropMask drop, bool f16, hipStream_t st) {
  return f16 ? rowdot_dispatch<F16>(X, M, K, A, r, s, U, part, drop, false, st)
             : rowdot_dispatch<Bf16>(X, M, K, A, r, s, U, part, drop, false, st);
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
