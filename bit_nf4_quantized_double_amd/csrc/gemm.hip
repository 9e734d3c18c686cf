// Fused NF4-dequant bf16 MFMA GEMMs of the QLoRA linear.
//
// Forward ([P1] "The mechanism in brief"; [P4] "The idea in one line"):
//     Y[m][n]  = sum_k X[m][k] * Wbf[n][k]  +  sum_j U~[m][j] * B[n][j]
// dX (backward for the activations):
//     dX[m][c] = sum_n dY[m][n] * Wbf[n][c] +  sum_j V~[m][j] * A[j][c]
//
// Wbf is never materialised: each 64-deep reduction step the workgroup reads
// the packed codes of the W tile it needs, decodes them to bf16 (level * block
// scale, round to nearest even) and stores them in LDS, where they feed
// v_mfma_f32_32x32x16_bf16.  The rank-r adapter term runs as one extra
// reduction step over the r adapter columns, into the same accumulators.
//
// Tile: BM x BN outputs per 256-thread workgroup, 2 x 2 waves, each wave
// (BM/2) x (BN/2) as (BM/64) x (BN/64) MFMA tiles of 32 x 32.
//   NT (forward): W tile = BN rows n x 64 k, stored [n][k] (k contiguous),
//                 read with ds_read_b128 like the activation tile.
//   NN (dX):      W tile = 64 rows n x BN columns c, stored [n][c] (c
//                 contiguous) exactly as decoded; the MFMA B operand needs 8
//                 consecutive n per lane and gets them with gfx950's
//                 transposing LDS read ds_read_b64_tr_b16.
#include "gemm_args.h"

namespace qlora {


namespace {

constexpr int kThreads = 256;

typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// ---- shared-memory tile geometry ------------------------------------------
// Activation tile / NT weight tile: rows of 64 bf16 (128 B), 16-byte chunks
// XOR-swizzled by swz(row).
__device__ __forceinline__ uint32_t kt_off(uint32_t row, uint32_t chunk) {
  return row * 64u + ((chunk ^ swz(row)) << 3);
}
// NN weight tile: 64 rows (n) of BN bf16, padded by 16 elements so the 4 rows
// touched by one transposing read land in different banks.
template <int BN>
__device__ __forceinline__ uint32_t nn_off(uint32_t row, uint32_t col) {
  return row * (uint32_t)(BN + 16) + col;
}

template <int BM, int BN, bool NN>
struct Smem {
  static constexpr int kAct = BM * 64;                         // elements per buffer
  static constexpr int kW = NN ? 64 * (BN + 16) : BN * 64;
  static constexpr int kBytes = 2 * 2 * (kAct + kW);            // double-buffered bf16
};

// ---- activation tile: BM rows x 64 reduction columns ----------------------
template <int BM>
struct ActLoader {
  static constexpr int kChunks = BM * 8 / kThreads;  // 16-byte chunks per thread
  uint4 v[kChunks];

  __device__ __forceinline__ void load(const GemmArgs& a, int m0, int r0, int tid) {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      int q = tid + i * kThreads;
      int row = q >> 3, ch = q & 7;
      int m = m0 + row, rr = r0 + ch * 8;
      if (m < a.M && rr < a.R)
        v[i] = *reinterpret_cast<const uint4*>(a.act + (int64_t)m * a.ld_act + rr);
      else
        v[i] = make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(uint16_t* s, int tid) const {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      int q = tid + i * kThreads;
      *reinterpret_cast<uint4*>(s + kt_off(q >> 3, q & 7)) = v[i];
    }
  }
};

// ---- W tile: each thread decodes 32 consecutive weights of one W row ------
// NT: BN rows (n = c0 + row) x 64 k starting at r0.
// NN: 64 rows (n = r0 + row) x BN columns starting at c0.
template <int BN, bool NN>
struct WLoader {
  static constexpr int kRows = NN ? 64 : BN;
  static constexpr int kSegs = (NN ? BN : 64) / 32;            // 32-weight segments per row
  static constexpr int kPer = kRows * kSegs / kThreads;         // segments per thread
  static_assert(kRows * kSegs % kThreads == 0, "tile/thread mismatch");
  uint4 code[kPer];
  float scale[kPer];

  __device__ __forceinline__ void load(const GemmArgs& a, int c0, int r0, int tid) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      int s = tid + i * kThreads;
      int row = s / kSegs, seg = s % kSegs;
      int n, k;
      bool ok;
      if (NN) { n = r0 + row; k = c0 + seg * 32; ok = n < a.R && k < a.C; }
      else    { n = c0 + row; k = r0 + seg * 32; ok = n < a.C; }
      if (ok) {
        uint32_t e = (uint32_t)n * (uint32_t)a.K + (uint32_t)k;   // weight index
        code[i] = *reinterpret_cast<const uint4*>(a.codes + (e >> 1));
        scale[i] = block_scale(a.q8, a.s2, e >> 6);
      } else {
        code[i] = make_uint4(0x77777777u, 0x77777777u, 0x77777777u, 0x77777777u);  // level 0.0
        scale[i] = 0.f;
      }
    }
  }
  __device__ __forceinline__ void store(uint16_t* s, int tid, const float* lv) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      int sg = tid + i * kThreads;
      int row = sg / kSegs, seg = sg % kSegs;
      uint4 w0 = decode8(code[i].x, scale[i], lv);
      uint4 w1 = decode8(code[i].y, scale[i], lv);
      uint4 w2 = decode8(code[i].z, scale[i], lv);
      uint4 w3 = decode8(code[i].w, scale[i], lv);
      if (NN) {
        uint16_t* p = s + nn_off<BN>(row, seg * 32);
        reinterpret_cast<uint4*>(p)[0] = w0;
        reinterpret_cast<uint4*>(p)[1] = w1;
        reinterpret_cast<uint4*>(p)[2] = w2;
        reinterpret_cast<uint4*>(p)[3] = w3;
      } else {
        *reinterpret_cast<uint4*>(s + kt_off(row, seg * 4 + 0)) = w0;
        *reinterpret_cast<uint4*>(s + kt_off(row, seg * 4 + 1)) = w1;
        *reinterpret_cast<uint4*>(s + kt_off(row, seg * 4 + 2)) = w2;
        *reinterpret_cast<uint4*>(s + kt_off(row, seg * 4 + 3)) = w3;
      }
    }
  }
};

// B operand (W side) for one 32 x 32 x 16 MFMA: output columns col0..col0+31,
// reduction rows 16*ks .. 16*ks+15 of the current step.
template <int BN, bool NN>
__device__ __forceinline__ bf16x8 load_bfrag(const uint16_t* s, int col0, int ks, int lane) {
  if (!NN) {
    uint4 v = *reinterpret_cast<const uint4*>(s + kt_off(col0 + (lane & 31), ks * 2 + (lane >> 5)));
    return __builtin_bit_cast(bf16x8, v);
  } else {
    // lane (within its 16-lane group g) = p + 4q addresses row k0 + q, columns
    // cb + 4p..4p+3; it receives column cb + (lane & 15), rows k0..k0+3.
    int g = lane >> 4, i = lane & 15;
    int p = i & 3, q = i >> 2;
    int cb = col0 + (g & 1) * 16 + 4 * p;
    int k0 = ks * 16 + (g >> 1) * 8;
    i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(s + nn_off<BN>(k0 + q, cb)));
    i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(s + nn_off<BN>(k0 + 4 + q, cb)));
    typedef __attribute__((ext_vector_type(8))) short i16x8;
    i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
  }
}

template <int BM>
__device__ __forceinline__ bf16x8 load_afrag(const uint16_t* s, int row0, int ks, int lane) {
  uint4 v = *reinterpret_cast<const uint4*>(s + kt_off(row0 + (lane & 31), ks * 2 + (lane >> 5)));
  return __builtin_bit_cast(bf16x8, v);
}

template <int BM, int BN, bool NN>
__global__ __launch_bounds__(kThreads) void k_gemm_nf4(GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  using S = Smem<BM, BN, NN>;
  constexpr int TM = BM / 64, TN = BN / 64;  // MFMA tiles per wave
  // buffer b: activations at smem + b*kAct, W tile at smem + 2*kAct + b*kW
  auto s_act = [&](int b) { return smem + b * S::kAct; };
  auto s_w = [&](int b) { return smem + 2 * S::kAct + b * S::kW; };
  __shared__ float s_lv[16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM, c0 = blockIdx.x * BN;
  if (tid < 16) s_lv[tid] = a.nf4.level[tid];

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  ActLoader<BM> al;
  WLoader<BN, NN> wl;
  const int nsteps = (a.R + 63) / 64;

  al.load(a, m0, 0, tid);
  wl.load(a, c0, 0, tid);
  __syncthreads();  // s_lv visible
  al.store(s_act(0), tid);
  wl.store(s_w(0), tid, s_lv);
  __syncthreads();

  for (int step = 0; step < nsteps; ++step) {
    const int buf = step & 1;
    const bool more = step + 1 < nsteps;
    if (more) {
      al.load(a, m0, (step + 1) * 64, tid);
      wl.load(a, c0, (step + 1) * 64, tid);
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = load_afrag<BM>(s_act(buf), wm * (BM / 2) + 32 * i, ks, lane);
#pragma unroll
      for (int j = 0; j < TN; ++j) bfr[j] = load_bfrag<BN, NN>(s_w(buf), wn * (BN / 2) + 32 * j, ks, lane);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      al.store(s_act(buf ^ 1), tid);
      wl.store(s_w(buf ^ 1), tid, s_lv);
    }
    __syncthreads();
  }

  // ---- adapter step: r extra reduction columns ---------------------------
  if (a.r > 0) {
    const int buf = nsteps & 1;
    const int rp = (a.r + 15) & ~15;
    uint16_t* sa = s_act(buf);
    uint16_t* sw = s_w(buf);
    for (int idx = tid; idx < BM * rp; idx += kThreads) {
      int row = idx / rp, j = idx % rp;
      int m = m0 + row;
      uint16_t v = (m < a.M && j < a.r) ? a.lora_act[(int64_t)m * a.r + j] : (uint16_t)0;
      sa[kt_off(row, j >> 3) + (j & 7)] = v;
    }
    for (int idx = tid; idx < BN * rp; idx += kThreads) {
      if (!NN) {
        int col = idx / rp, j = idx % rp;
        int n = c0 + col;
        uint16_t v = (n < a.C && j < a.r) ? a.lora_w[(int64_t)n * a.r + j] : (uint16_t)0;
        sw[kt_off(col, j >> 3) + (j & 7)] = v;
      } else {
        int j = idx / BN, col = idx % BN;
        int c = c0 + col;
        uint16_t v = (c < a.C && j < a.r) ? a.lora_w[(int64_t)j * a.K + c] : (uint16_t)0;
        sw[nn_off<BN>(j, col)] = v;
      }
    }
    __syncthreads();
    for (int ks = 0; ks < rp / 16; ++ks) {
      bf16x8 af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = load_afrag<BM>(sa, wm * (BM / 2) + 32 * i, ks, lane);
#pragma unroll
      for (int j = 0; j < TN; ++j) bfr[j] = load_bfrag<BN, NN>(sw, wn * (BN / 2) + 32 * j, ks, lane);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }

  // ---- epilogue: fp32 -> bf16 (round to nearest even) ---------------------
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = c0 + wn * (BN / 2) + 32 * j + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; v += 2) {
        const int row = m0 + wm * (BM / 2) + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        uint32_t pk = pack_bf16x2(acc[i][j][v], acc[i][j][v + 1]);
        if (col < a.C) {
          if (row < a.M) a.out[(int64_t)row * a.ld_out + col] = (uint16_t)(pk & 0xFFFFu);
          if (row + 1 < a.M) a.out[(int64_t)(row + 1) * a.ld_out + col] = (uint16_t)(pk >> 16);
        }
      }
    }
}

thread_local hipEvent_t t_ev_start = nullptr, t_ev_stop = nullptr;

template <int BM, int BN, bool NN>
hipError_t launch(const GemmArgs& a, hipStream_t st) {
  auto kern = k_gemm_nf4<BM, BN, NN>;
  constexpr int bytes = Smem<BM, BN, NN>::kBytes;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  hipEvent_t ev0 = t_ev_start, ev1 = t_ev_stop;
  t_ev_start = t_ev_stop = nullptr;
  if (ev0 && (e = hipEventRecord(ev0, st)) != hipSuccess) return e;
  dim3 grid((a.C + BN - 1) / BN, (a.M + BM - 1) / BM);
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), bytes, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ev1 && (e = hipEventRecord(ev1, st)) != hipSuccess) return e;
  return hipSuccess;
}

}  // namespace

void time_next_gemm(hipEvent_t start, hipEvent_t stop) {
  if (start && stop) { t_ev_start = start; t_ev_stop = stop; }
  else { t_ev_start = t_ev_stop = nullptr; }
}

hipError_t launch_gemm_fwd(const GemmArgs& a, hipStream_t st) { return launch<128, 128, false>(a, st); }
hipError_t launch_gemm_dx(const GemmArgs& a, hipStream_t st) { return launch<128, 128, true>(a, st); }

}  // namespace qlora
