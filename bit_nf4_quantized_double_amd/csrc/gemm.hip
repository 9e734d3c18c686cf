// Fused NF4-dequant bf16 MFMA GEMMs of the QLoRA linear.
//
// Forward ([P1] "The mechanism in brief"; [P4] "The idea in one line"):
//     Y[m][n]  = sum_k X[m][k] * Wbf[n][k]  +  sum_j U~[m][j] * B[n][j]
// dX (backward for the activations):
//     dX[m][c] = sum_n dY[m][n] * Wbf[n][c] +  sum_j V~[m][j] * A[j][c]
//
// Wbf is never materialised.  Each 64-deep reduction step a workgroup reads
// the packed codes of the W tile it needs, decodes them to bf16
// (round-to-nearest-even of level * block scale) in registers and stores the
// tile in LDS, where all four waves read it as the MFMA B operand.  The rank-r
// adapter term is one extra reduction step into the same accumulators.
//
// Workgroup tile 256 (rows) x 128 (columns), 4 waves stacked along the rows;
// each wave owns 64 rows x 128 columns = 2 x 4 tiles of
// v_mfma_f32_32x32x16_bf16.  A wave's activation rows are private to it: it
// copies them with coalesced buffer_load ... lds (8 lanes per 128-byte row
// slice, straight into a wave-private LDS ring, no VGPR round trip) and reads
// them back in MFMA operand layout.  The decoded W tile is double-buffered
// and shared by the four waves (one barrier per step).
//
//   NT (forward): W tile = 128 rows n x 64 k, stored [n][k], read with
//                 ds_read_b128.
//   NN (dX):      W tile = 64 rows n x 128 columns c, stored [n][c] as
//                 decoded; the B operand needs 8 consecutive n per lane and
//                 gets them with gfx950's transposing ds_read_b64_tr_b16.
// Rows of 64 bf16 (128 B) keep their 16-byte chunks XOR-swizzled by swz(row)
// so row-consecutive operand reads are bank-conflict-free.
//
// Decode: each thread decodes 32 consecutive weights of one 64-weight block
// (one block scale).  The 16 values bf16(level[c] * scale) form a per-block
// lookup table held as byte planes in registers and indexed with v_perm_b32;
// the two lanes sharing a block each build half the table and swap halves
// with one DPP move.  No LDS traffic for the lookup.
//
// Few output tiles (at most half as many as compute units): grid z splits the
// reduction into ksplit ranges; each workgroup stores its fp32 tile and
// k_splitk_reduce adds the tiles in split order and rounds once.
#include <algorithm>

#include "dropout.h"
#include "gemm_args.h"
#include "nf4_lut.h"

namespace qlora {

// Pending measurement request of qlora_time_next_gemm (thread-local): the
// events to record around the next fused-GEMM launch; taking clears it.
void take_gemm_events(hipEvent_t& start, hipEvent_t& stop);

namespace {

constexpr int kThreads = 256;
constexpr int BM = 256, BN = 128;

typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(8))) short i16x8;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// ---- LDS tile geometry -----------------------------------------------------
// NT W tile: rows of 64 bf16 (128 B), 16-byte chunks XOR-swizzled by swz(row).
__device__ __forceinline__ uint32_t kt_off(uint32_t row, uint32_t chunk) {
  return row * 64u + ((chunk ^ swz(row)) << 3);
}
// NN W tile: 64 rows of BN bf16, padded by 32 elements; 16-byte chunk ch of
// row n is stored at chunk ch ^ 2 (ch >> 3) ^ (n & 3).  Both the producers'
// ds_write_b128 (4 threads per row at 64-byte stride) and the consumers'
// transposing ds_read_b64_tr_b16 are then free of LDS bank conflicts
// (measured with SQ_LDS_BANK_CONFLICT; a 16-element pad with only the upper
// half-row flipped, conflict-free in a 32-bank model, cost 2 conflict cycles
// per transposing read).
constexpr int kNNPitch = BN + 32;
__device__ __forceinline__ uint32_t nn_off(uint32_t row, uint32_t col) {
  const uint32_t ch = col >> 3;
  return row * kNNPitch + ((((ch ^ ((ch >> 3) << 1) ^ (row & 3)) & 15u) << 3) | (col & 7));
}

template <bool NN>
struct Tile {
  static constexpr int kElems = NN ? 64 * kNNPitch : BN * 64;  // bf16 per buffer
};

// ---- global -> register loads (raw buffer loads: out of range reads 0) ----
struct Srcs {
  __amdgpu_buffer_rsrc_t act, codes, q8, s2;
  __amdgpu_buffer_rsrc_t lora_act, lora_w;  // U~ or V~ [M x r]; B [C x r] (NT) or A [r x K] (NN)
};

template <bool NN>
__device__ __forceinline__ Srcs make_srcs(const GemmArgs& a) {
  Srcs s;
  // W is [n_out x k_in]: n_out = C (forward) or R (dX)
  const uint64_t wn = (uint64_t)a.K * (uint64_t)(NN ? a.R : a.C);
  const uint32_t nb = (uint32_t)(wn >> 6);
  s.act = make_rsrc(a.act, (uint32_t)((uint64_t)a.M * a.ld_act * 2));
  s.codes = make_rsrc(a.codes, (uint32_t)(wn >> 1));
  s.q8 = make_rsrc(a.q8, nb);
  s.s2 = make_rsrc(a.s2, ((nb + 255) >> 8) * 4);
  s.lora_act = make_rsrc(a.lora_act, (uint32_t)((uint64_t)a.M * a.r * 2));
  s.lora_w = make_rsrc(a.lora_w, (uint32_t)((uint64_t)(NN ? a.K : a.C) * a.r * 2));
  return s;
}

// 8 consecutive 16-bit elements starting at element e of a buffer, of which the first
// `valid` (clamped to 0..8) are real and the rest read as zero; nothing at
// all when !ok.  vec: e is a multiple of 8 (one 16-byte load); otherwise the
// elements are loaded one by one (all loads independent).
__device__ __forceinline__ uint4 load_e16x8(__amdgpu_buffer_rsrc_t r, uint32_t e, bool ok, int valid,
                                             bool vec) {
  if (!ok || valid <= 0) return make_uint4(0, 0, 0, 0);
  if (vec && valid >= 8) return buf_load16(r, 2u * e);
  uint32_t h[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    h[i] = i < valid ? __builtin_amdgcn_raw_buffer_load_b16(r, 2u * (e + i), 0, 0) : 0u;
  return make_uint4(h[0] | h[1] << 16, h[2] | h[3] << 16, h[4] | h[5] << 16, h[6] | h[7] << 16);
}

// Codes of the 32 weights this thread decodes for the step starting at r0.
struct CodeSeg {
  uint4 code;
  uint32_t q;  // 8-bit block absmax code
  float s2;    // second-level scale of its group
};

template <bool NN>
__device__ __forceinline__ CodeSeg load_codes(const GemmArgs& a, const Srcs& src, int c0, int r0, int tid) {
  int n, k;
  bool ok;
  if (NN) { n = r0 + (tid >> 2); k = c0 + (tid & 3) * 32; ok = n < a.R && k < a.C; }
  else    { n = c0 + (tid >> 1); k = r0 + (tid & 1) * 32; ok = n < a.C && k < a.R; }
  const uint32_t e = (uint32_t)n * (uint32_t)a.K + (uint32_t)k;  // weight index
  CodeSeg cs;  // out of range: all zero, which decodes to zeros
  cs.code = buf_load16(src.codes, ok ? (e >> 1) : kOOB);
  cs.q = buf_load1(src.q8, ok ? (e >> 6) : kOOB);
  cs.s2 = __builtin_bit_cast(float, buf_load4(src.s2, ok ? ((e >> 14) << 2) : kOOB));
  return cs;
}

template <bool NN, typename E>
__device__ __forceinline__ void decode_store(uint16_t* s, const CodeSeg& cs, const float th[8],
                                             const LaneMask& lm, int tid) {
  const Lut L = build_lut<LutPartner::kXor1, E>(th, (float)cs.q * cs.s2);  // a' = fp32(q8 * s2)
  const uint4 w0 = decode8_lut(L, cs.code.x, lm);
  const uint4 w1 = decode8_lut(L, cs.code.y, lm);
  const uint4 w2 = decode8_lut(L, cs.code.z, lm);
  const uint4 w3 = decode8_lut(L, cs.code.w, lm);
  if (NN) {
    const int row = tid >> 2, c = (tid & 3) * 32;
    *reinterpret_cast<uint4*>(s + nn_off(row, c + 0)) = w0;
    *reinterpret_cast<uint4*>(s + nn_off(row, c + 8)) = w1;
    *reinterpret_cast<uint4*>(s + nn_off(row, c + 16)) = w2;
    *reinterpret_cast<uint4*>(s + nn_off(row, c + 24)) = w3;
  } else {
    const int row = tid >> 1, c = (tid & 1) * 4;
    *reinterpret_cast<uint4*>(s + kt_off(row, c + 0)) = w0;
    *reinterpret_cast<uint4*>(s + kt_off(row, c + 1)) = w1;
    *reinterpret_cast<uint4*>(s + kt_off(row, c + 2)) = w2;
    *reinterpret_cast<uint4*>(s + kt_off(row, c + 3)) = w3;
  }
}

// ---- activations: coalesced copies into a wave-private LDS ring ----------
// One stage = the wave's 64 rows x 64 reduction columns (8 KB), row r at
// byte r * 128 with chunk lc stored at physical chunk lc ^ swz(r).
constexpr uint32_t kActStage = 64 * 128;
constexpr int kActStages = 3;

// Byte offsets of the 8 rows this lane copies (row 8j + (lane >> 3) of the
// wave's 64 rows for copy instruction j; kOOB past the last row).
struct ActRows {
  uint32_t off[8];
};

__device__ __forceinline__ ActRows act_rows(const GemmArgs& a, int row0, int lane) {
  ActRows ar;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int m = row0 + 8 * j + (lane >> 3);
    ar.off[j] = m < a.M ? (uint32_t)m * (uint32_t)a.ld_act * 2u : kOOB;
  }
  return ar;
}

typedef __attribute__((address_space(3))) uint8_t lds_u8;

// Issue the 8 coalesced copies of one step (reduction columns r0..r0+63) into
// the LDS stage at byte offset `stage`.  Lane l of copy j lands at stage +
// 1024 j + 16 l = row (8j + l / 8), physical chunk l % 8.
__device__ __forceinline__ void copy_act(const GemmArgs& a, const Srcs& src, const ActRows& rows, lds_u8* stage,
                                         int r0, int lane) {
  const uint32_t pc = lane & 7, rl = lane >> 3;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t lc = pc ^ ((rl ^ (uint32_t)j) & 7u);  // logical chunk = pc ^ swz(8j + rl)
    const int k = r0 + 8 * (int)lc;
    const uint32_t off = k < a.R ? rows.off[j] + 2u * (uint32_t)k : kOOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src.act, stage + 1024u * j, 16, off, 0, 0, 0);
  }
}

// A operand for MFMA sub-step ks, rows 32 i .. 32 i + 31 of the wave's slice.
__device__ __forceinline__ uint4 load_afrag(const uint16_t* st, int i, int ks, int lane) {
  const uint32_t r = 32 * i + (lane & 31);
  return *reinterpret_cast<const uint4*>(st + r * 64u + (((2u * ks + (lane >> 5)) ^ swz(r)) << 3));
}

// B operand for MFMA sub-step ks, columns col0..col0+31.
template <bool NN>
__device__ __forceinline__ uint4 load_bfrag(const uint16_t* s, int col0, int ks, int lane) {
  if (!NN) {
    return *reinterpret_cast<const uint4*>(s + kt_off(col0 + (lane & 31), 2 * ks + (lane >> 5)));
  } else {
    // 16-lane group g: lanes 0-31 are half 0 (rows 16 ks .. +7), 32-63 half 1
    // (rows 16 ks + 8 .. +15); odd groups take columns 16..31.  Lane p + 4q addresses row nb + q, columns cb + 4p and
    // receives column cb + (lane & 15), rows nb .. nb + 3.
    const int g = lane >> 4, i = lane & 15;
    const int cb = col0 + (g & 1) * 16 + 4 * (i & 3);
    const int nb = 16 * ks + 8 * (g >> 1) + (i >> 2);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(s + nn_off(nb, cb)));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(s + nn_off(nb + 4, cb)));
    const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(uint4, v);
  }
}

// One reduction step of MFMAs: A operand from the wave's activation stage,
// B operand from the shared W tile.  If cs is given, the next W tile is
// decoded into s_next alongside: MFMA sub-step ks is paired with code dword ks
// of this thread's 32 weights, so the decode VALU work issues while the matrix
// core runs (sub-steps are fenced so the compiler keeps that pairing).  B
// operands of sub-step ks + 1 are read during sub-step ks.
template <bool NN>
__device__ __forceinline__ void store_w8(uint16_t* s_next, const uint4& w, int q, int tid) {
  if (NN) *reinterpret_cast<uint4*>(s_next + nn_off(tid >> 2, (tid & 3) * 32 + 8 * q)) = w;
  else *reinterpret_cast<uint4*>(s_next + kt_off(tid >> 1, (tid & 1) * 4 + q)) = w;
}

template <bool NN, bool DECODE, typename E>
__device__ __forceinline__ void mma_step(f32x16 (&acc)[2][4], const uint16_t* act, const uint16_t* sw,
                                         uint16_t* s_next, const CodeSeg& cs, const float th[8],
                                         const LaneMask& lm, int tid, int lane) {
  uint4 nb[4], na[2];
#pragma unroll
  for (int j = 0; j < 4; ++j) nb[j] = load_bfrag<NN>(sw, 32 * j, 0, lane);
#pragma unroll
  for (int i = 0; i < 2; ++i) na[i] = load_afrag(act, i, 0, lane);
  Lut L;
  if (DECODE) L = build_lut<LutPartner::kXor1, E>(th, (float)cs.q * cs.s2);  // a' = fp32(q8 * s2)
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    uint4 bf[4], af[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) bf[j] = nb[j];
#pragma unroll
    for (int i = 0; i < 2; ++i) af[i] = na[i];
    if (ks < 3) {
#pragma unroll
      for (int j = 0; j < 4; ++j) nb[j] = load_bfrag<NN>(sw, 32 * j, ks + 1, lane);
#pragma unroll
      for (int i = 0; i < 2; ++i) na[i] = load_afrag(act, i, ks + 1, lane);
    }
    if (DECODE) {
      const uint32_t d = ks == 0 ? cs.code.x : ks == 1 ? cs.code.y : ks == 2 ? cs.code.z : cs.code.w;
      store_w8<NN>(s_next, decode8_lut(L, d, lm), ks, tid);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = E::mfma32(E::vec(af[i]), E::vec(bf[j]), acc[i][j]);
    if (DECODE) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // then up to 4 VALU
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// s_waitcnt with only a vmcnt limit (gfx9 encoding: vmcnt in bits 3:0 and
// 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their "no wait" maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Step hand-off barrier of the main loop.  A plain __syncthreads() carries a
// workgroup release fence, which would also drain the activation copies
// still in flight for later steps; here each wave first waits only for its
// own LDS operations (lgkmcnt(0): decoded-tile stores, operand reads), and
// producers additionally wait for the copies the next step needs before
// calling this (wait_vmcnt).
__device__ __forceinline__ void step_barrier() {
  __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0) only
  __builtin_amdgcn_s_barrier();
}

// XCD-aware tile order.  Workgroups are dealt round-robin to the 8 XCDs, so
// lin % 8 picks the XCD; each XCD gets a contiguous run t of the tile order
// below.  Tiles are ordered in bands of 2 row blocks, column-major inside a
// band: with 8 row blocks (2048 tokens) an XCD owns 2 row blocks x half the
// column tiles, so its L2 is shared by 2 activation row blocks and half the
// weight (instead of 1 row block and the whole weight).
__device__ __forceinline__ void tile_coords(int& tm, int& tn) {
  constexpr int RB = 2;  // row blocks per band
  const int nt = gridDim.x, mt = gridDim.y, total = nt * mt;
  const int lin = blockIdx.x + blockIdx.y * nt;
  const int t = (total % 8 == 0) ? (lin % 8) * (total / 8) + lin / 8 : lin;
  const int band = t / (RB * nt);
  const int rows = min(RB, mt - band * RB);  // the last band may be partial
  const int within = t - band * RB * nt;
  tn = within / rows;
  tm = band * RB + within % rows;
}

// Wave-specialised workgroup of 8 waves, two per SIMD:
//   waves 0-3 (consumers) run only the MFMAs of their 64 x 128 output slice;
//   waves 4-7 (producers) copy activations for consumer (wave - 4) into its
//   LDS ring, load codes and decode the next W tile.
// The SIMD co-issues a producer's VALU work with its consumer's MFMAs, so the
// decode runs in the matrix core's shadow without hand interleaving.  One
// barrier per 64-deep step hands tile s + 1 (and activation stage s + 1) from
// producers to consumers.
//
// Producer pipeline at step s: load codes of step s + 2 (2-slot register
// ring), copy activations of step s + 2 (3-stage LDS ring), decode codes of
// step s + 1 into W buffer (s + 1) % 2, then wait for the copies of step s + 1.
template <bool NN, typename E>
__global__ __launch_bounds__(2 * kThreads) void k_gemm_nf4(GemmArgs a) {
  // Two distinct LDS objects: the compiler can then tell that the producers'
  // stores of decoded W tiles never alias the activation copies in flight
  // (otherwise it drains every copy before each such store).
  __shared__ __attribute__((aligned(16))) uint16_t s_w[2 * Tile<NN>::kElems];
  __shared__ __attribute__((aligned(16))) uint8_t s_act[4 * kActStages * kActStage];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool producer = wave >= 4;
  const int slice = wave & 3;               // consumer slice this wave works on / feeds
  const int ptid = tid & (kThreads - 1);    // producer thread index 0..255
  int tm, tn;
  tile_coords(tm, tn);
  const int m0 = tm * BM, c0 = tn * BN;
  const int row0 = m0 + 64 * slice;
  uint16_t* const w_buf0 = s_w;
  uint16_t* const w_buf1 = s_w + Tile<NN>::kElems;
  auto act_lds = [&](int st) {
    return (lds_u8*)s_act + ((uint32_t)slice * kActStages + st) * kActStage;
  };
  auto act_ptr = [&](int st) {
    return reinterpret_cast<uint16_t*>(s_act + ((uint32_t)slice * kActStages + st) * kActStage);
  };

  const int nsteps = (a.R + 63) / 64;
  // Split reduction: this workgroup takes steps [s0, s0 + nloc) of the
  // nsteps; every split loops over the same even step count nst (an all-zero
  // step adds nothing).
  const int kz = blockIdx.z;
  const int spl = a.ksplit > 1 ? (nsteps + a.ksplit - 1) / a.ksplit : nsteps;
  const int s0 = kz * spl;
  const int nloc = max(0, min(spl, nsteps - s0));
  const int nst = (spl + 1) & ~1;
  const int kend = ((nsteps + 1) & ~1) * 64;  // >= R: loads there read zeros
  // All tiles walk the reduction in the same order, so the workgroups of
  // one XCD read the same activation / weight slices at about the same time
  // and share them in L2.
  auto kofs = [&](int step) {  // reduction offset of logical step; >= R past the end
    return step < nloc ? (s0 + step) * 64 : kend;
  };
  auto stage_of = [](int step) { return step % kActStages; };

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // ---- adapter step: r extra reduction columns j = 16 ks + 8 h + e --------
  // (sw: a W buffer, sa: this slice's activation stage, both free)
  auto adapter_step = [&](uint16_t* sw, uint16_t* sa) {
    __syncthreads();
    if (producer) {
      const Srcs src = make_srcs<NN>(a);
      // All loads of the fill are issued before any LDS store (16-byte
      // chunks of 8 ranks; out of range reads zero), so the fill costs one
      // memory latency, not one per element.
      const bool vec = (a.r & 7) == 0;
      // W-side operand: NT: B[n][j] -> sw[col][j]; NN: A[j][c] -> sw[j][col]
      uint4 wv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int idx = ptid + u * kThreads;  // 0 .. 1023 chunk slots
        if (!NN) {
          const int col = idx >> 3, jc = idx & 7, n = c0 + col;
          wv[u] = load_e16x8(src.lora_w, (uint32_t)n * (uint32_t)a.r + 8u * jc, n < a.C, a.r - 8 * jc, vec);
        } else {
          const int j = idx >> 4, cc = idx & 15, c = c0 + 8 * cc;
          wv[u] = load_e16x8(src.lora_w, (uint32_t)j * (uint32_t)a.K + (uint32_t)c, j < a.r && c < a.C, 8, true);
        }
      }
      // token-side operand: U~ / V~ rows of this producer's consumer slice
      uint4 av[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int idx = lane + 64 * u;  // 0 .. 511: row idx >> 3, chunk idx & 7
        const int rr = idx >> 3, jc = idx & 7, m = row0 + rr;
        av[u] = load_e16x8(src.lora_act, (uint32_t)m * (uint32_t)a.r + 8u * jc, m < a.M, a.r - 8 * jc, vec);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int idx = ptid + u * kThreads;
        if (!NN) {
          const int col = idx >> 3, jc = idx & 7;
          *reinterpret_cast<uint4*>(sw + kt_off(col, jc)) = wv[u];
        } else {
          const int j = idx >> 4, cc = idx & 15;
          *reinterpret_cast<uint4*>(sw + nn_off(j, 8 * cc)) = wv[u];
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t idx = lane + 64u * u, rr = idx >> 3, jc = idx & 7;
        *reinterpret_cast<uint4*>(sa + rr * 64u + ((jc ^ swz(rr)) << 3)) = av[u];
      }
    }
    __syncthreads();
    if (!producer) {
      const CodeSeg none{};
      const float th0[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      const LaneMask lm0{0, 0, 0};
      mma_step<NN, false, E>(acc, sa, sw, sw, none, th0, lm0, 0, lane);
    }
  };

  // ---- dX with LoRA dropout: the adapter's part of dX passes through the
  // dropout mask of the adapter input, mask * (V~ A).  The adapter step then
  // runs first, alone in the accumulators, which are masked before the main
  // reduction adds dY Wbf.  The producer of each slice draws the slice's
  // 64 x 128 keep bytes into activation stage 1 meanwhile.
  const bool drop_first = NN && a.drop.thr != 0 && a.r > 0 && kz == 0;
  if (drop_first) {
    adapter_step(w_buf0, act_ptr(0));
    uint8_t* keep = reinterpret_cast<uint8_t*>(act_ptr(1));
    if (producer) {
#pragma unroll 4
      for (int t = 0; t < 32; ++t) {  // (row, 4-column group) pairs q = lane + 64 t
        const int q = lane + 64 * t, rl = q >> 5, g = q & 31;
        const uint64_t e = (uint64_t)(row0 + rl) * (uint64_t)a.C + (uint64_t)(c0 + 4 * g);
        const uint64_t ctr = e >> 2;
        const uint4 u = philox4x32_10(make_uint4((uint32_t)ctr, (uint32_t)(ctr >> 32), 0u, 0u), a.drop.k0, a.drop.k1);
        const uint32_t kb = (u.x >= a.drop.thr ? 1u : 0u) | (u.y >= a.drop.thr ? 1u << 8 : 0u) |
                            (u.z >= a.drop.thr ? 1u << 16 : 0u) | (u.w >= a.drop.thr ? 1u << 24 : 0u);
        *reinterpret_cast<uint32_t*>(keep + 4 * q) = kb;  // byte rl * 128 + 4 g + i
      }
    }
    __syncthreads();
    if (!producer) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int rl = 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3), cl = 32 * j + (lane & 31);
            if (!keep[rl * 128 + cl]) acc[i][j][v] = 0.f;
          }
    }
    __syncthreads();  // stages 0 / 1 and W buffer 0 are refilled below
  }

  if (producer) {
    const bool odd = lane & 1;
    float th[8];
    lane_levels(a.nf4, odd, th);
    const LaneMask lm = lane_mask(odd);
    const Srcs src = make_srcs<NN>(a);
    const ActRows rows = act_rows(a, row0, lane);

    // Issue order inside a step: code loads first, then activation copies,
    // so that waiting for the codes of step s + 1 (decoded at step s) never
    // waits for the copies issued after them (vmcnt retires in order).
    CodeSeg c0s = load_codes<NN>(a, src, c0, kofs(0), ptid);
    copy_act(a, src, rows, act_lds(stage_of(0)), kofs(0), lane);
    CodeSeg c1s = load_codes<NN>(a, src, c0, kofs(1), ptid);
    copy_act(a, src, rows, act_lds(stage_of(1)), kofs(1), lane);
    decode_store<NN, E>(w_buf0, c0s, th, lm, ptid);
    // copies of step 0 done: younger are the codes (3) and copies (8) of step 1
    wait_vmcnt<11>();
    __syncthreads();

    auto body = [&](int step, CodeSeg& load_slot, const CodeSeg& dec, uint16_t* w_next) {
      load_slot = load_codes<NN>(a, src, c0, kofs(step + 2), ptid);
      __builtin_amdgcn_sched_barrier(0);  // keep all code loads ahead of the copies
      copy_act(a, src, rows, act_lds(stage_of(step + 2)), kofs(step + 2), lane);
      decode_store<NN, E>(w_next, dec, th, lm, ptid);
      // copies of step s + 1 done: younger are the codes (3) and copies (8)
      // of step s + 2
      wait_vmcnt<11>();
      step_barrier();
    };
    for (int step = 0; step < nst; step += 2) {
      body(step, c0s, c1s, w_buf1);
      body(step + 1, c1s, c0s, w_buf0);
    }
    wait_vmcnt<0>();  // nothing left in flight into the activation ring
  } else {
    __syncthreads();  // tile 0 and activations of step 0 are ready
    const CodeSeg none{};
    const float th0[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    const LaneMask lm0{0, 0, 0};
    for (int step = 0; step < nst; step += 2) {
      mma_step<NN, false, E>(acc, act_ptr(stage_of(step)), w_buf0, w_buf1, none, th0, lm0, 0, lane);
      step_barrier();
      mma_step<NN, false, E>(acc, act_ptr(stage_of(step + 1)), w_buf1, w_buf0, none, th0, lm0, 0, lane);
      step_barrier();
    }
  }

  // ---- adapter step at the end (no dropout): W buffer 0 and activation
  // stage nst % 3 are no longer read
  if (a.r > 0 && !drop_first && kz == 0) adapter_step(w_buf0, act_ptr(stage_of(nst)));

  // ---- split reduction: this split's fp32 tile, added up by a second pass
  if (a.part) {
    if (!producer) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = c0 + 32 * j + (lane & 31);
          if (col >= a.C) continue;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int row = row0 + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            if (row < a.M) a.part[((int64_t)kz * a.M + row) * a.C + col] = acc[i][j][v];
          }
        }
    }
    return;
  }

  // ---- epilogue: fp32 -> bf16 (round to nearest even) ---------------------
  if (!producer) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = c0 + 32 * j + (lane & 31);
        if (col >= a.C) continue;
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          const int row = row0 + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          const uint32_t pk = E::pack2(acc[i][j][v], acc[i][j][v + 1]);
          if (row < a.M) a.out[(int64_t)row * a.ld_out + col] = (uint16_t)(pk & 0xFFFFu);
          if (row + 1 < a.M) a.out[(int64_t)(row + 1) * a.ld_out + col] = (uint16_t)(pk >> 16);
        }
      }
  }
}

// out[m][c] = E(sum over z of part[z][m][c]), z in order; 8 columns per
// thread (C % 8 == 0, rows of out 16-byte aligned).
template <typename E>
__global__ __launch_bounds__(256) void k_splitk_reduce(const float* __restrict__ part, int ksplit, int M, int C,
                                                       uint16_t* __restrict__ out, int64_t ld_out) {
  const int c8 = C >> 3;
  const int64_t n = (int64_t)M * c8;
  const int64_t zs = (int64_t)M * C;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int m = (int)(i / c8), c = (int)(i - (int64_t)m * c8) * 8;
    const float4* p = reinterpret_cast<const float4*>(part + (int64_t)m * C + c);
    float4 lo = p[0], hi = p[1];
    for (int z = 1; z < ksplit; ++z) {
      const float4* q = reinterpret_cast<const float4*>(part + z * zs + (int64_t)m * C + c);
      const float4 a = q[0], b = q[1];
      lo.x += a.x; lo.y += a.y; lo.z += a.z; lo.w += a.w;
      hi.x += b.x; hi.y += b.y; hi.z += b.z; hi.w += b.w;
    }
    *reinterpret_cast<uint4*>(out + (int64_t)m * ld_out + c) =
        make_uint4(E::pack2(lo.x, lo.y), E::pack2(lo.z, lo.w), E::pack2(hi.x, hi.y), E::pack2(hi.z, hi.w));
  }
}

thread_local hipEvent_t t_ev_start = nullptr, t_ev_stop = nullptr;

template <bool NN>
hipError_t launch(GemmArgs a, hipStream_t st) {
  auto kern = a.f16 ? k_gemm_nf4<NN, F16> : k_gemm_nf4<NN, Bf16>;
  hipError_t e;
  hipEvent_t ev0, ev1;
  take_gemm_events(ev0, ev1);
  if (ev0 && (e = hipEventRecord(ev0, st)) != hipSuccess) return e;
  a.ksplit = a.part ? gemm_ksplit(a.M, a.C, a.R, device_compute_units()) : 1;
  if (a.ksplit < 2) a.part = nullptr;
  dim3 grid((a.C + BN - 1) / BN, (a.M + BM - 1) / BM, a.ksplit);
  hipLaunchKernelGGL(kern, grid, dim3(2 * kThreads), 0, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.part && (e = launch_splitk_reduce(a.part, a.ksplit, a.M, a.C, a.out, a.ld_out, a.f16, st)) != hipSuccess)
    return e;
  if (ev1 && (e = hipEventRecord(ev1, st)) != hipSuccess) return e;
  return hipSuccess;
}

}  // namespace

void take_gemm_events(hipEvent_t& start, hipEvent_t& stop) {
  start = t_ev_start;
  stop = t_ev_stop;
  t_ev_start = t_ev_stop = nullptr;
}

void time_next_gemm(hipEvent_t start, hipEvent_t stop) {
  if (start && stop) { t_ev_start = start; t_ev_stop = stop; }
  else { t_ev_start = t_ev_stop = nullptr; }
}

int gemm_ksplit(int64_t M, int64_t C, int64_t R, int cus) {
  const int64_t tiles = ((M + BM - 1) / BM) * ((C + BN - 1) / BN);
  const int64_t nsteps = (R + 63) / 64;
  if (cus <= 0 || tiles <= 0 || tiles * 2 > cus || C % 8 != 0) return 1;
  // at most 8 splits, a grid of at most one workgroup per compute unit, and
  // at least 8 steps (512 reduction columns) per split -- so no split is
  // empty: ceil(nsteps / ks) >= 8 >= ks
  const int64_t ks = std::min<int64_t>(std::min<int64_t>(8, cus / tiles), nsteps / 8);
  return ks > 1 ? (int)ks : 1;
}

size_t gemm_part_bytes(int64_t M, int64_t C, int64_t R, int cus) {
  const int ks = gemm_ksplit(M, C, R, cus);
  return ks > 1 ? (size_t)ks * (size_t)M * (size_t)C * 4u : 0;
}

// out = E(sum over z of part[z]) for an fp32 [ksplit][M][C] partial buffer
// (C % 8 == 0, out rows 16-byte aligned); also the second pass of the
// few-token kernel's reduction split.
hipError_t launch_splitk_reduce(const float* part, int ksplit, int M, int C, uint16_t* out, int64_t ld_out, bool f16,
                                hipStream_t st) {
  const int64_t n = (int64_t)M * (C / 8);
  const int blocks = (int)std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 2048));
  if (f16) hipLaunchKernelGGL(k_splitk_reduce<F16>, dim3(blocks), dim3(256), 0, st, part, ksplit, M, C, out, ld_out);
  else hipLaunchKernelGGL(k_splitk_reduce<Bf16>, dim3(blocks), dim3(256), 0, st, part, ksplit, M, C, out, ld_out);
  return hipGetLastError();
}

hipError_t launch_gemm_fwd(const GemmArgs& a, hipStream_t st) { return launch<false>(a, st); }
hipError_t launch_gemm_dx(const GemmArgs& a, hipStream_t st) { return launch<true>(a, st); }

}  // namespace qlora
