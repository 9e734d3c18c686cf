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
// tile in LDS, where all four consumer waves read it as the MFMA B operand.
// The rank-r adapter term is one extra reduction step into the same
// accumulators.
//
// Workgroup tile 256 (rows) x 128 (columns), 4 consumer waves stacked along
// the rows; each owns 64 rows x 128 columns = 2 x 4 tiles of
// v_mfma_f32_32x32x16_bf16.  A wave's activation rows are private to it: it
// loads them from the fragment-tiled copy of X or dY (gemm_args.h), one
// coalesced 1 KB load per MFMA operand, into registers two steps ahead.  The
// decoded W tile is the only thing in LDS (a 4-deep ring; one barrier per two
// steps).
//
//   NT (forward): W tile = 128 rows n x 64 k, stored [n][k], read with
//                 ds_read_b128.
//   NN (dX):      W tile = 64 rows n x 128 columns c, stored [n][c] as
//                 decoded (each group of 8 columns in the order 0, 2, 4, 6,
//                 1, 3, 5, 7, which the epilogue undoes); the B operand
//                 needs 8 consecutive n per lane and gets them with gfx950's
//                 transposing ds_read_b64_tr_b16.
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
  __amdgpu_buffer_rsrc_t codes, q8, s2;
  __amdgpu_buffer_rsrc_t lora_act, lora_w;  // U~ or V~ [M x r]; B [C x r] (NT) or A [r x K] (NN)
};

template <bool NN>
__device__ __forceinline__ Srcs make_srcs(const GemmArgs& a) {
  Srcs s;
  // W is [n_out x k_in]: n_out = C (forward) or R (dX)
  const uint64_t wn = (uint64_t)a.K * (uint64_t)(NN ? a.R : a.C);
  const uint32_t nb = (uint32_t)(wn >> 6);
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

// The W-tile segment (row n of W, 32 weights from reduction offset k) that
// producer thread tid decodes.  NT: 128 rows x 64; lanes l and l ^ 16 of a
// producer wave hold the two halves of one 64-weight block (a 16-lane row
// swap exchanges their halves of the block's table).  NN: 64 rows x 128;
// threads tid and tid ^ 1 share a block (a quad swap exchanges them).
template <bool NN>
__device__ __forceinline__ void seg_of(int tid, int& row, int& half) {
  if (NN) {
    row = tid >> 2;
    half = tid & 3;  // 32-weight segment of the 128-wide row
  } else {
    const int w = tid >> 6, l = tid & 63;
    row = 32 * w + (l & 15) + 16 * (l >> 5);
    half = (l >> 4) & 1;
  }
}

template <bool NN>
__device__ __forceinline__ CodeSeg load_codes(const GemmArgs& a, const Srcs& src, int c0, int r0, int tid) {
  int row, half;
  seg_of<NN>(tid, row, half);
  int n, k;
  bool ok;
  if (NN) { n = r0 + row; k = c0 + half * 32; ok = n < a.R && k < a.C; }
  else    { n = c0 + row; k = r0 + half * 32; ok = n < a.C && k < a.R; }
  const uint32_t e = (uint32_t)n * (uint32_t)a.K + (uint32_t)k;  // weight index
  CodeSeg cs;  // out of range: all zero, which decodes to zeros
  cs.code = buf_load16(src.codes, ok ? (e >> 1) : kOOB);
  cs.q = buf_load1(src.q8, ok ? (e >> 6) : kOOB);
  cs.s2 = __builtin_bit_cast(float, buf_load4(src.s2, ok ? ((e >> 14) << 2) : kOOB));
  return cs;
}

// Per-lane decode constants: the half of the levels this lane's table share
// covers, and the lookup masks.
struct DecodeConsts {
  float th[8];
  EoConsts eo;
};

template <bool NN>
__device__ __forceinline__ DecodeConsts decode_consts(const Nf4Consts& nf4, int tid) {
  DecodeConsts dc;
  int row, half;
  seg_of<NN>(tid, row, half);
  const bool odd = NN ? (half & 1) : half;  // the lane building levels 8..15
  lane_levels(nf4, odd, dc.th);
  dc.eo = eo_consts(NN && odd);  // NN (kXor1 tables): that lane's own half is "a"
  return dc;
}

// Decode 32 weights and store them in the W tile with the element-order
// lookup (16 permutes + 7 operations per 8 codes), which leaves each group
// of 8 columns in the order 0, 2, 4, 6, 1, 3, 5, 7.  NT: those are reduction
// columns, and the tiled X copy the forward reads carries the same order, so
// the products pair up.  NN: they are output columns; the epilogue (and the
// adapter operand, and the dropout mask) use the same order (eo_col).
template <bool NN, typename E>
__device__ __forceinline__ void decode_store(uint16_t* s, const CodeSeg& cs, const DecodeConsts& dc, int tid) {
  int row, half;
  seg_of<NN>(tid, row, half);
  const float scale = (float)cs.q * cs.s2;  // a' = fp32(q8 * s2)
  if (NN) {
    const Lut L = build_lut<LutPartner::kXor1, E>(dc.th, scale);
    const int c = half * 32;
    *reinterpret_cast<uint4*>(s + nn_off(row, c + 0)) = decode8_lut_hl(L, cs.code.x, dc.eo);
    *reinterpret_cast<uint4*>(s + nn_off(row, c + 8)) = decode8_lut_hl(L, cs.code.y, dc.eo);
    *reinterpret_cast<uint4*>(s + nn_off(row, c + 16)) = decode8_lut_hl(L, cs.code.z, dc.eo);
    *reinterpret_cast<uint4*>(s + nn_off(row, c + 24)) = decode8_lut_hl(L, cs.code.w, dc.eo);
  } else {
    const Lut L = build_lut<LutPartner::kRows16, E>(dc.th, scale);
    const int c = half * 4;
    *reinterpret_cast<uint4*>(s + kt_off(row, c + 0)) = decode8_lut_hl(L, cs.code.x, dc.eo);
    *reinterpret_cast<uint4*>(s + kt_off(row, c + 1)) = decode8_lut_hl(L, cs.code.y, dc.eo);
    *reinterpret_cast<uint4*>(s + kt_off(row, c + 2)) = decode8_lut_hl(L, cs.code.z, dc.eo);
    *reinterpret_cast<uint4*>(s + kt_off(row, c + 3)) = decode8_lut_hl(L, cs.code.w, dc.eo);
  }
}

// Output column held at NN tile column p (group of 8 in the decode's element
// order 0, 2, 4, 6, 1, 3, 5, 7).
__device__ __forceinline__ int eo_col(int p) { return (p & ~7) | ((p & 3) << 1) | ((p >> 2) & 1); }

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

// ---- A operand: fragments of the tiled activation copy ---------------------
// A wave's 64 rows are two 32-row fragment blocks; a 64-deep step of them is
// 2 x 4 fragments, each one coalesced 16-byte-per-lane load into the
// registers the MFMA reads.  Rows past M (whole blocks past the copy) and
// steps past the reduction read zeros.
struct AFrags {
  uint4 f[4][2];  // [sub-step ks][row half i]
};

// B operands of one 16-deep sub-step from the W tile in LDS.
template <bool NN>
__device__ __forceinline__ void read_b(const uint16_t* sw, int ks, int lane, uint4 (&b)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) b[j] = load_bfrag<NN>(sw, 32 * j, ks, lane);
}

// s_waitcnt with only a vmcnt limit (gfx9 encoding: vmcnt in bits 3:0 and
// 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their "no wait" maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Hand-off barrier of the main loop: each wave first waits for its own LDS
// operations only (lgkmcnt(0): decoded-tile stores, operand reads), not for
// the global loads it has in flight for later steps (a plain
// __syncthreads() would drain those too).
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

// Steps per barrier phase and the W ring: producers decode the two steps of
// phase p + 1 while consumers multiply those of phase p.
constexpr int kPhase = 2;
constexpr int kWBufs = 2 * kPhase;
// Output staging of the epilogue: each consumer wave's 64 x 128 tile, rows
// padded to 136 elements so the two rows one 16-bit store instruction
// touches fall in different LDS banks.
constexpr int kOutPitch = BN + 8;
constexpr int kOutElems = 4 * 64 * kOutPitch;

template <bool NN>
struct Lds {
  static constexpr int kRing = kWBufs * Tile<NN>::kElems;
  static constexpr int kMain = kRing > kOutElems ? kRing : kOutElems;  // ring, then output staging
  static constexpr int kAdapter = Tile<NN>::kElems;                    // adapter W-side operand
};

// A-operand fragments in flight: NT two steps ahead; NN one (its transposing
// B reads need more registers, and two steps would spill).
template <bool NN>
struct ARing {
  static constexpr int kSteps = NN ? 1 : 2;
};

// The adapter's token-side operand from the row pass's fp32 partial sums
// (gemm_args.h): element (m, j) = E(scale * sum over z, in order, of
// part[z][m][j]), rows past M and ranks past r zero, for the lane's rows
// row0 + 32 i + (lane & 31) and ranks 16 ks + 8 (lane >> 5) .. + 7.  `store`:
// also write those elements to lora_out [M x r].
template <typename E>
__device__ __forceinline__ void adapter_from_partials(const GemmArgs& a, int row0, int lane, int nks, bool store,
                                                      uint4 (&uf)[4][2]) {
  // one buffer resource per split over this wave's 64 rows (rows past M
  // read zeros); the loads of 4 splits are in flight together.  row0 is
  // uniform across the wave: say so, or the resource needs a waterfall loop.
  const int urow0 = __builtin_amdgcn_readfirstlane(row0);
  const uint32_t rbytes = (uint32_t)a.lora_rp * 4u;
  const uint32_t pbytes = __builtin_amdgcn_readfirstlane((uint32_t)max(0, min(64, a.M - urow0)) * rbytes);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int j = 16 * ks + 8 * (lane >> 5);
    const bool ok = ks < nks && j < a.r;
    float s[2][8];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) s[i][e] = 0.f;
    if (ks < nks) {
      for (int z0 = 0; z0 < a.lora_ns; z0 += 4) {
        uint4 v[4][2][2];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int z = min(z0 + q, a.lora_ns - 1);
          const __amdgpu_buffer_rsrc_t rs =
              make_rsrc(a.lora_part + ((size_t)z * (size_t)a.M + (size_t)urow0) * (size_t)a.lora_rp,
                        pbytes);
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const uint32_t off = (uint32_t)(32 * i + (lane & 31)) * rbytes + 4u * (uint32_t)j;
            v[q][i][0] = buf_load16(rs, ok ? off : kOOB);
            v[q][i][1] = buf_load16(rs, ok ? off + 16u : kOOB);
          }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (z0 + q >= a.lora_ns) break;
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              s[i][4 * h + 0] += __builtin_bit_cast(float, v[q][i][h].x);
              s[i][4 * h + 1] += __builtin_bit_cast(float, v[q][i][h].y);
              s[i][4 * h + 2] += __builtin_bit_cast(float, v[q][i][h].z);
              s[i][4 * h + 3] += __builtin_bit_cast(float, v[q][i][h].w);
            }
        }
      }
    }
    const float c = a.lora_scale;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int m = row0 + 32 * i + (lane & 31);
      uf[ks][i] = ok ? make_uint4(E::pack2(c * s[i][0], c * s[i][1]), E::pack2(c * s[i][2], c * s[i][3]),
                                  E::pack2(c * s[i][4], c * s[i][5]), E::pack2(c * s[i][6], c * s[i][7]))
                     : make_uint4(0, 0, 0, 0);
      if (store && ok && m < a.M && a.lora_out) {
        uint16_t* o = a.lora_out + (size_t)m * (size_t)a.r + j;
        const int64_t oi = (int64_t)m * a.r + j, on = (int64_t)a.M * a.r;
        if ((a.r & 7) == 0) {
          if (in_bounds(oi, 8, on)) *reinterpret_cast<uint4*>(o) = uf[ks][i];
        } else {
          const uint32_t w[4] = {uf[ks][i].x, uf[ks][i].y, uf[ks][i].z, uf[ks][i].w};
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (j + e < a.r && in_bounds(oi + e, 1, on)) o[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
        }
      }
    }
  }
}

// Wave-specialised workgroup of 8 waves, two per SIMD:
//   waves 0-3 (consumers) run the MFMAs of their 64 x 128 output slice; they
//   load their activation fragments themselves from the tiled copy (one or
//   two steps ahead, in registers) and read the shared decoded W tile from
//   LDS;
//   waves 4-7 (producers) load codes (four steps ahead) and decode W tiles
//   into a 4-deep LDS ring.
// The SIMD co-issues a producer's VALU decode with its consumer's MFMAs.  The
// LDS carries only the decoded weight: 16 KB written and 64 KB read per
// 64-deep step, against 48 KB and 96 KB when the activations were staged
// there too -- LDS writes run at about 64 B per clock per CU on this GPU and
// were the bottleneck.  One barrier per two steps.  The adapter term goes
// first, from its own LDS region filled during the prologue, so its loads
// overlap the first decode; the output leaves through LDS as coalesced
// 16-byte stores.
template <bool NN, typename E>
__global__ __launch_bounds__(2 * kThreads) void k_gemm_nf4(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t s_w[Lds<NN>::kMain];
  __shared__ __attribute__((aligned(16))) uint16_t s_ad[Lds<NN>::kAdapter];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool producer = wave >= 4;
  const int slice = wave & 3;               // consumer slice this wave works on / feeds
  const int ptid = tid & (kThreads - 1);    // producer thread index 0..255
  int tm, tn;
  tile_coords(tm, tn);
  const int m0 = tm * BM, c0 = tn * BN;
  const int row0 = m0 + 64 * slice;
  auto wbuf = [&](int step) { return s_w + (step & (kWBufs - 1)) * Tile<NN>::kElems; };

  const int nsteps = (a.R + 63) / 64;
  // Split reduction: this workgroup takes steps [s0, s0 + nloc) of the
  // nsteps; every split loops over the same step count nst, a multiple of 2
  // phases (all-zero steps add nothing).
  const int kz = blockIdx.z;
  const int spl = a.ksplit > 1 ? (nsteps + a.ksplit - 1) / a.ksplit : nsteps;
  const int s0 = kz * spl;
  const int nloc = max(0, min(spl, nsteps - s0));
  const int nst = (spl + 2 * kPhase - 1) & ~(2 * kPhase - 1);
  const int kend = ((nsteps + 1) & ~1) * 64;  // >= R: code loads there read zeros
  // All tiles walk the reduction in the same order, so the workgroups of
  // one XCD read the same activation / weight slices at about the same time
  // and share them in L2.
  auto kofs = [&](int step) {  // reduction offset of logical step; >= R past the end
    return step < nloc ? (s0 + step) * 64 : kend;
  };
  // The adapter term (split 0 only): r extra reduction columns
  // j = 16 ks + 8 h + e.  With LoRA dropout on dX it is masked before the
  // main reduction adds dY Wbf (mask * (V~ A)).
  const bool adapter = a.r > 0 && kz == 0;
  const bool drop_first = NN && a.drop.thr != 0 && adapter;

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const Srcs src = make_srcs<NN>(a);
  const bool vec = (a.r & 7) == 0;

  if (producer) {
    const DecodeConsts dc = decode_consts<NN>(a.nf4, ptid);
    // codes of step s in slot s % 4, loaded four steps before their decode;
    // each slot is 3 loads, so before decoding step s the loads of steps
    // s + 1 .. s + 3 may still be in flight (vmcnt <= 9)
    CodeSeg cr[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) cr[u] = load_codes<NN>(a, src, c0, kofs(u), ptid);
    if (adapter) {
      // the adapter's W-side operand into its region (NT: B[n][j] ->
      // s_ad[col][j]; NN: A[j][c] -> s_ad[j][col]); loads in flight together
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
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int idx = ptid + u * kThreads;
        if (!NN) *reinterpret_cast<uint4*>(s_ad + kt_off(idx >> 3, idx & 7)) = wv[u];
        else *reinterpret_cast<uint4*>(s_ad + nn_off(idx >> 4, 8 * (idx & 15))) = x_order_even_odd(wv[u]);
      }
    }
    if (drop_first) {
      // keep bytes of the consumer slice this producer feeds, 64 x 128, into
      // W buffers 2-3 (not decoded into before the mask is applied)
      uint8_t* keep = reinterpret_cast<uint8_t*>(wbuf(2)) + slice * (64 * BN);
      const int plane = tid & 63;
#pragma unroll 4
      for (int t = 0; t < 32; ++t) {  // (row, 4-column group) pairs q = lane + 64 t
        const int q = plane + 64 * t, rl = q >> 5, g = q & 31;
        const uint64_t e = (uint64_t)(row0 + rl) * (uint64_t)a.C + (uint64_t)(c0 + 4 * g);
        const uint64_t ctr = e >> 2;
        const uint4 u = philox4x32_10(make_uint4((uint32_t)ctr, (uint32_t)(ctr >> 32), 0u, 0u), a.drop.k0, a.drop.k1);
        const uint32_t kb = (u.x >= a.drop.thr ? 1u : 0u) | (u.y >= a.drop.thr ? 1u << 8 : 0u) |
                            (u.z >= a.drop.thr ? 1u << 16 : 0u) | (u.w >= a.drop.thr ? 1u << 24 : 0u);
        *reinterpret_cast<uint32_t*>(keep + 4 * q) = kb;  // byte rl * 128 + 4 g + i
      }
    }
    auto dec = [&](int step, CodeSeg& slot) {
      wait_vmcnt<9>();
      decode_store<NN, E>(wbuf(step), slot, dc, ptid);
      __builtin_amdgcn_sched_barrier(0);
      slot = load_codes<NN>(a, src, c0, kofs(step + 4), ptid);
    };
    dec(0, cr[0]);
    dec(1, cr[1]);
    step_barrier();  // steps 0 and 1 decoded; adapter operand (and keep bytes) staged
    if (drop_first) step_barrier();  // consumers applied the mask: W buffers 2-3 free
    for (int step = 0; step < nst; step += 2 * kPhase) {
      // phase of steps (step, step + 1): decode steps + 2, + 3
      if (step + 2 < nst) { dec(step + 2, cr[2]); dec(step + 3, cr[3]); }
      step_barrier();
      // phase of steps (step + 2, step + 3): decode steps + 4, + 5
      if (step + 4 < nst) { dec(step + 4, cr[0]); dec(step + 5, cr[1]); }
      step_barrier();
    }
    wait_vmcnt<0>();
  } else {
    constexpr int DA = ARing<NN>::kSteps;
    const int mbp = tiled_mbp(a.M);
    const __amdgpu_buffer_rsrc_t ract = make_rsrc(a.act_t, (uint32_t)tiled_bytes(a.M, a.R));
    // byte offsets of this lane in the two fragment blocks of the wave's rows
    const int mb0 = row0 >> 5;
    uint32_t abase[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
      abase[i] = mb0 + i < mbp ? (uint32_t)(mb0 + i) * (uint32_t)a.kbp * 1024u + 16u * (uint32_t)lane : kOOB;
    auto load_a = [&](int step, int ks, uint4 (&dst)[2]) {
      const bool ok = step < nloc;
      const uint32_t kb = 4u * (uint32_t)(s0 + step) + (uint32_t)ks;
#pragma unroll
      for (int i = 0; i < 2; ++i) dst[i] = buf_load16(ract, ok && abase[i] != kOOB ? abase[i] + kb * 1024u : kOOB);
    };
    AFrags ar[DA];  // A fragments of steps s .. s + DA - 1 (step s in ar[s % DA])
    // step 0's fragments first, so that their loads and the adapter
    // operand's are in flight together
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) load_a(0, ks, ar[0].f[ks]);
    // The adapter's token-side operand (U~ or V~) in MFMA A-operand layout,
    // formed before the later steps' activation loads are issued (fewer live
    // registers).
    const int nks = (a.r + 15) >> 4;  // 16-rank sub-steps that hold ranks
    uint4 uf[4][2];
    if (adapter) {
      if (a.lora_part) {
        adapter_from_partials<E>(a, row0, lane, nks, tn == 0, uf);
      } else {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const int m = row0 + 32 * i + (lane & 31), j = 16 * ks + 8 * (lane >> 5);
            uf[ks][i] = ks < nks ? load_e16x8(src.lora_act, (uint32_t)m * (uint32_t)a.r + (uint32_t)j, m < a.M,
                                              a.r - j, vec)
                                 : make_uint4(0, 0, 0, 0);
          }
      }
    }
#pragma unroll
    for (int d = 1; d < DA; ++d)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) load_a(d, ks, ar[d].f[ks]);

    if (adapter) {
      step_barrier();  // adapter operand staged; steps 0 and 1 decoded
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        if (ks >= nks) break;  // uniform; the loop stays unrolled (static register indices)
        uint4 bf[4];
        read_b<NN>(s_ad, ks, lane, bf);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = E::mfma32(E::vec(uf[ks][i]), E::vec(bf[j]), acc[i][j]);
      }
      if (drop_first) {
        const uint8_t* keep = reinterpret_cast<const uint8_t*>(wbuf(2)) + slice * (64 * BN);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int rl = 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3), cl = 32 * j + (lane & 31);
              if (!keep[rl * 128 + eo_col(cl)]) acc[i][j][v] = 0.f;
            }
        step_barrier();  // mask read: producers may decode into W buffers 2-3
      }
    } else {
      step_barrier();  // steps 0 and 1 decoded
    }

    uint4 bc[4], bn[4];
    // One step of MFMAs from A registers and the W buffer of `step`; the B
    // operands of the next sub-step are read while these MFMAs run, and each
    // sub-step's A fragments are replaced by those of step + DA once used.
    // `last`: the final step of a phase, whose successor's W buffer is only
    // ready after the barrier (read there).
    auto cstep = [&](int step, AFrags& af, bool last) {
      const uint16_t* sw = wbuf(step);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        if (ks < 3) read_b<NN>(sw, ks + 1, lane, bn);
        else if (!last) read_b<NN>(wbuf(step + 1), 0, lane, bn);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = E::mfma32(E::vec(af.f[ks][i]), E::vec(bc[j]), acc[i][j]);
        load_a(step + DA, ks, af.f[ks]);
        // interleave: one MFMA, then one (NT) or two (NN) operand reads, ...
        // the two fragment loads after the fifth and sixth MFMA
        constexpr int kDs = NN ? 2 : 1;
        const bool reads = ks < 3 || !last;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);            // MFMA
          if (reads) __builtin_amdgcn_sched_group_barrier(0x100, kDs, 0);  // DS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 4; ++j) bc[j] = bn[j];
      }
    };
    read_b<NN>(wbuf(0), 0, lane, bc);
    for (int step = 0; step < nst; step += 2 * kPhase) {
      cstep(step, ar[0], false);
      cstep(step + 1, ar[DA - 1], true);
      step_barrier();
      read_b<NN>(wbuf(step + 2), 0, lane, bc);
      cstep(step + 2, ar[0], false);
      cstep(step + 3, ar[DA - 1], true);
      step_barrier();
      if (step + 4 < nst) read_b<NN>(wbuf(step + 4), 0, lane, bc);
    }
  }

  // ---- split reduction: this split's fp32 tile, added up by a second pass
  if (a.part) {
    if (!producer) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int cl = 32 * j + (lane & 31);
          const int col = c0 + (NN ? eo_col(cl) : cl);
          if (col >= a.C) continue;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int row = row0 + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            const int64_t pi = ((int64_t)kz * a.M + row) * a.C + col;
            // non-temporal: the split tiles go out to memory while the
            // kernel runs (512 tokens on the 7B layer: 2 % faster step)
            if (row < a.M && in_bounds(pi, 1, (int64_t)a.ksplit * a.M * a.C))
              __builtin_nontemporal_store(acc[i][j][v], a.part + pi);
          }
        }
    }
    return;
  }

  // ---- epilogue: fp32 -> bf16 (round to nearest even), through LDS -------
  // The ring is free (every wave passed the last barrier).  Each consumer
  // stages its 64 x 128 tile in rows of its own LDS region, then reads it
  // back 16 bytes per lane: every global store instruction writes 4 rows of
  // 256 contiguous bytes instead of 2-byte pieces.  The stores are
  // non-temporal (the output is not read again here): about 1 us less per
  // launch than plain stores on the 7B shapes.
  if (!producer) {
    typedef __attribute__((ext_vector_type(4))) unsigned v4u;
    uint16_t* so = s_w + slice * (64 * kOutPitch);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = NN ? eo_col(32 * j + (lane & 31)) : 32 * j + (lane & 31);
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          const int rl = 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          const uint32_t pk = E::pack2(acc[i][j][v], acc[i][j][v + 1]);
          so[rl * kOutPitch + col] = (uint16_t)(pk & 0xFFFFu);
          so[(rl + 1) * kOutPitch + col] = (uint16_t)(pk >> 16);
        }
      }
    // LDS operations of one wave complete in order: the reads see the writes
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int rl = 4 * t + (lane >> 4), cl = 8 * (lane & 15);
      const uint4 v = *reinterpret_cast<const uint4*>(so + rl * kOutPitch + cl);
      const int row = row0 + rl, col = c0 + cl;
      if (row < a.M && col < a.C && in_bounds((int64_t)row * a.ld_out + col, 8, (int64_t)a.M * a.ld_out))
        __builtin_nontemporal_store(v4u{v.x, v.y, v.z, v.w}, reinterpret_cast<v4u*>(a.out + (int64_t)row * a.ld_out + col));
    }
  }
}

// Fragment-tiled copy of act[M][R] (see gemm_args.h): one thread per 16-byte
// piece, rows past M and columns past R written as zeros.
__global__ __launch_bounds__(256) void k_tile_act(const uint16_t* __restrict__ act, int M, int R, int kbp, bool eo,
                                                  uint16_t* __restrict__ act_t, int64_t npieces) {
  for (int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x; p < npieces; p += (int64_t)gridDim.x * 256) {
    // piece p: lane l = p & 63 of fragment f = p >> 6 = mb * kbp + kb
    const int l = (int)(p & 63);
    const int64_t f = p >> 6;
    const int mb = (int)(f / kbp), kb = (int)(f - (int64_t)mb * kbp);
    const int m = 32 * mb + (l & 31), k = 16 * kb + 8 * (l >> 5);
    uint4 v = make_uint4(0, 0, 0, 0);
    if (m < M && k < R && in_bounds((int64_t)m * R + k, 8, (int64_t)M * R))
      v = *reinterpret_cast<const uint4*>(act + (int64_t)m * R + k);
    if (in_bounds(p, 1, npieces)) reinterpret_cast<uint4*>(act_t)[p] = eo ? x_order_even_odd(v) : v;
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
    if (!in_bounds((int64_t)(ksplit - 1) * zs + (int64_t)m * C + c, 8, (int64_t)ksplit * zs)) continue;
    const float4* p = reinterpret_cast<const float4*>(part + (int64_t)m * C + c);
    float4 lo = p[0], hi = p[1];
    for (int z = 1; z < ksplit; ++z) {
      const float4* q = reinterpret_cast<const float4*>(part + z * zs + (int64_t)m * C + c);
      const float4 a = q[0], b = q[1];
      lo.x += a.x; lo.y += a.y; lo.z += a.z; lo.w += a.w;
      hi.x += b.x; hi.y += b.y; hi.z += b.z; hi.w += b.w;
    }
    if (in_bounds((int64_t)m * ld_out + c, 8, (int64_t)M * ld_out))
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

QLORA_OOB_READER(oob_count_gemm)

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

hipError_t launch_tile_act(const uint16_t* act, int M, int R, bool eo, uint16_t* act_t, hipStream_t st) {
  const int kbp = tiled_kbp(R);
  const int64_t npieces = (int64_t)tiled_mbp(M) * kbp * 64;
  if (npieces == 0) return hipSuccess;
  const int blocks = (int)std::max<int64_t>(1, std::min<int64_t>((npieces + 255) / 256, 4096));
  hipLaunchKernelGGL(k_tile_act, dim3(blocks), dim3(256), 0, st, act, M, R, kbp, eo, act_t, npieces);
  return hipGetLastError();
}

hipError_t launch_gemm_fwd(const GemmArgs& a, hipStream_t st) { return launch<false>(a, st); }
hipError_t launch_gemm_dx(const GemmArgs& a, hipStream_t st) { return launch<true>(a, st); }

}  // namespace qlora
