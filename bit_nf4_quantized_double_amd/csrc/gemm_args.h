// Launch arguments of the fused NF4-dequant GEMMs (see gemm.hip), and the
// fragment-tiled activation layout they read.
#pragma once

#include "common.h"
#include "dropout.h"

namespace qlora {

// Fragment-tiled copy of an activation matrix act[M][R] (R: the reduction
// length of the product that reads it).  It is stored as 1 KB fragments of
// 32 rows x 16 reduction columns, in the A-operand layout of
// v_mfma_f32_32x32x16: fragment (mb, kb) starts at element
// (mb * kbp + kb) * 512 and its lane l (0..63) holds the 8 elements
// act[32 mb + (l & 31)][16 kb + 8 (l >> 5) + e], e = 0..7.  kbp = 4 ceil(R / 64)
// fragments per 32-row block (whole 64-deep steps), mbp = ceil(M / 32)
// blocks; rows past M and columns past R hold zeros.  The adapter kernels
// that read act anyway (U~ over X, V~ over dY) write it; a GEMM wave then
// loads each operand fragment with one coalesced 1 KB load, straight into
// registers.  The forward's copy of X permutes each lane's 8 elements to the
// order 0, 2, 4, 6, 1, 3, 5, 7 (e above runs over that order), the order in
// which the forward GEMM decodes W; the dX product's copy of dY keeps the
// natural order.
__host__ __device__ inline int tiled_kbp(int64_t R) { return (int)(4 * ((R + 63) / 64)); }
__host__ __device__ inline int tiled_mbp(int64_t M) { return (int)((M + 31) / 32); }
__host__ __device__ inline size_t tiled_bytes(int64_t M, int64_t R) { return (size_t)tiled_mbp(M) * (size_t)tiled_kbp(R) * 1024u; }

// Element offset in the tiled copy of act[m][k .. k + 7], k a multiple of 8.
__host__ __device__ inline uint32_t tiled_elem(int m, int k, int kbp) {
  return (uint32_t)(((m >> 5) * kbp + (k >> 4)) * 512 + ((m & 31) + 32 * ((k >> 3) & 1)) * 8);
}

struct GemmArgs {
  const uint16_t* act_t;     // fragment-tiled X (forward) or dY (dX), 16-bit elements
  int kbp;                   // fragments per 32-row block of act_t (tiled_kbp(R))
  int M;                     // rows (tokens)
  int R;                     // reduction length: k_in (forward) or n_out (dX)
  int C;                     // output columns: n_out (forward) or k_in (dX)
  const uint8_t* codes;      // packed NF4 codes of W [n_out x k_in]
  const uint8_t* q8;         // 8-bit block absmax codes
  const float* s2;           // fp32 step per group of 256 blocks
  int K;                     // W row length (k_in)
  const uint16_t* lora_act;  // U~ or V~ [M x r] bf16 (unused when r == 0 or lora_part is set)
  const uint16_t* lora_w;    // forward: B [n_out x r]; dX: A [r x k_in]
  int r;                     // adapter rank, 0..64
  // The adapter's token-side operand from row-pass partial sums instead of
  // lora_act (when lora_part is set): E(lora_scale * sum over z < lora_ns,
  // in order, of lora_part[z][m][j]), row pitch lora_rp (rank_pitch(r)),
  // formed in the prologue of the split-0 workgroups; those of column tile
  // 0 also store it to lora_out [M x r] when that is set.
  const float* lora_part;
  int lora_ns, lora_rp;
  float lora_scale;
  uint16_t* lora_out;
  uint16_t* out;             // Y [M x n_out] or dX [M x k_in], bf16
  int64_t ld_out;
  Nf4Consts nf4;
  DropMask drop;             // dX only: dropout of the adapter input (thr 0: none)
  bool f16;                  // element type of act, lora_*, out and the decoded W: fp16 (else bf16)
  // Split reduction (set by the launcher): workgroup z of the grid takes
  // reduction steps [z * spl, (z + 1) * spl) and stores its fp32 tile in
  // part[z][M][C]; a second pass adds the ksplit tiles in order and rounds.
  int ksplit;
  float* part;
};

// Reduction splits for a product of M x C outputs over R on a device with
// `cus` compute units: more than one only when the grid of 256 x 128 tiles
// would leave at least half of them idle.  The fp32 bytes the split needs
// (0 if unsplit).
int gemm_ksplit(int64_t M, int64_t C, int64_t R, int cus);
size_t gemm_part_bytes(int64_t M, int64_t C, int64_t R, int cus);

// out = E(sum over z of part[z]) for fp32 partial sums [ksplit][M][C], z in
// order (C % 8 == 0, rows of out 16-byte aligned).
hipError_t launch_splitk_reduce(const float* part, int ksplit, int M, int C, uint16_t* out, int64_t ld_out, bool f16,
                                hipStream_t st);

// ---- adapter passes (adapter.hip) -----------------------------------------
// Row pass over act [M x R]: nch 128-wide chunks of the reduction, S splits
// of cps chunks each (S <= 8), one partial sum per split.
struct RowpassPlan {
  int nch, cps, S;
};
RowpassPlan rowpass_plan(int64_t M, int64_t R, int cus);
int rank_pitch(int r);  // r rounded up to a multiple of 8
size_t rowpass_part_bytes(int64_t M, int64_t R, int r, int cus);

// One read of act [M x R] (R % 8 == 0) writes the fragment-tiled copy
// (when `tiled` is set) and the fp32 partial sums part[z][m][j] =
// sum over split z's columns k of act'[m][k] w(j, k), pitch rank_pitch(r).
// contig: w(j, k) = A[j][k] (A [r x R]; the forward's X A^T, act' = the
// dropout mask times X, the tiled copy in the forward's element order);
// else w(j, k) = B[k][j] (B [R x r]; dY B, natural order, no mask).
// mbits (with mdrop.thr != 0): the pass also writes the keep mask mdrop of
// an [M x mK] adapter input as bits, word w of row m = elements 32 w ..
// 32 w + 31 (mK % 32 == 0; M * mK / 8 bytes), for the column pass.
hipError_t launch_rowpass(const uint16_t* act, int M, int R, const uint16_t* w, int r, bool contig, DropMask drop,
                          float* part, uint16_t* tiled, bool f16, int cus, hipStream_t st, uint32_t* mbits = nullptr,
                          int mK = 0, DropMask mdrop = DropMask{});

// U = E(scale * sum over z, in order, of part[z][m][j]) [M x r]: the U~ the
// forward GEMM forms from the same partials, bit for bit.
hipError_t launch_rowpass_finalize(const float* part, int S, int M, int r, float scale, uint16_t* U, bool f16,
                                   hipStream_t st);

// Column pass over all M tokens, one dispatch, fixed summation order:
// dA = V~^T (mask * X) [r x K] and dB = dY^T U~ stored [N x r], fp32.  The
// mask comes from mbits (the row pass's bits) when set, else from drop.
hipError_t launch_colpass(const uint16_t* X, int K, const uint16_t* Vt, const uint16_t* dY, int N,
                          const uint16_t* Ut, int M, int r, DropMask drop, float* dA, float* dB, bool f16,
                          hipStream_t st, const uint32_t* mbits = nullptr);

// The fragment-tiled copy of act[M][R] (row pitch R elements, R % 8 == 0)
// alone, for products whose adapter kernels do not run (r == 0); eo: the
// forward's element order (see above).
hipError_t launch_tile_act(const uint16_t* act, int M, int R, bool eo, uint16_t* act_t, hipStream_t st);

}  // namespace qlora
