// Launch arguments of the fused NF4-dequant GEMMs (see gemm.hip).
#pragma once

#include "common.h"
#include "dropout.h"

namespace qlora {

struct GemmArgs {
  const uint16_t* act;       // X [M x R] (forward) or dY [M x R] (dX), row-major bf16
  int64_t ld_act;            // row pitch of act in elements (= R)
  int M;                     // rows (tokens)
  int R;                     // reduction length: k_in (forward) or n_out (dX)
  int C;                     // output columns: n_out (forward) or k_in (dX)
  const uint8_t* codes;      // packed NF4 codes of W [n_out x k_in]
  const uint8_t* q8;         // 8-bit block absmax codes
  const float* s2;           // fp32 step per group of 256 blocks
  int K;                     // W row length (k_in)
  const uint16_t* lora_act;  // U~ or V~ [M x r] bf16 (unused when r == 0)
  const uint16_t* lora_w;    // forward: B [n_out x r]; dX: A [r x k_in]
  int r;                     // adapter rank, 0..64
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

}  // namespace qlora
