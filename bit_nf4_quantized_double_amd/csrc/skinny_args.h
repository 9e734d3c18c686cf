// Arguments of the few-token fused forward kernel (skinny.hip).
#pragma once

#include "common.h"

namespace qlora {

struct SkinnyArgs {
  const uint16_t* X;  // [M x K] tokens (16-bit elements, see f16)
  const uint8_t* codes;
  const uint8_t* q8;
  const float* s2;
  const uint16_t* U;  // [M x r] bf16 scaled adapter activation, or null (r == 0 or upart set)
  // U~ from the down projection's fp32 split partial sums instead of U (when
  // set): U~ = E(uscale * (upart[0] + upart[1] + ... + upart[uns - 1])),
  // each [M x r]; the partials are staged in LDS at the kernel's start.  The
  // workgroup of tile group 0 stores U~ to Uout when that is set.
  const float* upart;
  int uns;
  float uscale;
  uint16_t* Uout;
  int uoff;           // LDS byte offset of the staged partials; set by the launcher
  const uint16_t* B;  // [N x r] bf16, or null (r == 0)
  uint16_t* Y;        // [M x N] bf16, written
  int M, N, K, r;
  int tiles;          // W tiles per workgroup (= nwt * TPW); set by the launcher
  int nwk_log2;       // log2 of the waves sharing one tile group; set by the launcher
  int nci;            // chunk iterations per wave; set by the launcher
  int kchunks;        // 128-wide reduction chunks per workgroup row of the grid; set by the launcher
  float* part;        // fp32 [ksplit][M][N] partial sums when the reduction is split, else null
  Nf4Consts nf4;
  bool f16;           // X, U, B, Y and the decoded W are fp16 (else bf16)
};

int skinny_max_tokens();
// Reduction split across workgroups for these sizes on a device with `cus`
// compute units: ks splits of kchunks 128-wide chunks each (ks = 1:
// unsplit), every split non-empty: (ks - 1) * kchunks < chunks <= ks * kchunks.
struct SkinnySplit {
  int ks, kchunks;
};
SkinnySplit skinny_split(int64_t M, int64_t N, int64_t K, int cus);
// fp32 bytes the split's partial sums take (0 if unsplit)
size_t skinny_part_bytes(int64_t M, int64_t N, int64_t K, int cus);
// With upart set and the partials too large to stage, the launcher first
// rounds them into U (which must then be set) with a finalize pass.
hipError_t launch_skinny_fwd(SkinnyArgs a, hipStream_t st);

}  // namespace qlora
