// Few-token fused forward of the QLoRA linear (M <= 16 token rows):
//     Y[m][n] = sum_k X[m][k] * Wbf[n][k] + sum_j U~[m][j] * B[n][j]
// ([P1] "The mechanism in brief": W x plus (alpha / r) B A x on a frozen
// 4-bit base; [P4] "The idea in one line": W is dequantized to bf16 only for
// the product that uses it).
//
// With a handful of tokens the layer is bound by reading the packed weight
// (0.516 B per weight), and decoding it is the only real arithmetic.  Every
// weight is decoded exactly once, from its codes straight into MFMA operand
// registers -- no LDS tile, no barrier in the main loop.  The product uses
// v_mfma_f32_16x16x32_bf16 (or _f16) with 16 W rows on one side and the (zero-padded)
// 16 tokens on the other.
//
// Workgroup: 8 waves (two per SIMD, so up to 256 VGPRs per lane for deep
// prefetch), or 16 (four per SIMD) when each wave holds 2 tiles of an unsplit
// reduction at fewer than 8 tokens; `tiles` 16-row W tiles (a tile = 16 output features),
// the whole reduction length.  Wave (a, b): tiles a*TPW .. a*TPW + TPW - 1
// of the group, 128-wide reduction chunks b, b + nwk, b + 2 nwk, ...
// Lane l: W row (l & 15) of a tile, reduction columns 32 (l >> 4) .. + 31 of
// a chunk -- one 16-byte code load, half of a 64-weight block; lane l ^ 16
// holds the other half and shares the block's lookup table.  The X fragment
// of a chunk is loaded once and reused by all TPW tiles of the wave.  At the
// end, the nwk partial tiles of each output tile are added in LDS in a fixed
// order (deterministic; with 16 waves after a pairwise fold); the b == 0 wave
// adds the adapter term first.
//
// The reduction index is permuted consistently in both operands (lane group
// g, dword i of a chunk <-> columns kc + 32 g + 8 i .. + 7, and inside each
// such group of 8 the order 0,2,4,6,1,3,5,7), which only changes the fp32
// summation order.
#include <algorithm>

#include "nf4_lut.h"
#include "skinny_args.h"

namespace qlora {

void take_gemm_events(hipEvent_t& start, hipEvent_t& stop);  // gemm.hip
hipError_t launch_splitk_reduce(const float* part, int ksplit, int M, int C, uint16_t* out, int64_t ld_out, bool f16,
                                hipStream_t st);  // gemm.hip
hipError_t launch_rowdot_finalize(const float* part, int nsplit, int M, int r, float s, uint16_t* U, bool f16,
                                  hipStream_t st);  // lora.hip

namespace {

// A workgroup has NW = 8 waves (two per SIMD, up to 256 VGPRs each), or 16
// (four per SIMD, up to 128 VGPRs: at most 2 W tiles per wave) where a wave
// has few tiles and a long reduction -- there more waves hide more load and
// MFMA latency than the larger tile groups save.
constexpr int kSkUpBytes = 32 * 1024;  // staged U~ partials
template <int NW>
struct SkGeom {
  static_assert(NW == 8 || NW == 16, "8 or 16 waves per workgroup");
  static constexpr int kThreads = 64 * NW;
  static constexpr int kStageLoads = 4096 / kThreads;  // 16-byte staged-scale loads per thread: sbytes <= 60 KB
  static constexpr int kUpLoads = kSkUpBytes / 16 / kThreads;  // 16-byte staged U~-partial loads per thread
  // The nwk partial tiles of an output tile meet in LDS after one pairwise
  // fold (wave b + nwk / 2 into wave b) with 16 waves, so the reduction
  // buffer stays at tiles * 8 / nwt KB <= 64 KB.
  static constexpr int kFold = NW > 8 ? 1 : 0;
};

struct SkSeg {
  uint4 code;  // 32 codes
  uint32_t q;  // block absmax code
  float s2;    // group scale
};

struct SkSrcs {
  __amdgpu_buffer_rsrc_t codes, q8, s2, X;
};

// SL: the workgroup's block scales (absmax codes of its rows, and the
// second-level scales they use) are staged in LDS once, with coalesced loads,
// instead of two scattered small loads per 32 weights.
template <int TPW, int RD, bool SL, typename E, int NW>
__global__ __launch_bounds__(64 * NW) void k_skinny_fwd(SkinnyArgs a) {
  using G = SkGeom<NW>;
  constexpr int kSkThreads = G::kThreads;
  constexpr int kSkMaxStageLoads = G::kStageLoads;
  constexpr int kSkUpLoads = G::kUpLoads;
  extern __shared__ __attribute__((aligned(16))) float4 s_dyn[];
  float4* const s_red = s_dyn;  // [tiles][nwk][64], used after the main loop
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nwk = 1 << a.nwk_log2;
  const int wa = wave >> a.nwk_log2, wb = wave & (nwk - 1);
  const int row = lane & 15, g = lane >> 4;
  const int nch = (a.K + 127) >> 7;
  // reduction split across workgroups: grid row kz takes chunks
  // [cbase, cbase + nchl) of the nch
  const int kz = blockIdx.y;
  const int cbase = kz * a.kchunks;
  const int nchl = min(a.kchunks, nch - cbase);

  const uint32_t nw = (uint32_t)a.N * (uint32_t)a.K;  // < 2^32 (checked on the host)
  SkSrcs src;
  src.codes = make_rsrc(a.codes, nw >> 1);
  src.q8 = make_rsrc(a.q8, nw >> 6);
  src.s2 = make_rsrc(a.s2, (((nw >> 6) + 255) >> 8) * 4);
  src.X = make_rsrc(a.X, (uint32_t)a.M * (uint32_t)a.K * 2u);

  // first W row of this lane in tile 0 of the wave; tile t adds 16 rows
  const int n0 = (blockIdx.x * a.tiles + wa * TPW) * 16 + row;

  // staged scales: q8 of the workgroup's R = 16 tiles rows, all nbr blocks of
  // each, then the s2 values they refer to.  When nbr % 4 == 0 the rows are
  // stored qp = nbr + 4 bytes apart, so that the 16 rows one read
  // instruction touches fall in 16 different LDS banks (rows a multiple of
  // 128 bytes apart hit 2 banks: about 30 conflict cycles per read).
  const int nbr = a.K >> 6;
  // Blocks of each row the workgroup reads: all of them, or with the
  // reduction split only those of its own chunks, [blk0, blk0 + nbl).
  const int blk0 = 2 * cbase;
  const int nbl = max(1, min(2 * a.kchunks, nbr - blk0));
  const uint32_t R = (uint32_t)a.tiles * 16u;
  const uint32_t qp = (nbl & 3) ? (uint32_t)nbl : (uint32_t)nbl + 4u;  // LDS row pitch in bytes
  const uint32_t rowbase = (uint32_t)blockIdx.x * R;                  // first W row
  const uint32_t qbase = rowbase * (uint32_t)nbr;                     // its first block
  const uint32_t g_first = (qbase + (uint32_t)blk0) >> 8;
  const uint8_t* const s_q8 = reinterpret_cast<const uint8_t*>(s_dyn);
  const float* const s_s2 = reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(s_dyn) + R * qp);

  // U~ partials [uns][M][rp] (rp = r rounded up to 8, ranks past r zero) ->
  // LDS, for the workgroups that add the adapter term; requested here,
  // stored with the staged scales
  const bool ustage = a.upart != nullptr && a.r > 0 && kz == 0;
  const int urp = (a.r + 7) & ~7;
  float* const s_up = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(s_dyn) + a.uoff);
  const uint32_t un = ustage ? (uint32_t)(a.uns * a.M * urp) : 0u;  // floats staged, <= kSkUpBytes / 4
  const bool uvec = (a.r & 7) == 0;  // then the LDS copy is the global array
  uint4 upv[kSkUpLoads];
  float ups[4 * kSkUpLoads];
  if (ustage) {
    if (uvec) {
#pragma unroll
      for (int u = 0; u < kSkUpLoads; ++u) {
        const uint32_t i = (uint32_t)tid + (uint32_t)u * kSkThreads;
        upv[u] = i < un / 4 && in_bounds(4 * (int64_t)i, 4, (int64_t)a.uns * a.M * a.r)
                     ? *reinterpret_cast<const uint4*>(a.upart + 4 * i)
                     : make_uint4(0, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int u = 0; u < 4 * kSkUpLoads; ++u) {
        const uint32_t i = (uint32_t)tid + (uint32_t)u * kSkThreads;
        const uint32_t zm = i / (uint32_t)urp, j = i - zm * (uint32_t)urp;
        ups[u] = i < un && j < (uint32_t)a.r && in_bounds((int64_t)zm * a.r + j, 1, (int64_t)a.uns * a.M * a.r)
                     ? a.upart[zm * (uint32_t)a.r + j]
                     : 0.f;
      }
    }
  }
  auto store_up = [&]() {
    if (!ustage) return;
    if (uvec) {
#pragma unroll
      for (int u = 0; u < kSkUpLoads; ++u) {
        const uint32_t i = (uint32_t)tid + (uint32_t)u * kSkThreads;
        if (i < un / 4) *reinterpret_cast<uint4*>(s_up + 4 * i) = upv[u];
      }
    } else {
#pragma unroll
      for (int u = 0; u < 4 * kSkUpLoads; ++u) {
        const uint32_t i = (uint32_t)tid + (uint32_t)u * kSkThreads;
        if (i < un) s_up[i] = ups[u];
      }
    }
  };
  if (SL) {
    uint8_t* q8w = reinterpret_cast<uint8_t*>(s_dyn);
    float* s2w = reinterpret_cast<float*>(q8w + R * qp);
    const uint32_t ngs = ((qbase + (R - 1) * (uint32_t)nbr + (uint32_t)(blk0 + nbl) - 1) >> 8) - g_first + 1;
    float sv = 0.f;
    if ((uint32_t)tid < ngs) sv = __builtin_bit_cast(float, buf_load4(src.s2, (g_first + tid) * 4));
    if (nbl == nbr) {
      // whole rows: one contiguous run of R * nbr bytes (a multiple of 16)
      const uint32_t qbytes = R * (uint32_t)nbr;
      uint4 qv[kSkMaxStageLoads];  // all staged loads in flight at once
#pragma unroll
      for (int u = 0; u < kSkMaxStageLoads; ++u) {
        const uint32_t i = (uint32_t)tid + (uint32_t)u * kSkThreads;
        qv[u] = buf_load16(src.q8, i < qbytes / 16 ? qbase + 16 * i : kOOB);
      }
#pragma unroll
      for (int u = 0; u < kSkMaxStageLoads; ++u) {
        const uint32_t i = (uint32_t)tid + (uint32_t)u * kSkThreads;
        if (i < qbytes / 16) {
          if (qp == (uint32_t)nbr) {
            *reinterpret_cast<uint4*>(q8w + 16 * i) = qv[u];
          } else {
            // dwords 4 i .. 4 i + 3 of the rows: row r = 16 i / nbr, byte b (a multiple of 4)
            uint32_t r = (16 * i) / (uint32_t)nbr, b = 16 * i - r * (uint32_t)nbr;
            const uint32_t dw[4] = {qv[u].x, qv[u].y, qv[u].z, qv[u].w};
#pragma unroll
            for (int d = 0; d < 4; ++d) {
              *reinterpret_cast<uint32_t*>(q8w + r * qp + b) = dw[d];
              b += 4;
              if (b == (uint32_t)nbr) { b = 0; ++r; }
            }
          }
        }
      }
    } else if (((nbr | blk0 | nbl) & 3) == 0) {
      // a split: nbl bytes of each row, as dwords (every piece 4-byte aligned)
      // (batches of kSkMaxStageLoads dwords per thread, all in flight at once)
      const uint32_t pr = (uint32_t)nbl / 4, n = R * pr;
      for (uint32_t i0 = 0; i0 < n; i0 += kSkMaxStageLoads * kSkThreads) {
        uint32_t qv[kSkMaxStageLoads];
#pragma unroll
        for (int u = 0; u < kSkMaxStageLoads; ++u) {
          const uint32_t i = i0 + (uint32_t)tid + (uint32_t)u * kSkThreads, r = i / pr, d = i - r * pr;
          qv[u] = buf_load4(src.q8, i < n ? (rowbase + r) * (uint32_t)nbr + (uint32_t)blk0 + 4 * d : kOOB);
        }
#pragma unroll
        for (int u = 0; u < kSkMaxStageLoads; ++u) {
          const uint32_t i = i0 + (uint32_t)tid + (uint32_t)u * kSkThreads, r = i / pr, d = i - r * pr;
          if (i < n) *reinterpret_cast<uint32_t*>(q8w + r * qp + 4 * d) = qv[u];
        }
      }
    } else {
      // a split with unaligned pieces: byte by byte
      for (uint32_t i = (uint32_t)tid; i < R * (uint32_t)nbl; i += kSkThreads) {
        const uint32_t r = i / (uint32_t)nbl, b = i - r * (uint32_t)nbl;
        q8w[r * qp + b] = (uint8_t)buf_load1(src.q8, (rowbase + r) * (uint32_t)nbr + (uint32_t)blk0 + b);
      }
    }
    if ((uint32_t)tid < ngs) s2w[tid] = sv;
    store_up();
    __syncthreads();
  } else if (ustage) {
    store_up();
    __syncthreads();
  }
  // block scale a' = fp32(q8 * s2) of tile t, chunk c for this lane; chunks
  // past the split (padding: X == 0 there) take any staged finite scale
  auto lds_scale = [&](int t, int c) {
    const int bl = min(min(2 * c + (g >> 1), nbr - 1) - blk0, nbl - 1);  // staged block index
    const uint32_t rw = (uint32_t)((wa * TPW + t) * 16 + row);
    const uint32_t gb = qbase + rw * (uint32_t)nbr + (uint32_t)(blk0 + bl);  // global block index
    return (float)s_q8[rw * qp + (uint32_t)bl] * s_s2[(gb >> 8) - g_first];
  };
  const uint32_t e0 = (uint32_t)n0 * (uint32_t)a.K + 32u * (uint32_t)g;  // weight index at chunk 0

  // Code loads carry no range check of their own: a row past n_out lies past
  // the end of the codes (reads zeros, or -- if the index wraps -- some other
  // row's finite weights, into an output row that is never stored), and
  // columns past k_in (the tail of the last chunk, padding chunks) read the
  // next row's finite weights, and padding chunks of a split the next
  // split's, which meet X == 0 there (X loads are range checked).  Either way
  // nothing reaches a stored output.
  auto load = [&](int t, int i) {
    const int c = cbase + wb + (i << a.nwk_log2);
    const uint32_t e = e0 + (uint32_t)t * 16u * (uint32_t)a.K + (uint32_t)c * 128u;
    SkSeg s;
    s.code = buf_load16(src.codes, e >> 1);
    if (!SL) {
      s.q = buf_load1(src.q8, e >> 6);
      s.s2 = __builtin_bit_cast(float, buf_load4(src.s2, (e >> 14) << 2));
    } else {
      s.q = 0;
      s.s2 = 0.f;
    }
    return s;
  };
  // X fragment of chunk i: tokens m = lane & 15, columns kc + 32 g + 8 j
  const bool xrow = row < a.M;
  const uint32_t xoff0 = (uint32_t)row * (uint32_t)a.K * 2u + 64u * (uint32_t)g;
  auto load_x = [&](int i, uint4 xf[4]) {
    const int cl = wb + (i << a.nwk_log2), c = cbase + cl;
    const bool ok = xrow && (cl < nchl) && (c * 128 + 32 * g < a.K);
    const uint32_t o = xoff0 + (uint32_t)c * 256u;
#pragma unroll
    for (int j = 0; j < 4; ++j) xf[j] = buf_load16(src.X, ok ? o + 16u * j : kOOB);
  };
  // The decoded W fragments come out in the element order 0,2,4,6,1,3,5,7 of
  // each 8-column group (decode8_lut_hl); the X fragment is put in the same
  // order once per chunk and reused by every tile.
  auto order_x = [&](const uint4 (&xc)[4], uint4 (&xo)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) xo[j] = x_order_even_odd(xc[j]);
  };

  // lanes l and l ^ 16 share a block: the even row (g even) builds the
  // entries of levels 0..7, the odd row those of levels 8..15
  float th[8];
  lane_levels(a.nf4, g & 1, th);
  const EoConsts kc = eo_consts();

  f32x4 acc[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Issue order is pinned with full scheduling barriers: the X fragment of
  // chunk i + 1 is requested at the start of chunk i, and the codes of (tile
  // t, chunk i + RD) right after tile t of chunk i is decoded, so each load
  // has a whole chunk of decode work to arrive in.  Between two barriers the
  // MFMAs of tile t - 1 interleave with the decode of tile t.
  SkSeg ring[RD][TPW];
  uint4 xa[4], xb[4];
  load_x(0, xa);
#pragma unroll
  for (int d = 0; d < RD; ++d)
#pragma unroll
    for (int t = 0; t < TPW; ++t) ring[d][t] = load(t, d);
  __builtin_amdgcn_sched_barrier(0);

  auto chunk = [&](int i, SkSeg (&rg)[TPW], const uint4 (&xraw)[4], uint4 (&xn)[4]) {
    uint4 xc[4];
    order_x(xraw, xc);
    load_x(i + 1, xn);
    float sc[TPW];
    if (SL) {
      const int c = cbase + wb + (i << a.nwk_log2);
#pragma unroll
      for (int t = 0; t < TPW; ++t) sc[t] = lds_scale(t, c);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const SkSeg cs = rg[t];
      const float scale = SL ? sc[t] : (float)cs.q * cs.s2;  // a' = fp32(q8 * s2)
      const Lut L = build_lut<LutPartner::kRows16, E>(th, scale);
      const uint4 w0 = decode8_lut_hl(L, cs.code.x, kc);
      const uint4 w1 = decode8_lut_hl(L, cs.code.y, kc);
      const uint4 w2 = decode8_lut_hl(L, cs.code.z, kc);
      const uint4 w3 = decode8_lut_hl(L, cs.code.w, kc);
      rg[t] = load(t, i + RD);  // the same tile, RD chunks ahead
      __builtin_amdgcn_sched_barrier(0);
      acc[t] = E::mfma16(E::vec(w0), E::vec(xc[0]), acc[t]);
      acc[t] = E::mfma16(E::vec(w1), E::vec(xc[1]), acc[t]);
      acc[t] = E::mfma16(E::vec(w2), E::vec(xc[2]), acc[t]);
      acc[t] = E::mfma16(E::vec(w3), E::vec(xc[3]), acc[t]);
    }
  };
  // unrolled by U = max(RD, 2): static ring slot (u % RD) and X buffer (u % 2)
  constexpr int U = RD > 2 ? RD : 2;
  for (int it = 0; it < a.nci; it += U) {
#pragma unroll
    for (int u = 0; u < U; u += 2) {
      chunk(it + u, ring[u % RD], xa, xb);
      chunk(it + u + 1, ring[(u + 1) % RD], xb, xa);
    }
  }

  // adapter term U~ B^T, once per output tile (by the b == 0 wave): W-side
  // operand B[n][j], token-side operand U~[m][j], 32 ranks per MFMA
  if (wb == 0 && a.r > 0 && kz == 0) {
    const bool vec = (a.r & 7) == 0;
    for (int j0 = 0; j0 < a.r; j0 += 32) {
      const int j = j0 + 8 * g;
      uint4 uf = make_uint4(0, 0, 0, 0);
      if (row < a.M && j < a.r && ustage) {
        // U~[row][j .. j + 7] = E(uscale * (p0 + p1 + ...)) from the staged
        // partials, split 0 first then the others in order (as the finalize
        // pass of the down projection adds them)
        f32x4 lo = *reinterpret_cast<const f32x4*>(s_up + row * urp + j);
        f32x4 hi = *reinterpret_cast<const f32x4*>(s_up + row * urp + j + 4);
        for (int z = 1; z < a.uns; ++z) {
          lo += *reinterpret_cast<const f32x4*>(s_up + (z * a.M + row) * urp + j);
          hi += *reinterpret_cast<const f32x4*>(s_up + (z * a.M + row) * urp + j + 4);
        }
        const float c = a.uscale;
        uf = make_uint4(E::pack2(c * lo[0], c * lo[1]), E::pack2(c * lo[2], c * lo[3]), E::pack2(c * hi[0], c * hi[1]),
                        E::pack2(c * hi[2], c * hi[3]));
        if (a.Uout && blockIdx.x == 0 && wa == 0) {
          uint16_t* o = a.Uout + (int64_t)row * a.r + j;
          const int64_t oi = (int64_t)row * a.r + j, on = (int64_t)a.M * a.r;
          if (vec) {
            if (in_bounds(oi, 8, on)) *reinterpret_cast<uint4*>(o) = uf;
          } else {
            const uint32_t w[4] = {uf.x, uf.y, uf.z, uf.w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (j + e < a.r && in_bounds(oi + e, 1, on)) o[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
          }
        }
      } else if (row < a.M && j < a.r) {
        const uint16_t* p = a.U + (int64_t)row * a.r + j;
        const int64_t ui = (int64_t)row * a.r + j, un_ = (int64_t)a.M * a.r;
        if (vec) {
          if (in_bounds(ui, 8, un_)) uf = *reinterpret_cast<const uint4*>(p);
        } else {
          uint16_t v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = j + e < a.r && in_bounds(ui + e, 1, un_) ? p[e] : (uint16_t)0;
          uf = make_uint4(v[0] | (uint32_t)v[1] << 16, v[2] | (uint32_t)v[3] << 16,
                          v[4] | (uint32_t)v[5] << 16, v[6] | (uint32_t)v[7] << 16);
        }
      }
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int n = n0 + 16 * t;
        uint4 bf = make_uint4(0, 0, 0, 0);
        if (n < a.N && j < a.r) {
          const uint16_t* p = a.B + (int64_t)n * a.r + j;
          const int64_t bi = (int64_t)n * a.r + j, bn_ = (int64_t)a.N * a.r;
          if (vec) {
            if (in_bounds(bi, 8, bn_)) bf = *reinterpret_cast<const uint4*>(p);
          } else {
            uint16_t v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = j + e < a.r && in_bounds(bi + e, 1, bn_) ? p[e] : (uint16_t)0;
            bf = make_uint4(v[0] | (uint32_t)v[1] << 16, v[2] | (uint32_t)v[3] << 16,
                            v[4] | (uint32_t)v[5] << 16, v[6] | (uint32_t)v[7] << 16);
          }
        }
        acc[t] = E::mfma16(E::vec(bf), E::vec(uf), acc[t]);
      }
    }
  }

  // partial tiles -> LDS [tile][b][lane] (over the staged scales: wait for
  // every wave to leave the main loop), then a fixed-order sum over b.
  // With the fold, waves b >= nred first hand their tiles to wave b - nred,
  // which adds them to its own: slot b then holds acc_b + acc_(b + nred).
  constexpr int kFold = G::kFold;
  const int red_log2 = a.nwk_log2 - kFold, nred = 1 << red_log2;
  __syncthreads();
  if (!kFold || wb >= nred) {
    const int slot = kFold ? wb - nred : wb;
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int tt = wa * TPW + t;
      s_red[((tt << red_log2) + slot) * 64 + lane] = float4{acc[t][0], acc[t][1], acc[t][2], acc[t][3]};
    }
  }
  if (kFold) {
    __syncthreads();
    if (wb < nred) {
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        float4* slot = s_red + (((wa * TPW + t) << red_log2) + wb) * 64 + lane;
        const float4 v = *slot;
        *slot = float4{acc[t][0] + v.x, acc[t][1] + v.y, acc[t][2] + v.z, acc[t][3] + v.w};
      }
    }
  }
  __syncthreads();
  for (int idx = tid; idx < a.tiles * 64; idx += kSkThreads) {
    const int tt = idx >> 6, l = idx & 63;
    float4 s = s_red[(tt << red_log2) * 64 + l];
    for (int b = 1; b < nred; ++b) {
      const float4 v = s_red[((tt << red_log2) + b) * 64 + l];
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    // fragment element v of lane l: W row 4 (l >> 4) + v of the tile, token l & 15
    const int m = l & 15;
    const int n = (blockIdx.x * a.tiles + tt) * 16 + 4 * (l >> 4);
    if (m < a.M && n < a.N && a.part) {  // this split's fp32 partial sums
      if (in_bounds(((int64_t)kz * a.M + m) * a.N + n, 4, (int64_t)gridDim.y * a.M * a.N))
        *reinterpret_cast<float4*>(a.part + ((int64_t)kz * a.M + m) * a.N + n) = s;
    } else if (m < a.M && n < a.N) {  // n_out % 8 == 0: the 4 rows are all in range
      uint2 o;
      o.x = E::pack2(s.x, s.y);
      o.y = E::pack2(s.z, s.w);
      if (in_bounds((int64_t)m * a.N + n, 4, (int64_t)a.M * a.N)) *reinterpret_cast<uint2*>(a.Y + (int64_t)m * a.N + n) = o;
    }
  }
}

template <int TPW, int RD, int NW = 8>
hipError_t sk_launch(const SkinnyArgs& a, dim3 grid, size_t lds, bool sl, hipStream_t st) {
  constexpr int kSkThreads = SkGeom<NW>::kThreads;
  hipEvent_t ev0, ev1;
  take_gemm_events(ev0, ev1);
  hipError_t e;
  if (ev0 && (e = hipEventRecord(ev0, st)) != hipSuccess) return e;
  if (a.f16) {
    if (sl) hipLaunchKernelGGL((k_skinny_fwd<TPW, RD, true, F16, NW>), dim3(grid), dim3(kSkThreads), lds, st, a);
    else hipLaunchKernelGGL((k_skinny_fwd<TPW, RD, false, F16, NW>), dim3(grid), dim3(kSkThreads), lds, st, a);
  } else {
    if (sl) hipLaunchKernelGGL((k_skinny_fwd<TPW, RD, true, Bf16, NW>), dim3(grid), dim3(kSkThreads), lds, st, a);
    else hipLaunchKernelGGL((k_skinny_fwd<TPW, RD, false, Bf16, NW>), dim3(grid), dim3(kSkThreads), lds, st, a);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.part && (e = launch_splitk_reduce(a.part, (int)grid.y, a.M, a.N, a.Y, a.N, a.f16, st)) != hipSuccess) return e;
  if (ev1 && (e = hipEventRecord(ev1, st)) != hipSuccess) return e;
  return hipSuccess;
}

}  // namespace

QLORA_OOB_READER(oob_count_skinny)

// Largest M the few-token kernel handles.
int skinny_max_tokens() { return 16; }

// Work split: about one workgroup per compute unit.  A workgroup takes
// `tiles` = nwt * TPW W tiles; its 8 waves form nwt tile groups of TPW
// tiles, each split over nwk = 8 / nwt waves along the reduction.  The
// prefetch depth RD (chunks ahead) keeps about 8 code loads in flight per
// lane.  LDS: tiles * nwk KB <= 64 KB.
// Reduction split across workgroups: with 8 tokens or more, a weight whose
// tiles number at most 2 per compute unit (few outputs, a long reduction)
// would have every workgroup read all of X for those 2 tiles.  Instead a
// workgroup takes 8 tiles over 1 / ks of the reduction (at least 16 chunks
// of 128), when that still gives a workgroup per compute unit; the ks fp32
// partial sums are added in split order by a second pass.
SkinnySplit skinny_split(int64_t M, int64_t N, int64_t K, int cus) {
  const int64_t ntiles = (N + 15) / 16, nch = (K + 127) / 128;
  SkinnySplit sp{1, (int)nch};
  if (cus <= 0 || M < 8 || M > 16 || ntiles == 0 || (ntiles + cus - 1) / cus > 2) return sp;
  const int64_t groups = (ntiles + 7) / 8;
  const int64_t ks = std::min<int64_t>(cus / groups, nch / 16);
  if (ks < 2 || groups * ks < cus) return sp;
  // chunks per split, then the splits those chunks actually need (none empty)
  const int64_t kc = (nch + ks - 1) / ks;
  sp.kchunks = (int)kc;
  sp.ks = (int)((nch + kc - 1) / kc);
  return sp;
}

size_t skinny_part_bytes(int64_t M, int64_t N, int64_t K, int cus) {
  const int ks = skinny_split(M, N, K, cus).ks;
  return ks > 1 ? (size_t)ks * (size_t)M * (size_t)N * 4u : 0;
}

hipError_t launch_skinny_fwd(SkinnyArgs a, hipStream_t st) {
  const int ntiles = (a.N + 15) / 16;
  const int nch = (a.K + 127) / 128;
  const int num_cu = device_compute_units();
  SkinnySplit sp = skinny_split(a.M, a.N, a.K, num_cu);
  if (!a.part || sp.ks < 2) sp = SkinnySplit{1, nch};
  if (sp.ks < 2) a.part = nullptr;
  const int ks = sp.ks;
  a.kchunks = sp.kchunks;
  const int tpg = ks > 1 ? 8 : std::max(1, (ntiles + num_cu - 1) / num_cu);
  int tpw = std::min(tpg, 8);
  int nwt = 1;
  while (nwt * tpw < tpg && nwt < 8) nwt *= 2;
  tpw = std::min(8, (tpg + nwt - 1) / nwt);
  // 16 waves when a wave holds 2 tiles of an unsplit reduction and X is
  // short (fewer than 8 tokens): measured 3-4 % faster on a 8192 x 28672
  // weight at 1 and 4 tokens; with 1 tile per wave, or 16 tokens, no gain
  const bool w16 = ks == 1 && tpw == 2 && a.M < 8;
  const int nw = w16 ? 16 : 8;
  int nwk_log2 = 0;
  while ((nwt << (nwk_log2 + 1)) <= nw) ++nwk_log2;
  const int nwk = 1 << nwk_log2;
  int nci = (a.kchunks + nwk - 1) / nwk;
  // prefetch depth; with 16 waves (128 VGPRs) 2 chunks
  int rd = tpw >= 5 ? 1 : (tpw >= 3 ? 2 : (tpw == 2 ? (w16 ? 2 : 4) : 8));
  while (rd > 2 && nci % rd) rd /= 2;
  const int unroll = std::max(rd, 2);
  nci = (nci + unroll - 1) / unroll * unroll;  // padding chunks read nothing and add zeros
  a.tiles = nwt * tpw;
  a.nwk_log2 = nwk_log2;
  a.nci = nci;
  const dim3 grid((ntiles + a.tiles - 1) / a.tiles, ks);
  const size_t red = (size_t)a.tiles * (nwk >> (w16 ? SkGeom<16>::kFold : 0)) * 64 * sizeof(float4);
  // staged scales: q8 of 16 * tiles rows (the blocks of one split's chunks
  // when the reduction is split; the first split has the most), plus the
  // s2 groups the rows span
  const size_t nbr = (size_t)(a.K / 64);
  const size_t nbl = std::max<size_t>(1, std::min<size_t>(2 * (size_t)a.kchunks, nbr));
  const size_t rows = (size_t)a.tiles * 16;
  const size_t qbytes = rows * nbl;
  const size_t qpad = (nbl & 3) ? 0 : rows * 4;  // row padding of the LDS copy
  const size_t ngs = rows * nbr / 256 + 2;       // s2 groups, one staging thread each
  const size_t sbytes = qbytes + qpad + 4 * ngs;
  // within the default 64 KB of dynamic LDS (so the whole-row copy takes at
  // most kSkMaxStageLoads 16-byte pieces per thread), one thread per s2 group
  const bool sl = a.K >= 64 && sbytes <= 60 * 1024 && ngs <= (size_t)(64 * nw);
  size_t lds = std::max(red, sl ? sbytes : (size_t)0);
  if (a.upart) {
    // the U~ partials go after the staged scales; when they do not fit, a
    // finalize pass rounds them into U first
    const size_t ubytes = (size_t)a.uns * (size_t)a.M * (size_t)((a.r + 7) & ~7) * 4u;
    const size_t uoff = sl ? (sbytes + 15) & ~(size_t)15 : 0;
    if (a.r <= 0 || ubytes > (size_t)kSkUpBytes || uoff + ubytes > 64 * 1024) {
      if (a.r > 0) {
        if (!a.U) return hipErrorInvalidValue;
        // U is then the caller's U~ buffer (U_out or workspace), writable
        hipError_t e = launch_rowdot_finalize(a.upart, a.uns, a.M, a.r, a.uscale, const_cast<uint16_t*>(a.U), a.f16, st);
        if (e != hipSuccess) return e;
      }
      a.upart = nullptr;
    } else {
      a.uoff = (int)uoff;
      lds = std::max(lds, uoff + ubytes);
    }
  }
  if (w16) {
    switch (tpw * 16 + rd) {
      case 2 * 16 + 2: return sk_launch<2, 2, 16>(a, grid, lds, sl, st);
      default: return hipErrorInvalidValue;
    }
  }
  switch (tpw * 16 + rd) {
    case 1 * 16 + 1: return sk_launch<1, 1>(a, grid, lds, sl, st);
    case 1 * 16 + 2: return sk_launch<1, 2>(a, grid, lds, sl, st);
    case 1 * 16 + 4: return sk_launch<1, 4>(a, grid, lds, sl, st);
    case 1 * 16 + 8: return sk_launch<1, 8>(a, grid, lds, sl, st);
    case 2 * 16 + 1: return sk_launch<2, 1>(a, grid, lds, sl, st);
    case 2 * 16 + 2: return sk_launch<2, 2>(a, grid, lds, sl, st);
    case 2 * 16 + 4: return sk_launch<2, 4>(a, grid, lds, sl, st);
    case 3 * 16 + 1: return sk_launch<3, 1>(a, grid, lds, sl, st);
    case 3 * 16 + 2: return sk_launch<3, 2>(a, grid, lds, sl, st);
    case 4 * 16 + 1: return sk_launch<4, 1>(a, grid, lds, sl, st);
    case 4 * 16 + 2: return sk_launch<4, 2>(a, grid, lds, sl, st);
    case 5 * 16 + 1: return sk_launch<5, 1>(a, grid, lds, sl, st);
    case 6 * 16 + 1: return sk_launch<6, 1>(a, grid, lds, sl, st);
    case 7 * 16 + 1: return sk_launch<7, 1>(a, grid, lds, sl, st);
    case 8 * 16 + 1: return sk_launch<8, 1>(a, grid, lds, sl, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qlora
