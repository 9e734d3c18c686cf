// extern "C" entry points of libqlora: argument checks on the host, workspace
// layout, and the launch sequence of each operation on the caller's stream.
// Declarations and the contract of every entry point: include/qlora.h.
#include <algorithm>
#include <climits>
#include <cmath>
#include <cstring>
#include <string>

#include "../../include/qlora.h"
#include "common.h"
#include "gemm_args.h"
#include "skinny_args.h"

namespace qlora {
hipError_t launch_quantize(const float* W, int64_t nweights, uint8_t* codes, uint8_t* q8, float* s2,
                           hipStream_t st);
hipError_t launch_quantize_bf16(const uint16_t* W, int64_t nweights, uint8_t* codes, uint8_t* q8, float* s2,
                                hipStream_t st);
hipError_t launch_dequant(const uint8_t* codes, const uint8_t* q8, const float* s2, int64_t nweights,
                          uint16_t* out, bool f16, hipStream_t st);
hipError_t launch_quantize_fmt(const float* W, int64_t nweights, bool uniform, bool dq, uint8_t* codes,
                               uint8_t* q8, float* s2, float* absmax, hipStream_t st);
hipError_t launch_dequant_fmt(const uint8_t* codes, const uint8_t* q8, const float* s2, const float* absmax,
                              int64_t nweights, bool uniform, bool dq, bool f16, uint16_t* out, hipStream_t st);
hipError_t launch_merge(const uint8_t* codes, const uint8_t* q8, const float* s2, int N, int K, const uint16_t* A,
                        const uint16_t* B, int r, float s, uint16_t* out, hipStream_t st);
hipError_t launch_gemm_fwd(const GemmArgs& a, hipStream_t st);
hipError_t launch_gemm_dx(const GemmArgs& a, hipStream_t st);
void time_next_gemm(hipEvent_t start, hipEvent_t stop);
hipError_t launch_lora_down(const uint16_t* X, int M, int K, const uint16_t* A, int r, float s, uint16_t* U,
                            float* part, DropMask drop, bool f16, hipStream_t st);
size_t rowdot_part_bytes(int64_t M, int64_t Kd, int r);
int coldot_chunk_rows();
hipError_t launch_coldot(const uint16_t* v, int r, const uint16_t* in, int M, int C, float* part,
                         DropMask drop, bool f16, hipStream_t st);
hipError_t launch_finalize(const float* part, int nmc, int r, int C, float* out, bool trans, hipStream_t st);
hipError_t launch_vt_and_db(const uint16_t* dY, int M, int N, const uint16_t* B, const uint16_t* U, int r,
                            float s, uint16_t* V, float* vpart, float* cpart, float* dB, bool f16, hipStream_t st);
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t st);
hipError_t launch_zero_u16(uint16_t* p, int64_t n, hipStream_t st);
}  // namespace qlora

namespace {

thread_local std::string g_last_error;

int fail(int status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(QLORA_ERR_HIP, std::string(where) + ": " + hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round_up(size_t x) { return (x + 255) & ~(size_t)255; }

// Validates the frozen weight descriptor.
int check_weight(const qlora_nf4_weight* w) {
  if (!w) return fail(QLORA_ERR_INVALID_ARG, "weight descriptor is NULL");
  if (w->n_out < 0 || w->k_in < 0) return fail(QLORA_ERR_INVALID_ARG, "negative weight shape");
  if (w->k_in % 64 != 0) return fail(QLORA_ERR_SHAPE, "k_in must be a multiple of 64");
  if (w->n_out % 8 != 0) return fail(QLORA_ERR_SHAPE, "n_out must be a multiple of 8");
  if (w->n_out > 0 && w->k_in > 0 && w->n_out > (int64_t)(UINT32_MAX - 64) / w->k_in)
    return fail(QLORA_ERR_SHAPE, "n_out * k_in exceeds 2^32 weights");
  if (w->n_out > INT_MAX || w->k_in > INT_MAX) return fail(QLORA_ERR_SHAPE, "dimension exceeds INT_MAX");
  if (w->n_out * w->k_in > 0) {
    if (!w->codes || !w->absmax_q8 || !w->absmax_scale)
      return fail(QLORA_ERR_INVALID_ARG, "weight buffer pointer is NULL");
    if (!aligned16(w->codes) || !aligned16(w->absmax_q8) || !aligned16(w->absmax_scale))
      return fail(QLORA_ERR_ALIGN, "weight buffers must be 16-byte aligned");
  }
  return QLORA_OK;
}

int check_adapter(int32_t r, const uint16_t* A, const uint16_t* B) {
  if (r < 0) return fail(QLORA_ERR_INVALID_ARG, "r < 0");
  if (r > QLORA_MAX_RANK) return fail(QLORA_ERR_SHAPE, "r exceeds QLORA_MAX_RANK (64)");
  if (r > 0) {
    if (!A || !B) return fail(QLORA_ERR_INVALID_ARG, "A or B is NULL with r > 0");
    if (!aligned16(A) || !aligned16(B)) return fail(QLORA_ERR_ALIGN, "A and B must be 16-byte aligned");
  }
  return QLORA_OK;
}

int check_rows(int64_t M, int64_t n_out, int64_t k_in) {
  if (M < 0) return fail(QLORA_ERR_INVALID_ARG, "M < 0");
  if (M > INT_MAX) return fail(QLORA_ERR_SHAPE, "M exceeds INT_MAX");
  const int64_t widest = n_out > k_in ? n_out : k_in;
  // every activation / output buffer stays within 2^31 bytes (32-bit buffer offsets)
  if (widest > 0 && M > ((int64_t)1 << 30) / widest) return fail(QLORA_ERR_SHAPE, "M * width exceeds 2^30 elements");
  return QLORA_OK;
}

float lora_scale(float alpha, int32_t r) { return r > 0 ? alpha / (float)r : 0.f; }

// Dropout of the adapter input: keep threshold floor(p 2^32), key = seed, and
// the adapter scale with the 1 / (1 - p) of inverted dropout folded in,
// fp32(alpha / (r (1 - p))).  p = 0 is the plain layer.
int dropout_setup(int32_t r, float alpha, double p, uint64_t seed, qlora::DropMask* dm, float* s) {
  if (!(p >= 0.0 && p < 1.0)) return fail(QLORA_ERR_INVALID_ARG, "dropout_p must be in [0, 1)");
  *dm = qlora::DropMask{};
  if (p == 0.0) {
    *s = lora_scale(alpha, r);
    return QLORA_OK;
  }
  dm->thr = (uint32_t)std::floor(p * 4294967296.0);  // < 2^32 since p < 1
  dm->k0 = (uint32_t)seed;
  dm->k1 = (uint32_t)(seed >> 32);
  *s = r > 0 ? (float)((double)alpha / ((double)r * (1.0 - p))) : 0.f;
  return QLORA_OK;
}

struct BwdLayout {
  size_t u, v, part, cpart, total;  // part: U~ / V~ split-K partials; cpart: dA / dB row-chunk partials
  int nmc;
  size_t req;   // bytes required (U~, V~ and the reduction partials)
  size_t gemm;  // split-reduction tiles of the dX product, from `part` on
};

BwdLayout bwd_layout(int64_t M, int64_t n_out, int64_t k_in, int32_t r) {
  BwdLayout L{};
  if (M <= 0) return L;
  if (r > 0) {
    const int mch = qlora::coldot_chunk_rows();
    L.nmc = (int)((M + mch - 1) / mch);
    const int64_t widest = n_out > k_in ? n_out : k_in;
    L.u = 0;
    L.v = L.u + round_up((size_t)M * r * 2);
    L.part = L.v + round_up((size_t)M * r * 2);
    // U~ and V~ split-K partials share one region (stream order); the dB and
    // dA row-chunk partials share another (dB's are produced alongside V~'s)
    const size_t part = std::max(qlora::rowdot_part_bytes(M, k_in, r), qlora::rowdot_part_bytes(M, n_out, r));
    L.cpart = L.part + round_up(part);
    L.req = L.cpart + round_up((size_t)L.nmc * r * widest * 4);
  }
  // the dX product's split-reduction tiles reuse everything from L.part on
  // (dead by then); they need not fit: without room the product runs unsplit
  L.gemm = round_up(qlora::gemm_part_bytes(M, k_in, n_out));
  L.total = std::max(L.req, L.part + L.gemm);
  return L;
}

// Storage-format variants: checks shared by quantize and dequant.
int check_format(int format, int64_t n_out, int64_t k_in, const void* codes, const void* scales,
                 const void* s2, bool* uniform, bool* dq) {
  if (format < QLORA_FORMAT_NF4_DQ || format > QLORA_FORMAT_INT4) return fail(QLORA_ERR_INVALID_ARG, "unknown format");
  *uniform = format == QLORA_FORMAT_INT4_DQ || format == QLORA_FORMAT_INT4;
  *dq = format == QLORA_FORMAT_NF4_DQ || format == QLORA_FORMAT_INT4_DQ;
  qlora_nf4_weight w{n_out, k_in, static_cast<const uint8_t*>(codes), static_cast<const uint8_t*>(scales),
                     *dq ? static_cast<const float*>(s2) : reinterpret_cast<const float*>(scales)};
  return check_weight(&w);
}

}  // namespace

extern "C" {

const char* qlora_status_string(int status) {
  switch (status) {
    case QLORA_OK: return "QLORA_OK";
    case QLORA_ERR_INVALID_ARG: return "QLORA_ERR_INVALID_ARG: invalid argument";
    case QLORA_ERR_SHAPE: return "QLORA_ERR_SHAPE: unsupported shape";
    case QLORA_ERR_ALIGN: return "QLORA_ERR_ALIGN: pointer not 16-byte aligned";
    case QLORA_ERR_WORKSPACE: return "QLORA_ERR_WORKSPACE: workspace too small";
    case QLORA_ERR_HIP: return "QLORA_ERR_HIP: HIP runtime error";
    default: return "unknown qlora status";
  }
}

const char* qlora_last_error(void) { return g_last_error.c_str(); }

void qlora_time_next_gemm(hipEvent_t start, hipEvent_t stop) { qlora::time_next_gemm(start, stop); }

void qlora_nf4_table(float out[16]) {
  if (!out) return;
  const qlora::Nf4Consts& c = qlora::nf4_consts();
  std::memcpy(out, c.level, sizeof(c.level));
}

size_t qlora_workspace_bytes(int op, int64_t M, int64_t n_out, int64_t k_in, int32_t r) {
  if (M < 0 || n_out < 0 || k_in < 0 || r < 0 || r > QLORA_MAX_RANK) return 0;
  if (op == QLORA_OP_FWD) {
    if (M == 0) return 0;
    // [U~][U~ partials | split-reduction tiles of the main product]
    const size_t u = r > 0 ? round_up((size_t)M * r * 2) : 0;
    const size_t upart = r > 0 ? round_up(qlora::rowdot_part_bytes(M, k_in, r)) : 0;
    const size_t gpart = round_up(M > qlora::skinny_max_tokens() ? qlora::gemm_part_bytes(M, n_out, k_in)
                                                                  : qlora::skinny_part_bytes(M, n_out, k_in));
    return u + std::max(upart, gpart);
  }
  if (op == QLORA_OP_BWD) return bwd_layout(M, n_out, k_in, r).total;
  return 0;
}

int qlora_quantize_nf4_dq(const float* W, int64_t n_out, int64_t k_in, uint8_t* codes, uint8_t* absmax_q8,
                          float* absmax_scale, hipStream_t stream) {
  qlora_nf4_weight w{n_out, k_in, codes, absmax_q8, absmax_scale};
  int st = check_weight(&w);
  if (st) return st;
  if (n_out * k_in == 0) return QLORA_OK;
  if (!W) return fail(QLORA_ERR_INVALID_ARG, "W is NULL");
  if (!aligned16(W)) return fail(QLORA_ERR_ALIGN, "W must be 16-byte aligned");
  hipError_t e = qlora::launch_quantize(W, n_out * k_in, codes, absmax_q8, absmax_scale, stream);
  return e == hipSuccess ? QLORA_OK : hip_fail(e, "quantize launch");
}

int qlora_quantize_nf4_dq_bf16(const uint16_t* W, int64_t n_out, int64_t k_in, uint8_t* codes,
                               uint8_t* absmax_q8, float* absmax_scale, hipStream_t stream) {
  qlora_nf4_weight w{n_out, k_in, codes, absmax_q8, absmax_scale};
  int st = check_weight(&w);
  if (st) return st;
  if (n_out * k_in == 0) return QLORA_OK;
  if (!W) return fail(QLORA_ERR_INVALID_ARG, "W is NULL");
  if (!aligned16(W)) return fail(QLORA_ERR_ALIGN, "W must be 16-byte aligned");
  hipError_t e = qlora::launch_quantize_bf16(W, n_out * k_in, codes, absmax_q8, absmax_scale, stream);
  return e == hipSuccess ? QLORA_OK : hip_fail(e, "quantize launch");
}

int qlora_merge(const qlora_nf4_weight* w, const uint16_t* A, const uint16_t* B, int32_t r, float alpha,
                uint16_t* W_merged, hipStream_t stream) {
  int st = check_weight(w);
  if (st) return st;
  if ((st = check_adapter(r, A, B))) return st;
  if (w->n_out * w->k_in == 0) return QLORA_OK;
  if (!W_merged) return fail(QLORA_ERR_INVALID_ARG, "W_merged is NULL");
  if (!aligned16(W_merged)) return fail(QLORA_ERR_ALIGN, "W_merged must be 16-byte aligned");
  hipError_t e;
  if (r == 0) {
    // no adapter: the merged weight is the dequantized weight
    e = qlora::launch_dequant(w->codes, w->absmax_q8, w->absmax_scale, w->n_out * w->k_in, W_merged, false, stream);
  } else {
    e = qlora::launch_merge(w->codes, w->absmax_q8, w->absmax_scale, (int)w->n_out, (int)w->k_in, A, B, r,
                            lora_scale(alpha, r), W_merged, stream);
  }
  return e == hipSuccess ? QLORA_OK : hip_fail(e, "merge launch");
}

static int dequant_impl(const qlora_nf4_weight* w, uint16_t* W16, bool f16, hipStream_t stream) {
  int st = check_weight(w);
  if (st) return st;
  if (w->n_out * w->k_in == 0) return QLORA_OK;
  if (!W16) return fail(QLORA_ERR_INVALID_ARG, "output weight is NULL");
  if (!aligned16(W16)) return fail(QLORA_ERR_ALIGN, "output weight must be 16-byte aligned");
  hipError_t e = qlora::launch_dequant(w->codes, w->absmax_q8, w->absmax_scale, w->n_out * w->k_in, W16, f16,
                                       stream);
  return e == hipSuccess ? QLORA_OK : hip_fail(e, "dequant launch");
}

int qlora_dequant(const qlora_nf4_weight* w, uint16_t* W_bf16, hipStream_t stream) {
  return dequant_impl(w, W_bf16, false, stream);
}

int qlora_dequant_f16(const qlora_nf4_weight* w, uint16_t* W_f16, hipStream_t stream) {
  return dequant_impl(w, W_f16, true, stream);
}

static int linear_fwd_impl(const qlora_nf4_weight* w, const uint16_t* X, int64_t M, const uint16_t* A,
                           const uint16_t* B, int32_t r, float alpha, const qlora::DropMask& dm, float s,
                           uint16_t* Y, uint16_t* U_out, void* ws, size_t ws_bytes, bool f16, hipStream_t stream) {
  int st = check_weight(w);
  if (st) return st;
  if ((st = check_adapter(r, A, B))) return st;
  if ((st = check_rows(M, w->n_out, w->k_in))) return st;
  if (M == 0 || w->n_out == 0) return QLORA_OK;
  if (!X || !Y) return fail(QLORA_ERR_INVALID_ARG, "X or Y is NULL");
  if (!aligned16(X) || !aligned16(Y)) return fail(QLORA_ERR_ALIGN, "X and Y must be 16-byte aligned");
  if (U_out && !aligned16(U_out)) return fail(QLORA_ERR_ALIGN, "U_out must be 16-byte aligned");
  uint16_t* U = nullptr;
  float* part = nullptr;
  // workspace: [U~ when U_out is NULL][split-K partials of U~, later reused
  // for the split-reduction tiles of the main product (optional)]
  const size_t ubytes = r > 0 && !U_out ? round_up((size_t)M * r * 2) : 0;
  if (r > 0) {
    const size_t pbytes = qlora::rowdot_part_bytes(M, w->k_in, r);
    if (ubytes + pbytes > 0) {
      if (!ws || ws_bytes < ubytes + pbytes) return fail(QLORA_ERR_WORKSPACE, "forward workspace too small");
      if (!aligned16(ws)) return fail(QLORA_ERR_ALIGN, "workspace must be 16-byte aligned");
    }
    char* base = static_cast<char*>(ws);
    U = U_out ? U_out : reinterpret_cast<uint16_t*>(base);
    if (pbytes) part = reinterpret_cast<float*>(base + ubytes);
  }
  hipError_t e;
  if (r > 0 && w->k_in > 0) {
    e = qlora::launch_lora_down(X, (int)M, (int)w->k_in, A, r, s, U, part, dm, f16, stream);
    if (e != hipSuccess) return hip_fail(e, "lora_down launch");
  } else if (r > 0) {
    // k_in == 0: X A^T is an empty sum
    if ((e = qlora::launch_zero_u16(U, M * r, stream)) != hipSuccess) return hip_fail(e, "zero U");
  }
  if (M <= qlora::skinny_max_tokens()) {
    // few tokens: bound by reading the packed weight; decode straight into
    // MFMA operands, no LDS tile
    qlora::SkinnyArgs k{};
    k.X = X; k.codes = w->codes; k.q8 = w->absmax_q8; k.s2 = w->absmax_scale;
    k.U = U; k.B = B; k.Y = Y;
    k.M = (int)M; k.N = (int)w->n_out; k.K = (int)w->k_in; k.r = r;
    k.nf4 = qlora::nf4_consts();
    k.f16 = f16;
    // split partial sums after U~ (the U~ partials are consumed by then);
    // without room the kernel runs unsplit
    const size_t kbytes = qlora::skinny_part_bytes(M, w->n_out, w->k_in);
    if (kbytes && ws && aligned16(ws) && ws_bytes >= ubytes + kbytes)
      k.part = reinterpret_cast<float*>(static_cast<char*>(ws) + ubytes);
    e = qlora::launch_skinny_fwd(k, stream);
    return e == hipSuccess ? QLORA_OK : hip_fail(e, "few-token forward launch");
  }
  qlora::GemmArgs g{};
  g.act = X; g.ld_act = w->k_in; g.M = (int)M; g.R = (int)w->k_in; g.C = (int)w->n_out;
  g.codes = w->codes; g.q8 = w->absmax_q8; g.s2 = w->absmax_scale; g.K = (int)w->k_in;
  g.lora_act = U; g.lora_w = B; g.r = r;
  g.out = Y; g.ld_out = w->n_out;
  g.nf4 = qlora::nf4_consts();
  g.f16 = f16;
  const size_t gbytes = qlora::gemm_part_bytes(M, w->n_out, w->k_in);
  if (gbytes && ws && aligned16(ws) && ws_bytes >= ubytes + gbytes)
    g.part = reinterpret_cast<float*>(static_cast<char*>(ws) + ubytes);
  e = qlora::launch_gemm_fwd(g, stream);
  return e == hipSuccess ? QLORA_OK : hip_fail(e, "forward GEMM launch");
}

static int linear_bwd_impl(const qlora_nf4_weight* w, const uint16_t* X, const uint16_t* dY, int64_t M,
                           const uint16_t* A, const uint16_t* B, int32_t r, float alpha,
                           const qlora::DropMask& dm, float s, const uint16_t* U, uint16_t* dX, float* dA,
                           float* dB, void* ws, size_t ws_bytes, bool f16, hipStream_t stream) {
  int st = check_weight(w);
  if (st) return st;
  if ((st = check_adapter(r, A, B))) return st;
  if ((st = check_rows(M, w->n_out, w->k_in))) return st;
  const int64_t N = w->n_out, K = w->k_in;
  if (r > 0) {
    if (!dA || !dB) return fail(QLORA_ERR_INVALID_ARG, "dA or dB is NULL with r > 0");
    if (!aligned16(dA) || !aligned16(dB)) return fail(QLORA_ERR_ALIGN, "dA and dB must be 16-byte aligned");
  }
  if (M > 0 && K > 0) {
    if (!dX) return fail(QLORA_ERR_INVALID_ARG, "dX is NULL");
    if (!aligned16(dX)) return fail(QLORA_ERR_ALIGN, "dX must be 16-byte aligned");
  }
  if (M > 0 && (K > 0 || N > 0)) {
    if ((K > 0 && !X) || (N > 0 && !dY)) return fail(QLORA_ERR_INVALID_ARG, "X or dY is NULL");
    if ((X && !aligned16(X)) || (dY && !aligned16(dY))) return fail(QLORA_ERR_ALIGN, "X and dY must be 16-byte aligned");
  }
  if (U && !aligned16(U)) return fail(QLORA_ERR_ALIGN, "U must be 16-byte aligned");
  const BwdLayout L = bwd_layout(M, N, K, r);
  if (r > 0 && M > 0) {
    if (!ws || ws_bytes < L.req) return fail(QLORA_ERR_WORKSPACE, "backward workspace too small");
    if (!aligned16(ws)) return fail(QLORA_ERR_ALIGN, "workspace must be 16-byte aligned");
  }

  hipError_t e;
  if (M == 0 || N == 0 || K == 0) {
    // An empty dimension makes the token reductions (dA = V~^T X, dB = dY^T U~)
    // and, for n_out == 0, dX empty sums: write zeros.
    if (r > 0) {
      if ((e = qlora::launch_fill_zero(dA, (int64_t)r * K, stream)) != hipSuccess) return hip_fail(e, "zero dA");
      if ((e = qlora::launch_fill_zero(dB, N * r, stream)) != hipSuccess) return hip_fail(e, "zero dB");
    }
    if (M > 0 && K > 0) {
      if ((e = qlora::launch_zero_u16(dX, M * K, stream)) != hipSuccess) return hip_fail(e, "zero dX");
    }
    return QLORA_OK;
  }

  char* base = static_cast<char*>(ws);
  uint16_t* Ut = nullptr;
  uint16_t* Vt = nullptr;
  float* part = nullptr;
  if (r > 0) {
    Vt = reinterpret_cast<uint16_t*>(base + L.v);
    part = reinterpret_cast<float*>(base + L.part);
    if (U) {
      Ut = const_cast<uint16_t*>(U);
    } else {
      Ut = reinterpret_cast<uint16_t*>(base + L.u);
      if ((e = qlora::launch_lora_down(X, (int)M, (int)K, A, r, s, Ut, part, dm, f16, stream)) != hipSuccess)
        return hip_fail(e, "lora_down launch");
    }
    // V~ = bf16(s dY B) and dB = dY^T U~ (stored [N x r]): both read dY
    float* cpart = reinterpret_cast<float*>(base + L.cpart);
    if ((e = qlora::launch_vt_and_db(dY, (int)M, (int)N, B, Ut, r, s, Vt, part, cpart, dB, f16, stream)) != hipSuccess)
      return hip_fail(e, "V~ / dB launch");
    // dA = V~^T (mask * X)  ([r x K])
    if ((e = qlora::launch_coldot(Vt, r, X, (int)M, (int)K, cpart, dm, f16, stream)) != hipSuccess)
      return hip_fail(e, "dA partials launch");
    if ((e = qlora::launch_finalize(cpart, L.nmc, r, (int)K, dA, false, stream)) != hipSuccess)
      return hip_fail(e, "dA finalize launch");
  }
  qlora::GemmArgs g{};
  g.act = dY; g.ld_act = N; g.M = (int)M; g.R = (int)N; g.C = (int)K;
  g.codes = w->codes; g.q8 = w->absmax_q8; g.s2 = w->absmax_scale; g.K = (int)K;
  g.lora_act = Vt; g.lora_w = A; g.r = r;
  g.out = dX; g.ld_out = K;
  g.nf4 = qlora::nf4_consts();
  g.drop = dm;
  g.f16 = f16;
  // split-reduction tiles, from L.part on (U~ / V~ partials and dA / dB
  // partials are consumed by now); without room the product runs unsplit
  if (L.gemm && ws && aligned16(ws) && ws_bytes >= L.part + L.gemm)
    g.part = reinterpret_cast<float*>(static_cast<char*>(ws) + L.part);
  e = qlora::launch_gemm_dx(g, stream);
  return e == hipSuccess ? QLORA_OK : hip_fail(e, "dX GEMM launch");
}

int qlora_linear_fwd(const qlora_nf4_weight* w, const uint16_t* X, int64_t M, const uint16_t* A,
                     const uint16_t* B, int32_t r, float alpha, uint16_t* Y, uint16_t* U_out, void* ws,
                     size_t ws_bytes, hipStream_t stream) {
  return linear_fwd_impl(w, X, M, A, B, r, alpha, qlora::DropMask{}, lora_scale(alpha, r), Y, U_out, ws, ws_bytes,
                         false, stream);
}

int qlora_linear_fwd_f16(const qlora_nf4_weight* w, const uint16_t* X, int64_t M, const uint16_t* A,
                         const uint16_t* B, int32_t r, float alpha, uint16_t* Y, uint16_t* U_out, void* ws,
                         size_t ws_bytes, hipStream_t stream) {
  return linear_fwd_impl(w, X, M, A, B, r, alpha, qlora::DropMask{}, lora_scale(alpha, r), Y, U_out, ws, ws_bytes,
                         true, stream);
}

int qlora_linear_bwd(const qlora_nf4_weight* w, const uint16_t* X, const uint16_t* dY, int64_t M,
                     const uint16_t* A, const uint16_t* B, int32_t r, float alpha, const uint16_t* U,
                     uint16_t* dX, float* dA, float* dB, void* ws, size_t ws_bytes, hipStream_t stream) {
  return linear_bwd_impl(w, X, dY, M, A, B, r, alpha, qlora::DropMask{}, lora_scale(alpha, r), U, dX, dA, dB, ws,
                         ws_bytes, false, stream);
}

int qlora_linear_bwd_f16(const qlora_nf4_weight* w, const uint16_t* X, const uint16_t* dY, int64_t M,
                         const uint16_t* A, const uint16_t* B, int32_t r, float alpha, const uint16_t* U,
                         uint16_t* dX, float* dA, float* dB, void* ws, size_t ws_bytes, hipStream_t stream) {
  return linear_bwd_impl(w, X, dY, M, A, B, r, alpha, qlora::DropMask{}, lora_scale(alpha, r), U, dX, dA, dB, ws,
                         ws_bytes, true, stream);
}

int qlora_linear_fwd_dropout(const qlora_nf4_weight* w, const uint16_t* X, int64_t M, const uint16_t* A,
                             const uint16_t* B, int32_t r, float alpha, double dropout_p, uint64_t seed,
                             uint16_t* Y, uint16_t* U_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  qlora::DropMask dm{};
  float s = 0.f;
  const int st = dropout_setup(r, alpha, dropout_p, seed, &dm, &s);
  if (st) return st;
  return linear_fwd_impl(w, X, M, A, B, r, alpha, dm, s, Y, U_out, ws, ws_bytes, false, stream);
}

int qlora_linear_bwd_dropout(const qlora_nf4_weight* w, const uint16_t* X, const uint16_t* dY, int64_t M,
                             const uint16_t* A, const uint16_t* B, int32_t r, float alpha, double dropout_p,
                             uint64_t seed, const uint16_t* U, uint16_t* dX, float* dA, float* dB, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  qlora::DropMask dm{};
  float s = 0.f;
  const int st = dropout_setup(r, alpha, dropout_p, seed, &dm, &s);
  if (st) return st;
  return linear_bwd_impl(w, X, dY, M, A, B, r, alpha, dm, s, U, dX, dA, dB, ws, ws_bytes, false, stream);
}

int qlora_format_table(int format, float out[16]) {
  if (format < QLORA_FORMAT_NF4_DQ || format > QLORA_FORMAT_INT4) return fail(QLORA_ERR_INVALID_ARG, "unknown format");
  if (!out) return fail(QLORA_ERR_INVALID_ARG, "out is NULL");
  const bool uniform = format == QLORA_FORMAT_INT4_DQ || format == QLORA_FORMAT_INT4;
  const qlora::Nf4Consts& c = uniform ? qlora::int4_consts() : qlora::nf4_consts();
  std::memcpy(out, c.level, sizeof(c.level));
  return QLORA_OK;
}

int qlora_quantize_format(int format, const float* W, int64_t n_out, int64_t k_in, uint8_t* codes, void* scales,
                          float* absmax_scale, hipStream_t stream) {
  bool uniform = false, dq = false;
  int st = check_format(format, n_out, k_in, codes, scales, absmax_scale, &uniform, &dq);
  if (st) return st;
  if (n_out * k_in == 0) return QLORA_OK;
  if (!W) return fail(QLORA_ERR_INVALID_ARG, "W is NULL");
  if (!aligned16(W)) return fail(QLORA_ERR_ALIGN, "W must be 16-byte aligned");
  hipError_t e = qlora::launch_quantize_fmt(W, n_out * k_in, uniform, dq, codes,
                                            dq ? static_cast<uint8_t*>(scales) : nullptr,
                                            dq ? absmax_scale : nullptr,
                                            dq ? nullptr : static_cast<float*>(scales), stream);
  return e == hipSuccess ? QLORA_OK : hip_fail(e, "quantize launch");
}

int qlora_dequant_format(int format, int64_t n_out, int64_t k_in, const uint8_t* codes, const void* scales,
                         const float* absmax_scale, uint16_t* W_bf16, hipStream_t stream) {
  bool uniform = false, dq = false;
  int st = check_format(format, n_out, k_in, codes, scales, absmax_scale, &uniform, &dq);
  if (st) return st;
  if (n_out * k_in == 0) return QLORA_OK;
  if (!W_bf16) return fail(QLORA_ERR_INVALID_ARG, "W_bf16 is NULL");
  if (!aligned16(W_bf16)) return fail(QLORA_ERR_ALIGN, "W_bf16 must be 16-byte aligned");
  hipError_t e = qlora::launch_dequant_fmt(codes, dq ? static_cast<const uint8_t*>(scales) : nullptr,
                                           dq ? absmax_scale : nullptr,
                                           dq ? nullptr : static_cast<const float*>(scales), n_out * k_in,
                                           uniform, dq, false, W_bf16, stream);
  return e == hipSuccess ? QLORA_OK : hip_fail(e, "dequant launch");
}

}  // extern "C"
