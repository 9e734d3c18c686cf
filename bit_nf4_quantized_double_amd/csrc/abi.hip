// extern "C" entry points of libqlora: argument checks on the host, workspace
// layout, and the launch sequence of each operation on the caller's stream.
// Declarations and the contract of every entry point: include/qlora.h.
#include <algorithm>
#include <atomic>
#include <climits>
#include <cmath>
#include <cstring>
#include <mutex>
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
hipError_t launch_lora_down_partials(const uint16_t* X, int M, int K, const uint16_t* A, int r, float* part,
                                     DropMask drop, bool f16, hipStream_t st);
int rowdot_nsplit(int64_t M, int64_t Kd, int r);
// the per-source-file out-of-bounds counters of the bounds-checked build
uint64_t oob_count_codec(bool reset);
uint64_t oob_count_gemm(bool reset);
uint64_t oob_count_skinny(bool reset);
uint64_t oob_count_lora(bool reset);
uint64_t oob_count_adapter(bool reset);
uint64_t oob_count_merge(bool reset);
hipError_t launch_lora_down(const uint16_t* X, int M, int K, const uint16_t* A, int r, float s, uint16_t* U,
                            float* part, DropMask drop, bool f16, hipStream_t st);
size_t rowdot_part_bytes(int64_t M, int64_t Kd, int r);
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t st);
hipError_t launch_zero_u16(uint16_t* p, int64_t n, hipStream_t st);
}  // namespace qlora

// Workspace of qlora_linear_fwd_noalloc: one array per GPU, held until the
// process ends.  Host code never passes `scratch` itself to a kernel (on the
// host it is only a stand-in for the device symbol); it passes the device
// address hipGetSymbolAddress gives for the current device.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace qlora {

int device_compute_units() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cached[kMaxDev];  // 0: not queried yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < kMaxDev) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
  if (dev < kMaxDev) cached[dev].store(v, std::memory_order_relaxed);
  return v;
}

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
  // every activation / output buffer stays within 2^31 bytes (32-bit buffer
  // offsets), the fragment-tiled activation copies (rows padded to 32,
  // columns to 64) included
  if (widest > 0 && M > ((int64_t)1 << 30) / widest) return fail(QLORA_ERR_SHAPE, "M * width exceeds 2^30 elements");
  const int64_t mpad = (M + 31) / 32 * 32, wpad = (widest + 63) / 64 * 64;
  if (widest > 0 && mpad > ((int64_t)1 << 30) / wpad)
    return fail(QLORA_ERR_SHAPE, "M * width, padded to whole MFMA fragments, exceeds 2^30 elements");
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
  size_t u, v, dyt, part, total;  // part: row-pass partials of V~ (and of U~ when it is recomputed)
  size_t mask;  // keep-mask bits of X (M x k_in / 8 bytes) for the column pass under dropout
  size_t req;   // bytes required (U~, V~, the tiled dY and the partials)
  size_t gemm;  // offset of the dX product's split-reduction tiles (optional room past req)
};

// [U~][V~][fragment-tiled dY][V~ partials | U~ recompute partials][split
// tiles of the dX product]; U~, V~ and partials only with an adapter (r > 0)
BwdLayout bwd_layout(int64_t M, int64_t n_out, int64_t k_in, int32_t r) {
  BwdLayout L{};
  if (M <= 0) return L;
  const int cus = qlora::device_compute_units();
  const size_t urow = r > 0 ? round_up((size_t)M * r * 2) : 0;
  L.u = 0;
  L.v = urow;
  L.dyt = 2 * urow;
  L.part = L.dyt + round_up(qlora::tiled_bytes(M, n_out));
  L.req = L.part;
  if (r > 0) {
    // a U~ recompute (no U given) is done with its partials -- those of the
    // forward's own method at this token count -- before the row pass over
    // dY writes the V~ partials: one region serves both
    const size_t ure = M <= qlora::skinny_max_tokens() ? qlora::rowdot_part_bytes(M, k_in, r)
                                                       : qlora::rowpass_part_bytes(M, k_in, r, cus);
    const size_t part = std::max(ure, qlora::rowpass_part_bytes(M, n_out, r, cus));
    L.mask = L.part + round_up(part);
    L.req = L.mask + round_up((size_t)M * (size_t)(k_in / 32) * 4u);
  }
  // the dX product reads the V~ partials while it runs: its split tiles go
  // after them; they need not fit (without room the product runs unsplit)
  L.gemm = L.req;
  L.total = L.req + round_up(qlora::gemm_part_bytes(M, k_in, n_out, cus));
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

int qlora_debug_oob_count(uint64_t* count, int reset) {
  if (!count) return fail(QLORA_ERR_INVALID_ARG, "count is NULL");
  if (!qlora::kBoundsChecked) return fail(QLORA_ERR_INVALID_ARG, "not the bounds-checked build");
  const bool rs = reset != 0;
  const uint64_t c[] = {qlora::oob_count_codec(rs), qlora::oob_count_gemm(rs), qlora::oob_count_skinny(rs),
                        qlora::oob_count_lora(rs), qlora::oob_count_adapter(rs), qlora::oob_count_merge(rs)};
  uint64_t total = 0;
  for (uint64_t v : c) {
    if (v == ~(uint64_t)0) return fail(QLORA_ERR_HIP, "reading the out-of-bounds counters failed");
    total += v;
  }
  *count = total;
  return QLORA_OK;
}

void qlora_nf4_table(float out[16]) {
  if (!out) return;
  const qlora::Nf4Consts& c = qlora::nf4_consts();
  std::memcpy(out, c.level, sizeof(c.level));
}

int qlora_plan(int op, int64_t M, int64_t n_out, int64_t k_in, int compute_units, int64_t out[4]) {
  if (!out) return fail(QLORA_ERR_INVALID_ARG, "out is NULL");
  if ((op != QLORA_OP_FWD && op != QLORA_OP_BWD) || M < 0 || n_out < 0 || k_in < 0)
    return fail(QLORA_ERR_INVALID_ARG, "invalid plan arguments");
  const int cus = compute_units > 0 ? compute_units : qlora::device_compute_units();
  if (op == QLORA_OP_FWD && M <= qlora::skinny_max_tokens()) {
    const qlora::SkinnySplit sp = qlora::skinny_split(M, n_out, k_in, cus);
    out[0] = 2;
    out[1] = sp.ks;
    out[2] = sp.kchunks;
    out[3] = (k_in + 127) / 128;
    return QLORA_OK;
  }
  // the fused GEMM: forward reduces over k_in into n_out columns, dX over n_out into k_in
  const int64_t C = op == QLORA_OP_FWD ? n_out : k_in, R = op == QLORA_OP_FWD ? k_in : n_out;
  const int64_t nsteps = (R + 63) / 64;
  const int ks = qlora::gemm_ksplit(M, C, R, cus);
  out[0] = 1;
  out[1] = ks;
  out[2] = (nsteps + ks - 1) / ks;
  out[3] = nsteps;
  return QLORA_OK;
}

size_t qlora_workspace_bytes(int op, int64_t M, int64_t n_out, int64_t k_in, int32_t r) {
  if (M < 0 || n_out < 0 || k_in < 0 || r < 0 || r > QLORA_MAX_RANK) return 0;
  if (op == QLORA_OP_FWD) {
    if (M == 0) return 0;
    const int cus = qlora::device_compute_units();
    if (M <= qlora::skinny_max_tokens()) {
      // few tokens: [U~][U~ partials][split partials of the main product]
      const size_t u = r > 0 ? round_up((size_t)M * r * 2) : 0;
      const size_t upart = r > 0 ? round_up(qlora::rowdot_part_bytes(M, k_in, r)) : 0;
      return u + upart + round_up(qlora::skinny_part_bytes(M, n_out, k_in, cus));
    }
    // [fragment-tiled X][U~ partials of the row pass][split tiles of the main product]
    const size_t xt = round_up(qlora::tiled_bytes(M, k_in));
    const size_t upart = r > 0 ? round_up(qlora::rowpass_part_bytes(M, k_in, r, cus)) : 0;
    return xt + upart + round_up(qlora::gemm_part_bytes(M, n_out, k_in, cus));
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
  char* base = static_cast<char*>(ws);
  const int cus = qlora::device_compute_units();
  hipError_t e;
  if (M <= qlora::skinny_max_tokens()) {
    // Few tokens: U~ first (split partial sums over k_in, then rounded),
    // then the few-token kernel, bound by reading the packed weight.
    // Workspace: [U~ when U_out is NULL][U~ partials, later the split
    // partials of the main product (optional)].
    const size_t ubytes = r > 0 && !U_out ? round_up((size_t)M * r * 2) : 0;
    const size_t pbytes = r > 0 ? round_up(qlora::rowdot_part_bytes(M, w->k_in, r)) : 0;
    if (ubytes + pbytes > 0) {
      if (!ws || ws_bytes < ubytes + pbytes) return fail(QLORA_ERR_WORKSPACE, "forward workspace too small");
      if (!aligned16(ws)) return fail(QLORA_ERR_ALIGN, "workspace must be 16-byte aligned");
    }
    qlora::SkinnyArgs k{};
    uint16_t* U = nullptr;
    if (r > 0) {
      U = U_out ? U_out : reinterpret_cast<uint16_t*>(base);
      if (w->k_in > 0) {
        // the down projection's split partials; the few-token kernel adds
        // them (and stores U~ to U_out)
        float* part = reinterpret_cast<float*>(base + ubytes);
        e = qlora::launch_lora_down_partials(X, (int)M, (int)w->k_in, A, r, part, dm, f16, stream);
        if (e != hipSuccess) return hip_fail(e, "lora_down launch");
        k.upart = part;
        k.uns = qlora::rowdot_nsplit(M, w->k_in, r);
        k.uscale = s;
        k.Uout = U_out;
      } else if ((e = qlora::launch_zero_u16(U, M * r, stream)) != hipSuccess) {
        return hip_fail(e, "zero U");
      }
    }
    k.X = X; k.codes = w->codes; k.q8 = w->absmax_q8; k.s2 = w->absmax_scale;
    k.U = U; k.B = B; k.Y = Y;
    k.M = (int)M; k.N = (int)w->n_out; k.K = (int)w->k_in; k.r = r;
    k.nf4 = qlora::nf4_consts();
    k.f16 = f16;
    // the split partials of the main product go after the U~ partials (the
    // kernel reads those while it writes these); without room the kernel
    // runs unsplit
    const size_t kbytes = qlora::skinny_part_bytes(M, w->n_out, w->k_in, cus);
    if (kbytes && ws && aligned16(ws) && ws_bytes >= ubytes + pbytes + kbytes)
      k.part = reinterpret_cast<float*>(base + ubytes + pbytes);
    e = qlora::launch_skinny_fwd(k, stream);
    return e == hipSuccess ? QLORA_OK : hip_fail(e, "few-token forward launch");
  }
  // The fused GEMM.  Workspace: [fragment-tiled X][U~ partials of the row
  // pass][split tiles of the main product (optional)].  One row pass over X
  // writes the tiled copy and the U~ partial sums; the GEMM adds them up in
  // its prologue (and stores U~ to U_out, when given).
  const size_t xbytes = round_up(qlora::tiled_bytes(M, w->k_in));
  const size_t pbytes = r > 0 ? round_up(qlora::rowpass_part_bytes(M, w->k_in, r, cus)) : 0;
  if (xbytes + pbytes > 0) {
    if (!ws || ws_bytes < xbytes + pbytes) return fail(QLORA_ERR_WORKSPACE, "forward workspace too small");
    if (!aligned16(ws)) return fail(QLORA_ERR_ALIGN, "workspace must be 16-byte aligned");
  }
  uint16_t* Xt = reinterpret_cast<uint16_t*>(base);
  float* upart = r > 0 ? reinterpret_cast<float*>(base + xbytes) : nullptr;
  if (r > 0) {
    e = qlora::launch_rowpass(X, (int)M, (int)w->k_in, A, r, true, dm, upart, Xt, f16, cus, stream);
    if (e != hipSuccess) return hip_fail(e, "row pass launch");
  } else if ((e = qlora::launch_tile_act(X, (int)M, (int)w->k_in, true, Xt, stream)) != hipSuccess) {
    return hip_fail(e, "tile X launch");
  }
  qlora::GemmArgs g{};
  g.act_t = Xt; g.kbp = qlora::tiled_kbp(w->k_in); g.M = (int)M; g.R = (int)w->k_in; g.C = (int)w->n_out;
  g.codes = w->codes; g.q8 = w->absmax_q8; g.s2 = w->absmax_scale; g.K = (int)w->k_in;
  g.lora_w = B; g.r = r;
  g.lora_part = upart; g.lora_ns = qlora::rowpass_plan(M, w->k_in, cus).S; g.lora_rp = qlora::rank_pitch(r);
  g.lora_scale = s; g.lora_out = r > 0 ? U_out : nullptr;
  g.out = Y; g.ld_out = w->n_out;
  g.nf4 = qlora::nf4_consts();
  g.f16 = f16;
  const size_t gbytes = qlora::gemm_part_bytes(M, w->n_out, w->k_in, cus);
  if (gbytes && ws_bytes >= xbytes + pbytes + gbytes) g.part = reinterpret_cast<float*>(base + xbytes + pbytes);
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
  if (M > 0 && N > 0 && K > 0) {
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
  const int cus = qlora::device_compute_units();
  uint16_t* Ut = nullptr;
  uint16_t* Vt = nullptr;
  float* part = nullptr;
  uint32_t* mbits = nullptr;
  uint16_t* dYt = reinterpret_cast<uint16_t*>(base + L.dyt);
  if (r > 0) {
    Vt = reinterpret_cast<uint16_t*>(base + L.v);
    part = reinterpret_cast<float*>(base + L.part);
    if (dm.thr) mbits = reinterpret_cast<uint32_t*>(base + L.mask);
    if (U) {
      Ut = const_cast<uint16_t*>(U);
    } else {
      // recompute U~ exactly as the forward formed it at this token count
      Ut = reinterpret_cast<uint16_t*>(base + L.u);
      if (M <= qlora::skinny_max_tokens()) {
        if ((e = qlora::launch_lora_down(X, (int)M, (int)K, A, r, s, Ut, part, dm, f16, stream)) != hipSuccess)
          return hip_fail(e, "lora_down launch");
      } else {
        if ((e = qlora::launch_rowpass(X, (int)M, (int)K, A, r, true, dm, part, nullptr, f16, cus, stream)) !=
            hipSuccess)
          return hip_fail(e, "row pass launch");
        if ((e = qlora::launch_rowpass_finalize(part, qlora::rowpass_plan(M, K, cus).S, (int)M, r, s, Ut, f16,
                                                stream)) != hipSuccess)
          return hip_fail(e, "U~ finalize launch");
      }
    }
    // one row pass over dY: the tiled dY the dX product reads and the V~
    // partial sums, added up (and V~ stored) in the dX product's prologue
    // (under dropout it also writes the keep mask of X as bits for the
    // column pass, which then need not regenerate it)
    if ((e = qlora::launch_rowpass(dY, (int)M, (int)N, B, r, false, qlora::DropMask{}, part, dYt, f16, cus,
                                   stream, mbits, (int)K, dm)) != hipSuccess)
      return hip_fail(e, "row pass launch");
  } else if ((e = qlora::launch_tile_act(dY, (int)M, (int)N, false, dYt, stream)) != hipSuccess) {
    return hip_fail(e, "tile dY launch");
  }
  qlora::GemmArgs g{};
  g.act_t = dYt; g.kbp = qlora::tiled_kbp(N); g.M = (int)M; g.R = (int)N; g.C = (int)K;
  g.codes = w->codes; g.q8 = w->absmax_q8; g.s2 = w->absmax_scale; g.K = (int)K;
  g.lora_w = A; g.r = r;
  g.lora_part = part; g.lora_ns = qlora::rowpass_plan(M, N, cus).S; g.lora_rp = qlora::rank_pitch(r);
  g.lora_scale = s; g.lora_out = Vt;
  g.out = dX; g.ld_out = K;
  g.nf4 = qlora::nf4_consts();
  g.drop = dm;
  g.f16 = f16;
  // split-reduction tiles past the required part; without room the product runs unsplit
  if (ws_bytes >= L.total && L.total > L.gemm) g.part = reinterpret_cast<float*>(base + L.gemm);
  e = qlora::launch_gemm_dx(g, stream);
  if (e != hipSuccess) return hip_fail(e, "dX GEMM launch");
  // dA = V~^T (mask * X) [r x K] and dB = dY^T U~ [N x r], over all tokens
  if (r > 0 && (e = qlora::launch_colpass(X, (int)K, Vt, dY, (int)N, Ut, (int)M, r, dm, dA, dB, f16, stream,
                                          mbits)) != hipSuccess)
    return hip_fail(e, "dA / dB launch");
  return QLORA_OK;
}

int qlora_linear_fwd(const qlora_nf4_weight* w, const uint16_t* X, int64_t M, const uint16_t* A,
                     const uint16_t* B, int32_t r, float alpha, uint16_t* Y, uint16_t* U_out, void* ws,
                     size_t ws_bytes, hipStream_t stream) {
  return linear_fwd_impl(w, X, M, A, B, r, alpha, qlora::DropMask{}, lora_scale(alpha, r), Y, U_out, ws, ws_bytes,
                         false, stream);
}

// Device address of `scratch` on the calling thread's current device,
// looked up once per device (with that device current) and cached.
static int noalloc_scratch(void** out) {
  constexpr int kMaxDev = 64;
  static std::mutex mu;
  static void* ptrs[kMaxDev] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDev) return fail(QLORA_ERR_INVALID_ARG, "device index beyond the no-alloc scratch table");
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(QLORA_ERR_HIP, "hipGetSymbolAddress(scratch) gave NULL");
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return QLORA_OK;
}

int qlora_linear_fwd_noalloc(const qlora_nf4_weight* w, const uint16_t* X, int64_t M, const uint16_t* A,
                             const uint16_t* B, int32_t r, float alpha, uint16_t* Y, uint16_t* U_out,
                             hipStream_t stream) {
  int st = check_weight(w);
  if (st) return st;
  if ((st = check_adapter(r, A, B))) return st;
  if ((st = check_rows(M, w->n_out, w->k_in))) return st;
  const size_t need = qlora_workspace_bytes(QLORA_OP_FWD, M, w->n_out, w->k_in, r);
  if (need > kNoAllocScratchBytes)
    return fail(QLORA_ERR_WORKSPACE, "the forward at these sizes needs " + std::to_string(need) +
                                         " workspace bytes, beyond the no-alloc scratch of " +
                                         std::to_string(kNoAllocScratchBytes));
  if (M == 0 || w->n_out == 0) return QLORA_OK;
  void* ws = nullptr;
  if ((st = noalloc_scratch(&ws))) return st;
  return linear_fwd_impl(w, X, M, A, B, r, alpha, qlora::DropMask{}, lora_scale(alpha, r), Y, U_out, ws,
                         kNoAllocScratchBytes, false, stream);
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

int qlora_linear_fwd_dropout_f16(const qlora_nf4_weight* w, const uint16_t* X, int64_t M, const uint16_t* A,
                                 const uint16_t* B, int32_t r, float alpha, double dropout_p, uint64_t seed,
                                 uint16_t* Y, uint16_t* U_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  qlora::DropMask dm{};
  float s = 0.f;
  const int st = dropout_setup(r, alpha, dropout_p, seed, &dm, &s);
  if (st) return st;
  return linear_fwd_impl(w, X, M, A, B, r, alpha, dm, s, Y, U_out, ws, ws_bytes, true, stream);
}

int qlora_linear_bwd_dropout_f16(const qlora_nf4_weight* w, const uint16_t* X, const uint16_t* dY, int64_t M,
                                 const uint16_t* A, const uint16_t* B, int32_t r, float alpha, double dropout_p,
                                 uint64_t seed, const uint16_t* U, uint16_t* dX, float* dA, float* dB, void* ws,
                                 size_t ws_bytes, hipStream_t stream) {
  qlora::DropMask dm{};
  float s = 0.f;
  const int st = dropout_setup(r, alpha, dropout_p, seed, &dm, &s);
  if (st) return st;
  return linear_bwd_impl(w, X, dY, M, A, B, r, alpha, dm, s, U, dX, dA, dB, ws, ws_bytes, true, stream);
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
