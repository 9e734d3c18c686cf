// Device-side types and helpers shared by the gfx950 kernels of libqlora.
//
// Page legend for citations in csrc/:
//   [P1] "QLoRA, in depth: when a 4-bit base is worth it for small language
//        models, and how to ship the result"
//   [P4] "QLoRA and Fine-Tuning on One Consumer GPU"
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlora {

constexpr int kBlock = 64;    // weights per absmax block
constexpr int kGroup = 256;   // blocks per second-level scale
constexpr int kMaxRank = 64;

// NF4 levels and decision thresholds, built on the host and passed to every
// codec kernel by value (kernel arguments live in SGPRs; no device globals).
struct Nf4Consts {
  float level[16];  // ascending NF4 levels
  float thr[15];    // thr[i] = largest fp32 <= (level[i] + level[i+1]) / 2
};

const Nf4Consts& nf4_consts();  // host, built once

// Table-guided code search for quantization.  With x in [-1, 1] split into
// 256 cells of width 1/128 (cell i = int(x * 128 + 128), clamped), cand[i] is
// the number of thresholds below the start of cell i - 1.  No three
// consecutive cells hold two thresholds (they are > 3/128 apart), so the
// code -- the number of thresholds below x -- is cand[i] + (x > thr16[cand[i]])
// even when rounding of x * 128 + 128 moves x into a neighbouring cell
// (thr16[15] = +inf).
struct QuantSearch {
  uint8_t cand[256];
  float thr16[16];
};

const QuantSearch& quant_search();  // host, built once

// Compute units of the calling thread's current device: queried once per
// device and cached; 256 (an MI355X) when no device can be queried, as on a
// host without a GPU.  Work splits and the workspace sizes that hold their
// partial sums are both derived from it, so the two always agree.
int device_compute_units();

// Format variants: 16 evenly spaced levels -1 + 2 i / 15 with the same
// round-down midpoint thresholds, and their code search (host, built once).
const Nf4Consts& int4_consts();
const QuantSearch& quant_search_int4();

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

// 16-bit element type of a product: the weights are decoded to it, and
// the activations, adapter operands and outputs are stored in it.  bf16 is
// the pages' compute dtype ([P1] "A complete run on a 12 GB-class GPU" sets
// bnb_4bit_compute_dtype=torch.bfloat16); fp16 is the one the same listing
// names for GPUs without bf16.  Each kernel is instantiated once per type.
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;

struct Bf16 {
  typedef bf16x8 v8;
  // two fp32 -> packed pair, round to nearest even (v_cvt_pk_bf16_f32)
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) { return pack_bf16x2(lo, hi); }
  static __device__ __forceinline__ float widen(uint16_t b) { return bf16_to_f32(b); }
  static __device__ __forceinline__ v8 vec(uint4 u) { return __builtin_bit_cast(v8, u); }
  static __device__ __forceinline__ f32x16 mfma32(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16(v8 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

struct F16 {
  typedef f16x8 v8;
  // two fp32 -> packed pair, round to nearest even (v_cvt_pk_f16_f32)
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  }
  static __device__ __forceinline__ float widen(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
  static __device__ __forceinline__ v8 vec(uint4 u) { return __builtin_bit_cast(v8, u); }
  static __device__ __forceinline__ f32x16 mfma32(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16(v8 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

// Decode 8 packed NF4 codes (one dword, element 0 in the low nibble) with
// block scale a into 4 dwords of element pairs: w = E(level[c] * a).
// `lv` is the 16-entry level table in LDS (16 distinct banks: conflict-free).
template <typename E = Bf16>
__device__ __forceinline__ uint4 decode8(uint32_t d, float a, const float* lv) {
  uint4 o;
  o.x = E::pack2(lv[d & 15u] * a, lv[(d >> 4) & 15u] * a);
  o.y = E::pack2(lv[(d >> 8) & 15u] * a, lv[(d >> 12) & 15u] * a);
  o.z = E::pack2(lv[(d >> 16) & 15u] * a, lv[(d >> 20) & 15u] * a);
  o.w = E::pack2(lv[(d >> 24) & 15u] * a, lv[d >> 28] * a);
  return o;
}

// Block scale of block b: a' = fp32(q8[b] * s2[b / 256]).
__device__ __forceinline__ float block_scale(const uint8_t* q8, const float* s2, uint32_t b) {
  return (float)q8[b] * s2[b >> 8];
}

// ---- raw buffer loads: an offset at or past the buffer size reads zeros ----
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
constexpr uint32_t kOOB = 0x80000000u;  // callers keep every buffer <= 2^31 bytes

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t buf_load1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}

// ---- bounds-checked build ---------------------------------------------------
// Every raw global store, and every raw global load of caller-sized data
// (buffer loads are range checked by the hardware), is guarded by
// in_bounds(i, w, n): elements [i, i + w) of a buffer the caller sized to n
// elements (w == 0: no access, always in bounds).  In the normal build the guard is constant true and compiles
// away.  Built with -DQLORA_BOUNDS_CHECK (libqlora_checked.so), an access
// outside the buffer is skipped (a load reads zeros) and counted in a device
// counter of the translation unit, which qlora_debug_oob_count reads: a wrong
// index shows up as a count, not as a memory fault.
#ifdef QLORA_BOUNDS_CHECK
constexpr bool kBoundsChecked = true;
namespace {
__device__ unsigned int g_oob_count;
}  // namespace
__device__ __forceinline__ bool in_bounds(int64_t i, int64_t w, int64_t n) {
  if (w == 0 || (i >= 0 && w > 0 && i + w <= n)) return true;
  __hip_atomic_fetch_add(&g_oob_count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return false;
}
// host: this translation unit's count, cleared when `reset`
#define QLORA_OOB_READER(fn)                                                          \
  uint64_t fn(bool reset) {                                                           \
    unsigned int v = 0;                                                               \
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_oob_count), sizeof(v), 0, hipMemcpyDeviceToHost) != hipSuccess) \
      return ~(uint64_t)0;                                                            \
    if (reset) {                                                                      \
      const unsigned int z = 0;                                                       \
      if (hipMemcpyToSymbol(HIP_SYMBOL(g_oob_count), &z, sizeof(z), 0, hipMemcpyHostToDevice) != hipSuccess) \
        return ~(uint64_t)0;                                                          \
    }                                                                                 \
    return v;                                                                         \
  }
#else
constexpr bool kBoundsChecked = false;
__device__ __forceinline__ constexpr bool in_bounds(int64_t, int64_t, int64_t) { return true; }
#define QLORA_OOB_READER(fn) \
  uint64_t fn(bool) { return 0; }
#endif

// 16-byte chunk swizzle inside a 64-element (128-byte) bf16 LDS row: keeps
// ds_read_b128 / ds_write_b128 conflict-free for row-consecutive and for
// 8-row-strided access patterns.
__device__ __forceinline__ uint32_t swz(uint32_t row) { return (row ^ (row >> 3)) & 7u; }

}  // namespace qlora
