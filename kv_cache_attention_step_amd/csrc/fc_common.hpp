// Shared device/host helpers for the gfx950 kernels of libflashcache.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/flashcache.h"

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

#define FC_DEVICE __device__ __forceinline__

// ---------------------------------------------------------------------------
// bf16 <-> fp32 (bf16 is the upper half of an fp32)
// ---------------------------------------------------------------------------
FC_DEVICE float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
FC_DEVICE float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
FC_DEVICE float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// round to nearest even; NaN stays NaN
FC_DEVICE uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
FC_DEVICE uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}
// the same with the hardware pack-convert (round to nearest even, NaN stays NaN)
FC_DEVICE uint32_t pack2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// MFMA wrappers: D = A * B + C with A [32 x 16] (lane l: row l%32, k = 8*(l/32)..+7),
// B [16 x 32] (lane l: column l%32, same k), C/D [32 x 32] (lane l: column l%32,
// register i: row 8*(i/4) + 4*(l/32) + i%4).
FC_DEVICE f32x16_t mfma32x32x16(const bf16x8_t& a, const bf16x8_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Raw buffer descriptor over [base, base + bytes): loads past the end return 0.
FC_DEVICE __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
}

FC_DEVICE bf16x8_t as_bf16x8(const u32x4_t& v) { return __builtin_bit_cast(bf16x8_t, v); }

// LDS pointer type of the direct-to-LDS buffer loads
typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt with vmcnt = n and the LDS/export counters left unconstrained
#define FC_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

// ---------------------------------------------------------------------------
// host-side error plumbing (fc_status.cpp)
// ---------------------------------------------------------------------------
fc_status_t fc_fail(fc_status_t st, const char* fmt, ...);
fc_status_t fc_check_launch(const char* what);
void fc_clear_error();

// FC_DEBUG checks (validate.cpp): with the environment variable FC_DEBUG set to
// a non-zero value, entry points read their index inputs back (waiting for the
// stream) and reject invalid ones before anything is enqueued.
bool fc_debug_enabled();
fc_status_t fc_debug_check_qkv(const int32_t* positions, const int32_t* cu_seqlens_q, int B,
                               int T_q, const int32_t* block_table, int maxp, int page_size,
                               bool write_cache, hipStream_t st);
fc_status_t fc_debug_check_attention(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                     int B, int max_seqlen_q, int T_k,
                                     const int32_t* block_table, int maxp, int page_size,
                                     hipStream_t st);
fc_status_t fc_debug_check_offsets(const int32_t* cu, int B, int total, const char* name,
                                   const char* what, hipStream_t st);
fc_status_t fc_debug_check_views(const int32_t* cu_seqlens_k, const int32_t* verify_start,
                                 int B, const int32_t* block_table, int maxp, int page_size,
                                 int pages_per_view, hipStream_t st);

#define FC_REQUIRE(cond, st, ...)                   \
  do {                                              \
    if (!(cond)) return fc_fail((st), __VA_ARGS__); \
  } while (0)

static inline bool fc_is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
static inline int fc_log2i(int x) { int r = 0; while ((1 << r) < x) ++r; return r; }

// Compute units of the current device, cached per device id (256 if the query
// fails). Entries are read and written atomically; concurrent first calls on
// one device store the same value.
constexpr int FC_MAX_DEVICES = 64;
inline int fc_num_cus() {
  static int n_cu[FC_MAX_DEVICES] = {};
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < FC_MAX_DEVICES) {
    v = __atomic_load_n(&n_cu[dev], __ATOMIC_RELAXED);
    if (v > 0) return v;
  }
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
    v = 256;
  if (dev < FC_MAX_DEVICES) __atomic_store_n(&n_cu[dev], v, __ATOMIC_RELAXED);
  return v;
}
