// Shared device helpers for the gfx950 compressed-attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdarg>
#include <cstdio>
#include <string>

#include "csahca.h"

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define CSAHCA_DEV __device__ __forceinline__

// ---------------------------------------------------------------------------------------
// host-side status handling
// ---------------------------------------------------------------------------------------
namespace csahca {

void set_error(const char* fmt, ...);
void clear_error();

inline int fail(int code, const char* msg) {
  set_error("%s", msg);
  return code;
}

inline int launch_status(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("%s: launch failed: %s", what, hipGetErrorString(e));
    return CSAHCA_ELAUNCH;
  }
  clear_error();
  return CSAHCA_OK;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace csahca

// ---------------------------------------------------------------------------------------
// number formats
// ---------------------------------------------------------------------------------------
CSAHCA_DEV float bf16_to_f32(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// round to nearest even; inputs are finite
// float -> bfloat16, round to nearest even: gfx950's v_cvt_pk_bf16_f32 (two values per
// instruction)
typedef __bf16 bf16x2_hw __attribute__((ext_vector_type(2)));

CSAHCA_DEV uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

CSAHCA_DEV uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_hw v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// the float value of f rounded to bf16 (nearest even): low 16 bits cleared
CSAHCA_DEV float round_bf16(float f) { return __uint_as_float((uint32_t)f32_to_bf16(f) << 16); }


// float16, round to nearest even (the hardware conversion); two halves in one word
CSAHCA_DEV uint32_t pack_f16x2(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
}
CSAHCA_DEV float f16_lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu)); }
CSAHCA_DEV float f16_hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

// Order-preserving map of a float score to an unsigned key (larger score -> larger key);
// -0.0 is folded onto +0.0 so that the two compare equal.
CSAHCA_DEV uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

CSAHCA_DEV float key_score(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// 64-bit selection key: score first, then the LOWER index wins among equal scores.
// Every visible entry maps to a distinct nonzero key; 0 marks "no entry".
CSAHCA_DEV uint64_t entry_key(float score, uint32_t idx) {
  return ((uint64_t)score_key(score) << 32) | (uint64_t)(0xFFFFFFFFu - idx);
}

CSAHCA_DEV uint32_t key_index(uint64_t key) { return 0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFu); }

// ---------------------------------------------------------------------------------------
// wave-level helpers (wave64)
// ---------------------------------------------------------------------------------------
CSAHCA_DEV float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }

CSAHCA_DEV uint64_t shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  lo = __shfl_xor(lo, m, 64);
  hi = __shfl_xor(hi, m, 64);
  return ((uint64_t)hi << 32) | lo;
}

CSAHCA_DEV uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// x[l] + x[l ^ 16] + x[l ^ 32] + x[l ^ 48] in every lane (gfx950 permlane swaps, no LDS);
// the additions happen in the same order in all four lanes, so they agree bit for bit.
CSAHCA_DEV float sum_over_row_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// max over lanes l, l^16, l^32, l^48
CSAHCA_DEV float max_over_row_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// max over the 16 lanes of each row (DPP: xor 1, xor 2, rotate 4, rotate 8)
CSAHCA_DEV float row16_max(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false)));
  return x;
}

// inclusive prefix sum over the 64 lanes of a wave (DPP: shifts inside each row of 16,
// then row broadcasts; lanes without a source add 0)
CSAHCA_DEV uint32_t wave_incl_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false); // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false); // row_bcast:31
  return v;
}

// bitwise AND / OR over the 64 lanes of a wave, result in every lane
CSAHCA_DEV uint32_t wave_and(uint32_t x) {
  x &= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false);
  x &= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false);
  x &= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x124, 0xF, 0xF, false);
  x &= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x128, 0xF, 0xF, false);
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = a[0] & a[1];
  const auto b = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return b[0] & b[1];
}
CSAHCA_DEV uint32_t wave_or(uint32_t x) {
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false);
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false);
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x124, 0xF, 0xF, false);
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x128, 0xF, 0xF, false);
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = a[0] | a[1];
  const auto b = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return b[0] | b[1];
}

// Optional per-workgroup timestamps for latency studies (compiled out by default; a
// study includes one kernel source with CSAHCA_TRACE_ENABLED defined):
// shader-clock stamps in slots 0..13, fixed-rate stamps in slots 14 and 15.
#ifdef CSAHCA_TRACE_ENABLED
__device__ unsigned long long csahca_trace[8192 * 16];
#define CSAHCA_TRACE_WG (blockIdx.x + blockIdx.y * gridDim.x)
#define CSAHCA_TRACE(slot)                                                              \
  do {                                                                                  \
    if (threadIdx.x == 0 && CSAHCA_TRACE_WG < 8192)                                     \
      csahca_trace[CSAHCA_TRACE_WG * 16 + (slot)] = __builtin_amdgcn_s_memtime();       \
  } while (0)
#define CSAHCA_TRACE_RT(slot)                                                           \
  do {                                                                                  \
    if (threadIdx.x == 0 && CSAHCA_TRACE_WG < 8192)                                     \
      csahca_trace[CSAHCA_TRACE_WG * 16 + (slot)] = __builtin_amdgcn_s_memrealtime();   \
  } while (0)
#else
#define CSAHCA_TRACE(slot) \
  do {                     \
  } while (0)
#define CSAHCA_TRACE_RT(slot) \
  do {                        \
  } while (0)
#endif

// ceil-div for host and device
template <typename T>
__host__ __device__ constexpr T cdiv(T a, T b) {
  return (a + b - 1) / b;
}
