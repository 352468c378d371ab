// RMSNorm + partial RoPE of rows in place or out of place (queries, window rows, cache
// entries built elsewhere).
//
// Source: "DeepSeek-V4 Hybrid Attention: CSA, HCA, mHC, MoE", section IV (RMSNorm on the
// queries and the compressed KV entries, RoPE on the last 64 dimensions only); the MLA
// walk-through's "The Code: RoPE Helpers" (consecutive pairs, theta^(-2i/d)).
//
// HBM-bound streaming: a row of c channels is held by c/8 consecutive lanes (a whole wave
// at c = 512, so a wave moves one contiguous 1 KiB bf16 row); the mean square is a lane
// reduction inside those lanes; lanes holding the last d channels rotate their four pairs.
#include "normrope.hpp"

namespace {

using csahca::NormRope;
using csahca::Vec8;
using csahca::VEC;

template <typename T>
__global__ __launch_bounds__(256) void norm_rope_rows(const T* __restrict__ x, T* y, NormRope nr,
                                                      const int* __restrict__ pos, int T_, int H,
                                                      int c, int pstride, long long rows,
                                                      long long x_bs, long long y_bs) {
  const int CV = c / VEC;
  const long long item = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  long long row;
  int cv, t, b;
  if (rows * CV <= 0x7FFFFFFFLL) {  // 32-bit index math (64-bit division is a long sequence)
    const uint32_t it = (uint32_t)item, r32 = it / (uint32_t)CV, bt = r32 / (uint32_t)H;
    row = r32;
    cv = (int)(it - r32 * (uint32_t)CV);
    b = (int)(bt / (uint32_t)T_);
    t = (int)(bt - (uint32_t)b * (uint32_t)T_);
  } else {
    row = item / CV;
    cv = (int)(item - row * CV);
    const long long bt = row / H;
    t = (int)(bt % T_);
    b = (int)(bt / T_);
  }
  if (row >= rows) return;  // whole rows leave together (CV divides 64)
  const long long in_seq = (row - (long long)b * T_ * H) * c;  // (t, h) offset
  const long long p = (pos ? (long long)pos[b] : 0LL) + (long long)t * pstride;
  csahca::norm_rope_row8<T>(x + b * x_bs + in_seq, y + b * y_bs + in_seq, nr, p, cv, CV, c);
}

}  // namespace

extern "C" int csahca_norm_rope(const void* x, void* y, const float* gamma, const int* pos, int B,
                                int T, int H, int c, int pstride, int d_rope, float eps,
                                float theta, int norm, int dtype, long long x_bstride,
                                long long y_bstride, void* stream) {
  using namespace csahca;
  if (B < 1 || T < 0 || H < 1 || (norm != 0 && norm != 1))
    return fail(CSAHCA_EINVAL, "csahca_norm_rope: need B >= 1, T >= 0, H >= 1 and norm 0 or 1");
  if (!norm_rope_args_ok(c, d_rope, eps, theta))
    return fail(CSAHCA_EINVAL, "csahca_norm_rope: need c / 8 a power of two <= 64, d_rope % 8 == 0 "
                               "and <= c, eps >= 0 and theta > 0");
  if (dtype != CSAHCA_F32 && dtype != CSAHCA_BF16)
    return fail(CSAHCA_ENOTSUP, "csahca_norm_rope: dtype must be CSAHCA_F32 or CSAHCA_BF16");
  if (T == 0) {
    clear_error();
    return CSAHCA_OK;
  }
  if (!x || !y) return fail(CSAHCA_EINVAL, "csahca_norm_rope: x and y must be non-NULL");
  if (!aligned16(x) || !aligned16(y) || !aligned16(gamma))
    return fail(CSAHCA_EINVAL, "csahca_norm_rope: x, y and gamma must be 16-byte aligned");
  const long long seq = (long long)T * H * c;
  if (x_bstride < seq || y_bstride < seq || x_bstride % 8 || y_bstride % 8)
    return fail(CSAHCA_EINVAL, "csahca_norm_rope: batch strides must be >= T*H*c and multiples of 8");
  const long long rows = (long long)B * T * H;
  const long long threads = rows * (c / VEC);
  if (cdiv<long long>(threads, 256) > 0x7FFFFFFFLL) return fail(CSAHCA_ENOTSUP, "csahca_norm_rope: too many rows");
  const NormRope nr{gamma, eps, theta, d_rope, norm};
  const dim3 grid((unsigned)cdiv<long long>(threads, 256));
  hipStream_t st = (hipStream_t)stream;
  if (dtype == CSAHCA_BF16)
    hipLaunchKernelGGL(norm_rope_rows<uint16_t>, grid, dim3(256), 0, st, (const uint16_t*)x, (uint16_t*)y, nr,
                       pos, T, H, c, pstride, rows, x_bstride, y_bstride);
  else
    hipLaunchKernelGGL(norm_rope_rows<float>, grid, dim3(256), 0, st, (const float*)x, (float*)y, nr, pos, T,
                       H, c, pstride, rows, x_bstride, y_bstride);
  return launch_status("csahca_norm_rope");
}
