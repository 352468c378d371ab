// Kernel 1: softmax-gated block pooling (csa_compress / hca_compress).
//
// Source: "DeepSeek-V4 Hybrid Attention: CSA, HCA, mHC, MoE", section V.1 (an entry is
// the channel-wise weighted sum of its block's raw entries, the weights a softmax over
// the compression scores plus a positional bias) and section VI (the non-overlapping m'
// form); "DeepSeek-V4 Architecture From Kernels", section 6 (a blockwise softmax plus a
// weighted reduction).
//
// HBM-bound streaming: each thread owns 8 channels of one block and walks the block's m
// tokens with an online (running-max) softmax, so that X and Z are each read exactly
// once.  Consecutive threads own consecutive 8-channel slices of the same token row, so
// one wave reads a contiguous 64 x 16 B = 1 KiB row segment per token (bf16).
#include "common.hpp"

namespace {

constexpr int VEC = 8;      // channels per thread
constexpr int UNROLL = 8;   // tokens whose loads are issued together

template <typename T>
struct Vec8;

template <>
struct Vec8<uint16_t> {
  u32x4 raw;
  CSAHCA_DEV void load(const uint16_t* p) { raw = *reinterpret_cast<const u32x4*>(p); }
  CSAHCA_DEV float get(int i) const {
    uint32_t w = raw[i >> 1];
    return (i & 1) ? __uint_as_float(w & 0xFFFF0000u) : __uint_as_float(w << 16);
  }
  static CSAHCA_DEV void store(uint16_t* p, const float* v) {
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    *reinterpret_cast<u32x4*>(p) = o;
  }
};

template <>
struct Vec8<float> {
  f32x4 a, b;
  CSAHCA_DEV void load(const float* p) {
    a = *reinterpret_cast<const f32x4*>(p);
    b = *reinterpret_cast<const f32x4*>(p + 4);
  }
  CSAHCA_DEV float get(int i) const { return i < 4 ? a[i] : b[i - 4]; }
  static CSAHCA_DEV void store(float* p, const float* v) {
    *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
  }
};

template <typename T>
__global__ __launch_bounds__(256) void pool_kernel(const T* __restrict__ X,
                                                   const T* __restrict__ Z,
                                                   const float* __restrict__ P,
                                                   T* __restrict__ out, int N, int c, int m,
                                                   long long in_bs, long long out_bs,
                                                   long long total) {
  const long long item = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (item >= total) return;
  const int CV = c / VEC;
  const int cv = (int)(item % CV);
  const long long rest = item / CV;
  const int i = (int)(rest % N);
  const int b = (int)(rest / N);

  const long long base = (long long)b * in_bs + (long long)i * m * c + (long long)cv * VEC;
  const T* xp = X + base;
  const T* zp = Z + base;

  float mx[VEC], sum[VEC], acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    mx[e] = -INFINITY;
    sum[e] = 0.f;
    acc[e] = 0.f;
  }

  for (int j0 = 0; j0 < m; j0 += UNROLL) {
    const int cnt = min(UNROLL, m - j0);
    Vec8<T> xv[UNROLL], zv[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      if (u < cnt) {
        xv[u].load(xp + (long long)(j0 + u) * c);
        zv[u].load(zp + (long long)(j0 + u) * c);
      }
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      float z[UNROLL];
      float cm = mx[e];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        if (u < cnt) {
          z[u] = zv[u].get(e);
          if (P) z[u] += P[(j0 + u) * c + cv * VEC + e];
          cm = fmaxf(cm, z[u]);
        }
      }
      // cm is finite: at least one finite logit has been seen
      const float alpha = __expf(mx[e] - cm);  // exp(-inf) = 0 on the first chunk
      float s = sum[e] * alpha, a = acc[e] * alpha;
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        if (u < cnt) {
          const float p = __expf(z[u] - cm);
          s += p;
          a = fmaf(p, xv[u].get(e), a);
        }
      }
      mx[e] = cm;
      sum[e] = s;
      acc[e] = a;
    }
  }
  float res[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) res[e] = acc[e] / sum[e];
  Vec8<T>::store(out + (long long)b * out_bs + (long long)i * c + (long long)cv * VEC, res);
}

// Few blocks (a cache append at decode): one workgroup per (sequence, block).  Its
// threads split the block's m tokens into S contiguous sub-ranges per 8-channel slice,
// each with its own running softmax; the S partial states are merged in LDS in a fixed
// order, so the result does not depend on timing.
template <typename T>
__global__ __launch_bounds__(1024) void pool_block_kernel(const T* __restrict__ X,
                                                         const T* __restrict__ Z,
                                                         const float* __restrict__ P,
                                                         T* __restrict__ out, int N, int c,
                                                         int m, int S, long long in_bs,
                                                         long long out_bs) {
  extern __shared__ float part[];  // [S][CV][3][VEC]
  const int CV = c / VEC;
  const int cv = threadIdx.x % CV, s = threadIdx.x / CV;
  const int b = blockIdx.x / N, i = blockIdx.x % N;
  const int span = cdiv(m, S);
  const int j_lo = min(m, s * span), j_hi = min(m, j_lo + span);
  const long long base = (long long)b * in_bs + (long long)i * m * c + (long long)cv * VEC;
  float mx[VEC], sum[VEC], acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    mx[e] = -INFINITY;
    sum[e] = 0.f;
    acc[e] = 0.f;
  }
  for (int j0 = j_lo; j0 < j_hi; j0 += UNROLL) {
    const int cnt = min(UNROLL, j_hi - j0);
    Vec8<T> xv[UNROLL], zv[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      if (u < cnt) {
        xv[u].load(X + base + (long long)(j0 + u) * c);
        zv[u].load(Z + base + (long long)(j0 + u) * c);
      }
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      float z[UNROLL];
      float cm = mx[e];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        if (u < cnt) {
          z[u] = zv[u].get(e);
          if (P) z[u] += P[(j0 + u) * c + cv * VEC + e];
          cm = fmaxf(cm, z[u]);
        }
      }
      const float alpha = __expf(mx[e] - cm);
      float sm = sum[e] * alpha, a = acc[e] * alpha;
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        if (u < cnt) {
          const float p = __expf(z[u] - cm);
          sm += p;
          a = fmaf(p, xv[u].get(e), a);
        }
      }
      mx[e] = cm;
      sum[e] = sm;
      acc[e] = a;
    }
  }
  float* mine = part + ((size_t)s * CV + cv) * 3 * VEC;
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    mine[e] = mx[e];
    mine[VEC + e] = sum[e];
    mine[2 * VEC + e] = acc[e];
  }
  __syncthreads();
  if (s != 0) return;
  float res[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    float M = -INFINITY;
    for (int r = 0; r < S; ++r) M = fmaxf(M, part[((size_t)r * CV + cv) * 3 * VEC + e]);
    float sm = 0.f, a = 0.f;
    for (int r = 0; r < S; ++r) {
      const float* pr = part + ((size_t)r * CV + cv) * 3 * VEC;
      const float w = __expf(pr[e] - M);  // empty sub-range: exp(-inf) = 0
      sm = fmaf(pr[VEC + e], w, sm);
      a = fmaf(pr[2 * VEC + e], w, a);
    }
    res[e] = a / sm;
  }
  Vec8<T>::store(out + (long long)b * out_bs + (long long)i * c + (long long)cv * VEC, res);
}

int pool_entry(const char* name, const void* kv, const void* gate, const float* pos_bias,
               void* out, int B, int n, int c, int m, int dtype, long long in_bs,
               long long out_bs, void* stream) {
  using namespace csahca;
  if (B < 1 || n < 0 || c < 8 || (c % 8) != 0 || m < 1 || m > 4096)
    return fail(CSAHCA_EINVAL, "pool: need B >= 1, n >= 0, c >= 8 with c % 8 == 0, 1 <= m <= 4096");
  if (dtype != CSAHCA_F32 && dtype != CSAHCA_BF16)
    return fail(CSAHCA_ENOTSUP, "pool: dtype must be CSAHCA_F32 or CSAHCA_BF16");
  const long long N = n / m;
  if (N == 0) {  // no complete block: nothing to emit, nothing is read
    clear_error();
    return CSAHCA_OK;
  }
  if (!kv || !gate || !out) return fail(CSAHCA_EINVAL, "pool: kv, gate and out must be non-NULL");
  if (in_bs < (long long)n * c || out_bs < N * c)
    return fail(CSAHCA_EINVAL, "pool: in_bstride must be >= n*c and out_bstride >= (n/m)*c");
  if ((in_bs % 8) != 0 || (out_bs % 8) != 0)
    return fail(CSAHCA_EINVAL, "pool: strides must be multiples of 8 elements");
  if (!aligned16(kv) || !aligned16(gate) || !aligned16(out))
    return fail(CSAHCA_EINVAL, "pool: kv, gate and out must be 16-byte aligned");
  const long long total = (long long)B * N * (c / 8);
  hipStream_t st = (hipStream_t)stream;
  // few blocks of many tokens: split each block's tokens over more threads
  int S = min(m / 8, 1024 / (c / 8));
  if (S > 8) S = 8;
  if (total < 32768 && S >= 2) {
    const size_t lds = (size_t)S * (c / 8) * 3 * VEC * sizeof(float);
    if (lds <= 65536) {
      const unsigned grid = (unsigned)(B * N);
      const unsigned threads = (unsigned)(S * (c / 8));
      if (dtype == CSAHCA_BF16)
        hipLaunchKernelGGL(pool_block_kernel<uint16_t>, dim3(grid), dim3(threads), lds, st,
                           (const uint16_t*)kv, (const uint16_t*)gate, pos_bias, (uint16_t*)out,
                           (int)N, c, m, S, in_bs, out_bs);
      else
        hipLaunchKernelGGL(pool_block_kernel<float>, dim3(grid), dim3(threads), lds, st,
                           (const float*)kv, (const float*)gate, pos_bias, (float*)out, (int)N, c,
                           m, S, in_bs, out_bs);
      return launch_status(name);
    }
  }
  const int threads = 256;
  const long long blocks = cdiv<long long>(total, threads);
  if (blocks > 0x7FFFFFFFLL) return fail(CSAHCA_ENOTSUP, "pool: problem too large for one launch");
  if (dtype == CSAHCA_BF16) {
    hipLaunchKernelGGL(pool_kernel<uint16_t>, dim3((unsigned)blocks), dim3(threads), 0, st,
                       (const uint16_t*)kv, (const uint16_t*)gate, pos_bias, (uint16_t*)out,
                       (int)N, c, m, in_bs, out_bs, total);
  } else {
    hipLaunchKernelGGL(pool_kernel<float>, dim3((unsigned)blocks), dim3(threads), 0, st,
                       (const float*)kv, (const float*)gate, pos_bias, (float*)out, (int)N, c,
                       m, in_bs, out_bs, total);
  }
  return launch_status(name);
}

}  // namespace

extern "C" int csa_compress(const void* kv, const void* gate, const float* pos_bias, void* out,
                            int B, int n, int c, int m, int dtype, long long in_bstride,
                            long long out_bstride, void* stream) {
  return pool_entry("csa_compress", kv, gate, pos_bias, out, B, n, c, m, dtype, in_bstride,
                    out_bstride, stream);
}

extern "C" int hca_compress(const void* kv, const void* gate, const float* pos_bias, void* out,
                            int B, int n, int c, int m, int dtype, long long in_bstride,
                            long long out_bstride, void* stream) {
  return pool_entry("hca_compress", kv, gate, pos_bias, out, B, n, c, m, dtype, in_bstride,
                    out_bstride, stream);
}
