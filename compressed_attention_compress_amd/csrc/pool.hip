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
//
// Overlapped two-stream form (csa_compress_overlap, section V.1's equation with two KV
// streams): entry i walks stream a over block i and then stream b over block i-1 with
// the same running softmax, which is one joint softmax over the 2m logits.
#include "pool.hpp"

namespace {

constexpr int VEC = 8;      // channels per thread

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

// Online softmax-weighted sum over tokens [j_lo, j_hi) of one 8-channel slice.  Full
// chunks of UB tokens issue all their loads first and reduce the chunk as balanced trees
// (max, sum of weights, sum of weighted values), so the dependent chain per chunk is
// log2(UB) deep instead of UB; a partial last chunk takes the guarded path.
template <typename T, int UB, bool HAS_P>
CSAHCA_DEV void pool_run(const T* __restrict__ xp, const T* __restrict__ zp,
                         const float* __restrict__ pp, int c, int j_lo, int j_hi,
                         float (&mx)[VEC], float (&sum)[VEC], float (&acc)[VEC]) {
  int j0 = j_lo;
  for (; j0 + UB <= j_hi; j0 += UB) {
    Vec8<T> xv[UB], zv[UB];
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      xv[u].load(xp + (long long)(j0 + u) * c);
      zv[u].load(zp + (long long)(j0 + u) * c);
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      float z[UB], t[UB];
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        z[u] = zv[u].get(e);
        if (HAS_P) z[u] += pp[(j0 + u) * c + e];
        t[u] = z[u];
      }
#pragma unroll
      for (int w = UB / 2; w >= 1; w /= 2)
#pragma unroll
        for (int u = 0; u < w; ++u) t[u] = fmaxf(t[u], t[u + w]);
      const float cm = fmaxf(mx[e], t[0]);
      const float alpha = __expf(mx[e] - cm);  // exp(-inf) = 0 on the first chunk
      float pw[UB], px[UB];
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        pw[u] = __expf(z[u] - cm);
        px[u] = pw[u] * xv[u].get(e);
      }
#pragma unroll
      for (int w = UB / 2; w >= 1; w /= 2)
#pragma unroll
        for (int u = 0; u < w; ++u) {
          pw[u] += pw[u + w];
          px[u] += px[u + w];
        }
      mx[e] = cm;
      sum[e] = fmaf(sum[e], alpha, pw[0]);
      acc[e] = fmaf(acc[e], alpha, px[0]);
    }
  }
  for (; j0 < j_hi; ++j0) {  // tail: one token at a time
    Vec8<T> xv, zv;
    xv.load(xp + (long long)j0 * c);
    zv.load(zp + (long long)j0 * c);
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      float z = zv.get(e);
      if (HAS_P) z += pp[j0 * c + e];
      const float cm = fmaxf(mx[e], z);
      const float alpha = __expf(mx[e] - cm);
      const float p = __expf(z - cm);
      mx[e] = cm;
      sum[e] = fmaf(sum[e], alpha, p);
      acc[e] = fmaf(acc[e], alpha, p * xv.get(e));
    }
  }
}

template <typename T, int UB, bool HAS_P, bool OV>
__global__ __launch_bounds__(256) void pool_kernel(const T* __restrict__ X,
                                                   const T* __restrict__ Z,
                                                   const T* __restrict__ Xb,
                                                   const T* __restrict__ Zb,
                                                   const float* __restrict__ P,
                                                   T* __restrict__ out, int N, int c, int m,
                                                   int prev, long long in_bs, long long out_bs,
                                                   long long total) {
  const long long item = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (item >= total) return;
  const int CV = c / VEC;
  int cv, i, b;
  if (total <= 0x7FFFFFFFLL) {  // 32-bit index math (64-bit division is a long sequence)
    const uint32_t it = (uint32_t)item, rest = it / (uint32_t)CV;
    cv = (int)(it - rest * (uint32_t)CV);
    b = (int)(rest / (uint32_t)N);
    i = (int)(rest - (uint32_t)b * (uint32_t)N);
  } else {
    cv = (int)(item % CV);
    const long long rest = item / CV;
    i = (int)(rest % N);
    b = (int)(rest / N);
  }
  const int blk = OV ? i + prev : i;  // block of X (stream a)
  const long long base = (long long)b * in_bs + (long long)blk * m * c + (long long)cv * VEC;
  float mx[VEC], sum[VEC], acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    mx[e] = -INFINITY;
    sum[e] = 0.f;
    acc[e] = 0.f;
  }
  pool_run<T, UB, HAS_P>(X + base, Z + base, HAS_P ? P + cv * VEC : nullptr, c, 0, m, mx, sum, acc);
  if (OV && blk >= 1)  // stream b over the previous block, bias rows m .. 2m-1
    pool_run<T, UB, HAS_P>(Xb + base - (long long)m * c, Zb + base - (long long)m * c,
                           HAS_P ? P + (long long)m * c + cv * VEC : nullptr, c, 0, m, mx, sum, acc);
  float res[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) res[e] = acc[e] / sum[e];
  Vec8<T>::store(out + (long long)b * out_bs + (long long)i * c + (long long)cv * VEC, res);
}

// Few blocks (a cache append at decode): the workgroups of one (sequence, block) split
// its channels into groups of CVG 8-channel slices, and a workgroup's threads split the
// block's tokens into S contiguous sub-ranges per slice, each with its own running
// softmax.  The S partial states of a channel are merged in LDS in a fixed order (the
// result does not depend on timing), one thread per channel.
template <typename T>
CSAHCA_DEV void store_one(T* p, float v);
template <>
CSAHCA_DEV void store_one<uint16_t>(uint16_t* p, float v) { *p = f32_to_bf16(v); }
template <>
CSAHCA_DEV void store_one<float>(float* p, float v) { *p = v; }

template <typename T, int UB, bool HAS_P, bool OV>
__global__ __launch_bounds__(256) void pool_block_kernel(const T* __restrict__ X,
                                                        const T* __restrict__ Z,
                                                        const T* __restrict__ Xb,
                                                        const T* __restrict__ Zb,
                                                        const float* __restrict__ P,
                                                        T* __restrict__ out, int N, int c,
                                                        int m, int prev, int S, int CVG,
                                                        long long in_bs, long long out_bs) {
  extern __shared__ float part[];  // [S][CVG][3][VEC]
  const int CG = c / VEC / CVG;
  const int cvl = threadIdx.x % CVG, s = threadIdx.x / CVG;
  const int cg = blockIdx.x % CG, bi = blockIdx.x / CG;
  const int b = bi / N, i = bi - b * N;
  const int cv = cg * CVG + cvl;
  const int blk = OV ? i + prev : i;
  // the entry's tokens: stream a's m, then (overlapped, after the first block) stream b's
  // m of the previous block; thread s takes the s-th sub-range of them
  const int mt = (OV && blk >= 1) ? 2 * m : m;
  const int span = cdiv(OV ? 2 * m : m, S);
  const int j_lo = min(mt, s * span), j_hi = min(mt, j_lo + span);
  const long long base = (long long)b * in_bs + (long long)blk * m * c + (long long)cv * VEC;
  float mx[VEC], sum[VEC], acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    mx[e] = -INFINITY;
    sum[e] = 0.f;
    acc[e] = 0.f;
  }
  pool_run<T, UB, HAS_P>(X + base, Z + base, HAS_P ? P + cv * VEC : nullptr, c, j_lo, min(j_hi, m),
                         mx, sum, acc);
  if (OV && j_hi > m)
    pool_run<T, UB, HAS_P>(Xb + base - (long long)m * c, Zb + base - (long long)m * c,
                           HAS_P ? P + (long long)m * c + cv * VEC : nullptr, c, max(j_lo, m) - m,
                           j_hi - m, mx, sum, acc);
  float* mine = part + ((size_t)s * CVG + cvl) * 3 * VEC;
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    mine[e] = mx[e];
    mine[VEC + e] = sum[e];
    mine[2 * VEC + e] = acc[e];
  }
  __syncthreads();
  T* orow = out + (long long)b * out_bs + (long long)i * c + (long long)cg * CVG * VEC;
  for (int t = threadIdx.x; t < CVG * VEC; t += blockDim.x) {
    const int sl = t / VEC, e = t - sl * VEC;
    float M = -INFINITY;
    for (int r = 0; r < S; ++r) M = fmaxf(M, part[((size_t)r * CVG + sl) * 3 * VEC + e]);
    float sm = 0.f, av = 0.f;
    for (int r = 0; r < S; ++r) {
      const float* pr = part + ((size_t)r * CVG + sl) * 3 * VEC;
      const float w = __expf(pr[e] - M);  // empty sub-range: exp(-inf) = 0
      sm = fmaf(pr[VEC + e], w, sm);
      av = fmaf(pr[2 * VEC + e], w, av);
    }
    store_one<T>(orow + t, av / sm);
  }
}

template <typename T, bool HAS_P, bool OV>
void launch_pool(const void* kv, const void* gate, const void* kv_b, const void* gate_b,
                 const float* pos_bias, void* out, int B, long long N, int c, int m, int prev,
                 long long in_bs, long long out_bs, hipStream_t st) {
  const long long total = (long long)B * N * (c / 8);
  const int CV = c / VEC;
  const int mt = OV ? 2 * m : m;  // tokens an entry reads
  const T *X = (const T*)kv, *Z = (const T*)gate, *Xb = (const T*)kv_b, *Zb = (const T*)gate_b;
  if (total < 32768 && mt >= 8) {
    // few blocks of many tokens: 8-channel slices in groups of up to 8 per workgroup,
    // tokens in sub-ranges of at least 4, at most 256 threads per workgroup
    int CVG = 8;
    while (CV % CVG != 0) CVG /= 2;
    const int smax = 256 / CVG;
    const int span = max(4, cdiv(mt, smax));
    const int S = cdiv(mt, span);
    const size_t lds = (size_t)S * CVG * 3 * VEC * sizeof(float);
    const unsigned grid = (unsigned)(B * N * (CV / CVG)), threads = (unsigned)(S * CVG);
    if (span % 8 == 0 && m % 8 == 0)
      hipLaunchKernelGGL((pool_block_kernel<T, 8, HAS_P, OV>), dim3(grid), dim3(threads), lds, st,
                         X, Z, Xb, Zb, pos_bias, (T*)out, (int)N, c, m, prev, S, CVG, in_bs, out_bs);
    else
      hipLaunchKernelGGL((pool_block_kernel<T, 4, HAS_P, OV>), dim3(grid), dim3(threads), lds, st,
                         X, Z, Xb, Zb, pos_bias, (T*)out, (int)N, c, m, prev, S, CVG, in_bs, out_bs);
    return;
  }
  const unsigned blocks = (unsigned)cdiv<long long>(total, 256);
  if (m % 8 == 0)
    hipLaunchKernelGGL((pool_kernel<T, 8, HAS_P, OV>), dim3(blocks), dim3(256), 0, st, X, Z, Xb, Zb,
                       pos_bias, (T*)out, (int)N, c, m, prev, in_bs, out_bs, total);
  else
    hipLaunchKernelGGL((pool_kernel<T, 4, HAS_P, OV>), dim3(blocks), dim3(256), 0, st, X, Z, Xb, Zb,
                       pos_bias, (T*)out, (int)N, c, m, prev, in_bs, out_bs, total);
}

}  // namespace

namespace csahca {

int pool_entry(const char* name, const void* kv, const void* gate, const void* kv_b,
               const void* gate_b, bool ov, int prev, const float* pos_bias, void* out, int B,
               int n, int c, int m, int dtype, long long in_bs, long long out_bs, void* stream) {
  using namespace csahca;
  if (B < 1 || n < 0 || c < 8 || (c % 8) != 0 || m < 1 || m > 4096) {
    set_error("%s: need B >= 1, n >= 0, c >= 8 with c %% 8 == 0, 1 <= m <= 4096", name);
    return CSAHCA_EINVAL;
  }
  if (prev != 0 && prev != 1) {
    set_error("%s: prev must be 0 or 1", name);
    return CSAHCA_EINVAL;
  }
  if (dtype != CSAHCA_F32 && dtype != CSAHCA_BF16) {
    set_error("%s: dtype must be CSAHCA_F32 or CSAHCA_BF16", name);
    return CSAHCA_ENOTSUP;
  }
  const long long N = n / m - prev;  // entries to emit
  if (N <= 0) {  // no complete block to emit: nothing is read
    clear_error();
    return CSAHCA_OK;
  }
  if (!kv || !gate || !out || (ov && (!kv_b || !gate_b))) {
    set_error("%s: the KV, gate and out pointers must be non-NULL", name);
    return CSAHCA_EINVAL;
  }
  if (in_bs < (long long)n * c || out_bs < N * c) {
    set_error("%s: in_bstride must be >= n*c and out_bstride >= entries*c", name);
    return CSAHCA_EINVAL;
  }
  if ((in_bs % 8) != 0 || (out_bs % 8) != 0) {
    set_error("%s: strides must be multiples of 8 elements", name);
    return CSAHCA_EINVAL;
  }
  if (!aligned16(kv) || !aligned16(gate) || !aligned16(out) || (ov && (!aligned16(kv_b) || !aligned16(gate_b)))) {
    set_error("%s: the KV, gate and out pointers must be 16-byte aligned", name);
    return CSAHCA_EINVAL;
  }
  const long long total = (long long)B * N * (c / 8);
  if (cdiv<long long>(total, 256) > 0x7FFFFFFFLL) {
    set_error("%s: problem too large for one launch", name);
    return CSAHCA_ENOTSUP;
  }
  hipStream_t st = (hipStream_t)stream;
#define CSAHCA_POOL_LAUNCH(T, HP, O) \
  launch_pool<T, HP, O>(kv, gate, kv_b, gate_b, pos_bias, out, B, N, c, m, prev, in_bs, out_bs, st)
  if (dtype == CSAHCA_BF16) {
    if (ov) {
      if (pos_bias) CSAHCA_POOL_LAUNCH(uint16_t, true, true);
      else CSAHCA_POOL_LAUNCH(uint16_t, false, true);
    } else {
      if (pos_bias) CSAHCA_POOL_LAUNCH(uint16_t, true, false);
      else CSAHCA_POOL_LAUNCH(uint16_t, false, false);
    }
  } else {
    if (ov) {
      if (pos_bias) CSAHCA_POOL_LAUNCH(float, true, true);
      else CSAHCA_POOL_LAUNCH(float, false, true);
    } else {
      if (pos_bias) CSAHCA_POOL_LAUNCH(float, true, false);
      else CSAHCA_POOL_LAUNCH(float, false, false);
    }
  }
#undef CSAHCA_POOL_LAUNCH
  return launch_status(name);
}

}  // namespace csahca

using csahca::pool_entry;

extern "C" int csa_compress(const void* kv, const void* gate, const float* pos_bias, void* out,
                            int B, int n, int c, int m, int dtype, long long in_bstride,
                            long long out_bstride, void* stream) {
  return pool_entry("csa_compress", kv, gate, nullptr, nullptr, false, 0, pos_bias, out, B, n, c,
                    m, dtype, in_bstride, out_bstride, stream);
}

extern "C" int hca_compress(const void* kv, const void* gate, const float* pos_bias, void* out,
                            int B, int n, int c, int m, int dtype, long long in_bstride,
                            long long out_bstride, void* stream) {
  return pool_entry("hca_compress", kv, gate, nullptr, nullptr, false, 0, pos_bias, out, B, n, c,
                    m, dtype, in_bstride, out_bstride, stream);
}

extern "C" int csa_compress_overlap(const void* kv_a, const void* gate_a, const void* kv_b,
                                    const void* gate_b, const float* pos_bias, void* out, int B,
                                    int n, int c, int m, int prev, int dtype,
                                    long long in_bstride, long long out_bstride, void* stream) {
  return pool_entry("csa_compress_overlap", kv_a, gate_a, kv_b, gate_b, true, prev, pos_bias, out,
                    B, n, c, m, dtype, in_bstride, out_bstride, stream);
}
