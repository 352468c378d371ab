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
#include "normrope.hpp"
#include "pool.hpp"

namespace {

using csahca::NormRope;
using csahca::Vec8;
using csahca::VEC;

// Online softmax-weighted sum over tokens [j_lo, j_hi) of one 8-channel slice.  Full
// chunks of UB tokens issue all their loads first and reduce the chunk as balanced trees
// (max, sum of weights, sum of weighted values), so the dependent chain per chunk is
// log2(UB) deep instead of UB; a partial last chunk takes the guarded path.
// With ST the tokens read are also written to a doubled ring (row j to sx + j*c and
// sx + j*c + rs, likewise for the logits), so that an append stores what it pools.
template <typename T, int UB, bool HAS_P, bool ST = false>
CSAHCA_DEV void pool_run(const T* __restrict__ xp, const T* __restrict__ zp,
                         const float* __restrict__ pp, int c, int j_lo, int j_hi,
                         float (&mx)[VEC], float (&sum)[VEC], float (&acc)[VEC],
                         T* sx = nullptr, T* sz = nullptr, long long rs = 0) {
  int j0 = j_lo;
  for (; j0 + UB <= j_hi; j0 += UB) {
    Vec8<T> xv[UB], zv[UB];
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      xv[u].load(xp + (long long)(j0 + u) * c);
      zv[u].load(zp + (long long)(j0 + u) * c);
    }
    if (ST) {
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        const long long o = (long long)(j0 + u) * c;
        xv[u].put(sx + o);
        xv[u].put(sx + o + rs);
        zv[u].put(sz + o);
        zv[u].put(sz + o + rs);
      }
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
    if (ST) {
      const long long o = (long long)j0 * c;
      xv.put(sx + o);
      xv.put(sx + o + rs);
      zv.put(sz + o);
      zv.put(sz + o + rs);
    }
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

// Append mode: the entries are those an append of tokens n_old .. to a sequence
// completes.  Row j of entry e (position e*m + j) comes from the new tokens (X, row
// e*m + j - n_old) or, for the block begun by earlier appends, from the doubled ring
// (row (e*m + j) mod R; a block never wraps, R being a multiple of m).  With `store`, the
// new tokens read are also written to the ring (only when that overwrites none of the
// ring rows read in the same launch).
struct AppendRows {
  const void* ring_x;
  const void* ring_z;
  int R;
  int store;
  long long n_old;
  long long ring_bs;  // elements
};

constexpr int PLAIN = 0, TWO_STREAM = 1, APPEND = 2;

// Pool tokens [j_lo, j_hi) of entry e (absolute index) in append mode.
template <typename T, int UB, bool HAS_P>
CSAHCA_DEV void pool_append_run(const T* X, const T* Z, const AppendRows& ap, const float* pp,
                                int b, long long e, int m, int c, int cv, long long in_bs,
                                int j_lo, int j_hi, float (&mx)[VEC], float (&sum)[VEC],
                                float (&acc)[VEC]) {
  const long long p0 = e * m;  // position of the block's first token
  const int js = (int)max(0LL, min((long long)m, ap.n_old - p0));  // tokens from the ring
  const long long ro = (long long)b * ap.ring_bs + (p0 % ap.R) * c + (long long)cv * VEC;
  if (j_lo < js)
    pool_run<T, UB, HAS_P>((const T*)ap.ring_x + ro, (const T*)ap.ring_z + ro, pp, c, j_lo,
                           min(j_hi, js), mx, sum, acc);
  if (j_hi > js) {
    // rows j >= js of the new tokens: row j sits at new row p0 + j - n_old >= 0
    const long long no = (long long)b * in_bs + (p0 - ap.n_old) * c + (long long)cv * VEC;
    const int lo = max(j_lo, js);
    if (ap.store)
      pool_run<T, UB, HAS_P, true>(X + no, Z + no, pp, c, lo, j_hi, mx, sum, acc,
                                   (T*)ap.ring_x + ro, (T*)ap.ring_z + ro, (long long)ap.R * c);
    else
      pool_run<T, UB, HAS_P>(X + no, Z + no, pp, c, lo, j_hi, mx, sum, acc);
  }
}

// One thread per (sequence, entry, 8-channel slice); `bid` is the workgroup's index among
// those of this pooling (a paired launch offsets it).
template <typename T, int UB, bool HAS_P, int MODE, bool NR>
CSAHCA_DEV void pool_items(const T* __restrict__ X, const T* __restrict__ Z,
                           const T* __restrict__ Xb, const T* __restrict__ Zb,
                           const float* __restrict__ P, T* __restrict__ out, int N, int c, int m,
                           int prev, long long in_bs, long long out_bs, long long total,
                           const NormRope& nr, long long entry0, const AppendRows& ap, int bid) {
  constexpr bool OV = MODE == TWO_STREAM;
  const long long item = (long long)bid * blockDim.x + threadIdx.x;
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
  float g[VEC];  // NR: the channels' gains, loaded with the first tokens
  if (NR) csahca::load_gain8(nr, cv * VEC, g);
  float mx[VEC], sum[VEC], acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    mx[e] = -INFINITY;
    sum[e] = 0.f;
    acc[e] = 0.f;
  }
  if (MODE == APPEND)
    pool_append_run<T, UB, HAS_P>(X, Z, ap, HAS_P ? P + cv * VEC : nullptr, b, entry0 + i, m, c, cv,
                                  in_bs, 0, m, mx, sum, acc);
  else
    pool_run<T, UB, HAS_P>(X + base, Z + base, HAS_P ? P + cv * VEC : nullptr, c, 0, m, mx, sum, acc);
  if (OV && blk >= 1)  // stream b over the previous block, bias rows m .. 2m-1
    pool_run<T, UB, HAS_P>(Xb + base - (long long)m * c, Zb + base - (long long)m * c,
                           HAS_P ? P + (long long)m * c + cv * VEC : nullptr, c, 0, m, mx, sum, acc);
  float res[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) res[e] = acc[e] / sum[e];
  // the CV lanes of one entry are consecutive and aligned, so the row sum stays in them
  if (NR) csahca::norm_rope8(res, g, cv * VEC, CV, c, nr, (long long)m * (entry0 + i));
  Vec8<T>::store(out + (long long)b * out_bs + (long long)i * c + (long long)cv * VEC, res);
}

template <typename T, int UB, bool HAS_P, int MODE, bool NR>
__global__ __launch_bounds__(256) void pool_kernel(const T* __restrict__ X,
                                                   const T* __restrict__ Z,
                                                   const T* __restrict__ Xb,
                                                   const T* __restrict__ Zb,
                                                   const float* __restrict__ P,
                                                   T* __restrict__ out, int N, int c, int m,
                                                   int prev, long long in_bs, long long out_bs,
                                                   long long total, NormRope nr, long long entry0,
                                                   AppendRows ap) {
  pool_items<T, UB, HAS_P, MODE, NR>(X, Z, Xb, Zb, P, out, N, c, m, prev, in_bs, out_bs, total, nr,
                                     entry0, ap, (int)blockIdx.x);
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

// `bid` is the workgroup's index among those of this pooling (a paired launch offsets it);
// the workgroup has exactly S * CVG threads.
template <typename T, int UB, bool HAS_P, int MODE, bool NR>
CSAHCA_DEV void pool_block(const T* __restrict__ X, const T* __restrict__ Z,
                           const T* __restrict__ Xb, const T* __restrict__ Zb,
                           const float* __restrict__ P, T* __restrict__ out, int N, int c, int m,
                           int prev, int S, int CVG, long long in_bs, long long out_bs,
                           const NormRope& nr, long long entry0, const AppendRows& ap, int bid) {
  constexpr bool OV = MODE == TWO_STREAM;
  extern __shared__ float part[];  // [S][CVG][3][VEC], then (NR) [c] results + [16] sums
  const int CG = c / VEC / CVG;
  const int cvl = threadIdx.x % CVG, s = threadIdx.x / CVG;
  const int cg = bid % CG, bi = bid / CG;
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
  if (MODE == APPEND)
    pool_append_run<T, UB, HAS_P>(X, Z, ap, HAS_P ? P + cv * VEC : nullptr, b, entry0 + i, m, c, cv,
                                  in_bs, j_lo, min(j_hi, m), mx, sum, acc);
  else
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
  float* fin = part + (size_t)S * CVG * 3 * VEC;  // NR: the entry's c pooled values
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
    if (NR)
      fin[t] = av / sm;
    else
      store_one<T>(orow + t, av / sm);
  }
  if (NR) {
    // the workgroup holds the whole entry (CVG * VEC == c): RMS over the c values, then
    // the gain and the rotation of the last d channels, pairs read from LDS
    float* wsum = fin + c;
    __syncthreads();
    float inv = 1.f;
    if (nr.norm) {
      float ss = 0.f;
      for (int t = threadIdx.x; t < c; t += blockDim.x) ss = fmaf(fin[t], fin[t], ss);
      ss = csahca::row_sum(ss, 64);
      if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = ss;
      __syncthreads();
      ss = 0.f;
      for (int w = 0; w < (int)(blockDim.x + 63) / 64; ++w) ss += wsum[w];  // fixed order
      inv = 1.0f / sqrtf(ss / (float)c + nr.eps);
    }
    const long long pos = (long long)m * (entry0 + i);
    for (int t = threadIdx.x; t < c; t += blockDim.x) {
      const int u = t ^ 1;  // the pair's other channel
      const float gt = nr.gamma ? nr.gamma[t] : 1.f, gu = nr.gamma ? nr.gamma[u] : 1.f;
      float v = fin[t] * (inv * gt);
      if (t >= c - nr.d) {
        const float w = fin[u] * (inv * gu);
        float a = (t & 1) ? w : v, bb = (t & 1) ? v : w;
        csahca::rope_rotate(a, bb, pos, (t - (c - nr.d)) >> 1, nr.d, nr.theta);
        v = (t & 1) ? bb : a;
      }
      store_one<T>(orow + t, v);
    }
  }
}

template <typename T, int UB, bool HAS_P, int MODE, bool NR>
__global__ __launch_bounds__(NR ? 512 : 256) void pool_block_kernel(const T* __restrict__ X,
                                                        const T* __restrict__ Z,
                                                        const T* __restrict__ Xb,
                                                        const T* __restrict__ Zb,
                                                        const float* __restrict__ P,
                                                        T* __restrict__ out, int N, int c,
                                                        int m, int prev, int S, int CVG,
                                                        long long in_bs, long long out_bs,
                                                        NormRope nr, long long entry0,
                                                        AppendRows ap) {
  pool_block<T, UB, HAS_P, MODE, NR>(X, Z, Xb, Zb, P, out, N, c, m, prev, S, CVG, in_bs, out_bs, nr,
                                     entry0, ap, (int)blockIdx.x);
}

// Launch plan of a plain pooling (no bias, no norm) of N entries of m tokens: many entries
// take pool_kernel (one thread per 8-channel slice of an entry); few entries of many tokens
// take pool_block_kernel (the entry's tokens split over S sub-ranges per slice).
struct PoolPlan {
  bool block;   // pool_block_kernel
  int ub;       // tokens per load round: 4 or 8
  int S, CVG;   // block path: sub-ranges and slices per workgroup
  unsigned grid, threads;
  size_t lds;
  long long total;
};

PoolPlan plan_plain(int B, long long N, int c, int m) {
  PoolPlan p{};
  p.total = (long long)B * N * (c / 8);
  const int CV = c / VEC;
  p.block = p.total < 32768 && m >= 8;
  if (p.block) {
    int CVG = 8;
    while (CV % CVG != 0) CVG /= 2;
    const int smax = 256 / CVG;
    const int span = max(4, cdiv(m, smax));
    p.S = cdiv(m, span);
    p.CVG = CVG;
    p.lds = (size_t)p.S * CVG * 3 * VEC * sizeof(float);
    p.grid = (unsigned)(B * N * (CV / CVG));
    p.threads = (unsigned)(p.S * CVG);
    p.ub = (span % 8 == 0 && m % 8 == 0) ? 8 : 4;
  } else {
    p.grid = (unsigned)cdiv<long long>(p.total, 256);
    p.threads = 256;
    p.ub = m % 8 == 0 ? 8 : 4;
  }
  return p;
}

// One side of a paired pooling launch
template <typename T>
struct PoolSide {
  const T *X, *Z;
  T* out;
  int N, c, m, S, CVG;
  long long in_bs, out_bs, total;
};

// Two plain poolings in one launch: workgroups [0, gridA) run side A on pool_kernel's
// layout, the rest run side B on pool_block_kernel's (256 threads each).
template <typename T, int UBA, int UBB>
__global__ __launch_bounds__(256) void pool_pair_kernel(PoolSide<T> A, PoolSide<T> Bs, int gridA,
                                                        NormRope nr0, AppendRows ap0) {
  if ((int)blockIdx.x < gridA)
    pool_items<T, UBA, false, PLAIN, false>(A.X, A.Z, nullptr, nullptr, nullptr, A.out, A.N, A.c, A.m, 0,
                                            A.in_bs, A.out_bs, A.total, nr0, 0, ap0, (int)blockIdx.x);
  else
    pool_block<T, UBB, false, PLAIN, false>(Bs.X, Bs.Z, nullptr, nullptr, nullptr, Bs.out, Bs.N, Bs.c,
                                            Bs.m, 0, Bs.S, Bs.CVG, Bs.in_bs, Bs.out_bs, nr0, 0, ap0,
                                            (int)blockIdx.x - gridA);
}

template <typename T, bool HAS_P, int MODE, bool NR>
void launch_pool(const void* kv, const void* gate, const void* kv_b, const void* gate_b,
                 const float* pos_bias, void* out, int B, long long N, int c, int m, int prev,
                 long long in_bs, long long out_bs, const NormRope& nr, long long entry0,
                 const AppendRows& ap, hipStream_t st) {
  constexpr bool OV = MODE == TWO_STREAM;
  const long long total = (long long)B * N * (c / 8);
  const int CV = c / VEC;
  const int mt = OV ? 2 * m : m;  // tokens an entry reads
  const T *X = (const T*)kv, *Z = (const T*)gate, *Xb = (const T*)kv_b, *Zb = (const T*)gate_b;
  if (total < 32768 && mt >= 8) {
    // few blocks of many tokens: 8-channel slices in groups of up to 8 per workgroup,
    // tokens in sub-ranges of at least 4, at most 256 threads per workgroup.  With the
    // norm the workgroup holds the whole entry (all CV slices, at most 512 threads, a
    // whole number of waves).
    int CVG = 8, smax, unit = 1;
    if (NR) {
      CVG = CV;
      smax = 512 / CV;
      unit = CV >= 64 ? 1 : 64 / CV;
    } else {
      while (CV % CVG != 0) CVG /= 2;
      smax = 256 / CVG;
    }
    const int span = max(4, cdiv(mt, smax));
    const int S = cdiv(cdiv(mt, span), unit) * unit;
    const size_t lds = ((size_t)S * CVG * 3 * VEC + (NR ? (size_t)c + 16 : 0)) * sizeof(float);
    const unsigned grid = (unsigned)(B * N * (CV / CVG)), threads = (unsigned)(S * CVG);
    if (span % 8 == 0 && m % 8 == 0)
      hipLaunchKernelGGL((pool_block_kernel<T, 8, HAS_P, MODE, NR>), dim3(grid), dim3(threads), lds, st,
                         X, Z, Xb, Zb, pos_bias, (T*)out, (int)N, c, m, prev, S, CVG, in_bs, out_bs,
                         nr, entry0, ap);
    else
      hipLaunchKernelGGL((pool_block_kernel<T, 4, HAS_P, MODE, NR>), dim3(grid), dim3(threads), lds, st,
                         X, Z, Xb, Zb, pos_bias, (T*)out, (int)N, c, m, prev, S, CVG, in_bs, out_bs,
                         nr, entry0, ap);
    return;
  }
  const unsigned blocks = (unsigned)cdiv<long long>(total, 256);
  if (m % 8 == 0)
    hipLaunchKernelGGL((pool_kernel<T, 8, HAS_P, MODE, NR>), dim3(blocks), dim3(256), 0, st, X, Z, Xb,
                       Zb, pos_bias, (T*)out, (int)N, c, m, prev, in_bs, out_bs, total, nr, entry0,
                       ap);
  else
    hipLaunchKernelGGL((pool_kernel<T, 4, HAS_P, MODE, NR>), dim3(blocks), dim3(256), 0, st, X, Z, Xb,
                       Zb, pos_bias, (T*)out, (int)N, c, m, prev, in_bs, out_bs, total, nr, entry0,
                       ap);
}

struct PoolArgs {
  const void *kv, *gate, *kv_b, *gate_b;
  const float* pos_bias;
  void* out;
  int B;
  long long N;
  int c, m, prev;
  long long in_bs, out_bs;
  NormRope nr;
  long long entry0;
  AppendRows ap;
  hipStream_t st;
};

template <typename T, bool HP, int MODE, bool NR>
void run_pool(const PoolArgs& a) {
  launch_pool<T, HP, MODE, NR>(a.kv, a.gate, a.kv_b, a.gate_b, a.pos_bias, a.out, a.B, a.N, a.c,
                               a.m, a.prev, a.in_bs, a.out_bs, a.nr, a.entry0, a.ap, a.st);
}

template <typename T>
void pick_pool(const PoolArgs& a, bool hp, int mode, bool nr) {
  using F = void (*)(const PoolArgs&);
  static const F tab[12] = {
      run_pool<T, false, PLAIN, false>,      run_pool<T, false, PLAIN, true>,
      run_pool<T, false, TWO_STREAM, false>, run_pool<T, false, TWO_STREAM, true>,
      run_pool<T, false, APPEND, false>,     run_pool<T, false, APPEND, true>,
      run_pool<T, true, PLAIN, false>,       run_pool<T, true, PLAIN, true>,
      run_pool<T, true, TWO_STREAM, false>,  run_pool<T, true, TWO_STREAM, true>,
      run_pool<T, true, APPEND, false>,      run_pool<T, true, APPEND, true>};
  tab[(hp ? 6 : 0) + 2 * mode + (nr ? 1 : 0)](a);
}

}  // namespace

namespace csahca {

// Argument checks of one pooling; *N_out receives the number of entries to emit (0: the
// call has nothing to do and succeeds).
int pool_check(const char* name, const void* kv, const void* gate, const void* kv_b,
               const void* gate_b, bool ov, int prev, void* out, int B, int n, int c, int m,
               int dtype, long long in_bs, long long out_bs, long long* N_out) {
  using namespace csahca;
  *N_out = 0;
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
  if (N <= 0) return CSAHCA_OK;       // no complete block to emit: nothing is read
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
  *N_out = N;
  return CSAHCA_OK;
}

int pool_entry(const char* name, const void* kv, const void* gate, const void* kv_b,
               const void* gate_b, bool ov, int prev, const float* pos_bias, void* out, int B,
               int n, int c, int m, int dtype, long long in_bs, long long out_bs, void* stream,
               const NormRope* nr, long long entry0) {
  using namespace csahca;
  long long N = 0;
  int rc = pool_check(name, kv, gate, kv_b, gate_b, ov, prev, out, B, n, c, m, dtype, in_bs, out_bs, &N);
  if (rc != CSAHCA_OK) return rc;
  if (N == 0) {
    clear_error();
    return CSAHCA_OK;
  }
  if (nr && (!norm_rope_args_ok(c, nr->d, nr->eps, nr->theta) || entry0 < 0 || !aligned16(nr->gamma))) {
    set_error("%s: the norm needs c / 8 a power of two <= 64, d_rope %% 8 == 0 and <= c, "
              "eps >= 0, theta > 0, entry0 >= 0 and gamma 16-byte aligned", name);
    return CSAHCA_EINVAL;
  }
  PoolArgs a{kv, gate, kv_b, gate_b, pos_bias, out, B, N, c, m, prev, in_bs, out_bs,
             nr ? *nr : NormRope{nullptr, 0.f, 1.f, 0, 0}, entry0, AppendRows{nullptr, nullptr, 1, 0, 0, 0},
             (hipStream_t)stream};
  if (dtype == CSAHCA_BF16)
    pick_pool<uint16_t>(a, pos_bias != nullptr, ov ? TWO_STREAM : PLAIN, nr != nullptr);
  else
    pick_pool<float>(a, pos_bias != nullptr, ov ? TWO_STREAM : PLAIN, nr != nullptr);
  return launch_status(name);
}

// Two plain poolings of one layer pair (csa_compress and hca_compress arguments) in one
// launch when one takes pool_kernel's layout and the other pool_block_kernel's at 256
// threads; otherwise one launch each.  The entries are the same bits either way.
int pool_pair(const void* kv_a, const void* gate_a, void* out_a, int n_a, int m_a, long long in_bs_a,
              long long out_bs_a, const void* kv_b, const void* gate_b, void* out_b, int n_b, int m_b,
              long long in_bs_b, long long out_bs_b, int B, int c, int dtype, void* stream) {
  const char* name = "csahca_compress_pair";
  long long NA = 0, NB = 0;
  int rc = pool_check(name, kv_a, gate_a, nullptr, nullptr, false, 0, out_a, B, n_a, c, m_a, dtype,
                      in_bs_a, out_bs_a, &NA);
  if (rc != CSAHCA_OK) return rc;
  rc = pool_check(name, kv_b, gate_b, nullptr, nullptr, false, 0, out_b, B, n_b, c, m_b, dtype, in_bs_b,
                  out_bs_b, &NB);
  if (rc != CSAHCA_OK) return rc;
  hipStream_t st = (hipStream_t)stream;
  const PoolPlan pa = plan_plain(B, NA, c, m_a), pb = plan_plain(B, NB, c, m_b);
  const bool swap = pa.block && !pb.block;  // side 1 takes pool_kernel's layout
  const PoolPlan &p1 = swap ? pb : pa, &p2 = swap ? pa : pb;
  if (NA > 0 && NB > 0 && !p1.block && p2.block && p2.threads == 256 &&
      (long long)p1.grid + p2.grid <= 0x7FFFFFFFLL) {
    const NormRope nr0{nullptr, 0.f, 1.f, 0, 0};
    const AppendRows ap0{nullptr, nullptr, 1, 0, 0, 0};
    auto go = [&](auto tag) {
      using T = decltype(tag);
      const PoolSide<T> sa{(const T*)kv_a, (const T*)gate_a, (T*)out_a, (int)NA, c, m_a,
                           pa.S, pa.CVG, in_bs_a, out_bs_a, pa.total};
      const PoolSide<T> sb{(const T*)kv_b, (const T*)gate_b, (T*)out_b, (int)NB, c, m_b,
                           pb.S, pb.CVG, in_bs_b, out_bs_b, pb.total};
      const PoolSide<T>& s1 = swap ? sb : sa;
      const PoolSide<T>& s2 = swap ? sa : sb;
      const dim3 grid(p1.grid + p2.grid);
      const int g1 = (int)p1.grid;
      if (p1.ub == 8 && p2.ub == 8)
        hipLaunchKernelGGL((pool_pair_kernel<T, 8, 8>), grid, dim3(256), p2.lds, st, s1, s2, g1, nr0, ap0);
      else if (p1.ub == 8)
        hipLaunchKernelGGL((pool_pair_kernel<T, 8, 4>), grid, dim3(256), p2.lds, st, s1, s2, g1, nr0, ap0);
      else if (p2.ub == 8)
        hipLaunchKernelGGL((pool_pair_kernel<T, 4, 8>), grid, dim3(256), p2.lds, st, s1, s2, g1, nr0, ap0);
      else
        hipLaunchKernelGGL((pool_pair_kernel<T, 4, 4>), grid, dim3(256), p2.lds, st, s1, s2, g1, nr0, ap0);
    };
    if (dtype == CSAHCA_BF16)
      go(uint16_t{});
    else
      go(float{});
    return launch_status(name);
  }
  if (NA > 0) {
    rc = pool_entry(name, kv_a, gate_a, nullptr, nullptr, false, 0, nullptr, out_a, B, n_a, c, m_a, dtype,
                    in_bs_a, out_bs_a, stream);
    if (rc != CSAHCA_OK) return rc;
  }
  if (NB > 0)
    return pool_entry(name, kv_b, gate_b, nullptr, nullptr, false, 0, nullptr, out_b, B, n_b, c, m_b, dtype,
                      in_bs_b, out_bs_b, stream);
  clear_error();
  return CSAHCA_OK;
}

int pool_append(const char* name, const void* kv_new, const void* gate_new, const void* ring_x,
                const void* ring_z, int R, long long n_old, bool store, const float* pos_bias,
                void* entries, int B, long long first, long long count, int c, int m, int dtype,
                long long new_bs, long long ring_bs, long long ent_bs, void* stream) {
  if (count <= 0) return CSAHCA_OK;
  // N entries, the first being entry `first` of the cache; `out` addresses entry `first`
  const long long total = (long long)B * count * (c / 8);
  if (cdiv<long long>(total, 256) > 0x7FFFFFFFLL || count > 0x7FFFFFFFLL) {
    set_error("%s: problem too large for one launch", name);
    return CSAHCA_ENOTSUP;
  }
  const int e = dtype == CSAHCA_BF16 ? 2 : 4;
  PoolArgs a{kv_new, gate_new, nullptr, nullptr, pos_bias, (char*)entries + first * c * e, B, count, c, m, 0,
             new_bs, ent_bs, NormRope{nullptr, 0.f, 1.f, 0, 0}, first,
             AppendRows{ring_x, ring_z, R, store ? 1 : 0, n_old, ring_bs}, (hipStream_t)stream};
  if (dtype == CSAHCA_BF16)
    pick_pool<uint16_t>(a, pos_bias != nullptr, APPEND, false);
  else
    pick_pool<float>(a, pos_bias != nullptr, APPEND, false);
  return launch_status(name);
}

}  // namespace csahca

using csahca::pool_entry;

extern "C" int csa_compress(const void* kv, const void* gate, const float* pos_bias, void* out,
                            int B, int n, int c, int m, int dtype, long long in_bstride,
                            long long out_bstride, void* stream) {
  return pool_entry("csa_compress", kv, gate, nullptr, nullptr, false, 0, pos_bias, out, B, n, c,
                    m, dtype, in_bstride, out_bstride, stream, nullptr, 0);
}

extern "C" int csahca_compress_pair(const void* kv_a, const void* gate_a, void* out_a, int n_a,
                                    int m_a, long long in_bstride_a, long long out_bstride_a,
                                    const void* kv_b, const void* gate_b, void* out_b, int n_b,
                                    int m_b, long long in_bstride_b, long long out_bstride_b, int B,
                                    int c, int dtype, void* stream) {
  return csahca::pool_pair(kv_a, gate_a, out_a, n_a, m_a, in_bstride_a, out_bstride_a, kv_b, gate_b, out_b,
                           n_b, m_b, in_bstride_b, out_bstride_b, B, c, dtype, stream);
}

extern "C" int hca_compress(const void* kv, const void* gate, const float* pos_bias, void* out,
                            int B, int n, int c, int m, int dtype, long long in_bstride,
                            long long out_bstride, void* stream) {
  return pool_entry("hca_compress", kv, gate, nullptr, nullptr, false, 0, pos_bias, out, B, n, c,
                    m, dtype, in_bstride, out_bstride, stream, nullptr, 0);
}

extern "C" int csa_compress_overlap(const void* kv_a, const void* gate_a, const void* kv_b,
                                    const void* gate_b, const float* pos_bias, void* out, int B,
                                    int n, int c, int m, int prev, int dtype,
                                    long long in_bstride, long long out_bstride, void* stream) {
  return pool_entry("csa_compress_overlap", kv_a, gate_a, kv_b, gate_b, true, prev, pos_bias, out,
                    B, n, c, m, dtype, in_bstride, out_bstride, stream, nullptr, 0);
}

extern "C" int csahca_compress_norm_rope(const void* kv, const void* gate, const float* pos_bias,
                                         const float* gamma, void* out, int B, int n, int c,
                                         int m, long long entry0, int d_rope, float eps,
                                         float theta, int dtype, long long in_bstride,
                                         long long out_bstride, void* stream) {
  const NormRope nr{gamma, eps, theta, d_rope, 1};
  return pool_entry("csahca_compress_norm_rope", kv, gate, nullptr, nullptr, false, 0, pos_bias,
                    out, B, n, c, m, dtype, in_bstride, out_bstride, stream, &nr, entry0);
}

extern "C" int csa_compress_overlap_norm_rope(const void* kv_a, const void* gate_a,
                                              const void* kv_b, const void* gate_b,
                                              const float* pos_bias, const float* gamma,
                                              void* out, int B, int n, int c, int m, int prev,
                                              long long entry0, int d_rope, float eps,
                                              float theta, int dtype, long long in_bstride,
                                              long long out_bstride, void* stream) {
  const NormRope nr{gamma, eps, theta, d_rope, 1};
  return pool_entry("csa_compress_overlap_norm_rope", kv_a, gate_a, kv_b, gate_b, true, prev,
                    pos_bias, out, B, n, c, m, dtype, in_bstride, out_bstride, stream, &nr,
                    entry0);
}
