// Device side of the softmax-gated block pooling shared by the pooling kernels
// (pool.hip) and the launches that pool a decode step's new block beside other work
// (topk_select.hip): the per-slice online softmax over a block's tokens, and the item
// layout of one thread per (sequence, entry, 8-channel slice).
//
// Source: "DeepSeek-V4 Hybrid Attention: CSA, HCA, mHC, MoE", section V.1 (an entry is
// the channel-wise weighted sum of its block's raw entries, the weights a softmax over
// the compression scores plus a positional bias).
#pragma once

#include "normrope.hpp"

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

}  // namespace
