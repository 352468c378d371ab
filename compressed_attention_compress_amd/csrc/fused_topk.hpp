// The per-chunk half of the exact top-k selection, fused into the decode scoring kernel
// (workgroups of 256 threads).
//
// Source: "DeepSeek-V4 Hybrid Attention: CSA, HCA, mHC, MoE", section V.2 (the selector
// keeps the k best blocks by index score); "DeepSeek-V4: Anatomy of an Open-Source
// Frontier Model", "Worked example" (no more entries than exist can be picked).
//
// Keys: an entry's 64-bit key is (order-preserving score bits << 32) | (~index), so all
// keys differ and the larger key is the better score, or the lower index on equal scores.
//
// Each scoring workgroup holds the scores of its chunk in LDS.  It lists its entries whose
// 32-bit score key is at least a cut, chosen by one or two radix histogram passes so that
// between JT and JMAX entries pass (every entry when the chunk holds at most JMAX), in
// index order, together with a bound `edge`: every entry it did not list has a key below
// edge.  The selection kernel (topk_select.hip) then takes the k-th largest key K of the
// union of a query's lists.  If every chunk's edge is at most K, the union holds the whole
// top k (an unlisted entry scores below K, and k listed keys are >= K): those are the
// union's keys >= K, in index order (chunks are index ranges, each list is in index
// order).  Otherwise (the best entries cluster in a few chunks) it selects from the group
// maxima and scores that every chunk also wrote.
#pragma once

#include "indexer.hpp"

namespace csahca {

constexpr int FT_NT = 256;                    // threads per workgroup
constexpr int FT_NW = FT_NT / 64;
constexpr int FT_LKPT = SCORE_STAGE / FT_NT;  // chunk keys per thread

// LDS of the cut, laid over the scoring kernel's key ring once the key loop is done
struct FtScratch {
  uint32_t hist[FT_NT];              // one 8-bit digit
  uint32_t jw[FT_LKPT * FT_NW];      // per (j, wave) counts, then their exclusive prefix
  uint32_t red_and[FT_NW], red_or[FT_NW];
  uint32_t scan[FT_NW];
  uint32_t first[FT_NW];
  uint32_t total, found_count, found_bin;
};

// ---------------------------------------------------------------------------------------
// block-wide helpers (FT_NT threads; every thread calls them)
// ---------------------------------------------------------------------------------------
// Workgroup barrier for LDS traffic only: this wave's LDS operations have completed, then
// s_barrier.  __syncthreads would also wait for the wave's outstanding global stores (the
// chunk's scores, just issued), which nothing here reads back.
CSAHCA_DEV void ft_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

CSAHCA_DEV int ft_lane() { return threadIdx.x & 63; }
CSAHCA_DEV int ft_wave() { return threadIdx.x >> 6; }

// exclusive prefix over FT_NT threads of one count each, and the total
CSAHCA_DEV uint32_t ft_block_scan(uint32_t c, uint32_t& total, FtScratch& sc) {
  const uint32_t incl = wave_incl_scan(c);
  if (ft_lane() == 63) sc.scan[ft_wave()] = incl;
  ft_barrier();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < FT_NW; ++w) {
    before += w < ft_wave() ? sc.scan[w] : 0u;
    all += sc.scan[w];
  }
  ft_barrier();
  total = all;
  return before + incl - c;
}

// Write out, in slot order (j, thread), every key with pred set: slot j of thread t is
// position t + FT_NT*j of the sequence.  Returns how many were written (uniform).
template <int KP, typename Pred, typename Sink>
CSAHCA_DEV uint32_t ft_compact(const uint64_t (&kr)[KP], Pred pred, Sink sink, FtScratch& sc) {
  static_assert(KP * FT_NW <= FT_LKPT * FT_NW, "the (j, wave) counts fit the scratch");
  static_assert(KP * FT_NW <= 4 * 64, "one wave scans the (j, wave) counts, at most four per lane");
  uint64_t bal[KP];
#pragma unroll
  for (int j = 0; j < KP; ++j) {
    bal[j] = __ballot(pred(kr[j]));
    if (ft_lane() == 0) sc.jw[j * FT_NW + ft_wave()] = (uint32_t)__popcll(bal[j]);
  }
  ft_barrier();
  if (ft_wave() == 0) {
    constexpr int PER = (KP * FT_NW + 63) / 64;
    uint32_t c[PER], sum = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int x = ft_lane() * PER + i;
      c[i] = x < KP * FT_NW ? sc.jw[x] : 0u;
      sum += c[i];
    }
    const uint32_t incl = wave_incl_scan(sum);
    uint32_t run = incl - sum;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int x = ft_lane() * PER + i;
      if (x < KP * FT_NW) sc.jw[x] = run;
      run += c[i];
    }
    if (ft_lane() == 63) sc.total = incl;
  }
  ft_barrier();
  // this wave's offsets, read before any sink writes (which may alias them for the
  // compiler: each read would wait for the writes before it)
  uint32_t off[KP];
#pragma unroll
  for (int j = 0; j < KP; ++j) off[j] = sc.jw[j * FT_NW + ft_wave()];
#pragma unroll
  for (int j = 0; j < KP; ++j) {
    if ((bal[j] >> ft_lane()) & 1ull) {
      const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal[j] >> 32),
                                                       __builtin_amdgcn_mbcnt_lo((uint32_t)bal[j], 0u));
      sink(off[j] + below, kr[j]);
    }
  }
  const uint32_t total = sc.total;
  ft_barrier();
  return total;
}

// ---------------------------------------------------------------------------------------
// 1. the chunk's cut
// ---------------------------------------------------------------------------------------
// u[j]: 32-bit score key of the chunk's entry threadIdx.x + FT_NT*j, 0 if none (a finite
// score never maps to 0); LKPT keys per thread cover the chunk.  Returns the cut as a
// 33-bit bound: the listed keys are those with u >= cut; 0 lists every entry.  count: how
// many are listed.
struct FtCut {
  uint64_t cut;
  uint32_t count;
};

template <int LKPT>
CSAHCA_DEV FtCut ft_local_cut(const uint32_t (&u)[LKPT], int n, int JT, int JMAX, FtScratch& sc) {
  static_assert(LKPT <= FT_LKPT, "a chunk holds at most SCORE_STAGE keys");
  if (n <= JMAX) return {0ull, (uint32_t)n};
  uint32_t a = ~0u, o = 0u;
#pragma unroll
  for (int j = 0; j < LKPT; ++j)
    if (u[j]) {
      a &= u[j];
      o |= u[j];
    }
  a = wave_and(a);
  o = wave_or(o);
  if (ft_lane() == 0) {
    sc.red_and[ft_wave()] = a;
    sc.red_or[ft_wave()] = o;
  }
  ft_barrier();
  a = ~0u;
  o = 0u;
#pragma unroll
  for (int w = 0; w < FT_NW; ++w) {
    a &= sc.red_and[w];
    o |= sc.red_or[w];
  }
  ft_barrier();
  if (a == o) return {(uint64_t)a + 1, 0u};  // all equal: no cut separates them
  int hb = 31 - __builtin_clz(a ^ o);          // highest bit on which the keys differ
  uint32_t prefix = a & (hb == 31 ? 0u : ~0u << (hb + 1));
  uint32_t above = 0;                          // keys above the current range
  for (;;) {
    const int lo = hb >= 7 ? hb - 7 : 0;
    const uint32_t dmask = (2u << (hb - lo)) - 1u;  // digit: bits lo .. hb
    const uint32_t hmask = hb == 31 ? 0u : ~0u << (hb + 1);
    sc.hist[threadIdx.x] = 0u;  // FT_NT == 256 bins
    ft_barrier();
#pragma unroll
    for (int j = 0; j < LKPT; ++j)
      if (u[j] && (u[j] & hmask) == prefix) atomicAdd(&sc.hist[(u[j] >> lo) & dmask], 1u);
    ft_barrier();
    // thread t owns digit 255 - t: cum = keys whose digit is >= it, plus those above
    const uint32_t c = sc.hist[255 - threadIdx.x];
    uint32_t tot;
    const uint32_t cum = ft_block_scan(c, tot, sc) + c + above;
    // the largest digit D with cum(D) >= JT: the first thread whose cum reaches JT
    const uint64_t hit = __ballot(cum >= (uint32_t)JT);
    if (ft_lane() == 0) sc.first[ft_wave()] = hit ? (uint32_t)(ft_wave() * 64 + __builtin_ctzll(hit)) : 0xFFFFu;
    ft_barrier();
    uint32_t tf = 0xFFFFu;
#pragma unroll
    for (int w = 0; w < FT_NW; ++w) tf = min(tf, sc.first[w]);
    if (threadIdx.x == tf) {
      sc.found_count = cum;
      sc.found_bin = c;
    }
    ft_barrier();
    const uint32_t D = 255u - tf, cD = sc.found_count, hD = sc.found_bin;
    ft_barrier();
    if (cD <= (uint32_t)JMAX) return {(uint64_t)(prefix | (D << lo)), cD};
    if (lo == 0) return {(uint64_t)(prefix | D) + 1, cD - hD};  // one key value: list those above
    above = cD - hD;
    prefix |= D << lo;
    hb = lo - 1;
  }
}

}  // namespace csahca
