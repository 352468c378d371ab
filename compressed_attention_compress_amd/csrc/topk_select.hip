// Kernel 2b: exact top-k selection over the lightning-indexer scores.
//
// Source: "DeepSeek-V4 Hybrid Attention: CSA, HCA, mHC, MoE", section V.2 (the selector
// keeps the k best blocks by index score); "DeepSeek-V4: Anatomy of an Open-Source
// Frontier Model" (lesson 6.7): no more entries than exist can be picked.
//
// Selection: one workgroup per query.  Selection keys are
// (order-preserving score bits << 32) | (~index), so all keys are distinct and "larger
// key" means "better, lower index on ties".  A group of 16 entries is keyed by its maximum
// score, then by the lower group index (groups are index ranges, so this orders equal
// maxima as their best entries are ordered).  Let T1 be the K-th largest group key and s1
// its score.  The K selected groups hold K entries whose keys beat every entry of an
// unselected group, so every top-K entry lies in a selected group and scores at least s1.
// The exact top-K is then taken from the entries of those K groups that score >= s1.
// Both K-th-largest searches are MSB-first radix selects over register-resident keys (an
// LDS histogram per 11-bit digit) that skip the bits all remaining candidates share and
// rank the last few candidates directly.  The candidates are kept in index order, so the
// output comes out ascending without a sort.
#include "indexer.hpp"

namespace {

using namespace csahca;

// ---------------------------------------------------------------------------------------
// selection
// ---------------------------------------------------------------------------------------
constexpr int DBITS = 11;                // radix digit
constexpr int NBIN = 1 << DBITS;
constexpr int BPT = NBIN / SEL_THREADS;  // digits each thread scans
constexpr int NWAVE = SEL_THREADS / 64;

struct SelScratch {
  uint32_t hist[2][NBIN];
  uint32_t jw[KPT * NWAVE];  // per (j, wave) counts, then their exclusive prefix
  uint64_t red_and[NWAVE];
  uint64_t red_or[NWAVE];
  uint32_t scan[NWAVE];
  uint32_t total;
  uint32_t found_digit;
  uint32_t found_kth;
  uint32_t found_count;
  uint64_t result;
};

// K-th largest (1-based) of the distinct nonzero keys the workgroup holds in registers
// (KPT per thread; 0 = empty).  One AND/OR reduction finds the highest bit on which the
// keys differ; from there MSB-first radix passes of 11 bits narrow the candidates.  A
// pass builds an LDS histogram of the digit, then every wave scans 128 digits (two per
// lane, in descending order) and the lane whose range holds the K-th key reports the
// digit.  The search stops as soon as that digit holds a single candidate.  (All 1024
// threads run on one CU, so every phase costs its instruction count times 16 cycles:
// a second pass is cheaper than gathering and ranking even a hundred keys.)
CSAHCA_DEV uint64_t radix_select_kth(const uint64_t (&kr)[KPT], int kth, SelScratch& sc) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t alo = ~0u, ahi = ~0u, olo = 0u, ohi = 0u;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    if (kr[j] != 0ull) {
      alo &= (uint32_t)kr[j];
      ahi &= (uint32_t)(kr[j] >> 32);
      olo |= (uint32_t)kr[j];
      ohi |= (uint32_t)(kr[j] >> 32);
    }
  }
  alo = wave_and(alo);
  ahi = wave_and(ahi);
  olo = wave_or(olo);
  ohi = wave_or(ohi);
  if (lane == 0) {
    sc.red_and[wave] = ((uint64_t)ahi << 32) | alo;
    sc.red_or[wave] = ((uint64_t)ohi << 32) | olo;
  }
  for (int i = threadIdx.x; i < 2 * NBIN; i += SEL_THREADS) (&sc.hist[0][0])[i] = 0u;
  __syncthreads();
  uint64_t a = ~0ull, o = 0ull;
#pragma unroll
  for (int i = 0; i < NWAVE; ++i) {
    a &= sc.red_and[i];
    o |= sc.red_or[i];
  }
  const uint64_t diff = a ^ o;
  if (diff == 0ull) return a;  // a single key
  const int hb = 63 - __builtin_clzll(diff);
  // bits above hb are common to every key
  uint64_t mask = hb == 63 ? 0ull : (~0ull << (hb + 1));
  uint64_t prefix = a & mask;
  int buf = 0;
#ifdef CSAHCA_TRACE_ENABLED
  if (threadIdx.x == 0 && blockIdx.x < 8192) csahca_trace[blockIdx.x * 16 + 5] += 1ull << (8 * (hb / 11));
  const int tslot = csahca_trace[blockIdx.x * 16 + 6] == 0 ? 7 : 10;
  CSAHCA_TRACE(tslot);
  bool tfirst = true;
#endif
  for (int sh = hb >= DBITS - 1 ? hb - (DBITS - 1) : 0;; sh = sh >= DBITS ? sh - DBITS : 0) {
    uint32_t* h = sc.hist[buf];
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const uint64_t k = kr[j];
      if (k != 0ull && (k & mask) == prefix) atomicAdd(&h[(uint32_t)(k >> sh) & (NBIN - 1)], 1u);
    }
    for (int i = threadIdx.x; i < NBIN; i += SEL_THREADS) sc.hist[buf ^ 1][i] = 0u;
    __syncthreads();
#ifdef CSAHCA_TRACE_ENABLED
    if (threadIdx.x == 0 && blockIdx.x < 8192 && tfirst)
      csahca_trace[blockIdx.x * 16 + tslot + 1] = __builtin_amdgcn_s_memtime();
#endif
    // this lane's BPT digits, descending with the thread index
    const int d_hi = NBIN - 1 - BPT * (int)threadIdx.x;
    uint32_t c[BPT], csum = 0;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      c[i] = h[d_hi - i];
      csum += c[i];
    }
    const uint32_t incl = wave_incl_scan(csum);
    if (lane == 63) sc.scan[wave] = incl;
    __syncthreads();
    uint32_t above = incl - csum;
#pragma unroll
    for (int i = 0; i < NWAVE; ++i) above += i < wave ? sc.scan[i] : 0u;
    const uint32_t kk = (uint32_t)kth;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      if (above < kk && kk <= above + c[i]) {
        sc.found_digit = d_hi - i;
        sc.found_kth = kk - above;
        sc.found_count = c[i];
      }
      above += c[i];
    }
    __syncthreads();
#ifdef CSAHCA_TRACE_ENABLED
    if (threadIdx.x == 0 && blockIdx.x < 8192) {
      if (tfirst) csahca_trace[blockIdx.x * 16 + tslot + 2] = __builtin_amdgcn_s_memtime();
      csahca_trace[blockIdx.x * 16 + 6] += 1;
    }
    tfirst = false;
#endif
    const uint64_t dsel = sc.found_digit;
    kth = (int)sc.found_kth;
    const uint32_t count = sc.found_count;
    prefix = (prefix & ~((uint64_t)(NBIN - 1) << sh)) | (dsel << sh);
    mask |= (uint64_t)(NBIN - 1) << sh;
    if (sh == 0) return prefix;  // every bit decided
    if (count == 1) {            // the K-th key is the only candidate left
#pragma unroll
      for (int j = 0; j < KPT; ++j)
        if (kr[j] != 0ull && (kr[j] & mask) == prefix) sc.result = kr[j];
      __syncthreads();
      const uint64_t r = sc.result;
      __syncthreads();
      return r;
    }
    buf ^= 1;
  }
}

__global__ __launch_bounds__(SEL_THREADS) void select_topk(
    const float* __restrict__ scores, const uint32_t* __restrict__ gmax,
    const int* __restrict__ q_pos, int m, int Tq, int N_c, int NG, int k,
    int* __restrict__ topk_idx, float* __restrict__ topk_score) {
  __shared__ SelScratch sc;
  __shared__ int glist[MAX_K];
  static_assert(KPT * NWAVE == 4 * 64, "one wave scans the per-(j, wave) counts");
  static_assert(NWAVE * 64 == MAX_K, "one listed group per 16 lanes per key slot");
  CSAHCA_TRACE(0);
  CSAHCA_TRACE_RT(14);
  const int q = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // group maxima, coalesced: thread t holds groups j*SEL_THREADS + t (j < KPT); issued
  // before the visible count is known, masked afterwards.  A group's key is its maximum
  // score key, then the lower group index: as groups are index ranges, that orders equal
  // maxima as their best entries are ordered.
  const uint32_t* grow = gmax + (size_t)q * NG;
  uint64_t kr[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int gi = j * SEL_THREADS + (int)threadIdx.x;
    kr[j] = gi < NG ? ((uint64_t)grow[gi] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)gi) : 0ull;
  }
  const int b = q / Tq, t = q - b * Tq;
  const int V = visible_entries(q_pos, b, t, m, N_c);
  const int keff = min(k, V);
  const float* srow = scores + (size_t)q * N_c;
  int* orow = topk_idx + (size_t)q * k;
  float* osc = topk_score ? topk_score + (size_t)q * k : nullptr;

  if (keff == V) {  // everything usable is selected
    for (int i = threadIdx.x; i < k; i += SEL_THREADS) {
      orow[i] = i < V ? i : -1;
      if (osc) osc[i] = i < V ? srow[i] : -INFINITY;
    }
    return;
  }
  const int ng = cdiv(V, GROUP);
#pragma unroll
  for (int j = 0; j < KPT; ++j)
    if (j * SEL_THREADS + (int)threadIdx.x >= ng) kr[j] = 0ull;  // not (yet) complete groups
  // With fewer groups than K every group is a candidate (T1 = 0 keeps every usable key).
  const uint64_t T1 = keff < ng ? radix_select_kth(kr, keff, sc) : 0ull;
  // entries scoring below the T1 group's maximum cannot be among the top K
  const uint64_t T1s = T1 & 0xFFFFFFFF00000000ull;
  CSAHCA_TRACE(1);

  // exactly min(K, ng) groups have a maximum >= T1; list them in index order, which is
  // (j, wave, lane) order: per-(j, wave) counts by ballot, one scan over them
  uint32_t ngl;
  {
    uint64_t bal[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      bal[j] = __ballot(kr[j] != 0ull && kr[j] >= T1);
      if (lane == 0) sc.jw[j * NWAVE + wave] = (uint32_t)__popcll(bal[j]);
    }
    __syncthreads();
    if (wave == 0) {  // exclusive scan of the KPT*NWAVE counts, four per lane
      uint32_t c4[4], sum = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c4[i] = sc.jw[4 * lane + i];
        sum += c4[i];
      }
      const uint32_t incl = wave_incl_scan(sum);
      uint32_t run = incl - sum;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sc.jw[4 * lane + i] = run;
        run += c4[i];
      }
      if (lane == 63) sc.total = incl;
    }
    __syncthreads();
    ngl = sc.total;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      if ((bal[j] >> lane) & 1ull) {
        const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal[j] >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((uint32_t)bal[j], 0u));
        glist[sc.jw[j * NWAVE + wave] + below] = j * SEL_THREADS + (int)threadIdx.x;
      }
    }
    __syncthreads();
  }
  CSAHCA_TRACE(2);
  // candidates, coalesced: 16 lanes read the 16 scores of one listed group; key j of lane
  // (wave, lane) is element lane%16 of listed group wave*64 + j*4 + lane/16.  Every load
  // is issued (clamped to valid memory) before any is used, so they overlap.
  int ce[KPT];
  float cv[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int gp = wave * 64 + j * 4 + (lane >> 4);
    ce[j] = gp < (int)ngl ? glist[gp] * GROUP + (lane & 15) : V;
    cv[j] = srow[min(ce[j], N_c - 1)];
  }
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const uint64_t key = ce[j] < V ? entry_key(cv[j], (uint32_t)ce[j]) : 0ull;
    kr[j] = key >= T1s ? key : 0ull;
  }
  const uint64_t T2 = radix_select_kth(kr, keff, sc);
  CSAHCA_TRACE(3);
  {
    // candidate rank (index order) is wave*1024 + j*64 + lane: running count per wave
    uint32_t off[KPT];
    uint32_t run = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const uint64_t bl = __ballot(kr[j] != 0ull && kr[j] >= T2);
      off[j] = run + __builtin_amdgcn_mbcnt_hi((uint32_t)(bl >> 32),
                                               __builtin_amdgcn_mbcnt_lo((uint32_t)bl, 0u));
      run += (uint32_t)__popcll(bl);
    }
    if (lane == 0) sc.scan[wave] = run;
    __syncthreads();
    uint32_t before = 0;
#pragma unroll
    for (int i = 0; i < NWAVE; ++i) before += i < wave ? sc.scan[i] : 0u;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const uint64_t key = kr[j];
      if (key != 0ull && key >= T2) {
        orow[before + off[j]] = (int)key_index(key);
        if (osc) osc[before + off[j]] = key_score((uint32_t)(key >> 32));
      }
    }
  }
  for (int i = keff + threadIdx.x; i < k; i += SEL_THREADS) {
    orow[i] = -1;
    if (osc) osc[i] = -INFINITY;
  }
  CSAHCA_TRACE(4);
  CSAHCA_TRACE_RT(15);
}

}  // namespace

namespace csahca {

int index_select_impl(const float* scores, const uint32_t* gmax, const int* q_pos, int m, int B,
                      int Tq, int N_c, int k, int* topk_idx, float* topk_score, hipStream_t st) {
  using namespace csahca;
  const int nq = B * Tq;
  const int NG = cdiv(N_c, GROUP);
  hipLaunchKernelGGL(select_topk, dim3((unsigned)nq), dim3(SEL_THREADS), 0, st, scores,
                     gmax, q_pos, m, Tq, N_c, NG, k, topk_idx, topk_score);
  return launch_status("lightning_index_select");
}

}  // namespace csahca

extern "C" size_t lightning_index_topk_workspace_size(int B, int Tq, int n_ih, int N_c, int k) {
  (void)n_ih;
  (void)k;
  if (B < 1 || Tq < 1 || N_c < 1) return 0;
  return ws_layout((long long)B * Tq, N_c).total;
}

extern "C" int lightning_index_select(const float* scores, const int* q_pos, int m, int B,
                                      int Tq, int N_c, int k, int* topk_idx, float* topk_score,
                                      void* workspace, size_t ws_bytes, void* stream) {
  using namespace csahca;
  if (!scores || !q_pos || !topk_idx)
    return fail(CSAHCA_EINVAL, "lightning_index_select: scores, q_pos and topk_idx must be non-NULL");
  if (B < 1 || Tq < 1 || N_c < 1 || m < 1 || k < 1)
    return fail(CSAHCA_EINVAL, "lightning_index_select: B, Tq, N_c, m and k must be >= 1");
  if (N_c > MAX_NC || k > MAX_K)
    return fail(CSAHCA_ENOTSUP, "lightning_index_select: N_c <= 262144 and k <= 1024 are built");
  const WsLayout L = ws_layout((long long)B * Tq, N_c);
  if (!workspace || ws_bytes < L.total)
    return fail(CSAHCA_EWORKSPACE, "lightning_index_select: workspace missing or too small");
  return index_select_impl(scores, (const uint32_t*)((char*)workspace + L.gkeys_off), q_pos, m, B, Tq,
                     N_c, k, topk_idx, topk_score, (hipStream_t)stream);
}

extern "C" int lightning_index_topk(const void* q_idx, const float* w_idx, const void* k_idx,
                                    int idx_dtype, const int* q_pos, int m, int B, int Tq,
                                    int n_ih, int c_I, int N_c, int k, int* topk_idx,
                                    float* topk_score, float* all_scores, void* workspace,
                                    size_t ws_bytes, void* stream) {
  using namespace csahca;
  int st = index_check_common(q_idx, w_idx, k_idx, idx_dtype, q_pos, m, B, Tq, n_ih, c_I, N_c, k);
  if (st != CSAHCA_OK) return st;
  if (!topk_idx) return fail(CSAHCA_EINVAL, "lightning_index_topk: topk_idx must be non-NULL");
  const WsLayout L = ws_layout((long long)B * Tq, N_c);
  if (!workspace || ws_bytes < L.total)
    return fail(CSAHCA_EWORKSPACE, "lightning_index_topk: workspace missing or too small");
  if (all_scores && !aligned16(all_scores))
    return fail(CSAHCA_EINVAL, "lightning_index_topk: all_scores must be 16-byte aligned");
  float* scores = all_scores ? all_scores : (float*)((char*)workspace + L.scores_off);
  uint32_t* gkeys = (uint32_t*)((char*)workspace + L.gkeys_off);
  hipStream_t s = (hipStream_t)stream;
  st = index_score_impl(q_idx, w_idx, k_idx, idx_dtype, q_pos, m, B, Tq, n_ih, c_I, N_c, scores, gkeys, s);
  if (st != CSAHCA_OK) return st;
  return index_select_impl(scores, gkeys, q_pos, m, B, Tq, N_c, k, topk_idx, topk_score, s);
}

