// Kernel 2b: exact top-k selection over the lightning-indexer scores.
//
// Source: "DeepSeek-V4 Hybrid Attention: CSA, HCA, mHC, MoE", section V.2 (the selector
// keeps the k best blocks by index score); "DeepSeek-V4: Anatomy of an Open-Source
// Frontier Model" (lesson 6.7): no more entries than exist can be picked.
//
// Selection: one workgroup per query, or, without chunk lists when k <= 512 and there are
// at most 5120 groups (a prefill chunk), one wave per query (the second kernel below: the
// same two thresholds found by bisection).  Selection keys are
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
#include <mutex>

#include "indexer.hpp"
#include "pool.hpp"
#include "pool_device.hpp"

namespace {

using namespace csahca;

// ---------------------------------------------------------------------------------------
// selection (one workgroup of SEL_THREADS threads per query)
// ---------------------------------------------------------------------------------------
constexpr int DBITS = 11;                // radix digit
constexpr int NBIN = 1 << DBITS;
constexpr int BPT = NBIN / SEL_THREADS;  // digits each thread scans
constexpr int NWAVE = SEL_THREADS / 64;
constexpr int SEL_COMPACT = 4096;        // list keys compacted into LDS for the k-th search
constexpr int CPT = SEL_COMPACT / SEL_THREADS;
static_assert(NWAVE * KPT * 64 / GROUP == MAX_K, "the candidate gather holds k groups");
static_assert(FT_MAX_P <= 128 && SEL_THREADS >= 128, "the bounds are read by the first two waves");

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
// (KP per thread; 0 = empty).  One AND/OR reduction finds the highest bit on which the
// keys differ; from there MSB-first radix passes of 11 bits narrow the candidates.  A
// pass builds an LDS histogram of the digit, then every thread scans BPT digits (in
// descending order) and the thread whose range holds the K-th key reports the digit.  The
// search stops as soon as that digit holds a single candidate.
//
// With RANGE the caller passes bounds lo <= every key <= hi instead (and has zeroed both
// histograms, sc.hist): the keys share the bits above the highest bit where lo and hi
// differ, so the AND/OR reduction is skipped.
template <int KP, bool RANGE = false>
CSAHCA_DEV uint64_t radix_select_kth(const uint64_t (&kr)[KP], int kth, SelScratch& sc,
                                     uint64_t lo = 0ull, uint64_t hi = 0ull) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint64_t a = lo, o = hi;
  if constexpr (!RANGE) {
    uint32_t alo = ~0u, ahi = ~0u, olo = 0u, ohi = 0u;
#pragma unroll
    for (int j = 0; j < KP; ++j) {
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
    a = ~0ull;
    o = 0ull;
#pragma unroll
    for (int i = 0; i < NWAVE; ++i) {
      a &= sc.red_and[i];
      o |= sc.red_or[i];
    }
    __syncthreads();
  }
  const uint64_t diff = a ^ o;
  if (diff == 0ull) return a;  // a single key (with RANGE: lo == hi)
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
    for (int j = 0; j < KP; ++j) {
      const uint64_t k = kr[j];
      if (k != 0ull && (k & mask) == prefix) atomicAdd(&h[(uint32_t)(k >> sh) & (NBIN - 1)], 1u);
    }
    for (int i = threadIdx.x; i < NBIN; i += SEL_THREADS) sc.hist[buf ^ 1][i] = 0u;
    __syncthreads();
#ifdef CSAHCA_TRACE_ENABLED
    if (threadIdx.x == 0 && blockIdx.x < 8192 && tfirst)
      csahca_trace[blockIdx.x * 16 + tslot + 1] = __builtin_amdgcn_s_memtime();
#endif
    // this thread's BPT digits, descending with the thread index
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
    if (sh == 0) {  // every bit decided
      __syncthreads();
      return prefix;
    }
    if (count == 1) {  // the K-th key is the only candidate left
#pragma unroll
      for (int j = 0; j < KP; ++j)
        if (kr[j] != 0ull && (kr[j] & mask) == prefix) sc.result = kr[j];
      __syncthreads();
      const uint64_t r = sc.result;
      __syncthreads();
      return r;
    }
    buf ^= 1;
  }
}

// Hands every key of kr for which pred holds to sink(position, key, j), positions counted
// in the order (j, wave, lane) when JMAJOR, else (wave, j, lane); returns their number.
// Two ballot rounds (counts, then positions), so no ballot is held in registers.
template <int KP, bool JMAJOR, typename Pred, typename Sink>
CSAHCA_DEV uint32_t compact_in_order(const uint64_t (&kr)[KP], Pred pred, Sink sink, SelScratch& sc) {
  static_assert(KP * NWAVE <= 4 * 64, "one wave scans the (j, wave) counts, four per lane");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < KP; ++j) {
    const uint64_t bal = __ballot(pred(kr[j]));
    if (lane == 0) sc.jw[JMAJOR ? j * NWAVE + wave : wave * KP + j] = (uint32_t)__popcll(bal);
  }
  __syncthreads();
  if (wave == 0) {
    constexpr int N = KP * NWAVE, PER = (N + 63) / 64;
    uint32_t c[PER], sum = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int x = lane * PER + i;
      c[i] = x < N ? sc.jw[x] : 0u;
      sum += c[i];
    }
    const uint32_t incl = wave_incl_scan(sum);
    uint32_t run = incl - sum;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int x = lane * PER + i;
      if (x < N) sc.jw[x] = run;
      run += c[i];
    }
    if (lane == 63) sc.total = incl;
  }
  __syncthreads();
  // this wave's KP offsets, read before any sink writes (which the compiler cannot tell
  // apart from the offsets: each read would wait for the writes before it)
  uint32_t off[KP];
#pragma unroll
  for (int j = 0; j < KP; ++j) off[j] = sc.jw[JMAJOR ? j * NWAVE + wave : wave * KP + j];
#pragma unroll
  for (int j = 0; j < KP; ++j) {
    const bool p = pred(kr[j]);
    const uint64_t bal = __ballot(p);
    if (p)
      sink(off[j] + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u)),
           kr[j], j);
  }
  const uint32_t total = sc.total;
  __syncthreads();
  return total;
}

// Every key of kr that is >= T, written out in the order (j, wave, lane) when JMAJOR, else
// (wave, j, lane) (the callers make that the index order); then the padding up to k.
template <int KP, bool JMAJOR>
CSAHCA_DEV void write_selected(const uint64_t (&kr)[KP], uint64_t T, int keff, int k, int* orow,
                               float* osc, SelScratch& sc) {
  compact_in_order<KP, JMAJOR>(
      kr, [&](uint64_t key) { return key != 0ull && key >= T; },
      [&](uint32_t pos, uint64_t key, int) {
        orow[pos] = (int)key_index(key);
        if (osc) osc[pos] = key_score((uint32_t)(key >> 32));
      },
      sc);
  for (int i = keff + threadIdx.x; i < k; i += SEL_THREADS) {
    orow[i] = -1;
    if (osc) osc[i] = -INFINITY;
  }
}

// With chunk lists (decode; fused_topk.hpp) the selection first takes the k-th largest key
// K of the union of the query's lists: if no chunk left out an entry at or above K, the
// union's keys >= K are the top k.  Otherwise, and without lists, it selects through the
// group maxima as described at the top of this file.
// KP is the number of keys a thread holds: KPT in general; 8 for a selection without lists
// with k <= 512 and at most 8192 groups (a prefill chunk), which holds a thread to 64
// registers, so that two workgroups share a compute unit.  LKP (0: no lists) is the number
// of list slots a thread holds, the smallest power of two with P * JMAX <= SEL_THREADS * LKP,
// so that no loop of the list path runs over slots that no chunk can fill.
// Workgroups past the queries (the list selection only) pool a decode step's new CSA
// blocks instead, with csa_compress's arithmetic (one thread per 8-channel slice of an
// entry; with pb.norm, csahca_compress_norm_rope's), then normalise the step's window rows
// as csahca_norm_rope does.
template <int KP, int LKP>
__global__ __launch_bounds__(SEL_THREADS, KP == KPT ? 1 : 8) void select_topk(
    const float* __restrict__ scores, const uint32_t* __restrict__ gmax,
    const int* __restrict__ q_pos, int m, int Tq, int N_c, int NG, int k,
    int* __restrict__ topk_idx, float* __restrict__ topk_score, ChunkLists cl, int nq,
    PoolBeside pb) {
  if constexpr (LKP > 0) if ((int)blockIdx.x >= nq) {
    const int w = (int)blockIdx.x - nq;
    const AppendRows ap0{nullptr, nullptr, 1, 0, 0, 0};
    if (w < pb.pool_wgs) {
      if (pb.norm)
        pool_items<uint16_t, 4, false, PLAIN, true>(pb.X, pb.Z, nullptr, nullptr, nullptr, pb.out, pb.N, pb.c,
                                                    pb.m, 0, pb.in_bs, pb.out_bs, pb.total, pb.nr, pb.entry0,
                                                    ap0, w);
      else
        pool_items<uint16_t, 4, false, PLAIN, false>(pb.X, pb.Z, nullptr, nullptr, nullptr, pb.out, pb.N,
                                                     pb.c, pb.m, 0, pb.in_bs, pb.out_bs, pb.total,
                                                     NormRope{nullptr, 0.f, 1.f, 0, 0}, 0, ap0, w);
      return;
    }
    const int CV = pb.c / VEC;
    const long long item = (long long)(w - pb.pool_wgs) * blockDim.x + threadIdx.x;
    const long long row = item / CV;
    if (row >= pb.rows) return;  // whole rows leave together (CV divides 64)
    const int cv = (int)(item - row * CV);
    const int b = (int)(row / pb.rT), t = (int)(row - (long long)b * pb.rT);
    const long long p = (pb.rpos ? (long long)pb.rpos[b] : 0LL) + t;
    const NormRope nx{pb.nr.gamma, pb.nr.eps, pb.nr.theta, pb.nr.d, 1};
    norm_rope_row8<uint16_t>(pb.rx + b * pb.rx_bs + (long long)t * pb.c, pb.ry + b * pb.ry_bs + (long long)t * pb.c,
                             nx, p, cv, CV, pb.c);
    return;
  }
  __shared__ SelScratch sc;
  __shared__ int glist[MAX_K];
  CSAHCA_TRACE(0);
  CSAHCA_TRACE_RT(14);
  const int q = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = q / Tq, t = q - b * Tq;
  const int V = visible_entries(q_pos, b, t, m, N_c);
  const int keff = min(k, V);
  const float* srow = scores + (size_t)q * N_c;
  int* orow = topk_idx + (size_t)q * k;
  float* osc = topk_score ? topk_score + (size_t)q * k : nullptr;
  // With lists: every slot and bound of the query's lists is loaded together with its
  // ready word and the position (all of it is workspace memory), and masked to the usable
  // chunks once the position has arrived: chunks past the usable entries wrote nothing in
  // this call.  Thread (wave, lane) holds slots wave * 64 LKP + 64 j + lane.
  constexpr int LK = LKP > 0 ? LKP : 1;
  uint64_t lk[LK];
  uint64_t e = 0ull;
  uint32_t ready = 0u;
  if (LKP > 0 && cl.cand) {
    const uint64_t* cq = cl.cand + (size_t)q * cl.P * cl.JMAX;
    const int nall = cl.P * cl.JMAX;
    ready = cl.path[q];
    e = (int)threadIdx.x < cl.P ? cl.edge[(size_t)q * FT_MAX_P + threadIdx.x] : 0ull;
#pragma unroll
    for (int j = 0; j < LK; ++j) {
      const int s = wave * 64 * LK + 64 * j + lane;
      lk[j] = s < nall ? cq[s] : 0ull;
    }
  }

  if (keff == V) {  // everything usable is selected
    for (int i = threadIdx.x; i < k; i += SEL_THREADS) {
      orow[i] = i < V ? i : -1;
      if (osc) osc[i] = i < V ? srow[i] : -INFINITY;
    }
    if (cl.path && threadIdx.x == 0) cl.path[q] = FT_PATH_ALL;
    return;
  }
  constexpr int GPWk = KP * 64 / GROUP;  // listed groups per wave in the candidate gather
  uint64_t kr[KP];
  if constexpr (LKP > 0) if (cl.cand) {
    static_assert(LKP <= KPT, "the list slots fit the selection's registers");
    __shared__ uint64_t s_keys[SEL_COMPACT];
    // The union: slot s = chunk * JMAX + position (lists are padded with zero keys), held
    // so that (wave, j, lane) order is slot order, which is index order (chunks are index
    // ranges, each list is in index order).  The lists give the top k exactly when K, their
    // k-th largest key, is at least every chunk's bound E; so only keys >= max E matter,
    // and if fewer than k remain, the lists cannot decide.
    // (a thread may see its own workgroup's FT_PATH_GROUPS below instead of the old word:
    // either way not FT_LISTS_READY, so every thread takes the same branch)
    CSAHCA_TRACE(1);
    if (ready == FT_LISTS_READY) {
      const int P_eff = cdiv(V, cl.CH);
      const int nslots = P_eff * cl.JMAX;
      if ((int)threadIdx.x >= P_eff) e = 0ull;
#pragma unroll
      for (int j = 0; j < LKP; ++j)
        if (wave * 64 * LKP + 64 * j + lane >= nslots) lk[j] = 0ull;
      // the histograms of the k-th search are cleared while the loads are in flight
      for (int i = threadIdx.x; i < 2 * NBIN; i += SEL_THREADS) (&sc.hist[0][0])[i] = 0u;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) e = umax64(e, shfl_xor_u64(e, d));
      if (lane == 0) sc.red_or[wave] = e;
      __syncthreads();
      const uint64_t emax = umax64(sc.red_or[0], sc.red_or[1]);
      uint64_t kmax = 0ull;
#pragma unroll
      for (int j = 0; j < LKP; ++j) {
        lk[j] = lk[j] >= emax ? lk[j] : 0ull;
        kmax = umax64(kmax, lk[j]);
      }
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) kmax = umax64(kmax, shfl_xor_u64(kmax, d));
      if constexpr (LKP <= 8) {
        // Few slots per thread: the k-th search and the write run on the registers
        // themselves, with one barrier for the count of kept keys and their maximum.
        // (The counts sit in sc.scan, which the k-th search writes only after its first
        // barrier, and the write-out's compaction does not touch.)
        uint32_t cnt = 0;
#pragma unroll
        for (int j = 0; j < LKP; ++j) cnt += (uint32_t)__popcll(__ballot(lk[j] != 0ull));
        if (lane == 0) {
          sc.red_and[wave] = kmax;
          sc.scan[wave] = cnt;
        }
        __syncthreads();
        uint32_t total = 0;
#pragma unroll
        for (int i = 0; i < NWAVE; ++i) {
          kmax = umax64(kmax, sc.red_and[i]);
          total += sc.scan[i];
        }
        CSAHCA_TRACE(2);
        if (total >= (uint32_t)keff) {
          // every kept key lies in [emax (or 1 when every chunk listed everything), kmax]
          const uint64_t K = radix_select_kth<LKP, true>(lk, keff, sc, emax ? emax : 1ull, kmax);
          CSAHCA_TRACE(3);
          write_selected<LKP, false>(lk, K, keff, k, orow, osc, sc);
          if (threadIdx.x == 0) cl.path[q] = FT_PATH_LISTS;
          CSAHCA_TRACE(4);
          CSAHCA_TRACE_RT(15);
          return;
        }
      } else {
      if (lane == 0) sc.red_and[wave] = kmax;  // (the barriers inside the compaction order it)
      // the kept keys, compacted in slot order into LDS when few enough
      const uint32_t total = compact_in_order<LKP, false>(
          lk, [](uint64_t key) { return key != 0ull; },
          [&](uint32_t pos, uint64_t key, int) {
            if (pos < (uint32_t)SEL_COMPACT) s_keys[pos] = key;
          },
          sc);
      CSAHCA_TRACE(2);
      if (total >= (uint32_t)keff) {
#pragma unroll
        for (int i = 0; i < NWAVE; ++i) kmax = umax64(kmax, sc.red_and[i]);
        // every kept key lies in [lowest kept, kmax]; emax <= the lowest, and all of them
        // share the bits above the highest bit where emax (or 1, when every chunk listed
        // everything) and kmax differ
        const uint64_t lo = emax ? emax : 1ull;
        if (total <= (uint32_t)SEL_COMPACT) {
          uint64_t f[CPT];  // (j, thread) order is the compacted order
#pragma unroll
          for (int j = 0; j < CPT; ++j) {
            const uint32_t i = (uint32_t)(j * SEL_THREADS) + threadIdx.x;
            f[j] = i < total ? s_keys[i] : 0ull;
          }
          const uint64_t K = radix_select_kth<CPT, true>(f, keff, sc, lo, kmax);  // >= emax, so >= every bound
          CSAHCA_TRACE(3);
          write_selected<CPT, true>(f, K, keff, k, orow, osc, sc);
        } else {
          const uint64_t K = radix_select_kth<LKP, true>(lk, keff, sc, lo, kmax);
          CSAHCA_TRACE(3);
          write_selected<LKP, false>(lk, K, keff, k, orow, osc, sc);
        }
        if (threadIdx.x == 0) cl.path[q] = FT_PATH_LISTS;
        CSAHCA_TRACE(4);
        CSAHCA_TRACE_RT(15);
        return;
      }
      }
    }
  }
  if (cl.path && threadIdx.x == 0) cl.path[q] = FT_PATH_GROUPS;
  // group maxima, coalesced: thread t holds groups j*SEL_THREADS + t (j < KP).  A group's
  // key is its maximum score key, then the lower group index: as groups are index ranges,
  // that orders equal maxima as their best entries are ordered.
  const uint32_t* grow = gmax + (size_t)q * NG;
  const int ng = cdiv(V, GROUP);
#pragma unroll
  for (int j = 0; j < KP; ++j) {
    const int gi = j * SEL_THREADS + (int)threadIdx.x;
    kr[j] = gi < ng ? ((uint64_t)grow[gi] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)gi) : 0ull;
  }
  // With fewer groups than K every group is a candidate (T1 = 0 keeps every usable key).
  const uint64_t T1 = keff < ng ? radix_select_kth(kr, keff, sc) : 0ull;
  // entries scoring below the T1 group's maximum cannot be among the top K
  const uint64_t T1s = T1 & 0xFFFFFFFF00000000ull;
  CSAHCA_TRACE(1);
  // exactly min(K, ng) groups have a maximum >= T1; list them in index order, which is
  // (j, wave, lane) order
  const uint32_t ngl = compact_in_order<KP, true>(
      kr, [&](uint64_t key) { return key != 0ull && key >= T1; },
      [&](uint32_t pos, uint64_t, int j) { glist[pos] = j * SEL_THREADS + (int)threadIdx.x; }, sc);
  CSAHCA_TRACE(2);
  // candidates, coalesced: 16 lanes read the 16 scores of one listed group; key j of lane
  // (wave, lane) is element lane%16 of listed group wave*GPWk + j*4 + lane/16, so that
  // (wave, j, lane) order is index order.  Every load is issued (clamped to valid memory)
  // before any is used, so they overlap.
  int ce[KP];
  float cv[KP];
#pragma unroll
  for (int j = 0; j < KP; ++j) {
    const int gp = wave * GPWk + j * 4 + (lane >> 4);
    ce[j] = gp < (int)ngl ? glist[gp] * GROUP + (lane & 15) : V;
    cv[j] = srow[min(ce[j], N_c - 1)];
  }
#pragma unroll
  for (int j = 0; j < KP; ++j) {
    const uint64_t key = ce[j] < V ? entry_key(cv[j], (uint32_t)ce[j]) : 0ull;
    kr[j] = key >= T1s ? key : 0ull;
  }
  const uint64_t T2 = radix_select_kth(kr, keff, sc);
  CSAHCA_TRACE(3);
  write_selected<KP, false>(kr, T2, keff, k, orow, osc, sc);
  CSAHCA_TRACE(4);
  CSAHCA_TRACE_RT(15);
}

// ---------------------------------------------------------------------------------------
// selection by one wave per query (no lists, k <= WS_MAX_K, at most 64 WS_MAX_NGPL groups)
// ---------------------------------------------------------------------------------------
// The same two thresholds as above, found by bisection instead of histograms: the K-th
// largest of a set of 32-bit keys is the largest x for which at least K keys are >= x,
// decided one bit at a time from the highest bit on which the keys differ, each count a
// sum of ballot popcounts.  Once few keys are left undecided (inside the interval the
// decided bits leave), they are compacted into LDS and the search goes on over those
// alone.  No step needs more than the wave, so the four queries of a workgroup run
// independently, with no workgroup barrier.
//   T1: s1, the K-th largest group maximum (score key).  The groups above s1, and the
//       groups at s1 of lowest index up to K in all, are the K groups of the group-key
//       order above.
//   Candidates: the entries of those groups scoring >= s1, in index order (held in LDS up
//       to WS_CAP; beyond that every count re-reads the groups' scores).
//   T2: s2, the K-th largest candidate score key; the selected are the candidates above
//       s2 and, of those at s2, the lowest indices up to K.
// Score keys are nonzero for every non-NaN score, so 0 marks "no key".
constexpr int WS_WAVES = 4;      // queries per workgroup
constexpr int WS_MAX_K = 512;
constexpr int WS_CAP = 1024;     // candidates held in LDS per query
constexpr int WS_UNROLL = 16;    // candidate batches (4 groups each) per load round
constexpr int WS_MAX_NGPL = 80;  // group maxima per lane (5120 groups; four waves per SIMD)
constexpr int WS_SHRINK = 4;     // undecided keys per lane once compacted (256 per wave)

CSAHCA_DEV uint32_t lane_below(uint64_t bal) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
}

// LDS written by lanes of this wave is read back by other lanes of it: one wave's LDS
// operations complete in order, so only the compiler must not move them across this
CSAHCA_DEV void wave_lds_order() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// the lowest n set bits of m
CSAHCA_DEV uint64_t lowest_bits(uint64_t m, uint32_t n) {
  if (n >= (uint32_t)__popcll(m)) return m;
  uint64_t out = 0ull;
  for (uint32_t i = 0; i < n; ++i) {
    const uint64_t lowest = m & (~m + 1ull);
    out |= lowest;
    m ^= lowest;
  }
  return out;
}

// The lanes of one row (64 keys in index order) that are selected by the rule "above the
// threshold, or equal to it among the first `take` equal keys in index order"; eq_seen
// counts the equal keys of the rows before.
CSAHCA_DEV uint64_t row_selection(bool above, bool equal, uint32_t take, uint32_t& eq_seen) {
  uint64_t sel = __ballot(above);
  const uint64_t beq = __ballot(equal);
  if (beq) {
    sel |= lowest_bits(beq, take > eq_seen ? take - eq_seen : 0u);
    eq_seen += (uint32_t)__popcll(beq);
  }
  return sel;
}

template <int N>
CSAHCA_DEV uint32_t count_ge(const uint32_t (&v)[N], uint32_t x) {
  uint32_t c = 0;
#pragma unroll
  for (int j = 0; j < N; ++j) c += (uint32_t)__popcll(__ballot(v[j] >= x));
  return c;
}

// K-th largest of the nonzero keys v (n of them, n >= K; a and o the AND and OR of them).
// lds: 64 (WS_SHRINK + 1) words of this wave's LDS to compact the undecided keys into.
template <int N>
CSAHCA_DEV uint32_t wave_kth_largest(const uint32_t (&v)[N], uint32_t n, uint32_t K, uint32_t a, uint32_t o,
                                     uint32_t* lds) {
  a = __builtin_amdgcn_readfirstlane(a);  // (the same in every lane: scalar from here)
  o = __builtin_amdgcn_readfirstlane(o);
  const uint32_t diff = a ^ o;
  if (diff == 0u) return a;
  int bit = 31 - __builtin_clz(diff);
  uint32_t t = bit == 31 ? 0u : a & ~((2u << bit) - 1u);  // the bits every key shares
  uint32_t clo = n, chi = 0u;  // keys >= t; keys >= t + 2^(bit+1) (all below K)
  for (; bit >= 0; --bit) {
    if (N > WS_SHRINK && clo - chi <= (uint32_t)(64 * WS_SHRINK)) break;
    const uint32_t c = t | (1u << bit);
    const uint32_t cnt = count_ge(v, c);
    if (cnt >= K) {
      t = c;
      clo = cnt;
    } else {
      chi = cnt;
    }
  }
  if constexpr (N > WS_SHRINK) {
    if (bit < 0) return t;
    // the undecided keys lie in [t, t + 2^(bit+1)); compact them (in any order), each lane
    // writing its own in a row from its offset (the others to a slot of its own past them)
    const int lane = threadIdx.x & 63;
    uint32_t hmask = bit == 31 ? 0u : ~((2u << bit) - 1u);  // (t has none of the other bits)
    uint32_t mine = 0;
#pragma unroll
    for (int j = 0; j < N; ++j) mine += (v[j] != 0u && (v[j] & hmask) == t) ? 1u : 0u;
    const uint32_t incl = wave_incl_scan(mine);
    uint32_t pos = incl - mine;
    asm volatile("" : "+s"(hmask));  // (the tests are made again below, not kept)
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const bool in = v[j] != 0u && (v[j] & hmask) == t;
      lds[in ? pos : (uint32_t)(64 * WS_SHRINK + lane)] = v[j];
      pos += in ? 1u : 0u;
    }
    wave_lds_order();
    const uint32_t nu = clo - chi;
    uint32_t u[WS_SHRINK];
#pragma unroll
    for (int j = 0; j < WS_SHRINK; ++j) {
      const uint32_t i = (uint32_t)(64 * j + lane);
      u[j] = i < nu ? lds[i] : 0u;
    }
    wave_lds_order();  // (the caller may reuse the LDS)
    const uint32_t K2 = K - chi;
    for (; bit >= 0; --bit) {
      const uint32_t c = t | (1u << bit);
      if (count_ge(u, c) >= K2) t = c;
    }
  }
  return t;
}

// Calls f(i, e, key) for the candidate batches i = 0, 1, ... of a query: lane l of batch
// i holds entry e = 16 glist[4i + l/16] + l%16 and its score key (0 past V or the list),
// so that (i, lane) order is index order.  The loads of the next WS_UNROLL batches are
// issued before the current ones are used.
template <typename F>
CSAHCA_DEV void ws_for_candidates(const int* gl, int ngl, const float* srow, int V, int N_c, F f) {
  const int lane = threadIdx.x & 63;
  const int nb = cdiv(ngl, 4);
  auto issue = [&](int i0, int (&e)[WS_UNROLL], float (&v)[WS_UNROLL]) {
#pragma unroll
    for (int u = 0; u < WS_UNROLL; ++u) {
      const int gp = 4 * (i0 + u) + (lane >> 4);
      e[u] = gp < ngl ? gl[gp] * GROUP + (lane & 15) : V;
      v[u] = srow[min(e[u], N_c - 1)];
    }
  };
  int e[WS_UNROLL], e2[WS_UNROLL];
  float v[WS_UNROLL], v2[WS_UNROLL];
  issue(0, e, v);
  for (int i0 = 0; i0 < nb; i0 += WS_UNROLL) {
    const bool more = i0 + WS_UNROLL < nb;
    if (more) issue(i0 + WS_UNROLL, e2, v2);
#pragma unroll
    for (int u = 0; u < WS_UNROLL; ++u)
      if (i0 + u < nb) f(i0 + u, e[u], e[u] < V ? score_key(v[u]) : 0u);
    if (more) {
#pragma unroll
      for (int u = 0; u < WS_UNROLL; ++u) {
        e[u] = e2[u];
        v[u] = v2[u];
      }
    }
  }
}

template <int NGPL>
__global__ __launch_bounds__(64 * WS_WAVES, 4) void select_topk_wave(
    const float* __restrict__ scores, const uint32_t* __restrict__ gmax,
    const int* __restrict__ q_pos, int m, int Tq, int N_c, int NG, int nq, int k,
    int* __restrict__ topk_idx, float* __restrict__ topk_score) {
  __shared__ int s_glist[WS_WAVES][WS_MAX_K];
  __shared__ uint32_t s_ckey[WS_WAVES][WS_CAP];
  __shared__ int s_cidx[WS_WAVES][WS_CAP];
  static_assert(WS_CAP >= 64 * (WS_SHRINK + 1), "the key compaction reuses the candidate keys' LDS");
  // (the wave index is uniform in the wave: everything per query is scalar)
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q = blockIdx.x * WS_WAVES + wave;
  if (q >= nq) return;
  CSAHCA_TRACE(0);
  CSAHCA_TRACE_RT(14);
  const int b = q / Tq, t = q - b * Tq;
  const int V = visible_entries(q_pos, b, t, m, N_c);
  const int keff = min(k, V);
  const float* srow = scores + (size_t)q * N_c;
  int* orow = topk_idx + (size_t)q * k;
  float* osc = topk_score ? topk_score + (size_t)q * k : nullptr;
  for (int i = keff + lane; i < k; i += 64) {
    orow[i] = -1;
    if (osc) osc[i] = -INFINITY;
  }
  if (keff == V) {  // everything usable is selected
    for (int i = lane; i < V; i += 64) {
      orow[i] = i;
      if (osc) osc[i] = srow[i];
    }
    return;
  }
  int* gl = s_glist[wave];
  uint32_t* ckey = s_ckey[wave];
  int* cidx = s_cidx[wave];

  // T1 over the group maxima: lane l holds groups 64 j + l
  const int ng = cdiv(V, GROUP);
  const uint32_t* grow = gmax + (size_t)q * NG;
  // (loads clamped to the row; one per-lane limit decides which are past it, so that no
  // per-group index stays live)
  const int lim = ng - 1 - lane;
  const uint32_t* gp = grow + lane;
  uint32_t mx[NGPL];
#pragma unroll
  for (int j = 0; j < NGPL; ++j) mx[j] = gp[min(64 * j, lim)];
  uint32_t a = ~0u, o = 0u;
#pragma unroll
  for (int j = 0; j < NGPL; ++j) {
    if (64 * j > lim) mx[j] = 0u;
    a &= mx[j] ? mx[j] : ~0u;
    o |= mx[j];
  }
  a = wave_and(a);
  o = wave_or(o);
  CSAHCA_TRACE(1);
  // with no more groups than K every group is taken (threshold 0: every nonzero key is
  // above it) and every usable entry is a candidate
  const bool all_groups = keff >= ng;
  const uint32_t s1 = all_groups ? 0u : wave_kth_largest(mx, (uint32_t)ng, (uint32_t)keff, a, o, ckey);
  CSAHCA_TRACE(2);
  // the K groups, listed in index order
  {
    uint32_t above = 0;
#pragma unroll
    for (int j = 0; j < NGPL; ++j) above += (uint32_t)__popcll(__ballot(mx[j] > s1));
    const uint32_t take = all_groups ? 0u : (uint32_t)keff - above;  // groups at s1 to take
    uint32_t base = 0, eq_seen = 0;
    int gid = lane;
    asm volatile("" : "+v"(gid));  // (formed afresh here, not kept from the loads)
#pragma unroll
    for (int j = 0; j < NGPL; ++j) {
      const uint64_t sel = row_selection(mx[j] > s1, !all_groups && mx[j] == s1, take, eq_seen);
      if ((sel >> lane) & 1ull) gl[base + lane_below(sel)] = 64 * j + gid;
      base += (uint32_t)__popcll(sel);
    }
  }
  const int ngl = all_groups ? ng : keff;
  // every candidate key lies in [s1, the largest group maximum] (o bounds them above)
  wave_lds_order();
  CSAHCA_TRACE(3);

  // candidates: the listed groups' entries scoring >= s1, compacted in index order
  const uint32_t cmin = s1 ? s1 : 1u;
  uint32_t nc = 0;
  ws_for_candidates(gl, ngl, srow, V, N_c, [&](int, int e, uint32_t key) {
    const bool c = key >= cmin;
    const uint64_t bal = __ballot(c);
    const uint32_t pos = nc + lane_below(bal);
    if (c && pos < (uint32_t)WS_CAP) {
      ckey[pos] = key;
      cidx[pos] = e;
    }
    nc += (uint32_t)__popcll(bal);
  });
  CSAHCA_TRACE(4);
  constexpr int CPL = WS_CAP / 64;
  if (nc <= (uint32_t)WS_CAP) {
    wave_lds_order();
    uint32_t ck[CPL];
    uint32_t ca = ~0u, co = 0u;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const uint32_t i = 64 * j + lane;
      ck[j] = i < nc ? ckey[i] : 0u;
      ca &= ck[j] ? ck[j] : ~0u;
      co |= ck[j];
    }
    ca = wave_and(ca);
    co = wave_or(co);
    int cid[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) cid[j] = cidx[64 * j + lane];
    wave_lds_order();  // (the compaction below reuses the candidate keys' LDS)
    const uint32_t s2 = wave_kth_largest(ck, nc, (uint32_t)keff, ca, co, ckey);
    uint32_t above = 0;
#pragma unroll
    for (int j = 0; j < CPL; ++j) above += (uint32_t)__popcll(__ballot(ck[j] > s2));
    const uint32_t take = (uint32_t)keff - above;
    uint32_t base = 0, eq_seen = 0;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const uint64_t sel = row_selection(ck[j] > s2, ck[j] == s2, take, eq_seen);
      if ((sel >> lane) & 1ull) {
        const uint32_t pos = base + lane_below(sel);
        orow[pos] = cid[j];
        if (osc) osc[pos] = key_score(ck[j]);
      }
      base += (uint32_t)__popcll(sel);
    }
    CSAHCA_TRACE(5);
    CSAHCA_TRACE_RT(15);
    return;
  }
  // more candidates than LDS holds: every count re-reads the listed groups' scores
  const uint32_t hi = o;
  auto count_at_least = [&](uint32_t x) {
    uint32_t c = 0;
    ws_for_candidates(gl, ngl, srow, V, N_c, [&](int, int, uint32_t key) {
      c += (uint32_t)__popcll(__ballot(key >= x));
    });
    return c;
  };
  // largest x in [cmin, hi] with at least keff candidates >= x
  uint32_t s2 = cmin;
  {
    const uint32_t diff = cmin ^ hi;
    if (diff) {
      const int hb = 31 - __builtin_clz(diff);
      s2 = hb == 31 ? 0u : cmin & ~((2u << hb) - 1u);
      for (int bit = hb; bit >= 0; --bit) {
        const uint32_t c = s2 | (1u << bit);
        if (count_at_least(c) >= (uint32_t)keff) s2 = c;
      }
    }
  }
  const uint32_t take = (uint32_t)keff - count_at_least(s2 + 1u);
  uint32_t base = 0, eq_seen = 0;
  ws_for_candidates(gl, ngl, srow, V, N_c, [&](int, int e, uint32_t key) {
    const uint64_t sel = row_selection(key > s2, key == s2, take, eq_seen);
    if ((sel >> lane) & 1ull) {
      const uint32_t pos = base + lane_below(sel);
      orow[pos] = e;
      if (osc) osc[pos] = key_score(key);
    }
    base += (uint32_t)__popcll(sel);
  });
}

}  // namespace

namespace csahca {

int index_select_impl(const float* scores, const uint32_t* gmax, const int* q_pos, int m, int B,
                      int Tq, int N_c, int k, int* topk_idx, float* topk_score, hipStream_t st,
                      const ChunkLists* lists, const PoolBeside* pool, bool* pooled) {
  using namespace csahca;
  const int nq = B * Tq;
  if (pooled) *pooled = false;
  const PoolBeside no_pool{nullptr, nullptr, nullptr, 0, 8, 4, 0, 0, 0, 0, NormRope{nullptr, 0.f, 1.f, 0, 0},
                           0, 0, nullptr, nullptr, nullptr, 0, 0, 1, 0};
  const int NG = cdiv(N_c, GROUP);
  if (!lists && k <= WS_MAX_K && NG <= 64 * WS_MAX_NGPL) {
    const unsigned grid = (unsigned)cdiv(nq, WS_WAVES);
    auto kern = NG <= 64 * 16 ? select_topk_wave<16> : NG <= 64 * 48 ? select_topk_wave<48>
                                                                       : select_topk_wave<WS_MAX_NGPL>;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * WS_WAVES), 0, st, scores, gmax, q_pos, m, Tq, N_c, NG, nq,
                       k, topk_idx, topk_score);
    return launch_status("lightning_index_select");
  }
  // (the 8-key kernel gathers k <= 512 candidate groups and holds at most 8192 maxima)
  if (!lists && k <= NWAVE * 8 * 64 / GROUP && NG <= SEL_THREADS * 8)
    hipLaunchKernelGGL((select_topk<8, 0>), dim3((unsigned)nq), dim3(SEL_THREADS), 0, st, scores, gmax,
                       q_pos, m, Tq, N_c, NG, k, topk_idx, topk_score, ChunkLists{}, nq, no_pool);
  else if (!lists)
    hipLaunchKernelGGL((select_topk<KPT, 0>), dim3((unsigned)nq), dim3(SEL_THREADS), 0, st, scores, gmax,
                       q_pos, m, Tq, N_c, NG, k, topk_idx, topk_score, ChunkLists{}, nq, no_pool);
  else {
    // list slots per thread: the smallest power of two that holds every chunk's list
    const long long slots = (long long)lists->P * lists->JMAX;
    auto kern = slots <= SEL_THREADS * 2 ? select_topk<KPT, 2>
              : slots <= SEL_THREADS * 4 ? select_topk<KPT, 4>
              : slots <= SEL_THREADS * 8 ? select_topk<KPT, 8>
                                          : select_topk<KPT, KPT>;
    const bool with_pool = pool && (pool->total > 0 || pool->rows > 0);
    const long long gpool = with_pool ? pool->pool_wgs + cdiv<long long>(pool->rows * (pool->c / VEC), SEL_THREADS)
                                      : 0;
    hipLaunchKernelGGL(kern, dim3((unsigned)(nq + gpool)), dim3(SEL_THREADS), 0, st, scores, gmax, q_pos, m, Tq,
                       N_c, NG, k, topk_idx, topk_score, *lists, nq, with_pool ? *pool : no_pool);
    if (pooled) *pooled = with_pool;
  }
  return launch_status("lightning_index_select");
}

}  // namespace csahca

extern "C" size_t lightning_index_topk_workspace_size(int B, int Tq, int n_ih, int N_c, int k) {
  (void)n_ih;
  if (B < 1 || Tq < 1 || N_c < 1 || k < 1) return 0;
  return ws_layout((long long)B * Tq, N_c, k, Tq == 1).total;
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
  const WsLayout L = ws_layout((long long)B * Tq, N_c, k, Tq == 1);
  if (!workspace || ws_bytes < L.total)
    return fail(CSAHCA_EWORKSPACE, "lightning_index_select: workspace missing or too small");
  // the chunk lists are taken for the queries whose lists the scoring launch marked ready
  const ChunkLists cl = chunk_lists_of((char*)workspace, L, k);
  return index_select_impl(scores, (const uint32_t*)((char*)workspace + L.gkeys_off), q_pos, m, B, Tq,
                           N_c, k, topk_idx, topk_score, (hipStream_t)stream, cl.cand ? &cl : nullptr);
}

namespace {

// lightning_index_topk on a given workspace (the caller's, or the allocation-free variant's
// file-scope scratch); argument checks included
// The pooling of a decode step's new CSA block(s) enqueued with the indexer call
// (lightning_index_topk_csa_compress): csa_compress's arguments without the bias; with nr
// (lightning_index_topk_csa_compress_norm_rope_rows) csahca_compress_norm_rope's, and the
// step's window rows of csahca_compress_pair_norm_rope_rows's side a.
struct PoolReq {
  const void *kv, *gate;
  void* out;
  int n, c, dtype;
  long long in_bs, out_bs;
  const NormRope* nr;
  long long entry0;
  const PairRows* rows;
};

int index_topk_impl(const char* name, const void* q_idx, const float* w_idx, const void* k_idx,
                    int idx_dtype, const int* q_pos, int m, int B, int Tq, int n_ih, int c_I,
                    int N_c, int k, int* topk_idx, float* topk_score, float* all_scores,
                    void* workspace, size_t ws_bytes, hipStream_t s, const PoolReq* pr = nullptr) {
  using namespace csahca;
  int st = index_check_common(q_idx, w_idx, k_idx, idx_dtype, q_pos, m, B, Tq, n_ih, c_I, N_c, k);
  if (st != CSAHCA_OK) return st;
  if (!topk_idx) {
    set_error("%s: topk_idx must be non-NULL", name);
    return CSAHCA_EINVAL;
  }
  const WsLayout L = ws_layout((long long)B * Tq, N_c, k, Tq == 1);
  if (!workspace || ws_bytes < L.total) {
    set_error("%s: workspace missing or too small (%zu bytes needed)", name, L.total);
    return CSAHCA_EWORKSPACE;
  }
  if (all_scores && !aligned16(all_scores)) {
    set_error("%s: all_scores must be 16-byte aligned", name);
    return CSAHCA_EINVAL;
  }
  // the pooling's arguments, all checked before anything is enqueued
  long long NP = 0;
  const bool norm = pr && pr->nr;
  const int row_t = norm && pr->rows && pr->rows->x_a ? pr->rows->T : 0;  // window rows per sequence
  if (pr) {
    st = pool_check(name, pr->kv, pr->gate, nullptr, nullptr, false, 0, pr->out, B, pr->n, pr->c, m,
                    pr->dtype, pr->in_bs, pr->out_bs, &NP);
    if (st != CSAHCA_OK) return st;
    if (norm && (!norm_rope_args_ok(pr->c, pr->nr->d, pr->nr->eps, pr->nr->theta) || pr->entry0 < 0 ||
                 !aligned16(pr->nr->gamma))) {
      set_error("%s: the norm needs c / 8 a power of two <= 64, d_rope %% 8 == 0 and <= c, "
                "eps >= 0, theta > 0, entry0 >= 0 and gamma 16-byte aligned", name);
      return CSAHCA_EINVAL;
    }
    if (norm && pr->rows) {
      st = pair_rows_check(name, *pr->rows, pr->c);
      if (st != CSAHCA_OK) return st;
    }
  }
  // in the selection launch when it is the list selection (bfloat16, m < 8: csa_compress's
  // one-thread-per-slice layout with 4 tokens per load round), else its own launch after
  const bool beside = pr && (NP > 0 || row_t > 0) && pr->dtype == CSAHCA_BF16 && m < 8 && pr->c % 8 == 0 &&
                      (long long)B * NP * (pr->c / 8) <= 0x7FFFFFFFLL &&
                      (long long)B * row_t * (pr->c / 8) <= 0x7FFFFFFFLL;
  PoolBeside pb{};
  if (beside) {
    const PairRows* r = pr->rows;
    pb = PoolBeside{(const uint16_t*)pr->kv, (const uint16_t*)pr->gate, (uint16_t*)pr->out, (int)NP, pr->c, m,
                    pr->in_bs, pr->out_bs, (long long)B * NP * (pr->c / 8), norm ? 1 : 0,
                    norm ? *pr->nr : NormRope{nullptr, 0.f, 1.f, 0, 0}, pr->entry0,
                    (int)cdiv<long long>((long long)B * NP * (pr->c / 8), SEL_THREADS),
                    row_t ? (const uint16_t*)r->x_a : nullptr, row_t ? (uint16_t*)r->y_a : nullptr,
                    row_t ? r->pos_a : nullptr, row_t ? r->x_bs_a : 0, row_t ? r->y_bs_a : 0, row_t ? row_t : 1,
                    (long long)B * row_t};
    if (norm) pb.nr.norm = 1;
  }
  bool pooled = false;
  char* ws = (char*)workspace;
  float* scores = all_scores ? all_scores : (float*)(ws + L.scores_off);
  uint32_t* gkeys = (uint32_t*)(ws + L.gkeys_off);
  if (index_can_list(idx_dtype, Tq, c_I, n_ih, L.plan)) {
    // decode: the scoring launch also writes every chunk's list; the selection launch
    // selects from their union first
    const ChunkLists cl = chunk_lists_of(ws, L, k);
    st = index_score_impl(q_idx, w_idx, k_idx, idx_dtype, q_pos, m, B, Tq, n_ih, c_I, N_c, scores, gkeys,
                          s, &cl);
    if (st != CSAHCA_OK) return st;
    st = index_select_impl(scores, gkeys, q_pos, m, B, Tq, N_c, k, topk_idx, topk_score, s, &cl,
                           beside ? &pb : nullptr, &pooled);
  } else {
    st = index_score_impl(q_idx, w_idx, k_idx, idx_dtype, q_pos, m, B, Tq, n_ih, c_I, N_c, scores, gkeys, s);
    if (st != CSAHCA_OK) return st;
    st = index_select_impl(scores, gkeys, q_pos, m, B, Tq, N_c, k, topk_idx, topk_score, s);
  }
  if (st != CSAHCA_OK || !pr || pooled) return st;
  if (norm)  // the one-layer form of the paired pooling (side b empty)
    return pool_pair(name, pr->kv, pr->gate, pr->out, pr->n, m, pr->in_bs, pr->out_bs, nullptr, nullptr, nullptr,
                     0, m, pr->c, pr->c, B, pr->c, pr->dtype, pr->nr, pr->nr->gamma, pr->entry0, nullptr, 0, s,
                     pr->rows);
  if (NP == 0) return st;
  return pool_entry(name, pr->kv, pr->gate, nullptr, nullptr, false, 0, nullptr, pr->out, B, pr->n, pr->c, m,
                    pr->dtype, pr->in_bs, pr->out_bs, s);
}

}  // namespace

extern "C" int lightning_index_topk(const void* q_idx, const float* w_idx, const void* k_idx,
                                    int idx_dtype, const int* q_pos, int m, int B, int Tq,
                                    int n_ih, int c_I, int N_c, int k, int* topk_idx,
                                    float* topk_score, float* all_scores, void* workspace,
                                    size_t ws_bytes, void* stream) {
  return index_topk_impl("lightning_index_topk", q_idx, w_idx, k_idx, idx_dtype, q_pos, m, B, Tq,
                         n_ih, c_I, N_c, k, topk_idx, topk_score, all_scores, workspace, ws_bytes,
                         (hipStream_t)stream);
}

extern "C" int lightning_index_topk_csa_compress(
    const void* q_idx, const float* w_idx, const void* k_idx, int idx_dtype, const int* q_pos, int m, int B,
    int Tq, int n_ih, int c_I, int N_c, int k, int* topk_idx, float* topk_score, float* all_scores,
    void* workspace, size_t ws_bytes, const void* kv, const void* gate, void* out, int n, int c, int dtype,
    long long in_bstride, long long out_bstride, void* stream) {
  const PoolReq pr{kv, gate, out, n, c, dtype, in_bstride, out_bstride, nullptr, 0, nullptr};
  return index_topk_impl("lightning_index_topk_csa_compress", q_idx, w_idx, k_idx, idx_dtype, q_pos, m, B,
                         Tq, n_ih, c_I, N_c, k, topk_idx, topk_score, all_scores, workspace, ws_bytes,
                         (hipStream_t)stream, &pr);
}

extern "C" int lightning_index_topk_csa_compress_norm_rope_rows(
    const void* q_idx, const float* w_idx, const void* k_idx, int idx_dtype, const int* q_pos, int m, int B,
    int Tq, int n_ih, int c_I, int N_c, int k, int* topk_idx, float* topk_score, float* all_scores,
    void* workspace, size_t ws_bytes, const void* kv, const void* gate, const float* gamma, void* out, int n,
    int c, long long entry0, int d_rope, float eps, float theta, int dtype, long long in_bstride,
    long long out_bstride, int T, const void* row_x, void* row_y, const int* row_pos, long long row_x_bstride,
    long long row_y_bstride, void* stream) {
  const NormRope nr{gamma, eps, theta, d_rope, 1};
  const PairRows rows{T, row_x, nullptr, row_y, nullptr, row_pos, nullptr, row_x_bstride, row_y_bstride, c, c};
  const PoolReq pr{kv, gate, out, n, c, dtype, in_bstride, out_bstride, &nr, entry0, &rows};
  return index_topk_impl("lightning_index_topk_csa_compress_norm_rope_rows", q_idx, w_idx, k_idx, idx_dtype,
                         q_pos, m, B, Tq, n_ih, c_I, N_c, k, topk_idx, topk_score, all_scores, workspace,
                         ws_bytes, (hipStream_t)stream, &pr);
}

// ---------------------------------------------------------------------------------------
// allocation-free variant: the workspace is a file-scope device array
// ---------------------------------------------------------------------------------------
// Every GPU the library runs on holds its own copy of `scratch` (placed by the code-object
// loader, zero-filled) until the process ends.  In host code the array's name only stands
// for the symbol: its device address is taken once per device with hipGetSymbolAddress,
// and only that address is ever handed to a kernel.
static __device__ __align__(256) uint8_t scratch[CSAHCA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
void* scratch_dev[MAX_DEVICES];  // device address of `scratch` per device, null until set up

// The device address of this device's scratch array; set up on the first call per device
// (that device current).  Fails when the stream belongs to another device than the
// current one, whose copy of the array the kernels would then not be able to reach.
int scratch_for(const char* name, hipStream_t stream, void** out) {
  using namespace csahca;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) {
    set_error("%s: no current device (or device ordinal >= %d)", name, MAX_DEVICES);
    return CSAHCA_ELAUNCH;
  }
  if (stream) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess || (int)sdev != dev) {
      set_error("%s: the stream must belong to the current device", name);
      return CSAHCA_EINVAL;
    }
  }
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_dev[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      set_error("%s: cannot locate the scratch array on device %d: %s", name, dev, hipGetErrorString(e));
      return CSAHCA_ELAUNCH;
    }
    scratch_dev[dev] = p;
  }
  *out = scratch_dev[dev];
  return CSAHCA_OK;
}

}  // namespace

extern "C" int lightning_index_topk_noalloc(const void* q_idx, const float* w_idx,
                                            const void* k_idx, int idx_dtype, const int* q_pos,
                                            int m, int B, int Tq, int n_ih, int c_I, int N_c,
                                            int k, int* topk_idx, float* topk_score,
                                            float* all_scores, void* stream) {
  using namespace csahca;
  const char* name = "lightning_index_topk_noalloc";
  // shape checks first: the size test below needs sane B, Tq and N_c
  int st = index_check_common(q_idx, w_idx, k_idx, idx_dtype, q_pos, m, B, Tq, n_ih, c_I, N_c, k);
  if (st != CSAHCA_OK) return st;
  const size_t need = ws_layout((long long)B * Tq, N_c, k, Tq == 1).total;
  if (need > CSAHCA_NOALLOC_SCRATCH_BYTES) {
    set_error("%s: the call needs %zu bytes of scratch, above the built maximum of %zu "
              "(use lightning_index_topk with a workspace)", name, need,
              (size_t)CSAHCA_NOALLOC_SCRATCH_BYTES);
    return CSAHCA_EWORKSPACE;
  }
  void* ws = nullptr;
  st = scratch_for(name, (hipStream_t)stream, &ws);
  if (st != CSAHCA_OK) return st;
  return index_topk_impl(name, q_idx, w_idx, k_idx, idx_dtype, q_pos, m, B, Tq, n_ih, c_I, N_c, k,
                         topk_idx, topk_score, all_scores, ws, CSAHCA_NOALLOC_SCRATCH_BYTES,
                         (hipStream_t)stream);
}
