// Kernel 2: lightning-indexer scores and exact top-k selection.
//
// Source: "DeepSeek-V4 Hybrid Attention: CSA, HCA, mHC, MoE", section V.2: the score of
// compressed block s for query t is sum_h w_{t,h} * ReLU(q_{t,h} . K_s) over the indexer
// heads, and the selector keeps the k best blocks; "DeepSeek-V4: Anatomy of an
// Open-Source Frontier Model" (lesson 6.7): the indexer runs in low precision and can
// pick no more entries than exist.
//
// Scoring (index_score_fp8): the q_I . K_I contraction runs on MFMA (for c_I = 128 one
// v_mfma_scale_f32_16x16x128_f8f6f4 with unit block scales per 16 heads x 16 keys; for
// c_I = 32/64 v_mfma_f32_16x16x32_fp8_fp8).  Each lane streams C_I/4 contiguous bytes of
// one key row straight from HBM into the B operand (no LDS); A takes the same bytes of
// the indexer query row, so whatever order the instruction assigns to the contraction
// dimension, it is the same for both operands and the dot products are exact.  ReLU, the head weights and the
// cross-head sum are applied to the MFMA accumulators in registers.  Every score is
// written once (fp32) and every group of 16 consecutive keys also writes its maximum
// 64-bit selection key.
//
// Selection (select_topk): one workgroup per query.  Selection keys are
// (order-preserving score bits << 32) | (~index), so all keys are distinct and "larger
// key" means "better, lower index on ties".  Let T1 be the K-th largest group maximum.
// At least K keys are >= T1 (one per selected group), so the K-th largest key overall is
// >= T1 and every top-K key lies in one of exactly K selected groups.  The exact top-K is
// then taken from those K*16 candidates.  Both K-th-largest searches are MSB-first radix
// selects over register-resident keys (an LDS histogram per 11-bit digit) that skip the
// bits all remaining candidates share.  The candidates are kept in index order, so the
// output comes out ascending without a sort.
#include "common.hpp"

namespace {

#ifndef CSAHCA_SCORE_WGS
#define CSAHCA_SCORE_WGS 512  // scoring workgroups to aim for (about two per CU)
#endif
#ifndef CSAHCA_SCORE_CONTIG
#define CSAHCA_SCORE_CONTIG 0  // 1: each wave scores a contiguous quarter of its chunk
#endif

constexpr int GROUP = 16;           // keys per group maximum
constexpr int SEL_THREADS = 1024;
constexpr int KPT = 16;                              // selection keys per thread (registers)
constexpr int SEL_MAX_KEYS = SEL_THREADS * KPT;      // 16384 group maxima per query
constexpr int MAX_NC = GROUP * SEL_MAX_KEYS;
constexpr int MAX_K = SEL_THREADS;                   // one candidate group per thread
static_assert(KPT == GROUP, "a thread scans exactly one candidate group");

CSAHCA_DEV int visible_entries(const int* q_pos, int b, int t, int m, int N_c) {
  const long long p = (long long)q_pos[b] + t;
  long long v = (p + 1) / m;
  if (p + 1 <= 0) v = 0;
  return (int)(v < N_c ? v : N_c);
}

// ---------------------------------------------------------------------------------------
// scoring, FP8 E4M3FN keys on MFMA
// ---------------------------------------------------------------------------------------
// QPW queries per workgroup of 4 waves.  QPW = 1: the four waves split the key blocks of
// one query (decode).  QPW = 4: each wave scores its own query over the same key blocks
// (prefill; the repeated key reads hit in cache).  A wave walks its blocks with PF blocks
// of keys in flight in registers: block k is scored while blocks k+1 .. k+PF-1 load.
typedef int i32x8 __attribute__((ext_vector_type(8)));

template <int C_I>
struct KeyOperand;  // the C_I/4 contiguous key bytes one lane contributes per 16-key block

template <>
struct KeyOperand<128> {  // one v_mfma_scale_f32_16x16x128_f8f6f4 per head block
  i32x8 v;
  CSAHCA_DEV void load(const uint8_t* p) { v = *reinterpret_cast<const i32x8*>(p); }
  CSAHCA_DEV void zero() { v = i32x8{0, 0, 0, 0, 0, 0, 0, 0}; }
  CSAHCA_DEV static f32x4 mma(const KeyOperand& a, const KeyOperand& b, f32x4 c) {
    // operand formats 0 = FP8 E4M3; block scales 127 = 2^0 (E8M0), i.e. no scaling
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a.v, b.v, c, 0, 0, 0, 127, 0, 127);
  }
};

template <int C_I>
struct KeyOperand {  // C_I in {32, 64}: v_mfma_f32_16x16x32_fp8_fp8, C_I/32 K-steps
  static constexpr int KS = C_I / 32;
  long v[KS];
  CSAHCA_DEV void load(const uint8_t* p) {
    if constexpr (KS == 2) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(p);
      v[0] = (long)(((uint64_t)a[1] << 32) | a[0]);
      v[1] = (long)(((uint64_t)a[3] << 32) | a[2]);
    } else {
      const u32x2 a = *reinterpret_cast<const u32x2*>(p);
      v[0] = (long)(((uint64_t)a[1] << 32) | a[0]);
    }
  }
  CSAHCA_DEV void zero() {
#pragma unroll
    for (int i = 0; i < KS; ++i) v[i] = 0;
  }
  CSAHCA_DEV static f32x4 mma(const KeyOperand& a, const KeyOperand& b, f32x4 c) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      c = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a.v[ks], b.v[ks], c, 0, 0, 0);
    return c;
  }
};

template <int C_I, int HB, int QPW, int PF>
__global__ __launch_bounds__(256) void index_score_fp8(
    const uint8_t* __restrict__ qI, const float* __restrict__ w, const uint8_t* __restrict__ KI,
    const int* __restrict__ q_pos, int m, int Tq, int N_c, int CH, int nq, int NG,
    float* __restrict__ scores, uint64_t* __restrict__ gkeys) {
  constexpr int NIH = HB * 16;
  constexpr int WPQ = 4 / QPW;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int q = blockIdx.y * QPW + wave / WPQ;
  const int sub = wave % WPQ;
  if (q >= nq) return;  // this kernel has no barriers: a finished wave may leave
  const int b = q / Tq, t = q - b * Tq;
  const int V = visible_entries(q_pos, b, t, m, N_c);
  const int e_begin = blockIdx.x * CH;
  const int e_end = min(e_begin + CH, V);
  if (e_begin >= e_end) return;

  const int row = lane & 15, g = lane >> 4;
  // A operand: indexer query of head (16*hb + row), dims [g*C_I/4, (g+1)*C_I/4); the same
  // dims of a key row form the B operand, so the dot products are those of the full rows
  KeyOperand<C_I> a[HB];
  const uint8_t* qp = qI + (size_t)q * NIH * C_I;
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) a[hb].load(qp + (hb * 16 + row) * C_I + g * (C_I / 4));
  // head weights of the accumulator rows this lane holds: heads 16*hb + 4*g + i
  float wr[HB][4];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb)
#pragma unroll
    for (int i = 0; i < 4; ++i) wr[hb][i] = w[(size_t)q * NIH + hb * 16 + 4 * g + i];

  const uint8_t* kb = KI + (size_t)b * N_c * C_I + g * (C_I / 4);
  float* srow = scores + (size_t)q * N_c;
  uint64_t* grow = gkeys + (size_t)q * NG;
  const int nblk = cdiv(e_end - e_begin, GROUP);
#if CSAHCA_SCORE_CONTIG
  // block k of this wave is sub*per + k
  const int per = cdiv(nblk, WPQ);
  const int nmine = max(0, min(per, nblk - sub * per));
  auto blk_of = [&](int k) { return sub * per + k; };
#else
  const int nmine = nblk > sub ? cdiv(nblk - sub, WPQ) : 0;  // blocks sub, sub+WPQ, ...
  auto blk_of = [&](int k) { return sub + k * WPQ; };
#endif

  // blocks past the end load a valid row instead (their scores are never used)
  auto load_block = [&](KeyOperand<C_I>& dst, int k) {
    const int e = min(e_begin + blk_of(min(k, nmine - 1)) * GROUP + row, e_end - 1);
    dst.load(kb + (size_t)e * C_I);
  };
  // two register buffers of PF blocks: while one is scored the other is in flight, so
  // every load has a full iteration of scoring to arrive
  KeyOperand<C_I> kf0[PF], kf1[PF];
#pragma unroll
  for (int u = 0; u < PF; ++u) {
    load_block(kf0[u], u);
    load_block(kf1[u], PF + u);
  }
  auto score_blocks = [&](KeyOperand<C_I>(&kf)[PF], int k0) {
    f32x4 acc[PF][HB];
#pragma unroll
    for (int u = 0; u < PF; ++u)
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) acc[u][hb] = KeyOperand<C_I>::mma(a[hb], kf[u], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int u = 0; u < PF; ++u) load_block(kf[u], k0 + 2 * PF + u);  // refill: two rounds ahead
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int k = k0 + u;
      // lane holds key (row) for heads 16*hb + 4*g + i; sum over heads as a balanced tree
      float t[4 * HB];
#pragma unroll
      for (int hb = 0; hb < HB; ++hb)
#pragma unroll
        for (int i = 0; i < 4; ++i) t[4 * hb + i] = wr[hb][i] * fmaxf(acc[u][hb][i], 0.f);
#pragma unroll
      for (int wdt = 2 * HB; wdt >= 1; wdt /= 2)
#pragma unroll
        for (int v = 0; v < wdt; ++v) t[v] += t[v + wdt];
      const float score = sum_over_row_groups(t[0]);  // same value in lanes row, row+16, ...
      const int e0 = e_begin + blk_of(k) * GROUP;
      const int e = e0 + row;
      const bool valid = k < nmine && e < e_end;
      if (g == 0 && valid) srow[e] = score;
      // group maximum: the best score of the 16 keys, lowest index among equal scores
      const float sv = valid ? score : -INFINITY;
      const float best = row16_max(sv);
      const uint64_t hit = __ballot(valid && sv == best) & 0xFFFFull;
      if (lane == 0 && hit != 0ull) grow[e0 / GROUP] = entry_key(best, (uint32_t)(e0 + __builtin_ctzll(hit)));
    }
  };
  for (int k0 = 0; k0 < nmine; k0 += 2 * PF) {
    score_blocks(kf0, k0);
    if (k0 + PF < nmine) score_blocks(kf1, k0 + PF);
  }
}

// ---------------------------------------------------------------------------------------
// scoring, float32 keys (small heads; plain FMA)
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void index_score_f32(
    const float* __restrict__ qI, const float* __restrict__ w, const float* __restrict__ KI,
    const int* __restrict__ q_pos, int m, int Tq, int N_c, int n_ih, int c_I, int NG,
    float* __restrict__ scores, uint64_t* __restrict__ gkeys) {
  extern __shared__ float smem_f[];
  float* qs = smem_f;               // [n_ih * c_I]
  float* ws = smem_f + n_ih * c_I;  // [n_ih]
  const int q = blockIdx.y;
  const int b = q / Tq, t = q - b * Tq;
  for (int i = threadIdx.x; i < n_ih * c_I; i += blockDim.x) qs[i] = qI[(size_t)q * n_ih * c_I + i];
  for (int i = threadIdx.x; i < n_ih; i += blockDim.x) ws[i] = w[(size_t)q * n_ih + i];
  __syncthreads();
  const int V = visible_entries(q_pos, b, t, m, N_c);
  const int e = blockIdx.x * blockDim.x + threadIdx.x;  // blockDim is a multiple of 16
  const bool valid = e < V;
  float s = 0.f;
  if (valid) {
    const float* kr = KI + ((size_t)b * N_c + e) * c_I;
    for (int h = 0; h < n_ih; ++h) {
      float d = 0.f;
      for (int j = 0; j < c_I; ++j) d = fmaf(qs[h * c_I + j], kr[j], d);
      s = fmaf(ws[h], fmaxf(d, 0.f), s);
    }
    scores[(size_t)q * N_c + e] = s;
  }
  uint64_t key = valid ? entry_key(s, (uint32_t)e) : 0ull;
  key = umax64(key, shfl_xor_u64(key, 1));
  key = umax64(key, shfl_xor_u64(key, 2));
  key = umax64(key, shfl_xor_u64(key, 4));
  key = umax64(key, shfl_xor_u64(key, 8));
  if ((threadIdx.x & 15) == 0 && e < V) gkeys[(size_t)q * NG + e / GROUP] = key;
}

// ---------------------------------------------------------------------------------------
// selection
// ---------------------------------------------------------------------------------------
constexpr int NBIN = 2048;  // radix digit of 11 bits
constexpr int NWAVE = SEL_THREADS / 64;

struct SelScratch {
  uint32_t hist[2][NBIN];
  uint64_t red_and[NWAVE];
  uint64_t red_or[NWAVE];
  uint32_t scan[NWAVE];
  uint32_t total;
  uint32_t found_digit;
  uint32_t found_kth;
  uint32_t found_count;
  uint64_t result;
};

// exclusive prefix sum of v over the workgroup, in thread order; also returns the total
CSAHCA_DEV uint32_t block_exclusive_scan(uint32_t v, SelScratch& sc, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_scan(v);
  if (lane == 63) sc.scan[wave] = incl;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < NWAVE; ++i) {
    const uint32_t x = sc.scan[i];
    before += i < wave ? x : 0u;
    all += x;
  }
  total = all;
  __syncthreads();  // sc.scan may be reused right after
  return before + incl - v;
}

// K-th largest (1-based) of the distinct nonzero keys the workgroup holds in registers
// (KPT per thread; 0 = empty).  One AND/OR reduction finds the highest bit on which the
// keys differ; from there MSB-first radix passes of 11 bits narrow the candidates.  A
// pass builds an LDS histogram of the digit, then every wave scans 128 digits (two per
// lane, in descending order) and the lane whose range holds the K-th key reports the
// digit.  The search stops as soon as that digit holds a single candidate.
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
  for (int sh = hb >= 10 ? hb - 10 : 0;; sh = sh >= 11 ? sh - 11 : 0) {
    uint32_t* h = sc.hist[buf];
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const uint64_t k = kr[j];
      if (k != 0ull && (k & mask) == prefix) atomicAdd(&h[(uint32_t)(k >> sh) & (NBIN - 1)], 1u);
    }
    for (int i = threadIdx.x; i < NBIN; i += SEL_THREADS) sc.hist[buf ^ 1][i] = 0u;
    __syncthreads();
    // this lane's two digits, descending with the thread index
    const int d_hi = NBIN - 1 - 2 * (int)threadIdx.x;
    const uint32_t c_hi = h[d_hi], c_lo = h[d_hi - 1];
    const uint32_t incl = wave_incl_scan(c_hi + c_lo);
    if (lane == 63) sc.scan[wave] = incl;
    __syncthreads();
    uint32_t above = incl - (c_hi + c_lo);
#pragma unroll
    for (int i = 0; i < NWAVE; ++i) above += i < wave ? sc.scan[i] : 0u;
    const uint32_t kk = (uint32_t)kth;
    if (above < kk && kk <= above + c_hi) {
      sc.found_digit = d_hi;
      sc.found_kth = kk - above;
      sc.found_count = c_hi;
    } else if (above + c_hi < kk && kk <= above + c_hi + c_lo) {
      sc.found_digit = d_hi - 1;
      sc.found_kth = kk - above - c_hi;
      sc.found_count = c_lo;
    }
    __syncthreads();
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
    const float* __restrict__ scores, const uint64_t* __restrict__ gkeys,
    const int* __restrict__ q_pos, int m, int Tq, int N_c, int NG, int k,
    int* __restrict__ topk_idx, float* __restrict__ topk_score) {
  __shared__ SelScratch sc;
  __shared__ int glist[MAX_K];
  const int q = blockIdx.x;
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
  // group maxima: thread t holds groups t*KPT .. t*KPT+KPT-1
  const int ng = cdiv(V, GROUP);
  const uint64_t* grow = gkeys + (size_t)q * NG;
  uint64_t kr[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int gi = (int)threadIdx.x * KPT + j;
    kr[j] = gi < ng ? grow[gi] : 0ull;
  }
  // With fewer groups than K every group is a candidate (T1 = 0 keeps every usable key).
  const uint64_t T1 = keff < ng ? radix_select_kth(kr, keff, sc) : 0ull;

  // exactly min(K, ng) groups have a maximum >= T1; list them in index order
  uint32_t ngl;
  {
    uint32_t cnt = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) cnt += (kr[j] != 0ull && kr[j] >= T1);
    uint32_t off = block_exclusive_scan(cnt, sc, ngl);
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      if (kr[j] != 0ull && kr[j] >= T1) glist[off++] = (int)threadIdx.x * KPT + j;
    __syncthreads();
  }
  // candidates: thread t scans the 16 keys of listed group t, keeping those >= T1
#pragma unroll
  for (int j = 0; j < KPT; ++j) kr[j] = 0ull;
  if (threadIdx.x < ngl) {
    const int e0 = glist[threadIdx.x] * GROUP;
#pragma unroll
    for (int j = 0; j < GROUP; ++j) {
      const int e = e0 + j;
      if (e < V) {
        const uint64_t key = entry_key(srow[e], (uint32_t)e);
        kr[j] = key >= T1 ? key : 0ull;
      }
    }
  }
  const uint64_t T2 = radix_select_kth(kr, keff, sc);
  {
    uint32_t cnt = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) cnt += (kr[j] != 0ull && kr[j] >= T2);
    uint32_t total;
    uint32_t off = block_exclusive_scan(cnt, sc, total);
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const uint64_t key = kr[j];
      if (key != 0ull && key >= T2) {
        orow[off] = (int)key_index(key);
        if (osc) osc[off] = key_score((uint32_t)(key >> 32));
        ++off;
      }
    }
  }
  for (int i = keff + threadIdx.x; i < k; i += SEL_THREADS) {
    orow[i] = -1;
    if (osc) osc[i] = -INFINITY;
  }
}

// ---------------------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------------------
struct WsLayout {
  size_t gkeys_off, gkeys_bytes, scores_off, scores_bytes, total;
};

WsLayout ws_layout(long long nq, int N_c) {
  WsLayout L;
  const long long NG = cdiv<long long>(N_c, GROUP);
  L.gkeys_off = 0;
  L.gkeys_bytes = csahca::align_up((size_t)(nq * NG * 8), 256);
  L.scores_off = L.gkeys_bytes;
  L.scores_bytes = csahca::align_up((size_t)(nq * (long long)N_c * 4), 256);
  L.total = L.scores_off + L.scores_bytes;
  return L;
}

int check_common(const void* q_idx, const float* w_idx, const void* k_idx, int idx_dtype,
                 const int* q_pos, int m, int B, int Tq, int n_ih, int c_I, int N_c, int k) {
  using namespace csahca;
  if (!q_idx || !w_idx || !k_idx || !q_pos)
    return fail(CSAHCA_EINVAL, "indexer: q_idx, w_idx, k_idx and q_pos must be non-NULL");
  if (B < 1 || Tq < 1 || n_ih < 1 || c_I < 1 || N_c < 1 || m < 1 || k < 1)
    return fail(CSAHCA_EINVAL, "indexer: B, Tq, n_ih, c_I, N_c, m and k must be >= 1");
  if (N_c > MAX_NC) return fail(CSAHCA_ENOTSUP, "indexer: N_c above 262144 is not built");
  if (k > MAX_K) return fail(CSAHCA_ENOTSUP, "indexer: k above 1024 is not built");
  if ((long long)B * Tq > 0x7FFFFFFFLL / 2) return fail(CSAHCA_ENOTSUP, "indexer: too many queries");
  if (idx_dtype == CSAHCA_FP8_E4M3FN) {
    if (n_ih % 16 != 0 || n_ih > 128)
      return fail(CSAHCA_ENOTSUP, "indexer: FP8 keys need n_ih % 16 == 0 and n_ih <= 128");
    if (c_I != 32 && c_I != 64 && c_I != 128)
      return fail(CSAHCA_ENOTSUP, "indexer: FP8 keys need c_I in {32, 64, 128}");
  } else if (idx_dtype == CSAHCA_F32) {
    if (n_ih * c_I > 4096)
      return fail(CSAHCA_ENOTSUP, "indexer: float32 keys need n_ih * c_I <= 4096");
  } else {
    return fail(CSAHCA_ENOTSUP, "indexer: idx_dtype must be CSAHCA_FP8_E4M3FN or CSAHCA_F32");
  }
  if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned16(w_idx))
    return fail(CSAHCA_EINVAL, "indexer: q_idx, w_idx and k_idx must be 16-byte aligned");
  return CSAHCA_OK;
}

template <int C_I, int HB>
void launch_fp8(const void* q_idx, const float* w_idx, const void* k_idx, const int* q_pos,
                int m, int Tq, int N_c, int nq, int NG, float* scores, uint64_t* gkeys,
                hipStream_t st) {
  const bool decode = Tq == 1;
  const int QPW = decode ? 1 : 4;
  const int qgroups = cdiv(nq, QPW);
  // about two workgroups per CU, each streaming a long chunk of keys
  int chunks = cdiv(CSAHCA_SCORE_WGS, qgroups);
  chunks = max(1, min(chunks, cdiv(N_c, 256)));
  const int CH = cdiv(cdiv(N_c, chunks), 64) * 64;
  chunks = cdiv(N_c, CH);
  dim3 grid((unsigned)chunks, (unsigned)qgroups);
  if (decode)
    hipLaunchKernelGGL((index_score_fp8<C_I, HB, 1, 4>), grid, dim3(256), 0, st,
                       (const uint8_t*)q_idx, w_idx, (const uint8_t*)k_idx, q_pos, m, Tq, N_c,
                       CH, nq, NG, scores, gkeys);
  else
    hipLaunchKernelGGL((index_score_fp8<C_I, HB, 4, 4>), grid, dim3(256), 0, st,
                       (const uint8_t*)q_idx, w_idx, (const uint8_t*)k_idx, q_pos, m, Tq, N_c,
                       CH, nq, NG, scores, gkeys);
}

template <int C_I>
bool launch_fp8_heads(int n_ih, const void* q_idx, const float* w_idx, const void* k_idx,
                      const int* q_pos, int m, int Tq, int N_c, int nq, int NG, float* scores,
                      uint64_t* gkeys, hipStream_t st) {
  switch (n_ih / 16) {
    case 1: launch_fp8<C_I, 1>(q_idx, w_idx, k_idx, q_pos, m, Tq, N_c, nq, NG, scores, gkeys, st); return true;
    case 2: launch_fp8<C_I, 2>(q_idx, w_idx, k_idx, q_pos, m, Tq, N_c, nq, NG, scores, gkeys, st); return true;
    case 4: launch_fp8<C_I, 4>(q_idx, w_idx, k_idx, q_pos, m, Tq, N_c, nq, NG, scores, gkeys, st); return true;
    case 8: launch_fp8<C_I, 8>(q_idx, w_idx, k_idx, q_pos, m, Tq, N_c, nq, NG, scores, gkeys, st); return true;
    default: return false;
  }
}

int score_impl(const void* q_idx, const float* w_idx, const void* k_idx, int idx_dtype,
               const int* q_pos, int m, int B, int Tq, int n_ih, int c_I, int N_c,
               float* scores, uint64_t* gkeys, hipStream_t st) {
  using namespace csahca;
  const int nq = B * Tq;
  const int NG = cdiv(N_c, GROUP);
  if (idx_dtype == CSAHCA_FP8_E4M3FN) {
    bool ok = false;
    if (c_I == 128) ok = launch_fp8_heads<128>(n_ih, q_idx, w_idx, k_idx, q_pos, m, Tq, N_c, nq, NG, scores, gkeys, st);
    else if (c_I == 64) ok = launch_fp8_heads<64>(n_ih, q_idx, w_idx, k_idx, q_pos, m, Tq, N_c, nq, NG, scores, gkeys, st);
    else ok = launch_fp8_heads<32>(n_ih, q_idx, w_idx, k_idx, q_pos, m, Tq, N_c, nq, NG, scores, gkeys, st);
    if (!ok) return fail(CSAHCA_ENOTSUP, "indexer: FP8 keys need n_ih in {16, 32, 64, 128}");
  } else {
    const size_t lds = (size_t)(n_ih * c_I + n_ih) * sizeof(float);
    dim3 grid((unsigned)cdiv(N_c, 256), (unsigned)nq);
    hipLaunchKernelGGL(index_score_f32, grid, dim3(256), lds, st, (const float*)q_idx, w_idx,
                       (const float*)k_idx, q_pos, m, Tq, N_c, n_ih, c_I, NG, scores, gkeys);
  }
  return launch_status("lightning_index_score");
}

int select_impl(const float* scores, const uint64_t* gkeys, const int* q_pos, int m, int B,
                int Tq, int N_c, int k, int* topk_idx, float* topk_score, hipStream_t st) {
  using namespace csahca;
  const int nq = B * Tq;
  const int NG = cdiv(N_c, GROUP);
  hipLaunchKernelGGL(select_topk, dim3((unsigned)nq), dim3(SEL_THREADS), 0, st, scores,
                     gkeys, q_pos, m, Tq, N_c, NG, k, topk_idx, topk_score);
  return launch_status("lightning_index_select");
}

}  // namespace

extern "C" size_t lightning_index_topk_workspace_size(int B, int Tq, int n_ih, int N_c, int k) {
  (void)n_ih;
  (void)k;
  if (B < 1 || Tq < 1 || N_c < 1) return 0;
  return ws_layout((long long)B * Tq, N_c).total;
}

extern "C" int lightning_index_score(const void* q_idx, const float* w_idx, const void* k_idx,
                                     int idx_dtype, const int* q_pos, int m, int B, int Tq,
                                     int n_ih, int c_I, int N_c, int k, float* scores,
                                     void* workspace, size_t ws_bytes, void* stream) {
  using namespace csahca;
  int st = check_common(q_idx, w_idx, k_idx, idx_dtype, q_pos, m, B, Tq, n_ih, c_I, N_c, k);
  if (st != CSAHCA_OK) return st;
  if (!scores) return fail(CSAHCA_EINVAL, "lightning_index_score: scores must be non-NULL");
  const WsLayout L = ws_layout((long long)B * Tq, N_c);
  if (!workspace || ws_bytes < L.total)
    return fail(CSAHCA_EWORKSPACE, "lightning_index_score: workspace missing or too small");
  return score_impl(q_idx, w_idx, k_idx, idx_dtype, q_pos, m, B, Tq, n_ih, c_I, N_c, scores,
                    (uint64_t*)((char*)workspace + L.gkeys_off), (hipStream_t)stream);
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
  return select_impl(scores, (const uint64_t*)((char*)workspace + L.gkeys_off), q_pos, m, B, Tq,
                     N_c, k, topk_idx, topk_score, (hipStream_t)stream);
}

extern "C" int lightning_index_topk(const void* q_idx, const float* w_idx, const void* k_idx,
                                    int idx_dtype, const int* q_pos, int m, int B, int Tq,
                                    int n_ih, int c_I, int N_c, int k, int* topk_idx,
                                    float* topk_score, float* all_scores, void* workspace,
                                    size_t ws_bytes, void* stream) {
  using namespace csahca;
  int st = check_common(q_idx, w_idx, k_idx, idx_dtype, q_pos, m, B, Tq, n_ih, c_I, N_c, k);
  if (st != CSAHCA_OK) return st;
  if (!topk_idx) return fail(CSAHCA_EINVAL, "lightning_index_topk: topk_idx must be non-NULL");
  const WsLayout L = ws_layout((long long)B * Tq, N_c);
  if (!workspace || ws_bytes < L.total)
    return fail(CSAHCA_EWORKSPACE, "lightning_index_topk: workspace missing or too small");
  if (all_scores && !aligned16(all_scores))
    return fail(CSAHCA_EINVAL, "lightning_index_topk: all_scores must be 16-byte aligned");
  float* scores = all_scores ? all_scores : (float*)((char*)workspace + L.scores_off);
  uint64_t* gkeys = (uint64_t*)((char*)workspace + L.gkeys_off);
  hipStream_t s = (hipStream_t)stream;
  st = score_impl(q_idx, w_idx, k_idx, idx_dtype, q_pos, m, B, Tq, n_ih, c_I, N_c, scores, gkeys, s);
  if (st != CSAHCA_OK) return st;
  return select_impl(scores, gkeys, q_pos, m, B, Tq, N_c, k, topk_idx, topk_score, s);
}
