// Kernel 2a: lightning-indexer scores.
//
// Source: "DeepSeek-V4 Hybrid Attention: CSA, HCA, mHC, MoE", section V.2: the score of
// compressed block s for query t is sum_h w_{t,h} * ReLU(q_{t,h} . K_s) over the indexer
// heads; "DeepSeek-V4: Anatomy of an Open-Source Frontier Model" (lesson 6.7): the
// indexer runs in low precision.
//
// Scoring (index_score_fp8): the q_I . K_I contraction runs on MFMA (for c_I = 128 one
// v_mfma_scale_f32_16x16x128_f8f6f4 with unit block scales per 16 heads x 16 keys; for
// c_I = 32/64 v_mfma_f32_16x16x32_fp8_fp8).  Each lane streams C_I/4 contiguous bytes of
// one key row straight from HBM into the B operand (no LDS); A takes the same bytes of
// the indexer query row, so whatever order the instruction assigns to the contraction
// dimension, it is the same for both operands and the dot products are exact.  ReLU, the
// head weights and the cross-head sum are applied to the MFMA accumulators in registers.
// Every score is written once (fp32) and every group of 16 consecutive keys also writes
// the order-preserving 32-bit key of its maximum score.
#include "fused_topk.hpp"

namespace {

using namespace csahca;


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

// MX FP4 keys (c_I = 128): the B operand is the lane's 32 E2M1 elements (16 bytes, the
// low 4 registers; the instruction reads no more for FP4) and its 32-element block's E8M0
// scale; the queries stay FP8 with unit scale.  With an FP8 A and an FP4 B operand the
// instruction does not take K in the same order from both: when lane group g of B holds
// key elements [32g, 32g+32) (one scale block, so one scale per lane), lane group g of A
// supplies dimensions [16g, 16g+16) in its first 16 bytes and [64+16g, 80+16g) in its
// last 16.  The queries are loaded in that order.
// (Found with one-hot queries against random keys; the parity tests pin it.)
CSAHCA_DEV f32x4 mma_fp8_fp4(const i32x8& a, const u32x4& b, uint32_t scale_b, f32x4 c) {
  const i32x8 bv = i32x8{(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
  // formats: A 0 = FP8 E4M3, B 4 = FP4 E2M1; A scale 127 = 2^0, B scale from the lane
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, bv, c, 0, 4, 0, 127, 0, (int)scale_b);
}

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
    float* __restrict__ scores, uint32_t* __restrict__ gkeys) {
  constexpr int NIH = HB * 16;
  constexpr int WPQ = 4 / QPW;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int q = blockIdx.y * QPW + wave / WPQ;
  const int sub = wave % WPQ;
  if (q >= nq) return;  // QPW == 1: the four waves share q (the one barrier stays uniform)
  const int b = q / Tq, t = q - b * Tq;
  const int e_begin = blockIdx.x * CH;
  // the chunk's keys are loaded before the visible count is known (every key below N_c is
  // valid memory); scores past the visible count are never written
  const int e_lim = min(e_begin + CH, N_c);

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
  uint32_t* grow = gkeys + (size_t)q * NG;
  auto count_mine = [&](int nblk) { return nblk > sub ? cdiv(nblk - sub, WPQ) : 0; };
  auto blk_of = [&](int k) { return sub + k * WPQ; };  // blocks sub, sub+WPQ, ...
  int nmine = count_mine(cdiv(e_lim - e_begin, GROUP));
  int e_last = e_lim - 1;

  // blocks past the end load a valid row instead (their scores are never used)
  auto load_block = [&](KeyOperand<C_I>& dst, int k) {
    const int e = min(e_begin + blk_of(min(k, nmine - 1)) * GROUP + row, e_last);
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
  const int V = visible_entries(q_pos, b, t, m, N_c);
  const int e_end = min(e_lim, V);
  if (e_begin >= e_end) return;  // uniform over the workgroup when QPW == 1
  nmine = count_mine(cdiv(e_end - e_begin, GROUP));
  e_last = e_end - 1;
  // QPW == 1 (decode): scores and group maxima are staged in LDS and written after the
  // last key load.  Vector stores share the load counter and may complete out of order
  // with loads, so a store inside the loop would make every later wait for a key block a
  // wait for all of them.
  __shared__ float s_sc[QPW == 1 ? SCORE_STAGE : 1];
  __shared__ uint32_t s_gk[QPW == 1 ? SCORE_STAGE / GROUP : 1];
  auto score_blocks = [&](KeyOperand<C_I>(&kf)[PF], int k0) {
    f32x4 acc[PF][HB];
#pragma unroll
    for (int u = 0; u < PF; ++u)
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) acc[u][hb] = KeyOperand<C_I>::mma(a[hb], kf[u], f32x4{0.f, 0.f, 0.f, 0.f});
    // the refill may not move above the MFMAs that read the buffer: then the loads can
    // reuse its registers, and no load result is copied (waited for) at the loop edge
    __builtin_amdgcn_sched_barrier(0);
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
      if (g == 0 && valid) {
        if (QPW == 1) s_sc[e - e_begin] = score;
        else srow[e] = score;
      }
      // group maximum over the group's usable keys (a prefix of its 16)
      const float best = row16_max(valid ? score : -INFINITY);
      if (lane == 0 && valid) {
        if (QPW == 1) s_gk[(e0 - e_begin) / GROUP] = score_key(best);
        else grow[e0 / GROUP] = score_key(best);
      }
    }
  };
  // both buffers every iteration (blocks past nmine are masked), so that each buffer is
  // refilled in place and no load result has to be copied at the loop edge
  for (int k0 = 0; k0 < nmine; k0 += 2 * PF) {
    score_blocks(kf0, k0);
    score_blocks(kf1, k0 + PF);
  }
  if (QPW == 1) {  // coalesced write-out of the staged chunk
    __syncthreads();
    const int n = e_end - e_begin;
    for (int i = (int)threadIdx.x; i < n; i += 256) srow[e_begin + i] = s_sc[i];
    for (int i = (int)threadIdx.x; i < cdiv(n, GROUP); i += 256) grow[e_begin / GROUP + i] = s_gk[i];
  }
}

// ---------------------------------------------------------------------------------------
// scoring at decode, c_I = 128: key blocks streamed by row DMA into per-wave LDS rings
// ---------------------------------------------------------------------------------------
// One query per workgroup of 4 waves; wave w scores key blocks w, w+4, ... of the
// workgroup's chunk.  Each wave keeps RING - 1 blocks of 16 keys (2 KiB each) in flight
// with global_load_lds (the data bypasses registers, so no register rotation can force
// a drain) and waits for its own oldest block with an explicit vmcnt; the rings are
// private to a wave, so there is no barrier until the final write-out.  Inside a block,
// row r holds its 16-byte chunks in the order c ^ (r & 7): a lane reading 32 bytes of its
// key row then hits eight distinct bank groups per eight lanes.
// Four blocks per wave ring (three in flight, 12 KiB of DMA per workgroup): with the
// workgroup's LDS at 49 KiB, three workgroups fit a CU.  Measured at the 1M and 128K
// decode shapes: rings of 3 and 4 blocks 28.7 us per launch, 5 blocks 29.6, 6 blocks 30.1,
// 7 blocks 30.8.
#ifndef CSAHCA_SCORE_RING
#define CSAHCA_SCORE_RING 4  // key blocks per wave ring (RING - 1 in flight)
#endif
constexpr int RING = CSAHCA_SCORE_RING;

// s_waitcnt vmcnt(2 * min(n, MAXN)): n blocks (two row loads each) may stay in flight
template <int N>
CSAHCA_DEV void wait_vm_exact() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * N) : "memory");
}
template <int MAXN>
CSAHCA_DEV void wait_vm_le(int n) {
  static_assert(MAXN >= 0 && 2 * MAXN <= 63, "vmcnt holds at most 63");
  if constexpr (MAXN == 0) {
    wait_vm_exact<0>();
  } else {
    if (n >= MAXN) wait_vm_exact<MAXN>();
    else wait_vm_le<MAXN - 1>(n);
  }
}

// LISTS: the per-chunk half of the top-k selection runs in the same launch
// (fused_topk.hpp): every workgroup also lists the best entries of its chunk.
// SPT: the chunk's scores per thread in the write-out and the list (CH <= 256 * SPT), so
// that those loops run over no slot past the chunk.
template <int HB, bool F4, bool LISTS, int SPT>
__global__ __launch_bounds__(256, 2) void index_score_dec128(
    const uint8_t* __restrict__ qI, const float* __restrict__ w, const uint8_t* __restrict__ KI,
    const uint8_t* __restrict__ KS,
    const int* __restrict__ q_pos, int m, int N_c, int CH, int NG, float* __restrict__ scores,
    uint32_t* __restrict__ gkeys, ChunkLists cl) {
  static_assert(!LISTS || FT_NT == 256, "the chunk cut runs on the scoring workgroup");
  constexpr int C_I = 128, NIH = HB * 16;
  // a block of 16 keys: FP8 rows of 128 bytes, or FP4 rows of 64 bytes followed by a
  // 256-byte slot whose first 64 bytes are the 16 keys' four E8M0 scales each
  constexpr int KRB = F4 ? C_I / 2 : C_I, BLKB = GROUP * KRB + (F4 ? 256 : 0);
  __shared__ __attribute__((aligned(16))) uint8_t ring[4][RING][BLKB];
  __shared__ __attribute__((aligned(16))) uint8_t s_q[NIH * C_I];
  __shared__ float s_w[cdiv(NIH, 64) * 64];
  static_assert(SPT * 256 <= SCORE_STAGE, "a chunk's scores fit the LDS stage");
  __shared__ float s_sc[SPT * 256];
  __shared__ uint32_t s_gk[SPT * 256 / GROUP];
  CSAHCA_TRACE(0);
  CSAHCA_TRACE_RT(14);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int q = blockIdx.y;  // decode: one query token per sequence, b = q
  const int e_begin = blockIdx.x * CH;
  const int e_lim = min(e_begin + CH, N_c);
  const int row = lane & 15, g = lane >> 4;
  // read before any DMA is issued, so that it can be a scalar load with its own counter
  const int V = visible_entries(q_pos, q, 0, m, N_c);

  // blocks of this wave: wave + 4k, k < nmine; loads are clamped to the chunk's last key
  // (the first blocks are issued before the visible count is applied)
  int nmine = 0, e_last = e_lim - 1;
  auto count_mine = [&](int nblk) { return nblk > wave ? cdiv(nblk - wave, 4) : 0; };
  nmine = count_mine(cdiv(e_lim - e_begin, GROUP));
  const uint8_t* kb = KI + (size_t)q * N_c * KRB;
  const uint8_t* ksb = KS + (size_t)q * N_c * 4;  // FP4: four scale bytes per key
  // FP8, in each 1 KiB half of a block: lane l moves row l/8, chunk (l%8) ^ (l/8).
  // FP4: lane l moves row l/4, chunk l%4 (the 1 KiB is read back whole, conflict-free),
  // and lanes 0..15 move the scale words of rows 0..15 (the others repeat row 15).
  const int dma_row = F4 ? lane >> 2 : lane >> 3;
  const int dma_chunk = F4 ? lane & 3 : (lane & 7) ^ (lane >> 3);
  auto issue = [&](int k) {
    const int e0 = e_begin + (wave + 4 * min(k, nmine - 1)) * GROUP;
    uint8_t* dst = ring[wave][k % RING];
    if constexpr (F4) {
      const int e = min(e0 + dma_row, e_last);
      __builtin_amdgcn_global_load_lds(kb + (size_t)e * KRB + dma_chunk * 16,
                                       (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
      const int es = min(e0 + min(lane, GROUP - 1), e_last);
      __builtin_amdgcn_global_load_lds(ksb + (size_t)es * 4,
                                       (__attribute__((address_space(3))) void*)(dst + GROUP * KRB),
                                       4, 0, 0);
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int e = min(e0 + 8 * h + dma_row, e_last);
        __builtin_amdgcn_global_load_lds(kb + (size_t)e * C_I + dma_chunk * 16,
                                         (__attribute__((address_space(3))) void*)(dst + h * 1024),
                                         16, 0, 0);
      }
    }
  };
  // The query's indexer vectors and head weights come by DMA too, ahead of the key
  // blocks: with only DMA in flight, one counted wait covers exactly them.  Wave w moves
  // the 1 KiB pieces w, w+4, ... of q_I and the 64-weight pieces w, w+4, ... of w.
  constexpr int QPIECES = NIH * C_I / 1024, WPIECES = cdiv(NIH, 64);
  int nown = 0;
  const uint8_t* qsrc = qI + (size_t)q * NIH * C_I;
  for (int i = wave; i < QPIECES; i += 4, ++nown)
    __builtin_amdgcn_global_load_lds(qsrc + i * 1024 + lane * 16,
                                     (__attribute__((address_space(3))) void*)(s_q + i * 1024),
                                     16, 0, 0);
  for (int i = wave; i < WPIECES; i += 4, ++nown)
    __builtin_amdgcn_global_load_lds(w + (size_t)q * NIH + min(i * 64 + lane, NIH - 1),
                                     (__attribute__((address_space(3))) void*)(s_w + i * 64),
                                     4, 0, 0);
  const int nfill = min(RING - 1, nmine);
  for (int k = 0; k < nfill; ++k) issue(k);
  CSAHCA_TRACE(1);
  wait_vm_le<RING - 1>(nfill);  // this wave's q_I / w pieces have landed
  // ... and every other wave's (a bare barrier: __syncthreads would also drain the ring)
  asm volatile("s_barrier" ::: "memory");
  // A operand: indexer query of head (16*hb + row), dims [g*32, g*32 + 32); head weights
  // of the accumulator rows this lane holds: heads 16*hb + 4*g + i
  KeyOperand<C_I> a[HB];
  float wr[HB][4];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const uint8_t* qr = s_q + (hb * 16 + row) * C_I;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(qr + (F4 ? 16 * g : 32 * g));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(qr + (F4 ? 64 + 16 * g : 32 * g + 16));
    a[hb].v = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
#pragma unroll
    for (int i = 0; i < 4; ++i) wr[hb][i] = s_w[hb * 16 + 4 * g + i];
  }

  const int e_end = min(e_lim, V);
  if (e_begin >= e_end) {  // uniform: nothing usable in this chunk
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no DMA may target LDS at exit
    return;
  }
  const int nmine_lim = nmine;
  nmine = count_mine(cdiv(e_end - e_begin, GROUP));
  // reader offsets of this lane's 32 bytes (chunks 2g, 2g+1 of row `row`); FP4: its 16
  // bytes (elements 32g .. 32g+31 of row `row`) and its block's scale byte
  const int rd0 = F4 ? row * KRB + g * 16 : (row * 8 + ((2 * g) ^ (row & 7))) * 16;
  const int rd1 = F4 ? GROUP * KRB + row * 4 + g : (row * 8 + ((2 * g + 1) ^ (row & 7))) * 16;
  for (int k = 0; k < nmine; ++k) {
    // blocks k+1 .. min(nmine_lim, k+RING-1)-1 may stay in flight
    wait_vm_le<RING - 2>(min(nmine_lim, k + RING - 1) - 1 - k);
    const uint8_t* blk = ring[wave][k % RING];
    f32x4 acc[HB];
    if constexpr (F4) {
      const u32x4 kv = *reinterpret_cast<const u32x4*>(blk + rd0);
      const uint32_t ks = blk[rd1];
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) acc[hb] = mma_fp8_fp4(a[hb].v, kv, ks, f32x4{0.f, 0.f, 0.f, 0.f});
    } else {
      KeyOperand<C_I> kf;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(blk + rd0);
      const u32x4 hi = *reinterpret_cast<const u32x4*>(blk + rd1);
      kf.v = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) acc[hb] = KeyOperand<C_I>::mma(a[hb], kf, f32x4{0.f, 0.f, 0.f, 0.f});
    }
    // slot (k-1) % RING was read in the previous iteration: refill it
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (k + RING - 1 < nmine_lim) issue(k + RING - 1);
    // lane holds key (row) for heads 16*hb + 4*g + i; sum over heads as a balanced tree
    float t[4 * HB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int i = 0; i < 4; ++i) t[4 * hb + i] = wr[hb][i] * fmaxf(acc[hb][i], 0.f);
#pragma unroll
    for (int wdt = 2 * HB; wdt >= 1; wdt /= 2)
#pragma unroll
      for (int v = 0; v < wdt; ++v) t[v] += t[v + wdt];
    const float score = sum_over_row_groups(t[0]);  // same value in lanes row, row+16, ...
    const int e0 = e_begin + (wave + 4 * k) * GROUP;
    const bool valid = e0 + row < e_end;
    if (g == 0 && valid) s_sc[e0 - e_begin + row] = score;
    // group maximum over the group's usable keys (a prefix of its 16)
    const float best = row16_max(valid ? score : -INFINITY);
    if (lane == 0 && valid) s_gk[(e0 - e_begin) / GROUP] = score_key(best);
    if (k == 0) CSAHCA_TRACE(2);
  }
  CSAHCA_TRACE(3);
  // the loop waited for every block up to nmine - 1; blocks past it (issued before the
  // visible count was known) are waited for here, before the workgroup barrier
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  const int n = e_end - e_begin;
  float* srow = scores + (size_t)q * N_c;
  uint32_t* grow = gkeys + (size_t)q * NG;
  // the chunk's scores, entry threadIdx.x + 256 j: all LDS reads issued before the first
  // store (one wait, not one per store), kept for the list below
  float sv[SPT];
#pragma unroll
  for (int j = 0; j < SPT; ++j) {
    const int i = (int)threadIdx.x + 256 * j;
    sv[j] = i < n ? s_sc[i] : 0.f;
  }
#pragma unroll
  for (int j = 0; j < SPT; ++j) {
    const int i = (int)threadIdx.x + 256 * j;
    if (i < n) srow[e_begin + i] = sv[j];
  }
  for (int i = (int)threadIdx.x; i < cdiv(n, GROUP); i += 256) grow[e_begin / GROUP + i] = s_gk[i];
  if constexpr (LISTS) {
    const int keff = min(cl.k, V);
    if (keff < V) {  // (with keff == V the selection takes every usable entry)
      // the key ring is free (every DMA has landed and the workgroup passed the barrier)
      FtScratch& sc = *reinterpret_cast<FtScratch*>(&ring[0][0][0]);
      static_assert(sizeof(FtScratch) <= sizeof(ring), "the cut's scratch fits the key ring");
      uint32_t u[SPT];
      uint64_t kr[SPT];
#pragma unroll
      for (int j = 0; j < SPT; ++j) {
        const int i = (int)threadIdx.x + 256 * j;
        u[j] = i < n ? score_key(sv[j]) : 0u;
        kr[j] = i < n ? ((uint64_t)u[j] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)(e_begin + i)) : 0ull;
      }
      // list about this query's share of the top k per chunk plus four standard
      // deviations (the host sized the lists for the whole cache; a shorter sequence has
      // fewer chunks, each holding more of its top k)
      const int P_eff = cdiv(V, CH);
      const float per = (float)keff / (float)P_eff;
      const int JT = min(cl.JMAX, (int)(per + 4.f * sqrtf(per) + 8.f) + 1);
      const FtCut cut = ft_local_cut(u, n, JT, cl.JMAX, sc);
      const int chunk = blockIdx.x;
      uint64_t* list = cl.cand + ((size_t)q * cl.P + chunk) * cl.JMAX;
      ft_compact(
          kr, [&](uint64_t key) { return key != 0ull && (key >> 32) >= cut.cut; },
          [&](uint32_t pos, uint64_t key) { list[pos] = key; }, sc);
      for (int i = (int)cut.count + (int)threadIdx.x; i < cl.JMAX; i += 256) list[i] = 0ull;  // padding
      if (threadIdx.x == 0) cl.edge[(size_t)q * FT_MAX_P + chunk] = cut.cut == 0ull ? 0ull : cut.cut << 32;
    }
    if (threadIdx.x == 0 && blockIdx.x == 0) cl.path[q] = FT_LISTS_READY;
  }
  CSAHCA_TRACE(4);
  CSAHCA_TRACE_RT(15);
}

// ---------------------------------------------------------------------------------------
// scoring at prefill, c_I = 128: four queries per workgroup share key stages in LDS
// ---------------------------------------------------------------------------------------
// Wave w scores query 4*blockIdx.x + w (same sequence) over a range of PRE_KEYS keys.  Key
// stages of PRE_STG keys (four 16-key blocks, 8 KiB) arrive by row DMA into a ring of
// PRE_NSTG stages that all four waves read, so every key byte crosses the memory path once
// per four queries; one barrier per stage hands a slot back for refill.  Per stage a wave
// runs the 4 x HB MFMAs, reduces each lane's 4*HB accumulators over its heads, and then
// one reduce-scatter over the four row groups (two permlane16 swaps, one permlane32 swap)
// leaves every lane with the complete score of one key: lane l holds key 64*stage + l, so
// a stage's 64 scores leave in one coalesced store.  The waits on the row DMA count only
// the DMA issued after the awaited stage: as vector loads complete in order among
// themselves, that bound holds whatever the order in which the stores complete.
constexpr int PRE_STG = 64;
constexpr int PRE_NSTG = 4;
constexpr int PRE_KEYS = 8192;

template <int HB, bool F4>
__global__ __launch_bounds__(256, HB >= 8 ? 2 : 4) void index_score_pre128(
    const uint8_t* __restrict__ qI, const float* __restrict__ w, const uint8_t* __restrict__ KI,
    const uint8_t* __restrict__ KS,
    const int* __restrict__ q_pos, int m, int Tq, int N_c, int NG, float* __restrict__ scores,
    uint32_t* __restrict__ gkeys) {
  // a stage: FP8 rows of 128 bytes, or FP4 rows of 64 bytes then one 256-byte slot per
  // wave whose first 64 bytes hold the wave's 16 keys' four E8M0 scales each (a 4-byte
  // row DMA writes all 64 lanes; the rest of the slot takes repeats)
  constexpr int C_I = 128, NIH = HB * 16, NBS = PRE_STG / GROUP;
  constexpr int KRB = F4 ? C_I / 2 : C_I, STGB = PRE_STG * KRB + (F4 ? 4 * 256 : 0);
  static_assert(NBS == 4, "the reduce-scatter spreads four blocks over the four row groups");
  __shared__ __attribute__((aligned(16))) uint8_t ring[PRE_NSTG][STGB];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int row = lane & 15, g = lane >> 4;
  const int qgs = cdiv(Tq, 4);  // query groups per sequence
  const int b = blockIdx.x / qgs;
  const int t0 = (blockIdx.x - b * qgs) * 4;
  const int tl = min(t0 + 3, Tq - 1);       // the workgroup's last query
  const int t = min(t0 + wave, tl);         // waves past Tq repeat it and store nothing
  const bool qact = t0 + wave < Tq;
  const int q = b * Tq + t;
  const int e_begin = blockIdx.y * PRE_KEYS;
  // read before any DMA is issued, so that they can be scalar loads with their own counter
  const int Vmax = visible_entries(q_pos, b, tl, m, N_c);
  const int Vw = qact ? visible_entries(q_pos, b, t, m, N_c) : 0;
  if (e_begin >= Vmax) return;  // uniform over the workgroup, before any barrier
  const int nst = cdiv(min(e_begin + PRE_KEYS, Vmax) - e_begin, PRE_STG);

  // A operand: indexer query of head (16*hb + row), dims [g*32, g*32 + 32); head weights
  // of the accumulator rows this lane holds: heads 16*hb + 4*g + i
  KeyOperand<C_I> a[HB];
  f32x4 wr[HB];
  const uint8_t* qp = qI + (size_t)q * NIH * C_I;
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    if constexpr (F4) {
      const uint8_t* qr = qp + (hb * 16 + row) * C_I;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(qr + 16 * g);
      const u32x4 hi = *reinterpret_cast<const u32x4*>(qr + 64 + 16 * g);
      a[hb].v = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    } else {
      a[hb].load(qp + (hb * 16 + row) * C_I + g * 32);
    }
    wr[hb] = *reinterpret_cast<const f32x4*>(w + (size_t)q * NIH + hb * 16 + 4 * g);
  }

  // stage s: rows e_begin + 64*s + r; wave w moves the 1 KiB pieces w and w + 4 (rows
  // 8p .. 8p+7); in a piece lane l moves row l/8, 16-byte chunk (l%8) ^ (l/8), so that a
  // reader of 32 bytes of its row hits eight distinct bank groups per eight lanes
  const uint8_t* kb = KI + (size_t)b * N_c * KRB;
  const uint8_t* ksb = KS + (size_t)b * N_c * 4;
  // FP4: wave w moves the 1 KiB of rows 16w .. 16w+15 (lane l: row l/4, chunk l%4) and
  // lanes 0..15 the scale words of the same rows
  const int dma_row = F4 ? lane >> 2 : lane >> 3;
  const int dma_chunk = F4 ? lane & 3 : (lane & 7) ^ (lane >> 3);
  auto issue = [&](int st) {
    uint8_t* dst = ring[st % PRE_NSTG];
    if constexpr (F4) {
      const int e = min(e_begin + st * PRE_STG + 16 * wave + dma_row, N_c - 1);
      __builtin_amdgcn_global_load_lds(kb + (size_t)e * KRB + dma_chunk * 16,
                                       (__attribute__((address_space(3))) void*)(dst + wave * 1024),
                                       16, 0, 0);
      const int es = min(e_begin + st * PRE_STG + 16 * wave + min(lane, GROUP - 1), N_c - 1);
      __builtin_amdgcn_global_load_lds(
          ksb + (size_t)es * 4,
          (__attribute__((address_space(3))) void*)(dst + PRE_STG * KRB + wave * 256), 4, 0, 0);
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int p = wave + 4 * h;
        const int e = min(e_begin + st * PRE_STG + 8 * p + dma_row, N_c - 1);
        __builtin_amdgcn_global_load_lds(kb + (size_t)e * C_I + dma_chunk * 16,
                                         (__attribute__((address_space(3))) void*)(dst + p * 1024),
                                         16, 0, 0);
      }
    }
  };
  const int nfill = min(PRE_NSTG - 1, nst);
  for (int st = 0; st < nfill; ++st) issue(st);
  // the compiler does not order register loads and row DMAs: its wait for the query and
  // weights (forced here, once) also covers the first stages, which are needed next anyway
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) asm volatile("" : "+v"(a[hb].v), "+v"(wr[hb]));

  float* srow = scores + (size_t)q * N_c;
  uint32_t* grow = gkeys + (size_t)q * NG;
  // reader offsets of this lane's 32 bytes (chunks 2g, 2g+1 of row `row` of a block)
  const int rd0 = (row * 8 + ((2 * g) ^ (row & 7))) * 16;
  const int rd1 = (row * 8 + ((2 * g + 1) ^ (row & 7))) * 16;
  for (int st = 0; st < nst; ++st) {
    // stages st+1 .. min(nst, st+NSTG-1)-1 may stay in flight
    wait_vm_le<PRE_NSTG - 2>(min(nst - 1, st + PRE_NSTG - 2) - st);
    // every wave's part of stage st has landed, and every wave is done with stage st-1
    asm volatile("s_barrier" ::: "memory");
    if (st + PRE_NSTG - 1 < nst) issue(st + PRE_NSTG - 1);
    const uint8_t* stg = ring[st % PRE_NSTG];
    f32x4 acc[NBS][HB];
    if constexpr (F4) {
      u32x4 kv[NBS];
      uint32_t ks[NBS];
#pragma unroll
      for (int u = 0; u < NBS; ++u) {
        kv[u] = *reinterpret_cast<const u32x4*>(stg + (u * GROUP + row) * KRB + g * 16);
        ks[u] = stg[PRE_STG * KRB + u * 256 + row * 4 + g];
      }
#pragma unroll
      for (int u = 0; u < NBS; ++u)
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) acc[u][hb] = mma_fp8_fp4(a[hb].v, kv[u], ks[u], f32x4{0.f, 0.f, 0.f, 0.f});
    } else {
      KeyOperand<C_I> kf[NBS];
#pragma unroll
      for (int u = 0; u < NBS; ++u) {
        const u32x4 lo = *reinterpret_cast<const u32x4*>(stg + u * (GROUP * C_I) + rd0);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(stg + u * (GROUP * C_I) + rd1);
        kf[u].v = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
#pragma unroll
      for (int u = 0; u < NBS; ++u)
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) acc[u][hb] = KeyOperand<C_I>::mma(a[hb], kf[u], f32x4{0.f, 0.f, 0.f, 0.f});
    }
    // this lane's heads (16*hb + 4*g + i) of key `row` of block u
    float pu[NBS];
#pragma unroll
    for (int u = 0; u < NBS; ++u) {
      float th[HB];
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        float x = wr[hb][0] * fmaxf(acc[u][hb][0], 0.f);
#pragma unroll
        for (int i = 1; i < 4; ++i) x = fmaf(wr[hb][i], fmaxf(acc[u][hb][i], 0.f), x);
        th[hb] = x;
      }
#pragma unroll
      for (int wdt = HB / 2; wdt >= 1; wdt /= 2)
#pragma unroll
        for (int v = 0; v < wdt; ++v) th[v] += th[v + wdt];
      pu[u] = th[0];
    }
    // reduce-scatter over the row groups: afterwards row group r holds block r
    const auto x01 = __builtin_amdgcn_permlane16_swap(__float_as_uint(pu[0]), __float_as_uint(pu[1]), false, false);
    const auto x23 = __builtin_amdgcn_permlane16_swap(__float_as_uint(pu[2]), __float_as_uint(pu[3]), false, false);
    const float s01 = __uint_as_float(x01[0]) + __uint_as_float(x01[1]);
    const float s23 = __uint_as_float(x23[0]) + __uint_as_float(x23[1]);
    const auto y = __builtin_amdgcn_permlane32_swap(__float_as_uint(s01), __float_as_uint(s23), false, false);
    const float score = __uint_as_float(y[0]) + __uint_as_float(y[1]);
    const int e = e_begin + st * PRE_STG + lane;
    const bool valid = e < Vw;
    if (valid) srow[e] = score;
    // group maximum of each row group's usable keys (a prefix of its 16)
    const float best = row16_max(valid ? score : -INFINITY);
    if (row == 0 && valid) grow[e / GROUP] = score_key(best);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no DMA may target LDS at exit
}

// ---------------------------------------------------------------------------------------
// scoring, float32 keys (small heads; plain FMA)
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void index_score_f32(
    const float* __restrict__ qI, const float* __restrict__ w, const float* __restrict__ KI,
    const int* __restrict__ q_pos, int m, int Tq, int N_c, int n_ih, int c_I, int NG,
    float* __restrict__ scores, uint32_t* __restrict__ gkeys) {
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
  uint32_t key = valid ? score_key(s) : 0u;
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) key = max(key, (uint32_t)__shfl_xor((int)key, d, 64));
  if ((threadIdx.x & 15) == 0 && e < V) gkeys[(size_t)q * NG + e / GROUP] = key;
}


// ---------------------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------------------
template <int C_I, int HB, bool F4>
void launch_fp8(const void* q_idx, const float* w_idx, const void* k_idx, const int* q_pos,
                int m, int Tq, int N_c, int nq, int NG, float* scores, uint32_t* gkeys,
                hipStream_t st, const ChunkLists* cl) {
  const bool decode = Tq == 1;
  const int QPW = decode ? 1 : 4;
  const int qgroups = cdiv(nq, QPW);
  // about two workgroups per CU, each streaming a long chunk of keys (decode: at most
  // SCORE_STAGE keys, the LDS staging of its scores; the chunks of the decode kernel
  // follow the plan its fused selection is sized by)
  int chunks = cdiv(SCORE_WGS, qgroups);
  chunks = max(1, min(chunks, cdiv(N_c, 256)));
  if (decode) chunks = max(chunks, cdiv(N_c, SCORE_STAGE));
  int CH = cdiv(cdiv(N_c, chunks), 64) * 64;
  if (decode && C_I == 128) CH = topk_plan_decode(nq, N_c, cl ? cl->k : 1).CH;
  chunks = cdiv(N_c, CH);
  dim3 grid((unsigned)chunks, (unsigned)qgroups);
  const uint8_t* KI = (const uint8_t*)k_idx;
  // MX FP4 keys: [B, N_c, 64] E2M1 rows, then [B, N_c, 4] E8M0 scales
  const uint8_t* KS = F4 ? KI + (size_t)(nq / Tq) * N_c * (C_I / 2) : nullptr;
  if (decode && C_I == 128) {
    // the chunk's scores per thread in the write-out and the list: 8 for chunks of up to
    // 2048 keys (the plans of the 128K and 1M decode shapes), else 16
    const ChunkLists cla = cl ? *cl : ChunkLists{};
    auto kern = cl ? (CH <= 2048 ? index_score_dec128<HB, F4, true, 8> : index_score_dec128<HB, F4, true, 16>)
                   : (CH <= 2048 ? index_score_dec128<HB, F4, false, 8> : index_score_dec128<HB, F4, false, 16>);
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, (const uint8_t*)q_idx, w_idx, KI, KS, q_pos, m, N_c, CH,
                       NG, scores, gkeys, cla);
  }
  else if (C_I == 128)
    hipLaunchKernelGGL((index_score_pre128<HB, F4>),
                       dim3((unsigned)(nq / Tq * cdiv(Tq, 4)), (unsigned)cdiv(N_c, PRE_KEYS)), dim3(256), 0, st,
                       (const uint8_t*)q_idx, w_idx, KI, KS, q_pos, m, Tq, N_c, NG, scores, gkeys);
  else if (decode)
    hipLaunchKernelGGL((index_score_fp8<C_I, HB, 1, 4>), grid, dim3(256), 0, st,
                       (const uint8_t*)q_idx, w_idx, KI, q_pos, m, Tq, N_c, CH, nq, NG, scores, gkeys);
  else
    hipLaunchKernelGGL((index_score_fp8<C_I, HB, 4, 4>), grid, dim3(256), 0, st,
                       (const uint8_t*)q_idx, w_idx, KI, q_pos, m, Tq, N_c, CH, nq, NG, scores, gkeys);
}

template <int C_I, bool F4>
bool launch_fp8_heads(int n_ih, const void* q_idx, const float* w_idx, const void* k_idx,
                      const int* q_pos, int m, int Tq, int N_c, int nq, int NG, float* scores,
                      uint32_t* gkeys, hipStream_t st, const ChunkLists* cl) {
  switch (n_ih / 16) {
    case 1: launch_fp8<C_I, 1, F4>(q_idx, w_idx, k_idx, q_pos, m, Tq, N_c, nq, NG, scores, gkeys, st, cl); return true;
    case 2: launch_fp8<C_I, 2, F4>(q_idx, w_idx, k_idx, q_pos, m, Tq, N_c, nq, NG, scores, gkeys, st, cl); return true;
    case 4: launch_fp8<C_I, 4, F4>(q_idx, w_idx, k_idx, q_pos, m, Tq, N_c, nq, NG, scores, gkeys, st, cl); return true;
    case 8: launch_fp8<C_I, 8, F4>(q_idx, w_idx, k_idx, q_pos, m, Tq, N_c, nq, NG, scores, gkeys, st, cl); return true;
    default: return false;
  }
}

}  // namespace

namespace csahca {

int index_check_common(const void* q_idx, const float* w_idx, const void* k_idx, int idx_dtype,
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
    if (n_ih != 16 && n_ih != 32 && n_ih != 64 && n_ih != 128)
      return fail(CSAHCA_ENOTSUP, "indexer: FP8 keys need n_ih in {16, 32, 64, 128}");
    if (c_I != 32 && c_I != 64 && c_I != 128)
      return fail(CSAHCA_ENOTSUP, "indexer: FP8 keys need c_I in {32, 64, 128}");
  } else if (idx_dtype == CSAHCA_MXFP4) {
    if ((n_ih != 16 && n_ih != 32 && n_ih != 64 && n_ih != 128) || c_I != 128)
      return fail(CSAHCA_ENOTSUP, "indexer: MX FP4 keys need n_ih in {16, 32, 64, 128} and c_I == 128");
  } else if (idx_dtype == CSAHCA_F32) {
    if (n_ih * c_I > 4096)
      return fail(CSAHCA_ENOTSUP, "indexer: float32 keys need n_ih * c_I <= 4096");
  } else {
    return fail(CSAHCA_ENOTSUP, "indexer: idx_dtype must be CSAHCA_FP8_E4M3FN, CSAHCA_MXFP4 or CSAHCA_F32");
  }
  if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned16(w_idx))
    return fail(CSAHCA_EINVAL, "indexer: q_idx, w_idx and k_idx must be 16-byte aligned");
  return CSAHCA_OK;
}


bool index_can_list(int idx_dtype, int Tq, int c_I, int n_ih, const TopkPlan& plan) {
  return plan.lists && Tq == 1 && c_I == 128 && (n_ih == 16 || n_ih == 32 || n_ih == 64 || n_ih == 128) &&
         (idx_dtype == CSAHCA_FP8_E4M3FN || idx_dtype == CSAHCA_MXFP4);
}

int index_score_impl(const void* q_idx, const float* w_idx, const void* k_idx, int idx_dtype,
                     const int* q_pos, int m, int B, int Tq, int n_ih, int c_I, int N_c,
                     float* scores, uint32_t* gkeys, hipStream_t st, const ChunkLists* cl) {
  using namespace csahca;
  const int nq = B * Tq;
  const int NG = cdiv(N_c, GROUP);
  if (idx_dtype == CSAHCA_FP8_E4M3FN) {
    bool ok = false;
    if (c_I == 128) ok = launch_fp8_heads<128, false>(n_ih, q_idx, w_idx, k_idx, q_pos, m, Tq, N_c, nq, NG, scores, gkeys, st, cl);
    else if (c_I == 64) ok = launch_fp8_heads<64, false>(n_ih, q_idx, w_idx, k_idx, q_pos, m, Tq, N_c, nq, NG, scores, gkeys, st, nullptr);
    else ok = launch_fp8_heads<32, false>(n_ih, q_idx, w_idx, k_idx, q_pos, m, Tq, N_c, nq, NG, scores, gkeys, st, nullptr);
    if (!ok) return fail(CSAHCA_ENOTSUP, "indexer: FP8 keys need n_ih in {16, 32, 64, 128}");
  } else if (idx_dtype == CSAHCA_MXFP4) {
    if (!launch_fp8_heads<128, true>(n_ih, q_idx, w_idx, k_idx, q_pos, m, Tq, N_c, nq, NG, scores, gkeys, st, cl))
      return fail(CSAHCA_ENOTSUP, "indexer: MX FP4 keys need n_ih in {16, 32, 64, 128}");
  } else {
    const size_t lds = (size_t)(n_ih * c_I + n_ih) * sizeof(float);
    dim3 grid((unsigned)cdiv(N_c, 256), (unsigned)nq);
    hipLaunchKernelGGL(index_score_f32, grid, dim3(256), lds, st, (const float*)q_idx, w_idx,
                       (const float*)k_idx, q_pos, m, Tq, N_c, n_ih, c_I, NG, scores, gkeys);
  }
  return launch_status("lightning_index_score");
}

}  // namespace csahca

namespace {

// one word per thread set to zero (a fill kernel rather than hipMemsetAsync, so that a
// captured graph holds only kernels)
__global__ __launch_bounds__(256) void clear_words(uint32_t* p, int n) {
  const int i = (int)(blockIdx.x * 256 + threadIdx.x);
  if (i < n) p[i] = 0u;
}

}  // namespace

namespace csahca {

// The chunk lists of a decode workspace (null fields when the layout has none)
ChunkLists chunk_lists_of(char* ws, const WsLayout& L, int k) {
  ChunkLists cl{};
  if (!L.plan.lists) return cl;
  cl.edge = (uint64_t*)(ws + L.edge_off);
  cl.cand = (uint64_t*)(ws + L.cand_off);
  cl.path = (uint32_t*)(ws + L.path_off);
  cl.k = k;
  cl.P = L.plan.P;
  cl.JMAX = L.plan.JMAX;
  cl.CH = L.plan.CH;
  return cl;
}

}  // namespace csahca

extern "C" int lightning_index_score(const void* q_idx, const float* w_idx, const void* k_idx,
                                     int idx_dtype, const int* q_pos, int m, int B, int Tq,
                                     int n_ih, int c_I, int N_c, int k, float* scores,
                                     void* workspace, size_t ws_bytes, void* stream) {
  using namespace csahca;
  int st = index_check_common(q_idx, w_idx, k_idx, idx_dtype, q_pos, m, B, Tq, n_ih, c_I, N_c, k);
  if (st != CSAHCA_OK) return st;
  if (!scores) return fail(CSAHCA_EINVAL, "lightning_index_score: scores must be non-NULL");
  const WsLayout L = ws_layout((long long)B * Tq, N_c, k, Tq == 1);
  if (!workspace || ws_bytes < L.total)
    return fail(CSAHCA_EWORKSPACE, "lightning_index_score: workspace missing or too small");
  // as in lightning_index_topk, the decode launch also writes the chunk lists (and marks
  // each query's lists ready); a decode layout without them clears the marks
  char* ws = (char*)workspace;
  uint32_t* gkeys = (uint32_t*)(ws + L.gkeys_off);
  const hipStream_t s = (hipStream_t)stream;
  const ChunkLists cl = chunk_lists_of(ws, L, k);
  if (cl.cand && index_can_list(idx_dtype, Tq, c_I, n_ih, L.plan))
    return index_score_impl(q_idx, w_idx, k_idx, idx_dtype, q_pos, m, B, Tq, n_ih, c_I, N_c, scores, gkeys, s,
                            &cl);
  st = index_score_impl(q_idx, w_idx, k_idx, idx_dtype, q_pos, m, B, Tq, n_ih, c_I, N_c, scores, gkeys, s);
  if (st != CSAHCA_OK || !cl.path) return st;
  const int nq = B * Tq;
  hipLaunchKernelGGL(clear_words, dim3((unsigned)cdiv(nq, 256)), dim3(256), 0, s, cl.path, nq);
  return launch_status("lightning_index_score");
}
