// Kernels 3 and 4: multi-query attention over compressed entries plus the raw window.
//
// Source: "DeepSeek-V4 Hybrid Attention: CSA, HCA, mHC, MoE": section I (softmax of the
// scaled dot products, weighted sum of values), section V.3 (CSA core attention over the
// selected blocks, MQA: every head shares one compressed K = V row), section VI
// (equation o_{t,i}: key = value = the compressed entries, dense over all of them);
// "DeepSeek-V4: Anatomy of an Open-Source Frontier Model", "One query in a CSA layer",
// steps 3-5: the selected entries and the last 128 raw tokens are attended together.
//
// One joint softmax runs over the row list of a query: the compressed slots (CSA: the
// top-k list, -1 skipped; HCA: entries 0 .. N_h-1, those not yet complete skipped)
// followed by the window slots.  A workgroup takes a range of slots ("split") for one
// group of queries and a group of heads; splits are merged afterwards by log-sum-exp,
// which gives exactly the joint softmax.
//
// bf16 path (c = 512), per 32-slot tile:
//   * the 32 rows are read once from HBM straight into LDS (global_load_lds_dwordx4: each
//     wave instruction moves one 1 KiB row; rows keep a 16-byte pad), through a ring of
//     tiles so that the next tile is in flight while one is computed;
//   * every wave owns 16 (query, head) pairs.  S^T = E . Q^T on MFMA
//     (v_mfma_f32_16x16x32_bf16, A = 16 rows x 32 dims from LDS, B = Q from registers);
//     the accumulator layout puts one head per lane column, so the online-softmax
//     statistics of a head live in the lanes that also hold its output;
//   * O^T += E^T . P^T on MFMA: P stays in registers in exactly the layout the S
//     accumulator produced it; E^T comes from the same LDS tile through the gfx950
//     transpose read (ds_read_b64_tr_b16), two reads per MFMA.
// float32 path: plain FMA over LDS-resident scores (small heads only).
#include <mutex>

#include "normrope.hpp"

namespace {

constexpr int C = 512;            // head dim of the bf16 path
constexpr int TILE = 32;          // slots per LDS tile
constexpr int ROWB = C * 2 + 32;  // LDS row stride in bytes (rows are placed by row_base)
constexpr int KS = C / 32;        // MFMA K-steps of S (16 x 32 dims)

// LDS byte offset of row r of a tile.  Modulo the 256 bytes the 64 banks cover per cycle,
// row r starts at 32 (r % 8) + 16 ((r / 8) % 2): the S reads (16 bytes of 16 rows at one
// column per 16 lanes) hit the sixteen distinct 16-byte slots, and the transpose reads
// (32 bytes of 8 consecutive rows per 32 lanes) eight disjoint 32-byte windows.  With a
// plain 16-byte pad per row, neighbouring rows' 32-byte windows overlapped (a two-way
// bank conflict on every transpose read).  Rows stay 16-byte aligned for the row DMA,
// and row r + 16 lies exactly 16 strides after row r.
CSAHCA_DEV constexpr int row_base(int r) { return r * ROWB + 16 * ((r >> 3) & 1); }
static_assert(row_base(TILE - 1) + C * 2 <= TILE * ROWB, "a tile's rows fit its stage");
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// Per-head attention sink: a logit (natural-log units, the units of scale * q.k) that
// joins the softmax denominator only.  Folds it into a head's maximum m (log2 units) and
// sum l, and returns the factor that carries accumulators taken relative to the old
// maximum over to the new one.
CSAHCA_DEV float fold_sink(const float* sink, int h, float& m, float& l) {
  if (!sink) return 1.f;
  const float s2 = sink[h] * LOG2E;
  if (s2 == -INFINITY) return 1.f;
  const float M = fmaxf(m, s2);
  const float r = m == -INFINITY ? 0.f : exp2f(m - M);
  l = l * r + exp2f(s2 - M);
  m = M;
  return r;
}

// The same for a head that keeps two sums over one maximum: l, the mass of its fp32
// weights (for the log-sum-exp), and lq, the sum of the bf16-rounded weights the output
// was accumulated with (for normalising the output).
CSAHCA_DEV float fold_sink2(const float* sink, int h, float& m, float& l, float& lq) {
  if (!sink) return 1.f;
  const float s2 = sink[h] * LOG2E;
  if (s2 == -INFINITY) return 1.f;
  const float M = fmaxf(m, s2);
  const float r = m == -INFINITY ? 0.f : exp2f(m - M);
  const float e = exp2f(s2 - M);
  l = l * r + e;
  lq = lq * r + e;
  m = M;
  return r;
}

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* ckv;
  const int* topk;
  const uint16_t* win;
  const int* win_pos;
  const int* q_pos;
  uint16_t* out;
  float* lse;
  uint16_t* opart;  // [nq, n_splits, n_h, C] partial outputs O/l, scaled float16
  float* mlpart;    // [nq, n_splits, n_h, 4] running max (log2 units), sum, scale, pad
  const float* sink;  // [n_h] attention sink logits (natural-log units) or null
  // RMSNorm + partial RoPE of the queries as they are loaded (qnr; normrope.hpp), gain
  // nullable
  const float* q_gamma;
  int qnr, d_rope;
  float nr_eps, nr_theta;
  int B, Tq, n_h, Nc, k, L, W, m;
  int is_csa;
  int n_slots_c;  // compressed slots: k (CSA) or Nc (HCA)
  int n_slots;    // n_slots_c + W + Tg - 1
  int Tg;         // consecutive query tokens per workgroup (HCA prefill shares rows)
  int HPW;        // heads per workgroup
  int n_hg;       // head groups = n_h / HPW
  int nqg;        // query groups per sequence
  int n_splits, RS;
  int n_work;     // B * nqg * n_splits * n_hg
  int per_xcd;    // gridDim.x / 8
  float scale_log2;
};

// entries visible to position p: min(N, (p+1)/m); positions are below 2^31 (32-bit
// division: the 64-bit one is a long software sequence)
CSAHCA_DEV int vis_count(long long p, int m, int N) {
  if (p + 1 <= 0) return 0;
  const uint32_t v = (uint32_t)(p + 1) / (uint32_t)m;
  return v < (uint32_t)N ? (int)v : N;
}

// Wait until at most N of this wave's vector-memory operations are outstanding, then
// join the workgroup barrier.  Written as one asm statement with a memory clobber so the
// compiler neither adds a full vmcnt(0) drain nor moves LDS reads across the barrier.
template <int N>
CSAHCA_DEV void wait_vmcnt_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Every LDS read of this wave has completed; then join the workgroup barrier.
CSAHCA_DEV void lds_reads_done_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait until at most `inflight` tiles (LPW row loads each) of this wave are outstanding,
// inflight in [0, MAXF]; vmcnt takes an immediate, so dispatch on the value.
template <int MAXF, int LPW>
CSAHCA_DEV void wait_tiles(int inflight) {
  constexpr int c1 = LPW < 63 ? LPW : 63;
  constexpr int c2 = 2 * LPW < 63 ? 2 * LPW : 63;
  constexpr int c3 = 3 * LPW < 63 ? 3 * LPW : 63;
  if (MAXF >= 3 && inflight >= 3) wait_vmcnt_barrier<c3>();
  else if (MAXF >= 2 && inflight >= 2) wait_vmcnt_barrier<c2>();
  else if (MAXF >= 1 && inflight >= 1) wait_vmcnt_barrier<c1>();
  else wait_vmcnt_barrier<0>();
}

// LDS ring depth NS: 2 tiles when many workgroups run (two 4-wave workgroups share a CU
// and hide each other's latency: prefill), 4 tiles when few queries are split over
// workgroups (one workgroup per CU keeps three tiles in flight: decode).
// Column-split workgroups (CS) add an exchange area: P^T operands [TPI][NW][64 lanes]
// (16 bytes each), the per-head factors alpha [NW][16], one flag per wave, and at the end
// the running maxima and sums [NW][16], partial row maxima [NW][NW * 16] and the sums of
// the rounded weights [NW][16].
__host__ __device__ constexpr size_t xch_bytes(int NW, int TPI) {
  return (size_t)TPI * NW * 64 * 16 + (size_t)NW * 16 * 4 + 64 + 3 * (size_t)NW * 16 * 4 +
         (size_t)NW * NW * 16 * 4;
}

// ... and with the query RMSNorm + RoPE, its gains [C]
size_t attend_lds_bytes(int NS, int NW, int RS, bool csa, bool cs, bool nr) {
  const int TPI = NS >= 4 ? 2 : 1;
  const size_t x = csahca::align_up((size_t)NS * TILE * ROWB + (size_t)NS * NW * sizeof(uint32_t) +
                                        (csa ? (size_t)RS * sizeof(int) : 0), 16);
  return x + (cs ? xch_bytes(NW, TPI) : 0) + (nr ? (size_t)C * sizeof(float) : 0);
}

// bits [lo, hi) of a 32-bit mask, the bounds relative to `base` and clipped to [0, 32)
CSAHCA_DEV uint32_t range_bits(int lo, int hi, int base) {
  lo = min(max(lo - base, 0), 32);
  hi = min(max(hi - base, 0), 32);
  if (hi <= lo) return 0u;
  const uint32_t up = hi == 32 ? 0xFFFFFFFFu : ((1u << hi) - 1u);
  return up & ~((1u << lo) - 1u);
}

// 32-bit LDS byte address of a pointer into dynamic shared memory
CSAHCA_DEV uint32_t lds_addr(const uint8_t* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}

// O^T += E^T P^T as asm text (pv_asm.inc, written by gen_pv_asm.py): the transpose reads
// ds_read_b64_tr_b16 feed v_mfma_f32_16x16x32_bf16 with waits on LDS reads only.
#include "pv_asm.inc"
#define PV_ACC_OPERANDS                                                                   \
  "+v"(oacc[0]), "+v"(oacc[1]), "+v"(oacc[2]), "+v"(oacc[3]), "+v"(oacc[4]), "+v"(oacc[5]), \
      "+v"(oacc[6]), "+v"(oacc[7]), "+v"(oacc[8]), "+v"(oacc[9]), "+v"(oacc[10]),           \
      "+v"(oacc[11]), "+v"(oacc[12]), "+v"(oacc[13]), "+v"(oacc[14]), "+v"(oacc[15]),       \
      "+v"(oacc[16]), "+v"(oacc[17]), "+v"(oacc[18]), "+v"(oacc[19]), "+v"(oacc[20]),       \
      "+v"(oacc[21]), "+v"(oacc[22]), "+v"(oacc[23]), "+v"(oacc[24]), "+v"(oacc[25]),       \
      "+v"(oacc[26]), "+v"(oacc[27]), "+v"(oacc[28]), "+v"(oacc[29]), "+v"(oacc[30]),       \
      "+v"(oacc[31])

// One workgroup: queries t0 .. t0+Tg-1 of one sequence, HPW heads, slots
// [split*RS, (split+1)*RS).  Rows arrive by global_load_lds straight into an LDS ring of
// NS tiles; each wave issues its share of every tile (one 1 KiB row per instruction) and
// waits with an explicit vmcnt for the oldest tile only, so NS-1 tiles stay in flight
// without holding registers.  Skipped slots load a valid dummy row; a wave-uniform 32-bit
// mask per tile gives every skipped slot a zero weight.  The running maximum only moves
// when a score exceeds it by more than 2^8 (weights stay <= 256), so the output
// accumulators are rarely rescaled.  LDS operands are read in small groups, one group
// ahead of the MFMAs that use them, which bounds the registers in use so that two
// workgroups share a CU.
// CS (column split, NW = 2 or 4, one query per workgroup, one tile per iteration): each
// wave still computes the scores and softmax of its own 16 heads, but the P^T operands
// and rescale factors go through LDS, and for O^T += E^T P^T wave w owns the output
// columns [w*512/NW, (w+1)*512/NW) of all NW head blocks: every E^T fragment it reads
// from LDS feeds NW MFMAs, so the transpose reads per tile drop by NW.
template <int NW, int NS, bool CSA, bool CS>
__global__ __launch_bounds__(NW * 64, (NW == 4 && NS == 2) ? 2 : 1) void attend_bf16(AttnArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr int LPW = TILE / NW;  // rows each wave loads per tile
  constexpr float LAZY = 8.f;     // log2 headroom before the running maximum moves
  static_assert(!CS || NW == 2 || NW == 4, "column split: 2 or 4 waves");
  static_assert(!CS || NS == 2, "column split: one tile per iteration");
  uint8_t* tiles = smem;
  uint32_t* tmask = reinterpret_cast<uint32_t*>(smem + NS * TILE * ROWB);  // [NS][NW]
  int* sidx = reinterpret_cast<int*>(tmask + NS * NW);                     // [RS]
  // exchange area (CS): after sidx, 16-byte aligned.  Aligned as an offset from smem, so
  // that the pointer keeps its LDS address space (ds_read / ds_write, not flat accesses,
  // whose waits would also drain the row DMA in flight).
  uint8_t* xch = smem + ((NS * TILE * ROWB + NS * NW * 4 + (CSA ? a.RS * 4 : 0) + 15) & ~15);
  // the query norm gains after the exchange area
  float* s_gain = reinterpret_cast<float*>(xch + (CS ? xch_bytes(NW, NS >= 4 ? 2 : 1) : 0));

  // XCD-aware order: consecutive work items (the head groups of one row range first) run
  // on the same XCD, so the rows they share are read from HBM once into that XCD's L2.
  CSAHCA_TRACE(0);
  CSAHCA_TRACE_RT(14);
  const int Lb = blockIdx.x;
  const int wid = (Lb & 7) * a.per_xcd + (Lb >> 3);
  if (wid >= a.n_work) return;  // grid padding, before any barrier
  const int hg = wid % a.n_hg;
  const int rest = wid / a.n_hg;
  const int split = rest % a.n_splits;
  const int qg = rest / a.n_splits;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int row16 = lane & 15, g = lane >> 4;
  const int b = qg / a.nqg;
  const int t0 = (qg - b * a.nqg) * a.Tg;
  const int wpq = a.HPW / 16;
  const int tq = t0 + wave / wpq;
  const int h0 = hg * a.HPW + (wave % wpq) * 16;
  const bool active = tq < a.Tq;
  const int tlast = min(t0 + a.Tg, a.Tq) - 1;
  // positions first, while no DMA has been issued: uniform loads the compiler can make
  // scalar (their wait is then independent of the vector loads issued below)
  const long long qpos0 = a.q_pos[b];
  const long long wp = a.win_pos[b];
  const int slot_lo = split * a.RS;
  const int slot_hi = min(a.n_slots, slot_lo + a.RS);
  const long long qrow = (long long)b * a.Tq + (active ? tq : tlast);
  const uint16_t* ckv_b = a.ckv + (size_t)b * a.Nc * C;
  const uint16_t* win_b = a.win + (size_t)b * a.L * C;
  const int nsc = a.n_slots_c;
  const int ntile = slot_hi > slot_lo ? cdiv(slot_hi - slot_lo, TILE) : 0;
  constexpr int TPI = NS >= 4 ? 2 : 1;  // tiles consumed per iteration

  // Position-dependent ranges, set once the positions have arrived (below):
  // window slot j >= nsc holds raw position wpos0 + (j - nsc), i.e. source row
  // wrow0 + (j - nsc).  Usable raw positions: >= 0, inside the source rows, and in the
  // query's own window (p-W, p]; for loading, the union over the workgroup's queries.
  long long wrow0 = 0;
  int wu_lo = nsc, wu_hi = nsc, wq_lo = nsc, wq_hi = nsc;
  int Vu = 0, Vw = 0;  // HCA: entries visible to the last / to this wave's query

  // DMA of tile tt into its ring stage: each wave issues rows wave, wave + NW, ...  of
  // the tile, one 1 KiB row per instruction.  HCA with `spec`: compressed rows are
  // loaded before the positions are known (every row below N_h is valid memory;
  // visibility is applied by the score mask).  Tiles whose rows are all contiguous
  // compressed rows (HCA) or all window rows, and CSA tiles of selected entries only, take
  // short paths with no per-row branching; other tiles decide row by row.
  uint32_t mybits = 0;  // this wave's rows of a tile
#pragma unroll
  for (int i = 0; i < LPW; ++i) mybits |= 1u << (wave + i * NW);
  auto dma_row = [&](const uint16_t* src, uint8_t* st, int r) {
    __builtin_amdgcn_global_load_lds(src + lane * 8,
                                     (__attribute__((address_space(3))) void*)(st + row_base(r)),
                                     16, 0, 0);
  };
  auto issue = [&](int tt, bool spec) {
    const int stage = tt % NS;
    uint8_t* st = tiles + stage * (TILE * ROWB);
    const int base = slot_lo + tt * TILE;
    const int cend = min(slot_hi, nsc);  // end of this split's compressed slots
    uint32_t okbits = 0;
    if (!CSA && base + TILE <= cend && (spec || base + TILE <= Vu)) {
      const uint16_t* src = ckv_b + (size_t)(base + wave) * C;
#pragma unroll
      for (int i = 0; i < LPW; ++i) dma_row(src + (size_t)i * NW * C, st, wave + i * NW);
      okbits = mybits;
    } else if (base >= nsc && base >= wu_lo && base + TILE <= min(wu_hi, slot_hi)) {
      const uint16_t* src = win_b + (size_t)(wrow0 + (base - nsc) + wave) * C;
#pragma unroll
      for (int i = 0; i < LPW; ++i) dma_row(src + (size_t)i * NW * C, st, wave + i * NW);
      okbits = mybits;
    } else if (CSA && base + TILE <= cend) {
      // lane i < LPW fetches the entry index of row wave + i*NW; rows read them by lane
      const int ev = lane < LPW ? sidx[base - slot_lo + wave + lane * NW] : 0;
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const int e = __builtin_amdgcn_readlane(ev, i);
        const bool ok = (unsigned)e < (unsigned)a.Nc;
        dma_row(ckv_b + (size_t)(ok ? e : 0) * C, st, wave + i * NW);
        okbits |= ok ? (1u << (wave + i * NW)) : 0u;
      }
    } else {
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const int r = wave + i * NW;
        const int j = base + r;
        const uint16_t* src = ckv_b;  // dummy: any valid row
        bool ok = false;
        if (j < slot_hi) {
          if (j < nsc) {
            if (CSA) {
              const int e = __builtin_amdgcn_readfirstlane(sidx[j - slot_lo]);
              ok = (unsigned)e < (unsigned)a.Nc;
              if (ok) src = ckv_b + (size_t)e * C;
            } else if (spec || j < Vu) {
              ok = true;
              src = ckv_b + (size_t)j * C;
            }
          } else if (j >= wu_lo && j < wu_hi) {
            ok = true;
            src = win_b + (size_t)(wrow0 + (j - nsc)) * C;
          }
        }
        okbits |= ok ? (1u << r) : 0u;
        dma_row(src, st, r);
      }
    }
    if (lane == 0) tmask[stage * NW + wave] = okbits;
  };

  // Start-up, ordered so that independent latencies overlap: the Q fragments, then (CSA)
  // this split's entry indices or (HCA, when the first tiles hold only compressed rows)
  // the first tiles themselves, while the positions arrive.
  // query norm gains, this thread's share of the C channels (to LDS once Q has arrived)
  constexpr int GPT = C / (NW * 64);
  float gq[GPT];
  if (a.qnr) {
#pragma unroll
    for (int i = 0; i < GPT; ++i) gq[i] = a.q_gamma ? a.q_gamma[(int)threadIdx.x + i * NW * 64] : 1.f;
  }
  bf16x8 qf[KS];
  {
    const uint16_t* qp = a.q + (qrow * a.n_h + h0 + row16) * C + g * (C / 4);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qp + ks * 8));
  }
  if (CSA) {  // the split's selected entry indices, staged in LDS
    const int* tk = a.topk + ((long long)b * a.Tq + t0) * a.k;
    const int hi = min(slot_hi, nsc);
    for (int j = slot_lo + (int)threadIdx.x; j < hi; j += NW * 64) sidx[j - slot_lo] = tk[j];
  }
  const bool spec = !CSA && slot_lo + TPI * TILE <= nsc;
  if (spec)
    for (int tt = 0; tt < TPI && tt < ntile; ++tt) issue(tt, true);

  const long long pfirst = qpos0 + t0, plast = qpos0 + tlast;
  const long long p = qpos0 + (active ? tq : tlast);
  const long long wpos0 = pfirst - a.W + 1;
  wrow0 = wpos0 - wp;
  auto win_slots = [&](long long lo_pos, long long hi_pos, int& lo, int& hi) {
    lo_pos = max(lo_pos, max(0LL, wp));
    hi_pos = min(hi_pos, wp + a.L - 1);
    if (hi_pos < lo_pos) {
      lo = hi = nsc;
      return;
    }
    lo = nsc + (int)(lo_pos - wpos0);
    hi = nsc + (int)(hi_pos - wpos0) + 1;
  };
  win_slots(wpos0, plast, wu_lo, wu_hi);
  win_slots(p - a.W + 1, p, wq_lo, wq_hi);
  if (!CSA) {
    Vu = vis_count(plast, a.m, a.Nc);
    Vw = vis_count(p, a.m, a.Nc);
  }
  if (CSA) __syncthreads();  // sidx complete
  CSAHCA_TRACE(1);

  // Query RMSNorm + RoPE: the rotation angles depend only on the wave's query position,
  // so they are formed while Q is in flight (lane i < d_rope/2 forms pair i's)
  const int nr_P = a.d_rope / 2;  // <= 64 rotated pairs (the host checks)
  float nr_cs = 1.f, nr_sn = 0.f;
  if (a.qnr && lane < nr_P) csahca::rope_cos_sin(p, csahca::rope_freq(lane, a.d_rope, a.nr_theta), nr_cs, nr_sn);

  // The compiler does not assume that row DMAs and register loads complete in order, so
  // its wait for Q (forced here by the empty asm, once, rather than before the first MFMA
  // of every iteration) drains every load issued so far: only the tiles needed first.
  if (!spec)
    for (int tt = 0; tt < TPI && tt < ntile; ++tt) issue(tt, false);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(qf[ks]));
  if (a.qnr) {  // the gains arrived with Q
#pragma unroll
    for (int i = 0; i < GPT; ++i) s_gain[(int)threadIdx.x + i * NW * 64] = gq[i];
  }
  for (int tt = TPI; tt < NS && tt < ntile; ++tt) issue(tt, false);
  if (a.qnr) {
    // RMSNorm of the query row (this lane holds channels g*C/4 .. +C/4 of head h0+row16,
    // its three partners the rest), then RoPE on the last d_rope channels; the arithmetic
    // of the row kernel (norm_rope8), with the sum of squares in another order.  The
    // ring's DMA is in flight meanwhile (the barrier waits for LDS only).
    lds_reads_done_barrier();
    float ssp[4] = {0.f, 0.f, 0.f, 0.f};  // four chains (the sum's order is fixed)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 w4 = __builtin_bit_cast(u32x4, qf[ks]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = __uint_as_float(w4[e] << 16), hi = __uint_as_float(w4[e] & 0xFFFF0000u);
        ssp[e] = fmaf(lo, lo, ssp[e]);
        ssp[e] = fmaf(hi, hi, ssp[e]);
      }
    }
    const float ss = sum_over_row_groups((ssp[0] + ssp[1]) + (ssp[2] + ssp[3]));
    const float inv = 1.0f / sqrtf(ss / (float)C + a.nr_eps);
    // d_rope <= 128, so only lane group 3 (channels 384..511) holds rotated channels, and
    // in step ks it holds pairs i0 .. i0+3, i0 = (384 + 8 ks - (C - d_rope)) / 2, the same
    // for all its lanes: their angles come by readlane
    const int r0 = C - a.d_rope;  // first rotated channel
    constexpr int KB = 4;         // steps per batch of gain reads (one LDS wait per batch)
#pragma unroll
    for (int kb = 0; kb < KS; kb += KB) {
      f32x4 gv[KB][2];
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        const int d0 = g * (C / 4) + 8 * (kb + u);
        gv[u][0] = *reinterpret_cast<const f32x4*>(s_gain + d0);
        gv[u][1] = *reinterpret_cast<const f32x4*>(s_gain + d0 + 4);
      }
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        const int ks = kb + u;
        const u32x4 w4 = __builtin_bit_cast(u32x4, qf[ks]);
        const float gg[8] = {gv[u][0][0], gv[u][0][1], gv[u][0][2], gv[u][0][3],
                             gv[u][1][0], gv[u][1][1], gv[u][1][2], gv[u][1][3]};
        float v[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[2 * e] = __uint_as_float(w4[e] << 16) * (inv * gg[2 * e]);
          v[2 * e + 1] = __uint_as_float(w4[e] & 0xFFFF0000u) * (inv * gg[2 * e + 1]);
        }
        const int c3 = 3 * (C / 4) + 8 * ks;  // group 3's first channel in this step
        if (c3 >= r0) {                      // uniform
          const int i0 = (c3 - r0) / 2;
#pragma unroll
          for (int q2 = 0; q2 < 4; ++q2) {
            const float cq = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, nr_cs), i0 + q2));
            const float sq = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, nr_sn), i0 + q2));
            float a0 = v[2 * q2], a1 = v[2 * q2 + 1];
            csahca::rope_apply(a0, a1, cq, sq);
            if (g == 3) {
              v[2 * q2] = a0;
              v[2 * q2 + 1] = a1;
            }
          }
        }
        qf[ks] = __builtin_bit_cast(bf16x8, u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                                  pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])});
      }
    }
  }

  // l_run: mass of the fp32 weights (log-sum-exp, split records); lq_run: sum of the same
  // weights rounded to bf16, as they enter the PV product (normalises the output)
  float m_run = -INFINITY, l_run = 0.f, lq_run = 0.f;
  // O^T accumulators: without CS oacc[cb][i] is column 16*cb + 4*g + i of head
  // h0 + row16; with CS oacc[cbl*NW + hb][i] is column 16*(wave*32/NW + cbl) + 4*g + i of
  // head hg*HPW + 16*hb + row16
  f32x4 oacc[C / 16];
#pragma unroll
  for (int cb = 0; cb < C / 16; ++cb) oacc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // LDS byte offsets of this lane's operands inside a tile
  int s_off = row_base(row16) + g * (C / 4) * 2;                  // S: A = row, 8 dims
  int t_off = row_base(4 * g + (row16 >> 2)) + (row16 & 3) * 8;  // PV: transpose reads
  // (one register each: left to itself the compiler keeps their parts apart, and spills)
  asm volatile("" : "+v"(s_off), "+v"(t_off));

  auto tile_mask = [&](int stage, int base) -> uint32_t {
    uint32_t loaded = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) loaded |= tmask[stage * NW + w];
    loaded = __builtin_amdgcn_readfirstlane(loaded);
    uint32_t vm = range_bits(wq_lo, min(wq_hi, slot_hi), base);
    if (CSA)
      vm |= range_bits(slot_lo, min(nsc, slot_hi), base);
    else
      vm |= range_bits(0, min(min(Vw, nsc), slot_hi), base);
    return vm & loaded;
  };

  // Each iteration consumes TPI tiles: with a 4-tile ring two (64 slots: four independent
  // S chains, one softmax update, 64 PV MFMAs) while the next two are in flight; with a
  // 2-tile ring one, while the other is in flight.
  static_assert(NS % TPI == 0, "the ring holds whole iterations");
  for (int it = 0; it < ntile; it += TPI) {
    // tiles it .. min(ntile, it+NS)-1 are issued; all but the first TPI may stay in flight
    wait_tiles<NS - TPI, LPW>(min(ntile - it, NS) - TPI);
    if (it < 3 * TPI) CSAHCA_TRACE(2 + 2 * (it / TPI) + (it ? 4 : 0));
    const bool two = TPI == 2 && ntile - it >= 2;
    if (active) {
      const int stA = it % NS, stB = (it + 1) % NS;
      const uint8_t* tA = tiles + stA * (TILE * ROWB);
      const uint8_t* tB = two ? tiles + stB * (TILE * ROWB) : tA;
      const int base = slot_lo + it * TILE;
      const uint32_t vmA = tile_mask(stA, base);
      const uint32_t vmB = two ? tile_mask(stB, base + TILE) : 0u;

      // ---- S^T = E Q^T in 16-slot blocks, operands read one K-step ahead ----
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0, s2 = s0, s3 = s0;
      const uint8_t* spA = tA + s_off;
      const uint8_t* spB = tB + s_off;
      u32x4 r0 = *reinterpret_cast<const u32x4*>(spA);
      u32x4 r1 = *reinterpret_cast<const u32x4*>(spA + 16 * ROWB);
      u32x4 r2, r3;
      if (TPI == 2) {
        r2 = *reinterpret_cast<const u32x4*>(spB);
        r3 = *reinterpret_cast<const u32x4*>(spB + 16 * ROWB);
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4 n0, n1, n2, n3;
        if (ks + 1 < KS) {
          n0 = *reinterpret_cast<const u32x4*>(spA + (ks + 1) * 16);
          n1 = *reinterpret_cast<const u32x4*>(spA + 16 * ROWB + (ks + 1) * 16);
          if (TPI == 2) {
            n2 = *reinterpret_cast<const u32x4*>(spB + (ks + 1) * 16);
            n3 = *reinterpret_cast<const u32x4*>(spB + 16 * ROWB + (ks + 1) * 16);
          }
        }
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, r0), qf[ks], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, r1), qf[ks], s1, 0, 0, 0);
        if (TPI == 2) {
          s2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, r2), qf[ks], s2, 0, 0, 0);
          s3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, r3), qf[ks], s3, 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        r0 = n0;
        r1 = n1;
        if (TPI == 2) {
          r2 = n2;
          r3 = n3;
        }
      }
      if (it == TPI) CSAHCA_TRACE(12);
      // lane: head h0 + row16; sv[4*rb + i] is slot base + 16*rb + 4g + i (rb 2, 3: tile B):
      // the raw score q.k, -inf where the slot is masked (no masking when every slot of
      // the iteration is usable, the common case)
      constexpr int NSV = 8 * TPI;
      float sv[NSV];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[i] = s0[i];
        sv[4 + i] = s1[i];
        if (TPI == 2) {
          sv[(8 + i) % NSV] = s2[i];
          sv[(12 + i) % NSV] = s3[i];
        }
      }
      if ((vmA & (TPI == 2 ? vmB : ~0u)) != ~0u) {  // wave-uniform
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * g + i;
          sv[i] = ((vmA >> r) & 1u) ? sv[i] : -INFINITY;
          sv[4 + i] = ((vmA >> (16 + r)) & 1u) ? sv[4 + i] : -INFINITY;
          if (TPI == 2) {
            sv[(8 + i) % NSV] = ((vmB >> r) & 1u) ? sv[(8 + i) % NSV] : -INFINITY;
            sv[(12 + i) % NSV] = ((vmB >> (16 + r)) & 1u) ? sv[(12 + i) % NSV] : -INFINITY;
          }
        }
      }
      float mx[NSV / 2];
#pragma unroll
      for (int e = 0; e < NSV / 2; ++e) mx[e] = fmaxf(sv[e], sv[e + NSV / 2]);
#pragma unroll
      for (int w = NSV / 4; w >= 1; w >>= 1)
#pragma unroll
        for (int e = 0; e < w; ++e) mx[e] = fmaxf(mx[e], mx[e + w]);
      // in log2 units (the scale is positive, so the maximum commutes with it)
      const float mloc = max_over_row_groups(mx[0]) * a.scale_log2;
      // lazy running maximum: move it only when exceeded by more than LAZY
      const bool bump = mloc > m_run + LAZY;
      const float m_new = bump ? mloc : m_run;
      // hardware exp2: results below 2^-126 flush to zero, negligible next to the running
      // sum, which is at least 1 (it holds the term of the score that set the maximum)
      const float alpha = bump ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
      const float m_use = m_new == -INFINITY ? 0.f : m_new;  // nothing usable yet: all -inf
      float pe[NSV];
#pragma unroll
      for (int e = 0; e < NSV; ++e) pe[e] = __builtin_amdgcn_exp2f(fmaf(sv[e], a.scale_log2, -m_use));
      float ps[NSV / 2];
#pragma unroll
      for (int e = 0; e < NSV / 2; ++e) ps[e] = pe[e] + pe[e + NSV / 2];
#pragma unroll
      for (int w = NSV / 4; w >= 1; w >>= 1)
#pragma unroll
        for (int e = 0; e < w; ++e) ps[e] += ps[e + w];
      const float psum = sum_over_row_groups(ps[0]);
      l_run = l_run * alpha + psum;
      // the weights enter O^T += E^T P^T as bf16; their rounded sum normalises the output,
      // which is then an exact convex combination of its rows (a query with a single
      // usable row returns that row's bits)
      uint32_t pk[NSV / 2];  // consecutive weights as packed bf16 pairs, and their values
#pragma unroll
      for (int e = 0; e < NSV / 2; ++e) {
        pk[e] = pack_bf16x2(pe[2 * e], pe[2 * e + 1]);
        pe[2 * e] = __uint_as_float(pk[e] << 16);
        pe[2 * e + 1] = __uint_as_float(pk[e] & 0xFFFF0000u);
      }
#pragma unroll
      for (int e = 0; e < NSV / 2; ++e) ps[e] = pe[e] + pe[e + NSV / 2];
#pragma unroll
      for (int w = NSV / 4; w >= 1; w >>= 1)
#pragma unroll
        for (int e = 0; e < w; ++e) ps[e] += ps[e + w];
      lq_run = lq_run * alpha + sum_over_row_groups(ps[0]);
      m_run = m_new;
      // P^T as B operands: k-slot e <-> slot (e < 4 ? 4g+e : 16+4g+e-4) of its tile
      const bf16x8 pfA = __builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
      bf16x8 pfB;
      if (TPI == 2)
        pfB = __builtin_bit_cast(bf16x8, u32x4{pk[4 % (NSV / 2)], pk[5 % (NSV / 2)], pk[6 % (NSV / 2)],
                                               pk[7 % (NSV / 2)]});
      // ---- O^T += E^T P^T: E^T through LDS transpose reads, issued in asm ahead of use ----
      // ds_read_b64_tr_b16: in each 16-lane group, lane i receives column i%4 of the four
      // 4-element rows addressed by lanes i/4, i/4+4, i/4+8, i/4+12.  Lane j addresses row
      // (4g + j/4) at column 16*cb + 4*(j%4), so lane i gets column 16*cb + i of rows
      // 4g .. 4g+3 (and 16+4g .. 16+4g+3 with the second read): exactly its A operand.
      if (it == TPI) CSAHCA_TRACE(13);
      const uint32_t aA = lds_addr(tA + t_off), aB = lds_addr(tB + t_off);
      if constexpr (!CS) {
        if (__any(bump)) {
#pragma unroll
          for (int cb = 0; cb < C / 16; ++cb) oacc[cb] *= alpha;
        }
        if constexpr (TPI == 2) {
          asm volatile(CSAHCA_PV_ASM_2TILE
                       : PV_ACC_OPERANDS
                       : "v"(pfA), "v"(pfB), "v"(aA), "v"(aB)
                       : CSAHCA_PV_CLOBBERS, "memory");
        } else {
          asm volatile(CSAHCA_PV_ASM_1TILE
                       : PV_ACC_OPERANDS
                       : "v"(pfA), "v"(aA)
                       : CSAHCA_PV_CLOBBERS, "memory");
        }
      } else {
        // exchange: this wave's P^T operands, rescale factors and rescale flag, then every
        // wave's (the barrier also orders the previous iteration's reads before the writes)
        u32x4* xp = reinterpret_cast<u32x4*>(xch);                   // [TPI][NW][64]
        float* xa = reinterpret_cast<float*>(xch + TPI * NW * 1024);  // [NW][16]
        uint32_t* xf = reinterpret_cast<uint32_t*>(xa + NW * 16);     // [NW]
        xp[wave * 64 + lane] = __builtin_bit_cast(u32x4, pfA);
        if (TPI == 2) xp[(NW + wave) * 64 + lane] = __builtin_bit_cast(u32x4, pfB);
        if (g == 0) xa[wave * 16 + row16] = alpha;
        const uint32_t any_bump = __any(bump) ? 1u : 0u;
        if (lane == 0) xf[wave] = any_bump;
        lds_reads_done_barrier();
        u32x4 px[NW][TPI];
#pragma unroll
        for (int hb = 0; hb < NW; ++hb) {
#pragma unroll
          for (int tt = 0; tt < TPI; ++tt) px[hb][tt] = xp[(tt * NW + hb) * 64 + lane];
          if (__builtin_amdgcn_readfirstlane(xf[hb])) {
            const float al = xa[hb * 16 + row16];
#pragma unroll
            for (int cbl = 0; cbl < C / 16 / NW; ++cbl) oacc[cbl * NW + hb] *= al;
          }
        }
        if (it == TPI) CSAHCA_TRACE(6);
        const uint32_t cofs = (uint32_t)wave * (C / 16 / NW) * 32;  // the wave's first column block
        const uint32_t cA = aA + cofs;
        if constexpr (NW == 4) {
          asm volatile(CSAHCA_PVC_ASM_4W_1T
                       : PV_ACC_OPERANDS
                       : "v"(px[0][0]), "v"(px[1 % NW][0]), "v"(px[2 % NW][0]), "v"(px[3 % NW][0]), "v"(cA)
                       : CSAHCA_PV_CLOBBERS, "memory");
        } else {
          asm volatile(CSAHCA_PVC_ASM_2W_1T
                       : PV_ACC_OPERANDS
                       : "v"(px[0][0]), "v"(px[1 % NW][0]), "v"(cA)
                       : CSAHCA_PV_CLOBBERS, "memory");
        }
      }
    }
    lds_reads_done_barrier();  // the consumed stages are free for the next issue
    if (it < 3 * TPI) CSAHCA_TRACE(3 + 2 * (it / TPI) + (it ? 4 : 0));
    for (int tt = it + NS; tt < it + NS + TPI && tt < ntile; ++tt) issue(tt, false);
  }
  CSAHCA_TRACE(4);
  if constexpr (CS) {  // one query per workgroup: every wave is active
    constexpr int CPW = C / 16 / NW;   // column blocks per wave
    constexpr int EROWB = C * 2 + 16;  // staging row stride in bytes
    float* xm = reinterpret_cast<float*>(xch + TPI * NW * 1024 + NW * 16 * 4 + 64);  // [NW][16]
    float* xl = xm + NW * 16;                                                       // [NW][16]
    float* xam = xl + NW * 16;  // [NW][NW*16]: |O| maxima over a wave's columns, per head
    float* xlq = xam + NW * NW * 16;  // [NW][16]
    if (g == 0) {
      xm[wave * 16 + row16] = m_run;
      xl[wave * 16 + row16] = l_run;
      xlq[wave * 16 + row16] = lq_run;
    }
#pragma unroll
    for (int hb = 0; hb < NW; ++hb) {
      float pam = 0.f;
#pragma unroll
      for (int cbl = 0; cbl < CPW; ++cbl) {
        const f32x4 o = oacc[cbl * NW + hb];
        pam = fmaxf(pam, fmaxf(fmaxf(fabsf(o[0]), fabsf(o[1])), fmaxf(fabsf(o[2]), fabsf(o[3]))));
      }
      pam = max_over_row_groups(pam);
      if (g == 0) xam[wave * NW * 16 + hb * 16 + row16] = pam;
    }
    lds_reads_done_barrier();
    // every head block's values of this wave's columns, as 16-bit rows [head][column]
#pragma unroll
    for (int hb = 0; hb < NW; ++hb) {
      float lh = xl[hb * 16 + row16], mh = xm[hb * 16 + row16], lqh = xlq[hb * 16 + row16];
      const bool as_f16 = a.n_splits > 1;
      // one split: the sink joins here (with splits, in the merge)
      const float rs = as_f16 ? 1.f : fold_sink2(a.sink, hg * a.HPW + 16 * hb + row16, mh, lh, lqh);
      const float inv = lqh > 0.f ? rs / lqh : 0.f;
      float f = inv;
      if (as_f16) {  // partial O / l scaled by 2^-e per row (see the merge)
        float amax = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) amax = fmaxf(amax, xam[w * NW * 16 + hb * 16 + row16]);
        amax *= inv;
        const uint32_t ex = min(max((__float_as_uint(amax) >> 23) & 0xFFu, 1u), 253u);
        f = inv * __uint_as_float((254u - ex) << 23);
        if (hb == wave && g == 0) {
          const long long pr = (qrow * a.n_splits + split) * a.n_h + h0 + row16;
          *reinterpret_cast<f32x4*>(a.mlpart + pr * 4) = f32x4{mh, lh, __uint_as_float(ex << 23), 0.f};
        }
      } else if (hb == wave && a.lse && g == 0) {
        a.lse[qrow * a.n_h + h0 + row16] = lh > 0.f ? (mh + __log2f(lh)) * LN2 : -INFINITY;
      }
      uint8_t* srow = tiles + (hb * 16 + row16) * EROWB;
#pragma unroll
      for (int cbl = 0; cbl < CPW; ++cbl) {
        const f32x4 o = oacc[cbl * NW + hb];
        const int cb = wave * CPW + cbl;
        *reinterpret_cast<u32x2*>(srow + (16 * cb + 4 * g) * 2) =
            as_f16 ? u32x2{pack_f16x2(o[0] * f, o[1] * f), pack_f16x2(o[2] * f, o[3] * f)}
                   : u32x2{pack_bf16x2(o[0] * f, o[1] * f), pack_bf16x2(o[2] * f, o[3] * f)};
      }
    }
    lds_reads_done_barrier();
    // this wave's own head block: 16 whole rows, one 1 KiB store each
    uint16_t* dst = a.n_splits == 1 ? a.out + (qrow * a.n_h + h0) * C
                                    : a.opart + ((qrow * a.n_splits + split) * a.n_h + h0) * C;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr)
      *reinterpret_cast<u32x4*>(dst + rr * C + lane * 8) =
          *reinterpret_cast<const u32x4*>(tiles + (wave * 16 + rr) * EROWB + lane * 16);
    CSAHCA_TRACE(5);
    CSAHCA_TRACE_RT(15);
    return;
  }
  if (!active) return;

  // lane: head h0 + row16; oacc[cb][i] is column 16*cb + 4*g + i.  The wave's 16 output
  // rows (heads h0 .. h0+15) are contiguous in both destinations.
  const int h = h0 + row16;
  float f;              // multiplier from the accumulators to the stored 16-bit values
  uint16_t* dst;        // the wave's first output row
  bool as_f16;
  if (a.n_splits == 1) {
    float mm = m_run, ll = l_run, lq = lq_run;
    const float rs = fold_sink2(a.sink, h, mm, ll, lq);
    f = lq > 0.f ? rs / lq : 0.f;
    dst = a.out + (qrow * a.n_h + h0) * C;
    as_f16 = false;
    if (a.lse && g == 0) a.lse[qrow * a.n_h + h] = ll > 0.f ? (mm + __log2f(ll)) * LN2 : -INFINITY;
  } else {
    // Partial output O / l in float16, scaled by a power of two 2^-e chosen per row so
    // that its largest magnitude lies in [1, 2): no input range overflows, and every value
    // keeps float16's 11-bit precision relative to the row's largest.  The record (m, l,
    // 2^e) lets the merge weigh the row by l * 2^(m - M) * 2^e.
    const long long pr0 = (qrow * a.n_splits + split) * a.n_h + h0;
    const float inv = lq_run > 0.f ? 1.f / lq_run : 0.f;
    float amax = 0.f;
#pragma unroll
    for (int cb = 0; cb < C / 16; ++cb)
      amax = fmaxf(amax, fmaxf(fmaxf(fabsf(oacc[cb][0]), fabsf(oacc[cb][1])),
                               fmaxf(fabsf(oacc[cb][2]), fabsf(oacc[cb][3]))));
    amax = max_over_row_groups(amax) * inv;  // the head's four lanes hold its 512 columns
    const uint32_t ex = min(max((__float_as_uint(amax) >> 23) & 0xFFu, 1u), 253u);
    f = inv * __uint_as_float((254u - ex) << 23);  // 1 / (l * 2^(ex - 127))
    dst = a.opart + pr0 * C;
    as_f16 = true;
    if (g == 0) {
      *reinterpret_cast<f32x4*>(a.mlpart + (pr0 + row16) * 4) =
          f32x4{m_run, l_run, __uint_as_float(ex << 23), 0.f};
    }
  }
  auto pack = [&](float x, float y) { return as_f16 ? pack_f16x2(x * f, y * f) : pack_bf16x2(x * f, y * f); };
  constexpr int EROWB = C * 2 + 16;  // staging row stride in bytes
  if (NW * 16 * EROWB <= NS * TILE * ROWB) {
    // through LDS (the tiles are free: every wave passed the loop's last barrier and no
    // row load is outstanding), so that each store writes one whole 1 KiB row
    uint8_t* stg = tiles + wave * 16 * EROWB;
#pragma unroll
    for (int cb = 0; cb < C / 16; ++cb)
      *reinterpret_cast<u32x2*>(stg + row16 * EROWB + (16 * cb + 4 * g) * 2) =
          u32x2{pack(oacc[cb][0], oacc[cb][1]), pack(oacc[cb][2], oacc[cb][3])};
#pragma unroll
    for (int r = 0; r < 16; ++r)
      *reinterpret_cast<u32x4*>(dst + r * C + lane * 8) =
          *reinterpret_cast<const u32x4*>(stg + r * EROWB + lane * 16);
  } else {
    uint16_t* op = dst + row16 * C + 4 * g;
#pragma unroll
    for (int cb = 0; cb < C / 16; ++cb)
      *reinterpret_cast<u32x2*>(op + 16 * cb) = u32x2{pack(oacc[cb][0], oacc[cb][1]), pack(oacc[cb][2], oacc[cb][3])};
  }
  CSAHCA_TRACE(5);
  CSAHCA_TRACE_RT(15);
}

// Merge the splits of every (query, head) by their log-sum-exp.  One workgroup per pair:
// wave w takes the splits w, w+4, ..., eight partial rows in flight per lane (8 columns
// each); the four wave sums are then added in a fixed order.  A split's partial row holds
// its output normalised by the sum of its own (bf16-rounded) weights and scaled by 2^-e_s
// (float16); its weight in the merge is l_s * 2^(m_s - M) * 2^e_s, with l_s the mass of
// its fp32 weights and M the largest running maximum.
__global__ __launch_bounds__(256) void attend_combine(const uint16_t* __restrict__ opart,
                                                      const float* __restrict__ mlpart,
                                                      uint16_t* __restrict__ out,
                                                      float* __restrict__ lse,
                                                      const float* __restrict__ sink, int n_h,
                                                      int n_splits) {
  __shared__ float red[4][C + 4];
  const long long pair = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long long qrow = pair / n_h;
  const int h = (int)(pair - qrow * n_h);
  const long long pr0 = qrow * n_splits * n_h + h;  // partial row of split s: pr0 + s*n_h
  float M = -INFINITY;
  for (int s = lane; s < n_splits; s += 64) M = fmaxf(M, mlpart[(pr0 + (long long)s * n_h) * 4]);
  for (int d = 1; d < 64; d <<= 1) M = fmaxf(M, shfl_xor_f(M, d));
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float Ls = 0.f;
  if (M != -INFINITY) {
    for (int s0 = wave; s0 < n_splits; s0 += 32) {
      u32x4 x[8];
      f32x4 ml[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int s = s0 + 4 * u;
        if (s < n_splits) {
          const long long pr = pr0 + (long long)s * n_h;
          ml[u] = *reinterpret_cast<const f32x4*>(mlpart + pr * 4);
          x[u] = *reinterpret_cast<const u32x4*>(opart + pr * C + lane * 8);
        } else {
          ml[u] = f32x4{-INFINITY, 0.f, 0.f, 0.f};
          x[u] = u32x4{0u, 0u, 0u, 0u};
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float w = ml[u][0] == -INFINITY ? 0.f : ml[u][1] * exp2f(ml[u][0] - M);
        Ls += w;
        const float wgt = w * ml[u][2];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] = fmaf(wgt, f16_lo(x[u][i]), acc[2 * i]);
          acc[2 * i + 1] = fmaf(wgt, f16_hi(x[u][i]), acc[2 * i + 1]);
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) red[wave][lane * 8 + i] = acc[i];
  if (lane == 0) red[wave][C] = Ls;
  __syncthreads();
  if (wave != 0) return;
  float o8[8];
  float Lt = ((red[0][C] + red[1][C]) + red[2][C]) + red[3][C];
  const float rs = fold_sink(sink, h, M, Lt);
  const float inv = Lt > 0.f ? rs / Lt : 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = lane * 8 + i;
    o8[i] = (((red[0][c] + red[1][c]) + red[2][c]) + red[3][c]) * inv;
  }
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(o8[2 * i], o8[2 * i + 1]);
  *reinterpret_cast<u32x4*>(out + (qrow * n_h + h) * C + lane * 8) = o;
  if (lse && lane == 0) lse[qrow * n_h + h] = Lt > 0.f ? (M + __log2f(Lt)) * LN2 : -INFINITY;
}

constexpr int COMBINE_WAVE_SPLITS = 16;

// Merge of up to COMBINE_WAVE_SPLITS splits (one load round; more take attend_combine):
// every (query, head) by the log-sum-exp of its splits.  One wave per pair, four
// pairs per workgroup.  Lane l loads the record (m, l, 2^e) of split l (of splits 64j + l
// beyond 64); the partial rows are loaded 16 splits at a time, each lane holding 8
// columns of every row, the first 16 issued together with the records.  The records
// reach every lane by readlane, so no LDS and no barrier are needed, and the splits are
// added in index order.  A split's partial row holds its output normalised by the sum of
// its own (bf16-rounded) weights and scaled by 2^-e_s (float16); its weight in the merge
// is l_s * 2^(m_s - M) * 2^e_s, with l_s the mass of its fp32 weights and M the largest
// running maximum.
__global__ __launch_bounds__(256) void attend_combine_wave(const uint16_t* __restrict__ opart,
                                                           const float* __restrict__ mlpart,
                                                           uint16_t* __restrict__ out,
                                                           float* __restrict__ lse,
                                                           const float* __restrict__ sink, int n_h,
                                                           int n_splits, long long n_pairs) {
  constexpr int CH = COMBINE_WAVE_SPLITS;  // partial rows in flight per lane
  const int lane = threadIdx.x & 63;
  const long long pair = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (pair >= n_pairs) return;  // whole waves; no barrier follows
  const long long qrow = pair / n_h;
  const int h = (int)(pair - qrow * n_h);
  const long long pr0 = qrow * n_splits * n_h + h;  // partial row of split s: pr0 + s*n_h
  auto rec_of = [&](int s) {
    return s < n_splits ? *reinterpret_cast<const f32x4*>(mlpart + (pr0 + (long long)s * n_h) * 4)
                        : f32x4{-INFINITY, 0.f, 0.f, 0.f};
  };
  auto row_of = [&](int s) {
    return s < n_splits ? *reinterpret_cast<const u32x4*>(opart + (pr0 + (long long)s * n_h) * C + lane * 8)
                        : u32x4{0u, 0u, 0u, 0u};
  };
  f32x4 rec = rec_of(lane);
  u32x4 x[CH];
#pragma unroll
  for (int u = 0; u < CH; ++u) x[u] = row_of(u);
  float M = rec[0];
  for (int s = lane + 64; s < n_splits; s += 64) M = fmaxf(M, rec_of(s)[0]);
  for (int d = 1; d < 64; d <<= 1) M = fmaxf(M, shfl_xor_f(M, d));
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float Ls = 0.f;
  for (int s0 = 0; s0 < n_splits; s0 += CH) {
    if (s0 > 0) {
      if ((s0 & 63) == 0) rec = rec_of(s0 + lane);
#pragma unroll
      for (int u = 0; u < CH; ++u) x[u] = row_of(s0 + u);
    }
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int sl = (s0 + u) & 63;  // the lane holding split s0 + u's record
      const float ms = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rec[0]), sl));
      const float ls = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rec[1]), sl));
      const float es = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rec[2]), sl));
      const float w = ms == -INFINITY ? 0.f : ls * exp2f(ms - M);  // 0 past the last split
      Ls += w;
      const float wgt = w * es;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = fmaf(wgt, f16_lo(x[u][i]), acc[2 * i]);
        acc[2 * i + 1] = fmaf(wgt, f16_hi(x[u][i]), acc[2 * i + 1]);
      }
    }
  }
  float Lt = Ls;
  const float rs = fold_sink(sink, h, M, Lt);
  const float inv = Lt > 0.f ? rs / Lt : 0.f;
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i] * inv, acc[2 * i + 1] * inv);
  *reinterpret_cast<u32x4*>(out + (qrow * n_h + h) * C + lane * 8) = o;
  if (lse && lane == 0) lse[qrow * n_h + h] = Lt > 0.f ? (M + __log2f(Lt)) * LN2 : -INFINITY;
}

// ---------------------------------------------------------------------------------------
// float32 path (c <= 256): one workgroup per query, scores held in LDS
// ---------------------------------------------------------------------------------------
struct AttnF32Args {
  const float* q;
  const float* ckv;
  const int* topk;
  const float* win;
  const int* win_pos;
  const int* q_pos;
  float* out;
  float* lse;
  const float* sink;  // [n_h] or null
  int Tq, n_h, c, Nc, k, L, W, m, is_csa, n_slots_c, n_slots;
  float scale;
};

__global__ __launch_bounds__(256) void attend_f32(AttnF32Args a) {
  extern __shared__ float sm[];
  float* S = sm;                                          // [n_h, n_slots]
  float* stat = S + (size_t)a.n_h * a.n_slots;            // [n_h] sums
  float* mx = stat + a.n_h;                               // [n_h] maxima
  long long* src = reinterpret_cast<long long*>(mx + a.n_h + ((a.n_h * 2 + a.n_h * a.n_slots) & 1));
  const int qrow = blockIdx.x;
  const int b = qrow / a.Tq, t = qrow - b * a.Tq;
  const long long p = (long long)a.q_pos[b] + t;
  const long long wp = a.win_pos[b];
  const int V = a.is_csa ? 0 : vis_count(p, a.m, a.Nc);
  // slot -> element offset (>= 0: compressed cache; < -1: window, encoded -2 - off; -1: none)
  for (int j = threadIdx.x; j < a.n_slots; j += blockDim.x) {
    long long o = -1;
    if (j < a.n_slots_c) {
      if (a.is_csa) {
        const int e = a.topk[(long long)qrow * a.k + j];
        if (e >= 0 && e < a.Nc) o = ((long long)b * a.Nc + e) * a.c;
      } else if (j < V) {
        o = ((long long)b * a.Nc + j) * a.c;
      }
    } else {
      const long long pos = p - a.W + 1 + (j - a.n_slots_c);
      const long long r = pos - wp;
      if (pos >= 0 && r >= 0 && r < a.L) o = -2 - ((long long)b * a.L + r) * a.c;
    }
    src[j] = o;
  }
  __syncthreads();
  const float* qb = a.q + (long long)qrow * a.n_h * a.c;
  for (int idx = threadIdx.x; idx < a.n_h * a.n_slots; idx += blockDim.x) {
    const int h = idx / a.n_slots, j = idx - h * a.n_slots;
    const long long o = src[j];
    float v = -INFINITY;
    if (o != -1) {
      const float* row = o >= 0 ? a.ckv + o : a.win + (-2 - o);
      float d = 0.f;
      for (int x = 0; x < a.c; ++x) d = fmaf(qb[h * a.c + x], row[x], d);
      v = d * a.scale;
    }
    S[idx] = v;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int h = wave; h < a.n_h; h += blockDim.x / 64) {
    float mm = -INFINITY;
    for (int j = lane; j < a.n_slots; j += 64) mm = fmaxf(mm, S[h * a.n_slots + j]);
    for (int d = 1; d < 64; d <<= 1) mm = fmaxf(mm, shfl_xor_f(mm, d));
    float sum = 0.f;
    for (int j = lane; j < a.n_slots; j += 64) {
      const float x = S[h * a.n_slots + j];
      const float e = mm == -INFINITY ? 0.f : expf(x - mm);
      S[h * a.n_slots + j] = e;
      sum += e;
    }
    for (int d = 1; d < 64; d <<= 1) sum += shfl_xor_f(sum, d);
    if (lane == 0) {
      if (a.sink && a.sink[h] != -INFINITY) {  // the sink joins the denominator only
        const float M = fmaxf(mm, a.sink[h]);
        const float r = mm == -INFINITY ? 0.f : expf(mm - M);
        for (int j = 0; j < a.n_slots; ++j) S[h * a.n_slots + j] *= r;
        sum = sum * r + expf(a.sink[h] - M);
        mm = M;
      }
      stat[h] = sum;
      mx[h] = mm;
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < a.n_h * a.c; idx += blockDim.x) {
    const int h = idx / a.c, x = idx - h * a.c;
    float acc = 0.f;
    for (int j = 0; j < a.n_slots; ++j) {
      const long long o = src[j];
      if (o == -1) continue;
      const float* row = o >= 0 ? a.ckv + o : a.win + (-2 - o);
      acc = fmaf(S[h * a.n_slots + j], row[x], acc);
    }
    const float l = stat[h];
    a.out[((long long)qrow * a.n_h + h) * a.c + x] = l > 0.f ? acc / l : 0.f;
  }
  if (a.lse)
    for (int h = threadIdx.x; h < a.n_h; h += blockDim.x)
      a.lse[(long long)qrow * a.n_h + h] = stat[h] > 0.f ? mx[h] + logf(stat[h]) : -INFINITY;
}

// ---------------------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------------------
struct Plan {
  int Tg, HPW, NW, NS, n_hg, n_slots, n_splits, RS, nqg, n_work, per_xcd;
  bool CS;  // column-split PV (one query per workgroup, 2 or 4 waves)
  size_t opart_bytes, ml_bytes, ws, lds;
};

// Launch shape.  A workgroup holds up to 64 heads (4 waves; 8 waves when two prefill
// queries share the rows).  When the queries alone give fewer than 256 workgroups their
// rows are split over more, each split holding whole iterations (32 rows with the 2-tile
// ring, 64 with the 4-tile one).
Plan make_plan(int B, int Tq, int n_h, int n_slots_c, int W, bool csa) {
  Plan P;
  // heads per workgroup: the largest of 64, 32, 16 that divides n_h (n_h % 16 == 0), so
  // that the head groups tile the heads exactly; queries per workgroup (HCA prefill with
  // at most 64 heads): a power of two up to 128 / HPW, so that the wave count
  // Tg * HPW / 16 is 1, 2, 4 or 8.  Other head counts (float32 calls, which take only
  // the workspace size from this plan) keep one group of n_h heads.
  P.HPW = n_h % 64 == 0 ? 64 : n_h % 32 == 0 ? 32 : n_h % 16 == 0 ? 16 : n_h;
  P.Tg = 1;
  if (!csa && Tq > 1 && n_h <= 64) {
    const int lim = Tq < 128 / P.HPW ? Tq : 128 / P.HPW;
    while (P.Tg * 2 <= lim) P.Tg *= 2;
  }
  P.NW = P.Tg * P.HPW / 16;
  P.n_hg = n_h / P.HPW;
  P.n_slots = n_slots_c + W + P.Tg - 1;
  P.nqg = cdiv(Tq, P.Tg);
  const long long base = (long long)P.n_hg * B * P.nqg;
  // The 4-tile ring (two tiles per iteration) where it costs no occupancy: 4-wave
  // prefill workgroups when there are few, and 8-wave ones (a whole CU's registers
  // anyway).  Decode keeps the 2-tile ring: two workgroups fit a CU, so the CSA and HCA
  // calls of one step, run side by side on two streams, share CUs instead of waiting for
  // whole ones (Pro 1M decode 81.2 -> 78.3 us per step; the 128K shapes unchanged).
  P.NS = ((P.NW == 4 && base < 256 && Tq > 1) || P.NW == 8) ? 4 : 2;
  // splits hold whole iterations (TPI tiles), at least one each
  const int tpi = P.NS >= 4 ? 2 : 1;
  const int niter = cdiv(cdiv(P.n_slots, TILE), tpi);
  const long long want = cdiv<long long>(256, base);
  int ns = (int)(want < niter ? want : niter);
  if (ns < 1) ns = 1;
  P.RS = cdiv(niter, ns) * tpi * TILE;
  P.n_splits = cdiv(P.n_slots, P.RS);
  P.n_work = (int)(base * P.n_splits);
  P.per_xcd = cdiv(P.n_work, 8);
  const long long nqh = (long long)B * Tq * n_h;
  P.opart_bytes = P.n_splits > 1 ? csahca::align_up((size_t)(nqh * P.n_splits * C * 2), 256) : 0;
  P.ml_bytes = P.n_splits > 1 ? csahca::align_up((size_t)(nqh * P.n_splits * 4 * 4), 256) : 0;
  P.ws = P.opart_bytes + P.ml_bytes;
  // column split only with the 2-tile ring (many workgroups, one tile per iteration):
  // with two tiles per iteration the exchange costs what the fewer transpose reads save;
  // and not at decode, where each workgroup runs few iterations and the exchange costs
  // what it saves
  P.CS = P.Tg == 1 && (P.NW == 2 || P.NW == 4) && P.NS == 2 && Tq > 1;
  P.lds = attend_lds_bytes(P.NS, P.NW, P.RS, csa, P.CS, true);  // room for the query norm gains
  return P;
}

template <int NW, int NS, bool CSA, bool CS>
int launch_attend(const Plan& P, const AttnArgs& A, hipStream_t st) {
  // raise the kernel's dynamic LDS limit once per process, whichever thread calls first
  // (the attribute belongs to the kernel, for every device)
  static std::once_flag once;
  static hipError_t attr = hipSuccess;
  std::call_once(once, [] {
    attr = hipFuncSetAttribute((const void*)attend_bf16<NW, NS, CSA, CS>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024 - 1024);
  });
  if (attr != hipSuccess) return csahca::fail(CSAHCA_ELAUNCH, "attend: cannot raise the LDS limit");
  hipLaunchKernelGGL((attend_bf16<NW, NS, CSA, CS>), dim3((unsigned)(P.per_xcd * 8)),
                     dim3(NW * 64), P.lds, st, A);
  return CSAHCA_OK;
}

template <bool CSA>
int launch_attend_nw(const Plan& P, const AttnArgs& A, hipStream_t st) {
  switch (P.NW) {
    case 1: return launch_attend<1, 2, CSA, false>(P, A, st);
    case 2:
      return P.CS ? launch_attend<2, 2, CSA, true>(P, A, st) : launch_attend<2, 2, CSA, false>(P, A, st);
    case 4:
      if (P.CS) return launch_attend<4, 2, CSA, true>(P, A, st);
      return P.NS == 4 ? launch_attend<4, 4, CSA, false>(P, A, st) : launch_attend<4, 2, CSA, false>(P, A, st);
    case 8: return launch_attend<8, 4, CSA, false>(P, A, st);
    default: return csahca::fail(CSAHCA_ENOTSUP, "attend: unsupported wave count");
  }
}

int check_attend(const char* name, const void* q, const void* ckv, const void* win_kv,
                 const int* win_pos, const int* q_pos, int B, int Tq, int n_h, int c, int N,
                 int L, int W, int dtype, const void* out, int n_slots_c) {
  using namespace csahca;
  if (!q || !ckv || !win_kv || !win_pos || !q_pos || !out) {
    set_error("%s: q, ckv, win_kv, win_pos, q_pos and out must be non-NULL", name);
    return CSAHCA_EINVAL;
  }
  if (B < 1 || Tq < 1 || n_h < 1 || c < 1 || N < 1 || L < 1 || W < 0) {
    set_error("%s: need B, Tq, n_h, c, N, L >= 1 and W >= 0", name);
    return CSAHCA_EINVAL;
  }
  if (!aligned16(q) || !aligned16(ckv) || !aligned16(win_kv) || !aligned16(out)) {
    set_error("%s: q, ckv, win_kv and out must be 16-byte aligned", name);
    return CSAHCA_EINVAL;
  }
  if (dtype == CSAHCA_BF16) {
    if (c != C || n_h % 16 != 0 || n_h > 128) {
      set_error("%s: bfloat16 needs c == 512, n_h %% 16 == 0 and n_h <= 128", name);
      return CSAHCA_ENOTSUP;
    }
  } else if (dtype == CSAHCA_F32) {
    if (c > 256 || c % 4 != 0 || (long long)n_h * (n_slots_c + W) > 12288) {
      set_error("%s: float32 needs c <= 256, c %% 4 == 0 and n_h * slots <= 12288", name);
      return CSAHCA_ENOTSUP;
    }
  } else {
    set_error("%s: dtype must be CSAHCA_BF16 or CSAHCA_F32", name);
    return CSAHCA_ENOTSUP;
  }
  if ((long long)n_slots_c + W + 8 > 0x3FFFFFFFLL || (long long)B * Tq * n_h > 0x7FFFFFFFLL) {
    set_error("%s: problem too large", name);
    return CSAHCA_ENOTSUP;
  }
  return CSAHCA_OK;
}

// RMSNorm + partial RoPE of the queries inside the attention kernel
struct NrArgs {
  const float* q_gamma = nullptr;
  int q_norm = 0, d_rope = 0;
  float eps = 0.f, theta = 1.f;
};

int check_nr(const char* name, const NrArgs& nr, int dtype) {
  using namespace csahca;
  if (nr.q_norm == 0) return CSAHCA_OK;
  if (nr.q_norm != 1) {
    set_error("%s: q_norm must be 0 or 1", name);
    return CSAHCA_EINVAL;
  }
  if (dtype != CSAHCA_BF16) {
    set_error("%s: RMSNorm + RoPE inside attention needs bfloat16", name);
    return CSAHCA_ENOTSUP;
  }
  if (nr.d_rope < 0 || nr.d_rope % 8 != 0 || nr.d_rope > 128) {
    set_error("%s: d_rope must be a multiple of 8 in [0, 128]", name);
    return CSAHCA_EINVAL;
  }
  if (!(nr.eps >= 0.f) || !(nr.theta > 0.f) || nr.theta == INFINITY || nr.eps == INFINITY) {
    set_error("%s: need eps >= 0 and theta > 0, both finite", name);
    return CSAHCA_EINVAL;
  }
  return CSAHCA_OK;
}

// phase: PHASE_ALL the attention launch and, with several splits, the split merge;
// PHASE_BEGIN the attention launch only; PHASE_END the split merge only (nothing when the
// plan has one split, or on the float32 path, whose one launch is the begin phase).
constexpr int PHASE_ALL = 0, PHASE_BEGIN = 1, PHASE_END = 2;

int attend_impl(const char* name, bool csa, const void* q, const void* ckv, const int* topk,
                const void* win_kv, const int* win_pos, const int* q_pos, int m, int B, int Tq,
                int n_h, int c, int N, int k, int L, int W, float scale, const float* sink,
                const NrArgs& nr, int dtype, void* out, float* lse, void* workspace, size_t ws_bytes,
                hipStream_t st, int phase = PHASE_ALL) {
  using namespace csahca;
  const int n_slots_c = csa ? k : N;
  if (dtype == CSAHCA_F32 && phase == PHASE_END) {
    clear_error();
    return CSAHCA_OK;
  }
  if (dtype == CSAHCA_F32) {
    AttnF32Args A;
    A.q = (const float*)q;
    A.ckv = (const float*)ckv;
    A.topk = topk;
    A.win = (const float*)win_kv;
    A.win_pos = win_pos;
    A.q_pos = q_pos;
    A.out = (float*)out;
    A.lse = lse;
    A.sink = sink;
    A.Tq = Tq;
    A.n_h = n_h;
    A.c = c;
    A.Nc = N;
    A.k = k;
    A.L = L;
    A.W = W;
    A.m = m;
    A.is_csa = csa;
    A.n_slots_c = n_slots_c;
    A.n_slots = n_slots_c + W;
    A.scale = scale;
    const size_t lds = ((size_t)n_h * A.n_slots + 2 * n_h + 2) * 4 + (size_t)A.n_slots * 8;
    if (lds > 65536) {
      set_error("%s: float32 problem needs too much LDS", name);
      return CSAHCA_ENOTSUP;
    }
    hipLaunchKernelGGL(attend_f32, dim3((unsigned)(B * Tq)), dim3(256), lds, st, A);
    return launch_status(name);
  }
  const Plan P = make_plan(B, Tq, n_h, n_slots_c, W, csa);
  if (P.n_splits > 1 && (!workspace || ws_bytes < P.ws)) {
    set_error("%s: workspace missing or too small (%zu bytes needed)", name, P.ws);
    return CSAHCA_EWORKSPACE;
  }
  AttnArgs A;
  A.q = (const uint16_t*)q;
  A.ckv = (const uint16_t*)ckv;
  A.topk = topk;
  A.win = (const uint16_t*)win_kv;
  A.win_pos = win_pos;
  A.q_pos = q_pos;
  A.out = (uint16_t*)out;
  A.lse = lse;
  A.sink = sink;
  A.q_gamma = nr.q_gamma;
  A.qnr = nr.q_norm;
  A.d_rope = nr.d_rope;
  A.nr_eps = nr.eps;
  A.nr_theta = nr.theta;
  A.opart = P.n_splits > 1 ? (uint16_t*)workspace : nullptr;
  A.mlpart = P.n_splits > 1 ? (float*)((char*)workspace + P.opart_bytes) : nullptr;
  A.B = B;
  A.Tq = Tq;
  A.n_h = n_h;
  A.Nc = N;
  A.k = k;
  A.L = L;
  A.W = W;
  A.m = m;
  A.is_csa = csa;
  A.n_slots_c = n_slots_c;
  A.n_slots = P.n_slots;
  A.Tg = P.Tg;
  A.HPW = P.HPW;
  A.nqg = P.nqg;
  A.n_splits = P.n_splits;
  A.RS = P.RS;
  A.scale_log2 = scale * LOG2E;
  A.n_hg = P.n_hg;
  A.n_work = P.n_work;
  A.per_xcd = P.per_xcd;
  if (P.lds > 160 * 1024 - 1024) {
    set_error("%s: a split needs too much LDS", name);
    return CSAHCA_ENOTSUP;
  }
  if (phase != PHASE_END) {
    const int lrc = csa ? launch_attend_nw<true>(P, A, st) : launch_attend_nw<false>(P, A, st);
    if (lrc != CSAHCA_OK) return lrc;
    const int rc = launch_status(name);
    if (rc != CSAHCA_OK || P.n_splits == 1 || phase == PHASE_BEGIN) return rc;
  } else if (P.n_splits == 1) {
    clear_error();
    return CSAHCA_OK;
  }
  const long long nqh = (long long)B * Tq * n_h;
  // few splits: one wave per pair loads them all at once; many: four waves per pair
  if (P.n_splits <= COMBINE_WAVE_SPLITS)
    hipLaunchKernelGGL(attend_combine_wave, dim3((unsigned)cdiv<long long>(nqh, 4)), dim3(256), 0, st,
                       A.opart, A.mlpart, A.out, lse, sink, n_h, P.n_splits, nqh);
  else
    hipLaunchKernelGGL(attend_combine, dim3((unsigned)nqh), dim3(256), 0, st, A.opart, A.mlpart, A.out,
                       lse, sink, n_h, P.n_splits);
  return launch_status(name);
}

}  // namespace

extern "C" size_t csa_attend_workspace_size(int B, int Tq, int n_h, int c, int k, int W) {
  (void)c;
  if (B < 1 || Tq < 1 || n_h < 1 || k < 1 || W < 0) return 0;
  return make_plan(B, Tq, n_h, k, W, true).ws;
}

extern "C" size_t hca_attend_workspace_size(int B, int Tq, int n_h, int c, int N_h, int W) {
  (void)c;
  if (B < 1 || Tq < 1 || n_h < 1 || N_h < 1 || W < 0) return 0;
  return make_plan(B, Tq, n_h, N_h, W, false).ws;
}

namespace {

int csa_entry(const char* name, const void* q, const void* ckv, const int* topk_idx,
              const void* win_kv, const int* win_pos, const int* q_pos, int B, int Tq, int n_h,
              int c, int N_c, int k, int L, int W, float scale, const float* sink, const NrArgs& nr,
              int dtype, void* out, float* lse, void* workspace, size_t ws_bytes, void* stream,
              int phase = PHASE_ALL) {
  using namespace csahca;
  int rc = check_attend(name, q, ckv, win_kv, win_pos, q_pos, B, Tq, n_h, c, N_c, L, W, dtype, out, k);
  if (rc != CSAHCA_OK) return rc;
  if ((rc = check_nr(name, nr, dtype)) != CSAHCA_OK) return rc;
  if (!topk_idx || k < 1) {
    set_error("%s: topk_idx must be non-NULL and k >= 1", name);
    return CSAHCA_EINVAL;
  }
  if (!(scale > 0.f) || scale != scale) {
    set_error("%s: scale must be > 0", name);
    return CSAHCA_EINVAL;
  }
  return attend_impl(name, true, q, ckv, topk_idx, win_kv, win_pos, q_pos, 1, B, Tq, n_h, c, N_c, k,
                     L, W, scale, sink, nr, dtype, out, lse, workspace, ws_bytes, (hipStream_t)stream, phase);
}

int hca_entry(const char* name, const void* q, const void* ckv, const void* win_kv,
              const int* win_pos, const int* q_pos, int m, int B, int Tq, int n_h, int c, int N_h,
              int L, int W, float scale, const float* sink, const NrArgs& nr, int dtype, void* out,
              float* lse, void* workspace, size_t ws_bytes, void* stream, int phase = PHASE_ALL) {
  using namespace csahca;
  int rc = check_attend(name, q, ckv, win_kv, win_pos, q_pos, B, Tq, n_h, c, N_h, L, W, dtype, out, N_h);
  if (rc != CSAHCA_OK) return rc;
  if ((rc = check_nr(name, nr, dtype)) != CSAHCA_OK) return rc;
  if (m < 1) {
    set_error("%s: m must be >= 1", name);
    return CSAHCA_EINVAL;
  }
  if (!(scale > 0.f) || scale != scale) {
    set_error("%s: scale must be > 0", name);
    return CSAHCA_EINVAL;
  }
  return attend_impl(name, false, q, ckv, nullptr, win_kv, win_pos, q_pos, m, B, Tq, n_h, c, N_h, N_h,
                     L, W, scale, sink, nr, dtype, out, lse, workspace, ws_bytes, (hipStream_t)stream, phase);
}

}  // namespace

extern "C" int csa_attend(const void* q, const void* ckv, const int* topk_idx,
                          const void* win_kv, const int* win_pos, const int* q_pos, int B,
                          int Tq, int n_h, int c, int N_c, int k, int L, int W, float scale,
                          int dtype, void* out, float* lse, void* workspace, size_t ws_bytes,
                          void* stream) {
  return csa_entry("csa_attend", q, ckv, topk_idx, win_kv, win_pos, q_pos, B, Tq, n_h, c, N_c, k, L,
                   W, scale, nullptr, NrArgs{}, dtype, out, lse, workspace, ws_bytes, stream);
}

extern "C" int hca_attend(const void* q, const void* ckv, const void* win_kv, const int* win_pos,
                          const int* q_pos, int m, int B, int Tq, int n_h, int c, int N_h,
                          int L, int W, float scale, int dtype, void* out, float* lse,
                          void* workspace, size_t ws_bytes, void* stream) {
  return hca_entry("hca_attend", q, ckv, win_kv, win_pos, q_pos, m, B, Tq, n_h, c, N_h, L, W, scale,
                   nullptr, NrArgs{}, dtype, out, lse, workspace, ws_bytes, stream);
}

extern "C" int csa_attend_sink(const void* q, const void* ckv, const int* topk_idx,
                               const void* win_kv, const int* win_pos, const int* q_pos, int B,
                               int Tq, int n_h, int c, int N_c, int k, int L, int W, float scale,
                               const float* sink, int dtype, void* out, float* lse,
                               void* workspace, size_t ws_bytes, void* stream) {
  return csa_entry("csa_attend_sink", q, ckv, topk_idx, win_kv, win_pos, q_pos, B, Tq, n_h, c, N_c,
                   k, L, W, scale, sink, NrArgs{}, dtype, out, lse, workspace, ws_bytes, stream);
}

extern "C" int hca_attend_sink(const void* q, const void* ckv, const void* win_kv,
                               const int* win_pos, const int* q_pos, int m, int B, int Tq,
                               int n_h, int c, int N_h, int L, int W, float scale,
                               const float* sink, int dtype, void* out, float* lse,
                               void* workspace, size_t ws_bytes, void* stream) {
  return hca_entry("hca_attend_sink", q, ckv, win_kv, win_pos, q_pos, m, B, Tq, n_h, c, N_h, L, W,
                   scale, sink, NrArgs{}, dtype, out, lse, workspace, ws_bytes, stream);
}

extern "C" int csa_attend_ex(const void* q, const void* ckv, const int* topk_idx,
                             const void* win_kv, const int* win_pos, const int* q_pos, int B,
                             int Tq, int n_h, int c, int N_c, int k, int L, int W, float scale,
                             const float* sink, const float* q_gamma, int q_norm, int d_rope,
                             float eps, float theta, int dtype, void* out, float* lse,
                             void* workspace, size_t ws_bytes, void* stream) {
  return csa_entry("csa_attend_ex", q, ckv, topk_idx, win_kv, win_pos, q_pos, B, Tq, n_h, c, N_c, k,
                   L, W, scale, sink, NrArgs{q_gamma, q_norm, d_rope, eps, theta},
                   dtype, out, lse, workspace, ws_bytes, stream);
}

extern "C" int hca_attend_ex(const void* q, const void* ckv, const void* win_kv,
                             const int* win_pos, const int* q_pos, int m, int B, int Tq,
                             int n_h, int c, int N_h, int L, int W, float scale,
                             const float* sink, const float* q_gamma, int q_norm, int d_rope,
                             float eps, float theta, int dtype, void* out, float* lse,
                             void* workspace, size_t ws_bytes, void* stream) {
  return hca_entry("hca_attend_ex", q, ckv, win_kv, win_pos, q_pos, m, B, Tq, n_h, c, N_h, L, W,
                   scale, sink, NrArgs{q_gamma, q_norm, d_rope, eps, theta}, dtype,
                   out, lse, workspace, ws_bytes, stream);
}

// The two halves of csa_attend_ex / hca_attend_ex: the attention launch, and the split
// merge, so that a caller can run the merge on another stream than the attention.
extern "C" int csa_attend_begin(const void* q, const void* ckv, const int* topk_idx,
                                const void* win_kv, const int* win_pos, const int* q_pos, int B,
                                int Tq, int n_h, int c, int N_c, int k, int L, int W, float scale,
                                const float* sink, const float* q_gamma, int q_norm, int d_rope,
                                float eps, float theta, int dtype, void* out, float* lse,
                                void* workspace, size_t ws_bytes, void* stream) {
  return csa_entry("csa_attend_begin", q, ckv, topk_idx, win_kv, win_pos, q_pos, B, Tq, n_h, c, N_c, k,
                   L, W, scale, sink, NrArgs{q_gamma, q_norm, d_rope, eps, theta}, dtype, out, lse,
                   workspace, ws_bytes, stream, PHASE_BEGIN);
}

extern "C" int csa_attend_end(const void* q, const void* ckv, const int* topk_idx,
                              const void* win_kv, const int* win_pos, const int* q_pos, int B,
                              int Tq, int n_h, int c, int N_c, int k, int L, int W, float scale,
                              const float* sink, const float* q_gamma, int q_norm, int d_rope,
                              float eps, float theta, int dtype, void* out, float* lse,
                              void* workspace, size_t ws_bytes, void* stream) {
  return csa_entry("csa_attend_end", q, ckv, topk_idx, win_kv, win_pos, q_pos, B, Tq, n_h, c, N_c, k,
                   L, W, scale, sink, NrArgs{q_gamma, q_norm, d_rope, eps, theta}, dtype, out, lse,
                   workspace, ws_bytes, stream, PHASE_END);
}

extern "C" int hca_attend_begin(const void* q, const void* ckv, const void* win_kv,
                                const int* win_pos, const int* q_pos, int m, int B, int Tq,
                                int n_h, int c, int N_h, int L, int W, float scale,
                                const float* sink, const float* q_gamma, int q_norm, int d_rope,
                                float eps, float theta, int dtype, void* out, float* lse,
                                void* workspace, size_t ws_bytes, void* stream) {
  return hca_entry("hca_attend_begin", q, ckv, win_kv, win_pos, q_pos, m, B, Tq, n_h, c, N_h, L, W,
                   scale, sink, NrArgs{q_gamma, q_norm, d_rope, eps, theta}, dtype, out, lse, workspace,
                   ws_bytes, stream, PHASE_BEGIN);
}

extern "C" int hca_attend_end(const void* q, const void* ckv, const void* win_kv,
                              const int* win_pos, const int* q_pos, int m, int B, int Tq,
                              int n_h, int c, int N_h, int L, int W, float scale,
                              const float* sink, const float* q_gamma, int q_norm, int d_rope,
                              float eps, float theta, int dtype, void* out, float* lse,
                              void* workspace, size_t ws_bytes, void* stream) {
  return hca_entry("hca_attend_end", q, ckv, win_kv, win_pos, q_pos, m, B, Tq, n_h, c, N_h, L, W,
                   scale, sink, NrArgs{q_gamma, q_norm, d_rope, eps, theta}, dtype, out, lse, workspace,
                   ws_bytes, stream, PHASE_END);
}
