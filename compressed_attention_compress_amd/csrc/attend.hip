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
//   * the 32 rows are read once from HBM (each wave issues one 1 KiB row per load; rows
//     of the next tile are in flight in registers while the current tile is computed)
//     and staged in LDS with a 16-byte row pad;
//   * every wave owns 16 (query, head) pairs.  S^T = E . Q^T on MFMA
//     (v_mfma_f32_16x16x32_bf16, A = 16 rows x 32 dims from LDS, B = Q from registers);
//     the accumulator layout puts one head per lane column, so the online-softmax
//     statistics of a head live in the lanes that also hold its output;
//   * O^T += E^T . P^T on MFMA: P stays in registers in exactly the layout the S
//     accumulator produced it; E^T comes from LDS as 32-bit words holding two adjacent
//     columns, which feed an "even column" and an "odd column" MFMA each.
// float32 path: plain FMA over LDS-resident scores (small heads only).
#include "common.hpp"

namespace {

constexpr int C = 512;            // head dim of the bf16 path
constexpr int TILE = 32;          // slots per LDS tile
constexpr int ROWB = C * 2 + 16;  // LDS row stride in bytes
constexpr int KS = C / 32;        // MFMA K-steps of S (16 x 32 dims)
constexpr int CPAIRS = C / 32;    // 32-column blocks of O
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* ckv;
  const int* topk;
  const uint16_t* win;
  const int* win_pos;
  const int* q_pos;
  uint16_t* out;
  float* lse;
  float* opart;   // [nq, n_splits, n_h, C] unnormalised partial outputs
  float* mlpart;  // [nq, n_splits, n_h, 2] running max (log2 units) and sum
  int B, Tq, n_h, Nc, k, L, W, m;
  int is_csa;
  int n_slots_c;  // compressed slots: k (CSA) or Nc (HCA)
  int n_slots;    // n_slots_c + W + Tg - 1
  int Tg;         // consecutive query tokens per workgroup (HCA prefill shares rows)
  int HPW;        // heads per workgroup
  int nqg;        // query groups per sequence
  int n_splits, RS;
  float scale_log2;
};

CSAHCA_DEV int vis_count(long long p, int m, int N) {
  long long v = (p + 1) / m;
  if (p + 1 <= 0) v = 0;
  return (int)(v < N ? v : N);
}

template <int NW>
__global__ __launch_bounds__(NW * 64) void attend_bf16(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[TILE * ROWB];
  __shared__ int row_ok[TILE];
  constexpr int NT = NW * 64;
  constexpr int LOADS = TILE / NW;  // rows each wave loads per tile

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row16 = lane & 15, g = lane >> 4;
  const int split = blockIdx.x, hg = blockIdx.y, qg = blockIdx.z;
  const int b = qg / a.nqg;
  const int t0 = (qg - b * a.nqg) * a.Tg;
  const int wpq = a.HPW / 16;
  const int tq = t0 + wave / wpq;
  const int h0 = hg * a.HPW + (wave % wpq) * 16;
  const bool active = tq < a.Tq;
  const int tlast = min(t0 + a.Tg, a.Tq) - 1;
  const long long qpos0 = a.q_pos[b];
  const long long pfirst = qpos0 + t0, plast = qpos0 + tlast;
  const long long p = qpos0 + (active ? tq : tlast);
  const long long wp = a.win_pos[b];
  const int Vw = a.is_csa ? 0 : vis_count(p, a.m, a.Nc);
  const int Vu = a.is_csa ? 0 : vis_count(plast, a.m, a.Nc);
  const int slot_lo = split * a.RS;
  const int slot_hi = min(a.n_slots, slot_lo + a.RS);
  const long long qrow = (long long)b * a.Tq + (active ? tq : tlast);

  // source row of a slot for the union of this workgroup's queries (nullptr: skipped)
  auto slot_src = [&](int j) -> const uint16_t* {
    if (j >= slot_hi) return nullptr;
    if (j < a.n_slots_c) {
      if (a.is_csa) {
        const int e = a.topk[((long long)b * a.Tq + t0) * a.k + j];
        if (e < 0 || e >= a.Nc) return nullptr;
        return a.ckv + ((long long)b * a.Nc + e) * C;
      }
      if (j >= Vu) return nullptr;
      return a.ckv + ((long long)b * a.Nc + j) * C;
    }
    const long long pos = pfirst - a.W + 1 + (j - a.n_slots_c);
    if (pos < 0 || pos > plast) return nullptr;
    const long long r = pos - wp;
    if (r < 0 || r >= a.L) return nullptr;
    return a.win + ((long long)b * a.L + r) * C;
  };
  // is slot j (usable by the workgroup) usable by this wave's query?
  auto slot_mine = [&](int j) -> bool {
    if (j < a.n_slots_c) return a.is_csa || j < Vw;
    const long long pos = pfirst - a.W + 1 + (j - a.n_slots_c);
    return pos <= p && pos > p - a.W;
  };

  bf16x8 qf[KS];
  if (active) {
    const uint16_t* qp = a.q + (qrow * a.n_h + h0 + row16) * C + g * (C / 4);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qp + ks * 8));
  } else {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
  }

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 oacc[CPAIRS][2];
#pragma unroll
  for (int cp = 0; cp < CPAIRS; ++cp) {
    oacc[cp][0] = f32x4{0.f, 0.f, 0.f, 0.f};
    oacc[cp][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  u32x4 pre[LOADS];
  int pre_ok[LOADS];
  auto fetch = [&](int it) {
    const int base = slot_lo + it * TILE;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int r = wave + i * NW;  // wave-uniform row of the tile
      const uint16_t* src = slot_src(base + r);
      pre_ok[i] = src != nullptr;
      pre[i] = src ? *reinterpret_cast<const u32x4*>(src + lane * 8) : u32x4{0, 0, 0, 0};
    }
  };

  const int ntile = slot_hi > slot_lo ? cdiv(slot_hi - slot_lo, TILE) : 0;
  if (ntile > 0) fetch(0);
  for (int it = 0; it < ntile; ++it) {
    __syncthreads();  // the previous tile is no longer read
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int r = wave + i * NW;
      *reinterpret_cast<u32x4*>(tile + r * ROWB + lane * 16) = pre[i];
      if (lane == 0) row_ok[r] = pre_ok[i];
    }
    __syncthreads();
    if (it + 1 < ntile) fetch(it + 1);
    if (!active) continue;

    const int base = slot_lo + it * TILE;
    // ---- S^T = E Q^T for 2 blocks of 16 slots ----
    f32x4 s[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      s[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
      const uint8_t* rp = tile + (rb * 16 + row16) * ROWB + g * (C / 4) * 2;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 ef = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(rp + ks * 16));
        s[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ef, qf[ks], s[rb], 0, 0, 0);
      }
    }
    // lane: head h0 + row16, slots base + rb*16 + 4g + i
    float sv[8];
    float mloc = -INFINITY;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = rb * 16 + 4 * g + i;
        const int j = base + r;
        const bool ok = j < slot_hi && row_ok[r] && slot_mine(j);
        const float x = ok ? s[rb][i] * a.scale_log2 : -INFINITY;
        sv[rb * 4 + i] = x;
        mloc = fmaxf(mloc, x);
      }
    mloc = fmaxf(mloc, shfl_xor_f(mloc, 16));
    mloc = fmaxf(mloc, shfl_xor_f(mloc, 32));
    const float m_new = fmaxf(m_run, mloc);
    float alpha = 1.f;
    float pe[8];
    float psum = 0.f;
    if (m_new == -INFINITY) {
#pragma unroll
      for (int e = 0; e < 8; ++e) pe[e] = 0.f;
    } else {
      alpha = exp2f(m_run - m_new);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pe[e] = exp2f(sv[e] - m_new);
        psum += pe[e];
      }
    }
    psum += shfl_xor_f(psum, 16);
    psum += shfl_xor_f(psum, 32);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int cp = 0; cp < CPAIRS; ++cp)
#pragma unroll
        for (int par = 0; par < 2; ++par) oacc[cp][par] *= alpha;
    }
    // P^T as the B operand: k-slot e <-> slot (e < 4 ? 4g+e : 16+4g+e-4)
    const u32x4 pw = {pack_bf16x2(pe[0], pe[1]), pack_bf16x2(pe[2], pe[3]),
                      pack_bf16x2(pe[4], pe[5]), pack_bf16x2(pe[6], pe[7])};
    const bf16x8 pf = __builtin_bit_cast(bf16x8, pw);
    // ---- O^T += E^T P^T ----
#pragma unroll
    for (int cp = 0; cp < CPAIRS; ++cp) {
      const uint8_t* cpb = tile + (32 * cp + 2 * row16) * 2;
      uint32_t wv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4);
        wv[e] = *reinterpret_cast<const uint32_t*>(cpb + r * ROWB);
      }
      u32x4 ev, od;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ev[e] = (wv[2 * e] & 0xFFFFu) | (wv[2 * e + 1] << 16);
        od[e] = (wv[2 * e] >> 16) | (wv[2 * e + 1] & 0xFFFF0000u);
      }
      oacc[cp][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ev), pf,
                                                            oacc[cp][0], 0, 0, 0);
      oacc[cp][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, od), pf,
                                                            oacc[cp][1], 0, 0, 0);
    }
  }
  if (!active) return;

  // lane: head h0 + row16; oacc[cp][par][i] is column 32*cp + 8*g + 2*i + par
  const int h = h0 + row16;
  if (a.n_splits == 1) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    uint16_t* op = a.out + (qrow * a.n_h + h) * C + 8 * g;
#pragma unroll
    for (int cp = 0; cp < CPAIRS; ++cp) {
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(oacc[cp][0][i] * inv, oacc[cp][1][i] * inv);
      *reinterpret_cast<u32x4*>(op + 32 * cp) = o;
    }
    if (a.lse && g == 0)
      a.lse[qrow * a.n_h + h] = l_run > 0.f ? (m_run + __log2f(l_run)) * LN2 : -INFINITY;
  } else {
    const long long pr = (qrow * a.n_splits + split) * a.n_h + h;
    float* op = a.opart + pr * C + 8 * g;
#pragma unroll
    for (int cp = 0; cp < CPAIRS; ++cp) {
      const f32x4 lo = {oacc[cp][0][0], oacc[cp][1][0], oacc[cp][0][1], oacc[cp][1][1]};
      const f32x4 hi = {oacc[cp][0][2], oacc[cp][1][2], oacc[cp][0][3], oacc[cp][1][3]};
      *reinterpret_cast<f32x4*>(op + 32 * cp) = lo;
      *reinterpret_cast<f32x4*>(op + 32 * cp + 4) = hi;
    }
    if (g == 0) {
      a.mlpart[pr * 2 + 0] = m_run;
      a.mlpart[pr * 2 + 1] = l_run;
    }
  }
}

// merge the splits of every (query, head) by their log-sum-exp; one wave per pair
__global__ __launch_bounds__(256) void attend_combine(const float* __restrict__ opart,
                                                      const float* __restrict__ mlpart,
                                                      uint16_t* __restrict__ out,
                                                      float* __restrict__ lse, long long nqh,
                                                      int n_h, int n_splits) {
  const long long pair = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (pair >= nqh) return;
  const long long qrow = pair / n_h;
  const int h = (int)(pair - qrow * n_h);
  float M = -INFINITY;
  for (int s = 0; s < n_splits; ++s)
    M = fmaxf(M, mlpart[((qrow * n_splits + s) * n_h + h) * 2]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float Ls = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < n_splits; ++s) {
      const long long pr = (qrow * n_splits + s) * n_h + h;
      const float ms = mlpart[pr * 2], ls = mlpart[pr * 2 + 1];
      const float wgt = ms == -INFINITY ? 0.f : exp2f(ms - M);
      Ls = fmaf(wgt, ls, Ls);
      const f32x4 x0 = *reinterpret_cast<const f32x4*>(opart + pr * C + lane * 8);
      const f32x4 x1 = *reinterpret_cast<const f32x4*>(opart + pr * C + lane * 8 + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i] = fmaf(wgt, x0[i], acc[i]);
        acc[4 + i] = fmaf(wgt, x1[i], acc[4 + i]);
      }
    }
  }
  const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i] * inv, acc[2 * i + 1] * inv);
  *reinterpret_cast<u32x4*>(out + (qrow * n_h + h) * C + lane * 8) = o;
  if (lse && lane == 0) lse[qrow * n_h + h] = Ls > 0.f ? (M + __log2f(Ls)) * LN2 : -INFINITY;
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
  int Tg, HPW, NW, n_slots, n_splits, RS, nqg;
  size_t opart_bytes, ml_bytes, ws;
};

Plan make_plan(int B, int Tq, int n_h, int n_slots_c, int W, bool csa) {
  Plan P;
  P.Tg = 1;
  if (!csa && Tq > 1 && n_h <= 64) P.Tg = 128 / n_h < Tq ? 128 / n_h : Tq;
  if (P.Tg > 8) P.Tg = 8;
  P.HPW = n_h * P.Tg <= 128 ? n_h : 128 / P.Tg;
  P.NW = P.Tg * P.HPW / 16;
  P.n_slots = n_slots_c + W + P.Tg - 1;
  P.nqg = cdiv(Tq, P.Tg);
  const long long base = (long long)(n_h / P.HPW) * B * P.nqg;
  const int ntile = cdiv(P.n_slots, TILE);
  long long want = cdiv<long long>(512, base);
  int maxs = ntile / 2 > 1 ? ntile / 2 : 1;  // at least 2 tiles per split
  int ns = (int)(want < maxs ? want : maxs);
  if (ns < 1) ns = 1;
  P.RS = cdiv(ntile, ns) * TILE;
  P.n_splits = cdiv(P.n_slots, P.RS);
  const long long nqh = (long long)B * Tq * n_h;
  P.opart_bytes = P.n_splits > 1 ? csahca::align_up((size_t)(nqh * P.n_splits * C * 4), 256) : 0;
  P.ml_bytes = P.n_splits > 1 ? csahca::align_up((size_t)(nqh * P.n_splits * 2 * 4), 256) : 0;
  P.ws = P.opart_bytes + P.ml_bytes;
  return P;
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
      set_error("%s: bfloat16 needs c == 512, n_h % 16 == 0 and n_h <= 128", name);
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

int attend_impl(const char* name, bool csa, const void* q, const void* ckv, const int* topk,
                const void* win_kv, const int* win_pos, const int* q_pos, int m, int B, int Tq,
                int n_h, int c, int N, int k, int L, int W, float scale, int dtype, void* out,
                float* lse, void* workspace, size_t ws_bytes, hipStream_t st) {
  using namespace csahca;
  const int n_slots_c = csa ? k : N;
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
  A.opart = P.n_splits > 1 ? (float*)workspace : nullptr;
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
  dim3 grid((unsigned)P.n_splits, (unsigned)(n_h / P.HPW), (unsigned)(B * P.nqg));
  switch (P.NW) {
    case 1: hipLaunchKernelGGL(attend_bf16<1>, grid, dim3(64), 0, st, A); break;
    case 2: hipLaunchKernelGGL(attend_bf16<2>, grid, dim3(128), 0, st, A); break;
    case 4: hipLaunchKernelGGL(attend_bf16<4>, grid, dim3(256), 0, st, A); break;
    case 8: hipLaunchKernelGGL(attend_bf16<8>, grid, dim3(512), 0, st, A); break;
    default:
      set_error("%s: unsupported wave count %d", name, P.NW);
      return CSAHCA_ENOTSUP;
  }
  int rc = launch_status(name);
  if (rc != CSAHCA_OK || P.n_splits == 1) return rc;
  const long long nqh = (long long)B * Tq * n_h;
  hipLaunchKernelGGL(attend_combine, dim3((unsigned)cdiv<long long>(nqh, 4)), dim3(256), 0, st,
                     A.opart, A.mlpart, A.out, lse, nqh, n_h, P.n_splits);
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

extern "C" int csa_attend(const void* q, const void* ckv, const int* topk_idx,
                          const void* win_kv, const int* win_pos, const int* q_pos, int B,
                          int Tq, int n_h, int c, int N_c, int k, int L, int W, float scale,
                          int dtype, void* out, float* lse, void* workspace, size_t ws_bytes,
                          void* stream) {
  using namespace csahca;
  int rc = check_attend("csa_attend", q, ckv, win_kv, win_pos, q_pos, B, Tq, n_h, c, N_c, L, W,
                        dtype, out, k);
  if (rc != CSAHCA_OK) return rc;
  if (!topk_idx || k < 1) return fail(CSAHCA_EINVAL, "csa_attend: topk_idx must be non-NULL and k >= 1");
  if (!(scale > 0.f) || scale != scale) return fail(CSAHCA_EINVAL, "csa_attend: scale must be > 0");
  return attend_impl("csa_attend", true, q, ckv, topk_idx, win_kv, win_pos, q_pos, 1, B, Tq,
                     n_h, c, N_c, k, L, W, scale, dtype, out, lse, workspace, ws_bytes,
                     (hipStream_t)stream);
}

extern "C" int hca_attend(const void* q, const void* ckv, const void* win_kv, const int* win_pos,
                          const int* q_pos, int m, int B, int Tq, int n_h, int c, int N_h,
                          int L, int W, float scale, int dtype, void* out, float* lse,
                          void* workspace, size_t ws_bytes, void* stream) {
  using namespace csahca;
  int rc = check_attend("hca_attend", q, ckv, win_kv, win_pos, q_pos, B, Tq, n_h, c, N_h, L, W,
                        dtype, out, N_h);
  if (rc != CSAHCA_OK) return rc;
  if (m < 1) return fail(CSAHCA_EINVAL, "hca_attend: m must be >= 1");
  if (!(scale > 0.f) || scale != scale) return fail(CSAHCA_EINVAL, "hca_attend: scale must be > 0");
  return attend_impl("hca_attend", false, q, ckv, nullptr, win_kv, win_pos, q_pos, m, B, Tq, n_h,
                     c, N_h, N_h, L, W, scale, dtype, out, lse, workspace, ws_bytes,
                     (hipStream_t)stream);
}
