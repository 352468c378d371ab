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
#include <mutex>
#include <type_traits>

#include "normrope.hpp"
#include "pool.hpp"
#include "pool_device.hpp"

namespace {

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
  // NR: the gains of this thread's first channel of the epilogue (and its pair partner),
  // loaded now so that their latency hides under the pooling
  float g_t = 1.f, g_u = 1.f;
  if (NR && nr.gamma && (int)threadIdx.x < c) {
    g_t = nr.gamma[threadIdx.x];
    g_u = nr.gamma[threadIdx.x ^ 1];
  }
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
      const bool first = t == (int)threadIdx.x;  // gains loaded at the start
      const float gt = !nr.gamma ? 1.f : first ? g_t : nr.gamma[t];
      const float gu = !nr.gamma ? 1.f : first ? g_u : nr.gamma[u];
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

// Workgroup size cap of the norm's block path: 1024 threads (128 registers each) hold the
// plain bf16 pooling's loads in flight; the other forms (float, bias, two streams,
// append) need more registers per thread than 512-thread workgroups leave them (128), so
// they take 256
template <typename T, bool HAS_P, int MODE>
constexpr int nr_block_threads() {
  return (sizeof(T) == 2 && !HAS_P && MODE == PLAIN) ? 1024 : 256;
}

template <typename T, int UB, bool HAS_P, int MODE, bool NR>
__global__ __launch_bounds__((NR ? nr_block_threads<T, HAS_P, MODE>() : 256)) void pool_block_kernel(const T* __restrict__ X,
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

// ... and with the norm: the block path holds the whole entry (CVG = all slices) in at
// most 1024 threads, the per-slice path runs 1024-thread workgroups
PoolPlan plan_norm(int B, long long N, int c, int m) {
  PoolPlan p{};
  p.total = (long long)B * N * (c / 8);
  const int CV = c / VEC;
  p.block = p.total < 32768 && m >= 8;
  if (p.block) {
    const int unit = CV >= 64 ? 1 : 64 / CV;
    const int span = max(4, cdiv(m, 1024 / CV));
    p.S = cdiv(cdiv(m, span), unit) * unit;
    p.CVG = CV;
    p.lds = ((size_t)p.S * CV * 3 * VEC + (size_t)c + 16) * sizeof(float);
    p.grid = (unsigned)(B * N);
    p.threads = (unsigned)(p.S * CV);
    p.ub = (span % 8 == 0 && m % 8 == 0) ? 8 : 4;
  } else {
    p.grid = (unsigned)cdiv<long long>(p.total, 1024);
    p.threads = 1024;
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
  const float* gamma;  // NR: this side's gain
  long long entry0;    // NR: cache index of the first entry (its position is m * entry0)
};

// Rows normalised and rotated beside a paired pooling with the norm (a decode step's new
// window rows): T rows per sequence, row (b, t) at x + b * x_bs + t * c, position
// pos[b] + t (0 + t without pos), written to y likewise; the gain is the side's.
template <typename T>
struct RowSide {
  const T* x;
  T* y;
  const int* pos;
  long long x_bs, y_bs;
  const float* gamma;
  int T_;
};

// Two poolings in one launch: workgroups [0, gridA) run side A on pool_kernel's layout,
// workgroups [gridA, gridAB) side B on pool_block_kernel's (256 threads each; 1024 with
// the norm).  With the norm, the workgroups from gridAB on normalise the rows of RA then
// RB (B sequences each), one row per c/8 consecutive lanes.
template <typename T, int UBA, int UBB, bool NR>
__global__ __launch_bounds__(NR ? 1024 : 256) void pool_pair_kernel(PoolSide<T> A, PoolSide<T> Bs,
                                                                    int gridA, NormRope nr,
                                                                    AppendRows ap0, RowSide<T> RA,
                                                                    RowSide<T> RB, int gridAB, int B) {
  if constexpr (NR) {
    if ((int)blockIdx.x >= gridAB) {
      const int c = A.c, CV = c / VEC;
      const long long item = (long long)((int)blockIdx.x - gridAB) * blockDim.x + threadIdx.x;
      const long long row = item / CV, nra = (long long)B * RA.T_, nrows = nra + (long long)B * RB.T_;
      if (row >= nrows) return;  // whole rows leave together (CV divides 64)
      const int cv = (int)(item - row * CV);
      const bool sa = row < nra;
      const RowSide<T>& R = sa ? RA : RB;
      const long long r = sa ? row : row - nra;
      const int b = (int)(r / R.T_), t = (int)(r - (long long)b * R.T_);
      const long long p = (R.pos ? (long long)R.pos[b] : 0LL) + t;
      const NormRope nx{R.gamma, nr.eps, nr.theta, nr.d, 1};
      csahca::norm_rope_row8<T>(R.x + b * R.x_bs + (long long)t * c, R.y + b * R.y_bs + (long long)t * c, nx,
                                p, cv, CV, c);
      return;
    }
  }
  if ((int)blockIdx.x < gridA) {
    const NormRope na{A.gamma, nr.eps, nr.theta, nr.d, nr.norm};
    pool_items<T, UBA, false, PLAIN, NR>(A.X, A.Z, nullptr, nullptr, nullptr, A.out, A.N, A.c, A.m, 0,
                                         A.in_bs, A.out_bs, A.total, na, A.entry0, ap0, (int)blockIdx.x);
  } else {
    const NormRope nb{Bs.gamma, nr.eps, nr.theta, nr.d, nr.norm};
    pool_block<T, UBB, false, PLAIN, NR>(Bs.X, Bs.Z, nullptr, nullptr, nullptr, Bs.out, Bs.N, Bs.c,
                                         Bs.m, 0, Bs.S, Bs.CVG, Bs.in_bs, Bs.out_bs, nb, Bs.entry0, ap0,
                                         (int)blockIdx.x - gridA);
  }
}

// The norm's block path holds up to 1024 x 24 floats of partial states (96 KiB): raise
// the dynamic LDS limit of its kernels once per process (the attribute belongs to the
// kernel, for every device)
template <typename T, bool HAS_P, int MODE>
hipError_t raise_lds_limit() {
  static std::once_flag once;
  static hipError_t rc = hipSuccess;
  std::call_once(once, [] {
    rc = hipFuncSetAttribute((const void*)pool_block_kernel<T, 8, HAS_P, MODE, true>,
                             hipFuncAttributeMaxDynamicSharedMemorySize, 128 * 1024);
    if (rc == hipSuccess)
      rc = hipFuncSetAttribute((const void*)pool_block_kernel<T, 4, HAS_P, MODE, true>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, 128 * 1024);
  });
  return rc;
}

// the same for the paired launch with the norm (bf16)
hipError_t raise_pair_lds_limit() {
  using T = uint16_t;
  static std::once_flag once;
  static hipError_t rc = hipSuccess;
  std::call_once(once, [] {
    const void* k[4] = {(const void*)pool_pair_kernel<T, 8, 8, true>, (const void*)pool_pair_kernel<T, 8, 4, true>,
                        (const void*)pool_pair_kernel<T, 4, 8, true>, (const void*)pool_pair_kernel<T, 4, 4, true>};
    for (int i = 0; i < 4 && rc == hipSuccess; ++i)
      rc = hipFuncSetAttribute(k[i], hipFuncAttributeMaxDynamicSharedMemorySize, 128 * 1024);
  });
  return rc;
}

template <typename T, bool HAS_P, int MODE, bool NR>
int launch_pool(const void* kv, const void* gate, const void* kv_b, const void* gate_b,
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
    // norm the workgroup holds the whole entry (all CV slices, a whole number of waves, as
    // many threads as the form allows: a decode step pools one entry per sequence, so the
    // workgroups are few and each takes as many loads in flight as it can)
    int CVG = 8, smax, unit = 1;
    if (NR) {
      CVG = CV;
      smax = nr_block_threads<T, HAS_P, MODE>() / CV;
      unit = CV >= 64 ? 1 : 64 / CV;
    } else {
      while (CV % CVG != 0) CVG /= 2;
      smax = 256 / CVG;
    }
    const int span = max(4, cdiv(mt, smax));
    const int S = cdiv(cdiv(mt, span), unit) * unit;
    const size_t lds = ((size_t)S * CVG * 3 * VEC + (NR ? (size_t)c + 16 : 0)) * sizeof(float);
    const unsigned grid = (unsigned)(B * N * (CV / CVG)), threads = (unsigned)(S * CVG);
    if (NR && raise_lds_limit<T, HAS_P, MODE>() != hipSuccess)
      return csahca::fail(CSAHCA_ELAUNCH, "pooling: cannot raise the LDS limit");
    if (span % 8 == 0 && m % 8 == 0)
      hipLaunchKernelGGL((pool_block_kernel<T, 8, HAS_P, MODE, NR>), dim3(grid), dim3(threads), lds, st,
                         X, Z, Xb, Zb, pos_bias, (T*)out, (int)N, c, m, prev, S, CVG, in_bs, out_bs,
                         nr, entry0, ap);
    else
      hipLaunchKernelGGL((pool_block_kernel<T, 4, HAS_P, MODE, NR>), dim3(grid), dim3(threads), lds, st,
                         X, Z, Xb, Zb, pos_bias, (T*)out, (int)N, c, m, prev, S, CVG, in_bs, out_bs,
                         nr, entry0, ap);
    return CSAHCA_OK;
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
  return CSAHCA_OK;
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
int run_pool(const PoolArgs& a) {
  return launch_pool<T, HP, MODE, NR>(a.kv, a.gate, a.kv_b, a.gate_b, a.pos_bias, a.out, a.B, a.N, a.c,
                               a.m, a.prev, a.in_bs, a.out_bs, a.nr, a.entry0, a.ap, a.st);
}

template <typename T>
int pick_pool(const PoolArgs& a, bool hp, int mode, bool nr) {
  using F = int (*)(const PoolArgs&);
  static const F tab[12] = {
      run_pool<T, false, PLAIN, false>,      run_pool<T, false, PLAIN, true>,
      run_pool<T, false, TWO_STREAM, false>, run_pool<T, false, TWO_STREAM, true>,
      run_pool<T, false, APPEND, false>,     run_pool<T, false, APPEND, true>,
      run_pool<T, true, PLAIN, false>,       run_pool<T, true, PLAIN, true>,
      run_pool<T, true, TWO_STREAM, false>,  run_pool<T, true, TWO_STREAM, true>,
      run_pool<T, true, APPEND, false>,      run_pool<T, true, APPEND, true>};
  return tab[(hp ? 6 : 0) + 2 * mode + (nr ? 1 : 0)](a);
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
  const int lrc = dtype == CSAHCA_BF16
                      ? pick_pool<uint16_t>(a, pos_bias != nullptr, ov ? TWO_STREAM : PLAIN, nr != nullptr)
                      : pick_pool<float>(a, pos_bias != nullptr, ov ? TWO_STREAM : PLAIN, nr != nullptr);
  return lrc != CSAHCA_OK ? lrc : launch_status(name);
}

// Two poolings of one layer pair (csa_compress and hca_compress arguments; with nr, those
// of csahca_compress_norm_rope, each side with its own gain and first entry) in one
// launch when one takes pool_kernel's layout and the other pool_block_kernel's at the
// same workgroup size; otherwise one launch each.  The entries are the same bits either
// way.
int pair_rows_check(const char* name, const PairRows& r, int c) {
  const char* why = nullptr;
  const bool has_a = r.x_a || r.y_a, has_b = r.x_b || r.y_b;
  if (r.T < 0) why = "T must be >= 0";
  else if (r.T > 0 && ((has_a && (!r.x_a || !r.y_a)) || (has_b && (!r.x_b || !r.y_b))))
    why = "a side's row source and destination must both be set or both be NULL";
  else if (r.T > 0 && (!aligned16(r.x_a) || !aligned16(r.y_a) || !aligned16(r.x_b) || !aligned16(r.y_b)))
    why = "the row sources and destinations must be 16-byte aligned";
  else if (r.T > 0)
    for (int sd = 0; sd < 2; ++sd)
      if (sd == 0 ? has_a : has_b)
        for (long long bs : {sd == 0 ? r.x_bs_a : r.x_bs_b, sd == 0 ? r.y_bs_a : r.y_bs_b})
          if (bs < (long long)r.T * c || bs % 8) why = "row batch strides must be >= T*c and multiples of 8";
  if (!why) return CSAHCA_OK;
  set_error("%s: %s", name, why);
  return CSAHCA_EINVAL;
}

int pool_pair(const char* name, const void* kv_a, const void* gate_a, void* out_a, int n_a, int m_a,
              long long in_bs_a, long long out_bs_a, const void* kv_b, const void* gate_b, void* out_b,
              int n_b, int m_b, long long in_bs_b, long long out_bs_b, int B, int c, int dtype,
              const NormRope* nr, const float* gamma_a, long long entry0_a, const float* gamma_b,
              long long entry0_b, void* stream, const PairRows* rows) {
  long long NA = 0, NB = 0;
  int rc = pool_check(name, kv_a, gate_a, nullptr, nullptr, false, 0, out_a, B, n_a, c, m_a, dtype,
                      in_bs_a, out_bs_a, &NA);
  if (rc != CSAHCA_OK) return rc;
  rc = pool_check(name, kv_b, gate_b, nullptr, nullptr, false, 0, out_b, B, n_b, c, m_b, dtype, in_bs_b,
                  out_bs_b, &NB);
  if (rc != CSAHCA_OK) return rc;
  if (nr && (!norm_rope_args_ok(c, nr->d, nr->eps, nr->theta) || entry0_a < 0 || entry0_b < 0 ||
             !aligned16(gamma_a) || !aligned16(gamma_b))) {
    set_error("%s: the norm needs c / 8 a power of two <= 64, d_rope %% 8 == 0 and <= c, "
              "eps >= 0, theta > 0, entry0 >= 0 and gamma 16-byte aligned", name);
    return CSAHCA_EINVAL;
  }
  if (rows) {
    rc = pair_rows_check(name, *rows, c);
    if (rc != CSAHCA_OK) return rc;
  }
  const int nrow_t = rows ? rows->T : 0;  // rows per sequence and side
  hipStream_t st = (hipStream_t)stream;
  const PoolPlan pa = nr ? plan_norm(B, NA, c, m_a) : plan_plain(B, NA, c, m_a);
  const PoolPlan pb = nr ? plan_norm(B, NB, c, m_b) : plan_plain(B, NB, c, m_b);
  const unsigned wg = nr ? 1024u : 256u;
  const bool swap = pa.block && !pb.block;  // side 1 takes pool_kernel's layout
  const PoolPlan &p1 = swap ? pb : pa, &p2 = swap ? pa : pb;
  // (with the norm, bf16 only: the float form does not fit 1024-thread workgroups)
  if ((NA > 0 || NB > 0) && !p1.block && p2.block && p2.threads == wg && (!nr || dtype == CSAHCA_BF16) &&
      (long long)p1.grid + p2.grid + cdiv<long long>(2LL * B * nrow_t * (c / 8), wg) <= 0x7FFFFFFFLL) {
    if (nr && raise_pair_lds_limit() != hipSuccess)
      return fail(CSAHCA_ELAUNCH, "csahca_compress_pair: cannot raise the LDS limit");
    const NormRope n0 = nr ? *nr : NormRope{nullptr, 0.f, 1.f, 0, 0};
    const AppendRows ap0{nullptr, nullptr, 1, 0, 0, 0};
    auto go = [&](auto tag, auto nrtag) {
      using T = decltype(tag);
      constexpr bool NR = decltype(nrtag)::value;
      const PoolSide<T> sa{(const T*)kv_a, (const T*)gate_a, (T*)out_a, (int)NA, c, m_a,
                           pa.S, pa.CVG, in_bs_a, out_bs_a, pa.total, gamma_a, entry0_a};
      const PoolSide<T> sb{(const T*)kv_b, (const T*)gate_b, (T*)out_b, (int)NB, c, m_b,
                           pb.S, pb.CVG, in_bs_b, out_bs_b, pb.total, gamma_b, entry0_b};
      const PoolSide<T>& s1 = swap ? sb : sa;
      const PoolSide<T>& s2 = swap ? sa : sb;
      RowSide<T> ra{}, rb{};
      long long grid_rows = 0;
      if (NR && nrow_t > 0) {  // a side without rows gets T = 0
        const int ta = rows->x_a ? nrow_t : 0, tb = rows->x_b ? nrow_t : 0;
        ra = RowSide<T>{(const T*)rows->x_a, (T*)rows->y_a, rows->pos_a, rows->x_bs_a, rows->y_bs_a, gamma_a,
                        ta};
        rb = RowSide<T>{(const T*)rows->x_b, (T*)rows->y_b, rows->pos_b, rows->x_bs_b, rows->y_bs_b, gamma_b,
                        tb};
        grid_rows = cdiv<long long>((long long)B * (ta + tb) * (c / 8), wg);
      }
      const int g1 = (int)p1.grid, g12 = (int)(p1.grid + p2.grid);
      const dim3 grid((unsigned)(g12 + grid_rows)), blk(wg);
      if (p1.ub == 8 && p2.ub == 8)
        hipLaunchKernelGGL((pool_pair_kernel<T, 8, 8, NR>), grid, blk, p2.lds, st, s1, s2, g1, n0, ap0, ra, rb, g12, B);
      else if (p1.ub == 8)
        hipLaunchKernelGGL((pool_pair_kernel<T, 8, 4, NR>), grid, blk, p2.lds, st, s1, s2, g1, n0, ap0, ra, rb, g12, B);
      else if (p2.ub == 8)
        hipLaunchKernelGGL((pool_pair_kernel<T, 4, 8, NR>), grid, blk, p2.lds, st, s1, s2, g1, n0, ap0, ra, rb, g12, B);
      else
        hipLaunchKernelGGL((pool_pair_kernel<T, 4, 4, NR>), grid, blk, p2.lds, st, s1, s2, g1, n0, ap0, ra, rb, g12, B);
    };
    if (nr)
      go(uint16_t{}, std::true_type{});
    else if (dtype == CSAHCA_BF16)
      go(uint16_t{}, std::false_type{});
    else
      go(float{}, std::false_type{});
    return launch_status(name);
  }
  NormRope na{}, nb{};
  if (nr) {
    na = NormRope{gamma_a, nr->eps, nr->theta, nr->d, nr->norm};
    nb = NormRope{gamma_b, nr->eps, nr->theta, nr->d, nr->norm};
  }
  if (NA > 0) {
    rc = pool_entry(name, kv_a, gate_a, nullptr, nullptr, false, 0, nullptr, out_a, B, n_a, c, m_a, dtype,
                    in_bs_a, out_bs_a, stream, nr ? &na : nullptr, entry0_a);
    if (rc != CSAHCA_OK) return rc;
  }
  if (NB > 0) {
    rc = pool_entry(name, kv_b, gate_b, nullptr, nullptr, false, 0, nullptr, out_b, B, n_b, c, m_b, dtype,
                    in_bs_b, out_bs_b, stream, nr ? &nb : nullptr, entry0_b);
    if (rc != CSAHCA_OK) return rc;
  }
  if (nr && nrow_t > 0) {  // the rows in launches of their own
    if (rows->x_a) {
      rc = csahca_norm_rope(rows->x_a, rows->y_a, gamma_a, rows->pos_a, B, nrow_t, 1, c, 1, nr->d, nr->eps,
                            nr->theta, 1, dtype, rows->x_bs_a, rows->y_bs_a, stream);
      if (rc != CSAHCA_OK) return rc;
    }
    if (rows->x_b)
      return csahca_norm_rope(rows->x_b, rows->y_b, gamma_b, rows->pos_b, B, nrow_t, 1, c, 1, nr->d, nr->eps,
                              nr->theta, 1, dtype, rows->x_bs_b, rows->y_bs_b, stream);
  }
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
  const int lrc = dtype == CSAHCA_BF16 ? pick_pool<uint16_t>(a, pos_bias != nullptr, APPEND, false)
                                      : pick_pool<float>(a, pos_bias != nullptr, APPEND, false);
  return lrc != CSAHCA_OK ? lrc : launch_status(name);
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
  return csahca::pool_pair("csahca_compress_pair", kv_a, gate_a, out_a, n_a, m_a, in_bstride_a, out_bstride_a,
                           kv_b, gate_b, out_b, n_b, m_b, in_bstride_b, out_bstride_b, B, c, dtype, nullptr,
                           nullptr, 0, nullptr, 0, stream);
}

extern "C" int csahca_compress_pair_norm_rope(const void* kv_a, const void* gate_a, const float* gamma_a,
                                              void* out_a, int n_a, int m_a, long long entry0_a,
                                              long long in_bstride_a, long long out_bstride_a,
                                              const void* kv_b, const void* gate_b, const float* gamma_b,
                                              void* out_b, int n_b, int m_b, long long entry0_b,
                                              long long in_bstride_b, long long out_bstride_b, int B,
                                              int c, int d_rope, float eps, float theta, int dtype,
                                              void* stream) {
  const NormRope nr{nullptr, eps, theta, d_rope, 1};
  return csahca::pool_pair("csahca_compress_pair_norm_rope", kv_a, gate_a, out_a, n_a, m_a, in_bstride_a,
                           out_bstride_a, kv_b, gate_b, out_b, n_b, m_b, in_bstride_b, out_bstride_b, B, c,
                           dtype, &nr, gamma_a, entry0_a, gamma_b, entry0_b, stream);
}

extern "C" int csahca_compress_pair_norm_rope_rows(
    const void* kv_a, const void* gate_a, const float* gamma_a, void* out_a, int n_a, int m_a, long long entry0_a,
    long long in_bstride_a, long long out_bstride_a, const void* kv_b, const void* gate_b, const float* gamma_b,
    void* out_b, int n_b, int m_b, long long entry0_b, long long in_bstride_b, long long out_bstride_b, int B,
    int c, int d_rope, float eps, float theta, int dtype, int T, const void* row_x_a, void* row_y_a,
    const int* row_pos_a, long long row_x_bstride_a, long long row_y_bstride_a, const void* row_x_b,
    void* row_y_b, const int* row_pos_b, long long row_x_bstride_b, long long row_y_bstride_b, void* stream) {
  const NormRope nr{nullptr, eps, theta, d_rope, 1};
  const csahca::PairRows rows{T, row_x_a, row_x_b, row_y_a, row_y_b, row_pos_a, row_pos_b,
                              row_x_bstride_a, row_y_bstride_a, row_x_bstride_b, row_y_bstride_b};
  return csahca::pool_pair("csahca_compress_pair_norm_rope_rows", kv_a, gate_a, out_a, n_a, m_a, in_bstride_a,
                           out_bstride_a, kv_b, gate_b, out_b, n_b, m_b, in_bstride_b, out_bstride_b, B, c,
                           dtype, &nr, gamma_a, entry0_a, gamma_b, entry0_b, stream, &rows);
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
