// Shared definitions of the lightning-indexer kernels (scoring and exact top-k): the
// group size of the selection keys, the limits, the visibility rule, the launch plan of
// the decode scoring kernel and the workspace layout.  See index_score.hip,
// fused_topk.hpp and topk_select.hip.
#pragma once

#include "common.hpp"
#include "normrope.hpp"

namespace csahca {

constexpr int GROUP = 16;           // keys per group maximum
constexpr int SEL_THREADS = 1024;   // selection workgroup
constexpr int KPT = 16;                              // selection keys per thread (registers)
constexpr int SEL_MAX_KEYS = SEL_THREADS * KPT;      // 16384 group maxima per query
constexpr int MAX_NC = GROUP * SEL_MAX_KEYS;
constexpr int MAX_K = 1024;

constexpr int SCORE_WGS = 512;      // decode scoring workgroups to aim for (about two per CU)
constexpr int SCORE_STAGE = 4096;   // keys per decode workgroup (LDS-staged scores)

// Decode: every scoring workgroup lists the best entries of its chunk (fused_topk.hpp),
// and the selection kernel first selects from the union of a query's lists.
constexpr int FT_MAX_P = 128;                        // chunks per query
constexpr int FT_MAX_SLOTS = SEL_THREADS * KPT;      // chunks x list capacity per query

// how a query's selection went (the workspace's last words after a decode call)
constexpr uint32_t FT_PATH_LISTS = 1;   // the union of the chunk lists held the top k
constexpr uint32_t FT_PATH_GROUPS = 2;  // selected through the group maxima and scores
constexpr uint32_t FT_PATH_ALL = 3;     // k >= the usable entries: every one selected
// written to a query's word by the scoring launch that wrote its chunk lists, so that the
// selection launch (also through lightning_index_select) takes the lists only after them
constexpr uint32_t FT_LISTS_READY = 0x4C157EADu;

// number of usable entries for query t of sequence b: block s is usable iff
// m*(s+1) - 1 <= p, i.e. s < (p+1)/m
CSAHCA_DEV int visible_entries(const int* q_pos, int b, int t, int m, int N_c) {
  const long long p = (long long)q_pos[b] + t;
  long long v = (p + 1) / m;
  if (p + 1 <= 0) v = 0;
  return (int)(v < N_c ? v : N_c);
}

// Launch plan of the decode scoring kernel and its chunk lists.  P chunks of CH keys per
// query; a chunk lists between JT and JMAX of its best entries (every one when it holds at
// most JMAX).  JT is about the chunk's expected share of the top k plus four standard
// deviations (the kernel recomputes it from the query's usable entries), so that the union
// of the lists holds the whole top k unless the best entries cluster in a few chunks.
struct TopkPlan {
  bool lists;
  int P, CH, JT, JMAX;
};

inline int pow2_ceil(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

inline TopkPlan topk_plan_decode(long long nq, int N_c, int k) {
  TopkPlan T;
  int chunks = (int)cdiv<long long>(SCORE_WGS, nq);
  chunks = chunks < FT_MAX_P ? chunks : FT_MAX_P;
  const int lo = cdiv(N_c, SCORE_STAGE), hi = cdiv(N_c, 256);
  chunks = chunks < hi ? chunks : hi;
  const int keff = k < N_c ? k : N_c;
  for (;;) {
    chunks = chunks > lo ? chunks : lo;
    chunks = chunks > 1 ? chunks : 1;
    T.CH = cdiv(cdiv(N_c, chunks), 64) * 64;
    T.P = cdiv(N_c, T.CH);
    const double per = (double)keff / T.P;
    T.JT = (int)(per + 4.0 * __builtin_sqrt(per) + 8.0) + 1;
    const int cap = pow2_ceil(T.CH);
    T.JMAX = pow2_ceil(T.JT + T.JT / 2);
    T.JMAX = T.JMAX < cap ? T.JMAX : cap;
    if (T.JT > T.JMAX) T.JT = T.JMAX;
    // fewer, longer chunks until the lists of a query fit the selection's registers
    if ((long long)T.P * T.JMAX <= FT_MAX_SLOTS || chunks <= lo) break;
    chunks /= 2;
  }
  T.lists = T.P <= FT_MAX_P && (long long)T.P * T.JMAX <= FT_MAX_SLOTS;
  return T;
}

// Workspace: the maximum score key (score_key) of every group of GROUP entries, the fp32
// scores (used when the caller passes no all_scores buffer), then for a decode selection
// from chunk lists, per query and chunk the bound and the listed keys (zero-padded), and
// last, one word per query naming the way its selection went (FT_PATH_*).
struct WsLayout {
  size_t gkeys_off, gkeys_bytes, scores_off, scores_bytes;
  size_t edge_off, cand_off, path_off;
  TopkPlan plan;
  size_t total;
};

inline WsLayout ws_layout(long long nq, int N_c, int k, bool decode) {
  WsLayout L;
  const long long NG = cdiv<long long>(N_c, GROUP);
  L.gkeys_off = 0;
  L.gkeys_bytes = align_up((size_t)(nq * NG * 4), 256);
  L.scores_off = L.gkeys_off + L.gkeys_bytes;
  L.scores_bytes = align_up((size_t)(nq * (long long)N_c * 4), 256);
  L.total = L.scores_off + L.scores_bytes;
  L.plan = decode ? topk_plan_decode(nq, N_c, k) : TopkPlan{false, 0, 0, 0, 0};
  L.edge_off = L.cand_off = L.path_off = L.total;
  if (L.plan.lists) {
    L.edge_off = L.total;
    L.cand_off = L.edge_off + align_up((size_t)nq * FT_MAX_P * 8, 256);
    L.path_off = L.cand_off + align_up((size_t)nq * L.plan.P * L.plan.JMAX * 8, 256);
    L.total = L.path_off + align_up((size_t)nq * 4, 256);
  }
  return L;
}

// the chunk lists of a decode selection
struct ChunkLists {
  uint64_t* edge;  // [nq][FT_MAX_P] every unlisted entry of the chunk has a smaller key
  uint64_t* cand;  // [nq][P][JMAX] listed keys in index order, then zeros
  uint32_t* path;  // [nq] FT_LISTS_READY once the lists are written, then FT_PATH_*
  int k, P, JMAX, CH;  // top-k size; the plan's list layout and chunk length
};

// argument checks shared by lightning_index_score and lightning_index_topk
int index_check_common(const void* q_idx, const float* w_idx, const void* k_idx, int idx_dtype,
                       const int* q_pos, int m, int B, int Tq, int n_ih, int c_I, int N_c, int k);

// the chunk lists of a workspace laid out by ws_layout (all fields null without them)
ChunkLists chunk_lists_of(char* ws, const WsLayout& L, int k);

// whether index_score_impl can write chunk lists for these arguments
bool index_can_list(int idx_dtype, int Tq, int c_I, int n_ih, const TopkPlan& plan);

// enqueue the scoring kernel: scores [B*Tq, N_c] and group maxima [B*Tq, ceil(N_c/16)];
// with lists (decode, c_I = 128 FP8 or MX FP4 keys, a plan with lists) every chunk also
// writes its list
int index_score_impl(const void* q_idx, const float* w_idx, const void* k_idx, int idx_dtype,
                     const int* q_pos, int m, int B, int Tq, int n_ih, int c_I, int N_c,
                     float* scores, uint32_t* gkeys, hipStream_t st,
                     const ChunkLists* lists = nullptr);

// A decode step's new CSA block(s) to pool in the selection launch (bfloat16, no bias,
// m < 8: the one-thread-per-(sequence, entry, 8-channel slice) layout of csa_compress);
// total = B * N * (c / 8) items, N entries per sequence, in the first pool_wgs extra
// workgroups.  With norm, every entry is then normalised and rotated (nr, the first one
// being entry entry0 of the cache), and the workgroups after those normalise rT window
// rows per sequence (row (b, t) at rx + b * rx_bs + t * c, position rpos[b] + t, written
// to ry likewise; nr's gain), one row per c / 8 consecutive lanes: rows = B * rT.
struct PoolBeside {
  const uint16_t* X;
  const uint16_t* Z;
  uint16_t* out;
  int N, c, m;
  long long in_bs, out_bs, total;
  int norm;
  NormRope nr;
  long long entry0;
  int pool_wgs;
  const uint16_t* rx;
  uint16_t* ry;
  const int* rpos;
  long long rx_bs, ry_bs;
  int rT;
  long long rows;
};

// enqueue the selection kernel over scores and group maxima written by index_score_impl
// (and, with lists, the chunk lists, which it tries first).  With `pool` the selection
// launch also pools those blocks when it is the list selection (*pooled set to true);
// otherwise *pooled is false and the caller pools them itself.
int index_select_impl(const float* scores, const uint32_t* gkeys, const int* q_pos, int m,
                      int B, int Tq, int N_c, int k, int* topk_idx, float* topk_score,
                      hipStream_t st, const ChunkLists* lists = nullptr,
                      const PoolBeside* pool = nullptr, bool* pooled = nullptr);

}  // namespace csahca
