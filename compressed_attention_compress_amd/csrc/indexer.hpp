// Shared definitions of the lightning-indexer kernels (scoring and exact top-k): the
// group size of the selection keys, the limits, the visibility rule and the workspace
// layout.  See index_score.hip and topk_select.hip.
#pragma once

#include "common.hpp"

namespace csahca {

constexpr int GROUP = 16;           // keys per group maximum
constexpr int SEL_THREADS = 1024;
constexpr int KPT = 16;                              // selection keys per thread (registers)
constexpr int SEL_MAX_KEYS = SEL_THREADS * KPT;      // 16384 group maxima per query
constexpr int MAX_NC = GROUP * SEL_MAX_KEYS;
constexpr int MAX_K = SEL_THREADS;                   // one candidate group per thread
static_assert(KPT == GROUP, "a thread scans exactly one candidate group");

// number of usable entries for query t of sequence b: block s is usable iff
// m*(s+1) - 1 <= p, i.e. s < (p+1)/m
CSAHCA_DEV int visible_entries(const int* q_pos, int b, int t, int m, int N_c) {
  const long long p = (long long)q_pos[b] + t;
  long long v = (p + 1) / m;
  if (p + 1 <= 0) v = 0;
  return (int)(v < N_c ? v : N_c);
}

// Workspace: the maximum score key (score_key) of every group of GROUP entries, then the
// fp32 scores (used when the caller passes no all_scores buffer).
struct WsLayout {
  size_t gkeys_off, gkeys_bytes, scores_off, scores_bytes, total;
};

inline WsLayout ws_layout(long long nq, int N_c) {
  WsLayout L;
  const long long NG = cdiv<long long>(N_c, GROUP);
  L.gkeys_off = 0;
  L.gkeys_bytes = align_up((size_t)(nq * NG * 4), 256);
  L.scores_off = L.gkeys_bytes;
  L.scores_bytes = align_up((size_t)(nq * (long long)N_c * 4), 256);
  L.total = L.scores_off + L.scores_bytes;
  return L;
}

// argument checks shared by lightning_index_score and lightning_index_topk
int index_check_common(const void* q_idx, const float* w_idx, const void* k_idx, int idx_dtype,
                       const int* q_pos, int m, int B, int Tq, int n_ih, int c_I, int N_c, int k);

// enqueue the scoring kernel: scores [B*Tq, N_c] and group maxima [B*Tq, ceil(N_c/16)]
int index_score_impl(const void* q_idx, const float* w_idx, const void* k_idx, int idx_dtype,
                     const int* q_pos, int m, int B, int Tq, int n_ih, int c_I, int N_c,
                     float* scores, uint32_t* gkeys, hipStream_t st);

// enqueue the selection kernel over scores and group maxima written by index_score_impl
int index_select_impl(const float* scores, const uint32_t* gkeys, const int* q_pos, int m,
                      int B, int Tq, int N_c, int k, int* topk_idx, float* topk_score,
                      hipStream_t st);

}  // namespace csahca
