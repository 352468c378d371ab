// Pooling launcher shared by the compress entry points and the KV-cache append.
#pragma once

#include "common.hpp"
#include "normrope.hpp"

namespace csahca {

// Validates, then enqueues softmax-gated pooling of whole blocks (see csa_compress and
// csa_compress_overlap in csahca.h for the arguments; `ov` selects the two-stream form,
// `prev` its one-block look-back).  With `nr` non-NULL every entry is then normalised and
// rotated (csahca_compress_norm_rope), the first emitted entry being entry `entry0` of the
// cache.  Returns a CSAHCA_* status; `name` prefixes errors.
int pool_entry(const char* name, const void* kv, const void* gate, const void* kv_b,
               const void* gate_b, bool ov, int prev, const float* pos_bias, void* out, int B,
               int n, int c, int m, int dtype, long long in_bs, long long out_bs, void* stream,
               const NormRope* nr = nullptr, long long entry0 = 0);

// Host-side validation of a pooling call (csa_compress's rules; `ov`/`prev` the two-stream
// form): *N_out receives the number of entries per sequence the call emits.
int pool_check(const char* name, const void* kv, const void* gate, const void* kv_b,
               const void* gate_b, bool ov, int prev, void* out, int B, int n, int c, int m,
               int dtype, long long in_bs, long long out_bs, long long* N_out);

// Window rows normalised beside a paired pooling with the norm (csahca_norm_rope's
// arguments for one side, H = 1, pstride 1): none when T == 0.
struct PairRows {
  int T;
  const void *x_a, *x_b;
  void *y_a, *y_b;
  const int *pos_a, *pos_b;
  long long x_bs_a, y_bs_a, x_bs_b, y_bs_b;
};

// Host-side validation of the rows; a side's rows are skipped when both its pointers are
// NULL.
int pair_rows_check(const char* name, const PairRows& r, int c);

// Two poolings of one layer pair (csahca_compress_pair and, with nr, its norm forms; with
// rows, csahca_compress_pair_norm_rope_rows).  A side with n = 0 pools nothing.
int pool_pair(const char* name, const void* kv_a, const void* gate_a, void* out_a, int n_a, int m_a,
              long long in_bs_a, long long out_bs_a, const void* kv_b, const void* gate_b, void* out_b,
              int n_b, int m_b, long long in_bs_b, long long out_bs_b, int B, int c, int dtype,
              const NormRope* nr, const float* gamma_a, long long entry0_a, const float* gamma_b,
              long long entry0_b, void* stream, const PairRows* rows = nullptr);

// Pools the `count` entries first .. first+count-1 that an append of tokens n_old .. to B
// sequences completes, in one launch: rows before n_old come from the doubled rings
// (R rows, batch stride ring_bs), the others from the new tokens (batch stride new_bs).
// With `store` the new tokens read are also written to the rings (the caller guarantees
// that this overwrites no ring row read here).  Arguments are validated by the caller.
int pool_append(const char* name, const void* kv_new, const void* gate_new, const void* ring_x,
                const void* ring_z, int R, long long n_old, bool store, const float* pos_bias,
                void* entries, int B, long long first, long long count, int c, int m, int dtype,
                long long new_bs, long long ring_bs, long long ent_bs, void* stream);

}  // namespace csahca
