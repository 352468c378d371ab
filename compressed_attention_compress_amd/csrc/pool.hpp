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

}  // namespace csahca
