// Pooling launcher shared by the compress entry points and the KV-cache append.
#pragma once

#include "common.hpp"

namespace csahca {

// Validates, then enqueues softmax-gated pooling of whole blocks (see csa_compress and
// csa_compress_overlap in csahca.h for the arguments; `ov` selects the two-stream form,
// `prev` its one-block look-back).  Returns a CSAHCA_* status; `name` prefixes errors.
int pool_entry(const char* name, const void* kv, const void* gate, const void* kv_b,
               const void* gate_b, bool ov, int prev, const float* pos_bias, void* out, int B,
               int n, int c, int m, int dtype, long long in_bs, long long out_bs, void* stream);

}  // namespace csahca
