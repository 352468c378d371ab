// KV-cache lifecycle of one layer: appending raw tokens, pooling the blocks they complete,
// keeping the exact recent window, forking a request at a shared prefix.
//
// Source: "DeepSeek-V4 Architecture From Kernels ... C-Kernel-Engine", section 9
// (heterogeneous KV cache: per request the recent window, compressed entries one per m
// tokens, and the uncompressed tail of an incomplete block; an entry is created whenever
// a block completes, the last W tokens stay exact, tails are kept across prefix hits).
//
// Layout: the raw tokens (values and gate logits) of a sequence live in a ring of
// R = m * ceil((W + m - 1) / m) rows, each token written twice, at row p mod R and
// p mod R + R.  R holds the window and any tail, a block never wraps (R is a multiple of
// m and blocks start at multiples of m), and any R consecutive positions are R contiguous
// rows of the doubled ring, so the attention call reads its window straight from it.
#include "pool.hpp"

namespace {

// Rows [n0, n0 + n) of the new tokens (source rows s0 .. s0 + n - 1) to ring rows
// (p mod R) and (p mod R) + R, p = p0 + s; values and gate logits; 16 bytes per thread.
__global__ __launch_bounds__(256) void ring_store(const uint8_t* __restrict__ kv, const uint8_t* __restrict__ gate,
                                                  uint8_t* __restrict__ kv_ring, uint8_t* __restrict__ gate_ring,
                                                  int s0, int n, long long p0, int R, int row_bytes,
                                                  long long src_bs, long long ring_bs, long long total) {
  const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= total) return;
  const int vec = row_bytes / 16;
  const long long rest = t / vec;
  const int v = (int)(t - rest * vec);
  const int j = (int)(rest % n);
  const int b = (int)(rest / n);
  const long long p = p0 + s0 + j;
  const int slot = (int)(p % R);
  const long long src = b * src_bs + (long long)(s0 + j) * row_bytes + v * 16;
  const long long d0 = b * ring_bs + (long long)slot * row_bytes + v * 16;
  const long long d1 = d0 + (long long)R * row_bytes;
  const u32x4 xv = *reinterpret_cast<const u32x4*>(kv + src);
  const u32x4 zv = *reinterpret_cast<const u32x4*>(gate + src);
  *reinterpret_cast<u32x4*>(kv_ring + d0) = xv;
  *reinterpret_cast<u32x4*>(kv_ring + d1) = xv;
  *reinterpret_cast<u32x4*>(gate_ring + d0) = zv;
  *reinterpret_cast<u32x4*>(gate_ring + d1) = zv;
}

int store_rows(const void* kv, const void* gate, void* kv_ring, void* gate_ring, int B, int s0,
               int n, long long p0, int R, int row_bytes, long long src_bs, long long ring_bs,
               hipStream_t st) {
  if (n <= 0) return CSAHCA_OK;
  const long long total = (long long)B * n * (row_bytes / 16);
  hipLaunchKernelGGL(ring_store, dim3((unsigned)cdiv<long long>(total, 256)), dim3(256), 0, st,
                     (const uint8_t*)kv, (const uint8_t*)gate, (uint8_t*)kv_ring, (uint8_t*)gate_ring, s0, n,
                     p0, R, row_bytes, src_bs, ring_bs, total);
  return csahca::launch_status("csahca_kv_append");
}

int elem_bytes(int dtype) { return dtype == CSAHCA_BF16 ? 2 : 4; }

}  // namespace

extern "C" int csahca_kv_ring_rows(int W, int m) {
  if (W < 0 || m < 1) return 0;
  return m * ((W + m - 1 + m - 1) / m);
}

extern "C" int csahca_kv_append(void* kv_ring, void* gate_ring, void* entries, const void* kv_new,
                                const void* gate_new, const float* pos_bias, int B, long long n_old,
                                int n_new, int c, int m, int W, int dtype, long long new_bstride,
                                long long ring_bstride, long long ent_bstride, void* stream) {
  using namespace csahca;
  const char* name = "csahca_kv_append";
  if (B < 1 || n_old < 0 || n_new < 0 || c < 8 || c % 8 != 0 || m < 1 || m > 4096 || W < 0)
    return fail(CSAHCA_EINVAL, "csahca_kv_append: need B >= 1, n_old >= 0, n_new >= 0, c % 8 == 0, 1 <= m <= 4096, W >= 0");
  if (dtype != CSAHCA_F32 && dtype != CSAHCA_BF16)
    return fail(CSAHCA_ENOTSUP, "csahca_kv_append: dtype must be CSAHCA_F32 or CSAHCA_BF16");
  if (n_new == 0) {
    clear_error();
    return CSAHCA_OK;
  }
  const int R = csahca_kv_ring_rows(W, m);
  if (!kv_ring || !gate_ring || !kv_new || !gate_new)
    return fail(CSAHCA_EINVAL, "csahca_kv_append: ring and new-token pointers must be non-NULL");
  const long long first = n_old / m, last = (n_old + n_new) / m;  // entries [first, last) are made
  if (last > first && !entries)
    return fail(CSAHCA_EINVAL, "csahca_kv_append: entries must be non-NULL when a block completes");
  if (new_bstride < (long long)n_new * c || ring_bstride < 2LL * R * c || ent_bstride < last * c)
    return fail(CSAHCA_EINVAL, "csahca_kv_append: strides below n_new*c, 2*R*c or (entries made)*c");
  if (new_bstride % 8 || ring_bstride % 8 || ent_bstride % 8)
    return fail(CSAHCA_EINVAL, "csahca_kv_append: strides must be multiples of 8 elements");
  if (!aligned16(kv_ring) || !aligned16(gate_ring) || !aligned16(kv_new) || !aligned16(gate_new) ||
      (entries && !aligned16(entries)))
    return fail(CSAHCA_EINVAL, "csahca_kv_append: pointers must be 16-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  const int e = elem_bytes(dtype), rb = c * e;
  const long long nbs = new_bstride * e, rbs = ring_bstride * e;
  const int t = (int)(n_old % m);
  const int keep = n_new < R ? n_new : R;  // the last tokens, kept for the window and tail
  // With room for the old tail and all new tokens (decode, short chunks), the pooling
  // launch also stores the new tokens of the blocks it completes (it overwrites no ring
  // row it reads), and the new tail is stored beside it; otherwise the last tokens are
  // stored after the pooling, which may have read the rows they replace.
  const bool early = n_new + t <= R;
  int rc = pool_append(name, kv_new, gate_new, kv_ring, gate_ring, R, n_old, early, pos_bias, entries, B,
                       first, last - first, c, m, dtype, new_bstride, ring_bstride, ent_bstride, stream);
  if (rc) return rc;
  if (early) {  // tokens past the last completed block (all of them when none completes)
    const long long s0 = last * m > n_old ? last * m - n_old : 0;
    return store_rows(kv_new, gate_new, kv_ring, gate_ring, B, (int)s0, n_new - (int)s0, n_old, R, rb, nbs,
                      rbs, st);
  }
  return store_rows(kv_new, gate_new, kv_ring, gate_ring, B, n_new - keep, keep, n_old, R, rb, nbs, rbs, st);
}

extern "C" int csahca_kv_fork(void* dst_kv_ring, void* dst_gate_ring, void* dst_entries,
                              const void* src_kv_ring, const void* src_gate_ring,
                              const void* src_entries, int B, long long n_entries, int c, int m,
                              int W, int dtype, long long ring_bstride, long long ent_bstride,
                              void* stream) {
  using namespace csahca;
  if (B < 1 || n_entries < 0 || c < 8 || c % 8 != 0 || m < 1 || m > 4096 || W < 0)
    return fail(CSAHCA_EINVAL, "csahca_kv_fork: need B >= 1, n_entries >= 0, c % 8 == 0, 1 <= m <= 4096, W >= 0");
  if (dtype != CSAHCA_F32 && dtype != CSAHCA_BF16)
    return fail(CSAHCA_ENOTSUP, "csahca_kv_fork: dtype must be CSAHCA_F32 or CSAHCA_BF16");
  const int R = csahca_kv_ring_rows(W, m);
  if (!dst_kv_ring || !dst_gate_ring || !src_kv_ring || !src_gate_ring ||
      (n_entries > 0 && (!dst_entries || !src_entries)))
    return fail(CSAHCA_EINVAL, "csahca_kv_fork: ring pointers (and entries when n_entries > 0) must be non-NULL");
  if (ring_bstride < 2LL * R * c || (n_entries > 0 && ent_bstride < n_entries * c))
    return fail(CSAHCA_EINVAL, "csahca_kv_fork: ring_bstride below 2*R*c or ent_bstride below n_entries*c");
  const size_t e = (size_t)elem_bytes(dtype);
  const size_t width = 2 * (size_t)R * c * e, pitch = (size_t)ring_bstride * e;
  hipStream_t st = (hipStream_t)stream;
  if (width > 0 &&  // m = 1 with no window keeps no raw tokens
      (hipMemcpy2DAsync(dst_kv_ring, pitch, src_kv_ring, pitch, width, B, hipMemcpyDeviceToDevice, st) != hipSuccess ||
       hipMemcpy2DAsync(dst_gate_ring, pitch, src_gate_ring, pitch, width, B, hipMemcpyDeviceToDevice, st) != hipSuccess))
    return fail(CSAHCA_ELAUNCH, "csahca_kv_fork: ring copy failed");
  if (n_entries > 0) {
    const size_t ew = (size_t)n_entries * c * e, ep = (size_t)ent_bstride * e;
    if (hipMemcpy2DAsync(dst_entries, ep, src_entries, ep, ew, B, hipMemcpyDeviceToDevice, st) != hipSuccess)
      return fail(CSAHCA_ELAUNCH, "csahca_kv_fork: entry copy failed");
  }
  clear_error();
  return CSAHCA_OK;
}
