/*
 * csahca.h -- C ABI of the MI355X (gfx950) compressed-attention library (libcsahca.so).
 *
 * DeepSeek-V4 compressed attention as the pages describe it:
 *   CSA  (Compressed Sparse Attention): pool every m raw KV tokens into one entry with
 *        softmax-gated weights, score every usable entry with the lightning indexer, keep
 *        the top-k, and run multi-query attention over them plus a sliding window of raw
 *        tokens.
 *   HCA  (Heavily Compressed Attention): pool every m' tokens and attend to every usable
 *        entry plus the same window.
 * Sources, cited by page and section:
 *   "DeepSeek-V4 Hybrid Attention: CSA, HCA, mHC, MoE" (trishampatil.com): section IV,
 *     V.1 (compression), V.2 (lightning indexer, equation I_{t,s}), V.3 (core attention),
 *     VI (HCA, equation o_{t,i}).
 *   "DeepSeek-V4: Anatomy of an Open-Source Frontier Model" (modernaiengineering.com
 *     lesson 6.7): "Hybrid attention with CSA and HCA", "One query in a CSA layer, step by
 *     step", "Worked example, step by step".
 *   "DeepSeek-V4 Architecture From Kernels ... C-Kernel-Engine" (shivasnotes.com):
 *     section 6 (CSA attention reference contract: index input, explicit scale), section 9
 *     (heterogeneous KV cache: compressed entries, tails, window, indexer cache).
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller, row-major and
 *     contiguous in the shapes given, 16-byte aligned.  The library never allocates,
 *     frees or synchronises; every kernel is enqueued on `stream` (a hipStream_t, NULL =
 *     the default stream) in call order.
 *   - Scratch memory is a caller-owned device `workspace` of at least the size that the
 *     matching *_workspace_size() returns for the same shape arguments.
 *   - Every argument is validated on the host before anything is enqueued.  On error the
 *     call returns a negative status, enqueues nothing and records a message readable
 *     with csahca_last_error().  Values stored in device memory (positions, indices) are
 *     not inspected on the host; their documented ranges are the caller's contract, and
 *     the kernels never read outside the buffers whatever those values are.
 *   - Positions: q_pos[b] (device int32) is the absolute position of query token 0 of
 *     sequence b; query token t sits at p = q_pos[b] + t.  Compressed entry s of a cache
 *     with block size m covers raw positions m*s .. m*s+m-1 and is usable by p iff
 *     m*(s+1)-1 <= p (the block is complete) and s < the cache length.
 *   - The sliding window of the query at p is raw positions max(0, p-W+1) .. p (the query's
 *     own token included).  Window rows come from win_kv [B, L, c], whose row 0 is raw
 *     position win_pos[b]; positions outside win_pos[b] .. win_pos[b]+L-1 are skipped.
 *   - Scores, softmax and accumulation are float32 on the GPU.  bfloat16 results are
 *     rounded to nearest even.
 */
#ifndef CSAHCA_H
#define CSAHCA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types */
#define CSAHCA_F32 0
#define CSAHCA_BF16 1
#define CSAHCA_FP8_E4M3FN 2 /* OCP FP8: 4 exponent bits (bias 7), 3 mantissa bits, no inf */
/* Indexer keys in OCP MX FP4 (E2M1 elements: 2 exponent bits, bias 1, 1 mantissa bit;
 * two per byte, the first in the low nibble; one E8M0 scale byte 2^(s-127) per 32
 * elements) with FP8 E4M3FN queries (unit scale).  Key layout: all rows
 * [B, N_c, c_I/2] bytes, then all scales [B, N_c, c_I/32] bytes, in one buffer. */
#define CSAHCA_MXFP4 3

/* status codes */
#define CSAHCA_OK 0
#define CSAHCA_EINVAL (-1)     /* a pointer, size or value is invalid                  */
#define CSAHCA_ENOTSUP (-2)    /* valid, but outside the shapes / types built here      */
#define CSAHCA_EWORKSPACE (-3) /* workspace missing or smaller than *_workspace_size() */
#define CSAHCA_ELAUNCH (-4)    /* the HIP runtime refused a launch                      */

/*
 * csa_compress / hca_compress -- softmax-gated block pooling.
 * Source: "DeepSeek-V4 Hybrid Attention: CSA, HCA, mHC, MoE", section V.1 (equation
 * C_i^comp) and VI (non-overlapping m' blocks); "DeepSeek-V4 Architecture From Kernels",
 * section 6 (a softmax within each block followed by a weighted sum).
 *
 *   out[b, i, ch] = sum_{j<m} S[b,i,j,ch] * kv[b, m*i+j, ch],
 *   S[b,i,.,ch]   = softmax_j( gate[b, m*i+j, ch] + pos_bias[j, ch] )
 * for i < n / m (floor: a trailing partial block is not emitted).  The softmax runs over
 * the m tokens of the block separately for every channel.
 *
 *   kv, gate   [B, n, c] of `dtype` (CSAHCA_F32 or CSAHCA_BF16); sequence b starts at
 *              kv + b * in_bstride elements (same stride for gate); in_bstride >= n*c.
 *   pos_bias   [m, c] float32, or NULL for zero bias.
 *   out        [B, n/m, c] of `dtype`; sequence b starts at out + b * out_bstride
 *              elements, out_bstride >= (n/m)*c.  A cache append is one call on the last
 *              m tokens with `out` pointing at the new entry.
 *   Limits: B >= 1, n >= 0, c >= 8 and c % 8 == 0, 1 <= m <= 4096.  With n < m nothing is
 *   read or written (the pointers may then be NULL).
 * The two names run the same kernel; they exist so that each branch's call reads as the
 * pages name it (m = 4 for CSA, m' = 128 for HCA in the V4 settings).
 */
int csa_compress(const void* kv, const void* gate, const float* pos_bias, void* out, int B,
                 int n, int c, int m, int dtype, long long in_bstride, long long out_bstride,
                 void* stream);
int hca_compress(const void* kv, const void* gate, const float* pos_bias, void* out, int B,
                 int n, int c, int m, int dtype, long long in_bstride, long long out_bstride,
                 void* stream);

/*
 * csahca_compress_pair -- the CSA and the HCA pooling of one layer pair (for instance the
 * blocks a decode step completes in both caches) in one launch.
 * Source: as csa_compress and hca_compress (the same per-block definition, run for two
 * caches); "DeepSeek-V4 Architecture From Kernels ... C-Kernel-Engine", section 9 (an entry
 * is made in each cache whenever a block of its size completes).
 * Side a and side b each take the arguments of csa_compress / hca_compress without the
 * bias: kv_x, gate_x [B, n_x, c] (batch stride in_bstride_x elements), out_x [B, n_x / m_x, c]
 * (batch stride out_bstride_x), sharing B, c and dtype.  Every argument rule of those
 * calls applies to both sides; a side with no complete block emits nothing.  The entries
 * are bit-identical to the two separate calls.  When one side has few entries of many
 * tokens and the other does not, both run in one kernel launch (the layout of a decode
 * step); otherwise the two poolings are enqueued one after the other.  Errors are checked
 * for both sides before anything is enqueued.
 */
int csahca_compress_pair(const void* kv_a, const void* gate_a, void* out_a, int n_a, int m_a,
                         long long in_bstride_a, long long out_bstride_a, const void* kv_b,
                         const void* gate_b, void* out_b, int n_b, int m_b,
                         long long in_bstride_b, long long out_bstride_b, int B, int c,
                         int dtype, void* stream);

/*
 * csa_compress_overlap -- the overlapped two-stream CSA compressor.
 * Source: "DeepSeek-V4 Hybrid Attention: CSA, HCA, mHC, MoE", section V.1 (two KV
 * streams a and b with their own compression scores; entry i combines stream a's block i
 * with stream b's block i-1, equation C_i^comp).
 *
 *   out[b, e, ch] = sum_{j<m} S[j, ch] * kv_a[b, m*i+j, ch]
 *                 + sum_{j<m} S[m+j, ch] * kv_b[b, m*(i-1)+j, ch],     i = e + prev,
 *   S[., ch] = softmax over the 2m logits ( gate_a[b, m*i+j, ch] + pos_bias[j, ch] ;
 *                                           gate_b[b, m*(i-1)+j, ch] + pos_bias[m+j, ch] )
 * One joint softmax per channel (the pages give the sum; normalising the 2m weights
 * together is the reading adopted).  Block i = 0 has no predecessor: its softmax runs
 * over stream a's m logits alone.  With prev = 1 the arrays start one block before the
 * first entry to emit (a cache append passes the last 2m tokens, blocks i-1 and i, and
 * gets entry i); n/m - prev entries are written.
 *
 *   kv_a, gate_a, kv_b, gate_b  [B, n, c] of `dtype` (CSAHCA_F32 or CSAHCA_BF16), all
 *              with the batch stride in_bstride (elements) >= n*c.
 *   pos_bias   [2m, c] float32 (rows 0..m-1 stream a positions, m..2m-1 stream b), or
 *              NULL for zero bias.
 *   out        [B, n/m - prev, c] of `dtype`, batch stride out_bstride.
 *   prev       0 or 1.
 *   Limits and errors as csa_compress; nothing is read or written when n/m - prev <= 0.
 */
int csa_compress_overlap(const void* kv_a, const void* gate_a, const void* kv_b,
                         const void* gate_b, const float* pos_bias, void* out, int B, int n,
                         int c, int m, int prev, int dtype, long long in_bstride,
                         long long out_bstride, void* stream);

/*
 * lightning_index_topk -- lightning-indexer scores and exact top-k selection.
 * Source: "DeepSeek-V4 Hybrid Attention: CSA, HCA, mHC, MoE", section V.2, equation
 * I_{t,s} and the top-k selector; "DeepSeek-V4: Anatomy of an Open-Source Frontier
 * Model", "Worked example" (top-k can pick no more entries than exist).
 *
 *   I[b,t,s] = sum_h w_idx[b,t,h] * max(0, sum_d q_idx[b,t,h,d] * k_idx[b,s,d])
 * for every usable entry s (V = min(N_c, (p+1)/m) of them).  The selection keeps
 * K = min(k, V) entries with the highest scores; equal scores go to the lower index and
 * -0.0 counts as +0.0.  topk_idx[b,t,:] lists them in ascending index order, followed by
 * k-K entries of -1.
 *
 *   q_idx      [B, Tq, n_ih, c_I] of idx_dtype (CSAHCA_FP8_E4M3FN or CSAHCA_F32; FP8 for
 *              CSAHCA_MXFP4).
 *   w_idx      [B, Tq, n_ih] float32.
 *   k_idx      [B, N_c, c_I] of idx_dtype (the compressed indexer-key cache); for
 *              CSAHCA_MXFP4 the packed rows and then the scales (see the define).
 *   q_pos      [B] int32 device; m = CSA block size of the cache.
 *   topk_idx   [B, Tq, k] int32 (out).
 *   topk_score [B, Tq, k] float32 (out, nullable): the selected scores, -inf on padding.
 *   all_scores [B, Tq, N_c] float32 (out, nullable): every score; entries s >= V are
 *              left unwritten.
 *   Limits: FP8 keys need n_ih in {16, 32, 64, 128} and c_I in {32, 64, 128}; MX FP4
 *   keys n_ih in {16, 32, 64, 128} and c_I = 128 (source: "DeepSeek-V4: Anatomy of an
 *   Open-Source Frontier Model", the indexer's query-key path trained down to FP4); F32 keys
 *   need n_ih * c_I <= 4096.  1 <= k <= 1024, N_c <= 262144.
 *
 * Workspace: lightning_index_topk_workspace_size() bytes, caller-owned, no initial
 * contents needed.  After a decode call that selected from chunk lists (Tq == 1,
 * c_I == 128) the workspace's last B*Tq 32-bit words (rounded up to 256 bytes) say how
 * each query's selection went: 1 the chunks' lists held the top k, 2 it went through the
 * group maxima (the best entries clustered in a few chunks), 3 every usable entry was
 * selected.
 */
size_t lightning_index_topk_workspace_size(int B, int Tq, int n_ih, int N_c, int k);
int lightning_index_topk(const void* q_idx, const float* w_idx, const void* k_idx,
                         int idx_dtype, const int* q_pos, int m, int B, int Tq, int n_ih,
                         int c_I, int N_c, int k, int* topk_idx, float* topk_score,
                         float* all_scores, void* workspace, size_t ws_bytes, void* stream);

/*
 * lightning_index_topk_noalloc -- lightning_index_topk for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): same arguments and results, minus the workspace.
 *
 * The workspace is instead a file-scope device array of CSAHCA_NOALLOC_SCRATCH_BYTES that
 * every GPU the library runs on holds until the process ends.  Its device address is
 * looked up once per device, on the first call with that device current; the stream must
 * belong to the current device (else CSAHCA_EINVAL).  The call allocates and frees
 * nothing.  A call whose lightning_index_topk_workspace_size() exceeds the maximum returns
 * CSAHCA_EWORKSPACE and enqueues nothing.  All calls on one GPU share that GPU's array:
 * calls that overlap on one GPU (different streams, or host threads without ordering)
 * race on it and their results are undefined; calls ordered on one stream are fine.
 */
#define CSAHCA_NOALLOC_SCRATCH_BYTES (32u << 20)
int lightning_index_topk_noalloc(const void* q_idx, const float* w_idx, const void* k_idx,
                                 int idx_dtype, const int* q_pos, int m, int B, int Tq,
                                 int n_ih, int c_I, int N_c, int k, int* topk_idx,
                                 float* topk_score, float* all_scores, void* stream);

/*
 * The two halves of lightning_index_topk, for callers that time or check them apart.
 * lightning_index_score writes every usable score to `scores` [B, Tq, N_c] and the
 * per-16-entry group maxima to the workspace (at decode, where lightning_index_topk
 * fuses the chunk lists into scoring, the lists too); lightning_index_select must then be
 * given the same scores, workspace and shape arguments.  Running both equals one
 * lightning_index_topk call, launch for launch.  Same limits and workspace size.
 */
int lightning_index_score(const void* q_idx, const float* w_idx, const void* k_idx,
                          int idx_dtype, const int* q_pos, int m, int B, int Tq, int n_ih,
                          int c_I, int N_c, int k, float* scores, void* workspace,
                          size_t ws_bytes, void* stream);
int lightning_index_select(const float* scores, const int* q_pos, int m, int B, int Tq,
                           int N_c, int k, int* topk_idx, float* topk_score, void* workspace,
                           size_t ws_bytes, void* stream);

/*
 * csa_attend -- multi-query attention over the selected compressed entries plus the
 * sliding window, one joint softmax.
 * Source: "DeepSeek-V4 Hybrid Attention: CSA, HCA, mHC, MoE", section V.3 (core attention
 * in MQA form over the selected blocks; one K = V row shared by all heads) and section I
 * (softmax(QK^T/sqrt(c))V); "DeepSeek-V4: Anatomy of an Open-Source Frontier Model",
 * "One query in a CSA layer", steps 3-5 (selected entries plus the last 128 raw tokens,
 * attended together).
 *
 *   rows(b,t) = { ckv[b, s] : s in topk_idx[b,t,:], s != -1 } followed by the window rows
 *   out[b,t,h] = sum_r softmax_r(scale * q[b,t,h] . row_r) * row_r
 *   lse[b,t,h] = log sum_r exp(scale * q[b,t,h] . row_r)   (natural log)
 *
 *   q       [B, Tq, n_h, c] of dtype; ckv [B, N_c, c]; topk_idx [B, Tq, k] int32 with
 *           entries in [0, N_c) or -1 (other values are treated as -1).
 *   win_kv  [B, L, c]; win_pos [B] int32 device; q_pos [B] int32 device.
 *   out     [B, Tq, n_h, c] of dtype; lse [B, Tq, n_h] float32 or NULL.
 *   dtype   CSAHCA_BF16: c == 512, n_h % 16 == 0, n_h <= 128.
 *           CSAHCA_F32:  c <= 256, c % 4 == 0, n_h * (k + W) <= 12288.
 *   A query with no row at all (not possible when W >= 1) gets out = 0, lse = -inf.
 */
size_t csa_attend_workspace_size(int B, int Tq, int n_h, int c, int k, int W);
int csa_attend(const void* q, const void* ckv, const int* topk_idx, const void* win_kv,
               const int* win_pos, const int* q_pos, int B, int Tq, int n_h, int c, int N_c,
               int k, int L, int W, float scale, int dtype, void* out, float* lse,
               void* workspace, size_t ws_bytes, void* stream);

/*
 * hca_attend -- multi-query attention over every usable compressed entry plus the window.
 * Source: "DeepSeek-V4 Hybrid Attention: CSA, HCA, mHC, MoE", section VI, equation
 * o_{t,i} (query q_{t,i}, key = value = C^comp, dense over all compressed entries, MQA);
 * "DeepSeek-V4: Anatomy of an Open-Source Frontier Model", "Hybrid attention with CSA and
 * HCA" (128-token uncompressed window in both layer types).
 *
 *   rows(b,t) = { ckv[b, s] : s < min(N_h, (p+1)/m) } followed by the window rows.
 * Arguments as csa_attend, with m the HCA block size (m') and N_h the cache length.
 *   dtype   CSAHCA_BF16: c == 512, n_h % 16 == 0, n_h <= 128.
 *           CSAHCA_F32:  c <= 256, c % 4 == 0, n_h * (N_h + W) <= 12288.
 */
size_t hca_attend_workspace_size(int B, int Tq, int n_h, int c, int N_h, int W);
int hca_attend(const void* q, const void* ckv, const void* win_kv, const int* win_pos,
               const int* q_pos, int m, int B, int Tq, int n_h, int c, int N_h, int L, int W,
               float scale, int dtype, void* out, float* lse, void* workspace,
               size_t ws_bytes, void* stream);

/*
 * csa_attend_sink / hca_attend_sink -- csa_attend / hca_attend with a per-head attention
 * sink.
 * Source: "DeepSeek-V4 Hybrid Attention: CSA, HCA, mHC, MoE", section IV (a learnable
 * attention sink per head, inside both branches).  Reading: the sink is a logit in the
 * units of scale * q.row that joins the softmax denominator and adds no value:
 *
 *   out[b,t,h] = sum_r e^{z_r} row_r / (e^{sink[h]} + sum_r e^{z_r}),  z_r = scale*q.row_r
 *   lse[b,t,h] = log(e^{sink[h]} + sum_r e^{z_r})
 *
 *   sink   [n_h] float32, device; NULL gives the plain call, an entry of -inf has no
 *          effect.
 * Every other argument, the limits and the errors are those of csa_attend / hca_attend
 * (same workspace size).
 */
int csa_attend_sink(const void* q, const void* ckv, const int* topk_idx, const void* win_kv,
                    const int* win_pos, const int* q_pos, int B, int Tq, int n_h, int c,
                    int N_c, int k, int L, int W, float scale, const float* sink, int dtype,
                    void* out, float* lse, void* workspace, size_t ws_bytes, void* stream);
int hca_attend_sink(const void* q, const void* ckv, const void* win_kv, const int* win_pos,
                    const int* q_pos, int m, int B, int Tq, int n_h, int c, int N_h, int L,
                    int W, float scale, const float* sink, int dtype, void* out, float* lse,
                    void* workspace, size_t ws_bytes, void* stream);

/*
 * csahca_compress_norm_rope / csa_compress_overlap_norm_rope / csahca_norm_rope -- RMSNorm
 * and partial RoPE, fused into pooling or on rows.
 * Source: "DeepSeek-V4 Hybrid Attention: CSA, HCA, mHC, MoE", section IV (both branches
 * apply RMSNorm to the queries and to the compressed KV entries, and RoPE to the last 64
 * dimensions only); the MLA walk-through's "The Code: RoPE Helpers" (the rotated
 * dimensions are consecutive pairs (2i, 2i+1), read as complex numbers and multiplied by
 * e^{i pos f_i}, f_i = theta^(-2i/d); theta = 10000 there).
 *
 *   norm_rope(x, pos)[ch] = rope_d( x / sqrt(mean_ch(x^2) + eps) * gamma , pos )
 * where rope_d rotates the last d channels as above and leaves the others unchanged.
 * Readings (the pages name RMSNorm but do not write it): the usual definition with a
 * per-channel gain and the caller's eps.  A compressed entry s carries position m * s,
 * the first raw position of its block.  Angles are formed in double precision, rotation
 * and normalisation in float32, the result rounded once to the row dtype.
 *
 * csahca_compress_norm_rope: csa_compress / hca_compress (same arguments and limits),
 *   then every emitted entry is normalised and rotated; the first emitted entry is
 *   entry `entry0` of the cache (0 for a whole pass, the entry's index for an append).
 * csa_compress_overlap_norm_rope: csa_compress_overlap, then the same.
 *   gamma   [c] float32 device (16-byte aligned), or NULL for unit gain.
 *   d_rope  rotated channels at the end of the row, d_rope % 8 == 0 and <= c (64 in the
 *           V4 settings, 0 for none).
 *   eps >= 0, theta > 0.  c / 8 must be a power of two no larger than 64 (c <= 512).
 *
 * csahca_norm_rope: rows x [B, T, H, c] of `dtype` -> y (same shape; y == x is allowed).
 *   Sequence b starts at x + b * x_bstride (y + b * y_bstride) elements; inside a
 *   sequence the rows are contiguous.  Strides >= T*H*c and multiples of 8.  Row (b, t, h) has position pos[b] + t * pstride: queries pass q_pos and
 *   pstride 1 (H = n_h), a window source its win_pos and 1 (H = 1), compressed entries
 *   built elsewhere NULL and m.  pos: [B] int32 device, or NULL for 0.  norm = 0 applies
 *   RoPE only.  Limits as above; T == 0 does nothing.
 */
int csahca_compress_norm_rope(const void* kv, const void* gate, const float* pos_bias,
                              const float* gamma, void* out, int B, int n, int c, int m,
                              long long entry0, int d_rope, float eps, float theta, int dtype,
                              long long in_bstride, long long out_bstride, void* stream);
int csa_compress_overlap_norm_rope(const void* kv_a, const void* gate_a, const void* kv_b,
                                   const void* gate_b, const float* pos_bias,
                                   const float* gamma, void* out, int B, int n, int c, int m,
                                   int prev, long long entry0, int d_rope, float eps,
                                   float theta, int dtype, long long in_bstride,
                                   long long out_bstride, void* stream);
int csahca_norm_rope(const void* x, void* y, const float* gamma, const int* pos, int B, int T,
                     int H, int c, int pstride, int d_rope, float eps, float theta, int norm,
                     int dtype, long long x_bstride, long long y_bstride, void* stream);

/*
 * csahca_compress_pair_norm_rope -- csahca_compress_pair with every emitted entry
 * normalised and rotated as csahca_compress_norm_rope does: the two poolings of one layer
 * pair (the blocks a decode step completes in both caches) in one launch.
 * Source: as csahca_compress_pair and csahca_compress_norm_rope.
 * Side x takes csahca_compress_norm_rope's arguments without the bias: its own gain
 * gamma_x ([c] float32 device, 16-byte aligned, or NULL) and first entry index entry0_x
 * (entry e carries position m_x * (entry0_x + e)); d_rope, eps and theta are shared.
 * Every argument rule of both calls applies; the entries are bit-identical to two
 * csahca_compress_norm_rope calls.  One launch when one side has few entries of many
 * tokens and the other does not; otherwise the two are enqueued one after the other.
 */
int csahca_compress_pair_norm_rope(const void* kv_a, const void* gate_a, const float* gamma_a,
                                   void* out_a, int n_a, int m_a, long long entry0_a,
                                   long long in_bstride_a, long long out_bstride_a,
                                   const void* kv_b, const void* gate_b, const float* gamma_b,
                                   void* out_b, int n_b, int m_b, long long entry0_b,
                                   long long in_bstride_b, long long out_bstride_b, int B, int c,
                                   int d_rope, float eps, float theta, int dtype, void* stream);

/*
 * csahca_compress_pair_norm_rope_rows -- csahca_compress_pair_norm_rope, and in the same
 * launch the T newest raw rows of each side normalised and rotated as window rows: a decode
 * step's new tokens enter both layers' windows while the blocks they complete are pooled.
 * Source: as csahca_compress_pair_norm_rope; "DeepSeek-V4 Hybrid Attention: CSA, HCA, mHC,
 * MoE", section IV (the window branch sees normalised, partially rotated keys too).
 * The pooling arguments and results are those of csahca_compress_pair_norm_rope.  The rows
 * of side x are those of
 *   csahca_norm_rope(row_x_x, row_y_x, gamma_x, row_pos_x, B, T, 1, c, 1, d_rope, eps,
 *                    theta, 1, dtype, row_x_bstride_x, row_y_bstride_x)
 * (the side's gain; row (b, t) at position row_pos_x[b] + t, or t when row_pos_x is NULL),
 * with the same bits.  T >= 0 (0: no rows, the call is csahca_compress_pair_norm_rope);
 * with T > 0 a side's row_x and row_y are both NULL (no rows for that side) or both
 * non-NULL and 16-byte aligned, its row strides then >= T*c and multiples of 8, and no
 * row range overlaps a pooling input or output.  A side may also pool nothing (n_x < m_x,
 * its pointers NULL): one layer's pooling and window rows in one launch.
 * One launch when the pooling is one launch (one side with few entries of many tokens,
 * bfloat16); otherwise the rows follow in csahca_norm_rope launches.  Errors as in the
 * two calls; nothing is enqueued on error.
 */
int csahca_compress_pair_norm_rope_rows(
    const void* kv_a, const void* gate_a, const float* gamma_a, void* out_a, int n_a, int m_a,
    long long entry0_a, long long in_bstride_a, long long out_bstride_a, const void* kv_b,
    const void* gate_b, const float* gamma_b, void* out_b, int n_b, int m_b, long long entry0_b,
    long long in_bstride_b, long long out_bstride_b, int B, int c, int d_rope, float eps,
    float theta, int dtype, int T, const void* row_x_a, void* row_y_a, const int* row_pos_a,
    long long row_x_bstride_a, long long row_y_bstride_a, const void* row_x_b, void* row_y_b,
    const int* row_pos_b, long long row_x_bstride_b, long long row_y_bstride_b, void* stream);

/*
 * csa_attend_ex / hca_attend_ex -- csa_attend_sink / hca_attend_sink with the RMSNorm and
 * partial RoPE of the queries done inside the attention kernel, as it loads them.
 * Source: "DeepSeek-V4 Hybrid Attention: CSA, HCA, mHC, MoE", section IV (queries and KV
 * entries normalised, the last 64 dimensions rotated, in both branches), with the
 * norm_rope definition above.
 *
 * With q_norm = 1 the result is that of csahca_norm_rope (norm = 1, pos = q_pos,
 * pstride 1) applied to q first, the normalised query rounded once to bfloat16 as there,
 * and then the _sink call, up to the order in which the row's sum of squares is taken (a
 * normalised element can round the other way); q itself is not written.  Keys are used as stored: compressed entries
 * are normalised when pooled (csahca_compress_norm_rope), and a window row is normalised
 * once, when its token arrives (csahca_norm_rope on the new rows), not at every step.
 *
 *   q_norm   1: RMSNorm + RoPE of the queries; 0: the _sink call.
 *   q_gamma  [c] float32 device, or NULL for unit gain.
 *   d_rope   rotated channels at the end of the row, a multiple of 8 in [0, 128].
 *   eps >= 0, theta > 0 (finite).
 *   sink     as in the _sink calls (NULL for none).
 * Every other argument, the limits and the errors are those of csa_attend / hca_attend
 * (same workspace size); with q_norm = 1 dtype must be CSAHCA_BF16 (else CSAHCA_ENOTSUP).
 */
int csa_attend_ex(const void* q, const void* ckv, const int* topk_idx, const void* win_kv,
                  const int* win_pos, const int* q_pos, int B, int Tq, int n_h, int c, int N_c,
                  int k, int L, int W, float scale, const float* sink, const float* q_gamma,
                  int q_norm, int d_rope, float eps, float theta, int dtype, void* out,
                  float* lse, void* workspace, size_t ws_bytes, void* stream);
int hca_attend_ex(const void* q, const void* ckv, const void* win_kv, const int* win_pos,
                  const int* q_pos, int m, int B, int Tq, int n_h, int c, int N_h, int L, int W,
                  float scale, const float* sink, const float* q_gamma, int q_norm, int d_rope,
                  float eps, float theta, int dtype, void* out, float* lse, void* workspace,
                  size_t ws_bytes, void* stream);

/*
 * lightning_index_topk_csa_compress -- lightning_index_topk, and with it
 *   csa_compress(kv, gate, NULL, out, B, n, c, m, dtype, in_bstride, out_bstride)
 * on the same stream: a decode step's new CSA block pooled while the indexer selects (the
 * indexer reads no pooled entry, so the two are independent).
 * Source: as lightning_index_topk and csa_compress.
 * Arguments: those of lightning_index_topk, then csa_compress's pooling arguments without
 * the bias (the block size is the indexer's m).  Every argument rule of both calls
 * applies, and all are checked before anything is enqueued; the results are those of the
 * two calls, bit for bit.  With bfloat16 entries, m < 8 and a decode selection from chunk
 * lists, the pooling runs in extra workgroups of the selection launch; otherwise its own
 * launch follows the indexer's.
 */
int lightning_index_topk_csa_compress(const void* q_idx, const float* w_idx, const void* k_idx,
                                      int idx_dtype, const int* q_pos, int m, int B, int Tq,
                                      int n_ih, int c_I, int N_c, int k, int* topk_idx,
                                      float* topk_score, float* all_scores, void* workspace,
                                      size_t ws_bytes, const void* kv, const void* gate, void* out,
                                      int n, int c, int dtype, long long in_bstride,
                                      long long out_bstride, void* stream);

/*
 * lightning_index_topk_csa_compress_norm_rope_rows -- lightning_index_topk, and with it
 *   csahca_compress_pair_norm_rope_rows with side a only: the CSA cache's new entries pooled,
 *   normalised and rotated (csahca_compress_norm_rope(kv, gate, NULL, gamma, out, B, n, c, m,
 *   entry0, d_rope, eps, theta, dtype, in_bstride, out_bstride)), and the step's T new window
 *   rows normalised and rotated (csahca_norm_rope(row_x, row_y, gamma, row_pos, B, T, 1, c, 1,
 *   d_rope, eps, theta, 1, dtype, row_x_bstride, row_y_bstride)); none of the three reads
 *   another's output.
 * Source: as lightning_index_topk, csa_compress and csahca_compress_norm_rope.
 * Arguments: those of lightning_index_topk, then those of the pooling and the rows (the
 * block size is the indexer's m; row_x and row_y both NULL, or T == 0, for no rows).
 * Every argument rule of the calls applies, all checked before anything is enqueued; the
 * results are those of the calls, bit for bit.  With bfloat16 entries, m < 8 and a
 * decode selection from chunk lists, the pooling and the rows run in extra workgroups of
 * the selection launch; otherwise in launches of their own after the indexer's.
 */
int lightning_index_topk_csa_compress_norm_rope_rows(
    const void* q_idx, const float* w_idx, const void* k_idx, int idx_dtype, const int* q_pos, int m,
    int B, int Tq, int n_ih, int c_I, int N_c, int k, int* topk_idx, float* topk_score,
    float* all_scores, void* workspace, size_t ws_bytes, const void* kv, const void* gate,
    const float* gamma, void* out, int n, int c, long long entry0, int d_rope, float eps,
    float theta, int dtype, long long in_bstride, long long out_bstride, int T,
    const void* row_x, void* row_y, const int* row_pos, long long row_x_bstride,
    long long row_y_bstride, void* stream);

/*
 * csa_attend_begin / csa_attend_end, hca_attend_begin / hca_attend_end -- the two halves
 * of csa_attend_ex / hca_attend_ex, for a caller that runs the split merge on another
 * stream than the attention (a decode step that joins its two attention layers on one
 * stream: the merge there waits only for the attention, already finished).
 * Source: as csa_attend / hca_attend (the split merge combines partial softmax results by
 * their log-sum-exp, which is exact for the joint softmax).
 * Arguments, limits, workspace and errors are those of csa_attend_ex / hca_attend_ex; both
 * halves take the same arguments.  _begin enqueues the attention: when the launch plan
 * has a single split (or dtype is CSAHCA_F32) it writes out and lse itself and _end does
 * nothing; otherwise it leaves per-split partial results in the workspace, and _end
 * (enqueued after _begin has completed, with the workspace untouched in between) merges
 * them into out and lse.  _begin then _end give the same bits as the _ex call.
 */
int csa_attend_begin(const void* q, const void* ckv, const int* topk_idx, const void* win_kv,
                     const int* win_pos, const int* q_pos, int B, int Tq, int n_h, int c, int N_c,
                     int k, int L, int W, float scale, const float* sink, const float* q_gamma,
                     int q_norm, int d_rope, float eps, float theta, int dtype, void* out,
                     float* lse, void* workspace, size_t ws_bytes, void* stream);
int csa_attend_end(const void* q, const void* ckv, const int* topk_idx, const void* win_kv,
                   const int* win_pos, const int* q_pos, int B, int Tq, int n_h, int c, int N_c,
                   int k, int L, int W, float scale, const float* sink, const float* q_gamma,
                   int q_norm, int d_rope, float eps, float theta, int dtype, void* out,
                   float* lse, void* workspace, size_t ws_bytes, void* stream);
int hca_attend_begin(const void* q, const void* ckv, const void* win_kv, const int* win_pos,
                     const int* q_pos, int m, int B, int Tq, int n_h, int c, int N_h, int L, int W,
                     float scale, const float* sink, const float* q_gamma, int q_norm,
                     int d_rope, float eps, float theta, int dtype, void* out, float* lse,
                     void* workspace, size_t ws_bytes, void* stream);
int hca_attend_end(const void* q, const void* ckv, const void* win_kv, const int* win_pos,
                   const int* q_pos, int m, int B, int Tq, int n_h, int c, int N_h, int L, int W,
                   float scale, const float* sink, const float* q_gamma, int q_norm, int d_rope,
                   float eps, float theta, int dtype, void* out, float* lse, void* workspace,
                   size_t ws_bytes, void* stream);

/*
 * csahca_kv_ring_rows / csahca_kv_append / csahca_kv_fork -- the cache lifecycle of one
 * layer: raw tokens arrive, completed blocks become compressed entries, the recent window
 * stays exact, a request can start from another's prefix.
 * Source: "DeepSeek-V4 Architecture From Kernels ... C-Kernel-Engine", section 9
 * (heterogeneous KV cache: per request the last W raw tokens, one compressed entry per m
 * tokens and the tail of the incomplete block; an entry is made when its block completes;
 * tails must stay consistent when a request reuses a cached prefix).
 *
 * Ring layout (the reading adopted): the raw values and gate logits of a sequence are kept
 * in rings of R = csahca_kv_ring_rows(W, m) = m * ceil((W + m - 1) / m) rows, the smallest
 * whole number of blocks holding the window and a tail.  Position p is stored twice, at
 * rows p mod R and p mod R + R, so
 *   - the last L <= R positions p0 .. p0+L-1 are the L contiguous rows from p0 mod R, and
 *   - with ring_bstride == 2*R*c, csa_attend / hca_attend read the window straight from
 *     the ring: win_kv = kv_ring, L = 2R, win_pos[b] = R * floor(max(0, n - R) / R) for a
 *     sequence of n tokens, valid for queries at positions >= n - R + W - 1 (decode and
 *     chunks of up to R - W + 1 tokens).
 *
 * csahca_kv_append: append n_new tokens to sequences that each hold n_old (the same for
 * every sequence of the call).  Entries s with n_old/m <= s < (n_old+n_new)/m are written,
 * each pooled as csa_compress does (the block that was a tail is pooled from the ring),
 * then the last min(n_new, R) tokens enter the ring.
 *   kv_ring, gate_ring  [B, 2R, c] of `dtype`, batch stride ring_bstride >= 2*R*c.
 *   entries   [B, >= (n_old+n_new)/m, c] of `dtype`, batch stride ent_bstride; may be NULL
 *             when no block completes.
 *   kv_new, gate_new  [B, n_new, c] of `dtype`, batch stride new_bstride >= n_new*c.
 *   pos_bias  [m, c] float32 or NULL (as csa_compress).
 *   Strides are in elements and multiples of 8.  Limits: c % 8 == 0, 1 <= m <= 4096,
 *   W >= 0, dtype CSAHCA_F32 or CSAHCA_BF16.  n_new == 0 does nothing.  Two appends to
 *   the same sequences must be ordered (same stream).
 *
 * csahca_kv_fork: a new request sharing the source's prefix.  Copies the source rings
 * (both halves, all B sequences) as they stand, i.e. the prefix is the source's current
 * length P, and its first n_entries = P / m entries; the copy then takes appends with
 * n_old = P.  Rings and entries use the batch strides of csahca_kv_append; dst and src
 * must not overlap.
 *
 * Both return CSAHCA_OK or a negative status as every entry point;
 * csahca_kv_ring_rows returns 0 for W < 0 or m < 1.
 */
int csahca_kv_ring_rows(int W, int m);
int csahca_kv_append(void* kv_ring, void* gate_ring, void* entries, const void* kv_new,
                     const void* gate_new, const float* pos_bias, int B, long long n_old,
                     int n_new, int c, int m, int W, int dtype, long long new_bstride,
                     long long ring_bstride, long long ent_bstride, void* stream);
int csahca_kv_fork(void* dst_kv_ring, void* dst_gate_ring, void* dst_entries,
                   const void* src_kv_ring, const void* src_gate_ring, const void* src_entries,
                   int B, long long n_entries, int c, int m, int W, int dtype,
                   long long ring_bstride, long long ent_bstride, void* stream);

/*
 * grouped_out_proj -- the grouped output projection shared by both branches.
 * Source: "DeepSeek-V4 Hybrid Attention: CSA, HCA, mHC, MoE", section V.3 (the c * n_h
 * concatenated head outputs are split into g groups of heads, each group projected by its
 * own smaller matrix to d_g dimensions, the g results concatenated) and section IV.
 *
 *   y[t, gi*d_g + j] = sum_{k < K_g} o[t, gi*K_g + k] * w[gi, j, k]     (gi < g, j < d_g)
 *
 *   o   [T, g*K_g] bf16, row stride ldo >= g*K_g elements: each token's concatenated head
 *       outputs in head order (an attention output [B, Tq, n_h, c] is T = B*Tq rows with
 *       K_g = n_h*c/g, so group gi holds heads gi*n_h/g .. (gi+1)*n_h/g - 1).
 *   w   [g, d_g, K_g] bf16: each group's matrix laid out as a linear layer's weight (out x
 *       in).
 *   y   [T, g*d_g] bf16, row stride ldy >= g*d_g; fp32 accumulation, rounded once.
 * Readings: contiguous head groups, outputs concatenated in group order, no bias.
 * Limits: dtype CSAHCA_BF16; K_g % 128 == 0; d_g % 16 == 0; strides multiples of 8;
 * T == 0 does nothing.  Up to 64 tokens (or d_g % 128 != 0) a kernel streams w once per 64
 * tokens; more tokens take 256 x 128 MFMA tiles.
 */
int grouped_out_proj(const void* o, const void* w, void* y, int T, int g, int K_g, int d_g,
                     long long ldo, long long ldy, int dtype, void* stream);

/* Message for the last non-OK status returned on the calling thread ("" if none). */
const char* csahca_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int csahca_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CSAHCA_H */
