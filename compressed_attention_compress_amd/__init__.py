"""Python binding of libcsahca.so, the gfx950 CSA / HCA compressed-attention library.

Argument marshalling only: every entry point forwards to the C function of the same name
(declared in include/csahca.h) and raises CsaHcaError on a non-zero status.  Pointer
arguments accept a torch tensor (its data_ptr is passed), a plain integer address or
None.  ``stream`` defaults to torch's current HIP stream.  There is no fallback: if the
shared library is missing or cannot be loaded, every call raises.
"""
import ctypes
import os

F32, BF16, FP8_E4M3FN = 0, 1, 2
OK, EINVAL, ENOTSUP, EWORKSPACE, ELAUNCH = 0, -1, -2, -3, -4

# CSAHCA_LIB selects another build of the same library (the host-sanitizer build in its
# tests); by default the library next to this file
LIB_PATH = os.environ.get("CSAHCA_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                        "libcsahca.so")

_P = ctypes.c_void_p
_I = ctypes.c_int
_LL = ctypes.c_longlong
_F = ctypes.c_float
_SZ = ctypes.c_size_t

_SIGNATURES = {
    "csa_compress": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _LL, _LL, _P]),
    "hca_compress": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _LL, _LL, _P]),
    "csahca_compress_pair": (_I, [_P, _P, _P, _I, _I, _LL, _LL, _P, _P, _P, _I, _I, _LL, _LL,
                                  _I, _I, _I, _P]),
    "csahca_compress_pair_norm_rope": (_I, [_P, _P, _P, _P, _I, _I, _LL, _LL, _LL, _P, _P, _P, _P,
                                            _I, _I, _LL, _LL, _LL, _I, _I, _I, _F, _F, _I, _P]),
    "csahca_compress_pair_norm_rope_rows": (_I, [_P, _P, _P, _P, _I, _I, _LL, _LL, _LL, _P, _P, _P,
                                                 _P, _I, _I, _LL, _LL, _LL, _I, _I, _I, _F, _F, _I,
                                                 _I, _P, _P, _P, _LL, _LL, _P, _P, _P, _LL, _LL,
                                                 _P]),
    "csa_compress_overlap": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _LL, _LL, _P]),
    "csahca_compress_norm_rope": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _LL, _I, _F, _F, _I,
                                       _LL, _LL, _P]),
    "csa_compress_overlap_norm_rope": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _LL,
                                            _I, _F, _F, _I, _LL, _LL, _P]),
    "csahca_norm_rope": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _F, _I, _I, _LL, _LL,
                              _P]),
    "grouped_out_proj": (_I, [_P, _P, _P, _I, _I, _I, _I, _LL, _LL, _I, _P]),
    "csahca_kv_ring_rows": (_I, [_I, _I]),
    "csahca_kv_append": (_I, [_P, _P, _P, _P, _P, _P, _I, _LL, _I, _I, _I, _I, _I, _LL, _LL, _LL,
                              _P]),
    "csahca_kv_fork": (_I, [_P, _P, _P, _P, _P, _P, _I, _LL, _I, _I, _I, _I, _LL, _LL, _P]),
    "lightning_index_topk_workspace_size": (_SZ, [_I, _I, _I, _I, _I]),
    "lightning_index_topk": (_I, [_P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P,
                                  _P, _SZ, _P]),
    "lightning_index_topk_noalloc": (_I, [_P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P,
                                          _P, _P]),
    "lightning_index_topk_csa_compress": (_I, [_P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _I, _I, _P,
                                               _P, _P, _P, _SZ, _P, _P, _P, _I, _I, _I, _LL, _LL,
                                               _P]),
    "lightning_index_topk_csa_compress_norm_rope_rows": (_I, [_P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _I, _I,
                                                           _P, _P, _P, _P, _SZ, _P, _P, _P, _P, _I, _I,
                                                           _LL, _I, _F, _F, _I, _LL, _LL, _I, _P, _P, _P,
                                                           _LL, _LL, _P]),
    "lightning_index_score": (_I, [_P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _SZ,
                                   _P]),
    "lightning_index_select": (_I, [_P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _SZ, _P]),
    "csa_attend_workspace_size": (_SZ, [_I, _I, _I, _I, _I, _I]),
    "csa_attend": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P, _P,
                        _P, _SZ, _P]),
    "hca_attend_workspace_size": (_SZ, [_I, _I, _I, _I, _I, _I]),
    "hca_attend": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P, _P, _P,
                        _SZ, _P]),
    "csa_attend_sink": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _P, _I,
                             _P, _P, _P, _SZ, _P]),
    "hca_attend_sink": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _P, _I, _P,
                             _P, _P, _SZ, _P]),
    "csa_attend_ex": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _I,
                           _I, _F, _F, _I, _P, _P, _P, _SZ, _P]),
    "hca_attend_ex": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _I, _I,
                           _F, _F, _I, _P, _P, _P, _SZ, _P]),
    "csa_attend_begin": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _I,
                              _I, _F, _F, _I, _P, _P, _P, _SZ, _P]),
    "hca_attend_begin": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _I, _I,
                              _F, _F, _I, _P, _P, _P, _SZ, _P]),
    "csa_attend_end": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _I,
                            _I, _F, _F, _I, _P, _P, _P, _SZ, _P]),
    "hca_attend_end": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _I, _I,
                            _F, _F, _I, _P, _P, _P, _SZ, _P]),
    "csahca_last_error": (ctypes.c_char_p, []),
    "csahca_version": (_I, []),
}

_lib = None


class CsaHcaError(RuntimeError):
    def __init__(self, name, status, msg):
        super().__init__(f"{name} returned {status}: {msg}")
        self.status = status


def load(path=LIB_PATH):
    """Load (once) and return the ctypes handle of the shared library."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise OSError(f"libcsahca.so not built ({path}); run __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(name, status):
    if status != OK:
        raise CsaHcaError(name, status, load().csahca_last_error().decode())
    return status


def version():
    return load().csahca_version()


def last_error():
    return load().csahca_last_error().decode()


def csa_compress(kv, gate, pos_bias, out, B, n, c, m, dtype, in_bstride, out_bstride,
                 stream=None):
    return _check("csa_compress", load().csa_compress(
        _ptr(kv), _ptr(gate), _ptr(pos_bias), _ptr(out), B, n, c, m, dtype, in_bstride,
        out_bstride, _stream(stream)))


def hca_compress(kv, gate, pos_bias, out, B, n, c, m, dtype, in_bstride, out_bstride,
                 stream=None):
    return _check("hca_compress", load().hca_compress(
        _ptr(kv), _ptr(gate), _ptr(pos_bias), _ptr(out), B, n, c, m, dtype, in_bstride,
        out_bstride, _stream(stream)))


def csa_compress_overlap(kv_a, gate_a, kv_b, gate_b, pos_bias, out, B, n, c, m, prev, dtype,
                         in_bstride, out_bstride, stream=None):
    return _check("csa_compress_overlap", load().csa_compress_overlap(
        _ptr(kv_a), _ptr(gate_a), _ptr(kv_b), _ptr(gate_b), _ptr(pos_bias), _ptr(out), B, n, c,
        m, prev, dtype, in_bstride, out_bstride, _stream(stream)))


def csahca_compress_pair(kv_a, gate_a, out_a, n_a, m_a, in_bstride_a, out_bstride_a, kv_b, gate_b,
                         out_b, n_b, m_b, in_bstride_b, out_bstride_b, B, c, dtype, stream=None):
    return _check("csahca_compress_pair", load().csahca_compress_pair(
        _ptr(kv_a), _ptr(gate_a), _ptr(out_a), n_a, m_a, in_bstride_a, out_bstride_a, _ptr(kv_b),
        _ptr(gate_b), _ptr(out_b), n_b, m_b, in_bstride_b, out_bstride_b, B, c, dtype,
        _stream(stream)))


def csahca_compress_pair_norm_rope(kv_a, gate_a, gamma_a, out_a, n_a, m_a, entry0_a, in_bstride_a,
                                   out_bstride_a, kv_b, gate_b, gamma_b, out_b, n_b, m_b, entry0_b,
                                   in_bstride_b, out_bstride_b, B, c, d_rope, eps, theta, dtype,
                                   stream=None):
    return _check("csahca_compress_pair_norm_rope", load().csahca_compress_pair_norm_rope(
        _ptr(kv_a), _ptr(gate_a), _ptr(gamma_a), _ptr(out_a), n_a, m_a, entry0_a, in_bstride_a,
        out_bstride_a, _ptr(kv_b), _ptr(gate_b), _ptr(gamma_b), _ptr(out_b), n_b, m_b, entry0_b,
        in_bstride_b, out_bstride_b, B, c, d_rope, float(eps), float(theta), dtype, _stream(stream)))


def csahca_compress_pair_norm_rope_rows(kv_a, gate_a, gamma_a, out_a, n_a, m_a, entry0_a,
                                        in_bstride_a, out_bstride_a, kv_b, gate_b, gamma_b, out_b,
                                        n_b, m_b, entry0_b, in_bstride_b, out_bstride_b, B, c,
                                        d_rope, eps, theta, dtype, T, row_x_a, row_y_a, row_pos_a,
                                        row_x_bstride_a, row_y_bstride_a, row_x_b, row_y_b,
                                        row_pos_b, row_x_bstride_b, row_y_bstride_b, stream=None):
    return _check("csahca_compress_pair_norm_rope_rows", load().csahca_compress_pair_norm_rope_rows(
        _ptr(kv_a), _ptr(gate_a), _ptr(gamma_a), _ptr(out_a), n_a, m_a, entry0_a, in_bstride_a,
        out_bstride_a, _ptr(kv_b), _ptr(gate_b), _ptr(gamma_b), _ptr(out_b), n_b, m_b, entry0_b,
        in_bstride_b, out_bstride_b, B, c, d_rope, float(eps), float(theta), dtype, T,
        _ptr(row_x_a), _ptr(row_y_a), _ptr(row_pos_a), row_x_bstride_a, row_y_bstride_a,
        _ptr(row_x_b), _ptr(row_y_b), _ptr(row_pos_b), row_x_bstride_b, row_y_bstride_b,
        _stream(stream)))


def csahca_compress_norm_rope(kv, gate, pos_bias, gamma, out, B, n, c, m, entry0, d_rope, eps,
                              theta, dtype, in_bstride, out_bstride, stream=None):
    return _check("csahca_compress_norm_rope", load().csahca_compress_norm_rope(
        _ptr(kv), _ptr(gate), _ptr(pos_bias), _ptr(gamma), _ptr(out), B, n, c, m, entry0, d_rope,
        eps, theta, dtype, in_bstride, out_bstride, _stream(stream)))


def csa_compress_overlap_norm_rope(kv_a, gate_a, kv_b, gate_b, pos_bias, gamma, out, B, n, c, m,
                                   prev, entry0, d_rope, eps, theta, dtype, in_bstride,
                                   out_bstride, stream=None):
    return _check("csa_compress_overlap_norm_rope", load().csa_compress_overlap_norm_rope(
        _ptr(kv_a), _ptr(gate_a), _ptr(kv_b), _ptr(gate_b), _ptr(pos_bias), _ptr(gamma), _ptr(out),
        B, n, c, m, prev, entry0, d_rope, eps, theta, dtype, in_bstride, out_bstride,
        _stream(stream)))


def csahca_norm_rope(x, y, gamma, pos, B, T, H, c, pstride, d_rope, eps, theta, norm, dtype,
                     x_bstride=None, y_bstride=None, stream=None):
    """Strides default to contiguous [B, T, H, c]."""
    seq = T * H * c
    return _check("csahca_norm_rope", load().csahca_norm_rope(
        _ptr(x), _ptr(y), _ptr(gamma), _ptr(pos), B, T, H, c, pstride, d_rope, eps, theta, norm,
        dtype, seq if x_bstride is None else x_bstride, seq if y_bstride is None else y_bstride,
        _stream(stream)))


def grouped_out_proj(o, w, y, T, g, K_g, d_g, ldo, ldy, dtype, stream=None):
    return _check("grouped_out_proj", load().grouped_out_proj(
        _ptr(o), _ptr(w), _ptr(y), T, g, K_g, d_g, ldo, ldy, dtype, _stream(stream)))


def csahca_kv_ring_rows(W, m):
    return load().csahca_kv_ring_rows(W, m)


def csahca_kv_append(kv_ring, gate_ring, entries, kv_new, gate_new, pos_bias, B, n_old, n_new,
                     c, m, W, dtype, new_bstride, ring_bstride, ent_bstride, stream=None):
    return _check("csahca_kv_append", load().csahca_kv_append(
        _ptr(kv_ring), _ptr(gate_ring), _ptr(entries), _ptr(kv_new), _ptr(gate_new),
        _ptr(pos_bias), B, n_old, n_new, c, m, W, dtype, new_bstride, ring_bstride, ent_bstride,
        _stream(stream)))


def csahca_kv_fork(dst_kv_ring, dst_gate_ring, dst_entries, src_kv_ring, src_gate_ring,
                   src_entries, B, n_entries, c, m, W, dtype, ring_bstride, ent_bstride,
                   stream=None):
    return _check("csahca_kv_fork", load().csahca_kv_fork(
        _ptr(dst_kv_ring), _ptr(dst_gate_ring), _ptr(dst_entries), _ptr(src_kv_ring),
        _ptr(src_gate_ring), _ptr(src_entries), B, n_entries, c, m, W, dtype, ring_bstride,
        ent_bstride, _stream(stream)))


def lightning_index_topk_workspace_size(B, Tq, n_ih, N_c, k):
    return load().lightning_index_topk_workspace_size(B, Tq, n_ih, N_c, k)


def lightning_index_topk(q_idx, w_idx, k_idx, idx_dtype, q_pos, m, B, Tq, n_ih, c_I, N_c, k,
                         topk_idx, topk_score, all_scores, workspace, ws_bytes, stream=None):
    return _check("lightning_index_topk", load().lightning_index_topk(
        _ptr(q_idx), _ptr(w_idx), _ptr(k_idx), idx_dtype, _ptr(q_pos), m, B, Tq, n_ih, c_I, N_c,
        k, _ptr(topk_idx), _ptr(topk_score), _ptr(all_scores), _ptr(workspace), ws_bytes,
        _stream(stream)))


def lightning_index_topk_csa_compress(q_idx, w_idx, k_idx, idx_dtype, q_pos, m, B, Tq, n_ih, c_I,
                                      N_c, k, topk_idx, topk_score, all_scores, workspace,
                                      ws_bytes, kv, gate, out, n, c, dtype, in_bstride,
                                      out_bstride, stream=None):
    return _check("lightning_index_topk_csa_compress", load().lightning_index_topk_csa_compress(
        _ptr(q_idx), _ptr(w_idx), _ptr(k_idx), idx_dtype, _ptr(q_pos), m, B, Tq, n_ih, c_I, N_c,
        k, _ptr(topk_idx), _ptr(topk_score), _ptr(all_scores), _ptr(workspace), ws_bytes,
        _ptr(kv), _ptr(gate), _ptr(out), n, c, dtype, in_bstride, out_bstride, _stream(stream)))


def lightning_index_topk_csa_compress_norm_rope_rows(
        q_idx, w_idx, k_idx, idx_dtype, q_pos, m, B, Tq, n_ih, c_I, N_c, k, topk_idx, topk_score,
        all_scores, workspace, ws_bytes, kv, gate, gamma, out, n, c, entry0, d_rope, eps, theta, dtype,
        in_bstride, out_bstride, T, row_x, row_y, row_pos, row_x_bstride, row_y_bstride, stream=None):
    return _check("lightning_index_topk_csa_compress_norm_rope_rows",
                  load().lightning_index_topk_csa_compress_norm_rope_rows(
                      _ptr(q_idx), _ptr(w_idx), _ptr(k_idx), idx_dtype, _ptr(q_pos), m, B, Tq, n_ih, c_I,
                      N_c, k, _ptr(topk_idx), _ptr(topk_score), _ptr(all_scores), _ptr(workspace),
                      ws_bytes, _ptr(kv), _ptr(gate), _ptr(gamma), _ptr(out), n, c, entry0, d_rope,
                      float(eps), float(theta), dtype, in_bstride, out_bstride, T, _ptr(row_x),
                      _ptr(row_y), _ptr(row_pos), row_x_bstride, row_y_bstride, _stream(stream)))


def lightning_index_topk_noalloc(q_idx, w_idx, k_idx, idx_dtype, q_pos, m, B, Tq, n_ih, c_I, N_c,
                                 k, topk_idx, topk_score, all_scores, stream=None):
    return _check("lightning_index_topk_noalloc", load().lightning_index_topk_noalloc(
        _ptr(q_idx), _ptr(w_idx), _ptr(k_idx), idx_dtype, _ptr(q_pos), m, B, Tq, n_ih, c_I, N_c,
        k, _ptr(topk_idx), _ptr(topk_score), _ptr(all_scores), _stream(stream)))


def lightning_index_score(q_idx, w_idx, k_idx, idx_dtype, q_pos, m, B, Tq, n_ih, c_I, N_c, k,
                          scores, workspace, ws_bytes, stream=None):
    return _check("lightning_index_score", load().lightning_index_score(
        _ptr(q_idx), _ptr(w_idx), _ptr(k_idx), idx_dtype, _ptr(q_pos), m, B, Tq, n_ih, c_I, N_c,
        k, _ptr(scores), _ptr(workspace), ws_bytes, _stream(stream)))


def lightning_index_select(scores, q_pos, m, B, Tq, N_c, k, topk_idx, topk_score, workspace,
                           ws_bytes, stream=None):
    return _check("lightning_index_select", load().lightning_index_select(
        _ptr(scores), _ptr(q_pos), m, B, Tq, N_c, k, _ptr(topk_idx), _ptr(topk_score),
        _ptr(workspace), ws_bytes, _stream(stream)))


def csa_attend_workspace_size(B, Tq, n_h, c, k, W):
    return load().csa_attend_workspace_size(B, Tq, n_h, c, k, W)


def csa_attend(q, ckv, topk_idx, win_kv, win_pos, q_pos, B, Tq, n_h, c, N_c, k, L, W, scale,
               dtype, out, lse, workspace, ws_bytes, stream=None):
    return _check("csa_attend", load().csa_attend(
        _ptr(q), _ptr(ckv), _ptr(topk_idx), _ptr(win_kv), _ptr(win_pos), _ptr(q_pos), B, Tq,
        n_h, c, N_c, k, L, W, float(scale), dtype, _ptr(out), _ptr(lse), _ptr(workspace),
        ws_bytes, _stream(stream)))


def hca_attend_workspace_size(B, Tq, n_h, c, N_h, W):
    return load().hca_attend_workspace_size(B, Tq, n_h, c, N_h, W)


def hca_attend(q, ckv, win_kv, win_pos, q_pos, m, B, Tq, n_h, c, N_h, L, W, scale, dtype, out,
               lse, workspace, ws_bytes, stream=None):
    return _check("hca_attend", load().hca_attend(
        _ptr(q), _ptr(ckv), _ptr(win_kv), _ptr(win_pos), _ptr(q_pos), m, B, Tq, n_h, c, N_h, L, W,
        float(scale), dtype, _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream)))


def csa_attend_sink(q, ckv, topk_idx, win_kv, win_pos, q_pos, B, Tq, n_h, c, N_c, k, L, W, scale,
                    sink, dtype, out, lse, workspace, ws_bytes, stream=None):
    return _check("csa_attend_sink", load().csa_attend_sink(
        _ptr(q), _ptr(ckv), _ptr(topk_idx), _ptr(win_kv), _ptr(win_pos), _ptr(q_pos), B, Tq,
        n_h, c, N_c, k, L, W, float(scale), _ptr(sink), dtype, _ptr(out), _ptr(lse),
        _ptr(workspace), ws_bytes, _stream(stream)))


def hca_attend_sink(q, ckv, win_kv, win_pos, q_pos, m, B, Tq, n_h, c, N_h, L, W, scale, sink,
                    dtype, out, lse, workspace, ws_bytes, stream=None):
    return _check("hca_attend_sink", load().hca_attend_sink(
        _ptr(q), _ptr(ckv), _ptr(win_kv), _ptr(win_pos), _ptr(q_pos), m, B, Tq, n_h, c, N_h, L, W,
        float(scale), _ptr(sink), dtype, _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
        _stream(stream)))


def csa_attend_ex(q, ckv, topk_idx, win_kv, win_pos, q_pos, B, Tq, n_h, c, N_c, k, L, W, scale,
                  sink, q_gamma, q_norm, d_rope, eps, theta, dtype, out, lse, workspace, ws_bytes,
                  stream=None):
    return _check("csa_attend_ex", load().csa_attend_ex(
        _ptr(q), _ptr(ckv), _ptr(topk_idx), _ptr(win_kv), _ptr(win_pos), _ptr(q_pos), B, Tq,
        n_h, c, N_c, k, L, W, float(scale), _ptr(sink), _ptr(q_gamma), q_norm, d_rope, float(eps),
        float(theta), dtype, _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream)))


def hca_attend_ex(q, ckv, win_kv, win_pos, q_pos, m, B, Tq, n_h, c, N_h, L, W, scale, sink,
                  q_gamma, q_norm, d_rope, eps, theta, dtype, out, lse, workspace, ws_bytes,
                  stream=None):
    return _check("hca_attend_ex", load().hca_attend_ex(
        _ptr(q), _ptr(ckv), _ptr(win_kv), _ptr(win_pos), _ptr(q_pos), m, B, Tq, n_h, c, N_h, L, W,
        float(scale), _ptr(sink), _ptr(q_gamma), q_norm, d_rope, float(eps), float(theta), dtype,
        _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream)))


def csa_attend_begin(q, ckv, topk_idx, win_kv, win_pos, q_pos, B, Tq, n_h, c, N_c, k, L, W, scale,
                     sink, q_gamma, q_norm, d_rope, eps, theta, dtype, out, lse, workspace, ws_bytes,
                     stream=None):
    return _check("csa_attend_begin", load().csa_attend_begin(
        _ptr(q), _ptr(ckv), _ptr(topk_idx), _ptr(win_kv), _ptr(win_pos), _ptr(q_pos), B, Tq,
        n_h, c, N_c, k, L, W, float(scale), _ptr(sink), _ptr(q_gamma), q_norm, d_rope, float(eps),
        float(theta), dtype, _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream)))


def hca_attend_begin(q, ckv, win_kv, win_pos, q_pos, m, B, Tq, n_h, c, N_h, L, W, scale, sink,
                     q_gamma, q_norm, d_rope, eps, theta, dtype, out, lse, workspace, ws_bytes,
                     stream=None):
    return _check("hca_attend_begin", load().hca_attend_begin(
        _ptr(q), _ptr(ckv), _ptr(win_kv), _ptr(win_pos), _ptr(q_pos), m, B, Tq, n_h, c, N_h, L, W,
        float(scale), _ptr(sink), _ptr(q_gamma), q_norm, d_rope, float(eps), float(theta), dtype,
        _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream)))


def csa_attend_end(q, ckv, topk_idx, win_kv, win_pos, q_pos, B, Tq, n_h, c, N_c, k, L, W, scale,
                   sink, q_gamma, q_norm, d_rope, eps, theta, dtype, out, lse, workspace, ws_bytes,
                   stream=None):
    return _check("csa_attend_end", load().csa_attend_end(
        _ptr(q), _ptr(ckv), _ptr(topk_idx), _ptr(win_kv), _ptr(win_pos), _ptr(q_pos), B, Tq,
        n_h, c, N_c, k, L, W, float(scale), _ptr(sink), _ptr(q_gamma), q_norm, d_rope, float(eps),
        float(theta), dtype, _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream)))


def hca_attend_end(q, ckv, win_kv, win_pos, q_pos, m, B, Tq, n_h, c, N_h, L, W, scale, sink,
                   q_gamma, q_norm, d_rope, eps, theta, dtype, out, lse, workspace, ws_bytes,
                   stream=None):
    return _check("hca_attend_end", load().hca_attend_end(
        _ptr(q), _ptr(ckv), _ptr(win_kv), _ptr(win_pos), _ptr(q_pos), m, B, Tq, n_h, c, N_h, L, W,
        float(scale), _ptr(sink), _ptr(q_gamma), q_norm, d_rope, float(eps), float(theta), dtype,
        _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream)))
