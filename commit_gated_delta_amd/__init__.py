"""Python binding of libgdn.so: gated-delta verify, ReplaySSM commit and
chunked prefill on MI355X (gfx950).

Argument marshalling only: every step of the path runs in the HIP kernels
behind the C ABI declared in ``include/gdn.h``.  torch provides device
memory and streams.  There is no fallback: if the built library is missing,
importing this package raises.

Names follow the C ABI: ``verify``, ``commit``, ``prefill_chunked``,
``records_bytes``, ``prefill_workspace_bytes``.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# GDN_LIBRARY names another build of the same library (the CPU tests load
# a sanitizer build of the host code this way).
LIB_PATH = os.environ.get("GDN_LIBRARY") or os.path.join(_HERE, "_build",
                                                         "libgdn.so")

GDN_OK, GDN_EINVAL, GDN_EUNSUPPORTED, GDN_EWORKSPACE, GDN_EHIP = 0, -1, -2, -3, -4
GDN_BF16, GDN_F32 = 0, 1
GDN_FLAG_L2NORM_QK = 1
GDN_FLAG_PREFILL_ONE_CHAIN = 2
GDN_FLAG_TOKENWISE = 4
GDN_MAX_LANES = 256
GDN_MAX_T = 64

EXPORTED = ("gdn_records_bytes", "gdn_verify", "gdn_commit",
            "gdn_commit_verify", "gdn_verify_tree", "gdn_commit_path",
            "gdn_kda_records_bytes", "gdn_kda_verify", "gdn_kda_commit",
            "gdn_state_snapshot", "gdn_state_restore",
            "gdn_prefill_workspace_bytes", "gdn_prefill_chunked",
            "gdn_prefill_chunked_noalloc", "gdn_strerror", "gdn_last_error")
PREFILL_SCRATCH_BYTES = 64 << 20


class GdnError(RuntimeError):
    def __init__(self, status, what):
        super().__init__("%s: %s (%d): %s" % (
            what, _strerror(status), status, lib.gdn_last_error().decode()))
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("n_lanes", ctypes.c_int32),
                ("h_v", ctypes.c_int32), ("h_k", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("t_max", ctypes.c_int32)]

    @classmethod
    def of(cls, n_layers, n_lanes, h_v, h_k, d_k, d_v, t_max):
        return cls(n_layers, n_lanes, h_v, h_k, d_k, d_v, t_max)


def _load_library():
    # torch ships its own HIP runtime (libamdhip64.so.7).  Load it first so
    # that libgdn.so binds to the same runtime instance as the streams and
    # device memory it is handed; a second runtime in the process would not
    # see torch's device state.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            "libgdn.so is not built (%s); run commit_gated_delta_amd/build.py "
            "or __graft_entry__.build()" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
    ip = ctypes.POINTER(ctypes.c_int32)
    dp = ctypes.POINTER(Dims)
    f = ctypes.c_float
    lib.gdn_records_bytes.argtypes = [dp]
    lib.gdn_records_bytes.restype = sz
    lib.gdn_verify.argtypes = [dp, ip, vp, vp, vp, ctypes.c_int, vp, vp, vp,
                               vp, vp, vp, f, ctypes.c_int, vp]
    lib.gdn_verify.restype = ctypes.c_int
    lib.gdn_commit.argtypes = [dp, ip, ip, vp, vp, vp]
    lib.gdn_commit.restype = ctypes.c_int
    lib.gdn_commit_verify.argtypes = [dp, ip, ip, vp, ip, vp, vp, vp,
                                      ctypes.c_int, vp, vp, vp, vp, vp, vp, f,
                                      ctypes.c_int, vp]
    lib.gdn_commit_verify.restype = ctypes.c_int
    lib.gdn_kda_records_bytes.argtypes = [dp]
    lib.gdn_kda_records_bytes.restype = sz
    lib.gdn_kda_verify.argtypes = lib.gdn_verify.argtypes
    lib.gdn_kda_verify.restype = ctypes.c_int
    lib.gdn_kda_commit.argtypes = lib.gdn_commit.argtypes
    lib.gdn_kda_commit.restype = ctypes.c_int
    lib.gdn_verify_tree.argtypes = [dp, ip, ip, vp, vp, vp, ctypes.c_int, vp,
                                    vp, vp, vp, vp, vp, f, ctypes.c_int, vp]
    lib.gdn_verify_tree.restype = ctypes.c_int
    lib.gdn_commit_path.argtypes = [dp, ip, ip, ip, ip, vp, vp, vp]
    lib.gdn_commit_path.restype = ctypes.c_int
    for fn in (lib.gdn_state_snapshot, lib.gdn_state_restore):
        fn.argtypes = [dp, i32, ip, vp, vp, vp]
        fn.restype = ctypes.c_int
    lib.gdn_prefill_workspace_bytes.argtypes = [i32] * 7
    lib.gdn_prefill_workspace_bytes.restype = sz
    lib.gdn_prefill_chunked.argtypes = [i32] * 8 + [vp] * 3 + [ctypes.c_int] + [
        vp] * 7 + [sz, f, ctypes.c_int, vp]
    lib.gdn_prefill_chunked.restype = ctypes.c_int
    lib.gdn_prefill_chunked_noalloc.argtypes = [i32] * 8 + [vp] * 3 + [
        ctypes.c_int] + [vp] * 6 + [f, ctypes.c_int, vp]
    lib.gdn_prefill_chunked_noalloc.restype = ctypes.c_int
    lib.gdn_strerror.argtypes = [ctypes.c_int]
    lib.gdn_strerror.restype = ctypes.c_char_p
    lib.gdn_last_error.argtypes = []
    lib.gdn_last_error.restype = ctypes.c_char_p
    return lib


lib = _load_library()


def _strerror(status):
    return lib.gdn_strerror(int(status)).decode()


def _check(status, what):
    if status != GDN_OK:
        raise GdnError(status, what)


def _ptr(t):
    """Device (or host) address of a tensor, or None."""
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _int_array(values, n):
    vals = [int(x) for x in values]
    if len(vals) != n:
        raise ValueError("expected %d per-lane values, got %d" % (n, len(vals)))
    return (ctypes.c_int32 * n)(*vals)


def _dtype_code(t):
    import torch
    if t is None:       # the C ABI reports the null pointer
        return GDN_BF16
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_F32
    raise TypeError("q/k/v must be bfloat16 or float32, got %s" % t.dtype)


def _stream(stream):
    """hipStream_t handle: torch's current stream by default, a
    torch.cuda.Stream, or a raw integer handle (0 = the null stream)."""
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def records_bytes(dims: Dims) -> int:
    return int(lib.gdn_records_bytes(ctypes.byref(dims)))


def _verify_flags(l2norm, tokenwise):
    return ((GDN_FLAG_L2NORM_QK if l2norm else 0) |
            (GDN_FLAG_TOKENWISE if tokenwise else 0))


def verify(dims: Dims, t_lane, q, k, v, beta, g, S, o, records,
           dbg_states=None, scale=1.0, l2norm=True, stream=None,
           raw_status=False, tokenwise=False):
    """gdn_verify on torch tensors (layouts in include/gdn.h;
    tokenwise=True sets GDN_FLAG_TOKENWISE)."""
    st = lib.gdn_verify(ctypes.byref(dims), _int_array(t_lane, dims.n_lanes),
                        _ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(beta),
                        _ptr(g), _ptr(S), _ptr(o), _ptr(records),
                        _ptr(dbg_states), float(scale),
                        _verify_flags(l2norm, tokenwise), _stream(stream))
    if raw_status:
        return st
    _check(st, "gdn_verify")


def commit(dims: Dims, m_lane, t_lane, records, S, stream=None,
           raw_status=False):
    """gdn_commit on torch tensors."""
    st = lib.gdn_commit(ctypes.byref(dims), _int_array(m_lane, dims.n_lanes),
                        _int_array(t_lane, dims.n_lanes), _ptr(records),
                        _ptr(S), _stream(stream))
    if raw_status:
        return st
    _check(st, "gdn_commit")


def commit_verify(dims: Dims, m_prev, t_prev, records_prev, t_lane, q, k, v,
                  beta, g, S, o, records, dbg_states=None, scale=1.0,
                  l2norm=True, stream=None, raw_status=False, tokenwise=False):
    """gdn_commit_verify on torch tensors: commit(m_prev) of the previous
    window's records, then verify of the new window, in one launch."""
    st = lib.gdn_commit_verify(
        ctypes.byref(dims), _int_array(m_prev, dims.n_lanes),
        _int_array(t_prev, dims.n_lanes), _ptr(records_prev),
        _int_array(t_lane, dims.n_lanes), _ptr(q), _ptr(k), _ptr(v),
        _dtype_code(q), _ptr(beta), _ptr(g), _ptr(S), _ptr(o), _ptr(records),
        _ptr(dbg_states), float(scale), _verify_flags(l2norm, tokenwise),
        _stream(stream))
    if raw_status:
        return st
    _check(st, "gdn_commit_verify")


def kda_records_bytes(dims: Dims) -> int:
    return int(lib.gdn_kda_records_bytes(ctypes.byref(dims)))


def kda_verify(dims: Dims, t_lane, q, k, v, beta, g, S, o, records,
               dbg_states=None, scale=1.0, l2norm=True, stream=None,
               raw_status=False, tokenwise=False):
    """gdn_kda_verify; g is [NL][N][T][Hv][d_k] (per-channel log-decay)."""
    st = lib.gdn_kda_verify(ctypes.byref(dims), _int_array(t_lane, dims.n_lanes),
                            _ptr(q), _ptr(k), _ptr(v), _dtype_code(q),
                            _ptr(beta), _ptr(g), _ptr(S), _ptr(o),
                            _ptr(records), _ptr(dbg_states), float(scale),
                            _verify_flags(l2norm, tokenwise),
                            _stream(stream))
    if raw_status:
        return st
    _check(st, "gdn_kda_verify")


def kda_commit(dims: Dims, m_lane, t_lane, records, S, stream=None,
               raw_status=False):
    st = lib.gdn_kda_commit(ctypes.byref(dims), _int_array(m_lane, dims.n_lanes),
                            _int_array(t_lane, dims.n_lanes), _ptr(records),
                            _ptr(S), _stream(stream))
    if raw_status:
        return st
    _check(st, "gdn_kda_commit")


def _table(rows, n, t_max, fill):
    """int32 [n][t_max] from per-lane sequences (padded with ``fill``)."""
    import numpy as np
    a = np.full((n, t_max), fill, dtype=np.int32)
    if len(rows) != n:
        raise ValueError("expected %d per-lane rows, got %d" % (n, len(rows)))
    for i, r in enumerate(rows):
        r = [int(x) for x in r]
        a[i, :len(r)] = r
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def verify_tree(dims: Dims, t_lane, parent, q, k, v, beta, g, S, o, records,
                dbg_states=None, scale=1.0, l2norm=True, stream=None,
                raw_status=False, tokenwise=False):
    """gdn_verify_tree; parent is [n_lanes][<= t_max] (-1: from S0)."""
    keep, pp = _table(parent, dims.n_lanes, dims.t_max, -1)
    st = lib.gdn_verify_tree(
        ctypes.byref(dims), _int_array(t_lane, dims.n_lanes), pp, _ptr(q),
        _ptr(k), _ptr(v), _dtype_code(q), _ptr(beta), _ptr(g), _ptr(S),
        _ptr(o), _ptr(records), _ptr(dbg_states), float(scale),
        _verify_flags(l2norm, tokenwise), _stream(stream))
    del keep
    if raw_status:
        return st
    _check(st, "gdn_verify_tree")


def commit_path(dims: Dims, paths, t_lane, parent, records, S, stream=None,
                raw_status=False):
    """gdn_commit_path; paths[n] lists the accepted nodes of lane n, root
    first (empty: nothing accepted)."""
    keep_p, pp = _table(paths, dims.n_lanes, dims.t_max, 0)
    keep_t, tp = _table(parent, dims.n_lanes, dims.t_max, -1)
    m = [len(p) for p in paths]
    st = lib.gdn_commit_path(ctypes.byref(dims), _int_array(m, dims.n_lanes),
                             pp, _int_array(t_lane, dims.n_lanes), tp,
                             _ptr(records), _ptr(S), _stream(stream))
    del keep_p, keep_t
    if raw_status:
        return st
    _check(st, "gdn_commit_path")


def _lane_list(lanes):
    vals = [int(x) for x in lanes]
    return len(vals), (ctypes.c_int32 * max(len(vals), 1))(*vals)


def state_snapshot(dims: Dims, lanes, S, snapshot, stream=None,
                   raw_status=False):
    """gdn_state_snapshot: snapshot[j] = S[:, lanes[j]] (device or pinned
    host tensor)."""
    n, arr = _lane_list(lanes)
    st = lib.gdn_state_snapshot(ctypes.byref(dims), n, arr, _ptr(S),
                                _ptr(snapshot), _stream(stream))
    if raw_status:
        return st
    _check(st, "gdn_state_snapshot")


def state_restore(dims: Dims, lanes, snapshot, S, stream=None,
                  raw_status=False):
    """gdn_state_restore: S[:, lanes[j]] = snapshot[j]."""
    n, arr = _lane_list(lanes)
    st = lib.gdn_state_restore(ctypes.byref(dims), n, arr, _ptr(snapshot),
                               _ptr(S), _stream(stream))
    if raw_status:
        return st
    _check(st, "gdn_state_restore")


def prefill_workspace_bytes(n_seqs, seq_len, h_v, h_k, d_k, d_v,
                            chunk=64) -> int:
    return int(lib.gdn_prefill_workspace_bytes(n_seqs, seq_len, h_v, h_k, d_k,
                                               d_v, chunk))


def _prefill_flags(l2norm, segments):
    return ((GDN_FLAG_L2NORM_QK if l2norm else 0) |
            (0 if segments else GDN_FLAG_PREFILL_ONE_CHAIN))


def prefill_chunked(n_seqs, seq_len, h_v, h_k, d_k, d_v, q, k, v, beta, g,
                    S_init, S_final, o, checkpoints, workspace,
                    ckpt_interval=8192, scale=1.0, l2norm=True, stream=None,
                    raw_status=False, chunk=64, segments=True):
    """gdn_prefill_chunked on torch tensors (segments=False sets
    GDN_FLAG_PREFILL_ONE_CHAIN)."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.gdn_prefill_chunked(
        n_seqs, seq_len, h_v, h_k, d_k, d_v, chunk, ckpt_interval, _ptr(q),
        _ptr(k), _ptr(v), _dtype_code(q), _ptr(beta), _ptr(g), _ptr(S_init),
        _ptr(S_final), _ptr(o), _ptr(checkpoints), _ptr(workspace), ws_bytes,
        float(scale), _prefill_flags(l2norm, segments), _stream(stream))
    if raw_status:
        return st
    _check(st, "gdn_prefill_chunked")


def prefill_chunked_noalloc(n_seqs, seq_len, h_v, h_k, d_k, d_v, q, k, v,
                            beta, g, S_init, S_final, o, checkpoints,
                            ckpt_interval=8192, scale=1.0, l2norm=True,
                            stream=None, raw_status=False, chunk=64,
                            segments=True):
    """gdn_prefill_chunked_noalloc: the prefill with the library's fixed
    scratch array as its workspace (no allocation; calls that overlap on
    one GPU race)."""
    st = lib.gdn_prefill_chunked_noalloc(
        n_seqs, seq_len, h_v, h_k, d_k, d_v, chunk, ckpt_interval, _ptr(q),
        _ptr(k), _ptr(v), _dtype_code(q), _ptr(beta), _ptr(g), _ptr(S_init),
        _ptr(S_final), _ptr(o), _ptr(checkpoints), float(scale),
        _prefill_flags(l2norm, segments), _stream(stream))
    if raw_status:
        return st
    _check(st, "gdn_prefill_chunked_noalloc")
