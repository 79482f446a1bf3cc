"""fp64 CPU oracle of the gated delta rule -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP library
(``commit_gated_delta_amd``) and never imports it.

The arithmetic lives in ``gdn_oracle.c`` (plain C, fp64, one loop nest per
step of the rule; OpenMP only across independent chains).  This module builds
it with gcc, loads it with ctypes and marshals numpy arrays.

What is computed (see the C file for the passage-by-passage account):
  * the gated delta rule of Yang, Kautz & Hatamizadeh, "Gated Delta Networks"
    (ICLR 2025), Sec. 3, with alpha = exp(g), optional L2 normalisation of q
    and k (eps = 1e-6 added to the sum of squares) and o_t = scale * S_t q_t;
  * commit(m) of the NInfer technical review (blog.123qwe.co.kr post 4624,
    section "Architecture 3: speculative decoding and ReplaySSM"): the state
    after the first m window steps from the untouched S_0;
  * prefill over a whole sequence with a state copy at every multiple of the
    checkpoint interval (same review, section "Architecture 2", the
    context_cache.checkpoint_interval setting);
  * draft-tree windows (the first page: draft trees with DFlash2): node t
    steps from its parent's state, and a commit replays an accepted
    root-to-node path from S_0;
  * KDA, the sibling rule with a per-key-channel decay (Kimi Delta
    Attention; the review names its state and a kda_replay contract);
  * snapshot / restore of the recurrent state of chosen lanes (same section:
    paused requests come back by replay or from a snapshot) -- exact copies,
    written here as numpy indexing.

Pins: every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_pins.py`` (closed forms, exact-rational brute force,
an autograd derivation of the delta rule, invariants) -- none is unpinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB_DIR = os.path.join(_HERE, "_build")
_LIB = os.path.join(_LIB_DIR, "liboracle.so")

EPS = 1e-6


def build(force: bool = True) -> str:
    """Compile gdn_oracle.c into oracle/_build/liboracle.so with gcc."""
    if not force and os.path.exists(_LIB):
        return _LIB
    os.makedirs(_LIB_DIR, exist_ok=True)
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-fno-fast-math", "-ffp-contract=off", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int32)
        i = ctypes.c_int
        lib.oracle_verify.argtypes = [i] * 7 + [ip] + [dp] * 6 + [
            ctypes.c_double, i, dp, dp]
        lib.oracle_verify.restype = i
        lib.oracle_commit.argtypes = [i] * 7 + [ip] + [dp] * 6 + [i]
        lib.oracle_commit.restype = i
        lib.oracle_verify_tree.argtypes = [i] * 7 + [ip, ip] + [dp] * 6 + [
            ctypes.c_double, i, dp, dp]
        lib.oracle_verify_tree.restype = i
        lib.oracle_commit_path.argtypes = [i] * 7 + [ip, ip] + [dp] * 6 + [i]
        lib.oracle_commit_path.restype = i
        lib.oracle_kda.argtypes = [i] * 7 + [ip, ip] + [dp] * 6 + [
            ctypes.c_double, i, dp, dp]
        lib.oracle_kda.restype = i
        lib.oracle_prefill.argtypes = [i] * 6 + [dp] * 6 + [
            ctypes.c_double, i, dp, dp, dp]
        lib.oracle_prefill.restype = i
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = i
        lib.oracle_set_num_threads.argtypes = [i]
        lib.oracle_set_num_threads.restype = None
        _lib = lib
    return _lib


def use_library(path):
    """Load the oracle from another build of gdn_oracle.c (the mutation test
    uses this to check that the pins reject planted mistakes).  Returns the
    previously loaded library handle so that it can be restored."""
    global _lib
    old = _load()
    _lib = None
    saved = globals()["_LIB"]
    globals()["_LIB"] = path
    try:
        _load()
    finally:
        globals()["_LIB"] = saved
    return old


def restore_library(handle):
    global _lib
    _lib = handle


def _d(a):
    """Contiguous float64 view/copy and its ctypes pointer."""
    a = np.ascontiguousarray(a, dtype=np.float64)
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the OpenMP loops over independent chains."""
    _load().oracle_set_num_threads(int(n))


def verify(q, k, v, beta, g, S0, t_lane, scale=1.0, l2norm=True,
           want_states=False):
    """Window verify.  Shapes:
      q, k  [NL, N, T, Hk, dk]; v [NL, N, T, Hv, dv]; beta, g [NL, N, T, Hv]
      S0    [NL, N, Hv, dk, dv]; t_lane [N] in 0..T
    Returns (o [NL, N, T, Hv, dv], states [NL, N, T, Hv, dk, dv] or None).
    Rows t >= t_lane of o (and states) are zero."""
    lib = _load()
    NL, N, T, Hk, dk = q.shape
    Hv, dv = v.shape[3], v.shape[4]
    assert k.shape == q.shape and v.shape == (NL, N, T, Hv, dv)
    assert beta.shape == (NL, N, T, Hv) and g.shape == beta.shape
    assert S0.shape == (NL, N, Hv, dk, dv)
    q, qp = _d(q); k, kp = _d(k); v, vp = _d(v)
    beta, bp = _d(beta); g, gp = _d(g); S0, sp = _d(S0)
    tl = np.ascontiguousarray(t_lane, dtype=np.int32)
    o = np.zeros((NL, N, T, Hv, dv))
    states = np.zeros((NL, N, T, Hv, dk, dv)) if want_states else None
    rc = lib.oracle_verify(
        NL, N, Hv, Hk, dk, dv, T, tl.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
        qp, kp, vp, bp, gp, sp, float(scale), int(bool(l2norm)),
        o.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
        states.ctypes.data_as(ctypes.POINTER(ctypes.c_double)) if want_states
        else None)
    if rc != 0:
        raise ValueError("oracle_verify failed: %d" % rc)
    return o, states


def commit(q, k, v, beta, g, S, m_lane, l2norm=True):
    """Commit: returns a new array, S advanced by the first m_lane[n] steps
    of each lane's window (lanes with m = 0 are unchanged)."""
    lib = _load()
    NL, N, T, Hk, dk = q.shape
    Hv, dv = v.shape[3], v.shape[4]
    q, qp = _d(q); k, kp = _d(k); v, vp = _d(v)
    beta, bp = _d(beta); g, gp = _d(g)
    out = np.array(S, dtype=np.float64, copy=True, order="C")
    ml = np.ascontiguousarray(m_lane, dtype=np.int32)
    rc = lib.oracle_commit(
        NL, N, Hv, Hk, dk, dv, T, ml.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
        qp, kp, vp, bp, gp, out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
        int(bool(l2norm)))
    if rc != 0:
        raise ValueError("oracle_commit failed: %d" % rc)
    return out


def verify_tree(q, k, v, beta, g, S0, t_lane, parent, scale=1.0,
                l2norm=True, want_states=False):
    """Draft-tree verify.  Shapes as verify(); parent int [N, T] with
    parent[n][t] in -1..t-1 (-1: the node steps from S0).  Returns
    (o, states or None): node t's output and state after its own step."""
    lib = _load()
    NL, N, T, Hk, dk = q.shape
    Hv, dv = v.shape[3], v.shape[4]
    q, qp = _d(q); k, kp = _d(k); v, vp = _d(v)
    beta, bp = _d(beta); g, gp = _d(g); S0, sp = _d(S0)
    tl = np.ascontiguousarray(t_lane, dtype=np.int32)
    pa = np.ascontiguousarray(parent, dtype=np.int32)
    assert pa.shape == (N, T)
    o = np.zeros((NL, N, T, Hv, dv))
    states = np.zeros((NL, N, T, Hv, dk, dv)) if want_states else None
    ip = ctypes.POINTER(ctypes.c_int32)
    dp = ctypes.POINTER(ctypes.c_double)
    rc = lib.oracle_verify_tree(
        NL, N, Hv, Hk, dk, dv, T, tl.ctypes.data_as(ip), pa.ctypes.data_as(ip),
        qp, kp, vp, bp, gp, sp, float(scale), int(bool(l2norm)),
        o.ctypes.data_as(dp), states.ctypes.data_as(dp) if want_states else None)
    if rc != 0:
        raise ValueError("oracle_verify_tree failed: %d" % rc)
    return o, states


def commit_path(q, k, v, beta, g, S, m_lane, path, l2norm=True):
    """Commit of accepted paths: a new array, S advanced by the steps of
    nodes path[n][0..m_lane[n]-1] of each lane's window, in that order."""
    lib = _load()
    NL, N, T, Hk, dk = q.shape
    Hv, dv = v.shape[3], v.shape[4]
    q, qp = _d(q); k, kp = _d(k); v, vp = _d(v)
    beta, bp = _d(beta); g, gp = _d(g)
    out = np.array(S, dtype=np.float64, copy=True, order="C")
    ml = np.ascontiguousarray(m_lane, dtype=np.int32)
    pa = np.zeros((N, T), dtype=np.int32)
    for n in range(N):
        pa[n, :int(ml[n])] = np.asarray(path[n][:int(ml[n])], dtype=np.int32)
    ip = ctypes.POINTER(ctypes.c_int32)
    rc = lib.oracle_commit_path(
        NL, N, Hv, Hk, dk, dv, T, ml.ctypes.data_as(ip), pa.ctypes.data_as(ip),
        qp, kp, vp, bp, gp, out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
        int(bool(l2norm)))
    if rc != 0:
        raise ValueError("oracle_commit_path failed: %d" % rc)
    return out


def kda_verify(q, k, v, beta, g, S0, t_lane, scale=1.0, l2norm=True,
               want_states=False):
    """KDA window verify.  Shapes as verify() except g [NL, N, T, Hv, dk]
    (log-decay per key channel).  Returns (o, states or None)."""
    lib = _load()
    NL, N, T, Hk, dk = q.shape
    Hv, dv = v.shape[3], v.shape[4]
    assert g.shape == (NL, N, T, Hv, dk)
    q, qp = _d(q); k, kp = _d(k); v, vp = _d(v)
    beta, bp = _d(beta); g, gp = _d(g)
    Sw = np.array(S0, dtype=np.float64, copy=True, order="C")
    tl = np.ascontiguousarray(t_lane, dtype=np.int32)
    o = np.zeros((NL, N, T, Hv, dv))
    states = np.zeros((NL, N, T, Hv, dk, dv)) if want_states else None
    ip = ctypes.POINTER(ctypes.c_int32)
    dp = ctypes.POINTER(ctypes.c_double)
    rc = lib.oracle_kda(NL, N, Hv, Hk, dk, dv, T, tl.ctypes.data_as(ip), None,
                        qp, kp, vp, bp, gp, Sw.ctypes.data_as(dp), float(scale),
                        int(bool(l2norm)), o.ctypes.data_as(dp),
                        states.ctypes.data_as(dp) if want_states else None)
    if rc != 0:
        raise ValueError("oracle_kda failed: %d" % rc)
    return o, states


def kda_commit(q, k, v, beta, g, S, m_lane, l2norm=True):
    """KDA commit: a new array, S advanced by the first m_lane[n] steps."""
    lib = _load()
    NL, N, T, Hk, dk = q.shape
    Hv, dv = v.shape[3], v.shape[4]
    q, qp = _d(q); k, kp = _d(k); v, vp = _d(v)
    beta, bp = _d(beta); g, gp = _d(g)
    out = np.array(S, dtype=np.float64, copy=True, order="C")
    ml = np.ascontiguousarray(m_lane, dtype=np.int32)
    ip = ctypes.POINTER(ctypes.c_int32)
    dp = ctypes.POINTER(ctypes.c_double)
    rc = lib.oracle_kda(NL, N, Hv, Hk, dk, dv, T, ml.ctypes.data_as(ip),
                        ml.ctypes.data_as(ip), qp, kp, vp, bp, gp,
                        out.ctypes.data_as(dp), 1.0, int(bool(l2norm)), None,
                        None)
    if rc != 0:
        raise ValueError("oracle_kda failed: %d" % rc)
    return out


def prefill(q, k, v, beta, g, S_init=None, ckpt_interval=8192, scale=1.0,
            l2norm=True):
    """Whole-sequence prefill.  Shapes: q, k [L, Hk, dk]; v [L, Hv, dv];
    beta, g [L, Hv]; S_init [Hv, dk, dv] or None (zero state).
    Returns (o [L, Hv, dv], ckpts [L // ckpt_interval, Hv, dk, dv], S_final)."""
    lib = _load()
    L, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    q, qp = _d(q); k, kp = _d(k); v, vp = _d(v)
    beta, bp = _d(beta); g, gp = _d(g)
    if S_init is not None:
        S_init, sip = _d(S_init)
    else:
        sip = None
    o = np.zeros((L, Hv, dv))
    n_ck = L // ckpt_interval if ckpt_interval > 0 else 0
    ck = np.zeros((max(n_ck, 0), Hv, dk, dv))
    Sf = np.zeros((Hv, dk, dv))
    dp = ctypes.POINTER(ctypes.c_double)
    rc = lib.oracle_prefill(
        L, Hv, Hk, dk, dv, int(ckpt_interval), qp, kp, vp, bp, gp, sip,
        float(scale), int(bool(l2norm)), o.ctypes.data_as(dp),
        ck.ctypes.data_as(dp) if n_ck > 0 else None, Sf.ctypes.data_as(dp))
    if rc != 0:
        raise ValueError("oracle_prefill failed: %d" % rc)
    return o, ck, Sf


def snapshot(S, lanes):
    """Snapshot of the recurrent state of the chosen lanes (NInfer technical
    review, "Architecture 2": paused requests resume from a snapshot).
    S [NL, N, Hv, dk, dv]; returns [len(lanes), NL, Hv, dk, dv] with entry j
    the state of lane lanes[j] in every layer -- an exact copy."""
    S = np.asarray(S)
    return np.stack([S[:, int(n)] for n in lanes]) if len(lanes) else \
        np.zeros((0,) + S.shape[:1] + S.shape[2:], S.dtype)


def restore(S, lanes, snap):
    """Inverse of snapshot: a copy of S with lane lanes[j] replaced by
    snap[j] in every layer.  A lane may not be listed twice."""
    lanes = [int(n) for n in lanes]
    if len(set(lanes)) != len(lanes):
        raise ValueError("a lane is restored twice")
    out = np.array(S, copy=True)
    for j, n in enumerate(lanes):
        out[:, n] = snap[j]
    return out
