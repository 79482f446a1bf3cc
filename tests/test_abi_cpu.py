"""The C ABI without a GPU: the library loads, exports every symbol that
include/gdn.h declares, and rejects bad arguments on the host with a status
code before any HIP call (so these calls are safe on a machine with no GPU).
"""
import ctypes
import os
import re

import numpy as np
import pytest

import commit_gated_delta_amd as gdn

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include",
                      "gdn.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", text)))


def test_header_declares_exactly_the_exported_set():
    assert _declared() == sorted(gdn.EXPORTED)


@pytest.mark.parametrize("sym", sorted(gdn.EXPORTED))
def test_symbol_exported(sym):
    assert hasattr(gdn.lib, sym)
    assert ctypes.cast(getattr(gdn.lib, sym), ctypes.c_void_p).value


def test_strerror():
    for st in (0, -1, -2, -3, -4, 17):
        assert isinstance(gdn.lib.gdn_strerror(st), bytes)


def _dims(**kw):
    base = dict(n_layers=1, n_lanes=2, h_v=4, h_k=2, d_k=128, d_v=128, t_max=8)
    base.update(kw)
    return gdn.Dims.of(**base)


def test_records_bytes():
    d = _dims()
    n = gdn.records_bytes(d)
    ntok = 1 * 2 * 8
    # raw key rows (f32 [h_k][d_k]) + ut (f32 [h_v][d_v]) + (fold, c)
    # (float2 [h_v])
    assert n >= ntok * (2 * 128 * 4 + 4 * 128 * 4 + 4 * 8)
    assert n < ntok * (2 * 128 * 4 + 4 * 128 * 4 + 4 * 8) + 3 * 256
    assert n % 256 == 0
    assert gdn.records_bytes(_dims(d_k=24)) == 0
    assert gdn.records_bytes(_dims(h_v=3)) == 0
    assert gdn.records_bytes(_dims(t_max=65)) == 0
    assert gdn.records_bytes(_dims(n_lanes=257)) == 0


class _Fake:
    """Stands in for a tensor: a 256-aligned host address, never touched
    because every call below is rejected before any memory access."""

    def __init__(self, dtype_code=gdn.GDN_BF16, addr=1 << 20):
        self.addr = addr
        import torch
        self.dtype = torch.bfloat16 if dtype_code == gdn.GDN_BF16 else torch.float32

    def data_ptr(self):
        return self.addr


def _verify(d, t_lane, **over):
    a = dict(q=_Fake(), k=_Fake(), v=_Fake(), beta=_Fake(gdn.GDN_F32),
             g=_Fake(gdn.GDN_F32), S=_Fake(gdn.GDN_F32), o=_Fake(gdn.GDN_F32),
             rec=_Fake(gdn.GDN_F32))
    a.update(over)
    return gdn.verify(d, t_lane, a["q"], a["k"], a["v"], a["beta"], a["g"],
                      a["S"], a["o"], a["rec"], stream=0, raw_status=True)


def test_verify_rejects_bad_arguments_on_host():
    d = _dims()
    assert _verify(_dims(d_k=24), [1, 1]) == gdn.GDN_EUNSUPPORTED
    assert _verify(_dims(h_v=3), [1, 1]) == gdn.GDN_EINVAL
    assert _verify(_dims(t_max=0), [1, 1]) == gdn.GDN_EINVAL
    assert _verify(_dims(t_max=65), [1, 1]) == gdn.GDN_EINVAL
    assert _verify(_dims(d_v=0), [1, 1]) == gdn.GDN_EINVAL
    assert _verify(_dims(d_v=1025), [1, 1]) == gdn.GDN_EINVAL
    assert _verify(d, [9, 1]) == gdn.GDN_EINVAL          # T > t_max
    assert _verify(d, [-1, 1]) == gdn.GDN_EINVAL
    assert _verify(d, [1, 1], q=None) == gdn.GDN_EINVAL
    assert _verify(d, [1, 1], rec=None) == gdn.GDN_EINVAL
    assert _verify(d, [1, 1], S=_Fake(gdn.GDN_F32, addr=(1 << 20) + 2)) == gdn.GDN_EINVAL
    assert _verify(d, [1, 1], rec=_Fake(gdn.GDN_F32, addr=(1 << 20) + 16)) == gdn.GDN_EINVAL
    # unknown flag bits
    st = gdn.lib.gdn_verify(ctypes.byref(d), (ctypes.c_int32 * 2)(1, 1),
                            *[ctypes.c_void_p(1 << 20)] * 3, gdn.GDN_BF16,
                            *[ctypes.c_void_p(1 << 20)] * 5, None,
                            ctypes.c_float(1.0), 6, None)
    assert st == gdn.GDN_EINVAL
    st = gdn.lib.gdn_verify(ctypes.byref(d), (ctypes.c_int32 * 2)(1, 1),
                            *[ctypes.c_void_p(1 << 20)] * 3, gdn.GDN_BF16,
                            *[ctypes.c_void_p(1 << 20)] * 5, None,
                            ctypes.c_float(1.0), 8, None)
    assert st == gdn.GDN_EINVAL
    # the norm and token-by-token flags are accepted (idle lanes: no launch)
    st = gdn.lib.gdn_verify(ctypes.byref(d), (ctypes.c_int32 * 2)(0, 0),
                            *[ctypes.c_void_p(1 << 20)] * 3, gdn.GDN_BF16,
                            *[ctypes.c_void_p(1 << 20)] * 5, None,
                            ctypes.c_float(1.0),
                            gdn.GDN_FLAG_L2NORM_QK | gdn.GDN_FLAG_TOKENWISE, None)
    assert st == gdn.GDN_OK
    # unknown dtype
    st = gdn.lib.gdn_verify(ctypes.byref(d), (ctypes.c_int32 * 2)(1, 1),
                            *[ctypes.c_void_p(1 << 20)] * 3, 7,
                            *[ctypes.c_void_p(1 << 20)] * 5, None,
                            ctypes.c_float(1.0), 1, None)
    assert st == gdn.GDN_EINVAL


def test_verify_with_only_idle_lanes_does_nothing():
    # t_lane all zero: valid, nothing to launch, returns OK without HIP
    assert _verify(_dims(), [0, 0]) == gdn.GDN_OK


def test_commit_rejects_bad_arguments_on_host():
    d = _dims()
    rec, S = _Fake(gdn.GDN_F32), _Fake(gdn.GDN_F32)
    c = lambda m, t, **kw: gdn.commit(kw.get("d", d), m, t, kw.get("rec", rec),
                                      kw.get("S", S), stream=0,
                                      raw_status=True)
    assert c([3, 1], [2, 1]) == gdn.GDN_EINVAL     # m > T
    assert c([-1, 0], [2, 1]) == gdn.GDN_EINVAL
    assert c([0, 0], [9, 1]) == gdn.GDN_EINVAL     # T > t_max
    assert c([0, 0], [2, 1], d=_dims(d_k=8)) == gdn.GDN_EUNSUPPORTED
    assert c([1, 0], [2, 1], rec=None) == gdn.GDN_EINVAL
    assert c([1, 0], [2, 1], S=_Fake(gdn.GDN_F32, addr=(1 << 20) + 1)) == gdn.GDN_EINVAL
    # every m = 0: a cancelled round, nothing is launched
    assert c([0, 0], [2, 1]) == gdn.GDN_OK


def _commit_verify(d, m_prev, t_prev, t_lane, **over):
    a = dict(rec_prev=_Fake(gdn.GDN_F32, addr=1 << 30), q=_Fake(), k=_Fake(),
             v=_Fake(), beta=_Fake(gdn.GDN_F32), g=_Fake(gdn.GDN_F32),
             S=_Fake(gdn.GDN_F32), o=_Fake(gdn.GDN_F32),
             rec=_Fake(gdn.GDN_F32))
    a.update(over)
    return gdn.commit_verify(d, m_prev, t_prev, a["rec_prev"], t_lane, a["q"],
                             a["k"], a["v"], a["beta"], a["g"], a["S"],
                             a["o"], a["rec"], stream=0, raw_status=True)


def test_commit_verify_rejects_bad_arguments_on_host():
    d = _dims()
    cv = _commit_verify
    assert cv(d, [3, 1], [2, 1], [1, 1]) == gdn.GDN_EINVAL    # m > t_prev
    assert cv(d, [0, 0], [9, 1], [1, 1]) == gdn.GDN_EINVAL    # t_prev > t_max
    assert cv(d, [0, 0], [2, 1], [9, 1]) == gdn.GDN_EINVAL    # T > t_max
    assert cv(_dims(d_k=24), [0, 0], [2, 1], [1, 1]) == gdn.GDN_EUNSUPPORTED
    assert cv(d, [1, 0], [2, 1], [1, 1], rec_prev=None) == gdn.GDN_EINVAL
    assert cv(d, [1, 0], [2, 1], [1, 1], q=None) == gdn.GDN_EINVAL
    assert cv(d, [1, 0], [2, 1], [1, 1],
              rec_prev=_Fake(gdn.GDN_F32, addr=(1 << 30) + 8)) == gdn.GDN_EINVAL
    # the two record buffers overlap
    n = gdn.records_bytes(d)
    assert cv(d, [1, 0], [2, 1], [1, 1],
              rec_prev=_Fake(gdn.GDN_F32, addr=(1 << 20) + 256 * (n // 512))
              ) == gdn.GDN_EINVAL
    assert "overlap" in gdn.lib.gdn_last_error().decode()
    # nothing to commit or verify: no launch
    assert cv(d, [0, 0], [2, 1], [0, 0], rec_prev=None) == gdn.GDN_OK


def test_kda_calls_reject_bad_arguments_on_host():
    d = _dims()
    n = gdn.kda_records_bytes(d)
    ntok = 1 * 2 * 8
    # raw keys f32 [h_k][d_k] + ut f32 [h_v][d_v] + alpha f32 [h_v][d_k]
    assert n >= ntok * (2 * 128 * 4 + 4 * 128 * 4 + 4 * 128 * 4)
    assert n % 256 == 0
    assert gdn.kda_records_bytes(_dims(d_k=64)) == 0
    f = dict(q=_Fake(), k=_Fake(), v=_Fake(), beta=_Fake(gdn.GDN_F32),
             g=_Fake(gdn.GDN_F32), S=_Fake(gdn.GDN_F32), o=_Fake(gdn.GDN_F32),
             rec=_Fake(gdn.GDN_F32))

    def kv(dims, t, **over):
        a = dict(f)
        a.update(over)
        return gdn.kda_verify(dims, t, a["q"], a["k"], a["v"], a["beta"],
                              a["g"], a["S"], a["o"], a["rec"], stream=0,
                              raw_status=True)

    assert kv(_dims(d_k=64), [1, 1]) == gdn.GDN_EUNSUPPORTED
    assert kv(d, [9, 1]) == gdn.GDN_EINVAL
    assert kv(d, [1, 1], g=None) == gdn.GDN_EINVAL
    assert kv(d, [0, 0]) == gdn.GDN_OK
    kc = lambda m, t, dims=d: gdn.kda_commit(dims, m, t, f["rec"], f["S"],
                                             stream=0, raw_status=True)
    assert kc([3, 0], [2, 1]) == gdn.GDN_EINVAL
    assert kc([0, 0], [2, 1], _dims(d_k=32)) == gdn.GDN_EUNSUPPORTED
    assert kc([0, 0], [2, 1]) == gdn.GDN_OK


def test_tree_calls_reject_bad_arguments_on_host():
    d = _dims(n_lanes=2, t_max=4)
    a = dict(q=_Fake(), k=_Fake(), v=_Fake(), beta=_Fake(gdn.GDN_F32),
             g=_Fake(gdn.GDN_F32), S=_Fake(gdn.GDN_F32), o=_Fake(gdn.GDN_F32),
             rec=_Fake(gdn.GDN_F32))

    def vt(parent, t=(4, 3), dims=d):
        return gdn.verify_tree(dims, t, parent, a["q"], a["k"], a["v"],
                               a["beta"], a["g"], a["S"], a["o"], a["rec"],
                               stream=0, raw_status=True)

    good = [[-1, 0, 0, 2], [-1, 0, 1]]
    assert vt([[-1, 0, 3, 2], [-1, 0, 1]]) == gdn.GDN_EINVAL   # parent after child
    assert vt([[-1, 0, 0, 2], [-1, -2, 1]]) == gdn.GDN_EINVAL  # below -1
    assert vt(good, dims=_dims(n_lanes=2, t_max=33)) == gdn.GDN_EUNSUPPORTED
    assert vt(good, t=(0, 0)) == gdn.GDN_OK                    # nothing to run

    def cp(paths, t=(4, 3), parent=good):
        return gdn.commit_path(d, paths, t, parent, a["rec"], a["S"], stream=0,
                               raw_status=True)

    assert cp([[1, 2], []]) == gdn.GDN_EINVAL       # does not start at a root
    assert cp([[0, 1, 3], []]) == gdn.GDN_EINVAL    # 3's parent is 2, not 1
    assert cp([[], [0, 1, 2, 0]]) == gdn.GDN_EINVAL  # m > t_lane
    assert cp([[], []]) == gdn.GDN_OK


def test_state_copy_rejects_bad_arguments_on_host():
    d = _dims(n_lanes=4)
    S, snap = _Fake(gdn.GDN_F32), _Fake(gdn.GDN_F32, addr=1 << 30)
    for fn in (gdn.state_snapshot, gdn.state_restore):
        assert fn(d, [0, 4], S, snap, stream=0, raw_status=True) == gdn.GDN_EINVAL
        assert fn(d, [-1], S, snap, stream=0, raw_status=True) == gdn.GDN_EINVAL
        assert fn(d, [0, 1, 2, 3, 0], S, snap, stream=0,
                  raw_status=True) == gdn.GDN_EINVAL            # n_sel > n_lanes
        assert fn(d, [1], None, snap, stream=0, raw_status=True) == gdn.GDN_EINVAL
        assert fn(d, [1], S, _Fake(gdn.GDN_F32, addr=(1 << 30) + 8), stream=0,
                  raw_status=True) == gdn.GDN_EINVAL            # alignment
        assert fn(d, [], S, snap, stream=0, raw_status=True) == gdn.GDN_OK
    # restoring one lane twice would race
    assert gdn.state_restore(d, [2, 2], snap, S, stream=0,
                             raw_status=True) == gdn.GDN_EINVAL
    assert "twice" in gdn.lib.gdn_last_error().decode()


def test_binding_checks_lane_count():
    with pytest.raises(ValueError):
        _verify(_dims(), [1, 1, 1])


def test_prefill_workspace_bytes():
    n = gdn.prefill_workspace_bytes(1, 32768, 32, 32, 128, 128)
    # per (chunk, head): the nonzero 16 x 32 blocks of the lower-triangular
    # T and P (6 each) as split bf16 (hi, lo: 1 KiB per fragment), four row
    # vectors of 64 floats and gamma_63
    assert n >= 512 * 32 * (2 * 6 * 2 * 1024 + 4 * 64 * 4 + 4)
    assert gdn.prefill_workspace_bytes(1, 100, 4, 3, 128, 128) == 0   # h_v % h_k
    assert gdn.prefill_workspace_bytes(1, 100, 4, 4, 64, 64) == 0     # d != 128
    assert gdn.prefill_workspace_bytes(0, 100, 4, 4, 128, 128) == 0
    # the same per-chunk block for every chunk length: 16-token chunks need
    # four times the blocks of 64-token chunks
    assert (gdn.prefill_workspace_bytes(1, 4096, 2, 2, 128, 128, 16) ==
            4 * gdn.prefill_workspace_bytes(1, 4096, 2, 2, 128, 128, 64))
    assert gdn.prefill_workspace_bytes(1, 100, 4, 4, 128, 128, 48) == 0
    assert gdn.prefill_workspace_bytes(1, 100, 4, 4, 128, 128, 0) == 0
    # sequences of more than 4,096 tokens, at most 8 sequence-heads, may run
    # in segments: room for each segment's transition and offset (all but the
    # last), and the start and end state of every segment (64 KiB per head)
    L, H = 3 * 4096 + 1000, 4
    per_chunk = gdn.prefill_workspace_bytes(1, 4096, 32, 32, 128, 128) // (64 * 32)
    p1 = (L + 63) // 64 * H * per_chunk
    seg = ((p1 + 255) // 256 * 256) + (2 * 3 + 2 * 4) * H * 65536
    assert gdn.prefill_workspace_bytes(1, L, H, H, 128, 128) == seg
    # several sequences: the same per sequence (sequences x heads <= 8)
    p1_2 = 2 * p1
    assert (gdn.prefill_workspace_bytes(2, L, H, H, 128, 128) ==
            ((p1_2 + 255) // 256 * 256) + 2 * (2 * 3 + 2 * 4) * H * 65536)
    # not for more than 8 sequence-heads, or one segment
    assert (gdn.prefill_workspace_bytes(3, L, H, H, 128, 128) ==
            3 * ((L + 63) // 64) * H * per_chunk)
    assert (gdn.prefill_workspace_bytes(1, L, 16, 16, 128, 128) ==
            (L + 63) // 64 * 16 * per_chunk)
    assert (gdn.prefill_workspace_bytes(1, 4096, H, H, 128, 128) ==
            64 * H * per_chunk)


def _prefill(**over):
    a = dict(n_seqs=1, L=256, hv=2, hk=1, dk=128, dv=128, interval=128,
             q=_Fake(), k=_Fake(), v=_Fake(), beta=_Fake(gdn.GDN_F32),
             g=_Fake(gdn.GDN_F32), Si=None, Sf=_Fake(gdn.GDN_F32),
             o=_Fake(gdn.GDN_F32), ck=_Fake(gdn.GDN_F32), ws_bytes=1 << 30)

    class _WS(_Fake):
        def __init__(self, nbytes):
            super().__init__(gdn.GDN_F32)
            self.nb = nbytes

        def numel(self):
            return self.nb

        def element_size(self):
            return 1

    a.update(over)
    return gdn.prefill_chunked(a["n_seqs"], a["L"], a["hv"], a["hk"], a["dk"],
                               a["dv"], a["q"], a["k"], a["v"], a["beta"],
                               a["g"], a["Si"], a["Sf"], a["o"], a["ck"],
                               _WS(a["ws_bytes"]),
                               ckpt_interval=a["interval"], stream=0,
                               raw_status=True, chunk=a.get("chunk", 64),
                               segments=a.get("segments", True))


def test_prefill_rejects_bad_arguments_on_host():
    assert _prefill(dk=64, dv=64) == gdn.GDN_EUNSUPPORTED
    assert _prefill(hv=3, hk=2) == gdn.GDN_EINVAL
    assert _prefill(L=0) == gdn.GDN_EINVAL
    assert _prefill(interval=100) == gdn.GDN_EINVAL      # not a multiple of 64
    assert _prefill(interval=0) == gdn.GDN_EINVAL
    assert _prefill(q=_Fake(gdn.GDN_F32), k=_Fake(gdn.GDN_F32),
                    v=_Fake(gdn.GDN_F32)) == gdn.GDN_EUNSUPPORTED
    assert _prefill(o=None) == gdn.GDN_EINVAL
    assert _prefill(ws_bytes=1024) == gdn.GDN_EWORKSPACE
    assert _prefill(q=_Fake(addr=(1 << 20) + 8)) == gdn.GDN_EINVAL
    assert b"prefill" in gdn.lib.gdn_last_error()
    # flag bits: the norm and the one-chain flag only (the accepted flag
    # lets the call go on to the workspace check)
    assert _prefill(segments=False, ws_bytes=1024) == gdn.GDN_EWORKSPACE
    P = gdn._ptr
    st = gdn.lib.gdn_prefill_chunked(
        1, 256, 2, 1, 128, 128, 64, 128, P(_Fake()), P(_Fake()), P(_Fake()),
        gdn.GDN_BF16, P(_Fake(gdn.GDN_F32)), P(_Fake(gdn.GDN_F32)), None,
        P(_Fake(gdn.GDN_F32)), P(_Fake(gdn.GDN_F32)), None,
        P(_Fake(gdn.GDN_F32)), 1 << 30, 1.0, 4, None)
    assert st == gdn.GDN_EINVAL and b"flag" in gdn.lib.gdn_last_error()
    # chunk length: 16, 32 or 64; the interval must be a multiple of it
    assert _prefill(chunk=48) == gdn.GDN_EUNSUPPORTED
    assert _prefill(chunk=128) == gdn.GDN_EUNSUPPORTED
    assert _prefill(chunk=0) == gdn.GDN_EINVAL
    assert _prefill(chunk=32, interval=48) == gdn.GDN_EINVAL
    assert _prefill(chunk=16, interval=48, ws_bytes=1024) == gdn.GDN_EWORKSPACE


def _prefill_noalloc(**over):
    a = dict(n_seqs=1, L=256, hv=2, hk=1, dk=128, dv=128, interval=128,
             q=_Fake(), k=_Fake(), v=_Fake(), beta=_Fake(gdn.GDN_F32),
             g=_Fake(gdn.GDN_F32), Si=None, Sf=_Fake(gdn.GDN_F32),
             o=_Fake(gdn.GDN_F32), ck=_Fake(gdn.GDN_F32))
    a.update(over)
    return gdn.prefill_chunked_noalloc(
        a["n_seqs"], a["L"], a["hv"], a["hk"], a["dk"], a["dv"], a["q"],
        a["k"], a["v"], a["beta"], a["g"], a["Si"], a["Sf"], a["o"], a["ck"],
        ckpt_interval=a["interval"], stream=0, raw_status=True)


def test_prefill_noalloc_rejects_bad_arguments_on_host():
    """The entry point without a workspace checks every argument, and that
    the fixed scratch array is large enough, before its first HIP call."""
    ws = gdn.prefill_workspace_bytes(1, 32768, 32, 32, 128, 128)
    assert ws > gdn.PREFILL_SCRATCH_BYTES
    assert _prefill_noalloc(L=32768, hv=32, hk=32,
                            interval=8192) == gdn.GDN_EWORKSPACE
    assert b"scratch" in gdn.lib.gdn_last_error()
    assert _prefill_noalloc(dk=64, dv=64) == gdn.GDN_EUNSUPPORTED
    assert _prefill_noalloc(hv=3, hk=2) == gdn.GDN_EINVAL
    assert _prefill_noalloc(interval=100) == gdn.GDN_EINVAL
    assert _prefill_noalloc(o=None) == gdn.GDN_EINVAL
    assert _prefill_noalloc(q=_Fake(gdn.GDN_F32), k=_Fake(gdn.GDN_F32),
                            v=_Fake(gdn.GDN_F32)) == gdn.GDN_EUNSUPPORTED
    assert _prefill_noalloc(q=_Fake(addr=(1 << 20) + 8)) == gdn.GDN_EINVAL


def test_missing_library_fails_loudly(tmp_path):
    """Without the built library the package refuses to import: there is no
    fallback path that computes anything elsewhere."""
    import shutil
    import subprocess
    import sys
    pkg = tmp_path / "commit_gated_delta_amd"
    pkg.mkdir()
    shutil.copy(os.path.join(os.path.dirname(gdn.__file__), "__init__.py"),
                pkg / "__init__.py")
    r = subprocess.run(
        [sys.executable, "-c", "import commit_gated_delta_amd"],
        cwd=str(tmp_path), capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "not built" in r.stderr
