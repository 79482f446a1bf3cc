"""GPU parity of gdn_verify / gdn_commit against the fp64 oracle, and the
bit-exact replay invariant (commit(m) == verify's own state after token m).

Every call goes through the C ABI (libgdn.so via the ctypes binding).
Tolerance: 2e-4 block-relative error on o and S (tests/gpu_util.py).
"""
import sys
import zlib

import numpy as np
import pytest

import gdn_synth as gs
import oracle
from tests.gpu_util import (TOL, o_rel_err, s_rel_err, to_dev,
                            window_to_dev)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import commit_gated_delta_amd as gdn  # noqa: E402  (fails loudly if not built)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _run_verify(dims, w, S_dev, dbg=False, scale=1.0, l2norm=True,
                tokenwise=False):
    q, k, v, beta, g = window_to_dev(w, torch)
    o = torch.full((dims.n_layers, dims.n_lanes, dims.t_max, dims.h_v,
                    dims.d_v), float("nan"), device="cuda")
    rec = torch.empty(gdn.records_bytes(dims), dtype=torch.uint8, device="cuda")
    dbg_t = None
    if dbg:
        dbg_t = torch.full((dims.n_layers, dims.n_lanes, dims.t_max, dims.h_v,
                            dims.d_k, dims.d_v), float("nan"), device="cuda")
    gdn.verify(dims, w.t_lane, q, k, v, beta, g, S_dev, o, rec, dbg_t,
               scale=scale, l2norm=l2norm, tokenwise=tokenwise)
    return o, rec, dbg_t


def _check_untouched_rows(o_np, t_lane):
    T = o_np.shape[2]
    for n, t in enumerate(t_lane):
        assert np.all(np.isfinite(o_np[:, n, :t])), "missing output rows"
        assert np.all(np.isnan(o_np[:, n, t:])), "rows past T_lane written"


SMALL = [
    # (name, NL, N, Hv, Hk, dk, dv, T, bf16, ragged, l2norm, scale)
    ("tiny_d16_t4", 1, 1, 2, 2, 16, 16, 4, False, False, True, 1.0),
    ("d128_two_col_blocks", 2, 3, 4, 2, 128, 128, 16, True, True, True, 1.0),
    ("d64_col_tail", 1, 2, 2, 1, 64, 96, 5, True, True, True, 1.0),
    ("d32_dv200_f32", 1, 1, 3, 3, 32, 200, 7, False, False, True, 1.0),
    ("d16_noscale_nonorm", 2, 2, 2, 2, 16, 16, 4, False, False, False, 0.5),
    ("d128_group4", 1, 2, 8, 2, 128, 64, 3, True, False, True, 1.0),
    # matrix-core verify (bf16, d_k = d_v = 128, one block): unnormalised
    # keys with an output scale, one key head per value head, T = 1 windows
    ("d128_noscale_nonorm", 1, 2, 4, 2, 128, 128, 8, True, True, False, 0.5),
    ("d128_group1", 1, 2, 2, 2, 128, 128, 5, True, True, True, 1.0),
    ("d128_t1", 2, 3, 2, 1, 128, 128, 1, True, False, True, 1.0),
    ("d128_dv256", 1, 2, 2, 1, 128, 256, 9, True, True, True, 1.0),
    # the longest windows the ABI takes (64 tokens): bf16 at d = 128 in four
    # blocks of 16 on the matrix cores, f32 at d_k = 64 token by token
    ("d128_t64_max_window", 1, 2, 4, 2, 128, 128, 64, True, True, True, 1.0),
    # f32 inputs on the matrix cores (key and query rows split into bf16
    # hi + lo): one block, and three blocks without the key norm
    ("f32_d128_t16", 1, 3, 4, 2, 128, 128, 16, False, True, True, 1.0),
    ("f32_d128_t40_blocks", 1, 2, 2, 1, 128, 256, 40, False, True, False, 0.5),
    # a second block of one token
    ("d128_t17_one_token_block", 1, 2, 2, 1, 128, 128, 17, True, False, True, 1.0),
    # three blocks with two 128-column blocks per head, no key norm, a scale
    ("d128_dv256_t40_blocks", 2, 2, 2, 1, 128, 256, 40, True, True, False, 0.5),
    ("d64_t33_f32", 1, 2, 2, 1, 64, 64, 33, False, True, True, 1.0),
    # the ABI's value-dimension limits: d_v = 1024 on both kernels (bf16:
    # eight 128-column blocks on the matrix cores; f32: token by token) and
    # d_v = 1
    ("d128_dv1024_max", 1, 1, 2, 1, 128, 1024, 6, True, True, True, 1.0),
    ("f32_d128_dv1024_max", 1, 1, 2, 1, 128, 1024, 5, False, True, True, 1.0),
    ("d32_dv1_min", 1, 2, 2, 1, 32, 1, 5, True, True, True, 1.0),
]


@pytest.mark.parametrize("T", [16, 40])
def test_tokenwise_flag_at_block_shapes(T):
    """GDN_FLAG_TOKENWISE at shapes the block form would take (bf16,
    d = 128): verify runs token by token and holds every intermediate state
    itself.  Its outputs and states meet the oracle, commit(m) is bit for bit
    the state it held after token m, and it agrees with the block form to
    the tolerance, not bit for bit (another kernel ran)."""
    shape = gs.WindowShape(1, 3, 4, 2, 128, 128, T)
    key = (104, T)
    w = gs.window_inputs(shape, key, ragged=True)
    w.t_lane[0] = T
    S0 = gs.initial_state(shape, key)
    dims = gdn.Dims.of(1, 3, 4, 2, 128, 128, T)
    o, rec, dbg = _run_verify(dims, w, to_dev(S0, torch), dbg=True,
                              tokenwise=True)
    ob, _, dbgb = _run_verify(dims, w, to_dev(S0, torch), dbg=True)
    torch.cuda.synchronize()
    o_np, dbg_np = o.cpu().numpy(), dbg.cpu().numpy()
    q64, k64, v64, b64, g64 = w.as_f64()
    o_ref, st_ref = oracle.verify(q64, k64, v64, b64, g64, S0, w.t_lane,
                                  want_states=True)
    e_o = o_rel_err(o_np, o_ref, w.t_lane)
    say("  T=%d tokenwise: o err %.3e" % (T, e_o))
    assert e_o <= TOL
    assert o_rel_err(o_np, ob.cpu().numpy(), w.t_lane) <= TOL
    assert not np.array_equal(o_np[:, 0, :T], ob.cpu().numpy()[:, 0, :T])
    for t in range(T):
        lanes = [n for n in range(3) if w.t_lane[n] > t]
        assert s_rel_err(dbg_np[:, lanes, t], st_ref[:, lanes, t]) <= TOL, t
        assert s_rel_err(dbg_np[:, lanes, t], dbgb.cpu().numpy()[:, lanes, t]) <= TOL, t
    for m in (1, T // 2, T):
        m_lane = np.minimum(m, w.t_lane)
        S_c = to_dev(S0, torch)
        gdn.commit(dims, m_lane, w.t_lane, rec, S_c)
        S_c = S_c.cpu().numpy()
        for n in range(3):
            mm = int(m_lane[n])
            want = S0[:, n] if mm == 0 else dbg_np[:, n, mm - 1]
            assert np.array_equal(S_c[:, n], want), (m, n)


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_window_parity_and_bitexact_replay(case):
    name, NL, N, Hv, Hk, dk, dv, T, bf16, ragged, l2norm, scale = case
    say("case", name)
    shape = gs.WindowShape(NL, N, Hv, Hk, dk, dv, T)
    key = (100, zlib.crc32(name.encode()) % 1000)
    w = gs.window_inputs(shape, key, bf16=bf16, ragged=ragged)
    if not l2norm:   # unnormalised keys must keep the rule stable
        if bf16:     # scale the values, stay bf16 (round to nearest even)
            w.k = gs.f32_to_bf16_bits(gs.bf16_bits_to_f32(w.k) / np.sqrt(dk))
            w.q = gs.f32_to_bf16_bits(gs.bf16_bits_to_f32(w.q) / np.sqrt(dk))
        else:
            w.k = (w.k.astype(np.float32) / np.sqrt(dk)).astype(np.float32)
            w.q = (w.q.astype(np.float32) / np.sqrt(dk)).astype(np.float32)
    S0 = gs.initial_state(shape, key)
    dims = gdn.Dims.of(NL, N, Hv, Hk, dk, dv, T)
    S_dev = to_dev(S0, torch)
    o, rec, dbg = _run_verify(dims, w, S_dev, dbg=True, scale=scale,
                              l2norm=l2norm)
    torch.cuda.synchronize()
    o_np = o.cpu().numpy()
    dbg_np = dbg.cpu().numpy()
    assert np.array_equal(S_dev.cpu().numpy(), S0), "verify wrote S0"
    _check_untouched_rows(o_np, w.t_lane)

    q64, k64, v64, b64, g64 = w.as_f64()
    o_ref, st_ref = oracle.verify(q64, k64, v64, b64, g64, S0, w.t_lane,
                                  scale=scale, l2norm=l2norm, want_states=True)
    e_o = o_rel_err(o_np, o_ref, w.t_lane)
    say("  o err %.3e" % e_o)
    assert e_o <= TOL
    for t in range(T):
        lanes = [n for n in range(N) if w.t_lane[n] > t]
        if lanes:
            e_s = s_rel_err(dbg_np[:, lanes, t], st_ref[:, lanes, t])
            assert e_s <= TOL, (t, e_s)

    # commit(m) for every m of every lane, bitwise against verify's column m
    for m in range(0, T + 1):
        m_lane = np.minimum(m, w.t_lane)
        S_c = to_dev(S0, torch)
        gdn.commit(dims, m_lane, w.t_lane, rec, S_c)
        S_c = S_c.cpu().numpy()
        for n in range(N):
            mm = int(m_lane[n])
            want = S0[:, n] if mm == 0 else dbg_np[:, n, mm - 1]
            assert np.array_equal(S_c[:, n], want), (m, n)
        S_ref = oracle.commit(q64, k64, v64, b64, g64, S0, m_lane,
                              l2norm=l2norm)
        assert s_rel_err(S_c, S_ref) <= TOL


@pytest.mark.parametrize("case", [("bf16_d128", 128, True), ("f32_d32", 32, False)],
                         ids=["bf16_d128", "f32_d32"])
def test_zero_key_and_query_rows(case):
    """All-zero key or query rows (the L2 norm then scales an exact 0): the
    token writes nothing into the state, or reads 0, exactly as the oracle
    has it; parity and bit-exact commit for every m."""
    name, dk, bf16 = case
    shape = gs.WindowShape(1, 3, 4, 2, dk, dk, 16)
    key = (103, zlib.crc32(name.encode()) % 1000)
    w = gs.window_inputs(shape, key, bf16=bf16, ragged=True)
    for n, t in ((0, 0), (0, 5), (1, 3), (2, 15)):
        w.k[:, n, t] = 0
    for n, t in ((0, 2), (1, 3), (2, 7)):
        w.q[:, n, t] = 0
    S0 = gs.initial_state(shape, key)
    dims = gdn.Dims.of(*shape.__dict__.values())
    S_dev = to_dev(S0, torch)
    o, rec, dbg = _run_verify(dims, w, S_dev, dbg=True)
    torch.cuda.synchronize()
    o_np, dbg_np = o.cpu().numpy(), dbg.cpu().numpy()
    q64, k64, v64, b64, g64 = w.as_f64()
    o_ref, st_ref = oracle.verify(q64, k64, v64, b64, g64, S0, w.t_lane,
                                  want_states=True)
    assert o_rel_err(o_np, o_ref, w.t_lane) <= TOL
    for t in range(16):
        lanes = [n for n in range(3) if w.t_lane[n] > t]
        if lanes:
            assert s_rel_err(dbg_np[:, lanes, t], st_ref[:, lanes, t]) <= TOL
    for m in range(17):
        m_lane = np.minimum(m, w.t_lane)
        S_c = to_dev(S0, torch)
        gdn.commit(dims, m_lane, w.t_lane, rec, S_c)
        S_c = S_c.cpu().numpy()
        for n in range(3):
            want = S0[:, n] if m_lane[n] == 0 else dbg_np[:, n, m_lane[n] - 1]
            assert np.array_equal(S_c[:, n], want), (m, n)


@pytest.mark.parametrize("case", [("bf16_d128", 128, True), ("f32_d32", 32, False)],
                         ids=["bf16_d128", "f32_d32"])
def test_orthonormal_keys_store_their_values(case):
    """Closed form of the delta write (no oracle involved): alpha = 1,
    beta = 1 and orthonormal keys (a permuted standard basis, exact in bf16;
    norm flag off) make the committed state map every key to its value:
    row j of the stored state (d_k x d_v) is the value written with e_j."""
    name, dk, bf16 = case
    T = 16
    shape = gs.WindowShape(1, 2, 2, 1, dk, dk, T)
    key = (104, zlib.crc32(name.encode()) % 1000)
    w = gs.window_inputs(shape, key, bf16=bf16)
    perm = np.random.default_rng(104).permutation(dk)[:T]
    kk = np.zeros((1, 2, T, 1, dk), np.float32)
    kk[:, :, np.arange(T), 0, perm] = 1.0
    w.k = gs.f32_to_bf16_bits(kk) if bf16 else kk
    w.beta[:] = 1.0
    w.g[:] = 0.0
    S0 = gs.initial_state(shape, key)
    dims = gdn.Dims.of(*shape.__dict__.values())
    S_dev = to_dev(S0, torch)
    _, rec, _ = _run_verify(dims, w, S_dev, l2norm=False)
    gdn.commit(dims, [T, T], [T, T], rec, S_dev)
    S = S_dev.cpu().numpy()
    v = gs.bf16_bits_to_f32(w.v) if bf16 else w.v.astype(np.float32)
    for n in range(2):
        for h in range(2):
            got = S[0, n, h][perm]
            ref = v[0, n, :, h]
            assert np.max(np.abs(got - ref)) / np.max(np.abs(ref)) <= TOL, (n, h)


MAX_LANES = [
    # (name, Hv, Hk, dk, dv, T, bf16): the matrix-core and the
    # token-by-token verify at the ABI's lane limit
    ("bf16_d128", 2, 1, 128, 128, 16, True),
    ("f32_d16", 2, 2, 16, 16, 8, False),
]


@pytest.mark.parametrize("case", MAX_LANES, ids=[c[0] for c in MAX_LANES])
def test_max_lanes(case):
    """GDN_MAX_LANES (256) lanes with ragged windows: outputs against the
    oracle, commit(m) bitwise against the debug states for every lane, and
    the fused call bitwise against commit + verify (the per-lane tables
    travel in the kernel arguments)."""
    name, Hv, Hk, dk, dv, T, bf16 = case
    N = gdn.GDN_MAX_LANES
    shape = gs.WindowShape(1, N, Hv, Hk, dk, dv, T)
    key = (102, zlib.crc32(name.encode()) % 1000)
    w = gs.window_inputs(shape, key, bf16=bf16, ragged=True)
    S0 = gs.initial_state(shape, key)
    m = gs.accepted_uniform(w.t_lane, key)
    dims = gdn.Dims.of(1, N, Hv, Hk, dk, dv, T)
    S_dev = to_dev(S0, torch)
    o, rec, dbg = _run_verify(dims, w, S_dev, dbg=True)
    gdn.commit(dims, m, w.t_lane, rec, S_dev)
    torch.cuda.synchronize()
    o_np, dbg_np, S_np = o.cpu().numpy(), dbg.cpu().numpy(), S_dev.cpu().numpy()
    _check_untouched_rows(o_np, w.t_lane)
    q64, k64, v64, b64, g64 = w.as_f64()
    o_ref, _ = oracle.verify(q64, k64, v64, b64, g64, S0, w.t_lane)
    e_o = o_rel_err(o_np, o_ref, w.t_lane)
    say("  %s: o err %.2e" % (name, e_o))
    assert e_o <= TOL
    for n in range(N):
        want = S0[:, n] if m[n] == 0 else dbg_np[:, n, m[n] - 1]
        assert np.array_equal(S_np[:, n], want), n
    S_ref = oracle.commit(q64, k64, v64, b64, g64, S0, m)
    assert s_rel_err(S_np, S_ref) <= TOL
    # one fused round on top: commit of this window + verify of the next
    w2 = gs.window_inputs(shape, key + (1,), bf16=bf16, ragged=True)
    q, k, v, beta, g = window_to_dev(w2, torch)
    S_a, S_b = to_dev(S0, torch), to_dev(S0, torch)
    o_a = torch.zeros((1, N, T, Hv, dv), device="cuda")
    o_b = torch.zeros_like(o_a)
    rec_a = torch.empty_like(rec)
    rec_b = torch.empty_like(rec)
    gdn.commit(dims, m, w.t_lane, rec, S_a)
    gdn.verify(dims, w2.t_lane, q, k, v, beta, g, S_a, o_a, rec_a)
    gdn.commit_verify(dims, m, w.t_lane, rec, w2.t_lane, q, k, v, beta, g,
                      S_b, o_b, rec_b)
    torch.cuda.synchronize()
    assert torch.equal(S_a, S_b)
    assert torch.equal(o_a, o_b)


def test_verify_is_deterministic_and_leaves_state():
    shape = gs.WindowShape(2, 4, 4, 2, 128, 128, 16)
    w = gs.window_inputs(shape, (101,), ragged=True)
    S0 = gs.initial_state(shape, (101,))
    dims = gdn.Dims.of(*shape.__dict__.values())
    S_dev = to_dev(S0, torch)
    o1, r1, _ = _run_verify(dims, w, S_dev)
    o2, r2, _ = _run_verify(dims, w, S_dev)
    torch.cuda.synchronize()
    assert torch.equal(torch.nan_to_num(o1, 7.0), torch.nan_to_num(o2, 7.0))
    # records: every byte that verify writes is identical (unwritten padding
    # rows of ragged lanes are compared through commit instead)
    m = w.t_lane.copy()
    Sa, Sb = to_dev(S0, torch), to_dev(S0, torch)
    gdn.commit(dims, m, w.t_lane, r1, Sa)
    gdn.commit(dims, m, w.t_lane, r2, Sb)
    assert torch.equal(Sa, Sb)
    assert np.array_equal(S_dev.cpu().numpy(), S0)


@pytest.mark.parametrize("case", [("bf16_T40_folds", 40, True),
                                  ("f32_T40_folds", 40, False),
                                  ("bf16_T64_alpha0", 64, True)],
                         ids=lambda c: c[0])
def test_debug_states_leave_outputs_unchanged(case):
    """Windows of several blocks: asking for the debug states (which run the
    token-by-token replay on a copy of the state) changes neither the
    outputs nor the records, bit for bit, also with folds and alpha = 0
    inside the blocks."""
    name, T, bf16 = case
    shape = gs.WindowShape(1, 3, 4, 2, 128, 128, T)
    key = (112, zlib.crc32(name.encode()) % 1000)
    w = gs.window_inputs(shape, key, bf16=bf16, ragged=True)
    w.t_lane[0] = T
    if "folds" in name:
        w.g[:] = -3.0 - 0.5 * np.arange(w.g.shape[-1])[None, None, None, :]
    else:
        w.g[:, :, 3] = -np.inf
        w.g[:, :, 20, ::2] = -200.0
        w.g[:, :, 37] = -np.inf
    S0 = gs.initial_state(shape, key)
    dims = gdn.Dims.of(*shape.__dict__.values())
    S_dev = to_dev(S0, torch)
    o1, r1, dbg = _run_verify(dims, w, S_dev, dbg=True)
    o2, r2, _ = _run_verify(dims, w, S_dev)
    torch.cuda.synchronize()
    assert torch.equal(torch.nan_to_num(o1, 7.0), torch.nan_to_num(o2, 7.0))
    m = w.t_lane.copy()
    Sa, Sb = to_dev(S0, torch), to_dev(S0, torch)
    gdn.commit(dims, m, w.t_lane, r1, Sa)
    gdn.commit(dims, m, w.t_lane, r2, Sb)
    assert torch.equal(Sa, Sb)
    dbg_np = dbg.cpu().numpy()
    Sa = Sa.cpu().numpy()
    for n in range(3):
        assert np.array_equal(Sa[:, n], dbg_np[:, n, int(w.t_lane[n]) - 1]), n
    say("  %s: outputs and records unchanged by debug states" % name)


def test_zero_gates_are_bitwise_identity():
    """beta = 0, g = 0: u = 0 and alpha = 1, so every step is
    fma(0, k, 1*S) = S exactly; commit(T) returns S0 bit for bit."""
    shape = gs.WindowShape(1, 2, 4, 2, 128, 128, 8)
    w = gs.window_inputs(shape, (102,))
    w.beta[:] = 0.0
    w.g[:] = 0.0
    S0 = gs.initial_state(shape, (102,))
    dims = gdn.Dims.of(*shape.__dict__.values())
    S_dev = to_dev(S0, torch)
    o, rec, _ = _run_verify(dims, w, S_dev)
    gdn.commit(dims, w.t_lane, w.t_lane, rec, S_dev)
    torch.cuda.synchronize()
    assert np.array_equal(S_dev.cpu().numpy(), S0)
    q64, k64, v64, b64, g64 = w.as_f64()
    o_ref, _ = oracle.verify(q64, k64, v64, b64, g64, S0, w.t_lane)
    assert o_rel_err(o.cpu().numpy(), o_ref, w.t_lane) <= TOL


def test_idle_lane_and_zero_accept():
    """t_lane = 0 lanes are neither read nor written; m = 0 lanes keep S."""
    shape = gs.WindowShape(1, 3, 2, 1, 64, 64, 4)
    w = gs.window_inputs(shape, (103,), t_lane=[4, 0, 2])
    S0 = gs.initial_state(shape, (103,))
    dims = gdn.Dims.of(*shape.__dict__.values())
    S_dev = to_dev(S0, torch)
    o, rec, dbg = _run_verify(dims, w, S_dev, dbg=True)
    o_np = o.cpu().numpy()
    assert np.all(np.isnan(o_np[:, 1]))
    assert np.all(np.isnan(dbg.cpu().numpy()[:, 1]))
    gdn.commit(dims, [0, 0, 2], w.t_lane, rec, S_dev)
    S1 = S_dev.cpu().numpy()
    assert np.array_equal(S1[:, 0], S0[:, 0])
    assert np.array_equal(S1[:, 1], S0[:, 1])
    assert np.array_equal(S1[:, 2], dbg.cpu().numpy()[:, 2, 1])


@pytest.mark.parametrize("case", [("bf16_d128", 128, True), ("f32_d32", 32, False)],
                         ids=lambda c: c[0])
def test_all_lanes_idle(case):
    """Degenerate batches on both verify kernels: with every lane idle
    (t_lane = 0, m = 0) verify, commit and the fused call read and write
    nothing (outputs, records and debug states keep their fill, the state
    its bits); a fused call whose next windows are all empty still commits
    the previous prefixes, bit for bit as commit alone."""
    name, d, bf16 = case
    shape = gs.WindowShape(2, 3, 2, 1, d, d, 16)
    dims = gdn.Dims.of(*shape.__dict__.values())
    S0 = gs.initial_state(shape, (109,))
    idle = np.zeros(3, dtype=np.int32)
    w0 = gs.window_inputs(shape, (109,), bf16=bf16, t_lane=[0, 0, 0])
    q, k, v, beta, g = window_to_dev(w0, torch)
    S_dev = to_dev(S0, torch)
    o = torch.full((2, 3, 16, 2, d), float("nan"), device="cuda")
    dbg = torch.full((2, 3, 16, 2, d, d), float("nan"), device="cuda")
    rec = torch.full((gdn.records_bytes(dims),), 0xA5, dtype=torch.uint8,
                     device="cuda")
    gdn.verify(dims, idle, q, k, v, beta, g, S_dev, o, rec, dbg)
    gdn.commit(dims, idle, idle, rec, S_dev)
    rec2 = rec.clone()
    gdn.commit_verify(dims, idle, idle, rec, idle, q, k, v, beta, g, S_dev,
                      o, rec2)
    torch.cuda.synchronize()
    assert torch.isnan(o).all() and torch.isnan(dbg).all()
    assert (rec == 0xA5).all() and (rec2 == 0xA5).all()
    assert np.array_equal(S_dev.cpu().numpy(), S0)
    # previous windows of 4, 0 and 2 tokens, accepted 3, 0 and 1; the next
    # windows empty: the fused call is the commit alone
    w1 = gs.window_inputs(shape, (109, 1), bf16=bf16, t_lane=[4, 0, 2])
    m = np.array([3, 0, 1], dtype=np.int32)
    S_v = to_dev(S0, torch)
    _, rec1, _ = _run_verify(dims, w1, S_v)
    S_c, S_f = to_dev(S0, torch), to_dev(S0, torch)
    gdn.commit(dims, m, w1.t_lane, rec1, S_c)
    o_f = torch.full_like(o, float("nan"))
    rec_f = torch.full_like(rec, 0xA5)
    gdn.commit_verify(dims, m, w1.t_lane, rec1, idle, q, k, v, beta, g, S_f,
                      o_f, rec_f)
    torch.cuda.synchronize()
    assert torch.equal(S_c, S_f)
    assert not np.array_equal(S_c.cpu().numpy()[:, 0], S0[:, 0])
    assert np.array_equal(S_c.cpu().numpy()[:, 1], S0[:, 1])
    assert torch.isnan(o_f).all() and (rec_f == 0xA5).all()
    say("  %s: idle batch untouched, empty next windows commit only" % name)


FOLD_CASES = [
    # (name, dk, dv, bf16): the matrix-core readout (bf16, d_k >= 32) and
    # the general loop (f32 inputs, d_k = 16)
    ("bf16_d128", 128, 128, True),
    ("bf16_d64", 64, 96, True),
    ("f32_d32", 32, 64, False),
    ("f32_d16", 16, 16, False),
]


def _fold_check(name, dk, dv, bf16, g_fill):
    shape = gs.WindowShape(1, 3, 4, 2, dk, dv, 16)
    key = (104, zlib.crc32(name.encode()) % 1000)
    w = gs.window_inputs(shape, key, bf16=bf16, t_lane=[16, 13, 7])
    g_fill(w.g)
    S0 = gs.initial_state(shape, key)
    dims = gdn.Dims.of(*shape.__dict__.values())
    S_dev = to_dev(S0, torch)
    o, rec, dbg = _run_verify(dims, w, S_dev, dbg=True)
    o_np, dbg_np = o.cpu().numpy(), dbg.cpu().numpy()
    q64, k64, v64, b64, g64 = w.as_f64()
    o_ref, st_ref = oracle.verify(q64, k64, v64, b64, g64, S0, w.t_lane,
                                  want_states=True)
    e_o = o_rel_err(o_np, o_ref, w.t_lane)
    say("  %s: o err %.2e" % (name, e_o))
    assert e_o <= TOL
    for t in range(16):
        lanes = [n for n in range(3) if w.t_lane[n] > t]
        assert s_rel_err(dbg_np[:, lanes, t], st_ref[:, lanes, t]) <= TOL, t
    for m in (1, 4, 5, 12, 16):
        m_lane = np.minimum(m, w.t_lane)
        S_c = to_dev(S0, torch)
        gdn.commit(dims, m_lane, w.t_lane, rec, S_c)
        S_c = S_c.cpu().numpy()
        for n in range(3):
            assert np.array_equal(S_c[:, n], dbg_np[:, n, m_lane[n] - 1]), (m, n)


@pytest.mark.parametrize("case", FOLD_CASES, ids=[c[0] for c in FOLD_CASES])
def test_zero_decay_tokens(case):
    """alpha = 0 exactly (g = -inf, and g = -200, which underflows in f32):
    the state is forgotten at that token (a fold by factor 0)."""
    name, dk, dv, bf16 = case

    def fill(g):
        g[:, :, 3] = -np.inf
        g[:, :, 9, ::2] = -200.0
        g[:, 1, 12] = -np.inf

    _fold_check("zero_" + name, dk, dv, bf16, fill)


@pytest.mark.parametrize("case", FOLD_CASES, ids=[c[0] for c in FOLD_CASES])
def test_strong_decay_folds(case):
    """g = -3 at every token: the scale leaves [2^-32, 2^32] every ~11
    tokens, so windows fold once or twice at head-dependent tokens."""
    name, dk, dv, bf16 = case

    def fill(g):
        g[:] = -3.0 - 0.5 * np.arange(g.shape[-1])[None, None, None, :]

    _fold_check("decay_" + name, dk, dv, bf16, fill)


def test_tiny_case_f32():
    """1 lane, 1 layer, 2 heads, d = 16, T = 4, f32 inputs; m ~ U{0..4}."""
    shape, key = gs.TINY, (gs.KEY_TINY, 0)
    w = gs.window_inputs(shape, key, bf16=False)
    S0 = gs.initial_state(shape, key)
    m = gs.accepted_uniform(w.t_lane, key)
    dims = gdn.Dims.of(*shape.__dict__.values())
    S_dev = to_dev(S0, torch)
    o, rec, dbg = _run_verify(dims, w, S_dev, dbg=True)
    gdn.commit(dims, m, w.t_lane, rec, S_dev)
    torch.cuda.synchronize()
    q64, k64, v64, b64, g64 = w.as_f64()
    o_ref, _ = oracle.verify(q64, k64, v64, b64, g64, S0, w.t_lane)
    S_ref = oracle.commit(q64, k64, v64, b64, g64, S0, m)
    S_gpu = S_dev.cpu().numpy()
    say("tiny case: m =", m, "o err %.2e S err %.2e" % (
        o_rel_err(o.cpu().numpy(), o_ref, w.t_lane), s_rel_err(S_gpu, S_ref)))
    assert o_rel_err(o.cpu().numpy(), o_ref, w.t_lane) <= TOL
    assert s_rel_err(S_gpu, S_ref) <= TOL
    want = S0 if m[0] == 0 else dbg.cpu().numpy()[:, :, m[0] - 1]
    assert np.array_equal(S_gpu, want)


def test_eight_lanes_48_layers_ragged():
    """8 lanes x 48 layers x 32/16 heads, d = 128, T_l ~ U{1..16},
    m_l ~ U{0..T_l}: full o and S parity against the oracle, and bit-exact
    replay on layer 0 (debug states)."""
    shape, key = gs.EIGHT_LANES, (gs.KEY_EIGHT_LANES, 0)
    say("8 lanes x 48 layers: generating inputs")
    w = gs.window_inputs(shape, key, ragged=True)
    S0 = gs.initial_state(shape, key)
    m = gs.accepted_uniform(w.t_lane, key)
    dims = gdn.Dims.of(*shape.__dict__.values())
    S_dev = to_dev(S0, torch)
    say("8 lanes x 48 layers: verify, T =", w.t_lane, "m =", m)
    o, rec, _ = _run_verify(dims, w, S_dev)
    o_np = o.cpu().numpy()
    _check_untouched_rows(o_np, w.t_lane)
    gdn.commit(dims, m, w.t_lane, rec, S_dev)
    S_gpu = S_dev.cpu().numpy()
    say("8 lanes x 48 layers: oracle")
    q64, k64, v64, b64, g64 = w.as_f64()
    o_ref, _ = oracle.verify(q64, k64, v64, b64, g64, S0, w.t_lane)
    e_o = o_rel_err(o_np, o_ref, w.t_lane)
    del o_ref
    S_ref = oracle.commit(q64, k64, v64, b64, g64, S0, m)
    e_s = s_rel_err(S_gpu, S_ref)
    say("8 lanes x 48 layers: o err %.3e  S err %.3e" % (e_o, e_s))
    assert e_o <= TOL and e_s <= TOL

    # bit-exact replay on layer 0 through a one-layer call with debug states
    d1 = gdn.Dims.of(1, shape.n_lanes, shape.h_v, shape.h_k, 128, 128,
                     shape.t_max)
    w1 = gs.WindowInputs(d1, True, w.q[:1], w.k[:1], w.v[:1], w.beta[:1],
                         w.g[:1], w.t_lane)
    S1 = to_dev(S0[:1], torch)
    _, rec1, dbg1 = _run_verify(d1, w1, S1, dbg=True)
    gdn.commit(d1, m, w.t_lane, rec1, S1)
    dbg1 = dbg1.cpu().numpy()
    S1 = S1.cpu().numpy()
    for n in range(shape.n_lanes):
        want = S0[:1, n] if m[n] == 0 else dbg1[:, n, m[n] - 1]
        assert np.array_equal(S1[:, n], want), n
    # the one-layer call and the 48-layer call agree bit for bit
    assert np.array_equal(S1, S_gpu[:1])


@pytest.mark.parametrize("T", [32, 64])
def test_eight_lanes_48_layers_long_windows(T):
    """8 lanes x 48 layers x 32/16 heads, d = 128, windows of up to 32 and
    64 tokens (blocks of 16, the bench's long-window shapes), m_l ~
    U{0..T_l}: the oracle follows layers 0 and 47 (o of every token and the
    committed state), and layer 0's commit is bit for bit a one-layer debug
    run's state."""
    base = gs.EIGHT_LANES
    shape = gs.WindowShape(base.n_layers, base.n_lanes, base.h_v, base.h_k,
                           128, 128, T)
    key = (gs.KEY_EIGHT_LANES, T)
    say("8 lanes x 48 layers, T = %d: generating inputs" % T)
    w = gs.window_inputs(shape, key, ragged=True)
    w.t_lane[0] = T
    S0 = gs.initial_state(shape, key)
    m = gs.accepted_uniform(w.t_lane, key)
    dims = gdn.Dims.of(*shape.__dict__.values())
    S_dev = to_dev(S0, torch)
    say("  verify, T =", w.t_lane, "m =", m)
    o, rec, _ = _run_verify(dims, w, S_dev)
    o_np = o.cpu().numpy()
    _check_untouched_rows(o_np, w.t_lane)
    gdn.commit(dims, m, w.t_lane, rec, S_dev)
    S_gpu = S_dev.cpu().numpy()
    sl = [0, base.n_layers - 1]
    q64, k64, v64, b64, g64 = (a[sl] for a in w.as_f64())
    o_ref, _ = oracle.verify(q64, k64, v64, b64, g64, S0[sl], w.t_lane)
    e_o = o_rel_err(o_np[sl], o_ref, w.t_lane)
    S_ref = oracle.commit(q64, k64, v64, b64, g64, S0[sl], m)
    e_s = s_rel_err(S_gpu[sl], S_ref)
    say("  layers %s: o err %.3e  S err %.3e" % (sl, e_o, e_s))
    assert e_o <= TOL and e_s <= TOL
    d1 = gdn.Dims.of(1, shape.n_lanes, shape.h_v, shape.h_k, 128, 128, T)
    w1 = gs.WindowInputs(d1, True, w.q[:1], w.k[:1], w.v[:1], w.beta[:1],
                         w.g[:1], w.t_lane)
    S1 = to_dev(S0[:1], torch)
    _, rec1, dbg1 = _run_verify(d1, w1, S1, dbg=True)
    gdn.commit(d1, m, w.t_lane, rec1, S1)
    dbg1 = dbg1.cpu().numpy()
    S1 = S1.cpu().numpy()
    for n in range(shape.n_lanes):
        want = S0[:1, n] if m[n] == 0 else dbg1[:, n, m[n] - 1]
        assert np.array_equal(S1[:, n], want), n
    assert np.array_equal(S1, S_gpu[:1])


def _chained(shape, case, rounds, acc, sample_layers, t_fixed, pool=8, say_every=16):
    """Chained verify -> commit(m) rounds; the oracle follows the sampled
    layers through every round.  Window inputs cycle through a pool of
    seeded sets, gates are redrawn every round.  Returns per-round errors."""
    dims = gdn.Dims.of(*shape.__dict__.values())
    S0 = gs.initial_state(shape, (case, 0))
    S_dev = to_dev(S0, torch)
    S_or = S0[sample_layers].astype(np.float64)
    pool_w = [gs.window_inputs(shape, (case, 1000 + p)) for p in range(pool)]
    o_buf = torch.empty((shape.n_layers, shape.n_lanes, shape.t_max, shape.h_v,
                         shape.d_v), device="cuda")
    rec = torch.empty(gdn.records_bytes(dims), dtype=torch.uint8, device="cuda")
    sl = list(sample_layers)
    errs = []
    t_lane = np.full(shape.n_lanes, t_fixed, dtype=np.int32)
    dev_pool = [window_to_dev(pw, torch)[:3] for pw in pool_w]
    for r in range(rounds):
        base = pool_w[r % pool]
        gw = gs.window_inputs(gs.WindowShape(shape.n_layers, shape.n_lanes,
                                             shape.h_v, 1, 1, 1, shape.t_max),
                              (case, 5000 + r))
        beta, g = gw.beta, gw.g
        m = acc(t_lane, (case, r))
        q, k, v = dev_pool[r % pool]
        beta_d, g_d = to_dev(beta, torch), to_dev(g, torch)
        # bit-exact replay, every round, on one sampled layer: a one-layer
        # verify with debug states on the same pre-commit state
        L = sl[r % len(sl)]
        d1 = gdn.Dims.of(1, shape.n_lanes, shape.h_v, shape.h_k, shape.d_k,
                         shape.d_v, shape.t_max)
        S_L = S_dev[L:L + 1].clone()
        o1 = torch.empty((1, shape.n_lanes, shape.t_max, shape.h_v,
                          shape.d_v), device="cuda")
        rec1 = torch.empty(gdn.records_bytes(d1), dtype=torch.uint8,
                           device="cuda")
        dbg1 = torch.empty((1, shape.n_lanes, shape.t_max, shape.h_v,
                            shape.d_k, shape.d_v), device="cuda")
        gdn.verify(d1, t_lane, q[L:L + 1], k[L:L + 1], v[L:L + 1],
                   beta_d[L:L + 1], g_d[L:L + 1], S_L, o1, rec1, dbg1)
        gdn.verify(dims, t_lane, q, k, v, beta_d, g_d, S_dev, o_buf, rec)
        gdn.commit(dims, m, t_lane, rec, S_dev)
        after = S_dev[L].cpu().numpy()
        before = S_L[0].cpu().numpy()
        snaps = dbg1[0].cpu().numpy()
        for n in range(shape.n_lanes):
            want = before[n] if m[n] == 0 else snaps[n, m[n] - 1]
            assert np.array_equal(after[n], want), ("replay not bit-exact",
                                                     r, L, n)
        o_np = o_buf[sl].cpu().numpy()
        q64, k64, v64 = (gs.bf16_bits_to_f64(a[sl]) for a in
                         (base.q, base.k, base.v))
        b64, g64 = beta[sl].astype(np.float64), g[sl].astype(np.float64)
        o_ref, _ = oracle.verify(q64, k64, v64, b64, g64, S_or, t_lane)
        S_or = oracle.commit(q64, k64, v64, b64, g64, S_or, m)
        e_o = o_rel_err(o_np, o_ref, t_lane)
        e_s = s_rel_err(S_dev[sl].cpu().numpy(), S_or)
        errs.append((e_o, e_s))
        if r % say_every == 0 or r == rounds - 1:
            say("  round %d: m=%s o err %.2e S err %.2e" % (r, m[:4], e_o, e_s))
    return errs


def test_one_lane_100_chained_rounds():
    """1 lane x 48 layers, T = 16, m ~ U{0..16}, 100 rounds carrying S."""
    say("1 lane x 48 layers, 100 rounds")
    errs = _chained(gs.ONE_LANE, gs.KEY_ONE_LANE, 100, gs.accepted_uniform, [0, 23, 47], 16)
    assert max(max(e) for e in errs) <= TOL


def test_twelve_lanes_256_chained_rounds():
    """12 lanes x 48 layers, T = 6, m ~ Binomial(6, 0.7), 256 rounds."""
    say("12 lanes x 48 layers, 256 rounds")
    errs = _chained(gs.TWELVE_LANES_T6, gs.KEY_TWELVE_LANES, 256, lambda t, key: gs.accepted_binomial(t, 0.7, key),
                    [5], 6, say_every=32)
    worst = max(max(e) for e in errs)
    assert worst <= TOL
    # the error does not drift upward over the chain (non-expansive rule)
    first = max(max(e) for e in errs[:64])
    last = max(max(e) for e in errs[-64:])
    say("  first-64 worst %.2e  last-64 worst %.2e" % (first, last))
    assert last <= 4 * first + 1e-6
