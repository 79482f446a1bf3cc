"""GPU parity of gdn_kda_verify / gdn_kda_commit (per-channel decay) against
the fp64 oracle, and bit-exact replay: commit(m) equals verify's own state
after token m.  Every call goes through the C ABI; tolerance 2e-4
block-relative."""
import sys
import zlib

import numpy as np
import pytest

import gdn_synth as gs
import oracle
from tests.gpu_util import TOL, o_rel_err, s_rel_err, to_dev, window_to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import commit_gated_delta_amd as gdn  # noqa: E402


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _kda_run(dims, w, gk, S_dev, dbg=True):
    q, k, v, beta, _ = window_to_dev(w, torch)
    g = to_dev(gk, torch)
    o = torch.full((dims.n_layers, dims.n_lanes, dims.t_max, dims.h_v,
                    dims.d_v), float("nan"), device="cuda")
    rec = torch.empty(gdn.kda_records_bytes(dims), dtype=torch.uint8,
                      device="cuda")
    d = None
    if dbg:
        d = torch.full((dims.n_layers, dims.n_lanes, dims.t_max, dims.h_v,
                        dims.d_k, dims.d_v), float("nan"), device="cuda")
    gdn.kda_verify(dims, w.t_lane, q, k, v, beta, g, S_dev, o, rec, d)
    return o, rec, d


CASES = [
    # (name, NL, N, Hv, Hk, dv, T, bf16, g_fill)
    ("bf16_two_col_blocks", 2, 3, 4, 2, 128, 16, True, None),
    ("f32_dv200", 1, 2, 3, 3, 200, 7, False, None),
    ("bf16_channel_forgetting", 1, 2, 4, 2, 64, 12, True, "zero"),
    ("bf16_strong_decay", 1, 2, 4, 2, 128, 16, True, "strong"),
    # the matrix-core KDA verify (bf16, d_v = 128, one block) with zero
    # decays on some channels
    ("bf16_channel_forgetting_d128", 1, 2, 4, 2, 128, 12, True, "zero"),
    # windows of 40 and 64 tokens: blocks of 16, each from the state left by
    # the blocks before it
    ("bf16_t40_blocks_forgetting", 1, 3, 2, 1, 128, 40, True, "zero"),
    ("bf16_t64_blocks_strong", 1, 2, 2, 2, 128, 64, True, "strong"),
    # f32 inputs on the matrix cores, one block and two blocks
    ("f32_d128_forgetting", 1, 3, 4, 2, 128, 16, False, "zero"),
    ("f32_t24_blocks_strong", 1, 2, 2, 1, 128, 24, False, "strong"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_kda_parity_and_bitexact_replay(case):
    name, NL, N, Hv, Hk, dv, T, bf16, fill = case
    say("case", name)
    shape = gs.WindowShape(NL, N, Hv, Hk, 128, dv, T)
    key = (600, zlib.crc32(name.encode()) % 1000)
    w = gs.window_inputs(shape, key, bf16=bf16, ragged=True)
    gk = gs.kda_gates(shape, key)
    if fill == "zero":
        gk[:, :, 2, :, ::3] = -np.inf     # alpha = 0 on every third channel
        gk[:, :, 7, :, :] = -200.0        # underflows to 0 in f32
    elif fill == "strong":
        gk[:] -= 4.0
    S0 = gs.initial_state(shape, key)
    dims = gdn.Dims.of(*shape.__dict__.values())
    S_dev = to_dev(S0, torch)
    o, rec, dbg = _kda_run(dims, w, gk, S_dev)
    torch.cuda.synchronize()
    assert torch.equal(S_dev.cpu(), torch.from_numpy(S0)), "verify wrote S0"
    o_np, dbg_np = o.cpu().numpy(), dbg.cpu().numpy()
    q64, k64, v64, b64, _ = w.as_f64()
    g64 = gk.astype(np.float64)
    o_ref, st_ref = oracle.kda_verify(q64, k64, v64, b64, g64, S0, w.t_lane,
                                      want_states=True)
    e_o = o_rel_err(o_np, o_ref, w.t_lane)
    say("  o err %.2e" % e_o)
    assert e_o <= TOL
    for t in range(T):
        lanes = [n for n in range(N) if w.t_lane[n] > t]
        if lanes:
            assert s_rel_err(dbg_np[:, lanes, t], st_ref[:, lanes, t]) <= TOL, t
    for m in range(0, T + 1, 3):
        m_lane = np.minimum(m, w.t_lane)
        S_c = to_dev(S0, torch)
        gdn.kda_commit(dims, m_lane, w.t_lane, rec, S_c)
        S_c = S_c.cpu().numpy()
        for n in range(N):
            mm = int(m_lane[n])
            want = S0[:, n] if mm == 0 else dbg_np[:, n, mm - 1]
            assert np.array_equal(S_c[:, n], want), (m, n)
        S_ref = oracle.kda_commit(q64, k64, v64, b64, g64, S0, m_lane)
        assert s_rel_err(S_c, S_ref) <= TOL


@pytest.mark.parametrize("case", [("bf16_t40_forgetting", 40, True),
                                  ("f32_t33_strong", 33, False)],
                         ids=lambda c: c[0])
def test_kda_debug_states_leave_outputs_unchanged(case):
    """Windows of several blocks: asking for the debug states (the
    token-by-token replay on a copy of the state) changes neither the
    outputs nor the records, bit for bit."""
    name, T, bf16 = case
    shape = gs.WindowShape(1, 3, 4, 2, 128, 128, T)
    key = (603, zlib.crc32(name.encode()) % 1000)
    w = gs.window_inputs(shape, key, bf16=bf16, ragged=True)
    w.t_lane[0] = T
    gk = gs.kda_gates(shape, key)
    if "forgetting" in name:
        gk[:, :, 2, :, ::3] = -np.inf
        gk[:, :, 21, :, 1::4] = -200.0
    else:
        gk[:] -= 4.0
    S0 = gs.initial_state(shape, key)
    dims = gdn.Dims.of(*shape.__dict__.values())
    S_dev = to_dev(S0, torch)
    o1, r1, dbg = _kda_run(dims, w, gk, S_dev)
    o2, r2, _ = _kda_run(dims, w, gk, S_dev, dbg=False)
    torch.cuda.synchronize()
    assert torch.equal(torch.nan_to_num(o1, 7.0), torch.nan_to_num(o2, 7.0))
    m = w.t_lane.copy()
    Sa, Sb = to_dev(S0, torch), to_dev(S0, torch)
    gdn.kda_commit(dims, m, w.t_lane, r1, Sa)
    gdn.kda_commit(dims, m, w.t_lane, r2, Sb)
    assert torch.equal(Sa, Sb)
    Sa, dbg_np = Sa.cpu().numpy(), dbg.cpu().numpy()
    for n in range(3):
        assert np.array_equal(Sa[:, n], dbg_np[:, n, int(w.t_lane[n]) - 1]), n
    say("  %s: outputs and records unchanged by debug states" % name)


def test_kda_full_batch_long_windows():
    """8 lanes x 48 layers x 32/16 heads, d = 128, windows of up to 40
    tokens (blocks of 16), ragged, m ~ U{0..T}: the oracle follows layers 0
    and 47 (o of every token and the committed state), and layer 0's commit
    is bit for bit a one-layer debug run's state."""
    T = 40
    shape = gs.WindowShape(48, 8, 32, 16, 128, 128, T)
    key = (604, T)
    w = gs.window_inputs(shape, key, ragged=True)
    w.t_lane[0] = T
    gk = gs.kda_gates(shape, key)
    S0 = gs.initial_state(shape, key)
    m = gs.accepted_uniform(w.t_lane, key)
    dims = gdn.Dims.of(*shape.__dict__.values())
    S_dev = to_dev(S0, torch)
    o, rec, _ = _kda_run(dims, w, gk, S_dev, dbg=False)
    gdn.kda_commit(dims, m, w.t_lane, rec, S_dev)
    torch.cuda.synchronize()
    sl = [0, 47]
    q64, k64, v64, b64, _ = (a[sl] for a in w.as_f64())
    g64 = gk[sl].astype(np.float64)
    o_ref, _ = oracle.kda_verify(q64, k64, v64, b64, g64, S0[sl], w.t_lane)
    e_o = o_rel_err(o.cpu().numpy()[sl], o_ref, w.t_lane)
    S_ref = oracle.kda_commit(q64, k64, v64, b64, g64, S0[sl], m)
    S_all = S_dev.cpu().numpy()
    e_s = s_rel_err(S_all[sl], S_ref)
    say("  kda full batch T=%d, layers %s: o err %.2e S err %.2e" % (T, sl, e_o, e_s))
    assert e_o <= TOL and e_s <= TOL
    d1 = gdn.Dims.of(1, 8, 32, 16, 128, 128, T)
    w1 = gs.WindowInputs(d1, True, w.q[:1], w.k[:1], w.v[:1], w.beta[:1],
                         w.g[:1], w.t_lane)
    S1 = to_dev(S0[:1], torch)
    _, rec1, dbg1 = _kda_run(d1, w1, gk[:1], S1)
    gdn.kda_commit(d1, m, w.t_lane, rec1, S1)
    torch.cuda.synchronize()
    dbg1, S1 = dbg1.cpu().numpy(), S1.cpu().numpy()
    for n in range(8):
        want = S0[:1, n] if m[n] == 0 else dbg1[:, n, m[n] - 1]
        assert np.array_equal(S1[:, n], want), n
    assert np.array_equal(S1, S_all[:1])


def test_kda_zero_gates_are_bitwise_identity():
    """beta = 0 and alpha = 1 on every channel: S * 1 then fma(0, k, S)
    leave the state bit for bit."""
    shape = gs.WindowShape(1, 2, 4, 2, 128, 128, 8)
    w = gs.window_inputs(shape, (601,))
    w.beta[:] = 0.0
    gk = np.zeros((1, 2, 8, 4, 128), np.float32)
    S0 = gs.initial_state(shape, (601,))
    dims = gdn.Dims.of(*shape.__dict__.values())
    S_dev = to_dev(S0, torch)
    _, rec, _ = _kda_run(dims, w, gk, S_dev, dbg=False)
    gdn.kda_commit(dims, w.t_lane, w.t_lane, rec, S_dev)
    torch.cuda.synchronize()
    assert np.array_equal(S_dev.cpu().numpy(), S0)


def test_kda_chained_rounds_48_layers():
    """48 layers x 2 lanes x 32/16 heads, T = 16, m ~ U{0..16}, 20 chained
    rounds; the oracle follows layers 0 and 47."""
    shape = gs.WindowShape(48, 2, 32, 16, 128, 128, 16)
    dims = gdn.Dims.of(*shape.__dict__.values())
    S0 = gs.initial_state(shape, (602,))
    S_dev = to_dev(S0, torch)
    sl = [0, 47]
    S_or = S0[sl].astype(np.float64)
    rec = torch.empty(gdn.kda_records_bytes(dims), dtype=torch.uint8,
                      device="cuda")
    o = torch.empty((48, 2, 16, 32, 128), device="cuda")
    t_lane = np.full(2, 16, np.int32)
    for r in range(20):
        w = gs.window_inputs(shape, (602, r))
        gk = gs.kda_gates(shape, (602, r), g_mean=-1.0)
        m = gs.accepted_uniform(t_lane, (602, r))
        q, k, v, beta, _ = window_to_dev(w, torch)
        gdn.kda_verify(dims, t_lane, q, k, v, beta, to_dev(gk, torch), S_dev,
                       o, rec)
        gdn.kda_commit(dims, m, t_lane, rec, S_dev)
        torch.cuda.synchronize()
        q64, k64, v64 = (gs.bf16_bits_to_f64(a[sl]) for a in (w.q, w.k, w.v))
        b64, g64 = w.beta[sl].astype(np.float64), gk[sl].astype(np.float64)
        o_ref, _ = oracle.kda_verify(q64, k64, v64, b64, g64, S_or, t_lane)
        S_or = oracle.kda_commit(q64, k64, v64, b64, g64, S_or, m)
        e_o = o_rel_err(o[sl].cpu().numpy(), o_ref, t_lane)
        e_s = s_rel_err(S_dev[sl].cpu().numpy(), S_or)
        if r % 5 == 0 or r == 19:
            say("  round %d: o err %.2e S err %.2e" % (r, e_o, e_s))
        assert e_o <= TOL and e_s <= TOL
