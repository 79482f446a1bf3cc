"""GPU tests of gdn_commit_verify, the fused commit of the previous window
and verify of the next one.

The fused call must reproduce the two-call sequence gdn_commit + gdn_verify
bit for bit (state, outputs, records, debug states) over chained rounds with
ragged windows, idle lanes, commit-only lanes and m = 0, and follow the fp64
oracle through the chain within 2e-4.  Every call goes through the C ABI.
"""
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


def _round_inputs(shape, key, r, bf16, idle_lane):
    w = gs.window_inputs(shape, key + (r,), bf16=bf16, ragged=True)
    t = w.t_lane.copy()
    if idle_lane is not None and r % 3 == 1:
        t[idle_lane] = 0          # a lane with nothing to verify this round
    w.t_lane = t
    m = gs.accepted_uniform(t, key + (r, 7))
    return w, m


CASES = [
    # (name, NL, N, Hv, Hk, dk, dv, T, bf16, rounds, dbg)
    ("d128_ragged", 2, 4, 4, 2, 128, 128, 16, True, 6, True),
    ("d64_col_tail", 1, 3, 2, 1, 64, 96, 5, True, 5, False),
    ("d32_f32", 1, 2, 3, 3, 32, 200, 7, False, 4, True),
    ("d16_f32", 2, 2, 2, 2, 16, 16, 4, False, 5, False),
    ("d128_dv256", 1, 3, 2, 1, 128, 256, 8, True, 4, True),
    ("d128_t40_long_window", 1, 3, 2, 1, 128, 128, 40, True, 3, False),
    ("d128_t64_blocks_dbg", 1, 2, 2, 1, 128, 128, 64, True, 3, True),
    ("d128_t17_blocks", 1, 4, 2, 1, 128, 128, 17, True, 4, True),
    ("f32_d128_blocks", 1, 3, 2, 1, 128, 128, 24, False, 4, True),
    # GDN_FLAG_TOKENWISE on both paths at a block-form shape
    ("d128_tokenwise", 1, 4, 2, 1, 128, 128, 16, True, 4, True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fused_equals_commit_then_verify(case):
    name, NL, N, Hv, Hk, dk, dv, T, bf16, rounds, dbg = case
    tw = name.endswith("tokenwise")
    say("case", name)
    shape = gs.WindowShape(NL, N, Hv, Hk, dk, dv, T)
    key = (200, zlib.crc32(name.encode()) % 1000)
    dims = gdn.Dims.of(NL, N, Hv, Hk, dk, dv, T)
    S0 = gs.initial_state(shape, key)
    S_a, S_b = to_dev(S0, torch), to_dev(S0, torch)
    nrec = gdn.records_bytes(dims)
    # record buffers alternate on both paths; the one a round writes is
    # cleared first so that unwritten bytes compare equal too
    rec_a = [torch.zeros(nrec, dtype=torch.uint8, device="cuda")
             for _ in range(2)]
    rec_b = [torch.zeros(nrec, dtype=torch.uint8, device="cuda")
             for _ in range(2)]
    oshape = (NL, N, T, Hv, dv)
    dshape = (NL, N, T, Hv, dk, dv)
    m_prev = np.zeros(N, np.int32)
    t_prev = np.zeros(N, np.int32)
    S_or = S0.astype(np.float64)
    for r in range(rounds):
        w, m = _round_inputs(shape, key, r, bf16, idle_lane=N - 1)
        q, k, v, beta, g = window_to_dev(w, torch)
        o_a = torch.full(oshape, float("nan"), device="cuda")
        o_b = torch.full(oshape, float("nan"), device="cuda")
        d_a = torch.full(dshape, float("nan"), device="cuda") if dbg else None
        d_b = torch.full(dshape, float("nan"), device="cuda") if dbg else None
        ap, an = rec_a[(r + 1) % 2], rec_a[r % 2]
        rp, rn = rec_b[(r + 1) % 2], rec_b[r % 2]
        an.zero_()
        rn.zero_()
        # two calls
        gdn.commit(dims, m_prev, t_prev, ap, S_a)
        gdn.verify(dims, w.t_lane, q, k, v, beta, g, S_a, o_a, an, d_a,
                   tokenwise=tw)
        # one fused call
        gdn.commit_verify(dims, m_prev, t_prev, None if r == 0 else rp,
                          w.t_lane, q, k, v, beta, g, S_b, o_b, rn, d_b,
                          tokenwise=tw)
        torch.cuda.synchronize()
        assert torch.equal(S_a, S_b), ("state", r)
        assert torch.equal(torch.nan_to_num(o_a, 7.0),
                           torch.nan_to_num(o_b, 7.0)), ("outputs", r)
        assert torch.equal(an, rn), ("records", r)
        if dbg:
            assert torch.equal(torch.nan_to_num(d_a, 7.0),
                               torch.nan_to_num(d_b, 7.0)), ("debug", r)
        # oracle: commit of the previous round, verify of this one
        q64, k64, v64, b64, g64 = w.as_f64()
        o_ref, _ = oracle.verify(q64, k64, v64, b64, g64, S_or, w.t_lane)
        e_o = o_rel_err(o_b.cpu().numpy(), o_ref, w.t_lane)
        e_s = s_rel_err(S_b.cpu().numpy(), S_or)
        say("  round %d: T=%s m_prev=%s o err %.2e S err %.2e" % (
            r, list(w.t_lane), list(m_prev), e_o, e_s))
        assert e_o <= TOL and e_s <= TOL
        S_or = oracle.commit(q64, k64, v64, b64, g64, S_or, m)
        m_prev, t_prev = m.astype(np.int32), w.t_lane.astype(np.int32)
    # the last round's commit alone (t_lane = 0 everywhere: commit only)
    zero = np.zeros(N, np.int32)
    gdn.commit(dims, m_prev, t_prev, rec_a[(rounds - 1) % 2], S_a)
    gdn.commit_verify(dims, m_prev, t_prev, rec_b[(rounds - 1) % 2], zero,
                      q, k, v, beta, g, S_b, o_b, rec_b[rounds % 2])
    torch.cuda.synchronize()
    assert torch.equal(S_a, S_b)
    assert s_rel_err(S_b.cpu().numpy(), S_or) <= TOL


def test_fused_one_lane_48_layers_chain():
    """48 layers x 1 lane x 32/16 heads, d = 128, T = 16, m ~ U{0..16}:
    30 fused rounds; the oracle follows layers 0 and 47 and the two-call
    path runs beside it (bitwise)."""
    shape = gs.ONE_LANE
    dims = gdn.Dims.of(*shape.__dict__.values())
    S0 = gs.initial_state(shape, (gs.KEY_ONE_LANE, 0))
    S_a, S_b = to_dev(S0, torch), to_dev(S0, torch)
    sl = [0, 47]
    S_or = S0[sl].astype(np.float64)
    nrec = gdn.records_bytes(dims)
    rec_a = torch.empty(nrec, dtype=torch.uint8, device="cuda")
    rec_b = [torch.empty(nrec, dtype=torch.uint8, device="cuda")
             for _ in range(2)]
    o_a = torch.empty((48, 1, 16, 32, 128), device="cuda")
    o_b = torch.empty_like(o_a)
    t = np.full(1, 16, np.int32)
    m_prev = np.zeros(1, np.int32)
    for r in range(30):
        w = gs.window_inputs(shape, (gs.KEY_ONE_LANE, 3000 + r))
        m = gs.accepted_uniform(t, (gs.KEY_ONE_LANE, r))
        q, k, v, beta, g = window_to_dev(w, torch)
        gdn.commit(dims, m_prev, t, rec_a, S_a)
        gdn.verify(dims, t, q, k, v, beta, g, S_a, o_a, rec_a)
        gdn.commit_verify(dims, m_prev, t, rec_b[(r + 1) % 2], t, q, k, v,
                          beta, g, S_b, o_b, rec_b[r % 2])
        torch.cuda.synchronize()
        assert torch.equal(S_a, S_b) and torch.equal(o_a, o_b), r
        q64, k64, v64 = (gs.bf16_bits_to_f64(a[sl]) for a in (w.q, w.k, w.v))
        b64, g64 = w.beta[sl].astype(np.float64), w.g[sl].astype(np.float64)
        o_ref, _ = oracle.verify(q64, k64, v64, b64, g64, S_or, t)
        e_o = o_rel_err(o_b[sl].cpu().numpy(), o_ref, t)
        e_s = s_rel_err(S_b[sl].cpu().numpy(), S_or)
        if r % 10 == 0 or r == 29:
            say("  round %d: m_prev=%d o err %.2e S err %.2e" % (
                r, m_prev[0], e_o, e_s))
        assert e_o <= TOL and e_s <= TOL
        S_or = oracle.commit(q64, k64, v64, b64, g64, S_or, m)
        m_prev = m.astype(np.int32)
