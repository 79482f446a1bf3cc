"""GPU tests of gdn_verify_tree / gdn_commit_path (draft-tree windows):
parity with the fp64 oracle per node, and the commit of an accepted
root-to-node path bit for bit equal to the state verify held at that node.
Every call goes through the C ABI; tolerance 2e-4 block-relative."""
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


def _run_tree(dims, w, parent, S_dev, dbg=True):
    q, k, v, beta, g = window_to_dev(w, torch)
    o = torch.full((dims.n_layers, dims.n_lanes, dims.t_max, dims.h_v,
                    dims.d_v), float("nan"), device="cuda")
    rec = torch.empty(gdn.records_bytes(dims), dtype=torch.uint8, device="cuda")
    d = None
    if dbg:
        d = torch.full((dims.n_layers, dims.n_lanes, dims.t_max, dims.h_v,
                        dims.d_k, dims.d_v), float("nan"), device="cuda")
    gdn.verify_tree(dims, w.t_lane, [list(p) for p in parent], q, k, v, beta,
                    g, S_dev, o, rec, d)
    return o, rec, d


def _check_tree(name, shape, bf16, parent_fn, g_fill=None, n_paths=4):
    key = (500, zlib.crc32(name.encode()) % 1000)
    w = gs.window_inputs(shape, key, bf16=bf16, ragged=True)
    if g_fill is not None:
        g_fill(w.g)
    parent = parent_fn(w.t_lane, shape.t_max, key)
    S0 = gs.initial_state(shape, key)
    dims = gdn.Dims.of(*shape.__dict__.values())
    S_dev = to_dev(S0, torch)
    o, rec, dbg = _run_tree(dims, w, parent, S_dev)
    torch.cuda.synchronize()
    assert torch.equal(S_dev.cpu(), torch.from_numpy(S0)), "verify wrote S0"
    o_np, dbg_np = o.cpu().numpy(), dbg.cpu().numpy()
    q64, k64, v64, b64, g64 = w.as_f64()
    o_ref, st_ref = oracle.verify_tree(q64, k64, v64, b64, g64, S0, w.t_lane,
                                       parent, want_states=True)
    e_o = o_rel_err(o_np, o_ref, w.t_lane)
    say("  %s: T=%s o err %.2e" % (name, list(w.t_lane), e_o))
    assert e_o <= TOL
    for t in range(shape.t_max):
        lanes = [n for n in range(shape.n_lanes) if w.t_lane[n] > t]
        if lanes:
            assert s_rel_err(dbg_np[:, lanes, t], st_ref[:, lanes, t]) <= TOL, t
    for r in range(n_paths):
        paths = gs.accepted_tree_paths(parent, w.t_lane, key + (r,))
        S_c = to_dev(S0, torch)
        gdn.commit_path(dims, paths, w.t_lane, [list(p) for p in parent], rec,
                        S_c)
        S_c = S_c.cpu().numpy()
        for n, p in enumerate(paths):
            want = S0[:, n] if not p else dbg_np[:, n, p[-1]]
            assert np.array_equal(S_c[:, n], want), (r, n, p)
        S_ref = oracle.commit_path(q64, k64, v64, b64, g64, S0,
                                   [len(p) for p in paths], paths)
        assert s_rel_err(S_c, S_ref) <= TOL


def _star(t_lane, t_max, key):
    p = np.full((len(t_lane), t_max), -1, dtype=np.int32)
    p[:, 1:] = 0
    for n, t in enumerate(t_lane):
        p[n, t:] = -1
    return p


CASES = [
    # (name, NL, N, Hv, Hk, dk, dv, T, bf16)
    ("bf16_d128", 2, 3, 4, 2, 128, 128, 16, True),
    ("bf16_d64_tail", 1, 3, 2, 1, 64, 96, 12, True),
    ("f32_d32", 1, 2, 3, 3, 32, 64, 9, False),
    ("f32_d16", 2, 2, 2, 2, 16, 16, 7, False),
    ("bf16_d128_dv256", 1, 2, 2, 1, 128, 256, 10, True),
    # f32 inputs on the matrix cores (rows as three bf16 parts)
    ("f32_d128", 1, 3, 4, 2, 128, 128, 16, False),
    # trees of more than 16 nodes (the ABI takes 32): two blocks of 16 on
    # the matrix cores
    ("bf16_d128_32_nodes", 1, 2, 2, 1, 128, 128, 32, True),
    ("bf16_d128_29_nodes", 2, 3, 4, 2, 128, 128, 29, True),
    ("f32_d128_32_nodes", 1, 2, 2, 1, 128, 128, 32, False),
    ("bf16_d128_dv256_24_nodes", 1, 2, 2, 1, 128, 256, 24, True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_tree_parity_and_bitexact_path_commit(case):
    name, NL, N, Hv, Hk, dk, dv, T, bf16 = case
    _check_tree("dfs_" + name, gs.WindowShape(NL, N, Hv, Hk, dk, dv, T), bf16,
                gs.tree_parents)


@pytest.mark.parametrize("T", [16, 32])
def test_star_tree_rebuilds_at_every_node(T):
    """Every node hangs off the root: verify rebuilds the root's state before
    every node after the first child (with 32 nodes, every node of the
    second block has its parent in the first)."""
    _check_tree("star%d" % T, gs.WindowShape(1, 3, 4, 2, 128, 128, T), True,
                _star)


@pytest.mark.parametrize("T", [16, 32])
def test_tree_with_scale_folds(T):
    """Strong decay along deep branches: folds happen on some paths only
    (with 32 nodes also on paths that cross blocks), and alpha = 0 nodes."""
    def fill(g):
        g[:] = -3.0 - 0.5 * np.arange(g.shape[-1])[None, None, None, :]
        g[:, :, 5] = -np.inf
        if g.shape[2] > 20:
            g[:, :, 20, ::2] = -200.0
    _check_tree("folds%d" % T, gs.WindowShape(1, 3, 4, 2, 128, 128, T), True,
                lambda t, T_, key: gs.tree_parents(t, T_, key, p_deeper=0.85),
                g_fill=fill)


@pytest.mark.parametrize("bf16", [True, False], ids=["bf16", "f32"])
def test_tree_debug_states_leave_outputs_unchanged(bf16):
    """32-node trees (two blocks): asking for the debug states changes
    neither the outputs nor the records, bit for bit."""
    shape = gs.WindowShape(1, 3, 4, 2, 128, 128, 32)
    key = (503, int(bf16))
    w = gs.window_inputs(shape, key, bf16=bf16, ragged=True)
    w.t_lane[0] = 32
    parent = gs.tree_parents(w.t_lane, 32, key)
    S0 = gs.initial_state(shape, key)
    dims = gdn.Dims.of(*shape.__dict__.values())
    S_dev = to_dev(S0, torch)
    o1, r1, dbg = _run_tree(dims, w, parent, S_dev)
    o2, r2, _ = _run_tree(dims, w, parent, S_dev, dbg=False)
    torch.cuda.synchronize()
    assert torch.equal(torch.nan_to_num(o1, 7.0), torch.nan_to_num(o2, 7.0))
    paths = gs.accepted_tree_paths(parent, w.t_lane, key)
    Sa, Sb = to_dev(S0, torch), to_dev(S0, torch)
    plist = [list(p) for p in parent]
    gdn.commit_path(dims, paths, w.t_lane, plist, r1, Sa)
    gdn.commit_path(dims, paths, w.t_lane, plist, r2, Sb)
    assert torch.equal(Sa, Sb)
    say("  %s: outputs and records unchanged by debug states"
        % ("bf16" if bf16 else "f32"))


def test_chain_tree_matches_the_linear_window():
    """parent[t] = t - 1 is an ordinary window: outputs within tolerance of
    gdn_verify's (the scales are formed in another order) and both commits
    bit-exact against their own states."""
    shape = gs.WindowShape(2, 3, 4, 2, 128, 128, 16)
    w = gs.window_inputs(shape, (501,), ragged=True)
    S0 = gs.initial_state(shape, (501,))
    dims = gdn.Dims.of(*shape.__dict__.values())
    chain = [[t - 1 for t in range(16)] for _ in range(3)]
    S_dev = to_dev(S0, torch)
    o_t, rec_t, _ = _run_tree(dims, w, np.array(chain), S_dev, dbg=False)
    q, k, v, b, g = window_to_dev(w, torch)
    o_l = torch.empty_like(o_t)
    rec_l = torch.empty_like(rec_t)
    gdn.verify(dims, w.t_lane, q, k, v, b, g, S_dev, o_l, rec_l)
    torch.cuda.synchronize()
    e = o_rel_err(o_t.cpu().numpy(), o_l.cpu().numpy(), w.t_lane)
    say("  chain vs linear: %.2e" % e)
    assert e <= TOL
    m = gs.accepted_uniform(w.t_lane, (501,))
    S_a, S_b = to_dev(S0, torch), to_dev(S0, torch)
    gdn.commit_path(dims, [list(range(mm)) for mm in m], w.t_lane, chain,
                    rec_t, S_a)
    gdn.commit(dims, m, w.t_lane, rec_l, S_b)
    torch.cuda.synchronize()
    assert s_rel_err(S_a.cpu().numpy(), S_b.cpu().numpy()) <= TOL


@pytest.mark.parametrize("T", [16, 32])
def test_tree_full_batch_sampled_layer(T):
    """48 layers x 8 lanes x 32/16 heads, d = 128, DFS trees of up to 16 and
    32 nodes (the bench's tree workloads): the oracle follows layer 0
    (outputs and an accepted-path commit per lane), and the 48-layer commit
    of layer 0 matches a one-layer debug run bitwise."""
    shape = gs.WindowShape(gs.EIGHT_LANES.n_layers, gs.EIGHT_LANES.n_lanes,
                           gs.EIGHT_LANES.h_v, gs.EIGHT_LANES.h_k, 128, 128, T)
    dims = gdn.Dims.of(*shape.__dict__.values())
    key = (502,) if T == 16 else (502, T)
    w = gs.window_inputs(shape, key, ragged=True)
    w.t_lane[0] = T
    parent = gs.tree_parents(w.t_lane, T, key)
    paths = gs.accepted_tree_paths(parent, w.t_lane, key)
    S0 = gs.initial_state(shape, key)
    S_dev = to_dev(S0, torch)
    say("tree full batch, %d nodes: verify" % T)
    o, rec, _ = _run_tree(dims, w, parent, S_dev, dbg=False)
    gdn.commit_path(dims, paths, w.t_lane, [list(p) for p in parent], rec,
                    S_dev)
    torch.cuda.synchronize()
    q64, k64, v64, b64, g64 = (a[:1] for a in w.as_f64())
    o_ref, _ = oracle.verify_tree(q64, k64, v64, b64, g64, S0[:1], w.t_lane,
                                  parent)
    e_o = o_rel_err(o[:1].cpu().numpy(), o_ref, w.t_lane)
    S_ref = oracle.commit_path(q64, k64, v64, b64, g64, S0[:1],
                               [len(p) for p in paths], paths)
    e_s = s_rel_err(S_dev[:1].cpu().numpy(), S_ref)
    say("  layer 0: o err %.2e S err %.2e" % (e_o, e_s))
    assert e_o <= TOL and e_s <= TOL
    d1 = gdn.Dims.of(1, 8, 32, 16, 128, 128, T)
    w1 = gs.WindowInputs(d1, True, w.q[:1], w.k[:1], w.v[:1], w.beta[:1],
                         w.g[:1], w.t_lane)
    S1 = to_dev(S0[:1], torch)
    _, _, dbg1 = _run_tree(d1, w1, parent, S1)
    torch.cuda.synchronize()
    dbg1 = dbg1.cpu().numpy()
    S_all = S_dev.cpu().numpy()
    for n, p in enumerate(paths):
        want = S0[0, n] if not p else dbg1[0, n, p[-1]]
        assert np.array_equal(S_all[0, n], want), n
