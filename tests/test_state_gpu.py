"""GPU tests of gdn_state_snapshot / gdn_state_restore: exact copies of the
recurrent state of chosen lanes to device or pinned host memory and back,
checked bit for bit against the oracle's definition, and a request that is
paused and resumed in another lane continuing bit for bit.  Every call goes
through the C ABI."""
import sys

import numpy as np
import pytest

import gdn_synth as gs
import oracle
from tests.gpu_util import to_dev, window_to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import commit_gated_delta_amd as gdn  # noqa: E402


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("pinned", [False, True], ids=["device", "pinned_host"])
def test_snapshot_and_restore_are_exact(pinned):
    shape = gs.WindowShape(3, 6, 4, 2, 64, 96, 4)
    dims = gdn.Dims.of(*shape.__dict__.values())
    S0 = gs.initial_state(shape, (300,))
    S = to_dev(S0, torch)
    lanes = [4, 1, 4, 0]
    shp = (len(lanes), 3, 4, 64, 96)
    snap = (torch.full(shp, float("nan"), pin_memory=True) if pinned
            else torch.full(shp, float("nan"), device="cuda"))
    gdn.state_snapshot(dims, lanes, S, snap)
    torch.cuda.synchronize()
    assert np.array_equal(snap.cpu().numpy(), oracle.snapshot(S0, lanes))
    # restore the snapshots of lanes 4 and 1 into lanes 2 and 5 (two
    # requests move), leaving the other lanes as they are
    gdn.state_restore(dims, [2, 5], snap[:2], S)
    torch.cuda.synchronize()
    want = oracle.restore(S0, [2, 5], oracle.snapshot(S0, [4, 1]))
    assert np.array_equal(S.cpu().numpy(), want)


def test_paused_request_resumes_bit_for_bit_in_another_lane():
    """Round 1 on all lanes; lane 1 is paused (snapshot to pinned host, its
    lane reused by another request), then resumed in lane 3 for round 2.
    Its outputs and state equal those of the same request never paused."""
    shape = gs.WindowShape(2, 4, 4, 2, 128, 128, 8)
    dims = gdn.Dims.of(*shape.__dict__.values())
    S0 = gs.initial_state(shape, (301,))
    w1 = gs.window_inputs(shape, (301, 1))
    m1 = gs.accepted_uniform(w1.t_lane, (301, 1))
    rec = torch.empty(gdn.records_bytes(dims), dtype=torch.uint8, device="cuda")
    o = torch.empty((2, 4, 8, 4, 128), device="cuda")

    def round_(S, w, m):
        q, k, v, b, g = window_to_dev(w, torch)
        out = torch.full_like(o, float("nan"))
        gdn.verify(dims, w.t_lane, q, k, v, b, g, S, out, rec)
        gdn.commit(dims, m, w.t_lane, rec, S)
        return out

    S_ref = to_dev(S0, torch)
    S_run = to_dev(S0, torch)
    round_(S_ref, w1, m1)
    round_(S_run, w1, m1)
    snap = torch.empty((1, 2, 4, 128, 128), pin_memory=True)
    gdn.state_snapshot(dims, [1], S_run, snap)
    torch.cuda.synchronize()
    # lane 1 is taken by another request; lane 3's old request finished
    S_run[:, 1].normal_()
    gdn.state_restore(dims, [3], snap, S_run)
    # round 2: the paused request's window goes to lane 3
    w2 = gs.window_inputs(shape, (301, 2))
    m2 = gs.accepted_uniform(w2.t_lane, (301, 2))
    w2m = gs.window_inputs(shape, (301, 2))
    m2m = m2.copy()
    for name in ("q", "k", "v", "beta", "g"):
        getattr(w2m, name)[:, 3] = getattr(w2, name)[:, 1]
    w2m.t_lane[3] = w2.t_lane[1]
    m2m[3] = m2[1]
    o_ref = round_(S_ref, w2, m2)
    o_run = round_(S_run, w2m, m2m)
    torch.cuda.synchronize()
    assert torch.equal(torch.nan_to_num(o_ref[:, 1], 7.0),
                       torch.nan_to_num(o_run[:, 3], 7.0))
    assert torch.equal(S_ref[:, 1], S_run[:, 3])


def test_full_batch_snapshot_round_trip():
    """8 lanes x 48 layers x 32 heads x 128 x 128 (768 MiB): snapshot of all
    lanes in reverse order to pinned host memory, restore, identical."""
    shape = gs.EIGHT_LANES
    dims = gdn.Dims.of(*shape.__dict__.values())
    say("full batch: state")
    S = torch.randn((48, 8, 32, 128, 128), device="cuda")
    ref = S.clone()
    lanes = list(range(7, -1, -1))
    snap = torch.empty((8, 48, 32, 128, 128), pin_memory=True)
    gdn.state_snapshot(dims, lanes, S, snap)
    torch.cuda.synchronize()
    for j in (0, 3, 7):
        assert torch.equal(snap[j].cuda(), ref[:, lanes[j]])
    S.zero_()
    gdn.state_restore(dims, lanes, snap, S)
    torch.cuda.synchronize()
    assert torch.equal(S, ref)
