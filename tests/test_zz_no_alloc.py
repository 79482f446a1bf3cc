"""gdn_prefill_chunked_noalloc (the prefill whose workspace is the
library's fixed scratch array) against gdn_prefill_chunked with a
caller-allocated workspace: bit for bit on the outputs, every checkpoint and
the final state, on two calls in a row, the second with a smaller input (the
scratch array keeps the first call's contents).  Both calls go through the C
ABI."""
import sys

import numpy as np
import pytest

import gdn_synth as gs
from tests.gpu_util import to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import commit_gated_delta_amd as gdn  # noqa: E402


def _inputs(n_seqs, L, Hv, Hk, seed):
    xs = [gs.prefill_inputs(L, Hv, Hk, 128, 128, (seed, s))
          for s in range(n_seqs)]
    st = lambda nm: to_dev(np.stack([getattr(x, nm) for x in xs]), torch)
    S0 = to_dev(np.stack([gs.prefill_state(Hv, 128, 128, (seed, s))
                          for s in range(n_seqs)]), torch)
    return st("q"), st("k"), st("v"), st("beta"), st("g"), S0


def _run(noalloc, n_seqs, L, Hv, Hk, interval, ins):
    q, k, v, beta, g, S0 = ins
    Sf = torch.full((n_seqs, Hv, 128, 128), float("nan"), device="cuda")
    o = torch.full((n_seqs, L, Hv, 128), float("nan"), device="cuda")
    n_ck = L // interval
    ck = torch.full((n_seqs, n_ck, Hv, 128, 128), float("nan"),
                    device="cuda") if n_ck else None
    if noalloc:
        gdn.prefill_chunked_noalloc(n_seqs, L, Hv, Hk, 128, 128, q, k, v,
                                    beta, g, S0, Sf, o, ck,
                                    ckpt_interval=interval)
    else:
        ws = torch.empty(gdn.prefill_workspace_bytes(n_seqs, L, Hv, Hk, 128,
                                                     128),
                         dtype=torch.uint8, device="cuda")
        gdn.prefill_chunked(n_seqs, L, Hv, Hk, 128, 128, q, k, v, beta, g,
                            S0, Sf, o, ck, ws, ckpt_interval=interval)
    torch.cuda.synchronize()
    return (o.cpu().numpy(), Sf.cpu().numpy(),
            None if ck is None else ck.cpu().numpy())


@pytest.mark.parametrize("sizes", [
    # (n_seqs, L, Hv, Hk, interval): the second call is smaller than the
    # first, and its chunk-head blocks sit where the first call left data
    ((2, 1000, 8, 4, 256), (1, 333, 4, 4, 128)),
    ((1, 4096, 16, 16, 1024), (1, 100, 2, 1, 64)),
    # both calls in segments (one sequence, few heads, more than 4,096
    # tokens): the segment buffers live in the scratch array too
    ((1, 3 * 4096 + 500, 2, 1, 4096), (1, 4096 + 64, 2, 2, 4096)),
    ((2, 2 * 4096 + 300, 4, 2, 8192), (3, 4096 + 1, 2, 1, 4096)),
])
def test_noalloc_matches_workspace_entry_point(sizes):
    for i, (n, L, Hv, Hk, iv) in enumerate(sizes):
        print("noalloc call %d: n_seqs=%d L=%d Hv=%d Hk=%d interval=%d"
              % (i, n, L, Hv, Hk, iv), flush=True)
        sys.stdout.flush()
        assert (gdn.prefill_workspace_bytes(n, L, Hv, Hk, 128, 128)
                <= gdn.PREFILL_SCRATCH_BYTES)
        ins = _inputs(n, L, Hv, Hk, 7000 + 10 * i + L)
        want = _run(False, n, L, Hv, Hk, iv, ins)
        got = _run(True, n, L, Hv, Hk, iv, ins)
        for a, b in zip(got, want):
            if b is None:
                assert a is None
                continue
            assert np.isfinite(b).all()
            assert np.array_equal(a, b)


def test_noalloc_refuses_sizes_beyond_the_scratch_array():
    L, Hv = 32768, 32
    assert (gdn.prefill_workspace_bytes(1, L, Hv, Hv, 128, 128)
            > gdn.PREFILL_SCRATCH_BYTES)
    x = torch.empty(16, dtype=torch.bfloat16, device="cuda")
    f = torch.empty(16, device="cuda")
    st = gdn.prefill_chunked_noalloc(1, L, Hv, Hv, 128, 128, x, x, x, f, f,
                                     None, f, f, None, raw_status=True)
    assert st == gdn.GDN_EWORKSPACE
