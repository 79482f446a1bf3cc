"""The entry points under HIP graph capture.

Every entry point launches kernels only (no memset, no allocation, no
synchronisation), so a caller can capture a serving loop into a HIP graph.
Each graph here is replayed three times, with eager work of the program
(state reset, a synchronisation) between the replays, and every replay is
checked bit for bit against the same calls run eagerly: chained fused
commit + verify rounds on both verify kernels, and the prefill entry point
that allocates nothing.  Every call goes through the C ABI.
"""
import sys

import numpy as np
import pytest

import gdn_synth as gs
from tests.gpu_util import to_dev, window_to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import commit_gated_delta_amd as gdn  # noqa: E402


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


ROUND_CASES = [
    # (name, NL, N, Hv, Hk, dk, dv, t_max, bf16): the matrix-core verify
    # (bf16, d = 128, t_max <= 16) and the token-by-token one (f32)
    ("matrix_core", 8, 4, 4, 2, 128, 128, 16, True),
    ("token_by_token", 2, 3, 4, 2, 64, 64, 8, False),
]


@pytest.mark.parametrize("case", ROUND_CASES, ids=[c[0] for c in ROUND_CASES])
def test_fused_rounds_replay_bitwise_from_a_graph(case):
    name, NL, N, Hv, Hk, dk, dv, tm, bf16 = case
    say("case", name)
    shape = gs.WindowShape(NL, N, Hv, Hk, dk, dv, tm)
    dims = gdn.Dims.of(*shape.__dict__.values())
    R = 4
    wins = [gs.window_inputs(shape, (800, r), bf16=bf16, ragged=True)
            for r in range(R)]
    ins = [window_to_dev(w, torch) for w in wins]
    m = [gs.accepted_uniform(w.t_lane, (800, r)) for r, w in enumerate(wins)]
    zero = np.zeros(N, dtype=np.int32)
    S0 = to_dev(gs.initial_state(shape, (800,)), torch)
    nrec = gdn.records_bytes(dims)

    def buffers():
        return (S0.clone(),
                torch.zeros((NL, N, tm, Hv, dv), device="cuda"),
                [torch.zeros(nrec, dtype=torch.uint8, device="cuda")
                 for _ in range(2)])

    def rounds(S, o, recs, stream):
        for r in range(R):
            mp, tp = (zero, zero) if r == 0 else (m[r - 1], wins[r - 1].t_lane)
            gdn.commit_verify(dims, mp, tp, recs[(r + 1) % 2], wins[r].t_lane,
                              *ins[r], S, o, recs[r % 2], stream=stream)

    S_e, o_e, rec_e = buffers()
    rounds(S_e, o_e, rec_e, None)
    torch.cuda.synchronize()
    want = (S_e.cpu(), o_e.cpu(), rec_e[(R - 1) % 2].cpu())

    S_g, o_g, rec_g = buffers()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            rounds(S_g, o_g, rec_g, None)
    torch.cuda.synchronize()
    for rep in range(3):
        S_g.copy_(S0)          # eager work between the replays
        o_g.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (S_g.cpu(), o_g.cpu(), rec_g[(R - 1) % 2].cpu())
        for a, b in zip(got, want):
            assert torch.equal(a, b), (name, rep)
        say("  replay %d bitwise equal to eager" % rep)


def test_noalloc_prefill_replays_bitwise_from_a_graph():
    L, Hv, Hk, interval = 1000, 4, 2, 256
    p = gs.prefill_inputs(L, Hv, Hk, 128, 128, (801,))
    q, k, v = (to_dev(x[None], torch) for x in (p.q, p.k, p.v))
    beta, gg = to_dev(p.beta[None], torch), to_dev(p.g[None], torch)
    S_init = to_dev(gs.prefill_state(Hv, 128, 128, (801,))[None], torch)
    n_ck = L // interval

    def outputs():
        return (torch.zeros((1, Hv, 128, 128), device="cuda"),
                torch.zeros((1, L, Hv, 128), device="cuda"),
                torch.zeros((1, n_ck, Hv, 128, 128), device="cuda"))

    def run(Sf, o, ck):
        gdn.prefill_chunked_noalloc(1, L, Hv, Hk, 128, 128, q, k, v, beta, gg,
                                    S_init, Sf, o, ck, ckpt_interval=interval)

    want = outputs()
    run(*want)
    torch.cuda.synchronize()
    want = tuple(x.cpu() for x in want)
    got = outputs()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            run(*got)
    torch.cuda.synchronize()
    for rep in range(3):
        for x in got:
            x.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(got, want):
            assert torch.equal(a.cpu(), b), rep
        say("  prefill replay %d bitwise equal to eager" % rep)
