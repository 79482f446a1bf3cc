"""GPU parity of gdn_prefill_chunked against the fp64 oracle; checkpoint
resume is bitwise; short prefills agree with verify.

Every call goes through the C ABI.  Tolerance: 2e-4 block-relative (per
head: max |x - ref| / max |ref| over the head's tokens and columns, or over
its state entries).
"""
import sys

import numpy as np
import pytest

import gdn_synth as gs
import oracle
from tests.gpu_util import TOL, block_rel_err, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import commit_gated_delta_amd as gdn  # noqa: E402


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_prefill(p, n_seqs_inputs, S_init=None, ckpt_interval=8192, scale=1.0,
                l2norm=True, chunk=64, segments=True):
    """p: list of PrefillInputs (one per sequence, equal shapes)."""
    n_seqs = len(n_seqs_inputs)
    L, Hv, Hk = p.seq_len, p.h_v, p.h_k
    stack = lambda name: np.stack([getattr(x, name) for x in n_seqs_inputs])
    q, k, v = (to_dev(stack(nm), torch) for nm in ("q", "k", "v"))
    beta, g = to_dev(stack("beta"), torch), to_dev(stack("g"), torch)
    Si = None if S_init is None else to_dev(np.ascontiguousarray(S_init), torch)
    Sf = torch.empty((n_seqs, Hv, 128, 128), device="cuda")
    o = torch.full((n_seqs, L, Hv, 128), float("nan"), device="cuda")
    n_ck = L // ckpt_interval
    ck = torch.full((n_seqs, max(n_ck, 1), Hv, 128, 128), float("nan"),
                    device="cuda") if n_ck > 0 else None
    ws = torch.empty(gdn.prefill_workspace_bytes(n_seqs, L, Hv, Hk, 128, 128,
                                                 chunk),
                     dtype=torch.uint8, device="cuda")
    gdn.prefill_chunked(n_seqs, L, Hv, Hk, 128, 128, q, k, v, beta, g, Si, Sf,
                        o, ck, ws, ckpt_interval=ckpt_interval, scale=scale,
                        l2norm=l2norm, chunk=chunk, segments=segments)
    torch.cuda.synchronize()
    return (o.cpu().numpy(), None if ck is None else ck.cpu().numpy(),
            Sf.cpu().numpy())


def oracle_prefill(p, S_init, ckpt_interval, scale=1.0, l2norm=True,
                   heads=None):
    q, k, v, b, g = p.as_f64()
    if heads is not None:   # heads are independent: run only some of them
        grp = p.h_v // p.h_k
        kidx = [h // grp for h in heads]
        q, k = q[:, kidx], k[:, kidx]
        v, b, g = v[:, heads], b[:, heads], g[:, heads]
        S_init = None if S_init is None else S_init[heads]
    return oracle.prefill(q, k, v, b, g, S_init, ckpt_interval=ckpt_interval,
                          scale=scale, l2norm=l2norm)


def o_err(o, ref):   # o: [L, H, dv] -> per head
    return block_rel_err(o, ref, 1, move=(1, 0, 2))


def o_err_blocks(o, ref, rows=64):
    """o: [L, H, dv]: the error per (head, block of `rows` tokens), each
    block against its own largest reference entry (so that small-magnitude
    stretches of a long sequence are not hidden by large ones)."""
    L, H, dv = o.shape
    nb = (L + rows - 1) // rows
    pad = nb * rows - L
    x = np.pad(np.asarray(o, np.float64), ((0, pad), (0, 0), (0, 0)))
    r = np.pad(np.asarray(ref, np.float64), ((0, pad), (0, 0), (0, 0)))
    x = x.reshape(nb, rows, H, dv).transpose(2, 0, 1, 3)
    r = r.reshape(nb, rows, H, dv).transpose(2, 0, 1, 3)
    return block_rel_err(x, r, 2)


def s_err(S, ref):   # S: [..., H, dk, dv] -> per head
    S = np.asarray(S).reshape(-1, 128, 128)
    ref = np.asarray(ref).reshape(-1, 128, 128)
    return block_rel_err(S, ref, 1)


CASES = [
    # (name, L, Hv, Hk, n_seqs, init, interval, scale, l2norm)
    ("one_chunk", 64, 2, 1, 1, False, 64, 1.0, True),
    ("tail_and_init", 200, 2, 1, 1, True, 64, 1.0, True),
    ("two_seqs_group2", 333, 4, 2, 2, True, 128, 0.5, True),
    ("eq_heads_no_init", 512, 4, 4, 1, False, 128, 1.0, True),
    ("short_tail", 70, 2, 2, 1, True, 64, 1.0, True),
    ("tiny", 5, 2, 1, 1, True, 64, 1.0, True),
    ("one_token", 1, 2, 1, 1, True, 64, 1.0, True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_prefill_parity(case):
    name, L, Hv, Hk, n_seqs, init, interval, scale, l2norm = case
    say("case", name)
    ins = [gs.prefill_inputs(L, Hv, Hk, 128, 128, (40, hash_case(name), s))
           for s in range(n_seqs)]
    S_init = None
    if init:
        S_init = np.stack([gs.prefill_state(Hv, 128, 128, (40, s))
                           for s in range(n_seqs)])
    o, ck, Sf = run_prefill(ins[0], ins, S_init, interval, scale, l2norm)
    for s in range(n_seqs):
        assert np.all(np.isfinite(o[s])), "unwritten output rows"
        o_ref, ck_ref, Sf_ref = oracle_prefill(
            ins[s], None if S_init is None else S_init[s].astype(np.float64),
            interval, scale, l2norm)
        e_o, e_s = o_err(o[s], o_ref), s_err(Sf[s], Sf_ref)
        say("  seq %d: o err %.2e  S err %.2e" % (s, e_o, e_s))
        assert e_o <= TOL and e_s <= TOL
        n_ck = L // interval
        for j in range(n_ck):
            assert s_err(ck[s, j], ck_ref[j]) <= TOL
        if n_ck and L % interval == 0:
            assert np.array_equal(ck[s, n_ck - 1], Sf[s])


def hash_case(name):
    import zlib
    return zlib.crc32(name.encode()) % 10000


def test_resume_from_checkpoint_is_bitwise():
    L, Hv, Hk, interval = 640, 4, 2, 128
    p = gs.prefill_inputs(L, Hv, Hk, 128, 128, (41,))
    S0 = gs.prefill_state(Hv, 128, 128, (41,))[None]
    o, ck, Sf = run_prefill(p, [p], S0, interval)
    for j in (0, 2):
        t = interval * (j + 1)
        tail = gs.PrefillInputs(L - t, Hv, Hk, 128, 128, True, p.q[t:], p.k[t:],
                                p.v[t:], p.beta[t:], p.g[t:])
        o2, _, Sf2 = run_prefill(tail, [tail], ck[:, j], interval)
        assert np.array_equal(Sf2, Sf), j
        assert np.array_equal(o2[0], o[0, t:]), j


def test_prefill_without_key_normalisation():
    """Flag L2NORM_QK off, with an output scale: the kernel takes the raw
    key and query rows.  Keys and queries are drawn pre-scaled by d_k^-1/2
    (rounded to bf16) so that the rule stays stable without the norm."""
    L, Hv, Hk, interval = 260, 4, 2, 128
    p = gs.prefill_inputs(L, Hv, Hk, 128, 128, (44,), g_mean=0.0)
    p.k = gs.f32_to_bf16_bits(gs.bf16_bits_to_f32(p.k) / np.sqrt(128.0))
    p.q = gs.f32_to_bf16_bits(gs.bf16_bits_to_f32(p.q) / np.sqrt(128.0))
    S0 = gs.prefill_state(Hv, 128, 128, (44,))[None]
    o, ck, Sf = run_prefill(p, [p], S0, interval, scale=0.7, l2norm=False)
    o_ref, ck_ref, Sf_ref = oracle_prefill(p, S0[0].astype(np.float64),
                                           interval, scale=0.7, l2norm=False)
    e_o, e_s = o_err(o[0], o_ref), s_err(Sf[0], Sf_ref)
    say("  no norm: o err %.2e  S err %.2e" % (e_o, e_s))
    assert e_o <= TOL and e_s <= TOL
    for j in range(L // interval):
        assert s_err(ck[0, j], ck_ref[j]) <= TOL


def test_prefill_zero_gates_keep_the_state_bitwise():
    """beta = 0 and g = 0: every chunk adds nothing and decays by exactly 1,
    so every checkpoint and S_final equal S_init bit for bit; the outputs
    are S_init q (parity)."""
    L, Hv, Hk, interval = 300, 2, 1, 128
    p = gs.prefill_inputs(L, Hv, Hk, 128, 128, (46,))
    p.beta[:] = 0.0
    p.g[:] = 0.0
    S0 = gs.prefill_state(Hv, 128, 128, (46,))[None]
    o, ck, Sf = run_prefill(p, [p], S0, interval)
    assert np.array_equal(Sf, S0)
    for j in range(L // interval):
        assert np.array_equal(ck[:, j], S0)
    o_ref, _, _ = oracle_prefill(p, S0[0].astype(np.float64), interval)
    assert o_err(o[0], o_ref) <= TOL


def test_prefill_orthonormal_keys_store_their_values():
    """Closed form of the delta write (no oracle involved): with alpha = 1,
    beta = 1 and orthonormal keys (a permuted standard basis, exact in
    bf16; norm flag off), the final state maps every key to its value: row
    j of the stored state (d_k x d_v) is the value written with key e_j."""
    L, Hv, Hk = 100, 2, 1
    p = gs.prefill_inputs(L, Hv, Hk, 128, 128, (47,), g_mean=0.0)
    perm = np.random.default_rng(47).permutation(128)[:L]
    k = np.zeros((L, Hk, 128), np.float32)
    k[np.arange(L), 0, perm] = 1.0
    p.k = gs.f32_to_bf16_bits(k)
    p.beta[:] = 1.0
    p.g[:] = 0.0
    S0 = gs.prefill_state(Hv, 128, 128, (47,))[None]
    _, _, Sf = run_prefill(p, [p], S0, 64, l2norm=False)
    v = gs.bf16_bits_to_f32(p.v)                      # [L, Hv, dv]
    for h in range(Hv):
        got = Sf[0, h][perm]                          # rows e_j -> values
        err = np.max(np.abs(got - v[:, h])) / np.max(np.abs(v[:, h]))
        say("  head %d: max rel err %.2e" % (h, err))
        assert err <= TOL


def test_prefill_zero_key_and_query_rows():
    """All-zero key or query rows inside chunks (the L2 norm then scales an
    exact 0): parity with the oracle on outputs, checkpoints and S_final."""
    L, Hv, Hk, interval = 200, 2, 1, 64
    p = gs.prefill_inputs(L, Hv, Hk, 128, 128, (45,), g_mean=0.0)
    for t in (0, 31, 64, 127, 150):
        p.k[t, 0] = 0
    for t in (3, 64, 199):
        p.q[t, 0] = 0
    S0 = gs.prefill_state(Hv, 128, 128, (45,))[None]
    o, ck, Sf = run_prefill(p, [p], S0, interval)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(Sf))
    o_ref, ck_ref, Sf_ref = oracle_prefill(p, S0[0].astype(np.float64), interval)
    assert o_err(o[0], o_ref) <= TOL and s_err(Sf[0], Sf_ref) <= TOL
    for j in range(L // interval):
        assert s_err(ck[0, j], ck_ref[j]) <= TOL


# positions (token, value head) of the planted gates: the first, a middle
# and the last token of chunks, two adjacent tokens, and the sequence's last
FORGET_AT = [(0, 0), (64, 1), (100, 0), (101, 0), (127, 1), (191, 0),
             (250, 1), (299, 0)]


@pytest.mark.parametrize("gate", ["alpha_zero", "strong_decay"])
def test_prefill_forgetting_gates(gate):
    """Tokens whose decay is exactly 0 (g = -inf) or vanishes in f32
    (g = -200) inside chunks: the state before them is forgotten.  Parity
    with the oracle on outputs, checkpoints and S_final, and bitwise resume
    from a checkpoint."""
    L, Hv, Hk, interval = 300, 2, 1, 128
    p = gs.prefill_inputs(L, Hv, Hk, 128, 128, (43, hash_case(gate)),
                          g_mean=0.0)
    val = -np.inf if gate == "alpha_zero" else -200.0
    for t, hh in FORGET_AT:
        p.g[t, hh] = val
    S0 = gs.prefill_state(Hv, 128, 128, (43,))[None]
    o, ck, Sf = run_prefill(p, [p], S0, interval)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(Sf))
    o_ref, ck_ref, Sf_ref = oracle_prefill(p, S0[0].astype(np.float64), interval)
    e_o, e_s = o_err(o[0], o_ref), s_err(Sf[0], Sf_ref)
    say("  %s: o err %.2e  S err %.2e" % (gate, e_o, e_s))
    assert e_o <= TOL and e_s <= TOL
    for j in range(L // interval):
        assert s_err(ck[0, j], ck_ref[j]) <= TOL
    t = interval
    tail = gs.PrefillInputs(L - t, Hv, Hk, 128, 128, True, p.q[t:], p.k[t:],
                            p.v[t:], p.beta[t:], p.g[t:])
    o2, _, Sf2 = run_prefill(tail, [tail], ck[:, 0], interval)
    assert np.array_equal(Sf2, Sf)
    assert np.array_equal(o2[0], o[0, t:])


def test_short_prefill_agrees_with_verify():
    """A prefill of T <= 16 tokens and a verify window over the same tokens
    run different kernels; both match the oracle, and each other."""
    T, Hv, Hk = 13, 4, 2
    p = gs.prefill_inputs(T, Hv, Hk, 128, 128, (42,), g_mean=0.0)
    S0 = gs.prefill_state(Hv, 128, 128, (42,))
    o_p, _, Sf_p = run_prefill(p, [p], S0[None], 64)
    dims = gdn.Dims.of(1, 1, Hv, Hk, 128, 128, T)
    q = to_dev(p.q[None, None], torch)
    k = to_dev(p.k[None, None], torch)
    v = to_dev(p.v[None, None], torch)
    b = to_dev(p.beta[None, None], torch)
    g = to_dev(p.g[None, None], torch)
    S = to_dev(S0[None, None], torch)
    o = torch.empty((1, 1, T, Hv, 128), device="cuda")
    rec = torch.empty(gdn.records_bytes(dims), dtype=torch.uint8, device="cuda")
    gdn.verify(dims, [T], q, k, v, b, g, S, o, rec)
    gdn.commit(dims, [T], [T], rec, S)
    o_v, S_v = o.cpu().numpy()[0, 0], S.cpu().numpy()[0, 0]
    assert o_err(o_p[0], o_v) <= TOL
    assert s_err(Sf_p[0], S_v) <= TOL


@pytest.mark.parametrize("hk", [32, 16])
def test_prefill_32k_tokens_32_heads(hk):
    """L = 32,768, 32 value heads, d = 128, g = -softplus(N(-2, 1)), zero
    initial state, checkpoints every 8,192 tokens, chunk 64.  The oracle runs
    all 32 heads; every checkpoint and S_final are compared per head, and
    the outputs per (head, 64-token block), each block against its own
    largest reference entry."""
    L, Hv = 32768, 32
    say("prefill 32k, h_k =", hk, ": generating")
    p = gs.prefill_inputs(L, Hv, hk, 128, 128, (4, hk))
    o, ck, Sf = run_prefill(p, [p], None, 8192)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(Sf))
    assert np.array_equal(ck[0, 3], Sf[0])
    say("  oracle on all %d heads" % Hv)
    o_ref, ck_ref, Sf_ref = oracle_prefill(p, None, 8192)
    e_o = o_err_blocks(o[0], o_ref)
    e_oh = o_err(o[0], o_ref)
    e_s = s_err(Sf[0], Sf_ref)
    e_c = max(s_err(ck[0, j], ck_ref[j]) for j in range(4))
    say("  o err per 64-token block %.2e (per head %.2e)  S err %.2e  "
        "ckpt err %.2e" % (e_o, e_oh, e_s, e_c))
    assert e_o <= TOL and e_s <= TOL and e_c <= TOL


def test_prefill_longest_sequence_of_the_pages():
    """The longest prefill the review reports (260,096 tokens: 4,064 chunks
    of 64, 31 checkpoints at 8,192), on 4 value heads sharing 2 key heads.
    The oracle runs value heads 0 and 3 (key heads 0 and 1): every
    checkpoint, S_final and the outputs per 64-token block."""
    L, Hv, Hk, interval = 260096, 4, 2, 8192
    heads = [0, 3]
    say("prefill %d tokens: generating" % L)
    p = gs.prefill_inputs(L, Hv, Hk, 128, 128, (49,))
    o, ck, Sf = run_prefill(p, [p], None, interval)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(Sf))
    n_ck = L // interval
    assert ck.shape[1] == n_ck == 31
    say("  oracle on value heads", heads)
    o_ref, ck_ref, Sf_ref = oracle_prefill(p, None, interval, heads=heads)
    e_o = o_err_blocks(o[0][:, heads], o_ref)
    e_s = s_err(Sf[0][heads], Sf_ref)
    e_c = max(s_err(ck[0, j][heads], ck_ref[j]) for j in range(n_ck))
    say("  o err per 64-token block %.2e  S err %.2e  ckpt err %.2e"
        % (e_o, e_s, e_c))
    assert e_o <= TOL and e_s <= TOL and e_c <= TOL


SEG = 4096  # tokens per segment of a segmented prefill


def _long_memory_inputs(L, Hv, Hk, key):
    """Prefill inputs whose state is remembered across a segment: slow
    gates (g = -softplus(N(-8, 1)), alpha^4096 ~ 0.25) and small write
    strengths (beta scaled by 0.02).  With the default synthetic gates and
    beta a chain forgets its start state within a few hundred tokens, and
    chains started from different states meet bit for bit long before a
    segment ends."""
    p = gs.prefill_inputs(L, Hv, Hk, 128, 128, key, g_mean=-8.0)
    p.beta[...] *= 0.02
    return p


def _tail_inputs(p, t):
    return gs.PrefillInputs(p.seq_len - t, p.h_v, p.h_k, 128, 128, True,
                            p.q[t:], p.k[t:], p.v[t:], p.beta[t:], p.g[t:])


def test_segmented_prefill_parity():
    """A sequence with few heads runs in segments of 4,096 tokens (each
    segment's transition and offset, a scan over the segments, then the
    outputs per segment).  Three full segments and a ragged tail, with an
    initial state and checkpoints at every segment boundary: the outputs
    per 64-token block, every checkpoint and S_final against the oracle.
    The same call with GDN_FLAG_PREFILL_ONE_CHAIN (one chain over the whole
    sequence) meets the same bar and agrees with it, but not bit for bit:
    the segments really ran."""
    L, Hv, Hk, interval = 3 * SEG + 1000, 2, 1, SEG
    p = _long_memory_inputs(L, Hv, Hk, (50,))
    S0 = gs.prefill_state(Hv, 128, 128, (50,))[None]
    seg = run_prefill(p, [p], S0, interval)
    one = run_prefill(p, [p], S0, interval, segments=False)
    o_ref, ck_ref, Sf_ref = oracle_prefill(p, S0[0].astype(np.float64),
                                           interval)
    for name, (o, ck, Sf) in (("segments", seg), ("one chain", one)):
        assert np.all(np.isfinite(o)) and np.all(np.isfinite(Sf))
        e_o, e_s = o_err_blocks(o[0], o_ref), s_err(Sf[0], Sf_ref)
        e_c = max(s_err(ck[0, j], ck_ref[j]) for j in range(L // interval))
        say("  %s: o err %.2e  S err %.2e  ckpt err %.2e"
            % (name, e_o, e_s, e_c))
        assert e_o <= TOL and e_s <= TOL and e_c <= TOL
    assert o_err_blocks(seg[0][0], one[0][0]) <= TOL
    assert s_err(seg[2][0], one[2][0]) <= TOL
    assert not np.array_equal(seg[2], one[2])


def test_segmented_prefill_resumes_bitwise():
    """Checkpoints every 8,192 tokens (two segments per interval): a prefill
    resumed from any checkpoint, itself in segments or a single segment,
    reproduces the rest bit for bit; a sequence that ends on a checkpoint
    has that checkpoint equal to S_final."""
    L, Hv, Hk, interval = 2 * 8192 + 3000, 2, 2, 8192
    p = _long_memory_inputs(L, Hv, Hk, (51,))
    o, ck, Sf = run_prefill(p, [p], None, interval)
    for j in range(L // interval):
        t = interval * (j + 1)
        tail = _tail_inputs(p, t)
        o2, _, Sf2 = run_prefill(tail, [tail], ck[:, j], interval)
        assert np.array_equal(Sf2, Sf), j
        assert np.array_equal(o2[0], o[0, t:]), j
    p2 = _long_memory_inputs(2 * 8192, Hv, Hk, (52,))
    _, ck2, Sf2 = run_prefill(p2, [p2], None, interval)
    assert np.array_equal(ck2[0, 1], Sf2[0])
    _, ck3, Sf3 = run_prefill(_tail_inputs(p2, 8192), [_tail_inputs(p2, 8192)],
                              ck2[:, 0], interval)
    assert np.array_equal(Sf3, Sf2)


def test_segmented_prefill_several_sequences():
    """Two sequences of 4 heads (8 sequence-heads, the most that run in
    segments), each with its own initial state and a ragged tail: every
    sequence's outputs per 64-token block, checkpoints and S_final against
    the oracle, and bit for bit the same sequence run alone (the segments of
    the sequences are independent parts of the same passes)."""
    L, Hv, Hk, interval = 2 * SEG + 700, 4, 2, SEG
    ps = [_long_memory_inputs(L, Hv, Hk, (54, i)) for i in range(2)]
    S0 = np.stack([gs.prefill_state(Hv, 128, 128, (54, i)) for i in range(2)])
    o, ck, Sf = run_prefill(ps[0], ps, S0, interval)
    for i, p in enumerate(ps):
        o_ref, ck_ref, Sf_ref = oracle_prefill(p, S0[i].astype(np.float64),
                                               interval)
        e_o, e_s = o_err_blocks(o[i], o_ref), s_err(Sf[i], Sf_ref)
        e_c = max(s_err(ck[i, j], ck_ref[j]) for j in range(L // interval))
        say("  sequence %d: o err %.2e  S err %.2e  ckpt err %.2e"
            % (i, e_o, e_s, e_c))
        assert e_o <= TOL and e_s <= TOL and e_c <= TOL
        o1, ck1, Sf1 = run_prefill(p, [p], S0[i:i + 1], interval)
        assert np.array_equal(o1[0], o[i]) and np.array_equal(Sf1[0], Sf[i])
        assert np.array_equal(ck1[0], ck[i])


@pytest.mark.parametrize("n_seqs,Hv,Hk,chunk", [(3, 2, 1, 32), (8, 1, 1, 64)])
def test_segmented_prefill_batch_matches_single_runs(n_seqs, Hv, Hk, chunk):
    """Batches at the segment limit in other shapes (3 x 2 heads with chunks
    of 32, 8 x 1 head): each sequence bit for bit its run alone, and within
    the tolerance of the one-chain call."""
    L = SEG + 300
    ps = [_long_memory_inputs(L, Hv, Hk, (55, n_seqs, i)) for i in range(n_seqs)]
    # an initial state, so that the scan multiplies by a transition (from
    # zero, two segments give exactly the one chain)
    S0 = np.stack([gs.prefill_state(Hv, 128, 128, (55, n_seqs, i))
                   for i in range(n_seqs)])
    o, _, Sf = run_prefill(ps[0], ps, S0, 8192, chunk=chunk)
    o2, _, Sf2 = run_prefill(ps[0], ps, S0, 8192, chunk=chunk, segments=False)
    for i, p in enumerate(ps):
        o1, _, Sf1 = run_prefill(p, [p], S0[i:i + 1], 8192, chunk=chunk)
        assert np.array_equal(o1[0], o[i]) and np.array_equal(Sf1[0], Sf[i]), i
        assert o_err_blocks(o[i], o2[i]) <= TOL and s_err(Sf[i], Sf2[i]) <= TOL
    assert not np.array_equal(Sf, Sf2)


def test_prefill_interval_off_the_segment_grid_runs_one_chain():
    """A checkpoint interval that is not a multiple of the segment length
    would put checkpoints inside segments: such a prefill runs as one chain,
    bit for bit the call with GDN_FLAG_PREFILL_ONE_CHAIN."""
    L, Hv, Hk, interval = 2 * SEG + 100, 2, 1, 2048
    p = gs.prefill_inputs(L, Hv, Hk, 128, 128, (53,))
    a = run_prefill(p, [p], None, interval)
    b = run_prefill(p, [p], None, interval, segments=False)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_segmented_prefill_chunk16():
    """Segments with 16-token chunks (256 chunks per segment) and a short
    tail, against the oracle."""
    L, Hv, Hk, interval = SEG + 500, 2, 2, SEG
    p = _long_memory_inputs(L, Hv, Hk, (54,))
    o, ck, Sf = run_prefill(p, [p], None, interval, chunk=16)
    o_ref, ck_ref, Sf_ref = oracle_prefill(p, None, interval)
    e_o, e_s = o_err_blocks(o[0], o_ref), s_err(Sf[0], Sf_ref)
    e_c = s_err(ck[0, 0], ck_ref[0])
    say("  o err %.2e  S err %.2e  ckpt err %.2e" % (e_o, e_s, e_c))
    assert e_o <= TOL and e_s <= TOL and e_c <= TOL


def test_chunk_sizes_agree():
    """The chunk length is an evaluation detail: chunks of 16, 32 and 64
    tokens give the same outputs, checkpoints and final state within the
    tolerance (each against the oracle and against each other), and for
    every chunk length a prefill resumed from a checkpoint reproduces the
    rest bit for bit.  A ragged tail (L % 64 != 0, L % 16 != 0) and an
    initial state are included."""
    L, Hv, Hk, interval = 650, 4, 2, 128
    p = gs.prefill_inputs(L, Hv, Hk, 128, 128, (48,))
    S0 = gs.prefill_state(Hv, 128, 128, (48,))[None]
    o_ref, ck_ref, Sf_ref = oracle_prefill(p, S0[0].astype(np.float64),
                                           interval)
    res = {}
    for C in (16, 32, 64):
        o, ck, Sf = run_prefill(p, [p], S0, interval, chunk=C)
        assert np.all(np.isfinite(o)) and np.all(np.isfinite(Sf))
        e_o, e_s = o_err_blocks(o[0], o_ref), s_err(Sf[0], Sf_ref)
        e_c = max(s_err(ck[0, j], ck_ref[j]) for j in range(L // interval))
        say("  chunk %d: o err %.2e  S err %.2e  ckpt err %.2e"
            % (C, e_o, e_s, e_c))
        assert e_o <= TOL and e_s <= TOL and e_c <= TOL
        res[C] = (o, ck, Sf)
        for j in (0, 3):
            t = interval * (j + 1)
            tail = gs.PrefillInputs(L - t, Hv, Hk, 128, 128, True, p.q[t:],
                                    p.k[t:], p.v[t:], p.beta[t:], p.g[t:])
            o2, _, Sf2 = run_prefill(tail, [tail], ck[:, j], interval,
                                     chunk=C)
            assert np.array_equal(Sf2, Sf), (C, j)
            assert np.array_equal(o2[0], o[0, t:]), (C, j)
    for a, b in ((16, 32), (32, 64), (16, 64)):
        assert o_err_blocks(res[a][0][0], res[b][0][0]) <= TOL, (a, b)
        assert s_err(res[a][2][0], res[b][2][0]) <= TOL, (a, b)
    # the chunks really differ in evaluation order: not bitwise the same
    assert not np.array_equal(res[16][2], res[64][2])
