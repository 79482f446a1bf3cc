"""Helpers shared by the GPU tests: device copies of seeded inputs and the
parity metric.

Parity metric (tolerance 2e-4): for every (layer, lane, value head) block,
max |x - ref| / max |ref| over the block's elements (all tokens and columns
of o, or all d_k x d_v entries of S); the test takes the maximum over
blocks.  Element-wise ratios are meaningless near zero, so the error is
measured against the block's largest reference magnitude.
"""
import numpy as np

TOL = 2e-4


def block_rel_err(x, ref, n_block_axes, move=None):
    """x, ref: arrays of equal shape.  If ``move`` is given it is a
    transpose that brings the block axes first.  Returns the max over blocks
    of max|x - ref| / max|ref| (blocks whose reference is all zero compare
    max|x| against 1)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if move is not None:
        x = np.transpose(x, move)
        ref = np.transpose(ref, move)
    nb = int(np.prod(x.shape[:n_block_axes]))
    x = x.reshape(nb, -1)
    ref = ref.reshape(nb, -1)
    num = np.max(np.abs(x - ref), axis=1)
    den = np.max(np.abs(ref), axis=1)
    den = np.where(den > 0, den, 1.0)
    return float(np.max(num / den))


def o_rel_err(o, o_ref, t_lane):
    """o: [NL, N, T, Hv, dv]; rows t >= t_lane are excluded (set to 0 on
    both sides after the caller checked them)."""
    o = np.array(o, dtype=np.float64, copy=True)
    ref = np.array(o_ref, dtype=np.float64, copy=True)
    T = o.shape[2]
    mask = np.arange(T)[None, :] < np.asarray(t_lane)[:, None]   # [N, T]
    m = mask[None, :, :, None, None]
    o = np.where(m, o, 0.0)
    ref = np.where(m, ref, 0.0)
    return block_rel_err(o, ref, 3, move=(0, 1, 3, 2, 4))


def s_rel_err(S, S_ref):
    """S: [NL, N, Hv, dk, dv]."""
    return block_rel_err(S, S_ref, 3)


def to_dev(a, torch, device="cuda"):
    """numpy -> torch device tensor; uint16 arrays are bf16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def window_to_dev(w, torch):
    return (to_dev(w.q, torch), to_dev(w.k, torch), to_dev(w.v, torch),
            to_dev(w.beta, torch), to_dev(w.g, torch))
