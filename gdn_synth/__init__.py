"""Seeded synthetic inputs for the gated-delta verify / commit / prefill path.

This module is the only code shared by the oracle side (tests, CPU baseline)
and the HIP side (binding tests, benchmark).  It holds none of the method's
arithmetic: it draws random numbers, applies the input distributions
(sigmoid / softplus of normal draws for the gates) and rounds to bf16.

Distributions (stand-ins for real activations, which need trained weights):
  q, k, v  ~ N(0, 1), rounded to bf16 (round-to-nearest-even) unless fp32 is
           asked for.  q and k are drawn raw; the L2 normalisation is part of
           the method and is done by the kernels and by the oracle.
  beta     = sigmoid(N(0, 1))                       fp32
  g        = -softplus(N(mu_g, 1)), mu_g = 0 (window) or -2 (prefill) fp32
  S0       ~ N(0, 0.1^2)                            fp32
  T_lane   fixed, or Uniform{1..t_max} per lane (ragged windows)
  m_lane   Uniform{0..T_lane} or Binomial(T_lane, p) -- drawn from its own
           stream so that the window inputs do not depend on it.

Seeding: numpy PCG64 seeded by SeedSequence([BASE_SEED, stream, *keys]).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

BASE_SEED = 20261202
_STREAM_WINDOW, _STREAM_STATE, _STREAM_M, _STREAM_T, _STREAM_PREFILL = 1, 2, 3, 4, 5


def rng(stream: int, *keys: int) -> np.random.Generator:
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence([BASE_SEED, stream, *keys])))


# ---------------------------------------------------------------- bf16 bits
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16
    bit patterns.  Inputs are finite draws, so NaN handling is not needed."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64."""
    u = (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16)
    return u.view(np.float32).astype(np.float64)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    u = (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16)
    return u.view(np.float32)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _softplus(x):
    return np.logaddexp(0.0, x)


# ------------------------------------------------------------- window inputs
@dataclass
class WindowShape:
    n_layers: int
    n_lanes: int
    h_v: int
    h_k: int
    d_k: int
    d_v: int
    t_max: int


@dataclass
class WindowInputs:
    shape: WindowShape
    bf16: bool
    # q, k: [NL, N, T, Hk, dk]; v: [NL, N, T, Hv, dv]
    # uint16 bf16 bit patterns when bf16 is True, else float32
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    beta: np.ndarray          # float32 [NL, N, T, Hv]
    g: np.ndarray             # float32 [NL, N, T, Hv]
    t_lane: np.ndarray        # int32 [N]
    extra: dict = field(default_factory=dict)

    def as_f64(self):
        """(q, k, v, beta, g) widened exactly to float64 (oracle input)."""
        if self.bf16:
            q, k, v = (bf16_bits_to_f64(a) for a in (self.q, self.k, self.v))
        else:
            q, k, v = (a.astype(np.float64) for a in (self.q, self.k, self.v))
        return q, k, v, self.beta.astype(np.float64), self.g.astype(np.float64)


def window_inputs(shape: WindowShape, key: tuple, bf16: bool = True,
                  t_lane=None, ragged: bool = False, g_mean: float = 0.0
                  ) -> WindowInputs:
    """Draw one verify window for every (layer, lane).  ``key`` is a tuple of
    ints naming the case (case key, round, ...)."""
    s = shape
    r = rng(_STREAM_WINDOW, *key)
    qk_shape = (s.n_layers, s.n_lanes, s.t_max, s.h_k, s.d_k)
    v_shape = (s.n_layers, s.n_lanes, s.t_max, s.h_v, s.d_v)
    g_shape = (s.n_layers, s.n_lanes, s.t_max, s.h_v)
    q = r.standard_normal(qk_shape, dtype=np.float32)
    k = r.standard_normal(qk_shape, dtype=np.float32)
    v = r.standard_normal(v_shape, dtype=np.float32)
    beta = _sigmoid(r.standard_normal(g_shape)).astype(np.float32)
    g = (-_softplus(r.standard_normal(g_shape) + g_mean)).astype(np.float32)
    if bf16:
        q, k, v = f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)
    if t_lane is None:
        if ragged:
            t_lane = rng(_STREAM_T, *key).integers(1, s.t_max + 1, size=s.n_lanes)
        else:
            t_lane = np.full(s.n_lanes, s.t_max)
    t_lane = np.asarray(t_lane, dtype=np.int32)
    assert t_lane.shape == (s.n_lanes,)
    return WindowInputs(s, bf16, q, k, v, beta, g, t_lane)


def initial_state(shape: WindowShape, key: tuple, sigma: float = 0.1
                  ) -> np.ndarray:
    """S0 ~ N(0, sigma^2), float32 [NL, N, Hv, dk, dv]."""
    s = shape
    r = rng(_STREAM_STATE, *key)
    return (r.standard_normal((s.n_layers, s.n_lanes, s.h_v, s.d_k, s.d_v))
            * sigma).astype(np.float32)


def window_lengths(n_lanes: int, t_max: int, key: tuple) -> np.ndarray:
    """Ragged per-lane window lengths T ~ Uniform{1..t_max} (MTP windows of
    1..5 and DFlash windows of up to 15 drafts plus the anchor)."""
    r = rng(_STREAM_T, 7, *key)
    return r.integers(1, t_max + 1, size=n_lanes).astype(np.int32)


def accepted_uniform(t_lane: np.ndarray, key: tuple) -> np.ndarray:
    """m_lane ~ Uniform{0..T_lane} per lane."""
    r = rng(_STREAM_M, *key)
    return np.array([r.integers(0, int(t) + 1) for t in t_lane], dtype=np.int32)


def accepted_binomial(t_lane: np.ndarray, p: float, key: tuple) -> np.ndarray:
    """m_lane ~ Binomial(T_lane, p) per lane."""
    r = rng(_STREAM_M, *key)
    return np.array([r.binomial(int(t), p) for t in t_lane], dtype=np.int32)


# ------------------------------------------------------------ prefill inputs
@dataclass
class PrefillInputs:
    seq_len: int
    h_v: int
    h_k: int
    d_k: int
    d_v: int
    bf16: bool
    q: np.ndarray      # [L, Hk, dk]
    k: np.ndarray      # [L, Hk, dk]
    v: np.ndarray      # [L, Hv, dv]
    beta: np.ndarray   # float32 [L, Hv]
    g: np.ndarray      # float32 [L, Hv]

    def as_f64(self):
        if self.bf16:
            q, k, v = (bf16_bits_to_f64(a) for a in (self.q, self.k, self.v))
        else:
            q, k, v = (a.astype(np.float64) for a in (self.q, self.k, self.v))
        return q, k, v, self.beta.astype(np.float64), self.g.astype(np.float64)


def prefill_inputs(seq_len: int, h_v: int, h_k: int, d_k: int, d_v: int,
                   key: tuple, bf16: bool = True, g_mean: float = -2.0
                   ) -> PrefillInputs:
    r = rng(_STREAM_PREFILL, *key)
    q = r.standard_normal((seq_len, h_k, d_k), dtype=np.float32)
    k = r.standard_normal((seq_len, h_k, d_k), dtype=np.float32)
    v = r.standard_normal((seq_len, h_v, d_v), dtype=np.float32)
    beta = _sigmoid(r.standard_normal((seq_len, h_v))).astype(np.float32)
    g = (-_softplus(r.standard_normal((seq_len, h_v)) + g_mean)).astype(np.float32)
    if bf16:
        q, k, v = f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)
    return PrefillInputs(seq_len, h_v, h_k, d_k, d_v, bf16, q, k, v, beta, g)


def prefill_state(h_v: int, d_k: int, d_v: int, key: tuple, sigma: float = 0.1):
    r = rng(_STREAM_STATE, 99, *key)
    return (r.standard_normal((h_v, d_k, d_v)) * sigma).astype(np.float32)


# ------------------------------------------------------------ named cases
# Window shapes of the synthetic workloads, with the first seed-key entry
# each case uses (a stream identifier only).
TINY = WindowShape(1, 1, 2, 2, 16, 16, 4)          # 1 lane, 1 layer, d = 16, T = 4
ONE_LANE = WindowShape(48, 1, 32, 16, 128, 128, 16)       # 1 lane x 48 layers
EIGHT_LANES = WindowShape(48, 8, 32, 16, 128, 128, 16)    # 8 lanes x 48 layers
TWELVE_LANES_T6 = WindowShape(48, 12, 32, 16, 128, 128, 6)  # 12 lanes, T = 6
KEY_TINY, KEY_ONE_LANE, KEY_EIGHT_LANES, KEY_TWELVE_LANES = 0, 1, 2, 3


# ------------------------------------------------------------- draft trees
_STREAM_TREE = 9


def tree_parents(t_lane, t_max: int, key: tuple, p_deeper: float = 0.6):
    """Random draft trees, one per lane, in depth-first preorder: node 0 is
    the root (parent -1); every later node's parent is the previous node
    (probability p_deeper) or an ancestor of it on the current path.
    Returns int32 [n_lanes, t_max]; entries past t_lane are -1."""
    r = rng(_STREAM_TREE, *key)
    out = np.full((len(t_lane), t_max), -1, dtype=np.int32)
    for n, T in enumerate(t_lane):
        stack = []  # path from the root to the previous node
        for t in range(int(T)):
            if t == 0:
                out[n, t] = -1
                stack = [0]
                continue
            if r.random() < p_deeper:
                par = stack[-1]
            else:
                par = stack[int(r.integers(0, len(stack)))]
            while stack[-1] != par:
                stack.pop()
            out[n, t] = par
            stack.append(t)
    return out


def tree_path(parent_row, node: int):
    """Nodes from the root to ``node`` (inclusive), root first."""
    path = []
    while node >= 0:
        path.append(int(node))
        node = int(parent_row[node])
    return path[::-1]


def accepted_tree_paths(parent, t_lane, key: tuple):
    """For each lane an accepted path: the root-to-node path of a uniformly
    drawn node, or [] (nothing accepted) with probability 1/(T+1)."""
    r = rng(_STREAM_TREE + 1, *key)
    paths = []
    for n, T in enumerate(t_lane):
        node = int(r.integers(-1, int(T)))
        paths.append([] if node < 0 else tree_path(parent[n], node))
    return paths


# ------------------------------------------------------------- KDA gates
_STREAM_KDA = 11


def kda_gates(shape: WindowShape, key: tuple, g_mean: float = 0.0):
    """Per-channel log-decays of a KDA window: g = -softplus(N(g_mean, 1)),
    f32 [n_layers, n_lanes, t_max, h_v, d_k]."""
    s = shape
    r = rng(_STREAM_KDA, *key)
    x = r.standard_normal((s.n_layers, s.n_lanes, s.t_max, s.h_v, s.d_k)) + g_mean
    return (-_softplus(x)).astype(np.float32)
