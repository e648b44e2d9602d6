"""Seeded layer cases shared by the GPU parity tests and the smoke check.

Inputs come from the seeded generator (synth); expected values from the CPU
oracle only. Nothing here calls the GPU library.
"""
from __future__ import annotations

import dataclasses

import numpy as np

import synth
from oracle import moe_oracle as O

REL_L2_BAR = 1e-3
MAX_ABS_BAR = 2e-2


@dataclasses.dataclass
class Case:
    H: int
    I: int
    E: int
    k: int
    G: int
    act: str
    T: int
    seed: int
    alpha: float = 0.0
    layer: int = 0
    x_bits: np.ndarray = None    # [T, H] act storage (uint16 bf16 bits or float32)
    x: np.ndarray = None         # [T, H] float64 values
    Wr_store: np.ndarray = None  # [E, H] act storage
    Wr: np.ndarray = None        # [E, H] float64 values
    b: np.ndarray = None         # [E] float32
    blobs: np.ndarray = None     # [E, expert_bytes] uint8
    bits: int = 4                # bits per weight code of the blobs


def make_case(H, I, E, k, G, act, T, seed, alpha=0.0, layer=0, std=0.02, only_experts=None, x_stream=0, bits=4):
    """A seeded layer. only_experts: if given, only those experts get generated weights;
    every other expert is filled with seeded random bytes (valid codes, finite scales)
    so that reading a wrong expert changes the result."""
    c = Case(H, I, E, k, G, act, T, seed, alpha, layer)
    c.x_bits = synth.activations(seed, x_stream, T, H, act, sub=layer)
    c.Wr_store = synth.router_weight(seed, layer, E, H, act)
    if act == "bf16":
        c.x = O.bf16_bits_to_f64(c.x_bits)
        c.Wr = O.bf16_bits_to_f64(c.Wr_store)
    else:
        c.x = c.x_bits.astype(np.float64)
        c.Wr = c.Wr_store.astype(np.float64)
    c.b = synth.router_bias(seed, layer, E, alpha)
    c.bits = bits
    eb = synth.expert_bytes(H, I, G, bits)
    if only_experts is None:
        c.blobs = synth.expert_blobs(seed, layer, 0, E, H, I, G, std, bits=bits)
    else:
        rng = np.random.default_rng(seed * 7919 + layer)
        c.blobs = rng.integers(0, 256, size=(E, eb), dtype=np.uint8)
        lay, _ = O.expert_layout(H, I, G, bits)
        # finite, small scales in the filler experts
        a0 = lay["s_gate"][0]
        c.blobs[:, a0:] = np.frombuffer(np.full((E * (eb - a0)) // 2, 0x2000, np.uint16).tobytes(),
                                        np.uint8).reshape(E, eb - a0)
        for e in sorted(set(int(v) for v in only_experts)):
            c.blobs[e] = synth.expert_blobs(seed, layer, e, 1, H, I, G, std, bits=bits)[0]
    return c


def oracle_logits(c: Case) -> np.ndarray:
    return O.router_logits(c.x, c.Wr, c.b)


def oracle_forward(c: Case, logits_in=None, tokens=None):
    return O.layer_forward(c.x, c.Wr, c.b, c.blobs, c.H, c.I, c.E, c.k, c.G, c.act, logits_in=logits_in,
                           tokens=tokens, bits=getattr(c, "bits", 4))


def rel_l2(a, ref):
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(a - ref) / max(np.linalg.norm(ref), 1e-300))


def max_abs(a, ref):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(ref, np.float64))))


def routing_margins(logits: np.ndarray, k: int) -> np.ndarray:
    """Per token, the smallest gap among the k+1 largest logits (ordering and cut)."""
    s = -np.sort(-np.asarray(logits, np.float64), axis=1)
    kk = min(k + 1, s.shape[1])
    return np.min(s[:, :kk - 1] - s[:, 1:kk], axis=1) if kk > 1 else np.full(s.shape[0], np.inf)


def valid_topk(logits_row, ids, k, tol):
    """ids (slot order) is the top-k of some logits within tol of logits_row."""
    l = np.asarray(logits_row, np.float64)
    sel = np.asarray(ids)
    if len(set(sel.tolist())) != k:
        return False
    rest = np.setdiff1d(np.arange(l.size), sel)
    if rest.size and l[sel].min() < l[rest].max() - 2 * tol:
        return False
    return bool(np.all(np.diff(l[sel]) <= 2 * tol))


def random_code_blobs(E, H, I, G, seed, p_minus8=0.3, bits=4):
    """Canonical blobs whose codes cover every value of the format: for 4-bit codes the code
    -8 (nibble 0x8) drawn with probability p_minus8 and the other 15 uniformly; for 2- and
    3-bit codes every n uniformly. fp16 group scales near 0.8 / sqrt(K E[q^2]), so that g, u
    and o stay of order one. Packed by the generator's C packers."""
    rng = np.random.default_rng(seed)
    eq2 = {4: 32.0, 3: 21.0, 2: 5.0}[bits]

    def codes(rows, K):
        if bits < 4:
            return rng.integers(0, 1 << bits, size=(rows, K)).astype(np.uint8)
        q = rng.integers(-7, 8, size=(rows, K)).astype(np.int8)
        q[rng.random((rows, K)) < p_minus8] = -8
        return q

    def scales(rows, K):
        s = 0.8 / np.sqrt(eq2 * K) * rng.uniform(0.5, 1.5, size=(rows, K // G))
        return s.astype(np.float16).view(np.uint16)

    out = []
    for _ in range(E):
        out.append(synth.pack_blob(codes(I, H), codes(I, H), codes(H, I), scales(I, H), scales(I, H),
                                   scales(H, I), bits=bits))
    return np.stack(out)


def tie_logits(T, E, k, seed):
    """Router logits [T, E] float32 with exact ties at the top-k cut and inside the
    top k, and +0.0 / -0.0 pairs: values from a small set {-1, -0.5, 0, 0.5, 1}
    with random zero signs; every 5th token has all logits zero (mixed signs, the
    answer is experts 0..k-1), every 5th + 1 one high logit at the last expert and a
    tie of every other expert at 0.5 or -0.0/+0.0, every 5th + 2 exactly k+1 experts
    tied at the maximum (the cut falls inside the tie)."""
    rng = np.random.default_rng(seed)
    vals = np.array([-1.0, -0.5, 0.0, 0.5, 1.0], np.float32)
    L = rng.choice(vals, size=(T, E)).astype(np.float32)
    for t in range(T):
        kind = t % 5
        if kind == 0:
            L[t] = 0.0
        elif kind == 1:
            L[t] = 0.5 if t % 2 else 0.0
            L[t, E - 1] = 1.0
        elif kind == 2:
            L[t] = -1.0
            top = rng.choice(E, size=min(k + 1, E), replace=False)
            L[t, top] = 0.0
    neg = (L == 0) & (rng.random((T, E)) < 0.5)
    L[neg] = -0.0
    return L
