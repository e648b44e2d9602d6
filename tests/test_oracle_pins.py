"""Pins of the CPU oracle against what mathematics and independent code fix.

Every check here compares the oracle with something other than itself: brute
force on tiny inputs, closed forms, invariants, library routines (NumPy, SciPy,
torch on the CPU) or the separately written C generator. A plausible mistake in
the oracle (a swapped gate/up, a transposed operand, a wrong group index, a
dropped bias, a wrong nibble order or tie-break) fails at least one of them.
"""
import itertools
import math
import os

import numpy as np
import pytest
import scipy.special

import synth
from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def sext4(n):
    """two's complement value of a 4-bit field, written arithmetically"""
    return n - 16 * (n >> 3)


# ----------------------------------------------------------------------------- int4 format


def test_unpack_inverts_c_packer_on_all_code_pairs():
    codes = np.array(list(itertools.product(range(-8, 8), repeat=2)), dtype=np.int8)  # [256, 2]
    packed = synth.pack_int4(codes)  # independent C packer
    assert packed.shape == (256, 1)
    np.testing.assert_array_equal(O.unpack_int4(packed), codes)


def test_unpack_then_pack_is_identity_on_all_bytes():
    b = np.arange(256, dtype=np.uint8).reshape(256, 1)
    q = O.unpack_int4(b)
    assert q.min() == -8 and q.max() == 7
    np.testing.assert_array_equal(synth.pack_int4(q), b)


def test_unpack_spec_bytes():
    # byte j = (q[2j] & 0xF) | (q[2j+1] & 0xF) << 4, nibbles two's complement
    for byte, lo, hi in [(0x00, 0, 0), (0x8F, -1, -8), (0x7F, -1, 7), (0x17, 7, 1), (0xF8, -8, -1),
                         (0x21, 1, 2)]:
        np.testing.assert_array_equal(O.unpack_int4(np.array([[byte]], np.uint8)), [[lo, hi]])
    for n in range(16):
        assert O.unpack_int4(np.array([[n]], np.uint8))[0, 0] == sext4(n)


def test_dequant_exact_in_fp32_for_every_code_and_fp16_scale():
    bits = np.arange(0, 0x7C00, dtype=np.uint16)  # every finite non-negative fp16
    s = bits.view(np.float16)
    s = np.concatenate([s, -s])
    for q in range(-8, 8):
        p32 = np.float32(q) * s.astype(np.float32)
        p64 = np.float64(q) * s.astype(np.float64)
        np.testing.assert_array_equal(p32.astype(np.float64), p64)


def test_dequant_group_indexing_brute_force():
    rng = np.random.default_rng(0)
    R, K, G = 3, 96, 32
    q = rng.integers(-8, 8, size=(R, K)).astype(np.int8)
    s = rng.standard_normal((R, K // G))
    W = O.dequant(q, s, G)
    for r in range(R):
        for k in range(K):
            assert W[r, k] == q[r, k] * s[r, k // G]


def _decode_bitstring(row_bytes, K, bits):
    """n codes of a canonical row, read off the row as one little-endian integer."""
    v = int.from_bytes(bytes(row_bytes), "little")
    return [(v >> (bits * i)) & ((1 << bits) - 1) for i in range(K)]


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_unpack_codes_every_code_at_every_alignment(bits):
    """Every pair of adjacent codes at every bit offset within a byte (3-bit codes cross
    byte boundaries), packed by the C packer and read back by the oracle, against a
    decode of the row as one integer and the format's q rule."""
    rng = np.random.default_rng(bits)
    L = 1 << bits
    rows = []
    for pos in range(8):
        for a in range(L):
            for c in range(L):
                n = rng.integers(0, L, size=32).astype(np.uint8)
                n[pos], n[pos + 1] = a, c
                rows.append(n)
    n = np.stack(rows)
    packed = synth.pack_codes(n, bits) if bits < 4 else synth.pack_int4(
        np.where(n >= 8, n.astype(np.int16) - 16, n).astype(np.int8))
    q = O.unpack_codes(packed, bits)
    for r in range(0, n.shape[0], 7):
        nn = _decode_bitstring(packed[r], 32, bits)
        assert nn == n[r].tolist()
    want = (n.astype(np.int16) - 16 * (n >= 8)) if bits == 4 else (2 * n.astype(np.int16) - (L - 1))
    np.testing.assert_array_equal(q, want)
    if bits == 4:
        np.testing.assert_array_equal(q, O.unpack_int4(packed))
    else:
        assert sorted(set(q.ravel().tolist())) == list(range(-(L - 1), L, 2))  # the odd levels


@pytest.mark.parametrize("bits", [2, 3])
def test_odd_level_quantiser_and_dequant(bits):
    """The generator's odd-level quantiser: |w - q s| <= s (1 + 2^-10) with q the nearest odd
    level; the expert blob of the generator holds exactly these codes and scales; q * s is
    exact in float32."""
    H, I, G = 128, 64, 64
    L = (1 << bits) - 1
    blob = synth.expert_blobs(9, 0, 3, 1, H, I, G, std=0.02, bits=bits)[0]
    Wg, Wu, Wd = O.expert_weights(blob, H, I, G, bits)
    for t, W, rows, K in ((0, Wg, I, H), (1, Wu, I, H), (2, Wd, H, I)):
        w = synth.expert_tensor_f32(9, 0, 3, t, rows, K)
        n, sb = synth.quantize_rows_odd(w, G, bits)
        s = O.fp16_bits_to_f64(sb)
        q = 2 * n.astype(np.float64) - L
        np.testing.assert_array_equal(W, q * np.repeat(s, G, axis=1))
        err = np.abs(w.astype(np.float64) - W)
        assert (err <= np.repeat(s, G, axis=1) * (1 + 2 ** -10) + 1e-12).all()
        p32 = (q.astype(np.float32) * np.repeat(s, G, axis=1).astype(np.float32)).astype(np.float64)
        np.testing.assert_array_equal(p32, W)


def test_expert_layout_sizes():
    assert O.expert_bytes(256, 128, 32) == 55296
    assert O.expert_bytes(2048, 768, 128) == 2433024
    assert O.expert_bytes(7168, 2048, 128) == 22708224
    assert O.expert_bytes(2048, 768, 128) == synth.expert_bytes(2048, 768, 128)
    for bits in (2, 3):
        assert O.expert_bytes(7168, 2048, 128, bits) == 3 * 7168 * 2048 * bits // 8 + 6 * 7168 * 2048 // 128
        assert O.expert_bytes(7168, 2048, 128, bits) == synth.expert_bytes(7168, 2048, 128, bits)


def test_expert_weights_split_matches_generator_tensors():
    # tiny expert built from known codes: every tensor and its scales land where the layout says
    rng = np.random.default_rng(1)
    H, I, G = 64, 32, 32
    qg, qu = rng.integers(-8, 8, (I, H)).astype(np.int8), rng.integers(-8, 8, (I, H)).astype(np.int8)
    qd = rng.integers(-8, 8, (H, I)).astype(np.int8)
    sg = np.array([[synth.f32_to_f16_bits(v) for v in row] for row in rng.uniform(0.1, 1, (I, H // G))], np.uint16)
    su = np.array([[synth.f32_to_f16_bits(v) for v in row] for row in rng.uniform(0.1, 1, (I, H // G))], np.uint16)
    sd = np.array([[synth.f32_to_f16_bits(v) for v in row] for row in rng.uniform(0.1, 1, (H, I // G))], np.uint16)
    blob = synth.pack_blob(qg, qu, qd, sg, su, sd)
    Wg, Wu, Wd = O.expert_weights(blob, H, I, G)
    for (W, q, s, K) in [(Wg, qg, sg, H), (Wu, qu, su, H), (Wd, qd, sd, I)]:
        sf = s.view(np.float16).astype(np.float64)
        for r in range(W.shape[0]):
            for k in range(K):
                assert W[r, k] == q[r, k] * sf[r, k // G]


# ----------------------------------------------------------------------------- rounding


def test_round_bf16_matches_torch_on_float32_values():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(2)
    v = np.concatenate([rng.standard_normal(20000).astype(np.float32),
                        (rng.standard_normal(2000) * 1e-39).astype(np.float32),  # subnormal range
                        (rng.standard_normal(2000) * 1e38).astype(np.float32),
                        np.array([0.0, -0.0, 3.3895314e38, 3.39e38], np.float32)])
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.round_bf16(v.astype(np.float64)), ref)


def test_round_bf16_ties_and_no_double_rounding():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even -> 1
    assert O.round_bf16(np.array([1 + 2 ** -8]))[0] == 1.0
    # 1 + 3*2^-8 is halfway between 1+2^-7 and 1+2^-6: even is 1+2^-6
    assert O.round_bf16(np.array([1 + 3 * 2 ** -8]))[0] == 1 + 2 ** -6
    # just above the tie (only representable in float64): rounds up; a float32 detour
    # would first round to the tie and then to even (down)
    v = 1 + 2 ** -8 + 2 ** -40
    assert np.float32(v) == np.float32(1 + 2 ** -8)
    assert O.round_bf16(np.array([v]))[0] == 1 + 2 ** -7
    assert O.round_bf16(np.array([-v]))[0] == -(1 + 2 ** -7)


def test_bf16_bits_to_f64_every_pattern_against_field_decode_and_torch():
    """All 65,536 bf16 bit patterns: the oracle's widening equals (a) the value the
    sign / 8-bit exponent / 7-bit fraction fields define, built with exact float64
    arithmetic (normal: (1 + f/128) 2^(e-127); subnormal: f/128 2^-126; e = 255:
    inf or NaN), and (b) torch's bfloat16 -> float64 conversion on the CPU."""
    torch = pytest.importorskip("torch")
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = O.bf16_bits_to_f64(bits)
    sign = np.where(bits >> 15, -1.0, 1.0)
    e = ((bits >> 7) & 0xFF).astype(np.int64)
    f = (bits & 0x7F).astype(np.float64)
    want = np.where(e == 0, np.ldexp(f / 128.0, -126), np.ldexp(1.0 + f / 128.0, (e - 127).clip(-126, 127)))
    want = sign * want
    special = e == 255
    want = np.where(special & (f == 0), sign * np.inf, want)
    want = np.where(special & (f != 0), np.nan, want)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    np.testing.assert_array_equal(got[ok], want[ok])
    np.testing.assert_array_equal(np.signbit(got[ok]), np.signbit(want[ok]))  # -0.0 stays -0.0
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(got[ok], ref[ok])
    assert np.isnan(ref[~ok]).all()
    # spot values: 1.0, -2.0, the largest finite, the smallest subnormal
    for b, v in [(0x3F80, 1.0), (0xC000, -2.0), (0x7F7F, float(np.ldexp(255.0, 120))), (0x0001, 2.0 ** -133)]:
        assert O.bf16_bits_to_f64(np.array([b], np.uint16))[0] == v


def test_round_act_f32_is_numpy_cast():
    v = np.array([1 / 3, 2 / 3, 1e-50, 1e300])
    np.testing.assert_array_equal(O.round_act(v, "f32"), v.astype(np.float32).astype(np.float64))


# ----------------------------------------------------------------------------- router / top-k


def test_router_logits_brute_force():
    rng = np.random.default_rng(3)
    T, E, H = 3, 5, 7
    # values with few significant bits so every product and sum is exact in float64
    x = rng.integers(-64, 64, (T, H)) / 16.0
    Wr = rng.integers(-64, 64, (E, H)) / 256.0
    b = rng.integers(-8, 8, E) / 4.0
    lg = O.router_logits(x, Wr, b)
    assert lg.dtype == np.float32
    for t in range(T):
        for e in range(E):
            ref = math.fsum(x[t, h] * Wr[e, h] for h in range(H)) + b[e]
            assert lg[t, e] == np.float32(ref)
    # the bias takes part: zero weights give logits equal to the bias
    np.testing.assert_array_equal(O.router_logits(x, np.zeros((E, H)), b), np.tile(b.astype(np.float32), (T, 1)))


def brute_rank(l, e):
    return sum(1 for f in range(len(l)) if l[f] > l[e] or (l[f] == l[e] and f < e))


@pytest.mark.parametrize("seed", range(20))
def test_topk_brute_force_rank(seed):
    rng = np.random.default_rng(seed)
    E = int(rng.integers(1, 40))
    k = int(rng.integers(1, E + 1))
    # few distinct values so ties are common
    l = rng.integers(-4, 4, E).astype(np.float32) / 2
    ids = O.topk_ids(l, k)
    for e in range(E):
        r = brute_rank(l, e)
        if r < k:
            assert ids[r] == e
        else:
            assert e not in ids
    np.testing.assert_array_equal(ids, np.lexsort((np.arange(E), -l.astype(np.float64)))[:k])


def test_topk_constructed_ties():
    np.testing.assert_array_equal(O.topk_ids(np.zeros(8, np.float32), 3), [0, 1, 2])
    l = np.array([0.0, -0.0, 0.0, 1.0], np.float32)  # -0.0 ties with +0.0
    np.testing.assert_array_equal(O.topk_ids(l, 3), [3, 0, 1])
    l = np.array([1.0, 5.0, 5.0, 2.0, 5.0], np.float32)
    np.testing.assert_array_equal(O.topk_ids(l, 4), [1, 2, 4, 3])


def test_topk_rejects_nan():
    with pytest.raises(AssertionError):
        O.topk_ids(np.array([0.0, np.nan], np.float32), 1)


def test_gate_weights_properties():
    rng = np.random.default_rng(4)
    for _ in range(50):
        E = int(rng.integers(2, 50))
        k = int(rng.integers(1, E + 1))
        l = (rng.standard_normal(E) * 3).astype(np.float32)
        ids = O.topk_ids(l, k)
        w = O.gate_weights(l[ids].astype(np.float64))
        assert abs(w.sum() - 1) < 1e-12
        assert np.all(np.diff(w) <= 0)  # slot order is logit order
        full = scipy.special.softmax(l.astype(np.float64))
        np.testing.assert_allclose(w, full[ids] / full[ids].sum(), rtol=1e-12)
        np.testing.assert_allclose(O.gate_weights(l[ids].astype(np.float64) + 123.0), w, rtol=1e-12)
    assert O.gate_weights(np.array([3.7]))[0] == 1.0
    # k = E: the plain softmax
    l = np.array([0.5, -1.0, 2.0])
    np.testing.assert_allclose(O.gate_weights(l[O.topk_ids(l, 3)]), np.sort(scipy.special.softmax(l))[::-1],
                               rtol=1e-14)


# ----------------------------------------------------------------------------- align / permute


@pytest.mark.parametrize("seed", range(10))
def test_align_permute_brute_force(seed):
    rng = np.random.default_rng(seed)
    E = int(rng.integers(1, 20))
    T, k = int(rng.integers(1, 12)), int(rng.integers(1, E + 1))
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    counts, offsets, sorted_, inv = O.align_permute(ids, E)
    a_ids = ids.ravel()
    n = a_ids.size
    for e in range(E):
        assert counts[e] == sum(1 for a in range(n) if a_ids[a] == e)
    assert offsets[0] == 0 and offsets[-1] == n == T * k
    for e in range(E):
        assert offsets[e + 1] - offsets[e] == counts[e]
    for a in range(n):
        p = sum(1 for b in range(n) if (a_ids[b], b) < (a_ids[a], a))
        assert sorted_[p] == a and inv[a] == p
    np.testing.assert_array_equal(sorted_[inv], np.arange(n))


# ----------------------------------------------------------------------------- expert FFN


def make_blob(Wq, H, I, G, scales=None):
    """blob from code matrices (gate, up, down) and optional fp16 scale arrays (default 1.0)."""
    qg, qu, qd = Wq
    one = synth.f32_to_f16_bits(1.0)
    sg = np.full((I, H // G), one, np.uint16) if scales is None else scales[0]
    su = np.full((I, H // G), one, np.uint16) if scales is None else scales[1]
    sd = np.full((H, I // G), one, np.uint16) if scales is None else scales[2]
    return synth.pack_blob(qg, qu, qd, sg, su, sd)


def f16(v):
    return synth.f32_to_f16_bits(float(v))


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_ffn_diagonal_closed_form(act):
    """Wg = diag(a), Wu = diag(b), Wd = c * P (a non-symmetric permutation):
    y[P(i)] = c_i * rho(silu(a_i x_i) * b_i x_i). Scales differ per group and the unused
    groups carry different scales, so a wrong group index, a gate/up swap, a transposed
    down matrix or a wrong nibble order all change y."""
    D, G = 64, 32
    rng = np.random.default_rng(5)
    perm = np.roll(np.arange(D), 5)  # i -> perm[i]
    qg = np.zeros((D, D), np.int8); qu = np.zeros((D, D), np.int8); qd = np.zeros((D, D), np.int8)
    a_q = rng.integers(1, 8, D); b_q = -rng.integers(1, 8, D)
    for i in range(D):
        qg[i, i] = a_q[i]
        qu[i, i] = b_q[i]
        qd[perm[i], i] = 1
    sg = np.zeros((D, D // G), np.uint16); su = np.zeros((D, D // G), np.uint16); sd = np.zeros((D, D // G), np.uint16)
    for r in range(D):
        for g in range(D // G):
            sg[r, g] = f16(0.25 * (1 + g) + 0.125 * (r % 3))
            su[r, g] = f16(0.5 * (2 - g) + 0.0625 * (r % 5))
            sd[r, g] = f16(2.0 ** (g - 1) * (1 + (r % 2)))
    blob = make_blob((qg, qu, qd), D, D, G, (sg, su, sd))
    x = rng.standard_normal((4, D))
    if act == "bf16":
        x = O.round_bf16(x)
    res = O.layer_forward(x, np.zeros((1, D)), None, blob[None], D, D, 1, 1, G, act)
    fs = lambda s: s.view(np.float16).astype(np.float64)
    for t in range(4):
        for i in range(D):
            g = a_q[i] * fs(sg)[i, i // G] * x[t, i]
            u = b_q[i] * fs(su)[i, i // G] * x[t, i]
            h = O.round_act(np.array([g / (1 + math.exp(-g)) * u]), act)[0]
            assert res["y"][t, perm[i]] == pytest.approx(fs(sd)[perm[i], i // G] * h, rel=1e-15, abs=0)


def test_ffn_identity_expert_closed_form():
    """Identity gate, up and down (q = 1 on the diagonal, s = 1): y = rho(x^2 * sigmoid(x))."""
    D, G = 32, 32
    eye = np.eye(D, dtype=np.int8)
    blob = make_blob((eye, eye, eye), D, D, G)
    x = O.round_bf16(np.random.default_rng(6).standard_normal((5, D)) * 3)
    y = O.layer_forward(x, np.zeros((1, D)), None, blob[None], D, D, 1, 1, G, "bf16")["y"]
    ref = O.round_bf16(x * x * scipy.special.expit(x))
    np.testing.assert_allclose(y, ref, rtol=1e-15, atol=0)


def tiny_layer(seed, H=64, I=32, E=6, G=32, bits=4):
    blobs = synth.expert_blobs(100 + seed, 0, 0, E, H, I, G, std=0.05, bits=bits)
    rng = np.random.default_rng(seed)
    x = O.round_bf16(rng.standard_normal((7, H)))
    Wr = O.round_bf16(rng.standard_normal((E, H)) * 0.1)
    b = (rng.standard_normal(E) * 0.5).astype(np.float32)
    return blobs, x, Wr, b


@pytest.mark.parametrize("k,bits", [(1, 4), (2, 4), (3, 4), (6, 4), (2, 3), (3, 2)])
def test_layer_matches_dense_brute_force(k, bits):
    """Every expert on every token (einsum over all experts at once), masked by top-k."""
    H, I, E, G = 64, 64 if bits < 4 else 32, 6, 64 if bits < 4 else 32
    blobs, x, Wr, b = tiny_layer(k, H, I, E, G, bits)
    res = O.layer_forward(x, Wr, b, blobs, H, I, E, k, G, "bf16", bits=bits)
    Ws = [O.expert_weights(blobs[e], H, I, G, bits) for e in range(E)]
    Wg = np.stack([w[0] for w in Ws]); Wu = np.stack([w[1] for w in Ws]); Wd = np.stack([w[2] for w in Ws])
    g = np.einsum("eih,th->tei", Wg, x)
    u = np.einsum("eih,th->tei", Wu, x)
    h = O.round_bf16(g * scipy.special.expit(g) * u)
    o = np.einsum("ehi,tei->teh", Wd, h)  # [T, E, H]
    logits = (x @ Wr.T + b.astype(np.float64)).astype(np.float32)
    mask = np.zeros((x.shape[0], E))
    for t in range(x.shape[0]):
        order = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))[:k]
        z = np.exp(logits[t, order].astype(np.float64) - logits[t, order].max())
        mask[t, order] = z / z.sum()
    y_dense = np.einsum("te,teh->th", mask, o)
    np.testing.assert_allclose(res["y"], y_dense, rtol=1e-12, atol=1e-14)


def test_layer_token_order_invariance_bitwise():
    H, I, E, G = 64, 32, 6, 32
    blobs, x, Wr, b = tiny_layer(11, H, I, E, G)
    res = O.layer_forward(x, Wr, b, blobs, H, I, E, 2, G, "bf16")
    perm = np.random.default_rng(0).permutation(x.shape[0])
    res_p = O.layer_forward(x[perm], Wr, b, blobs, H, I, E, 2, G, "bf16")
    np.testing.assert_array_equal(res_p["y"], res["y"][perm])
    np.testing.assert_array_equal(res_p["ids"], res["ids"][perm])


@pytest.mark.parametrize("k", [1, 2, 4])
def test_identical_experts_give_the_single_ffn(k):
    H, I, E, G = 64, 32, 4, 32
    one = synth.expert_blobs(7, 0, 0, 1, H, I, G, std=0.05)
    blobs = np.repeat(one, E, axis=0)
    _, x, Wr, b = tiny_layer(3, H, I, E, G)
    y = O.layer_forward(x, Wr, b, blobs, H, I, E, k, G, "bf16")["y"]
    y1 = O.layer_forward(x, Wr[:1], b[:1], one, H, I, 1, 1, G, "bf16")["y"]
    np.testing.assert_allclose(y, y1, rtol=1e-12, atol=1e-15)


def test_zero_expert_and_scale_doubling():
    H, I, G = 64, 32, 32
    blob = synth.expert_blobs(9, 0, 0, 1, H, I, G, std=0.05)[0]
    _, x, _, _ = tiny_layer(4, H, I, 1, G)
    lay, _ = O.expert_layout(H, I, G)
    zero = blob.copy()
    zero[lay["q_gate"][0]:lay["q_down"][1]] = 0
    y0 = O.layer_forward(x, np.zeros((1, H)), None, zero[None], H, I, 1, 1, G, "bf16")["y"]
    assert np.all(y0 == 0)
    y = O.layer_forward(x, np.zeros((1, H)), None, blob[None], H, I, 1, 1, G, "bf16")["y"]
    dbl = blob.copy()
    sd = dbl[lay["s_down"][0]:lay["s_down"][1]].view(np.uint16)
    sd[:] = (sd.view(np.float16).astype(np.float32) * 2).astype(np.float16).view(np.uint16)
    y2 = O.layer_forward(x, np.zeros((1, H)), None, dbl[None], H, I, 1, 1, G, "bf16")["y"]
    np.testing.assert_array_equal(y2, 2 * y)


def test_logits_in_overrides_router():
    H, I, E, G = 64, 32, 6, 32
    blobs, x, Wr, b = tiny_layer(12, H, I, E, G)
    lg = np.tile(np.arange(E, dtype=np.float32), (x.shape[0], 1))  # expert E-1 best
    res = O.layer_forward(x, Wr, b, blobs, H, I, E, 2, G, "bf16", logits_in=lg)
    assert np.all(res["ids"] == [E - 1, E - 2])
    sub = O.layer_forward(x, Wr, b, blobs, H, I, E, 2, G, "bf16", logits_in=lg, tokens=[3, 1])
    np.testing.assert_array_equal(sub["y"], res["y"][[3, 1]])


# ----------------------------------------------------------------------------- residency / cache


def test_link_accounting_recount():
    rng = np.random.default_rng(8)
    E, T, k = 10, 5, 3
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    res = rng.integers(0, 2, E)
    acc = O.link_accounting(ids, res, 100)
    hits = sum(1 for t in range(T) for j in range(k) if res[ids[t, j]])
    assert acc["hits"] == hits and acc["misses"] == T * k - hits
    uniq = set(ids.ravel().tolist())
    assert acc["bytes_hbm"] == 100 * sum(1 for e in uniq if res[e])
    assert acc["bytes_host"] == 100 * sum(1 for e in uniq if not res[e])


def test_cache_policy_hand_cases():
    # E = 5, 2 slots: experts 0, 1 resident. Counts favour 3 then 4.
    score, slot_of, done, ev = O.cache_policy_step(np.zeros(5), [0, 1, 0, 9, 5], [0, 1, -1, -1, -1], 2, 0.9, 8)
    assert done == [(3, 0), (4, 1)] and ev == [0, 1]
    np.testing.assert_array_equal(slot_of, [-1, -1, -1, 0, 1])
    # max_promotions = 1: only the best candidate, evicting the weakest resident (0, score 0 < 1)
    _, slot_of, done, ev = O.cache_policy_step(np.zeros(5), [0, 1, 0, 9, 5], [0, 1, -1, -1, -1], 2, 0.9, 1)
    assert done == [(3, 0)] and ev == [0]
    # a tie with a resident keeps the resident (resident first); ties among non-residents -> lower id
    _, slot_of, done, ev = O.cache_policy_step(np.zeros(4), [2, 0, 2, 2], [0, 1, -1, -1], 2, 0.9, 8)
    assert done == [(2, 1)] and ev == [1]
    # empty slots fill first, lowest slot first, with no victim
    _, slot_of, done, ev = O.cache_policy_step(np.zeros(4), [0, 3, 4, 0], [-1, -1, -1, 2], 3, 0.9, 8)
    assert done == [(2, 0), (1, 1)] and ev == []
    # decay then add, in float64
    score, *_ = O.cache_policy_step(np.array([10.0, 1.0]), [1, 2], [0, -1], 1, 0.9, 8)
    assert score[0] == 0.9 * 10.0 + 1 and score[1] == 0.9 * 1.0 + 2


def test_cache_policy_converges_to_top_counts():
    rng = np.random.default_rng(9)
    E, S = 40, 12
    p = 1.0 / np.arange(1, E + 1) ** 0.8
    p = p[rng.permutation(E)]
    slot_of = np.full(E, -1); slot_of[:S] = np.arange(S)
    score = np.zeros(E)
    for _ in range(200):
        counts = rng.multinomial(64, p / p.sum())
        score, slot_of, done, ev = O.cache_policy_step(score, counts, slot_of, S, 0.9, 4)
        assert len(done) <= 4
        assert sorted(slot_of[slot_of >= 0].tolist()) == list(range(S))  # slots stay a bijection
    top = set(np.argsort(-p, kind="stable")[:S].tolist())
    assert len(top & set(np.nonzero(slot_of >= 0)[0].tolist())) >= S - 2


def test_cache_set_resident_hand_cases():
    # residents 0 (slot 1) and 2 (slot 0); want {2, 3, 4} over 3 slots: 0 evicted (slot 1
    # freed), 3 takes slot 1, 4 the never-used slot 2; 2 keeps slot 0
    score, slot_of, done, ev = O.cache_set_resident(np.zeros(5), [1, 0, 2, 0, 0], [1, -1, 0, -1, -1],
                                                    [0, 0, 1, 1, 1], 3, 0.5)
    assert ev == [0] and done == [(3, 1), (4, 2)]
    assert slot_of.tolist() == [-1, -1, 0, 1, 2]
    assert score.tolist() == [1.0, 0.0, 2.0, 0.0, 0.0]
    # want nothing: every resident goes back to its host copy, nothing promoted
    _, slot_of, done, ev = O.cache_set_resident(np.zeros(3), [0, 0, 0], [0, 1, -1], [0, 0, 0], 2, 0.9)
    assert done == [] and ev == [0, 1] and (slot_of == -1).all()
    with pytest.raises(AssertionError):
        O.cache_set_resident(np.zeros(3), [0, 0, 0], [-1, -1, -1], [1, 1, 1], 2, 0.9)


def test_cache_set_resident_reaches_the_wanted_set():
    """From random tables to random wanted sets: afterwards exactly the wanted experts
    are resident, slots are distinct and in range, and a resident that stays wanted
    keeps its slot."""
    rng = np.random.default_rng(11)
    for _ in range(200):
        E, S = int(rng.integers(1, 40)), None
        S = int(rng.integers(0, E + 1))
        slot_of = np.full(E, -1)
        res = rng.choice(E, size=int(rng.integers(0, S + 1)), replace=False)
        slot_of[res] = rng.choice(S, size=res.size, replace=False) if S else []
        want = np.zeros(E, np.int32)
        want[rng.choice(E, size=int(rng.integers(0, S + 1)), replace=False)] = 1
        _, new, done, ev = O.cache_set_resident(np.zeros(E), np.zeros(E), slot_of, want, S, 0.9)
        assert ((new >= 0) == want.astype(bool)).all()
        assert len(set(new[new >= 0].tolist())) == int(want.sum()) and (new < S).all()
        kept = (slot_of >= 0) & want.astype(bool)
        assert (new[kept] == slot_of[kept]).all()
        assert sorted(ev) == sorted(np.nonzero((slot_of >= 0) & ~want.astype(bool))[0].tolist())
        assert [e for e, _ in done] == sorted(np.nonzero((slot_of < 0) & want.astype(bool))[0].tolist())


def test_prefetch_step_hand_cases():
    lg = np.array([[5, 4, 3, 2, 1, 0], [0, 1, 2, 3, 4, 5]], np.float32)
    host = np.array([1, 0, 1, 1, 1, 1])
    # empty slots: token 0's top 3 are 0, 1, 2 (1 is in HBM, skipped), token 1's first is 5
    pred, new, cp = O.prefetch_step(lg, 3, 3, host, np.full(3, -1), np.ones(3, bool))
    assert pred == [0, 2, 5] and new.tolist() == [0, 2, 5] and cp == [(0, 0), (1, 2), (2, 5)]
    # slot 1 holds 5, predicted again: kept; slot 2's 3 is not predicted: freed; 0 and 2
    # then take the lowest free slots 0 and 2
    pred, new, cp = O.prefetch_step(lg, 3, 3, host, np.array([-1, 5, 3]), np.ones(3, bool))
    assert pred == [0, 2, 5] and new.tolist() == [0, 5, 2] and cp == [(0, 0), (2, 2)]
    # a slot whose table entry was rewritten serves nothing: its expert is copied again
    pred, new, cp = O.prefetch_step(lg, 3, 3, host, np.array([2, -1, -1]), np.array([False, True, True]))
    assert pred == [0, 2, 5] and cp == [(0, 0), (1, 2), (2, 5)]
    # an HBM-resident expert held by a stale slot is not predicted
    host2 = np.array([1, 0, 0, 1, 1, 1])
    pred, new, cp = O.prefetch_step(lg, 3, 3, host2, np.array([2, -1, -1]), np.array([False, True, True]))
    assert pred == [0, 5, 4] and new.tolist() == [0, 5, 4]
    # ties go to the lower id (-0.0 ties +0.0); tokens repeating experts add nothing
    lt = np.array([[1, 1, 1, 1], [0.0, -0.0, 2, -1], [1, 1, 1, 1]], np.float32)
    pred, new, cp = O.prefetch_step(lt, 2, 4, np.ones(4, int), np.full(4, -1), np.ones(4, bool))
    assert pred == [0, 1, 2] and new.tolist() == [0, 1, 2, -1]
    # every candidate in HBM: nothing predicted, held slots freed
    pred, new, cp = O.prefetch_step(lg, 2, 2, np.zeros(6, int), np.array([3, -1]), np.ones(2, bool))
    assert pred == [] and new.tolist() == [-1, -1] and cp == []


def test_prefetch_step_invariants():
    """Random cases: the predicted experts are distinct host-read candidates taken in
    candidate order (none skipped while slots remain), the slots end up holding exactly
    them, a kept expert stays in its slot, and only the others are copied."""
    rng = np.random.default_rng(12)
    for _ in range(300):
        E = int(rng.integers(1, 30))
        T, kp, P = int(rng.integers(1, 5)), int(rng.integers(1, E + 1)), int(rng.integers(1, E + 1))
        lg = rng.integers(-3, 4, size=(T, E)).astype(np.float32)
        host = rng.integers(0, 2, size=E)
        occ = np.full(P, -1)
        held_e = rng.choice(E, size=int(rng.integers(0, min(P, E) + 1)), replace=False)
        occ[rng.choice(P, size=held_e.size, replace=False)] = held_e
        valid = rng.integers(0, 2, size=P).astype(bool)
        host_eff = host.copy()
        for i in range(P):
            if occ[i] >= 0 and valid[i]:
                host_eff[occ[i]] = 1
        pred, new, cp = O.prefetch_step(lg, kp, P, host, occ, valid)
        cand = [int(e) for t in range(T) for e in O.topk_ids(lg[t], kp)]
        want = []
        for e in cand:
            if host_eff[e] and e not in want:
                want.append(e)
        assert pred == want[:P]
        assert sorted(new[new >= 0].tolist()) == sorted(pred)
        for i in range(P):
            if occ[i] >= 0 and valid[i] and occ[i] in pred:
                assert new[i] == occ[i]
        assert sorted(e for _, e in cp) == sorted(e for e in pred
                                                  if not any(occ[i] == e and valid[i] for i in range(P)))
        assert all(new[i] == e for i, e in cp)


def test_residual_next_rounding():
    # 1 + 2^-8 is halfway between the bf16 neighbours 1 and 1 + 2^-7: ties to even
    assert O.residual_next(np.array([1.0]), np.array([2.0 ** -8]), "bf16")[0] == 1.0
    assert O.residual_next(np.array([1.0]), np.array([3 * 2.0 ** -9]), "bf16")[0] == 1.0 + 2.0 ** -7
    assert O.residual_next(np.array([1.0 + 2.0 ** -7]), np.array([2.0 ** -8]), "bf16")[0] == 1.0 + 2.0 ** -6
    # the sum is a float32 one first: 2^-30 is lost there, so the halfway case stays a tie
    # (the exact sum would round up)
    assert O.residual_next(np.array([1.0]), np.array([2.0 ** -8 + 2.0 ** -30]), "bf16")[0] == 1.0
    # float32 activations: the float32 sum itself; negatives and cancellation
    assert O.residual_next(np.array([1.0]), np.array([2.0 ** -30]), "f32")[0] == 1.0
    assert O.residual_next(np.array([-3.0, 0.5]), np.array([3.0, -0.25]), "bf16").tolist() == [0.0, 0.25]
    # against torch's own float32 add and bfloat16 conversion on random values
    import torch
    rng = np.random.default_rng(3)
    xb = O.round_bf16(rng.normal(size=4096))
    y = rng.normal(scale=0.1, size=4096).astype(np.float32)
    ref = (torch.tensor(xb, dtype=torch.float32) + torch.tensor(y)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.residual_next(xb, y, "bf16"), ref)


# ----------------------------------------------------------------------------- page structural figures


def test_page_residency_figures():
    vals = {}
    for line in open(os.path.join(GOLDEN, "pages_structural.txt"), encoding="utf-8"):
        line = line.split("#")[0].strip()
        if line:
            k, v = line.split()
            vals[k] = float(v)
    assert vals["routed_experts_per_layer"] * vals["layers"] == vals["routed_experts_total"]
    frac_off = vals["offloaded_experts_total"] / vals["routed_experts_total"]
    assert abs(frac_off - 0.30) < 1e-9
    # the deepseek-style plan: 30% of 384 on the host, coldest by Zipf rank
    E = int(vals["routed_experts_per_layer"])
    plan = synth.coldest_host_plan(2, 0, E, 1 - frac_off)
    n_host = int((plan == 0).sum())
    assert n_host == 115 and abs(n_host - vals["offloaded_experts_total"] / vals["layers"]) < 0.5
    ranks = synth.zipf_ranks(2, 0, E)
    assert ranks[plan == 0].min() > ranks[plan == 1].max()
    assert vals["cached_experts_min"] / vals["total_experts_min"] == pytest.approx(0.708, abs=0.01)
