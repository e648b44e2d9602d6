"""GPU edge cases against the CPU oracle, through the C ABI.

- Exact ties in the router logits (-0.0 equal to +0.0), at the top-k cut and inside
  the top k, on both routing paths: the one-launch decode routing (one wave per token,
  id-bit ballot grouping) and the multi-block top-k + scatter. Ties go to the lower
  expert id; ids, counts, offsets, the permutation and its inverse must match the
  oracle bit for bit.
- The int4 code -8 (nibble 0x8), which the fixture quantiser never emits, in every
  weight matrix, on every weight path: the bf16 GEMV (with the 16-row and 64-row fused
  down + combine, and the plain down GEMV + combine), the fp32 GEMV and the grouped
  MFMA GEMM at G = 32, 64, 128 and 256.
"""
import sys

import numpy as np
import pytest

import layer_cases as LC
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def moe():
    import expert_offloaded_ffn_moe_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    m.load_library()
    return m


def dev_x(c):
    if c.act == "bf16":
        return torch.from_numpy(c.x_bits.view(np.int16).copy()).view(torch.bfloat16).cuda()
    return torch.from_numpy(c.x_bits.copy()).cuda()


def route_bufs(T, E, k):
    A = T * k
    z = lambda n, dt=torch.int32: torch.full((n,), -7, dtype=dt, device="cuda")
    return dict(logits=torch.zeros(T * E, device="cuda"), topk_ids=z(A), topk_w=z(A, torch.float32),
                counts=z(E), offsets=z(E + 1), sorted=z(A), inv=z(A))


def forward(moe, c, lg, gemm_min_tokens=0):
    cfg = moe.make_config(c.H, c.I, c.E, c.k, c.G, c.act, max_tokens=c.T, gemm_min_tokens=gemm_min_tokens)
    plan = moe.Plan(cfg)
    plan.load_layer(0, c.Wr_store, c.b, c.blobs)
    rb = route_bufs(c.T, c.E, c.k)
    y = torch.full((c.T, c.H), float("nan"), device="cuda")
    plan.forward(0, dev_x(c), y, logits_in=torch.from_numpy(np.ascontiguousarray(lg)).cuda(), route=rb)
    torch.cuda.synchronize()
    plan.destroy()
    return y.cpu().numpy().astype(np.float64), rb


def check_routing(c, ref, rb, T=None):
    T = c.T if T is None else T
    np.testing.assert_array_equal(rb["topk_ids"].cpu().numpy().reshape(T, c.k), ref["ids"])
    np.testing.assert_array_equal(rb["counts"].cpu().numpy(), ref["counts"])
    np.testing.assert_array_equal(rb["offsets"].cpu().numpy(), ref["offsets"])
    np.testing.assert_array_equal(rb["sorted"].cpu().numpy(), ref["sorted"])
    np.testing.assert_array_equal(rb["inv"].cpu().numpy(), ref["inv"])
    w = rb["topk_w"].cpu().numpy().reshape(T, c.k).astype(np.float64)
    np.testing.assert_allclose(w, ref["w"], rtol=2e-6, atol=1e-7)


def check_y(y, ref_y, label):
    r, m = LC.rel_l2(y, ref_y), LC.max_abs(y, ref_y)
    _say("  %s: rel_l2=%.3e max_abs=%.3e" % (label, r, m))
    assert np.all(np.isfinite(y)), label
    assert r <= LC.REL_L2_BAR, (label, r)
    assert m <= LC.MAX_ABS_BAR, (label, m)


# ----------------------------------------------------------------------------- ties

TIES = [
    # E, k, T, act: bf16 T <= 4 and fp32 T <= 64 with T*k <= 256 take the one-launch
    # decode routing; the others the multi-block top-k and scatter
    (8, 2, 1, "bf16"), (8, 2, 4, "bf16"), (8, 2, 40, "bf16"), (8, 2, 2048, "bf16"), (8, 2, 40, "f32"),
    (128, 8, 1, "bf16"), (128, 8, 4, "bf16"), (128, 8, 40, "bf16"), (128, 8, 2048, "bf16"), (128, 8, 20, "f32"),
    (384, 6, 1, "bf16"), (384, 6, 4, "bf16"), (384, 6, 40, "bf16"), (384, 6, 2048, "bf16"), (384, 6, 10, "f32"),
]


@pytest.mark.parametrize("E,k,T,act", TIES)
def test_routing_ties_bit_exact(moe, E, k, T, act):
    _say("ties E=%d k=%d T=%d %s" % (E, k, T, act))
    H, I, G = 256, 64, 32
    c = LC.make_case(H, I, E, k, G, act, T, seed=40 + E + T)
    lg = LC.tie_logits(T, E, k, seed=E * 7 + T)
    toks = np.arange(min(T, 12))
    ref = O.layer_forward(c.x, c.Wr, c.b, c.blobs, H, I, E, k, G, act, logits_in=lg, tokens=toks)
    # the constructed rows have their textbook answers
    for t in range(0, min(T, 20), 5):
        np.testing.assert_array_equal(ref["ids"][t], np.arange(k))
    y, rb = forward(moe, c, lg)
    check_routing(c, ref, rb)
    check_y(y[toks], ref["y"], "y on %d tokens" % len(toks))


# ----------------------------------------------------------------------------- the code -8

MINUS8 = [
    # H, I, E, k, G, act, T, gemm_min_tokens, path
    (2048, 768, 32, 8, 128, "bf16", 1, 0, "bf16 GEMV, 16-row fused down + combine"),
    (1024, 2048, 16, 4, 128, "bf16", 1, 0, "bf16 GEMV, 16-row fused down + combine, h staged in LDS"),
    (4096, 256, 24, 6, 128, "bf16", 2, 0, "bf16 GEMV, 64-row fused down + combine"),
    (2048, 768, 32, 8, 128, "bf16", 8, -1, "bf16 GEMV (8-token), down GEMV + combine"),
    (2048, 256, 16, 4, 256, "bf16", 2, 0, "bf16 GEMV, G = 256"),
    (256, 128, 8, 2, 32, "f32", 16, 0, "fp32 GEMV"),
    (512, 256, 16, 4, 128, "f32", 3, 0, "fp32 GEMV, 4-token kernel"),
    (384, 96, 12, 3, 32, "bf16", 300, 0, "MFMA GEMM, G = 32"),
    (1024, 512, 32, 4, 64, "bf16", 700, 0, "MFMA GEMM, G = 64"),
    (2048, 768, 32, 8, 128, "bf16", 512, 0, "MFMA GEMM, G = 128"),
    (2048, 1536, 16, 8, 256, "bf16", 300, 0, "MFMA GEMM, G = 256"),
]


@pytest.mark.parametrize("H,I,E,k,G,act,T,gemm_min,path", MINUS8)
def test_code_minus8_every_weight_path(moe, H, I, E, k, G, act, T, gemm_min, path):
    _say("code -8: %s (H%d I%d E%d k%d G%d %s T%d)" % (path, H, I, E, k, G, act, T))
    c = LC.make_case(H, I, E, k, G, act, T, seed=60 + T, alpha=0.3, only_experts=[])
    c.blobs = LC.random_code_blobs(E, H, I, G, seed=H + I + T)
    # the blobs hold the code -8 in each of the three matrices of every expert
    lay, _ = O.expert_layout(H, I, G)
    for e in range(E):
        for name in ("q_gate", "q_up", "q_down"):
            a, b = lay[name]
            assert (O.unpack_int4(c.blobs[e, a:b].reshape(1, -1)) == -8).mean() > 0.2
    lg = LC.oracle_logits(c)
    toks = np.arange(T) if T <= 16 else np.sort(np.random.default_rng(T).choice(T, 24, replace=False))
    ref = LC.oracle_forward(c, logits_in=lg, tokens=toks)
    y, rb = forward(moe, c, lg, gemm_min_tokens=gemm_min)
    check_routing(c, ref, rb)
    check_y(y[toks], ref["y"], path)
