"""GPU parity of the 2- and 3-bit weight formats (odd levels q = 2n - (2^b - 1), fp16
group scales) against the CPU oracle, through the C ABI: routing bit-exact with the
oracle's logits, y within the tolerance bars, on the one-launch decode routing and
the multi-block routing, with generator-quantised and with random codes (every code
value), group sizes 64/128/256; y bitwise equal across residency plans; link
counters at the formats' expert bytes."""
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


def _x(c):
    return torch.from_numpy(c.x_bits.view(np.int16).copy()).view(torch.bfloat16).cuda()


def _route(T, E, k):
    A = T * k
    z = lambda n, dt=torch.int32: torch.full((n,), -7, dtype=dt, device="cuda")
    return dict(logits=torch.zeros(T * E, device="cuda"), topk_ids=z(A), topk_w=z(A, torch.float32),
                counts=z(E), offsets=z(E + 1), sorted=z(A), inv=z(A))


def _plan(moe, c, slots=None, resident=None):
    cfg = moe.make_config(c.H, c.I, c.E, c.k, c.G, "bf16", max_tokens=c.T, hbm_slots=c.E if slots is None else slots,
                          weight_bits=c.bits)
    p = moe.Plan(cfg)
    p.load_layer(0, c.Wr_store, c.b, c.blobs, resident)
    return p


def _run(plan, c, lg=None, route=None):
    y = torch.full((c.T, c.H), float("nan"), device="cuda")
    li = None if lg is None else torch.from_numpy(np.ascontiguousarray(lg)).cuda()
    plan.forward(0, _x(c), y, logits_in=li, route=route)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


CASES = [
    # H, I, E, k, G, bits, T, alpha, seed, codes
    (2048, 768, 128, 8, 128, 2, 1, 0.8, 1, "generated"),   # Qwen3-shaped decode, batch 1
    (2048, 768, 128, 8, 128, 3, 1, 0.8, 1, "generated"),
    (2048, 768, 128, 8, 128, 2, 4, 0.8, 2, "generated"),   # batch 4 (4-token passes)
    (2048, 768, 128, 8, 128, 3, 4, 0.8, 2, "generated"),
    (1024, 192, 16, 4, 64, 3, 3, 0.0, 3, "random"),    # G = 64, every code value
    (1024, 192, 16, 4, 64, 2, 3, 0.0, 3, "random"),
    (2048, 512, 16, 4, 256, 3, 2, 0.0, 4, "random"),        # G = 256
    (2048, 512, 16, 4, 256, 2, 2, 0.0, 4, "random"),
    (512, 256, 16, 4, 128, 3, 40, 0.5, 5, "random"),       # multi-block routing, 8-token passes (3-bit: 4)
    (512, 256, 16, 4, 128, 2, 40, 0.5, 5, "random"),
    (1024, 256, 32, 8, 128, 2, 300, 0.0, 6, "generated"),  # a prefill-sized batch on the GEMVs
    (4096, 512, 24, 6, 128, 3, 2, 0.5, 7, "generated"),    # K = 4096 rows staged in LDS for the down GEMV
]


@pytest.mark.parametrize("H,I,E,k,G,bits,T,alpha,seed,codes", CASES)
def test_lowbit_layer_parity(moe, H, I, E, k, G, bits, T, alpha, seed, codes):
    _say("low-bit case", H, I, E, k, G, bits, T, codes)
    a = alpha
    if codes == "generated":
        c = LC.make_case(H, I, E, k, G, "bf16", T, seed, a, bits=bits)
    else:
        c = LC.make_case(H, I, E, k, G, "bf16", T, seed, a, only_experts=[], bits=bits)
        c.blobs = LC.random_code_blobs(E, H, I, G, seed=seed, bits=bits)
    lg = LC.oracle_logits(c)
    toks = np.arange(T) if T <= 16 else np.sort(np.random.default_rng(T).choice(T, 24, replace=False))
    ref = LC.oracle_forward(c, logits_in=lg, tokens=toks)
    plan = _plan(moe, c)
    rb = _route(T, E, k)
    y = _run(plan, c, lg, rb)
    np.testing.assert_array_equal(rb["topk_ids"].cpu().numpy().reshape(T, k), ref["ids"])
    np.testing.assert_array_equal(rb["counts"].cpu().numpy(), ref["counts"])
    np.testing.assert_array_equal(rb["sorted"].cpu().numpy(), ref["sorted"])
    np.testing.assert_array_equal(rb["inv"].cpu().numpy(), ref["inv"])
    r, m = LC.rel_l2(y[toks], ref["y"]), LC.max_abs(y[toks], ref["y"])
    _say("  y: rel_l2=%.3e max_abs=%.3e" % (r, m))
    assert np.all(np.isfinite(y))
    assert r <= LC.REL_L2_BAR and m <= LC.MAX_ABS_BAR
    plan.destroy()


@pytest.mark.parametrize("bits", [2, 3])
def test_lowbit_residency_invariance_and_counters(moe, bits):
    """70/30 and all-host plans give y bitwise equal to the all-HBM plan; the link counters
    match an exact recount at the format's expert bytes (3*H*I*b/8 + 6*H*I/G)."""
    import synth
    c = LC.make_case(2048, 768, 128, 8, 128, "bf16", 4, 11, alpha=0.8, bits=bits)
    lg = LC.oracle_logits(c)
    res = synth.coldest_host_plan(11, 0, 128, 0.7)
    eb = synth.expert_bytes(2048, 768, 128, bits)
    assert eb == 3 * 2048 * 768 * bits // 8 + 6 * 2048 * 768 // 128
    ys = {}
    for name, slots, resident in (("hbm", 128, None), ("mixed", int(res.sum()), res), ("host", 0, None)):
        plan = _plan(moe, c, slots, resident)
        ys[name] = _run(plan, c, lg)
        st = plan.stats(0)
        in_hbm = np.ones(128) if name == "hbm" else (res if name == "mixed" else np.zeros(128))
        acc = O.link_accounting(O.route(lg, 8)[0], in_hbm, eb)
        assert (st["bytes_hbm"], st["bytes_host"]) == (acc["bytes_hbm"], acc["bytes_host"]), name
        assert (st["hits"], st["misses"]) == (acc["hits"], acc["misses"]), name
        plan.destroy()
    np.testing.assert_array_equal(ys["mixed"], ys["hbm"])
    np.testing.assert_array_equal(ys["host"], ys["hbm"])
    ref = LC.oracle_forward(c, logits_in=lg)
    assert LC.rel_l2(ys["hbm"], ref["y"]) <= LC.REL_L2_BAR


def test_lowbit_config_rules(moe):
    """2- and 3-bit plans need bf16 activations, G >= 64 and I a multiple of 64."""
    import ctypes
    lib = moe.load_library()
    for cfg in (moe.make_config(256, 128, 8, 2, 32, "bf16", weight_bits=2),
                moe.make_config(256, 128, 8, 2, 64, "f32", weight_bits=3),
                moe.make_config(256, 96, 8, 2, 32, "bf16", weight_bits=3),
                moe.make_config(256, 128, 8, 2, 64, "bf16", weight_bits=5)):
        out = ctypes.c_size_t()
        assert lib.moe_expert_bytes(ctypes.byref(cfg), ctypes.byref(out)) == moe.MOE_E_INVALID
