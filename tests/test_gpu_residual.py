"""moe_layer_forward_residual: y bitwise equal to moe_layer_forward's on the same plan
and inputs, and x_out equal, bit for bit, to the oracle's residual rule applied to x and
that y, on every path that writes y (the fused down + combine on 64- and 16-row tiles,
the separate combine for fp32 activations, the prefill GEMMs, 3-bit codes and host
computation of the offloaded experts); y also within the bars of the oracle forward."""
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
    if c.act == "bf16":
        return torch.from_numpy(c.x_bits.view(np.int16).copy()).view(torch.bfloat16).cuda()
    return torch.from_numpy(c.x_bits.copy()).cuda()


def _vals(t):
    if t.dtype == torch.bfloat16:
        return O.bf16_bits_to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.cpu().numpy().astype(np.float64)


CASES = [
    # H, I, E, k, G, act, T, bits, host_mode, alpha, seed
    (2048, 768, 128, 8, 128, "bf16", 1, 4, 0, 0.8, 1),    # fused down + combine, 16-row tiles
    (7168, 2048, 16, 6, 128, "bf16", 3, 4, 0, 0.5, 2),    # fused down + combine, 64-row tiles
    (256, 128, 8, 2, 32, "f32", 5, 4, 0, 0.0, 3),         # fp32: separate combine
    (1024, 512, 32, 4, 64, "bf16", 96, 4, 0, 0.3, 4),     # grouped MFMA GEMMs
    (1024, 512, 32, 4, 64, "bf16", 3, 3, 0, 0.3, 5),      # 3-bit codes
    (2048, 768, 128, 8, 128, "bf16", 4, 4, 1, 0.8, 6),    # offloaded experts computed by the host
]


@pytest.mark.parametrize("H,I,E,k,G,act,T,bits,host_mode,alpha,seed", CASES)
def test_residual_forward(moe, H, I, E, k, G, act, T, bits, host_mode, alpha, seed):
    import synth
    _say("residual:", H, I, E, k, G, act, T, "bits", bits, "host mode", host_mode)
    c = LC.make_case(H, I, E, k, G, act, T, seed, alpha, bits=bits)
    res = synth.coldest_host_plan(seed, 0, E, 0.7)
    cfg = moe.make_config(H, I, E, k, G, act, max_tokens=T, hbm_slots=int(res.sum()), weight_bits=bits)
    plan = moe.Plan(cfg, layers=[(c.Wr_store, c.b, c.blobs)], initial_hbm=res[None, :])
    if host_mode:
        plan.set_host_compute(0, host_mode)
    x = _x(c)
    y = torch.full((T, H), float("nan"), device="cuda")
    y2 = torch.full((T, H), float("nan"), device="cuda")
    xo = torch.full_like(x, float("nan"))
    ids = torch.empty(T * k, dtype=torch.int32, device="cuda")
    plan.forward(0, x, y)
    plan.forward_residual(0, x, y2, xo, route={"topk_ids": ids})
    torch.cuda.synchronize()
    assert torch.equal(y, y2), "y differs between the two entry points"
    yv = y2.cpu().numpy()
    want = O.residual_next(_vals(x), yv, act)
    assert np.array_equal(_vals(xo), want), "x_out differs from act(x + y)"
    toks = np.arange(T) if T <= 8 else np.sort(np.random.default_rng(T).choice(T, 8, replace=False))
    ref = LC.oracle_forward(c, tokens=toks)
    assert np.array_equal(ids.cpu().numpy().reshape(T, k)[toks], ref["ids"][toks]) or \
        LC.routing_margins(ref["logits"], k).min() < 1e-5
    r, m = LC.rel_l2(yv[toks].astype(np.float64), ref["y"]), LC.max_abs(yv[toks].astype(np.float64), ref["y"])
    _say("  rel_l2 %.3e max_abs %.3e" % (r, m))
    assert r <= LC.REL_L2_BAR and m <= LC.MAX_ABS_BAR
    plan.destroy()


def test_residual_argument_errors(moe):
    H, I, E, k, G, T = 256, 128, 8, 2, 32, 4
    c = LC.make_case(H, I, E, k, G, "bf16", T, 7)
    plan = moe.Plan(moe.make_config(H, I, E, k, G, "bf16", max_tokens=T),
                    layers=[(c.Wr_store, c.b, c.blobs)])
    x = _x(c)
    y = torch.empty((T, H), device="cuda")
    for bad in (None, x, x[1:]):  # missing, the same buffer as x, overlapping x
        with pytest.raises(moe.MoeError) as ei:
            plan.forward_residual(0, x, y, bad)
        assert ei.value.status == moe.MOE_E_INVALID
    with pytest.raises(moe.MoeError) as ei:  # overlapping y
        plan.forward_residual(0, x, y, y.view(torch.bfloat16)[:T])
    assert ei.value.status == moe.MOE_E_INVALID
    plan.destroy()
