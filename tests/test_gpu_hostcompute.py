"""Host computation of experts (moe_plan_set_host_compute) against the CPU oracle and
against the GPU path, through the C ABI: MOE_HOST_COMPUTE_MISSES (the host cores
compute the experts read from host memory, the GPU the rest) and
MOE_HOST_COMPUTE_LAYER (the host cores compute every expert); routing bit-exact, y
within the tolerance bars, the host-computed expert count equal to a recount from the
routing and the residency, and the GPU-only plan's y within tolerance of each."""
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


CASES = [
    # H, I, E, k, G, act, T, alpha, seed
    (2048, 768, 128, 8, 128, "bf16", 1, 0.8, 1),   # Qwen3-shaped decode
    (2048, 768, 128, 8, 128, "bf16", 4, 0.8, 2),
    (1024, 512, 32, 4, 64, "bf16", 40, 0.5, 3),    # multi-block routing, 8-token host passes
    (256, 128, 8, 2, 32, "f32", 16, 0.0, 4),       # fp32 activations
    (512, 256, 16, 4, 256, "bf16", 300, 0.0, 5),   # a prefill-sized batch (GEMV path), G = 256
]


@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("H,I,E,k,G,act,T,alpha,seed", CASES)
def test_host_compute_parity(moe, H, I, E, k, G, act, T, alpha, seed, mode):
    import synth
    _say("host compute mode %d:" % mode, H, I, E, k, G, act, T)
    c = LC.make_case(H, I, E, k, G, act, T, seed, alpha)
    lg = LC.oracle_logits(c)
    toks = np.arange(T) if T <= 16 else np.sort(np.random.default_rng(T).choice(T, 24, replace=False))
    ref = LC.oracle_forward(c, logits_in=lg, tokens=toks)
    res = synth.coldest_host_plan(seed, 0, E, 0.7)
    cfg = moe.make_config(H, I, E, k, G, act, max_tokens=T, hbm_slots=int(res.sum()))
    plan = moe.Plan(cfg, layers=[(c.Wr_store, c.b, c.blobs)], initial_hbm=res[None, :])
    gpu = moe.Plan(cfg, layers=[(c.Wr_store, c.b, c.blobs)], initial_hbm=res[None, :])
    plan.set_host_compute(0, mode, threads=8)
    li = torch.from_numpy(np.ascontiguousarray(lg)).cuda()
    ids = torch.empty(T * k, dtype=torch.int32, device="cuda")
    ys = []
    for p in (plan, gpu):
        y = torch.full((T, H), float("nan"), device="cuda")
        p.forward(0, _x(c), y, logits_in=li, route={"topk_ids": ids})
        torch.cuda.synchronize()
        ys.append(y.cpu().numpy().astype(np.float64))
    np.testing.assert_array_equal(ids.cpu().numpy().reshape(T, k), ref["ids"])
    for name, y in (("host compute", ys[0]), ("GPU only", ys[1])):
        r, m = LC.rel_l2(y[toks], ref["y"]), LC.max_abs(y[toks], ref["y"])
        _say("  %s: rel_l2=%.3e max_abs=%.3e" % (name, r, m))
        assert np.all(np.isfinite(y)) and r <= LC.REL_L2_BAR and m <= LC.MAX_ABS_BAR
    uniq = np.unique(ref["ids"])
    want = len(uniq) if mode == 2 else int((res[uniq] == 0).sum())
    st = plan.stats(0)
    _say("  host-computed experts %d of %d active" % (st["host_computed"], len(uniq)))
    assert st["host_computed"] == want
    acc = O.link_accounting(ref["ids"], res, synth.expert_bytes(H, I, G))
    assert (st["hits"], st["misses"]) == (acc["hits"], acc["misses"])
    # the same plan back on the GPU path gives the GPU-only result bit for bit
    plan.set_host_compute(0, 0)
    y = torch.full((T, H), float("nan"), device="cuda")
    plan.forward(0, _x(c), y, logits_in=li)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y.cpu().numpy().astype(np.float64), ys[1])
    plan.destroy()
    gpu.destroy()


def test_host_compute_steps_in_a_row_and_bad_arguments(moe):
    """Several forwards in a row on one stream, alternating layers with and without host
    computation (the pinned staging is reused across forwards), against the GPU path;
    argument checks."""
    L, H, I, E, k, G = 3, 1024, 256, 32, 4, 128
    layers = [LC.make_case(H, I, E, k, G, "bf16", 4, 20, alpha=0.8, layer=l) for l in range(L)]
    cfg = moe.make_config(H, I, E, k, G, "bf16", num_layers=L, max_tokens=4, hbm_slots=20)
    wts = [(c.Wr_store, c.b, c.blobs) for c in layers]
    plan, gpu = moe.Plan(cfg, layers=wts), moe.Plan(cfg, layers=wts)
    plan.set_host_compute(0, moe.HOST_COMPUTE_MISSES)
    plan.set_host_compute(2, moe.HOST_COMPUTE_LAYER)
    ya = torch.empty((12, 4, H), device="cuda")
    yb = torch.empty((12, 4, H), device="cuda")
    for step in range(12):
        l = step % L
        x = _x(layers[l])
        plan.forward(l, x, ya[step])
        gpu.forward(l, x, yb[step])
    torch.cuda.synchronize()
    for step in range(12):
        r = LC.rel_l2(ya[step].cpu().numpy(), yb[step].cpu().numpy())
        assert r <= 1e-4, (step, r)
    assert plan.stats(-1)["host_computed"] > 0
    for bad in ((5, 1), (0, 3), (0, -1)):
        with pytest.raises(moe.MoeError) as ei:
            plan.set_host_compute(*bad)
        assert ei.value.status == moe.MOE_E_INVALID
    cfg2 = moe.make_config(H, I, E, k, G, "bf16", max_tokens=4, weight_bits=2)
    p2 = moe.Plan(cfg2)
    with pytest.raises(moe.MoeError) as ei:
        p2.set_host_compute(0, 1)
    assert ei.value.status == moe.MOE_E_UNSUPPORTED
    for p in (plan, gpu, p2):
        p.destroy()
