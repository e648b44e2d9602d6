"""moe_layer_forward_noalloc, the forward whose workspace is the library's static
per-device array, against moe_layer_forward on the same plan and inputs: y and every
routing output bitwise equal, on two calls in a row with the second one smaller (the
array keeps the previous call's contents), on the decode, middle and prefill paths,
after switching plans; no allocation made by the calls; a forward whose workspace
exceeds the array refused with a clear error."""
import sys

import numpy as np
import pytest

import layer_cases as LC

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


def _route(T, E, k):
    A = T * k
    z = lambda n, dt=torch.int32: torch.full((n,), -7, dtype=dt, device="cuda")
    return dict(logits=torch.zeros(T * E, device="cuda"), topk_ids=z(A), topk_w=z(A, torch.float32),
                counts=z(E), offsets=z(E + 1), sorted=z(A), inv=z(A))


def _x(c, T):
    if c.act == "bf16":
        return torch.from_numpy(c.x_bits[:T].view(np.int16).copy()).view(torch.bfloat16).cuda()
    return torch.from_numpy(c.x_bits[:T].copy()).cuda()


def _both(plan, c, T, logits_in=None, moe=None):
    """(y, routing) of moe_layer_forward and of moe_layer_forward_noalloc. With `moe`,
    also checks that the no-alloc call changes neither the library's live allocations
    nor the device's free memory (every tensor is allocated before it)."""
    out = []
    for noalloc in (False, True):
        y = torch.full((T, c.H), float("nan"), device="cuda")
        r = _route(T, c.E, c.k)
        li = None if logits_in is None else torch.from_numpy(np.ascontiguousarray(logits_in[:T])).cuda()
        x = _x(c, T)
        torch.cuda.synchronize()
        if noalloc:
            before = (moe.debug_live_allocs(), torch.cuda.mem_get_info()[0]) if moe else None
            plan.forward_noalloc(0, x, y, logits_in=li, route=r)
            torch.cuda.synchronize()
            if moe:
                assert (moe.debug_live_allocs(), torch.cuda.mem_get_info()[0]) == before
        else:
            plan.forward(0, x, y, logits_in=li, route=r)
            torch.cuda.synchronize()
        out.append((y, r))
    return out


CASES = [
    # H, I, E, k, G, act, T first call, T second call, alpha, seed
    (2048, 768, 128, 8, 128, "bf16", 16, 3, 0.8, 1),    # grouped GEMM path, then the one-launch decode path
    (2048, 768, 128, 8, 128, "bf16", 4, 1, 0.8, 2),     # fused down + combine at batch 4, then batch 1
    (4096, 256, 24, 6, 128, "bf16", 2, 1, 0.5, 3),      # 64-row fused down + combine
    (384, 96, 12, 3, 32, "bf16", 13, 7, 0.5, 4),        # GEMM path twice, G = 32
    (256, 128, 8, 2, 32, "f32", 16, 5, 0.0, 5),         # fp32 activations
    (2048, 768, 128, 8, 128, "bf16", 40, 8, 0.0, 6),    # GEMM path with the GEMVs switched off below
]


@pytest.mark.parametrize("H,I,E,k,G,act,T1,T2,alpha,seed", CASES)
def test_noalloc_matches_forward_bitwise(moe, H, I, E, k, G, act, T1, T2, alpha, seed):
    _say("noalloc case", H, I, E, k, G, act, T1, T2)
    c = LC.make_case(H, I, E, k, G, act, T1, seed, alpha)
    gemm_min = -1 if seed == 6 else 0
    cfg = moe.make_config(H, I, E, k, G, act, max_tokens=T1, hbm_slots=(E * 2) // 3, gemm_min_tokens=gemm_min)
    plan = moe.Plan(cfg, layers=[(c.Wr_store, c.b, c.blobs)])
    lg = LC.oracle_logits(c)
    _both(plan, c, T1)  # warm-up of both entry points
    for T, logits_in in ((T1, None), (T2, None), (T1, lg), (T2, lg)):
        (ya, ra), (yb, rb) = _both(plan, c, T, logits_in, moe=moe)
        assert torch.isfinite(ya).all()
        assert torch.equal(ya, yb), (T, logits_in is None)
        for n in ra:
            assert torch.equal(ra[n], rb[n]), (T, n)
    plan.destroy()


def test_noalloc_refuses_a_workspace_beyond_the_array(moe):
    c = LC.make_case(2048, 768, 128, 8, 128, "bf16", 512, 9, 0.0)
    cfg = moe.make_config(2048, 768, 128, 8, 128, "bf16", max_tokens=512)
    plan = moe.Plan(cfg, layers=[(c.Wr_store, c.b, c.blobs)])
    y = torch.empty((512, 2048), device="cuda")
    with pytest.raises(moe.MoeError) as ei:
        plan.forward_noalloc(0, _x(c, 512), y)
    assert ei.value.status == moe.MOE_E_INVALID
    assert "bytes" in str(ei.value) and "static workspace" in str(ei.value)
    _say("  refused:", ei.value)
    # a smaller batch on the same plan still runs, and matches the plan-workspace forward
    (ya, _), (yb, _) = _both(plan, c, 24)
    assert torch.equal(ya, yb)
    plan.destroy()
