"""The C-ABI boundary on the GPU: plan creation with every layer's weights and an
initial residency set, residency sets chosen by the caller (want_resident) against the
oracle's rule, clean failure of plan creation at every allocation, plan info, and the
measured link ceilings."""
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


H, I, E, k, G, L = 512, 256, 24, 4, 128, 3


@pytest.fixture(scope="module")
def layers():
    return [LC.make_case(H, I, E, k, G, "bf16", 3, 51, alpha=0.8, layer=l) for l in range(L)]


def _x(c):
    return torch.from_numpy(c.x_bits.view(np.int16).copy()).view(torch.bfloat16).cuda()


def test_create_with_layers_and_initial_hbm(moe, layers):
    """moe_plan_create(cfg, layers, initial_hbm): the slot tables follow initial_hbm (slots
    in ascending expert id), and y equals that of a plan loaded layer by layer."""
    S = 10
    rng = np.random.default_rng(3)
    init = np.zeros((L, E), np.int32)
    for l in range(L):
        init[l, rng.choice(E, size=S - l, replace=False)] = 1
    cfg = moe.make_config(H, I, E, k, G, "bf16", num_layers=L, max_tokens=3, hbm_slots=S)
    a = moe.Plan(cfg, layers=[(c.Wr_store, c.b, c.blobs) for c in layers], initial_hbm=init)
    b = moe.Plan(cfg)
    for l, c in enumerate(layers):
        b.load_layer(l, c.Wr_store, c.b, c.blobs)
    for l in range(L):
        want = np.full(E, -1)
        ids = np.nonzero(init[l])[0]
        want[ids] = np.arange(ids.size)
        np.testing.assert_array_equal(a.residency(l), want)
        ya, yb = torch.empty((3, H), device="cuda"), torch.empty((3, H), device="cuda")
        a.forward(l, _x(layers[l]), ya)
        b.forward(l, _x(layers[l]), yb)
        torch.cuda.synchronize()
        assert torch.equal(ya, yb)
    info = a.info()
    _say("  plan info", info)
    assert info["host_pool_bytes"] == L * E * info["internal_expert_bytes"]
    assert info["hbm_slot_bytes"] == L * S * info["internal_expert_bytes"]
    assert info["workspace_bytes"] > 0
    a.destroy()
    b.destroy()
    # too many initially resident experts for the slots
    bad = np.ones((L, E), np.int32)
    with pytest.raises(moe.MoeError) as ei:
        moe.Plan(cfg, layers=[(c.Wr_store, c.b, c.blobs) for c in layers], initial_hbm=bad)
    assert ei.value.status == moe.MOE_E_INVALID


def test_want_resident_matches_oracle(moe, layers):
    """A caller-chosen residency set per layer and for all layers at once: slot tables equal
    the oracle's rule applied to the recounted assignment counts, y stays bitwise equal, the
    frequency policy continues from the scores afterwards, and a set larger than the slots
    is refused without change."""
    S = 12
    cfg = moe.make_config(H, I, E, k, G, "bf16", num_layers=L, max_tokens=3, hbm_slots=S)
    plan = moe.Plan(cfg, layers=[(c.Wr_store, c.b, c.blobs) for c in layers])
    slot = [np.where(np.arange(E) < S, np.arange(E), -1) for _ in range(L)]
    score = [np.zeros(E) for _ in range(L)]
    rng = np.random.default_rng(8)
    y0 = []
    for l, c in enumerate(layers):
        ids = torch.empty(3 * k, dtype=torch.int32, device="cuda")
        y = torch.empty((3, H), device="cuda")
        plan.forward(l, _x(c), y, route={"topk_ids": ids})
        torch.cuda.synchronize()
        y0.append(y.clone())
        c.counts = np.bincount(ids.cpu().numpy(), minlength=E)
    # one layer
    want1 = np.zeros(E, np.int32)
    want1[rng.choice(E, size=S, replace=False)] = 1
    plan.cache_update(1, want_resident=want1)
    score[1], slot[1], prom, ev = O.cache_set_resident(score[1], layers[1].counts, slot[1], want1, S, 0.9)
    np.testing.assert_array_equal(plan.residency(1), slot[1])
    assert plan.stats(1)["promotions"] == len(prom) and plan.stats(1)["evictions"] == len(ev)
    # every layer at once ([L][E]); layer 1's counts were used by the update above
    wantL = np.zeros((L, E), np.int32)
    for l in range(L):
        wantL[l, rng.choice(E, size=S - 2 * l, replace=False)] = 1
    plan.cache_update(-1, want_resident=wantL)
    for l in range(L):
        cnt = np.zeros(E) if l == 1 else layers[l].counts
        score[l], slot[l], _, _ = O.cache_set_resident(score[l], cnt, slot[l], wantL[l], S, 0.9)
        np.testing.assert_array_equal(plan.residency(l), slot[l])
    for l, c in enumerate(layers):
        y = torch.empty((3, H), device="cuda")
        plan.forward(l, _x(c), y)
        torch.cuda.synchronize()
        assert torch.equal(y, y0[l])
    # the frequency policy continues from the scores the counts went into
    ids = torch.empty(3 * k, dtype=torch.int32, device="cuda")
    y = torch.empty((3, H), device="cuda")
    plan.forward(0, _x(layers[0]), y, route={"topk_ids": ids})
    torch.cuda.synchronize()
    plan.cache_update(0, max_promotions=4)
    cnt = np.bincount(ids.cpu().numpy(), minlength=E)
    score[0], slot[0], _, _ = O.cache_policy_step(score[0], cnt, slot[0], S, 0.9, 4)
    np.testing.assert_array_equal(plan.residency(0), slot[0])
    # more wanted experts than slots: refused, tables unchanged
    with pytest.raises(moe.MoeError) as ei:
        plan.cache_update(2, want_resident=np.ones(E, np.int32))
    assert ei.value.status == moe.MOE_E_INVALID
    np.testing.assert_array_equal(plan.residency(2), slot[2])
    plan.destroy()


def _dev_free():
    torch.cuda.synchronize()
    return torch.cuda.mem_get_info()[0]


def _rss_bytes():
    with open("/proc/self/statm") as f:
        return int(f.read().split()[1]) * 4096


def test_alloc_failure_at_every_allocation_frees_everything(moe, layers):
    """moe_debug_fail_alloc makes the n-th device (or pinned host) allocation of plan
    creation fail, for every n until creation succeeds: each failure returns
    MOE_E_NOMEM (MOE_E_HOST_NOMEM), leaves no plan and no allocation held by the
    library (its live-allocation counters), and device free memory and resident host
    memory return to where they were (within the runtime's own granularity)."""
    cfg = moe.make_config(H, I, E, k, G, "bf16", num_layers=L, max_tokens=64, hbm_slots=8)
    wts = [(c.Wr_store, c.b, c.blobs) for c in layers]
    p = moe.Plan(cfg, layers=wts)  # warm the runtime's own pools
    p.destroy()
    live0 = moe.debug_live_allocs()
    dev0, rss0 = _dev_free(), _rss_bytes()
    for kind, status in ((0, moe.MOE_E_NOMEM), (1, moe.MOE_E_HOST_NOMEM)):
        n = 1
        while True:
            moe.debug_fail_alloc(kind, n)
            try:
                p = moe.Plan(cfg, layers=wts)
            except moe.MoeError as e:
                assert e.status == status, (kind, n, e)
                assert moe.debug_live_allocs() == live0, (kind, n)
                n += 1
                continue
            moe.debug_fail_alloc(kind, 0)
            p.destroy()
            break
        _say("  kind %d: %d allocations, each failure freed everything" % (kind, n - 1))
        assert n > 5
    assert moe.debug_live_allocs() == live0
    dev_diff = dev0 - _dev_free()
    _say("  device free memory moved by %d bytes" % dev_diff)
    assert abs(dev_diff) <= 4 << 20
    grow = _rss_bytes() - rss0
    _say("  resident host memory grew by %.1f MB over the failed creations" % (grow / 1e6))
    assert grow < 64 << 20


def test_link_ceilings_measured(moe):
    c = moe.measure_link_ceilings(256 << 20, 256 << 20, 3)
    _say("  ceilings", c)
    assert c["hbm_read_gbps"] > 500 and c["host_read_gbps"] > 1 and c["h2d_copy_gbps"] > 1
