"""Predictive prefetch: before the forward of layer l, the experts of layer l+1 that
the layer's router picks for the current activations are copied into its prefetch
slots on the plan's prefetch stream. Checked against
  - the oracle's prefetch rule on the same logits (predicted lists and slot tables
    equal, after every step, through slot reuse and cache updates),
  - an all-HBM plan on the same inputs (y bitwise equal: placement never changes values),
  - the oracle's link accounting under the residency each forward ran with (the base
    table plus the prefetched experts; exact counters),
  - the oracle forward on some (step, layer) pairs (tolerance bars).
"""
from __future__ import annotations

import numpy as np
import pytest

import layer_cases as LC
from oracle import moe_oracle as O

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import expert_offloaded_ffn_moe_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    m.load_library()
    return m


def _say(msg):
    print(msg, flush=True)


def _plans(moe, layers, dims, T, S, P, act="bf16"):
    H, I, E, k, G = dims
    L = len(layers)

    def make(slots, pf):
        cfg = moe.make_config(H, I, E, k, G, act, num_layers=L, max_tokens=T, hbm_slots=slots, prefetch_slots=pf)
        p = moe.Plan(cfg)
        for l, c in enumerate(layers):
            p.load_layer(l, c.Wr_store, c.b, c.blobs)
        return p

    return make(S, P), make(E, 0)


def _to_act(r, act):
    return r.to(torch.bfloat16) if act == "bf16" else r.clone()


def _x_f64(x, act):
    if act == "bf16":
        return O.bf16_bits_to_f64(x.view(torch.int16).cpu().numpy().view(np.uint16))
    return x.cpu().numpy().astype(np.float64)


def _run_chain(moe, dims, T, S, P, L, steps, seed, cand, act="bf16", update=None, oracle_every=5):
    """Steps of a chained decode over L layers with prefetch of layer l+1 before the
    forward of layer l; `update(step, plan)` optionally runs a cache update after a step
    and returns which layers' tables it rewrote."""
    import synth

    H, I, E, k, G = dims
    eb = synth.expert_bytes(H, I, G)
    layers = [LC.make_case(H, I, E, k, G, act, 1, seed, alpha=0.8, layer=l) for l in range(L)]
    pf, full = _plans(moe, layers, dims, T, S, P, act)
    occ_ref = [np.full(P, -1) for _ in range(L)]
    valid_ref = [np.ones(P, bool) for _ in range(L)]
    acc = dict(hits=0, misses=0, bytes_hbm=0, bytes_host=0)
    n_copied, checked, n_pred = 0, 0, 0
    r = torch.from_numpy(synth.activations(seed, 700, T, H, "f32")).cuda() * 1.0
    for step in range(steps):
        for l in range(L):
            x = _to_act(r, act)
            pred = None
            if l + 1 < L:
                pred = torch.full((P,), -7, dtype=torch.int32, device="cuda")
                pf.prefetch(l + 1, x=x, candidates=cand, predicted_out=pred)
            rb = dict(logits=torch.zeros(T * E, device="cuda"), topk_ids=torch.zeros(T * k, dtype=torch.int32,
                                                                                    device="cuda"))
            y = torch.full((T, H), float("nan"), device="cuda")
            yf = torch.full((T, H), float("nan"), device="cuda")
            res_l = pf.residency(l)
            pf.forward(l, x, y, route=rb)
            full.forward(l, x, yf)
            ref_lg = None
            if pred is not None:  # the next layer's logits of this x, by the library's own router
                rn = dict(logits=torch.zeros(T * E, device="cuda"))
                full.forward(l + 1, x, torch.empty((T, H), device="cuda"), route=rn)
                ref_lg = rn["logits"]
            torch.cuda.synchronize()
            assert torch.equal(y, yf), "step %d layer %d: y differs from the all-HBM plan" % (step, l)
            ids = rb["topk_ids"].cpu().numpy().reshape(T, k)
            # this forward read the base table plus the experts the last prefetch placed
            resident = res_l >= 0
            for i in range(P):
                if occ_ref[l][i] >= 0 and valid_ref[l][i]:
                    resident[occ_ref[l][i]] = True
            a = O.link_accounting(ids, resident, eb)
            for n in acc:
                acc[n] += a[n]
            if pred is not None:
                lg = ref_lg.cpu().numpy().reshape(T, E)
                host_read = pf.residency(l + 1) < 0
                want_pred, occ_ref[l + 1], copied = O.prefetch_step(lg, cand or k, P, host_read, occ_ref[l + 1],
                                                                    valid_ref[l + 1])
                valid_ref[l + 1] = np.ones(P, bool)
                n_copied += len(copied)
                n_pred += len(want_pred)
                got = pred.cpu().numpy()
                exp = np.full(P, -1)
                exp[:len(want_pred)] = want_pred
                assert np.array_equal(got, exp), "step %d layer %d: predicted %s, oracle %s" % (
                    step, l + 1, got.tolist(), exp.tolist())
                assert np.array_equal(pf.prefetch_slots(l + 1), occ_ref[l + 1]), "step %d layer %d slots" % (
                    step, l + 1)
            if (step * L + l) % oracle_every == 0:
                c = layers[l]
                lgl = rb["logits"].cpu().numpy().reshape(T, E).astype(np.float64)
                ref = O.layer_forward(_x_f64(x, act), c.Wr, c.b, c.blobs, H, I, E, k, G, act, logits_in=lgl)
                np.testing.assert_array_equal(ids, ref["ids"])
                yv = y.cpu().numpy().astype(np.float64)
                assert LC.rel_l2(yv, ref["y"]) <= LC.REL_L2_BAR
                assert LC.max_abs(yv, ref["y"]) <= LC.MAX_ABS_BAR
                checked += 1
            r = r + y
        if update is not None:
            for l in update(step, pf):
                valid_ref[l] = np.zeros(P, bool)  # the table upload pointed every expert elsewhere
    st = pf.stats(-1)
    _say("  hits %d misses %d prefetched %d predicted %d (oracle checks %d)" % (
        st["hits"], st["misses"], st["prefetched"], n_pred, checked))
    for n in acc:
        assert st[n] == acc[n], n
    assert st["prefetched"] == n_copied
    pf.destroy()
    full.destroy()
    return st, n_copied


@pytest.mark.parametrize("T,act,cand", [(1, "bf16", 0), (3, "bf16", 6), (2, "f32", 0), (4, "bf16", 0), (6, "f32", 3)])
def test_prefetch_follows_the_oracle(moe, T, act, cand):
    dims = (512, 256, 32, 4, 128)
    st, n = _run_chain(moe, dims, T, S=18, P=6, L=3, steps=6, seed=41, cand=cand, act=act)
    assert n > 0 and st["hits"] > 0


@pytest.mark.parametrize("overlap", [False, True])
def test_prefetch_across_cache_updates(moe, overlap):
    """Cache updates between steps rewrite the layers' tables: the experts the slots
    held are read from their host copies (or the HBM slot an update gave them) until a
    prefetch places them again, and stale slots are freed."""
    E, L, S = 32, 3, 18
    rng = np.random.default_rng(5)

    def update(step, plan):
        if overlap:
            plan.cache_update(-1, decay=0.9, max_promotions=3, overlap=True)
            return list(range(L))  # the pipelined update uploads every layer's table
        want = np.zeros((L, E), np.int32)
        for l in range(L):
            want[l, rng.choice(E, size=S, replace=False)] = 1
        before = [plan.residency(l) for l in range(L)]
        plan.cache_update(-1, want_resident=want)
        return [l for l in range(L) if not np.array_equal(plan.residency(l), before[l])]

    st, n = _run_chain(moe, (512, 256, E, 4, 128), 2, S=S, P=5, L=L, steps=6, seed=43, cand=0, update=update)
    assert n > 0


def test_prefetch_logits_path_side_stream_and_reload(moe):
    """Given logits: the prediction is the oracle rule on them exactly. A forward on
    another stream still waits for the prefetch. Reloading a layer frees its slots."""
    import synth

    H, I, E, k, G, T, P = 512, 256, 32, 4, 128, 4, 6
    c = LC.make_case(H, I, E, k, G, "bf16", T, 47, alpha=0.5)
    pf, full = _plans(moe, [c], (H, I, E, k, G), T, 10, P)
    lg = LC.oracle_logits(c).astype(np.float32)
    pred = torch.full((P,), -7, dtype=torch.int32, device="cuda")
    x = torch.from_numpy(c.x_bits.view(np.int16).copy()).view(torch.bfloat16).cuda()
    pf.prefetch(0, logits_in=torch.from_numpy(lg).cuda(), candidates=5, predicted_out=pred)
    want, occ, copied = O.prefetch_step(lg, 5, P, pf.residency(0) < 0, np.full(P, -1), np.ones(P, bool))
    side = torch.cuda.Stream()
    y = torch.full((T, H), float("nan"), device="cuda")
    yf = torch.empty((T, H), device="cuda")
    with torch.cuda.stream(side):
        pf.forward(0, x, y, logits_in=torch.from_numpy(lg).cuda(), stream=side)
    side.synchronize()
    full.forward(0, x, yf, logits_in=torch.from_numpy(lg).cuda())
    torch.cuda.synchronize()
    exp = np.full(P, -1)
    exp[:len(want)] = want
    assert np.array_equal(pred.cpu().numpy(), exp) and len(copied) > 0
    assert np.array_equal(pf.prefetch_slots(0), occ)
    assert torch.equal(y, yf)
    ids = np.stack([O.topk_ids(lg[t], k) for t in range(T)])
    resident = pf.residency(0) >= 0
    resident[occ[occ >= 0]] = True
    a = O.link_accounting(ids, resident, synth.expert_bytes(H, I, G))
    st = pf.stats(0)
    assert st["hits"] == a["hits"] and st["misses"] == a["misses"] and st["prefetched"] == len(copied)
    pf.load_layer(0, c.Wr_store, c.b, c.blobs)
    assert (pf.prefetch_slots(0) == -1).all()
    pf.forward(0, x, y, logits_in=torch.from_numpy(lg).cuda())
    torch.cuda.synchronize()
    assert torch.equal(y, yf)
    pf.destroy()
    full.destroy()


def test_prefetch_argument_errors(moe):
    H, I, E, k, G = 256, 128, 8, 2, 32
    c = LC.make_case(H, I, E, k, G, "f32", 2, 3)
    cfg = moe.make_config(H, I, E, k, G, "f32", num_layers=2, max_tokens=64, hbm_slots=4, prefetch_slots=3)
    p = moe.Plan(cfg)
    p.load_layer(0, c.Wr_store, c.b, c.blobs)
    x = torch.zeros((64, H), device="cuda")
    with pytest.raises(moe.MoeError) as ei:  # layer 1 not loaded
        p.prefetch(1, x=x[:1])
    assert ei.value.status == moe.MOE_E_INVALID
    for kw in (dict(x=x[:1], candidates=9), dict(x=x[:1], candidates=-1)):
        with pytest.raises(moe.MoeError) as ei:
            p.prefetch(0, **kw)
        assert ei.value.status == moe.MOE_E_INVALID
    with pytest.raises(moe.MoeError) as ei:  # 64 tokens x 8 candidates = 512 is fine; 2 layers: bad layer
        p.prefetch(2, x=x)
    assert ei.value.status == moe.MOE_E_INVALID
    p.prefetch(0, x=x, candidates=8)
    torch.cuda.synchronize()
    p.destroy()
    cfg0 = moe.make_config(H, I, E, k, G, "f32", max_tokens=2, hbm_slots=4)
    p0 = moe.Plan(cfg0)
    p0.load_layer(0, c.Wr_store, c.b, c.blobs)
    with pytest.raises(moe.MoeError) as ei:
        p0.prefetch(0, x=x[:1])
    assert ei.value.status == moe.MOE_E_STATE
    p0.destroy()


def test_prefetch_candidate_limit(moe):
    H, I, E, k, G = 256, 128, 64, 2, 32
    c = LC.make_case(H, I, E, k, G, "f32", 1, 4)
    cfg = moe.make_config(H, I, E, k, G, "f32", max_tokens=64, hbm_slots=4, prefetch_slots=3)
    p = moe.Plan(cfg)
    p.load_layer(0, c.Wr_store, c.b, c.blobs)
    x = torch.zeros((64, H), device="cuda")
    with pytest.raises(moe.MoeError) as ei:  # 64 x 33 > 2048 candidates
        p.prefetch(0, x=x, candidates=33)
    assert ei.value.status == moe.MOE_E_INVALID
    p.prefetch(0, x=x, candidates=32)
    torch.cuda.synchronize()
    p.destroy()


def test_prefetch_qwen3_shaped_chain(moe):
    """Qwen3-30B-A3B-shaped layers (H2048 I768 E128 k8 G128), 90 HBM slots and 8
    prefetch slots per layer, batch 1, chained over 4 layers for 3 steps."""
    _run_chain(moe, (2048, 768, 128, 8, 128), 1, S=90, P=8, L=4, steps=3, seed=3, cand=0, oracle_every=4)


@pytest.mark.parametrize("prefetch", [True, False])
def test_graph_replayed_steps_match_eager(moe, prefetch):
    """A chained decode step (prefetch of layer l+1, forward of layer l, residual add)
    captured once into a HIP graph and replayed step after step, with a pipelined cache
    update and host synchronisation between replays, against the same steps enqueued
    eagerly on a second plan: every layer's y bitwise equal on every replay, and the
    slot tables and counters equal."""
    import synth

    H, I, E, k, G, L, T, steps, seed, S, P = 512, 256, 32, 4, 128, 3, 1, 6, 53, 20, 5
    layers = [LC.make_case(H, I, E, k, G, "bf16", 1, seed, alpha=0.8, layer=l) for l in range(L)]

    def make():
        cfg = moe.make_config(H, I, E, k, G, "bf16", num_layers=L, max_tokens=T, hbm_slots=S,
                              prefetch_slots=P if prefetch else 0)
        p = moe.Plan(cfg)
        for l, c in enumerate(layers):
            p.load_layer(l, c.Wr_store, c.b, c.blobs)
        return p

    pg, pe = make(), make()
    x0 = [torch.from_numpy(synth.activations(seed, 800 + i, T, H, "bf16").view(np.int16).copy()).view(
        torch.bfloat16).cuda() for i in range(steps)]

    def bufs():
        return (torch.empty((L + 1, T, H), dtype=torch.bfloat16, device="cuda"),
                torch.full((L, T, H), float("nan"), device="cuda"), torch.empty((T, H), device="cuda"))

    (xg, yg, ag), (xe, ye, ae) = bufs(), bufs()

    def layers_pass(plan, xl, ys, acc, st):
        for l in range(L):
            if prefetch and l + 1 < L:
                plan.prefetch(l + 1, x=xl[l], stream=st)
            plan.forward(l, xl[l], ys[l], stream=st)
            torch.add(xl[l], ys[l], out=acc)
            xl[l + 1].copy_(acc)

    cur = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(cur)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        layers_pass(pg, xg, yg, ag, torch.cuda.current_stream())
    torch.cuda.synchronize()
    pg.reset_stats()
    for i in range(steps):
        xg[0].copy_(x0[i])
        g.replay()
        pg.cache_update(-1, decay=0.9, max_promotions=3, overlap=True, stream=cur)
        xe[0].copy_(x0[i])
        layers_pass(pe, xe, ye, ae, cur)
        pe.cache_update(-1, decay=0.9, max_promotions=3, overlap=True, stream=cur)
        torch.cuda.synchronize()
        assert torch.isfinite(yg).all()
        assert torch.equal(yg, ye), "replay %d: y differs from the eager steps" % i
        for l in range(L):
            assert np.array_equal(pg.residency(l), pe.residency(l)), "replay %d layer %d" % (i, l)
            if prefetch:
                assert np.array_equal(pg.prefetch_slots(l), pe.prefetch_slots(l)), "replay %d layer %d" % (i, l)
        yg.fill_(float("nan"))
    sg, se = pg.stats(-1), pe.stats(-1)
    _say("  replayed: hits %d misses %d prefetched %d" % (sg["hits"], sg["misses"], sg["prefetched"]))
    for n in ("forwards", "hits", "misses", "bytes_hbm", "bytes_host", "prefetched", "promotions"):
        assert sg[n] == se[n], n
    assert sg["forwards"] == steps * L
    del g
    pg.destroy()
    pe.destroy()
