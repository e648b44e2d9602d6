"""Expert-cache decode run in small dimensions: stacked layers, single-token steps with a
chained hidden state, a cache update after every step (cold start: experts 0..S-1 in the
slots), checked step by step against
  - an all-HBM plan on the same inputs (y bitwise equal: placement never changes values),
  - the oracle's cache policy fed with the counts recounted from the emitted expert ids
    (slot tables equal after every update),
  - the oracle's link accounting under the residency each step ran with (exact counters),
  - the oracle forward on a few (step, layer) pairs (tolerance bars).
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


@pytest.mark.parametrize("T,overlap", [(1, False), (3, False), (1, True), (3, True)])
def test_chained_cache_run(moe, T, overlap):
    """overlap: the pipelined update. Its policy reads the counts of the step before
    the one just run, and the experts it promotes are still read from host memory
    until the next update (their copies run meanwhile). A final synchronous update
    then adds the last staged counts and makes every promotion visible."""
    import synth

    H, I, E, k, G, L, steps, seed = 512, 256, 32, 4, 128, 4, 10, 31
    S = int(round(0.7 * E))
    eb = synth.expert_bytes(H, I, G)
    layers = [LC.make_case(H, I, E, k, G, "bf16", 1, seed, alpha=0.8, layer=l) for l in range(L)]

    def plan_with(slots):
        cfg = moe.make_config(H, I, E, k, G, "bf16", num_layers=L, max_tokens=T, hbm_slots=slots)
        p = moe.Plan(cfg)
        for l, c in enumerate(layers):
            p.load_layer(l, c.Wr_store, c.b, c.blobs)
        return p

    cached, full = plan_with(S), plan_with(E)
    slot_ref = [np.where(np.arange(E) < S, np.arange(E), -1) for _ in range(L)]
    table_ref = [v.copy() for v in slot_ref]  # what the kernels read
    score_ref = [np.zeros(E) for _ in range(L)]
    prev_counts, n_prom = None, 0
    for l in range(L):
        assert np.array_equal(cached.residency(l), slot_ref[l])
    acc = dict(hits=0, misses=0, bytes_hbm=0, bytes_host=0)
    checked = 0
    for step in range(steps):
        r = torch.from_numpy(synth.activations(seed, 500 + step, T, H, "f32")).cuda()
        counts = [np.zeros(E, np.int64) for _ in range(L)]
        for l in range(L):
            x = r.to(torch.bfloat16)
            A = T * k
            rb = dict(logits=torch.zeros(T * E, device="cuda"), topk_ids=torch.zeros(A, dtype=torch.int32,
                                                                                    device="cuda"))
            y = torch.full((T, H), float("nan"), device="cuda")
            yf = torch.full((T, H), float("nan"), device="cuda")
            cached.forward(l, x, y, route=rb)
            full.forward(l, x, yf)
            torch.cuda.synchronize()
            assert torch.equal(y, yf), "step %d layer %d: y differs between the cached and all-HBM plans" % (step, l)
            ids = rb["topk_ids"].cpu().numpy().reshape(T, k)
            counts[l] += np.bincount(ids.ravel(), minlength=E)
            a = O.link_accounting(ids, table_ref[l] >= 0, eb)
            for n in acc:
                acc[n] += a[n]
            if (step * L + l) % 7 == 0:  # oracle on the exact bf16 input and the GPU logits
                c = layers[l]
                xb = x.view(torch.int16).cpu().numpy().view(np.uint16)
                lg = rb["logits"].cpu().numpy().reshape(T, E).astype(np.float64)
                ref = O.layer_forward(O.bf16_bits_to_f64(xb), c.Wr, c.b, c.blobs, H, I, E, k, G, "bf16",
                                      logits_in=lg)
                np.testing.assert_array_equal(ids, ref["ids"])
                yv = y.cpu().numpy().astype(np.float64)
                assert LC.rel_l2(yv, ref["y"]) <= LC.REL_L2_BAR
                assert LC.max_abs(yv, ref["y"]) <= LC.MAX_ABS_BAR
                checked += 1
            r = r + y
        cached.cache_update(-1, decay=0.9, max_promotions=3, overlap=overlap)
        policy_counts = (prev_counts if overlap else counts)
        for l in range(L):
            promoted = []
            if policy_counts is not None:
                score_ref[l], slot_ref[l], promoted, _ = O.cache_policy_step(score_ref[l], policy_counts[l],
                                                                            slot_ref[l], S, 0.9, 3)
            n_prom += len(promoted)
            table_ref[l] = slot_ref[l].copy()
            if overlap:
                for e, _ in promoted:
                    table_ref[l][e] = -1
            assert np.array_equal(cached.residency(l), table_ref[l]), "step %d layer %d: slot table" % (step, l)
        prev_counts = counts
    if overlap:  # synchronous update: the counts the last pipelined update staged, then all visible
        cached.cache_update(-1, decay=0.9, max_promotions=3)
        for l in range(L):
            score_ref[l], slot_ref[l], promoted, _ = O.cache_policy_step(score_ref[l], prev_counts[l], slot_ref[l],
                                                                        S, 0.9, 3)
            n_prom += len(promoted)
            assert np.array_equal(cached.residency(l), slot_ref[l]), "final sync update, layer %d" % l
    st = cached.stats(-1)
    _say("  hits %d misses %d promotions %d evictions %d (oracle checks %d)" % (
        st["hits"], st["misses"], st["promotions"], st["evictions"], checked))
    for n in acc:
        assert st[n] == acc[n], n
    assert st["forwards"] == steps * L and st["tokens"] == steps * L * T
    assert st["promotions"] == n_prom > 0 and st["bytes_copied"] == st["promotions"] * eb
    cached.destroy()
    full.destroy()


def _replay_policy(ids_steps, E, S, L, decay, maxp, overlap):
    """The oracle's policy replayed over recorded expert ids ([steps][L][T*k]) from the
    cold start: per step, the tables the kernels read during that step (before the update
    that follows it) and the tables after the update."""
    slot = [np.where(np.arange(E) < S, np.arange(E), -1) for _ in range(L)]
    score = [np.zeros(E) for _ in range(L)]
    read_tables, after = [], []
    table = [v.copy() for v in slot]
    prev = None
    for step_ids in ids_steps:
        read_tables.append([t.copy() for t in table])
        counts = [np.bincount(np.asarray(step_ids[l]).ravel(), minlength=E) for l in range(L)]
        pol = prev if overlap else counts
        for l in range(L):
            promoted = []
            if pol is not None:
                score[l], slot[l], promoted, _ = O.cache_policy_step(score[l], pol[l], slot[l], S, decay, maxp)
            table[l] = slot[l].copy()
            if overlap:
                for e, _ in promoted:
                    table[l][e] = -1  # copy in flight: still read from host memory
        after.append([t.copy() for t in table])
        prev = counts
    return read_tables, after


@pytest.mark.parametrize("T", [1, 3])
def test_pipelined_updates_without_host_sync(moe, T):
    """Steps of forward + pipelined cache update queued back to back with no host
    synchronisation in the loop: the promotion copies run on the plan's copy stream while
    later forwards are queued, and each table upload waits for them on the device. The
    hidden state chains on the device. After one final synchronisation every step's y is
    compared bitwise with an all-HBM plan run in the same stream order, the slot tables
    recorded after every update with the oracle policy (one update late), and the link
    counters with an exact recount under the tables each step read."""
    import synth

    H, I, E, k, G, L, steps, seed = 512, 256, 32, 4, 128, 4, 12, 33
    S = int(round(0.7 * E))
    eb = synth.expert_bytes(H, I, G)
    layers = [LC.make_case(H, I, E, k, G, "bf16", 1, seed, alpha=0.8, layer=l) for l in range(L)]

    def plan_with(slots):
        cfg = moe.make_config(H, I, E, k, G, "bf16", num_layers=L, max_tokens=T, hbm_slots=slots)
        p = moe.Plan(cfg)
        for l, c in enumerate(layers):
            p.load_layer(l, c.Wr_store, c.b, c.blobs)
        return p

    cached, full = plan_with(S), plan_with(E)
    torch.cuda.synchronize()
    ys = torch.full((steps, L, T, H), float("nan"), device="cuda")
    yfs = torch.full((steps, L, T, H), float("nan"), device="cuda")
    ids = torch.full((steps, L, T * k), -1, dtype=torch.int32, device="cuda")
    r = torch.from_numpy(synth.activations(seed, 900, T, H, "f32")).cuda()
    tables = []
    for step in range(steps):
        for l in range(L):
            x = r.to(torch.bfloat16)
            cached.forward(l, x, ys[step, l], route={"topk_ids": ids[step, l]})
            full.forward(l, x, yfs[step, l])
            r = r + ys[step, l]
        cached.cache_update(-1, decay=0.9, max_promotions=3, overlap=True)
        tables.append([cached.residency(l) for l in range(L)])
    torch.cuda.synchronize()
    assert torch.isfinite(ys).all()
    assert torch.equal(ys, yfs), "y differs between the cached plan and the all-HBM plan"
    ids_h = ids.cpu().numpy()
    read_tables, after = _replay_policy([ids_h[s] for s in range(steps)], E, S, L, 0.9, 3, True)
    acc = dict(hits=0, misses=0, bytes_hbm=0, bytes_host=0)
    for s in range(steps):
        for l in range(L):
            assert np.array_equal(tables[s][l], after[s][l]), "step %d layer %d: slot table" % (s, l)
            a = O.link_accounting(ids_h[s, l].reshape(T, k), read_tables[s][l] >= 0, eb)
            for n in acc:
                acc[n] += a[n]
    st = cached.stats(-1)
    _say("  hits %d misses %d promotions %d" % (st["hits"], st["misses"], st["promotions"]))
    for n in acc:
        assert st[n] == acc[n], n
    assert st["promotions"] > 0
    cached.destroy()
    full.destroy()


CACHE_CHECKS = [(0, 0), (0, 47), (1, 1), (37, 20), (128, 30), (200, 5), (254, 46), (255, 47)]


@pytest.mark.timeout(1200)
def test_cache_run_full_size_48_layers(moe):
    """The benchmark's expert-cache run at its full size: 48 Qwen3-30B-A3B-shaped layers
    (H2048 I768 E128 k8 G128, Zipf alpha 0.8 seeded per layer), 90 HBM slots per layer from
    the cold start, 256 single-token steps on the benchmark's seeded activations, a
    pipelined cache update after every step and no host synchronisation in the loop.
    Checked: y bitwise equal to an all-HBM plan at every (step, layer); the oracle forward
    on sampled (step, layer) pairs (the exact bf16 input and the library's logits); the
    slot tables after every update against the oracle policy; the link counters against
    an exact recount."""
    import synth

    H, I, E, k, G, L, steps, seed, alpha = 2048, 768, 128, 8, 128, 48, 256, 3, 0.8
    S = int(round(0.7 * E))
    eb = synth.expert_bytes(H, I, G)
    cfgs = {}
    plans = {}
    for name, slots in (("cached", S), ("full", E)):
        cfgs[name] = moe.make_config(H, I, E, k, G, "bf16", num_layers=L, max_tokens=1, hbm_slots=slots)
        plans[name] = moe.Plan(cfgs[name])
    layer_data = []
    for l in range(L):
        blobs = synth.expert_blobs(seed, l, 0, E, H, I, G)
        Wr = synth.router_weight(seed, l, E, H, "bf16")
        b = synth.router_bias(seed, l, E, alpha)
        for p in plans.values():
            p.load_layer(l, Wr, b, blobs)
        layer_data.append((Wr, b))
        if l in {pair[1] for pair in CACHE_CHECKS}:
            layer_data[-1] = (Wr, b, blobs)
        if l % 8 == 7:
            _say("  %d layers generated and loaded" % (l + 1))
    xb = synth.activations(seed, 7000, steps * L, H, "bf16")  # the benchmark's (step, layer) inputs
    xs = torch.from_numpy(xb.view(np.int16).copy()).view(torch.bfloat16).cuda().view(steps * L, 1, H)
    ys = torch.full((steps * L, H), float("nan"), device="cuda")
    mism = torch.zeros((), dtype=torch.int64, device="cuda")
    ids = torch.full((steps, L, k), -1, dtype=torch.int32, device="cuda")
    chk_logits = {pair: torch.zeros(E, device="cuda") for pair in CACHE_CHECKS}
    yf = torch.empty((1, H), device="cuda")
    torch.cuda.synchronize()
    tables = []
    cached, full = plans["cached"], plans["full"]
    for s in range(steps):
        for l in range(L):
            i = s * L + l
            route = {"topk_ids": ids[s, l]}
            if (s, l) in chk_logits:
                route["logits"] = chk_logits[(s, l)]
            cached.forward(l, xs[i], ys[i:i + 1], route=route)
            full.forward(l, xs[i], yf)
            mism += (ys[i:i + 1] != yf).sum()
        cached.cache_update(-1, decay=0.9, max_promotions=8, overlap=True)
        tables.append([cached.residency(l) for l in range(L)])
        if s % 64 == 63:
            _say("  %d steps queued" % (s + 1))
    torch.cuda.synchronize()
    assert int(mism.item()) == 0, "y differs between the cached plan and the all-HBM plan"
    assert torch.isfinite(ys).all()
    ids_h = ids.cpu().numpy()
    for (s, l) in CACHE_CHECKS:
        Wr, b, blobs = layer_data[l]
        i = s * L + l
        lg = chk_logits[(s, l)].cpu().numpy().reshape(1, E).astype(np.float64)
        ref = O.layer_forward(O.bf16_bits_to_f64(xb[i:i + 1]), O.bf16_bits_to_f64(Wr), b, blobs, H, I, E, k, G,
                              "bf16", logits_in=lg)
        np.testing.assert_array_equal(ids_h[s, l].reshape(1, k), ref["ids"])
        yv = ys[i:i + 1].cpu().numpy().astype(np.float64)
        r, m = LC.rel_l2(yv, ref["y"]), LC.max_abs(yv, ref["y"])
        _say("  step %d layer %d: rel_l2=%.3e max_abs=%.3e" % (s, l, r, m))
        assert r <= LC.REL_L2_BAR and m <= LC.MAX_ABS_BAR
    read_tables, after = _replay_policy([ids_h[s] for s in range(steps)], E, S, L, 0.9, 8, True)
    acc = dict(hits=0, misses=0, bytes_hbm=0, bytes_host=0)
    for s in range(steps):
        for l in range(L):
            assert np.array_equal(tables[s][l], after[s][l]), "step %d layer %d: slot table" % (s, l)
            a = O.link_accounting(ids_h[s, l].reshape(1, k), read_tables[s][l] >= 0, eb)
            for n in acc:
                acc[n] += a[n]
    st = cached.stats(-1)
    _say("  hit rate %.4f, %d promotions" % (st["hits"] / max(1, st["hits"] + st["misses"]), st["promotions"]))
    for n in acc:
        assert st[n] == acc[n], n
    cached.destroy()
    full.destroy()
