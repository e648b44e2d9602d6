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
