"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Integers (ids, counts, offsets, permutation, counters) are compared bit-exactly,
with the oracle's own logits fed to the library (logits_in) so both sides route
from the same values. Floats: y within rel-L2 1e-3 and max-abs 2e-2 of the
oracle's float64 result. With the library's own router, ids are compared where
the oracle's routing margin exceeds the logit error, and checked for validity
elsewhere.
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


def make_plan(moe, c, hbm_slots=None, resident=None, max_tokens=None, layers=1, gemm_min_tokens=0,
              prefill_stage_slots=0):
    cfg = moe.make_config(c.H, c.I, c.E, c.k, c.G, c.act, num_layers=layers,
                          max_tokens=max_tokens or max(c.T, 1),
                          hbm_slots=c.E if hbm_slots is None else hbm_slots, gemm_min_tokens=gemm_min_tokens,
                          prefill_stage_slots=prefill_stage_slots)
    plan = moe.Plan(cfg)
    plan.load_layer(0, c.Wr_store, c.b, c.blobs, resident)
    return plan


def route_bufs(c):
    A = c.T * c.k
    z = lambda n, dt=torch.int32: torch.full((n,), -7, dtype=dt, device="cuda")
    return dict(logits=torch.zeros(c.T * c.E, device="cuda"), topk_ids=z(A), topk_w=z(A, torch.float32),
                counts=z(c.E), offsets=z(c.E + 1), sorted=z(A), inv=z(A))


def run(plan, c, logits_in=None, route=None):
    x = dev_x(c)
    y = torch.full((c.T, c.H), float("nan"), device="cuda")
    li = None if logits_in is None else torch.from_numpy(np.ascontiguousarray(logits_in, np.float32)).cuda()
    plan.forward(0, x, y, logits_in=li, route=route)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def check_routing_exact(c, ref, rb):
    A = c.T * c.k
    np.testing.assert_array_equal(rb["topk_ids"].cpu().numpy().reshape(c.T, c.k), ref["ids"])
    np.testing.assert_array_equal(rb["counts"].cpu().numpy(), ref["counts"])
    np.testing.assert_array_equal(rb["offsets"].cpu().numpy(), ref["offsets"])
    np.testing.assert_array_equal(rb["sorted"].cpu().numpy(), ref["sorted"])
    np.testing.assert_array_equal(rb["inv"].cpu().numpy(), ref["inv"])
    w = rb["topk_w"].cpu().numpy().reshape(c.T, c.k).astype(np.float64)
    np.testing.assert_allclose(w, ref["w"], rtol=2e-6, atol=1e-7)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, atol=1e-6)
    assert A == ref["sorted"].size


def check_y(y, ref_y, label):
    r, m = LC.rel_l2(y, ref_y), LC.max_abs(y, ref_y)
    _say("  %s: rel_l2=%.3e max_abs=%.3e" % (label, r, m))
    assert np.all(np.isfinite(y))
    assert r <= LC.REL_L2_BAR, (label, r)
    assert m <= LC.MAX_ABS_BAR, (label, m)


# ----------------------------------------------------------------------------- shapes

SMALL = [
    # H, I, E, k, G, act, T, alpha, seed
    (256, 128, 8, 2, 32, "f32", 16, 0.0, 0),     # the tiny reference layer
    (384, 96, 12, 3, 32, "bf16", 13, 0.5, 11),   # several tiles, ragged group split, bf16
    (384, 96, 12, 3, 32, "f32", 7, 0.5, 12),
    (512, 256, 16, 16, 128, "bf16", 5, 0.0, 13),  # k = E
    (256, 64, 5, 1, 64, "bf16", 9, 0.0, 14),     # k = 1
    (384, 96, 12, 3, 32, "bf16", 2, 0.5, 15),    # batch 2
    (256, 128, 8, 2, 32, "f32", 1, 0.0, 16),     # batch 1, fp32 activations
    (512, 256, 16, 16, 128, "bf16", 2, 0.0, 17),  # k = E = 16 at batch 2
    (2048, 768, 128, 8, 128, "bf16", 1, 0.8, 1),  # Qwen3-30B-A3B-shaped, decode batch 1
    (2048, 768, 128, 8, 128, "bf16", 4, 0.8, 1),  # and batch 4 (down projection fused with the combine)
    (4096, 256, 24, 6, 128, "bf16", 2, 0.5, 18),  # fused down + combine: 64 tiles x 2 tokens, 12 waves
    (8192, 128, 16, 2, 64, "bf16", 1, 0.0, 19),   # fused at batch 1: 128 tiles, k * splits = 2 * 2
    (256, 128, 8, 2, 32, "f32", 150, 0.5, 20),    # T*k > 256: multi-block grouping, fp32 GEMVs, ragged last block
    (2048, 256, 16, 4, 256, "bf16", 2, 0.5, 21),  # G = 256 with experts holding 2 tokens (4-token kernel)
    (512, 256, 16, 4, 128, "f32", 2, 0.0, 22),    # fp32 rows, experts holding 2 tokens (4-token kernel)
    (1024, 2048, 16, 4, 128, "bf16", 1, 0.5, 23),  # 16-row fused down + combine with h staged in LDS (I > 1024)
    (512, 1280, 8, 2, 64, "bf16", 3, 0.0, 24),    # the same, G = 64, 5 chunks per wave (ragged chunk quarters)
    (1024, 2048, 16, 6, 128, "bf16", 1, 0.5, 25),  # staged, both 4-chunk load batches issued before the staging
    (1024, 2048, 16, 10, 128, "bf16", 1, 0.5, 26),  # staged, 16 chunk iterations per lane: batches pipelined
]


# bf16 cases of at least 6 tokens take the grouped MFMA GEMM by default; these run
# them again with the GEMM switched off, through the GEMVs
SMALL_GEMV = [(c + ("gemv",)) for c in SMALL if c[5] == "bf16" and c[6] >= 6]


@pytest.mark.parametrize("H,I,E,k,G,act,T,alpha,seed,path", [c + ("default",) for c in SMALL] + SMALL_GEMV)
def test_layer_parity_oracle_logits(moe, H, I, E, k, G, act, T, alpha, seed, path):
    _say("case", H, I, E, k, G, act, T, alpha, seed, path)
    c = LC.make_case(H, I, E, k, G, act, T, seed, alpha)
    lg = LC.oracle_logits(c)
    ref = LC.oracle_forward(c, logits_in=lg)
    plan = make_plan(moe, c, gemm_min_tokens=-1 if path == "gemv" else 0)
    rb = route_bufs(c)
    y = run(plan, c, logits_in=lg, route=rb)
    check_routing_exact(c, ref, rb)
    np.testing.assert_array_equal(rb["logits"].cpu().numpy().reshape(T, E), lg)
    check_y(y, ref["y"], "y")
    plan.destroy()


@pytest.mark.parametrize("H,I,E,k,G,act,T,alpha,seed", SMALL)
def test_layer_parity_gpu_router(moe, H, I, E, k, G, act, T, alpha, seed):
    _say("case", H, I, E, k, G, act, T, alpha, seed)
    c = LC.make_case(H, I, E, k, G, act, T, seed, alpha)
    ref = LC.oracle_forward(c)
    plan = make_plan(moe, c)
    rb = route_bufs(c)
    y = run(plan, c, route=rb)
    glog = rb["logits"].cpu().numpy().reshape(T, E).astype(np.float64)
    err = np.abs(glog - ref["logits"]).max()
    scale = np.abs(ref["logits"]).max()
    _say("  logits max err %.3e (max |l| %.3f)" % (err, scale))
    assert err <= 1e-5 * max(1.0, scale)
    tol = 1e-5 * max(1.0, scale)
    margins = LC.routing_margins(ref["logits"], k)
    ids = rb["topk_ids"].cpu().numpy().reshape(T, k)
    clear = margins > 2 * tol
    np.testing.assert_array_equal(ids[clear], ref["ids"][clear])
    for t in np.nonzero(~clear)[0]:
        assert LC.valid_topk(ref["logits"][t], ids[t], k, tol)
    check_y(y[clear], ref["y"][clear], "y (unambiguous tokens %d/%d)" % (clear.sum(), T))
    plan.destroy()


@pytest.mark.parametrize("gemm_min", [-1, 0])
def test_all_tokens_one_expert_multi_pass(moe, gemm_min):
    """Every token routed to the same k experts: one expert gets T > 8 tokens (several
    GEMV passes with gemm_min -1; one GEMM tile of 21 rows per expert with the default)."""
    c = LC.make_case(384, 96, 12, 3, 32, "bf16", 21, 21)
    lg = np.tile(np.array([0.0] * 9 + [3.0, 2.0, 1.0], np.float32), (c.T, 1))
    ref = LC.oracle_forward(c, logits_in=lg)
    plan = make_plan(moe, c, gemm_min_tokens=gemm_min)
    rb = route_bufs(c)
    y = run(plan, c, logits_in=lg, route=rb)
    check_routing_exact(c, ref, rb)
    check_y(y, ref["y"], "y")
    plan.destroy()


def test_t0_is_noop_and_bad_args(moe):
    c = LC.make_case(256, 128, 8, 2, 32, "f32", 4, 0)
    plan = make_plan(moe, c, max_tokens=4)
    x = dev_x(c)
    y = torch.full((4, 256), 5.0, device="cuda")
    plan.forward(0, x[:0], y[:0])
    torch.cuda.synchronize()
    assert torch.all(y == 5.0)
    big = torch.zeros((5, 256), device="cuda")
    with pytest.raises(moe.MoeError) as ei:
        plan.forward(0, big, big)
    assert ei.value.status == moe.MOE_E_INVALID
    plan.destroy()


def test_residency_invariance_bitwise(moe):
    """all-HBM, 70/30 (cold start: experts 0..89 in the slots) and all-host plans give
    bitwise equal y, before and after cache updates that move experts."""
    c = LC.make_case(2048, 768, 128, 8, 128, "bf16", 4, 3, alpha=0.8)
    lg = LC.oracle_logits(c)
    y_router, y_given = [], []
    for slots in (128, 90, 0):
        plan = make_plan(moe, c, hbm_slots=slots)
        y_router.append(run(plan, c))
        y_given.append(run(plan, c, logits_in=lg))
        if slots == 90:
            for _ in range(3):
                plan.cache_update(0, max_promotions=16)
                y_router.append(run(plan, c))
                y_given.append(run(plan, c, logits_in=lg))
            assert plan.stats(0)["promotions"] > 0
        plan.destroy()
    for y in y_router[1:]:
        np.testing.assert_array_equal(y, y_router[0])
    for y in y_given[1:]:
        np.testing.assert_array_equal(y, y_given[0])
    ref = LC.oracle_forward(c, logits_in=lg)
    check_y(y_given[0], ref["y"], "y")


def test_counters_recount(moe):
    import synth
    c = LC.make_case(2048, 768, 128, 8, 128, "bf16", 4, 5, alpha=0.8)
    res = synth.coldest_host_plan(5, 0, 128, 0.7)
    plan = make_plan(moe, c, hbm_slots=int(res.sum()), resident=res)
    lg = LC.oracle_logits(c)
    ref = LC.oracle_forward(c, logits_in=lg)
    run(plan, c, logits_in=lg)
    run(plan, c, logits_in=lg)
    st = plan.stats(0)
    acc = O.link_accounting(ref["ids"], res, synth.expert_bytes(2048, 768, 128))
    assert st["forwards"] == 2 and st["tokens"] == 8
    assert st["hits"] == 2 * acc["hits"] and st["misses"] == 2 * acc["misses"]
    assert st["bytes_hbm"] == 2 * acc["bytes_hbm"] and st["bytes_host"] == 2 * acc["bytes_host"]
    slot_of = plan.residency(0)
    assert np.array_equal(slot_of >= 0, res.astype(bool))
    plan.destroy()


def test_token_order_invariance_bitwise(moe):
    c = LC.make_case(2048, 768, 128, 8, 128, "bf16", 4, 6, alpha=0.8)
    plan = make_plan(moe, c)
    y = run(plan, c)
    perm = np.array([2, 0, 3, 1])
    c2 = LC.make_case(2048, 768, 128, 8, 128, "bf16", 4, 6, alpha=0.8)
    c2.x_bits = c.x_bits[perm].copy()
    y2 = run(plan, c2)
    np.testing.assert_array_equal(y2, y[perm])
    plan.destroy()


@pytest.mark.parametrize("T,gemm_min", [(40, -1), (40, 0), (16, 0), (2048, 0)])
def test_large_batch_routing_and_sampled_outputs(moe, T, gemm_min):
    """T*k > 64: multi-block top-k and the block grouping path. Routing is compared
    bit-exactly for every token; y on a seeded sample of tokens (the whole batch for
    T <= 64). gemm_min -1: the GEMVs; 0: the default dispatch (the MFMA GEMM here)."""
    c = LC.make_case(2048, 768, 128, 8, 128, "bf16", T, 4)
    lg = LC.oracle_logits(c)
    rng = np.random.default_rng(T)
    toks = np.arange(T) if T <= 64 else np.sort(rng.choice(T, 48, replace=False))
    ref = LC.oracle_forward(c, logits_in=lg, tokens=toks)
    plan = make_plan(moe, c, gemm_min_tokens=gemm_min)
    rb = route_bufs(c)
    y = run(plan, c, logits_in=lg, route=rb)
    check_routing_exact(c, ref, rb)
    check_y(y[toks], ref["y"], "y (%d sampled tokens)" % len(toks))
    plan.destroy()


PREFILL = [
    # H, I, E, k, G, T, seed: T >= 256 takes the grouped MFMA GEMM path
    (384, 96, 12, 3, 32, 300, 21),     # G = 32, 3 gate/up n-tiles (one idle wave per workgroup)
    (512, 256, 16, 4, 128, 600, 22),
    (2048, 768, 128, 8, 128, 1024, 4),  # Qwen3-30B-A3B-shaped prefill micro-batch
    (1024, 512, 32, 4, 64, 700, 5),     # G = 64; the last tile of most experts has <= 32 rows
    (2048, 1536, 64, 8, 256, 500, 7),   # G = 256: two 128-wide passes per quantisation group
]


@pytest.mark.parametrize("H,I,E,k,G,T,seed", PREFILL)
def test_prefill_mfma_parity(moe, H, I, E, k, G, T, seed):
    c = LC.make_case(H, I, E, k, G, "bf16", T, seed, alpha=0.5 if E < 100 else 0.0)
    lg = LC.oracle_logits(c)
    rng = np.random.default_rng(seed)
    toks = np.sort(rng.choice(T, min(T, 64), replace=False))
    ref = LC.oracle_forward(c, logits_in=lg, tokens=toks)
    plan = make_plan(moe, c, gemm_min_tokens=256)
    rb = route_bufs(c)
    y = run(plan, c, logits_in=lg, route=rb)
    check_routing_exact(c, ref, rb)
    check_y(y[toks], ref["y"], "prefill y (%d sampled tokens of %d)" % (len(toks), T))
    # every token, a second run: the grouped GEMM has no order-dependent reductions,
    # so y repeats bit for bit (NaN compares equal here, so a NaN fails the checks above)
    y_again = run(plan, c, logits_in=lg, route=rb)
    assert np.all(np.isfinite(y))
    np.testing.assert_array_equal(y_again, y)
    # the MFMA router: logits within fp32 accumulation error, ids where unambiguous
    rb2 = route_bufs(c)
    y2 = run(plan, c, route=rb2)
    glog = rb2["logits"].cpu().numpy().reshape(T, E).astype(np.float64)
    err = np.abs(glog - lg).max()
    tol = 1e-5 * max(1.0, np.abs(lg).max())
    _say("  router logits max err %.3e" % err)
    assert err <= tol
    margins = LC.routing_margins(lg, k)
    clear = margins > 2 * tol
    ids = rb2["topk_ids"].cpu().numpy().reshape(T, k)
    np.testing.assert_array_equal(ids[clear], ref["ids"][clear])
    sel = [i for i, t in enumerate(toks) if clear[t]]
    check_y(y2[toks[sel]], ref["y"][sel], "prefill y, MFMA router (%d tokens)" % len(sel))
    plan.destroy()


@pytest.mark.parametrize("T,seed", [(512, 31), (300, 32)])
def test_prefill_offloaded_experts_staged(moe, T, seed):
    """GEMM-path forwards with offloaded experts: read in place, all staged into HBM
    slots first, partly staged (fewer slots than active offloaded experts), all
    experts offloaded and staged. y is bitwise equal to the all-HBM plan's (the
    same GEMMs read the same bytes from another place), the link counters match
    an exact recount, and the staged forward matches the oracle on sampled tokens."""
    import synth
    c = LC.make_case(2048, 768, 128, 8, 128, "bf16", T, seed, alpha=0.0)
    lg = LC.oracle_logits(c)
    res = synth.coldest_host_plan(seed, 0, 128, 0.7)
    eb = synth.expert_bytes(2048, 768, 128)
    plans = [("hbm", 128, 0, None), ("in place", 90, 0, res), ("staged", 90, 128, res),
             ("partly staged", 90, 5, res), ("all offloaded, staged", 0, 128, np.zeros(128, np.int32))]
    ys = {}
    for name, slots, stage, resident in plans:
        plan = make_plan(moe, c, hbm_slots=slots, resident=resident, gemm_min_tokens=256,
                         prefill_stage_slots=stage)
        ys[name] = run(plan, c, logits_in=lg)
        ys[name + " again"] = run(plan, c, logits_in=lg)
        st = plan.stats(0)
        if 0 < slots < 128:  # experts promoted and evicted under a staged plan: still the same y
            plan.cache_update(0, max_promotions=16)
            ys[name + " after a cache update"] = run(plan, c, logits_in=lg)
            assert plan.stats(0)["promotions"] > 0
        in_hbm = np.ones(128, np.int32) if resident is None else resident
        acc = O.link_accounting(O.route(lg, c.k)[0], in_hbm, eb)
        assert st["bytes_host"] == 2 * acc["bytes_host"] and st["bytes_hbm"] == 2 * acc["bytes_hbm"], name
        _say("  %s: %d offloaded experts touched" % (name, acc["bytes_host"] // eb))
        plan.destroy()
    for name, y in ys.items():
        np.testing.assert_array_equal(y, ys["hbm"], err_msg=name)
    rng = np.random.default_rng(seed)
    toks = np.sort(rng.choice(T, 48, replace=False))
    ref = LC.oracle_forward(c, logits_in=lg, tokens=toks)
    check_y(ys["staged"][toks], ref["y"], "staged prefill y (%d sampled tokens)" % len(toks))


# ----------------------------------------------------------------------------- full-size DeepSeek-style layer

DS_LAYER = dict(H=7168, I=2048, E=384, k=6, G=128, seed=2, alpha=1.0)
DS_CHECKED = {1: [0], 4: [0, 1, 2, 3], 16: [0, 2, 4, 6, 8, 10, 12, 14]}  # batch -> tokens whose outputs are compared


@pytest.fixture(scope="module")
def deepseek_layer(moe):
    """The DeepSeek-style layer at its full size (H7168 I2048 E384 k6 G128, Zipf bias alpha
    1.0), one seeded batch per size. Experts that the checked tokens route to carry their
    generated weights; every other expert is filled with its own constant code byte and
    small finite scales, so a read of a wrong expert changes the result. The oracle's y on
    the checked tokens is computed once here and shared by the plans tested below."""
    import concurrent.futures
    import synth
    d = DS_LAYER
    H, I, E, k, G, seed = d["H"], d["I"], d["E"], d["k"], d["G"], d["seed"]
    Wr_store = synth.router_weight(seed, 0, E, H, "bf16")
    Wr, b = O.bf16_bits_to_f64(Wr_store), synth.router_bias(seed, 0, E, d["alpha"])
    cases, need = {}, set()
    for T, toks in DS_CHECKED.items():
        c = LC.Case(H, I, E, k, G, "bf16", T, seed, d["alpha"], 0)
        c.x_bits = synth.activations(seed, 100 + T, T, H, "bf16")
        c.x, c.Wr_store, c.Wr, c.b = O.bf16_bits_to_f64(c.x_bits), Wr_store, Wr, b
        c.lg = LC.oracle_logits(c)
        need |= set(int(e) for e in O.route(c.lg, k)[0][toks].ravel())
        cases[T] = c
    eb = synth.expert_bytes(H, I, G)
    blobs = np.empty((E, eb), np.uint8)
    a0 = O.expert_layout(H, I, G)[0]["s_gate"][0]
    for e in range(E):
        blobs[e, :a0].fill((37 * e + 11) & 0xFF)
        blobs[e, a0:].view(np.uint16)[:] = 0x2000  # fp16 2^-7
    with concurrent.futures.ThreadPoolExecutor(8) as ex:
        for e, blob in zip(sorted(need), ex.map(lambda e: synth.expert_blobs(seed, 0, e, 1, H, I, G)[0],
                                                sorted(need))):
            blobs[e] = blob
    _say("  deepseek-shaped layer: %d generated experts" % len(need))
    for T, c in cases.items():
        c.blobs = blobs
        c.ref = LC.oracle_forward(c, logits_in=c.lg, tokens=np.array(DS_CHECKED[T]))
        _say("  oracle y for batch %d (%d tokens) done" % (T, len(DS_CHECKED[T])))
    res = synth.coldest_host_plan(seed, 0, E, 0.7)  # 269 experts in HBM, the 115 coldest on the host
    return cases, blobs, res


def _deepseek_plan(moe, deepseek_layer, plan_kind):
    cases, blobs, res = deepseek_layer
    d = DS_LAYER
    if plan_kind == "mixed":
        slots, resident = int(res.sum()), res
    else:  # every expert read from host memory over the host link
        slots, resident = 0, np.zeros(d["E"], np.int32)
    cfg = moe.make_config(d["H"], d["I"], d["E"], d["k"], d["G"], "bf16", max_tokens=max(DS_CHECKED),
                          hbm_slots=slots)
    plan = moe.Plan(cfg)
    c0 = cases[1]
    plan.load_layer(0, c0.Wr_store, c0.b, blobs, resident)
    return plan, resident


@pytest.mark.timeout(900)
@pytest.mark.parametrize("plan_kind", ["mixed", "host"])
def test_deepseek_shaped_full_size(moe, deepseek_layer, plan_kind):
    """Full-size DeepSeek-style layer in the launch configuration the benchmark times
    (default dispatch: GEMVs with the 16-row fused down + combine at batches 1 and 4, the
    grouped MFMA GEMM at 16), on the 70/30 plan (the 115 coldest experts read from host
    memory) and on the all-host plan (every expert over the host link). Routing bit-exact
    against the oracle for every token; y on the checked tokens (8 of 16 at batch 16), with
    the oracle's logits and with the library's router; link counters against an exact
    recount."""
    import synth
    cases = deepseek_layer[0]
    plan, resident = _deepseek_plan(moe, deepseek_layer, plan_kind)
    try:
        for T in sorted(DS_CHECKED):
            c = cases[T]
            toks = np.array(DS_CHECKED[T])
            ref = c.ref
            rb = route_bufs(c)
            plan.reset_stats()
            y = run(plan, c, logits_in=c.lg, route=rb)
            full = O.route(c.lg, c.k)
            counts, offsets, srt, inv = O.align_permute(full[0], c.E)
            np.testing.assert_array_equal(rb["topk_ids"].cpu().numpy().reshape(c.T, c.k), full[0])
            np.testing.assert_array_equal(rb["counts"].cpu().numpy(), counts)
            np.testing.assert_array_equal(rb["offsets"].cpu().numpy(), offsets)
            np.testing.assert_array_equal(rb["sorted"].cpu().numpy(), srt)
            np.testing.assert_array_equal(rb["inv"].cpu().numpy(), inv)
            assert np.all(np.isfinite(y))
            check_y(y[toks], ref["y"], "deepseek-shaped y, %s plan, batch %d (tokens %s)" % (
                plan_kind, T, toks.tolist()))
            st = plan.stats(0)
            acc = O.link_accounting(full[0], resident, synth.expert_bytes(c.H, c.I, c.G))
            assert (st["hits"], st["misses"]) == (acc["hits"], acc["misses"])
            assert (st["bytes_hbm"], st["bytes_host"]) == (acc["bytes_hbm"], acc["bytes_host"])
            if plan_kind == "host":
                assert st["bytes_hbm"] == 0 and st["hits"] == 0
            # the library's router: logits within fp32 accumulation error, y where the routing is clear
            rb2 = route_bufs(c)
            y2 = run(plan, c, route=rb2)
            glog = rb2["logits"].cpu().numpy().reshape(c.T, c.E).astype(np.float64)
            tol = 1e-5 * max(1.0, np.abs(c.lg).max())
            assert np.abs(glog - c.lg).max() <= tol
            clear = LC.routing_margins(c.lg, c.k)[toks] > 2 * tol
            if clear.any():
                check_y(y2[toks[clear]], ref["y"][clear], "deepseek-shaped y, library router, %s plan, batch %d" % (
                    plan_kind, T))
    finally:
        plan.destroy()
