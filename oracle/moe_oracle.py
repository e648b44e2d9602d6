"""CPU oracle for the forward pass of one routed MoE FFN layer.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline may import this module; the GPU library never calls it, and this
module imports nothing from the GPU package.

Plain NumPy float64, evaluated assignment by assignment, so that a reader can
check each step against its source by eye:

    y_t = sum_{j<k} w_{t,j} * FFN_{e_{t,j}}(x_t)
    FFN_e(x) = Wd_e . rho( silu(Wg_e x) * (Wu_e x) ),   W = q * s  (int4 code times fp16 scale)

Sources. The pages describe the problem; they fix no formula:
  * Page "763B MoE 塞进两张 96GB 显卡：闲置专家丢进主机内存", section
    "显存缺口从哪里来": each token, in each layer, is routed to a few of the
    layer's experts (6 of 384); the rest sit idle. Offloaded experts are read
    by GPU kernels from host memory through unified addressing, which moves
    bytes but not values.
  * Same page, section "同一个思路，vLLM 原生方案反而跑不通": a per-expert plan
    decides each expert's residency and read path individually; placement is
    a matter of data layout and read path, not of the computed result.
  * Page "我在 32GB 单卡上跑两万四千专家的 MoE:分层放置实测与三个坑",
    section "一、第一个坑:MoE 省算力,不省内存": which experts a token uses is
    decided at run time by the gate.
  * Same page, section "二、跑起来靠的是分层,不是激活": an expert cache in VRAM
    holds the most used experts and adapts with use (policy below).
The pages leave the numerics open. The readings taken here: softmax scores,
top-k on the logits with ties to the lower expert id, weights renormalised over
the selected k, SwiGLU experts, symmetric int4 codes with one fp16 scale per
group of G along K, the intermediate h rounded to the activation dtype, y in
fp32, gate weights applied after the down projection in slot order.

Parity pins: every function here is pinned by tests/test_oracle_pins.py
(brute force, closed forms, invariants, library cross-checks).
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------- formats


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """Canonical nibble decode along the last axis.

    Byte j of a row holds code 2j in its low nibble and code 2j+1 in its high
    nibble; a nibble n is two's complement, q = n - 16 when n >= 8, so every
    one of the 16 nibbles decodes (to [-8, 7]).
    """
    p = np.asarray(packed, dtype=np.uint8)
    lo = (p & 0x0F).astype(np.int16)
    hi = (p >> 4).astype(np.int16)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def unpack_codes(packed: np.ndarray, bits: int) -> np.ndarray:
    """Canonical b-bit decode along the last axis (the lower-bit formats; the pages name
    3-bit and about 2-bit packages without giving their layouts, so this is the library's
    own format). Code i of a row is the unsigned n at bits [b*i, b*i+b) of the row's
    little-endian bit string (bit j = bit j % 8 of byte j // 8). The weight code is
    q = n - 16 (n >= 8) for b = 4 (two's complement) and q = 2n - (2^b - 1) for b = 3, 2
    (odd levels, symmetric about zero)."""
    if bits == 4:
        return unpack_int4(packed)
    p = np.asarray(packed, dtype=np.uint8)
    stream = np.unpackbits(p, axis=-1, bitorder="little")  # bit j of byte i at 8i + j
    fields = stream.reshape(p.shape[:-1] + (-1, bits)).astype(np.int16)
    n = (fields * (1 << np.arange(bits, dtype=np.int16))).sum(axis=-1)
    return (2 * n - ((1 << bits) - 1)).astype(np.int8)


def fp16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """IEEE binary16 bit patterns to float64 (exact)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns to float64 (exact): the upper half of a float32."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u32.view(np.float32).astype(np.float64)


def expert_layout(H: int, I: int, G: int, bits: int = 4):
    """Byte ranges of the canonical expert blob, in order (b = bits per code):
    q_gate[I][H*b/8] | q_up[I][H*b/8] | q_down[H][I*b/8] | s_gate[I][H/G] | s_up[I][H/G] | s_down[H][I/G].
    """
    sizes = [("q_gate", I * H * bits // 8), ("q_up", I * H * bits // 8), ("q_down", H * I * bits // 8),
             ("s_gate", 2 * I * (H // G)), ("s_up", 2 * I * (H // G)), ("s_down", 2 * H * (I // G))]
    out, off = {}, 0
    for name, n in sizes:
        out[name] = (off, off + n)
        off += n
    return out, off


def expert_bytes(H: int, I: int, G: int, bits: int = 4) -> int:
    return expert_layout(H, I, G, bits)[1]


def dequant(q: np.ndarray, s: np.ndarray, G: int) -> np.ndarray:
    """W[n, k] = q[n, k] * s[n, k // G] in float64 (exact: a 4-bit by 11-bit product)."""
    q = np.asarray(q, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    return q * np.repeat(s, G, axis=1)


def expert_weights(blob: np.ndarray, H: int, I: int, G: int, bits: int = 4):
    """Dequantised (Wg [I,H], Wu [I,H], Wd [H,I]) of one canonical blob, float64."""
    lay, total = expert_layout(H, I, G, bits)
    blob = np.asarray(blob, dtype=np.uint8)
    assert blob.size == total, (blob.size, total)

    def part(name):
        a, b = lay[name]
        return blob[a:b]

    qg = unpack_codes(part("q_gate").reshape(I, H * bits // 8), bits)
    qu = unpack_codes(part("q_up").reshape(I, H * bits // 8), bits)
    qd = unpack_codes(part("q_down").reshape(H, I * bits // 8), bits)
    sg = fp16_bits_to_f64(part("s_gate").view(np.uint16).reshape(I, H // G))
    su = fp16_bits_to_f64(part("s_up").view(np.uint16).reshape(I, H // G))
    sd = fp16_bits_to_f64(part("s_down").view(np.uint16).reshape(H, I // G))
    return dequant(qg, sg, G), dequant(qu, su, G), dequant(qd, sd, G)


# ----------------------------------------------------------------------------- rounding


def round_bf16(v: np.ndarray) -> np.ndarray:
    """Round float64 to the nearest bfloat16 (ties to even), returned as float64.

    Direct from float64 (no detour through float32, which could round twice):
    with the binade exponent e of |v| (v = m * 2^e, 0.5 <= m < 1), the bf16
    spacing there is 2^(e-8) (8 significant bits), but never below the smallest
    bf16 subnormal 2^-133. v / spacing is exact, rint rounds half to even.
    Results above the largest finite bf16 become +-inf.
    """
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)
    spacing = np.ldexp(1.0, np.maximum(e - 8, -133))
    r = np.rint(v / spacing) * spacing
    max_bf16 = float(np.ldexp(255.0, 120))  # 0x7F7F = (2 - 2^-7) * 2^127
    return np.where(np.abs(r) > max_bf16, np.copysign(np.inf, v), r)


def round_act(v: np.ndarray, act: str) -> np.ndarray:
    """rho: round to the activation dtype ("bf16" or "f32"), result as float64."""
    if act == "bf16":
        return round_bf16(v)
    if act == "f32":
        return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)
    raise ValueError(act)


# ----------------------------------------------------------------------------- routing


def router_logits(x: np.ndarray, Wr: np.ndarray, b: np.ndarray | None) -> np.ndarray:
    """logits[t, e] = sum_h x[t, h] * Wr[e, h] + b[e], in float64, then rounded to float32.

    The gate that picks each token's experts at run time (page "我在 32GB 单卡上跑两万四千
    专家的 MoE…", section "一、第一个坑:MoE 省算力,不省内存"). The bias takes part in
    both selection and weights (plain reading; the pages give no bias).
    """
    x = np.asarray(x, dtype=np.float64)
    Wr = np.asarray(Wr, dtype=np.float64)
    lg = x @ Wr.T
    if b is not None:
        lg = lg + np.asarray(b, dtype=np.float64)[None, :]
    return lg.astype(np.float32)


def topk_ids(logits_row: np.ndarray, k: int) -> np.ndarray:
    """The k experts of one token: experts ordered by (logit descending, id ascending),
    first k taken; slot j holds the j-th of that order.

    "6 of 384" routed experts per token (page "763B MoE 塞进两张 96GB 显卡…", section
    "显存缺口从哪里来"). Ties go to the lower expert id; -0.0 equals +0.0.
    """
    l = np.asarray(logits_row, dtype=np.float64)
    assert not np.isnan(l).any(), "router logits must be finite"
    ids = np.arange(l.size)
    order = np.lexsort((ids, -l))  # primary key -l, then id
    return order[:k].astype(np.int32)


def gate_weights(sel_logits: np.ndarray) -> np.ndarray:
    """Softmax over the selected k logits (float64): w_j = exp(l_j - m) / sum exp(l_j' - m),
    m = max of the selected. Equals the full softmax renormalised over the selected."""
    l = np.asarray(sel_logits, dtype=np.float64)
    z = np.exp(l - l.max())
    return z / z.sum()


def route(logits: np.ndarray, k: int):
    """ids [T, k] int32 and weights [T, k] float64 for every token."""
    T = logits.shape[0]
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    for t in range(T):
        ids[t] = topk_ids(logits[t], k)
        w[t] = gate_weights(np.asarray(logits[t], dtype=np.float64)[ids[t]])
    return ids, w


def align_permute(ids: np.ndarray, E: int):
    """Token permutation grouped by expert, for assignments a = t*k + j.

    counts[e] = #assignments to e; offsets = exclusive prefix sum (E+1 entries);
    sorted = assignments grouped by expert ascending, ascending a within an expert;
    inv[sorted[p]] = p.
    """
    a = np.asarray(ids, dtype=np.int64).ravel()
    counts = np.bincount(a, minlength=E).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    sorted_ = np.argsort(a, kind="stable").astype(np.int32)
    inv = np.empty_like(sorted_)
    inv[sorted_] = np.arange(sorted_.size, dtype=np.int32)
    return counts, offsets, sorted_, inv


# ----------------------------------------------------------------------------- expert FFN


def silu(g: np.ndarray) -> np.ndarray:
    """silu(g) = g / (1 + exp(-g)) in float64."""
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def expert_ffn(x_t: np.ndarray, Wg: np.ndarray, Wu: np.ndarray, Wd: np.ndarray, act: str) -> np.ndarray:
    """o = Wd . rho(silu(Wg x) * (Wu x)), float64; rho rounds h to the activation dtype."""
    x_t = np.asarray(x_t, dtype=np.float64)
    g = Wg @ x_t
    u = Wu @ x_t
    h = round_act(silu(g) * u, act)
    return Wd @ h


class ExpertStore:
    """Dequantised experts of one layer, decoded on first use (float64)."""

    def __init__(self, blobs: np.ndarray, H: int, I: int, G: int, bits: int = 4):
        self.blobs, self.H, self.I, self.G, self.bits = blobs, H, I, G, bits
        self._cache = {}

    def get(self, e: int):
        if e not in self._cache:
            self._cache[e] = expert_weights(self.blobs[e], self.H, self.I, self.G, self.bits)
        return self._cache[e]

    def drop(self, e: int):
        self._cache.pop(e, None)


def layer_forward(x: np.ndarray, Wr: np.ndarray | None, b: np.ndarray | None, blobs: np.ndarray,
                  H: int, I: int, E: int, k: int, G: int, act: str,
                  logits_in: np.ndarray | None = None, tokens=None, bits: int = 4):
    """One routed MoE FFN layer, plain definition, float64.

    x: [T, H] float64 values of the activations (already in the activation dtype).
    logits_in: if given ([T, E] float32), routing uses these logits instead of the router.
    tokens: optional subset of token indices whose y rows are evaluated (routing is for all).
    bits: bits per weight code of the blobs (4, 3 or 2; see unpack_codes).

    Returns a dict with logits (float32), ids, w, counts, offsets, sorted, inv and y
    ([len(tokens), H] float64). Each FFN_e(x_t) is evaluated on its own; experts are
    decoded once each and freed after their last use, which changes no value.
    """
    x = np.asarray(x, dtype=np.float64)
    T = x.shape[0]
    logits = router_logits(x, Wr, b) if logits_in is None else np.asarray(logits_in, dtype=np.float32)
    assert logits.shape == (T, E)
    ids, w = route(logits, k)
    counts, offsets, sorted_, inv = align_permute(ids, E)
    toks = list(range(T)) if tokens is None else list(tokens)
    # o[(t, j)] for each evaluated assignment, then y_t summed in slot order j = 0..k-1
    need = {}
    for t in toks:
        for j in range(k):
            need.setdefault(int(ids[t, j]), []).append((t, j))
    store = ExpertStore(blobs, H, I, G, bits)
    o = {}
    for e in sorted(need):
        Wg, Wu, Wd = store.get(e)
        for (t, j) in need[e]:
            o[(t, j)] = expert_ffn(x[t], Wg, Wu, Wd, act)
        store.drop(e)
    y = np.zeros((len(toks), H), dtype=np.float64)
    for r, t in enumerate(toks):
        acc = np.zeros(H, dtype=np.float64)
        for j in range(k):
            acc = acc + w[t, j] * o[(t, j)]
        y[r] = acc
    return dict(logits=logits, ids=ids, w=w, counts=counts, offsets=offsets, sorted=sorted_, inv=inv, y=y)


# ----------------------------------------------------------------------------- residency / cache


def link_accounting(ids: np.ndarray, resident: np.ndarray, expert_bytes_: int):
    """Integer recount of one forward under a residency plan (resident[e] = 1 for HBM):
    hits / misses per assignment, and expert bytes per link over the unique experts touched
    (an offloaded expert crosses the host link, page "763B MoE …", section "显存缺口从哪里来")."""
    a = np.asarray(ids).ravel()
    res = np.asarray(resident).astype(bool)
    hits = int(res[a].sum())
    misses = int(a.size - hits)
    uniq = np.unique(a)
    bytes_hbm = int(res[uniq].sum()) * expert_bytes_
    bytes_host = int((~res[uniq]).sum()) * expert_bytes_
    return dict(hits=hits, misses=misses, bytes_hbm=bytes_hbm, bytes_host=bytes_host)


def cache_policy_step(score: np.ndarray, counts: np.ndarray, slot_of: np.ndarray, n_slots: int,
                      decay: float, max_promotions: int):
    """One expert-cache update (page "我在 32GB 单卡上跑两万四千专家的 MoE…", section
    "二、跑起来靠的是分层,不是激活": free VRAM holds the most used experts and the cache
    adapts with use; the pages give no policy, so this is the plain frequency reading).

    score_e <- decay * score_e + counts_e (float64, in that order).
    Desired set: the first n_slots experts in the order (score desc, resident first, id asc).
    Promotions: desired non-residents, in order (score desc, id asc). Each takes, while
    any is left, the lowest empty slot; then the slot of the next victim, victims being
    the residents outside the desired set in order (score asc, id desc). At most
    max_promotions promotions per update.

    slot_of[e] is the HBM slot of expert e, -1 when it is read from host memory.
    Returns (new_score, new_slot_of, [(expert, slot) promoted], [evicted experts]).
    """
    score = decay * np.asarray(score, dtype=np.float64) + np.asarray(counts, dtype=np.float64)
    slot_of = np.asarray(slot_of, dtype=np.int64).copy()
    E = score.size
    resident = slot_of >= 0
    order = sorted(range(E), key=lambda e: (-score[e], 0 if resident[e] else 1, e))
    desired = set(order[:n_slots])
    promos = sorted([e for e in desired if not resident[e]], key=lambda e: (-score[e], e))
    victims = sorted([e for e in range(E) if resident[e] and e not in desired], key=lambda e: (score[e], -e))
    free = sorted(set(range(n_slots)) - set(int(v) for v in slot_of[resident]))
    done, evicted = [], []
    for p in promos[:max(0, max_promotions)]:
        if free:
            s = free.pop(0)
        elif victims:
            v = victims.pop(0)
            s = int(slot_of[v])
            slot_of[v] = -1
            evicted.append(v)
        else:
            break
        slot_of[p] = s
        done.append((p, s))
    return score, slot_of, done, evicted


def cache_set_resident(score: np.ndarray, counts: np.ndarray, slot_of: np.ndarray, want: np.ndarray, n_slots: int,
                       decay: float):
    """An expert-cache update to a residency set the caller chose: the per-expert plan
    of page "763B MoE 塞进两张 96GB 显卡…", section "同一个思路，vLLM 原生方案反而跑不通",
    where residency is decided expert by expert, applied to the cache slots of page
    "我在 32GB 单卡上跑两万四千专家的 MoE…", section "二、跑起来靠的是分层,不是激活".

    score_e <- decay * score_e + counts_e, as in cache_policy_step. Every resident not in
    `want` is evicted (its slot freed); then every wanted non-resident, in ascending id,
    takes the lowest free slot. At most n_slots experts may be wanted.
    Returns (new_score, new_slot_of, [(expert, slot) promoted], [evicted experts]).
    """
    want = np.asarray(want).astype(bool)
    assert want.sum() <= n_slots, "more experts wanted than slots"
    score = decay * np.asarray(score, dtype=np.float64) + np.asarray(counts, dtype=np.float64)
    slot_of = np.asarray(slot_of, dtype=np.int64).copy()
    evicted = [e for e in range(slot_of.size) if slot_of[e] >= 0 and not want[e]]
    for e in evicted:
        slot_of[e] = -1
    free = sorted(set(range(n_slots)) - set(int(v) for v in slot_of[slot_of >= 0]))
    promoted = []
    for e in range(slot_of.size):
        if want[e] and slot_of[e] < 0:
            s = free.pop(0)
            slot_of[e] = s
            promoted.append((e, s))
    return score, slot_of, promoted, evicted


def prefetch_step(logits: np.ndarray, candidates: int, n_slots: int, host_read: np.ndarray,
                  slot_expert: np.ndarray, slot_valid: np.ndarray):
    """One predictive prefetch of a layer (page "我在 32GB 单卡上跑两万四千专家的 MoE…",
    section "二、跑起来靠的是分层,不是激活": the next layer's experts stream into VRAM
    while the current layer is computed). The page does not say how the experts are
    chosen; the reading taken: the layer's router logits of the activations at hand.

    logits [T, E] float32; host_read[e] = the expert's weights are read from host memory
    when no prefetch holds it; slot_expert [n_slots] = the expert each prefetch slot holds
    (-1 none); slot_valid[i] = slot i still serves its expert (no cache update has since
    pointed that expert elsewhere).
    Candidates: each token's `candidates` best experts (logit descending, id ascending),
    token by token. Predicted: the first n_slots distinct candidates that are host_read or
    held by a valid slot. A valid slot whose expert is predicted keeps it; every other
    slot is freed; each predicted expert not kept takes the lowest free slot, in
    prediction order, and is copied.
    Returns (predicted list, new slot_expert [n_slots], [(slot, expert) copied]).
    """
    logits = np.asarray(logits, dtype=np.float32)
    held = {int(slot_expert[i]): i for i in range(n_slots) if slot_expert[i] >= 0 and slot_valid[i]}
    predicted = []
    for t in range(logits.shape[0]):
        for e in topk_ids(logits[t], candidates):
            e = int(e)
            if len(predicted) < n_slots and e not in predicted and (host_read[e] or e in held):
                predicted.append(e)
    new = np.full(n_slots, -1, dtype=np.int64)
    for e, i in held.items():
        if e in predicted:
            new[i] = e
    copied = []
    for e in predicted:
        if e in held:
            continue
        i = int(np.flatnonzero(new < 0)[0])
        new[i] = e
        copied.append((i, e))
    return predicted, new, copied


def residual_next(x: np.ndarray, y: np.ndarray, act: str) -> np.ndarray:
    """The residual stream's next value after a MoE FFN layer: act(x + y), the sum formed
    in float32 (x in the activation dtype, y the layer's float32 output) and then
    rounded to the activation dtype (nearest, ties to even). The pages place the expert
    FFN inside transformer layers whose outputs add to the residual stream; they do not
    fix the precision of the add, and this is the plain reading for a float32 y.
    Returns float64 values."""
    s = np.asarray(x, dtype=np.float64).astype(np.float32) + np.asarray(y, dtype=np.float32)
    return round_act(s.astype(np.float64), act)
