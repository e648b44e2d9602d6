"""Checks of the seeded input generator (not the layer's arithmetic)."""
import numpy as np

import synth


def test_f16_converter_matches_numpy():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(5000) * s for s in (1e-7, 1e-5, 1e-2, 1, 1e3, 6e4)]).astype(np.float32)
    v = np.concatenate([v, np.float32([65504, 65519.99, 65520, 1e9, 0.0, -0.0, 2 ** -24, 2 ** -25, 3 * 2 ** -26])])
    ours = np.array([synth.f32_to_f16_bits(float(x)) for x in v], np.uint16)
    np.testing.assert_array_equal(ours, v.astype(np.float16).view(np.uint16))


def test_normals_are_standard_and_seeded():
    k = synth.key(1, synth.KIND_X, 0)
    z = synth.normal_f32(k, 400000).astype(np.float64)
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1) < 0.01
    assert abs(((z - z.mean()) ** 4).mean() / z.var() ** 2 - 3) < 0.05
    np.testing.assert_array_equal(z[1000:1010], synth.normal_f32(k, 10, first=1000))
    assert not np.array_equal(z[:10], synth.normal_f32(synth.key(1, synth.KIND_X, 1), 10))


def test_bf16_activation_bits_round_float32():
    k = synth.key(5, synth.KIND_X, 0)
    f = synth.normal_f32(k, 1000)
    b = synth.normal_bf16_bits(k, 1000)
    import torch
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(b, ref)


def test_quantiser_bounds():
    w = synth.expert_tensor_f32(1, 0, 3, 0, 16, 256)
    q, s = synth.quantize_rows(w, 128)
    sf = s.view(np.float16).astype(np.float32)
    assert q.min() >= -7 and q.max() <= 7
    deq = q.astype(np.float32) * np.repeat(sf, 128, axis=1)
    unclamped = np.abs(q) < 7
    step = np.repeat(sf, 128, axis=1)
    assert np.all(np.abs(w - deq)[unclamped] <= step[unclamped] / 2 * (1 + 1e-6))
    z, zs = synth.quantize_rows(np.zeros((2, 128), np.float32), 128)
    assert np.all(z == 0) and np.all(zs == 0)


def test_expert_blob_is_quantised_generator_weights():
    H, I, G = 256, 128, 32
    blob = synth.expert_blobs(0, 0, 5, 1, H, I, G)[0]
    w = synth.expert_tensor_f32(0, 0, 5, 1, I, H)  # up projection of expert 5
    q, s = synth.quantize_rows(w, G)
    off = I * H // 2
    np.testing.assert_array_equal(blob[off:2 * off], synth.pack_int4(q).ravel())
    soff = 3 * H * I // 2 + 2 * I * (H // G)
    np.testing.assert_array_equal(blob[soff:soff + 2 * I * (H // G)].view(np.uint16), s.ravel())


def test_zipf_bias():
    r = synth.zipf_ranks(1, 3, 128)
    assert sorted(r.tolist()) == list(range(1, 129))
    b = synth.router_bias(1, 3, 128, 0.8)
    np.testing.assert_allclose(b, -0.8 * np.log(r), rtol=1e-6)
    assert not np.array_equal(r, synth.zipf_ranks(1, 4, 128))  # per-layer permutation


def test_cut_codes_keeps_top_bits_and_scales():
    """The lower-bit copies the benchmark makes of generated 4-bit layers: every code is the
    top b bits of the 4-bit offset code (q + 8), read back by the oracle's decoders, and
    the fp16 scales are unchanged."""
    from oracle import moe_oracle as O
    H, I, G = 256, 128, 64
    b4 = synth.expert_blobs(5, 0, 0, 2, H, I, G)
    lay4, _ = O.expert_layout(H, I, G, 4)
    for bits in (2, 3):
        bb = synth.cut_codes(b4, H, I, G, bits)
        layb, _ = O.expert_layout(H, I, G, bits)
        assert bb.shape == (2, O.expert_bytes(H, I, G, bits))
        for e in range(2):
            for nm in ("q_gate", "q_up", "q_down"):
                q4 = O.unpack_int4(b4[e, lay4[nm][0]:lay4[nm][1]].reshape(1, -1)).astype(np.int16)
                qb = O.unpack_codes(bb[e, layb[nm][0]:layb[nm][1]].reshape(1, -1), bits).astype(np.int16)
                np.testing.assert_array_equal(qb, 2 * ((q4 + 8) >> (4 - bits)) - ((1 << bits) - 1))
            np.testing.assert_array_equal(bb[e, layb["s_gate"][0]:], b4[e, lay4["s_gate"][0]:])
