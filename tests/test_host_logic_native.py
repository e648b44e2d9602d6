"""The library's host-side logic (host_logic.cpp: configuration checks, the internal
expert layout and repack, the expert-cache policies) built on its own with g++ under
AddressSanitizer and UndefinedBehaviorSanitizer, driven through a pipe
(tests/native/host_logic_check.cpp) and compared with the oracle and with an
independent decoder of the internal layout written here from its documentation
(host_logic.h). Any sanitizer report, or a leak at exit, fails the module."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import synth
from oracle import moe_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "expert_offloaded_ffn_moe_amd", "csrc")


class Driver:
    def __init__(self, exe):
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=97",
                   UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=98")
        env.pop("LD_PRELOAD", None)
        self.p = subprocess.Popen([exe], stdin=subprocess.PIPE, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                  text=True, env=env)

    def ask(self, lines, n_out):
        for ln in lines:
            self.p.stdin.write(ln + "\n")
        self.p.stdin.flush()
        out = [self.p.stdout.readline().rstrip("\n") for _ in range(n_out)]
        assert self.p.poll() is None, "driver exited: %s" % self.p.stderr.read()
        return out

    def close(self):
        self.p.stdin.close()
        rc = self.p.wait(timeout=60)
        return rc, self.p.stderr.read()


@pytest.fixture(scope="module")
def drv(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.fail("g++ is required")
    exe = str(tmp_path_factory.mktemp("hl") / "host_logic_check")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-mavx512f", "-mavx512bw", "-mavx512vl", "-mf16c", "-mfma", "-pthread",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, os.path.join(CSRC, "host_logic.cpp"),
           os.path.join(CSRC, "host_ffn.cpp"), os.path.join(ROOT, "tests", "native", "host_logic_check.cpp"),
           "-o", exe]
    subprocess.check_call(cmd)
    d = Driver(exe)
    yield d
    rc, err = d.close()
    assert rc == 0 and "ERROR" not in err and "runtime error" not in err, err


SHAPES = [(256, 128, 32, 4), (384, 96, 32, 4), (512, 256, 64, 4), (256, 256, 256, 4), (2048, 768, 128, 4),
          (256, 128, 64, 2), (512, 256, 128, 2), (256, 128, 64, 3), (384, 192, 64, 3), (2048, 768, 128, 3)]


def layout_expected(H, I, G, B):
    """The documented rule: 16-byte lane words of kc = 32 (4-bit) or 64 (2-, 3-bit) values,
    regions in order (gate/up codes, gate/up high planes, gate/up scales, the same for
    down), each 256-byte aligned; high planes (512 bytes per block) only for 3-bit codes."""
    up = lambda v: (v + 255) // 256 * 256
    kc = 32 if B == 4 else 64
    hib = 512 if B == 3 else 0
    gu_t, gu_c, gu_g, dn_t, dn_c, dn_g = I // 32, H // kc, H // G, H // 64, I // kc, I // G
    o_guc = 0
    o_guh = up(o_guc + gu_t * gu_c * 1024)
    o_gus = up(o_guh + gu_t * gu_c * hib)
    o_dnc = up(o_gus + gu_t * gu_g * 128)
    o_dnh = up(o_dnc + dn_t * dn_c * 1024)
    o_dns = up(o_dnh + dn_t * dn_c * hib)
    end = up(o_dns + dn_t * dn_g * 128)
    return [kc, gu_t, gu_c, gu_g, dn_t, dn_c, dn_g, o_guc, o_guh, o_gus, o_dnc, o_dnh, o_dns, end,
            3 * H * I * B // 8 + 6 * H * I // G]


@pytest.mark.parametrize("H,I,G,B", SHAPES)
def test_layout(drv, H, I, G, B):
    got = [int(v) for v in drv.ask(["layout %d %d %d %d" % (H, I, G, B)], 1)[0].split()]
    assert got == layout_expected(H, I, G, B)


def decode_codes(region, tiles, chunks, B=4, hi_region=None):
    """[tiles, 64 lanes, chunks * kc] int codes q of a code region (and, for 3-bit codes,
    its high-plane region). 4-bit: dword d of a lane's 16 bytes covers K offsets
    8d..8d+7, offset 8d+2j in bits 4j..4j+3 and 8d+2j+1 in bits 16+4j..19+4j, stored as
    n = q + 8. 2-, 3-bit: dword d covers offsets 16d..16d+15, the low two bits of the
    code at 16d+2j in bits 2j..2j+1 and of 16d+2j+1 in bits 16+2j..17+2j; high-plane
    dword e covers offsets 32e..32e+31, bit 2 of the code at 32e+2i in bit i and of
    32e+2i+1 in bit 16+i; q = 2n - (2^B - 1)."""
    u = np.frombuffer(region.tobytes(), dtype="<u4").reshape(tiles, chunks, 64, 4)
    if B == 4:
        q = np.empty((tiles, chunks, 64, 32), dtype=np.int16)
        for d in range(4):
            for j in range(4):
                q[..., 8 * d + 2 * j] = ((u[..., d] >> (4 * j)) & 0xF).astype(np.int16) - 8
                q[..., 8 * d + 2 * j + 1] = ((u[..., d] >> (16 + 4 * j)) & 0xF).astype(np.int16) - 8
        return q.transpose(0, 2, 1, 3).reshape(tiles, 64, chunks * 32)
    n = np.zeros((tiles, chunks, 64, 64), dtype=np.int16)
    for d in range(4):
        for j in range(8):
            n[..., 16 * d + 2 * j] = (u[..., d] >> (2 * j)) & 3
            n[..., 16 * d + 2 * j + 1] = (u[..., d] >> (16 + 2 * j)) & 3
    if B == 3:
        h = np.frombuffer(hi_region.tobytes(), dtype="<u4").reshape(tiles, chunks, 64, 2)
        for e in range(2):
            for i in range(16):
                n[..., 32 * e + 2 * i] |= (((h[..., e] >> i) & 1) << 2).astype(np.int16)
                n[..., 32 * e + 2 * i + 1] |= (((h[..., e] >> (16 + i)) & 1) << 2).astype(np.int16)
    q = 2 * n - ((1 << B) - 1)
    return q.transpose(0, 2, 1, 3).reshape(tiles, 64, chunks * 64)


def decode_scales(region, tiles, groups):
    return np.frombuffer(region.tobytes(), dtype="<u2").reshape(tiles, groups, 64).transpose(0, 2, 1)


@pytest.mark.parametrize("H,I,G,B", SHAPES)
def test_repack_against_oracle_unpack(drv, tmp_path, H, I, G, B):
    """Random bytes cover every code value in every position; scales are random fp16 bits."""
    rng = np.random.default_rng(H + I + G + B)
    eb = O.expert_bytes(H, I, G, B)
    blob = rng.integers(0, 256, size=eb, dtype=np.uint8)
    src, dst = tmp_path / "c.bin", tmp_path / "i.bin"
    blob.tofile(src)
    assert drv.ask(["repack %d %d %d %d %s %s" % (H, I, G, B, src, dst)], 1) == ["done"]
    kc, gu_t, gu_c, gu_g, dn_t, dn_c, dn_g, o_guc, o_guh, o_gus, o_dnc, o_dnh, o_dns, end, _ = \
        layout_expected(H, I, G, B)
    internal = np.fromfile(dst, dtype=np.uint8)
    assert internal.size == end
    parts, _ = O.expert_layout(H, I, G, B)
    part = lambda n: blob[parts[n][0]:parts[n][1]]
    qg = O.unpack_codes(part("q_gate").reshape(I, H * B // 8), B)
    qu = O.unpack_codes(part("q_up").reshape(I, H * B // 8), B)
    qd = O.unpack_codes(part("q_down").reshape(H, I * B // 8), B)
    assert len(np.unique(qg)) == 1 << B
    hi = lambda o, t, c: internal[o:o + t * c * 512] if B == 3 else None
    gu = decode_codes(internal[o_guc:o_guc + gu_t * gu_c * 1024], gu_t, gu_c, B, hi(o_guh, gu_t, gu_c))
    np.testing.assert_array_equal(gu[:, :32].reshape(I, H), qg)
    np.testing.assert_array_equal(gu[:, 32:].reshape(I, H), qu)
    dn = decode_codes(internal[o_dnc:o_dnc + dn_t * dn_c * 1024], dn_t, dn_c, B, hi(o_dnh, dn_t, dn_c))
    np.testing.assert_array_equal(dn.reshape(H, I), qd)
    sgu = decode_scales(internal[o_gus:o_gus + gu_t * gu_g * 128], gu_t, gu_g)
    np.testing.assert_array_equal(sgu[:, :32].reshape(I, H // G), part("s_gate").view("<u2").reshape(I, H // G))
    np.testing.assert_array_equal(sgu[:, 32:].reshape(I, H // G), part("s_up").view("<u2").reshape(I, H // G))
    sdn = decode_scales(internal[o_dns:o_dns + dn_t * dn_g * 128], dn_t, dn_g)
    np.testing.assert_array_equal(sdn.reshape(H, I // G), part("s_down").view("<u2").reshape(H, I // G))


def _ints(v):
    return " ".join(str(int(a)) for a in v)


def _floats(v):
    return " ".join(float(a).hex() for a in v)


def _parse(out):
    score = np.array([float.fromhex(t) for t in out[0].split()])
    slot = np.array([int(t) for t in out[1].split()])
    prom = [tuple(int(u) for u in t.split(":")) for t in out[2].split()]
    ev = [int(t) for t in out[3].split()]
    return score, slot, prom, ev


def _random_state(rng, E, S):
    slot = np.full(E, -1)
    res = rng.choice(E, size=int(rng.integers(0, S + 1)), replace=False)
    if S:
        slot[res] = rng.choice(S, size=res.size, replace=False)
    score = rng.random(E) * rng.integers(0, 5, size=E)  # ties at zero and repeated values
    score[rng.random(E) < 0.3] = 1.0
    counts = rng.integers(0, 4, size=E) * (rng.random(E) < 0.6)
    return slot, score, counts


def test_cache_policy_matches_oracle(drv):
    rng = np.random.default_rng(5)
    for it in range(300):
        E = int(rng.integers(1, 70))
        S = int(rng.integers(0, E + 1))
        slot, score, counts = _random_state(rng, E, S)
        decay, maxp = float(rng.choice([0.0, 0.5, 0.9, 1.0])), int(rng.integers(0, 10))
        out = drv.ask(["policy %d %d %s %d" % (E, S, decay.hex(), maxp), _ints(counts), _floats(score),
                       _ints(slot)], 4)
        got = _parse(out)
        want = O.cache_policy_step(score, counts, slot, S, decay, maxp)
        np.testing.assert_array_equal(got[0], want[0])
        np.testing.assert_array_equal(got[1], want[1])
        assert got[2] == [(int(a), int(b)) for a, b in want[2]], it
        assert got[3] == [int(a) for a in want[3]], it


def test_cache_set_resident_matches_oracle(drv):
    rng = np.random.default_rng(6)
    for it in range(300):
        E = int(rng.integers(1, 70))
        S = int(rng.integers(0, E + 1))
        slot, score, counts = _random_state(rng, E, S)
        want = np.zeros(E, np.int32)
        n_want = int(rng.integers(0, E + 1)) if it % 10 == 0 else int(rng.integers(0, S + 1))
        want[rng.choice(E, size=n_want, replace=False)] = 1
        out = drv.ask(["setres %d %d %s" % (E, S, (0.9).hex()), _ints(counts), _floats(score), _ints(slot),
                       _ints(want)], 4)
        if n_want > S:
            assert out[0] == "refused"
            continue
        got = _parse(out)
        ref = O.cache_set_resident(score, counts, slot, want, S, 0.9)
        np.testing.assert_array_equal(got[0], ref[0])
        np.testing.assert_array_equal(got[1], ref[1])
        assert got[2] == [(int(a), int(b)) for a, b in ref[2]]
        assert got[3] == [int(a) for a in ref[3]]


def _valid(H, I, E, k, G, L, act, T, S, gmin, stage, bits):
    """The configuration rules as the header states them."""
    b = 4 if bits == 0 else bits
    low_ok = b == 4 or (act == 1 and G >= 64 and I % 64 == 0)
    return (H > 0 and I > 0 and G in (32, 64, 128, 256) and H % 64 == 0 and I % 32 == 0 and H % G == 0
            and I % G == 0 and 1 <= E <= 1024 and 1 <= k <= min(E, 32) and L >= 1 and act in (0, 1)
            and 1 <= T <= (1 << 20) and T * k <= (1 << 22) and 0 <= S <= E and 0 <= stage <= E
            and H <= 65536 and I <= 65536 and b in (2, 3, 4) and low_ok)


def test_check_config_matches_stated_rules(drv):
    rng = np.random.default_rng(7)
    base = [2048, 768, 128, 8, 128, 1, 1, 16, 90, 0, 0, 0]
    cases = [base]
    alts = {0: [0, -64, 64, 96, 65536, 65600], 1: [0, 32, 48, 96, 65536], 2: [0, 1, 1024, 1025], 3: [0, 1, 32, 33],
            4: [16, 32, 48, 64, 256, 512], 5: [0, 1, 48], 6: [-1, 0, 1, 2], 7: [0, 1, 1 << 20, (1 << 20) + 1],
            8: [-1, 0, 128, 129], 9: [-1, 0, 6], 10: [-1, 0, 128, 129], 11: [-1, 0, 1, 2, 3, 4, 5, 8]}
    for i, vals in alts.items():
        for v in vals:
            c = list(base)
            c[i] = v
            cases.append(c)
    for _ in range(200):
        c = list(base)
        for i in rng.choice(12, size=3, replace=False):
            c[i] = int(rng.choice(alts[int(i)]))
        cases.append(c)
    for c in cases:
        got = drv.ask(["check " + _ints(c)], 1)[0]
        assert (got == "OK") == _valid(*c), (c, got)


def _avx512():
    flags = open("/proc/cpuinfo").read()
    return all(f in flags for f in ("avx512f", "avx512bw", "avx512vl", "f16c"))


@pytest.mark.parametrize("H,I,G,M,threads,act", [(256, 128, 32, 1, 1, "bf16"), (512, 256, 128, 3, 4, "bf16"),
                                                 (1024, 768, 256, 9, 3, "bf16"), (2048, 768, 128, 2, 8, "bf16"),
                                                 (256, 128, 32, 5, 2, "f32"), (1024, 256, 64, 3, 4, "f32")])
def test_host_expert_ffn_against_oracle(drv, tmp_path, H, I, G, M, threads, act):
    """The host expert FFN (AVX-512, several worker threads, 8-token passes) on the library's
    internal layout against the oracle's FFN of the canonical blob: codes covering every
    value, bf16 activations, h rounded to bf16 on both sides; rel-L2 <= 1e-3, max-abs <= 2e-2."""
    if not _avx512():
        pytest.skip("host FFN needs AVX-512")
    import layer_cases as LC
    blob = LC.random_code_blobs(1, H, I, G, seed=H + M)[0]
    rng = np.random.default_rng(M)
    x = rng.standard_normal((M, H)).astype(np.float32)
    if act == "bf16":
        x = O.round_bf16(x.astype(np.float64)).astype(np.float32)
    bp, xp, op = tmp_path / "b.bin", tmp_path / "x.bin", tmp_path / "o.bin"
    blob.tofile(bp)
    x.tofile(xp)
    assert drv.ask(["ffn %d %d %d %d %d %d %s %s %s" % (H, I, G, M, threads, act == "bf16", bp, xp, op)],
                   1) == ["done"]
    o = np.fromfile(op, dtype=np.float32).reshape(M, H).astype(np.float64)
    Wg, Wu, Wd = O.expert_weights(blob, H, I, G)
    ref = np.stack([O.expert_ffn(x[m].astype(np.float64), Wg, Wu, Wd, act) for m in range(M)])
    r, m = LC.rel_l2(o, ref), LC.max_abs(o, ref)
    assert r <= (1e-3 if act == "bf16" else 1e-5) and m <= 2e-2, (r, m)
