"""Seeded synthetic inputs for the routed MoE FFN layer.

Shared by the oracle's tests, the GPU parity tests and the benchmark. This
package generates inputs only: it holds none of the layer's arithmetic. The
heavy lifting (normals, the fixture quantiser, canonical int4 packing) is in
``gen.c``, built with gcc into ``libmoesynth.so`` next to it.

Workloads (sizes, distributions and seeds) are described by ``WORKLOADS``.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB = os.path.join(_HERE, "libmoesynth.so")
_lib = None

# stream kinds of synth_key(base, kind, a, b, c)
KIND_X, KIND_EXPERT, KIND_ROUTER, KIND_RANK, KIND_RESID = 0, 1, 2, 3, 4


def build() -> str:
    """Compile gen.c into libmoesynth.so (gcc, OpenMP)."""
    tmp = _LIB + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    u64, i64, i32, f32, vp = (ctypes.c_uint64, ctypes.c_int64, ctypes.c_int, ctypes.c_float,
                              ctypes.c_void_p)
    lib.synth_key.restype = u64
    lib.synth_key.argtypes = [u64, u64, u64, u64, u64]
    lib.synth_u64.restype = u64
    lib.synth_u64.argtypes = [u64, u64]
    lib.synth_normal_f32.argtypes = [u64, i64, i64, f32, f32, vp]
    lib.synth_normal_bf16.argtypes = [u64, i64, i64, f32, f32, vp]
    lib.synth_f32_to_f16.restype = ctypes.c_uint16
    lib.synth_f32_to_f16.argtypes = [f32]
    lib.synth_f16_to_f32.restype = f32
    lib.synth_f16_to_f32.argtypes = [ctypes.c_uint16]
    lib.synth_quantize_row.argtypes = [vp, i32, i32, vp, vp]
    lib.synth_pack_int4.argtypes = [vp, i64, vp]
    lib.synth_expert_bytes.restype = i64
    lib.synth_expert_bytes.argtypes = [i32, i32, i32]
    lib.synth_experts.argtypes = [u64, i32, i32, i32, i32, i32, i32, f32, vp]
    lib.synth_expert_bytes_b.restype = i64
    lib.synth_expert_bytes_b.argtypes = [i32, i32, i32, i32]
    lib.synth_quantize_row_odd.argtypes = [vp, i32, i32, i32, vp, vp]
    lib.synth_pack_bits.argtypes = [vp, i64, i32, vp]
    lib.synth_experts_b.argtypes = [u64, i32, i32, i32, i32, i32, i32, f32, i32, vp]
    lib.synth_cut_codes.argtypes = [vp, i64, i32, i32, i32, i32, vp]
    lib.synth_expert_tensor_f32.argtypes = [u64, i32, i32, i32, i32, i32, f32, vp]
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def key(base: int, kind: int, a: int = 0, b: int = 0, c: int = 0) -> int:
    return int(_load().synth_key(base, kind, a, b, c))


def u64(k: int, n: int) -> np.ndarray:
    lib = _load()
    return np.array([lib.synth_u64(k, i) for i in range(n)], dtype=np.uint64)


def normal_f32(k: int, n: int, mean: float = 0.0, std: float = 1.0, first: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    _load().synth_normal_f32(k, first, n, mean, std, _ptr(out))
    return out


def normal_bf16_bits(k: int, n: int, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    """bf16 bit patterns (uint16) of round-to-nearest-even(mean + std * N)."""
    out = np.empty(n, dtype=np.uint16)
    _load().synth_normal_bf16(k, 0, n, mean, std, _ptr(out))
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def f32_to_f16_bits(v: float) -> int:
    return int(_load().synth_f32_to_f16(v))


def quantize_rows(w: np.ndarray, G: int):
    """Fixture quantiser on rows of w (float32 [R, K]) -> (codes int8 [R, K], fp16 bits [R, K/G])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    R, K = w.shape
    q = np.empty((R, K), dtype=np.int8)
    s = np.empty((R, K // G), dtype=np.uint16)
    lib = _load()
    for r in range(R):
        lib.synth_quantize_row(w[r].ctypes.data, K, G, q[r].ctypes.data, s[r].ctypes.data)
    return q, s


def pack_int4(q: np.ndarray) -> np.ndarray:
    """Canonical packing of int4 codes (int8 in [-8, 7]) along the last axis."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    out = np.empty(q.shape[:-1] + (q.shape[-1] // 2,), dtype=np.uint8)
    _load().synth_pack_int4(_ptr(q), q.size, _ptr(out))
    return out


def expert_bytes(H: int, I: int, G: int, bits: int = 4) -> int:
    if bits == 4:
        return int(_load().synth_expert_bytes(H, I, G))
    return int(_load().synth_expert_bytes_b(H, I, G, bits))


def expert_blobs(base: int, layer: int, e0: int, n: int, H: int, I: int, G: int,
                 std: float = 0.02, bits: int = 4) -> np.ndarray:
    """Canonical blobs of experts [e0, e0+n) of a layer, uint8 [n, expert_bytes]. bits = 3, 2:
    the same seeded weights quantised onto odd levels (synth_quantize_row_odd)."""
    out = np.empty((n, expert_bytes(H, I, G, bits)), dtype=np.uint8)
    if bits == 4:
        _load().synth_experts(base, layer, e0, n, H, I, G, std, _ptr(out))
    else:
        _load().synth_experts_b(base, layer, e0, n, H, I, G, std, bits, _ptr(out))
    return out


def cut_codes(blobs4: np.ndarray, H: int, I: int, G: int, bits: int) -> np.ndarray:
    """b-bit blobs from 4-bit blobs of the same shape (top b bits of each offset code, scales
    copied): seeded synthetic lower-bit experts for throughput runs, without regenerating."""
    blobs4 = np.ascontiguousarray(blobs4, dtype=np.uint8)
    out = np.empty((blobs4.shape[0], expert_bytes(H, I, G, bits)), dtype=np.uint8)
    _load().synth_cut_codes(_ptr(blobs4), blobs4.shape[0], H, I, G, bits, _ptr(out))
    return out


def quantize_rows_odd(w: np.ndarray, G: int, bits: int):
    """Odd-level fixture quantiser on rows of w (float32 [R, K]) -> (codes n uint8 [R, K],
    fp16 bits [R, K/G]); the weight code is q = 2n - (2^bits - 1)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    R, K = w.shape
    n = np.empty((R, K), dtype=np.uint8)
    s = np.empty((R, K // G), dtype=np.uint16)
    lib = _load()
    for r in range(R):
        lib.synth_quantize_row_odd(w[r].ctypes.data, K, G, bits, n[r].ctypes.data, s[r].ctypes.data)
    return n, s


def pack_codes(n: np.ndarray, bits: int) -> np.ndarray:
    """Canonical packing of unsigned b-bit codes n along the last axis (little-endian bit string)."""
    n = np.ascontiguousarray(n, dtype=np.uint8)
    K = n.shape[-1]
    rows = n.reshape(-1, K)
    out = np.empty((rows.shape[0], K * bits // 8), dtype=np.uint8)
    lib = _load()
    for r in range(rows.shape[0]):
        lib.synth_pack_bits(rows[r].ctypes.data, K, bits, out[r].ctypes.data)
    return out.reshape(n.shape[:-1] + (K * bits // 8,))


def expert_tensor_f32(base: int, layer: int, expert: int, tensor: int, rows: int, K: int,
                      std: float = 0.02) -> np.ndarray:
    """The unquantised fp32 weights behind tensor (0 gate, 1 up, 2 down) of one expert."""
    out = np.empty((rows, K), dtype=np.float32)
    _load().synth_expert_tensor_f32(base, layer, expert, tensor, rows, K, std, _ptr(out))
    return out


def pack_blob(q_gate, q_up, q_down, s_gate, s_up, s_down, bits: int = 4) -> np.ndarray:
    """Assemble one canonical blob from codes and fp16 scale bits (uint16): bits = 4 takes
    signed codes q (int8, -8..7); bits = 3, 2 take unsigned codes n (0 .. 2^bits - 1)."""
    pk = pack_int4 if bits == 4 else (lambda n: pack_codes(n, bits))
    parts = [pk(q_gate).ravel(), pk(q_up).ravel(), pk(q_down).ravel(),
             np.ascontiguousarray(s_gate, dtype=np.uint16).view(np.uint8).ravel(),
             np.ascontiguousarray(s_up, dtype=np.uint16).view(np.uint8).ravel(),
             np.ascontiguousarray(s_down, dtype=np.uint16).view(np.uint8).ravel()]
    return np.concatenate(parts)


# ---------------------------------------------------------------- activations / router


def activations(base: int, stream: int, T: int, H: int, act: str, sub: int = 0):
    """x [T, H] ~ N(0, 1): 'f32' -> float32 array; 'bf16' -> uint16 bf16 bit patterns."""
    k = key(base, KIND_X, stream, sub)
    if act == "f32":
        return normal_f32(k, T * H).reshape(T, H)
    return normal_bf16_bits(k, T * H).reshape(T, H)


def router_weight(base: int, layer: int, E: int, H: int, act: str, std: float = 0.02):
    """Wr [E, H] ~ N(0, std), in the activation dtype (float32 array or bf16 bits)."""
    k = key(base, KIND_ROUTER, layer)
    if act == "f32":
        return normal_f32(k, E * H, 0.0, std).reshape(E, H)
    return normal_bf16_bits(k, E * H, 0.0, std).reshape(E, H)


def zipf_ranks(base: int, layer: int, E: int) -> np.ndarray:
    """rank_e = 1 + pi(e), pi a seeded permutation of the experts of one layer."""
    k = key(base, KIND_RANK, layer)
    draws = u64(k, E)
    order = np.argsort(draws, kind="stable")  # order[r] = expert holding rank r+1
    ranks = np.empty(E, dtype=np.int64)
    ranks[order] = np.arange(1, E + 1)
    return ranks


def router_bias(base: int, layer: int, E: int, alpha: float) -> np.ndarray:
    """b_e = -alpha * ln(rank_e) as float32 (alpha = 0 gives zeros)."""
    if alpha == 0.0:
        return np.zeros(E, dtype=np.float32)
    return (-alpha * np.log(zipf_ranks(base, layer, E).astype(np.float64))).astype(np.float32)


def coldest_host_plan(base: int, layer: int, E: int, hbm_fraction: float) -> np.ndarray:
    """Residency by a-priori Zipf rank: the round(hbm_fraction*E) lowest ranks in HBM (1), rest host (0)."""
    n_hbm = int(round(hbm_fraction * E))
    ranks = zipf_ranks(base, layer, E)
    return (ranks <= n_hbm).astype(np.int32)


# ---------------------------------------------------------------- workloads


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    H: int
    I: int
    E: int
    k: int
    G: int
    act: str          # "f32" or "bf16"
    alpha: float      # Zipf bias exponent
    seed: int
    batches: tuple    # token counts T exercised
    layers: int = 1


WORKLOADS = {
    "tiny": Workload("tiny H256 I128 E8 k2 G32 f32", 256, 128, 8, 2, 32, "f32", 0.0, 0, (16,)),
    "qwen3_30b_a3b": Workload("Qwen3-30B-A3B-shaped layer H2048 I768 E128 k8 G128 bf16", 2048, 768, 128, 8,
                              128, "bf16", 0.8, 1, (1, 4)),
    "deepseek_384": Workload("DeepSeek-style layer H7168 I2048 E384 k6 G128 bf16", 7168, 2048, 384, 6, 128,
                             "bf16", 1.0, 2, (1, 4, 16)),
    "cache_48x": Workload("48 stacked Qwen3-30B-A3B-shaped layers, 90 HBM slots/layer", 2048, 768, 128, 8,
                          128, "bf16", 0.8, 3, (1,), 48),
    "prefill": Workload("prefill through the Qwen3-30B-A3B layer shape", 2048, 768, 128, 8, 128, "bf16",
                        0.0, 4, (2048, 1024)),
}
