"""Python binding of libmoe_offload.so (the C ABI in include/moe_offload.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels. torch supplies device memory (tensors) and streams. There is no
fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_offload.so")

MOE_OK, MOE_E_INVALID, MOE_E_NOMEM, MOE_E_HOST_NOMEM, MOE_E_HIP, MOE_E_UNSUPPORTED, MOE_E_STATE = range(7)
ACT_F32, ACT_BF16 = 0, 1
HOST_COMPUTE_NONE, HOST_COMPUTE_MISSES, HOST_COMPUTE_LAYER = 0, 1, 2


class Config(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("group_size", ctypes.c_int32), ("num_layers", ctypes.c_int32),
                ("act_dtype", ctypes.c_int32), ("max_tokens", ctypes.c_int32), ("hbm_slots", ctypes.c_int32),
                ("gemm_min_tokens", ctypes.c_int32), ("prefill_stage_slots", ctypes.c_int32),
                ("weight_bits", ctypes.c_int32), ("prefetch_slots", ctypes.c_int32)]


class LayerWeights(ctypes.Structure):
    _fields_ = [("router_w", ctypes.c_void_p), ("router_b", ctypes.c_void_p), ("experts", ctypes.c_void_p)]


class Routing(ctypes.Structure):
    _fields_ = [("logits", ctypes.c_void_p), ("topk_ids", ctypes.c_void_p), ("topk_w", ctypes.c_void_p),
                ("counts", ctypes.c_void_p), ("offsets", ctypes.c_void_p), ("sorted", ctypes.c_void_p),
                ("inv", ctypes.c_void_p)]


class Stats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("forwards", "tokens", "hits", "misses", "bytes_hbm", "bytes_host",
                                              "bytes_copied", "promotions", "evictions", "host_computed",
                                              "prefetched")]

    def as_dict(self):
        return {n: int(getattr(self, n)) for n, _ in self._fields_}


class CachePolicy(ctypes.Structure):
    _fields_ = [("decay", ctypes.c_double), ("max_promotions", ctypes.c_int32), ("overlap", ctypes.c_int32),
                ("want_resident", ctypes.c_void_p)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("device", ctypes.c_int32), ("gpu_numa_node", ctypes.c_int32), ("host_pool_node", ctypes.c_int32),
                ("numa_bound", ctypes.c_int32), ("internal_expert_bytes", ctypes.c_int64),
                ("host_pool_bytes", ctypes.c_int64), ("hbm_slot_bytes", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_int64)]

    def as_dict(self):
        return {n: int(getattr(self, n)) for n, _ in self._fields_}


class LinkCeilings(ctypes.Structure):
    _fields_ = [("hbm_read_gbps", ctypes.c_double), ("host_read_gbps", ctypes.c_double),
                ("h2d_copy_gbps", ctypes.c_double)]


KERNELS = ["router", "route", "gateup", "down", "combine", "gemm_gateup", "gemm_down", "stage"]


class KernelTimes(ctypes.Structure):
    _fields_ = [("launches", ctypes.c_int64 * 8), ("total_ms", ctypes.c_double * 8)]


class MoeError(RuntimeError):
    def __init__(self, status, fn, msg):
        super().__init__("%s failed: %s (%s)" % (fn, _status_name(status), msg))
        self.status = status


_lib = None


def _status_name(s):
    return ["MOE_OK", "MOE_E_INVALID", "MOE_E_NOMEM", "MOE_E_HOST_NOMEM", "MOE_E_HIP", "MOE_E_UNSUPPORTED",
            "MOE_E_STATE"][s] if 0 <= s < 7 else str(s)


def load_library(path: str = LIB_PATH, with_torch: bool = True):
    """Load the library. With torch, torch is imported first so that the library
    binds to the same HIP runtime as torch's tensors and streams."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libmoe_offload.so is not built (%s): run __graft_entry__.build() or "
                           "python expert_offloaded_ffn_moe_amd/build.py" % path)
    if with_torch:
        import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    vp, i32, st = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int
    lib.moe_expert_bytes.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(ctypes.c_size_t)]
    lib.moe_plan_create.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(LayerWeights), vp, vp, ctypes.POINTER(vp)]
    lib.moe_plan_load_layer.argtypes = [vp, i32, ctypes.POINTER(LayerWeights), vp, vp]
    lib.moe_plan_get_info.argtypes = [vp, ctypes.POINTER(PlanInfo)]
    lib.moe_measure_link_ceilings.argtypes = [ctypes.c_size_t, ctypes.c_size_t, i32, vp, ctypes.POINTER(LinkCeilings)]
    lib.moe_debug_fail_alloc.argtypes = [i32, i32]
    lib.moe_plan_set_host_compute.argtypes = [vp, i32, i32, i32]
    lib.moe_prefetch.argtypes = [vp, i32, i32, vp, vp, i32, vp, vp]
    lib.moe_plan_prefetch_slots.argtypes = [vp, i32, vp]
    lib.moe_debug_live_allocs.argtypes = [ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]
    lib.moe_layer_forward.argtypes = [vp, i32, i32, vp, vp, vp, ctypes.POINTER(Routing), vp]
    lib.moe_layer_forward_noalloc.argtypes = [vp, i32, i32, vp, vp, vp, ctypes.POINTER(Routing), vp]
    lib.moe_layer_forward_residual.argtypes = [vp, i32, i32, vp, vp, vp, vp, ctypes.POINTER(Routing), vp]
    lib.moe_cache_update.argtypes = [vp, i32, ctypes.POINTER(CachePolicy), vp]
    lib.moe_plan_stats.argtypes = [vp, i32, ctypes.POINTER(Stats)]
    lib.moe_plan_reset_stats.argtypes = [vp]
    lib.moe_plan_residency.argtypes = [vp, i32, vp]
    lib.moe_plan_profile.argtypes = [vp, i32]
    lib.moe_plan_kernel_times.argtypes = [vp, ctypes.POINTER(KernelTimes)]
    lib.moe_plan_destroy.argtypes = [vp]
    lib.moe_plan_destroy.restype = None
    lib.moe_status_str.argtypes = [st]
    lib.moe_status_str.restype = ctypes.c_char_p
    lib.moe_last_error.restype = ctypes.c_char_p
    for fn in ("moe_expert_bytes", "moe_plan_create", "moe_plan_load_layer", "moe_layer_forward",
               "moe_layer_forward_noalloc", "moe_layer_forward_residual",
               "moe_cache_update", "moe_plan_stats", "moe_plan_reset_stats", "moe_plan_residency",
               "moe_plan_profile", "moe_plan_kernel_times", "moe_plan_get_info", "moe_measure_link_ceilings",
               "moe_debug_fail_alloc", "moe_debug_live_allocs", "moe_plan_set_host_compute",
               "moe_prefetch", "moe_plan_prefetch_slots"):
        getattr(lib, fn).restype = st
    _lib = lib
    return lib


def _check(status, fn):
    if status != MOE_OK:
        raise MoeError(status, fn, _lib.moe_last_error().decode())


def _ptr(t):
    """Device/host address of a torch tensor or numpy array (None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        assert t.flags["C_CONTIGUOUS"]
        return t.ctypes.data
    assert t.is_contiguous()
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def measure_link_ceilings(hbm_bytes=1 << 30, host_bytes=1 << 30, iters=5, stream=None) -> dict:
    """Streaming-read GB/s over device memory and over pinned device-mapped host memory,
    and host -> device copy GB/s (moe_measure_link_ceilings)."""
    lib = load_library()
    out = LinkCeilings()
    _check(lib.moe_measure_link_ceilings(hbm_bytes, host_bytes, iters, _stream(stream), ctypes.byref(out)),
           "moe_measure_link_ceilings")
    return {n: float(getattr(out, n)) for n, _ in out._fields_}


def debug_fail_alloc(kind: int, n: int):
    """Test hook: the n-th next device (kind 0) or pinned host (kind 1) allocation fails."""
    lib = load_library()
    _check(lib.moe_debug_fail_alloc(kind, n), "moe_debug_fail_alloc")


def debug_live_allocs():
    """(device, pinned host) allocations the library currently holds."""
    lib = load_library()
    d, h = ctypes.c_int64(), ctypes.c_int64()
    _check(lib.moe_debug_live_allocs(ctypes.byref(d), ctypes.byref(h)), "moe_debug_live_allocs")
    return int(d.value), int(h.value)


def make_config(H, I, E, k, G, act="bf16", num_layers=1, max_tokens=16, hbm_slots=None, gemm_min_tokens=0,
                prefill_stage_slots=0, weight_bits=4, prefetch_slots=0):
    return Config(H, I, E, k, G, num_layers, ACT_BF16 if act == "bf16" else ACT_F32, max_tokens,
                  E if hbm_slots is None else hbm_slots, gemm_min_tokens, prefill_stage_slots, weight_bits,
                  prefetch_slots)


def expert_bytes(cfg: Config) -> int:
    lib = load_library()
    out = ctypes.c_size_t()
    _check(lib.moe_expert_bytes(ctypes.byref(cfg), ctypes.byref(out)), "moe_expert_bytes")
    return int(out.value)


def _layer_weights(router_w, router_b, experts):
    """(LayerWeights, the arrays it points into, kept alive by the caller)."""
    rw = np.ascontiguousarray(router_w)
    rb = None if router_b is None else np.ascontiguousarray(router_b, dtype=np.float32)
    ex = np.ascontiguousarray(experts, dtype=np.uint8)
    return LayerWeights(_ptr(rw), _ptr(rb), _ptr(ex)), (rw, rb, ex)


class Plan:
    """A residency plan: pools, pointer tables and workspace of `cfg.num_layers` layers.

    layers: optional list of (router_w, router_b, experts) per layer, loaded at create;
    initial_hbm: optional host [L, E] int (1 = the expert starts in an HBM slot)."""

    def __init__(self, cfg: Config, layers=None, initial_hbm=None, stream=None):
        self.lib = load_library()
        self.cfg = cfg
        h = ctypes.c_void_p()
        arr, keep, ih = None, [], None
        if layers is not None:
            assert len(layers) == cfg.num_layers
            arr = (LayerWeights * len(layers))()
            for i, (rw, rb, ex) in enumerate(layers):
                arr[i], k = _layer_weights(rw, rb, ex)
                keep.append(k)
            if initial_hbm is not None:
                ih = np.ascontiguousarray(initial_hbm, dtype=np.int32)
                assert ih.shape == (cfg.num_layers, cfg.num_experts)
        _check(self.lib.moe_plan_create(ctypes.byref(cfg), arr, _ptr(ih), _stream(stream), ctypes.byref(h)),
               "moe_plan_create")
        self.handle = h

    def load_layer(self, layer, router_w: np.ndarray, router_b, experts: np.ndarray, resident=None, stream=None):
        """router_w: host [E, H] float32 (f32 plans) or uint16 bf16 bits (bf16 plans);
        router_b: host [E] float32 or None; experts: host uint8 [E, expert_bytes];
        resident: host [E] int (1 = the expert starts in an HBM slot) or None."""
        w, keep = _layer_weights(router_w, router_b, experts)
        res = None if resident is None else np.ascontiguousarray(resident, dtype=np.int32)
        _check(self.lib.moe_plan_load_layer(self.handle, layer, ctypes.byref(w), _ptr(res), _stream(stream)),
               "moe_plan_load_layer")
        del keep

    def forward(self, layer, x, y, logits_in=None, route=None, stream=None):
        """x: cuda tensor [T, H] (float32 or bfloat16); y: cuda float32 [T, H];
        route: optional dict of cuda tensors named like the moe_routing fields."""
        T = int(x.shape[0])
        r = None
        if route is not None:
            r = Routing(*[_ptr(route.get(n)) for n, _ in Routing._fields_])
        _check(self.lib.moe_layer_forward(self.handle, layer, T, _ptr(x), _ptr(logits_in), _ptr(y),
                                          ctypes.byref(r) if r is not None else None, _stream(stream)),
               "moe_layer_forward")
        return y

    def forward_residual(self, layer, x, y, x_out, logits_in=None, route=None, stream=None):
        """forward() that also writes x_out = x + y in x's dtype (the residual stream's
        next value), from the kernel that writes y."""
        T = int(x.shape[0])
        r = None
        if route is not None:
            r = Routing(*[_ptr(route.get(n)) for n, _ in Routing._fields_])
        _check(self.lib.moe_layer_forward_residual(self.handle, layer, T, _ptr(x), _ptr(logits_in), _ptr(y),
                                                   _ptr(x_out), ctypes.byref(r) if r is not None else None,
                                                   _stream(stream)), "moe_layer_forward_residual")
        return y

    def forward_noalloc(self, layer, x, y, logits_in=None, route=None, stream=None):
        """forward() through moe_layer_forward_noalloc: the workspace comes from the
        library's static per-device array, and the call allocates nothing."""
        T = int(x.shape[0])
        r = None
        if route is not None:
            r = Routing(*[_ptr(route.get(n)) for n, _ in Routing._fields_])
        _check(self.lib.moe_layer_forward_noalloc(self.handle, layer, T, _ptr(x), _ptr(logits_in), _ptr(y),
                                                  ctypes.byref(r) if r is not None else None, _stream(stream)),
               "moe_layer_forward_noalloc")
        return y

    def cache_update(self, layer=-1, decay=0.9, max_promotions=8, overlap=False, want_resident=None, stream=None):
        """overlap=True: the pipelined update (decisions lag one update; copies on the
        plan's copy stream, promoted experts switched to HBM by the next update).
        want_resident: host [E] (one layer) or [L, E] (layer = -1) ints, the residency
        set to move to instead of the frequency policy's choice."""
        want = None if want_resident is None else np.ascontiguousarray(want_resident, dtype=np.int32)
        pol = CachePolicy(decay, max_promotions, 1 if overlap else 0, _ptr(want))
        _check(self.lib.moe_cache_update(self.handle, layer, ctypes.byref(pol), _stream(stream)),
               "moe_cache_update")

    def prefetch(self, layer, x=None, logits_in=None, candidates=0, predicted_out=None, stream=None):
        """Predict the layer's experts from x (cuda [T, H], the layer's router applied to
        it) or logits_in (cuda float32 [T, E]) and copy the host-read ones among them
        into the layer's prefetch slots, on the plan's prefetch stream, after the work
        enqueued on `stream` so far. predicted_out: optional cuda int32 [prefetch_slots]."""
        src = logits_in if logits_in is not None else x
        T = int(src.shape[0])
        _check(self.lib.moe_prefetch(self.handle, layer, T, _ptr(x), _ptr(logits_in), candidates,
                                     _ptr(predicted_out), _stream(stream)), "moe_prefetch")

    def prefetch_slots(self, layer) -> np.ndarray:
        """Expert held by each prefetch slot of the layer (-1 none); waits for its prefetch."""
        out = np.empty(self.cfg.prefetch_slots, dtype=np.int32)
        _check(self.lib.moe_plan_prefetch_slots(self.handle, layer, out.ctypes.data), "moe_plan_prefetch_slots")
        return out

    def set_host_compute(self, layer=-1, mode=HOST_COMPUTE_MISSES, threads=0):
        """Where the layer's experts are computed: HOST_COMPUTE_NONE (the GPU, offloaded ones
        read over the host link), HOST_COMPUTE_MISSES (the host cores compute the offloaded
        ones), HOST_COMPUTE_LAYER (the host cores compute all of them)."""
        _check(self.lib.moe_plan_set_host_compute(self.handle, layer, mode, threads), "moe_plan_set_host_compute")

    def info(self) -> dict:
        out = PlanInfo()
        _check(self.lib.moe_plan_get_info(self.handle, ctypes.byref(out)), "moe_plan_get_info")
        return out.as_dict()

    def stats(self, layer=-1) -> dict:
        s = Stats()
        _check(self.lib.moe_plan_stats(self.handle, layer, ctypes.byref(s)), "moe_plan_stats")
        return s.as_dict()

    def reset_stats(self):
        _check(self.lib.moe_plan_reset_stats(self.handle), "moe_plan_reset_stats")

    def residency(self, layer) -> np.ndarray:
        out = np.empty(self.cfg.num_experts, dtype=np.int32)
        _check(self.lib.moe_plan_residency(self.handle, layer, out.ctypes.data), "moe_plan_residency")
        return out

    def profile(self, enable: bool):
        _check(self.lib.moe_plan_profile(self.handle, 1 if enable else 0), "moe_plan_profile")

    def kernel_times(self) -> dict:
        """{kernel class: (launches, total ms)} of the recorded launches."""
        kt = KernelTimes()
        _check(self.lib.moe_plan_kernel_times(self.handle, ctypes.byref(kt)), "moe_plan_kernel_times")
        return {n: (int(kt.launches[i]), float(kt.total_ms[i])) for i, n in enumerate(KERNELS)}

    def destroy(self):
        if self.handle:
            self.lib.moe_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass
