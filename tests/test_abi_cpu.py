"""The C-ABI library loads and exports every symbol its header declares; calls
that need no GPU (sizes, validation, status strings) work on the CPU."""
import ctypes
import os
import re

import pytest

import expert_offloaded_ffn_moe_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    names = set()
    inc = os.path.join(ROOT, "include")
    for f in os.listdir(inc):
        if f.endswith(".h"):
            txt = open(os.path.join(inc, f)).read()
            txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
            names |= set(re.findall(r"\b(moe_\w+)\s*\(", txt))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(moe.LIB_PATH):
        pytest.fail("library not built: run __graft_entry__.build()")
    return moe.load_library(with_torch=False)


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n


def test_expert_bytes_and_validation(lib):
    for (H, I, G, want) in [(256, 128, 32, 55296), (2048, 768, 128, 2433024), (7168, 2048, 128, 22708224)]:
        assert moe.expert_bytes(moe.make_config(H, I, 8, 2, G)) == want
    bad = [moe.make_config(250, 128, 8, 2, 32), moe.make_config(256, 128, 8, 9, 32),
           moe.make_config(256, 128, 8, 2, 48), moe.make_config(256, 128, 2000, 2, 32),
           moe.make_config(256, 100, 8, 2, 32), moe.make_config(256, 128, 8, 2, 32, max_tokens=0),
           moe.make_config(256, 128, 8, 2, 32, hbm_slots=9), moe.make_config(256, 128, 8, 2, 32, prefill_stage_slots=9),
           moe.make_config(256, 128, 8, 2, 32, prefill_stage_slots=-1),
           moe.make_config(256, 128, 8, 2, 32, prefetch_slots=9),
           moe.make_config(256, 128, 128, 2, 32, prefetch_slots=65),
           moe.make_config(256, 128, 8, 2, 32, prefetch_slots=-1)]
    for cfg in bad:
        out = ctypes.c_size_t()
        assert lib.moe_expert_bytes(ctypes.byref(cfg), ctypes.byref(out)) == moe.MOE_E_INVALID
        h = ctypes.c_void_p(1)
        assert lib.moe_plan_create(ctypes.byref(cfg), None, None, None, ctypes.byref(h)) == moe.MOE_E_INVALID
        assert h.value is None
        assert len(lib.moe_last_error()) > 0


def test_status_strings_and_null_args(lib):
    assert lib.moe_status_str(0) == b"MOE_OK"
    assert lib.moe_status_str(4) == b"MOE_E_HIP"
    assert lib.moe_layer_forward(None, 0, 1, None, None, None, None, None) == moe.MOE_E_INVALID
    assert lib.moe_cache_update(None, 0, None, None) == moe.MOE_E_INVALID
    assert lib.moe_prefetch(None, 0, 1, None, None, 0, None, None) == moe.MOE_E_INVALID
    assert lib.moe_plan_prefetch_slots(None, 0, None) == moe.MOE_E_INVALID
    lib.moe_plan_destroy(None)


def _header_struct_fields(name):
    txt = open(os.path.join(ROOT, "include", "moe_offload.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    body = re.search(r"typedef struct \{([^}]*)\} %s;" % name, txt).group(1)
    return re.findall(r"(\w[\w\s\*]*?)\s*\*?\s*(\w+)\s*(?:\[[^\]]*\])?\s*;", body)


@pytest.mark.parametrize("cname,pyname", [("moe_layer_weights", "LayerWeights"), ("moe_routing", "Routing"),
                                          ("moe_stats", "Stats"), ("moe_cache_policy", "CachePolicy"),
                                          ("moe_plan_info", "PlanInfo"), ("moe_link_ceilings", "LinkCeilings"),
                                          ("moe_kernel_times", "KernelTimes")])
def test_binding_structs_match_header(cname, pyname):
    """Every struct the binding mirrors has the header's field names, in order, and the
    same size (ctypes lays fields out by the platform C ABI)."""
    fields = [n for _, n in _header_struct_fields(cname)]
    assert [n for n, _ in getattr(moe, pyname)._fields_] == fields, cname
    sizes = {"moe_layer_weights": 24, "moe_routing": 56, "moe_stats": 88, "moe_cache_policy": 24,
             "moe_plan_info": 48, "moe_link_ceilings": 24, "moe_kernel_times": 128}
    assert ctypes.sizeof(getattr(moe, pyname)) == sizes[cname]


def test_debug_fail_alloc_arguments(lib):
    assert lib.moe_debug_fail_alloc(2, 1) == moe.MOE_E_INVALID
    assert lib.moe_debug_fail_alloc(0, -1) == moe.MOE_E_INVALID
    assert lib.moe_debug_fail_alloc(0, 0) == moe.MOE_OK
    assert lib.moe_debug_fail_alloc(1, 0) == moe.MOE_OK


def test_link_ceiling_arguments_validated(lib):
    out = moe.LinkCeilings()
    assert lib.moe_measure_link_ceilings(1 << 10, 1 << 20, 1, None, ctypes.byref(out)) == moe.MOE_E_INVALID
    assert lib.moe_measure_link_ceilings(1 << 20, (1 << 20) + 1, 1, None, ctypes.byref(out)) == moe.MOE_E_INVALID
    assert lib.moe_measure_link_ceilings(1 << 20, 1 << 20, 0, None, ctypes.byref(out)) == moe.MOE_E_INVALID


def test_config_struct_matches_header():
    """The binding's moe_config mirror has the header's fields, in order and as int32."""
    txt = open(os.path.join(ROOT, "include", "moe_offload.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    body = re.search(r"typedef struct \{([^}]*)\} moe_config;", txt).group(1)
    fields = re.findall(r"int32_t\s+(\w+)\s*;", body)
    assert len(fields) == len(re.findall(r";", body)), "every moe_config field is an int32_t"
    assert [n for n, _ in moe.Config._fields_] == fields
    assert all(t is ctypes.c_int32 for _, t in moe.Config._fields_)
