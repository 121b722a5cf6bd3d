"""ctypes declarations mirroring include/pkv.h (argument marshalling only)."""

from __future__ import annotations

import ctypes
import os

# The in-tree library; PKV_LIB_PATH names another build of the same sources
# (the CPU sanitizer test loads a host-sanitized one this way).
LIB_PATH = os.environ.get("PKV_LIB_PATH") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpkv.so")

# pkv_status
OK, ERR_INVALID_ARG, ERR_METADATA, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_STALE_PLAN, ERR_HIP = range(7)
STATUS_NAMES = {0: "OK", 1: "INVALID_ARG", 2: "METADATA", 3: "UNSUPPORTED", 4: "WORKSPACE", 5: "STALE_PLAN",
                6: "HIP"}
# pkv_meta_reason
META_REASONS = {
    "batch_size": 1, "page_size": 2, "indptr_start": 3, "indptr_order": 4, "empty_page_list": 5,
    "last_page_len": 6, "page_index": 7, "indices_length": 8, "qo_exceeds_kv": 9, "head_group": 10,
    "decode_qo_len": 11, "append_collision": 12, "cascade_rows": 13, "cascade_nesting": 14,
}
F32, BF16, FP8_E4M3 = 0, 1, 2
NHD, HND = 0, 1
DECODE, PREFILL, MLA_DECODE = 0, 1, 2
KV_PAGED, KV_RAGGED = 0, 1
MASK_NONE, MASK_CUSTOM = 0, 1


class CacheDesc(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("page_stride", ctypes.c_int64),
                ("token_stride", ctypes.c_int64), ("head_stride", ctypes.c_int64),
                ("max_num_pages", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("layout", ctypes.c_int32), ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float)]


class PlanParams(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "mode", "batch_size", "num_qo_heads", "num_kv_heads", "head_dim_qk", "head_dim_vo", "page_size", "causal",
        "q_dtype", "kv_dtype", "num_cus", "fixed_split_pages", "target_per_cu", "mla_head_groups",
        "max_num_pages", "tail_split", "kv_format", "mask_mode", "merge_in_launch", "row_waves")]


class PlanInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "mode", "batch_size", "num_items", "num_merges", "num_partial_rows", "chunk_pages", "split",
        "rows_per_tile", "heads_y", "num_cus", "target", "total_rows")] + [
        ("workspace_bytes", ctypes.c_int64), ("staging_bytes", ctypes.c_int64), ("fingerprint", ctypes.c_uint64),
        ("mask_bits", ctypes.c_int64), ("merge_in_launch", ctypes.c_int32), ("row_waves", ctypes.c_int32)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


class GraphCaps(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "max_total_rows", "max_total_pages", "max_items", "max_merges", "max_partial_rows", "reserved")]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_ if name != "reserved"}


class CascadeLevel(ctypes.Structure):
    _fields_ = [("num_nodes", ctypes.c_int32), ("qo_indptr", ctypes.POINTER(ctypes.c_int32)),
                ("kv_indptr", ctypes.POINTER(ctypes.c_int32)), ("kv_indices", ctypes.POINTER(ctypes.c_int32)),
                ("num_indices", ctypes.c_int64), ("kv_last_page_len", ctypes.POINTER(ctypes.c_int32))]


class CascadeInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_levels", "total_rows", "num_items", "num_partial_rows", "num_merge_slots", "reserved")] + [
        ("workspace_bytes", ctypes.c_int64), ("staging_bytes", ctypes.c_int64), ("fingerprint", ctypes.c_uint64)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_ if name != "reserved"}


_i32p = ctypes.POINTER(ctypes.c_int32)
_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32

# name -> (restype, argtypes); exactly the functions include/pkv.h declares.
SIGNATURES = {
    "pkv_version": (ctypes.c_char_p, []),
    "pkv_last_error": (ctypes.c_char_p, []),
    "pkv_last_meta_reason": (_i32, []),
    "pkv_device_num_cus": (_i32, [_i32p]),
    "pkv_validate": (_i32, [_i32p, _i32p, _i32p, _i64, _i32p, _i32, _i32, _i32, _i32, _i32, _i32, _i32p]),
    "pkv_validate_append": (_i32, [_i32p, _i32p, _i32p, _i64, _i32p, _i32, _i32, _i32]),
    "pkv_append_paged_kv": (_i32, [_vp, _vp, _i64, _i64, _vp, _vp, _vp, _vp, _i32, _i32,
                                   ctypes.POINTER(CacheDesc), _vp]),
    "pkv_plan_compute": (_i32, [ctypes.POINTER(PlanParams), _i32p, _i32p, _i32p, _i64, _i32p, _i32p, _i64, _i32p,
                                _i64, ctypes.POINTER(PlanInfo)]),
    "pkv_plan_create": (_i32, [ctypes.POINTER(PlanParams), _i32p, _i32p, _i32p, _i64, _i32p, _vp, ctypes.c_size_t,
                               _vp, ctypes.c_size_t, _vp, ctypes.POINTER(_vp)]),
    "pkv_plan_get_info": (_i32, [_vp, ctypes.POINTER(PlanInfo)]),
    "pkv_plan_check": (_i32, [_vp, _i32p, _i32p, _i32p, _i64, _i32p]),
    "pkv_plan_destroy": (_i32, [_vp]),
    "pkv_graph_plan_size": (_i32, [ctypes.POINTER(PlanParams), ctypes.POINTER(GraphCaps), ctypes.POINTER(GraphCaps),
                                   ctypes.POINTER(_i64), ctypes.POINTER(_i64)]),
    "pkv_graph_plan_create": (_i32, [ctypes.POINTER(PlanParams), ctypes.POINTER(GraphCaps), _vp, ctypes.c_size_t, _vp,
                                     ctypes.c_size_t, _vp, ctypes.POINTER(_vp)]),
    "pkv_plan_update": (_i32, [_vp, _i32p, _i32p, _i32p, _i64, _i32p, _vp]),
    "pkv_run": (_i32, [_vp, _vp, _i64, _i64, ctypes.POINTER(CacheDesc), _vp, _vp, _i64, _i64, _vp, ctypes.c_float,
                       _vp]),
    "pkv_run_attention": (_i32, [_vp, _vp, _i64, _i64, ctypes.POINTER(CacheDesc), _vp, _vp, _i64, _i64, _vp,
                                 ctypes.c_float, _vp]),
    "pkv_run_merge": (_i32, [_vp, _vp, _i64, _i64, _vp, _vp]),
    "pkv_run_append": (_i32, [_vp, _vp, _i64, _i64, ctypes.POINTER(CacheDesc), _vp, _vp, _vp, _i64, _i64, _vp, _vp,
                              _vp, _i32, _vp, _i64, _i64, _vp, ctypes.c_float, _i32, _vp]),
    "pkv_time_next_attention": (_i32, [_vp, _vp]),
    "pkv_run_mla": (_i32, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _vp, _vp, _vp, ctypes.c_float, _vp]),
    "pkv_run_noalloc": (_i32, [ctypes.POINTER(PlanParams), _i32p, _i32p, _i32p, _i64, _i32p, _vp, _i64, _i64,
                               ctypes.POINTER(CacheDesc), _vp, _vp, _i64, _i64, _vp, ctypes.c_float, _vp]),
    "pkv_cascade_plan_compute": (_i32, [ctypes.POINTER(PlanParams), _i32, ctypes.POINTER(CascadeLevel),
                                        ctypes.POINTER(CascadeInfo), ctypes.POINTER(PlanInfo), _i32p, _i64, _i32p,
                                        _i64, _i32p, _i64]),
    "pkv_cascade_plan_create": (_i32, [ctypes.POINTER(PlanParams), _i32, ctypes.POINTER(CascadeLevel), _vp,
                                       ctypes.c_size_t, _vp, ctypes.c_size_t, _vp, ctypes.POINTER(_vp)]),
    "pkv_cascade_plan_get_info": (_i32, [_vp, ctypes.POINTER(CascadeInfo)]),
    "pkv_cascade_run": (_i32, [_vp, _vp, _i64, _i64, ctypes.POINTER(CacheDesc), _vp, _vp, _i64, _i64,
                               _vp, ctypes.c_float, _vp]),
    "pkv_cascade_plan_destroy": (_i32, [_vp]),
    "pkv_run_masked": (_i32, [_vp, _vp, _i64, _i64, ctypes.POINTER(CacheDesc), _vp, _vp, _vp, _i64, _i64, _vp,
                              ctypes.c_float, _vp]),
    "pkv_run_ragged": (_i32, [_vp, _vp, _i64, _i64, _vp, _vp, _i64, _i64, _vp, _vp, _vp, _i64, _i64, _vp,
                              ctypes.c_float, _vp]),
    "pkv_packbits": (_i32, [_vp, _i64, _vp, _vp]),
    "pkv_merge_state": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _vp]),
    "pkv_merge_states": (_i32, [_vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _vp]),
}


def load_library(path: str = LIB_PATH):
    """Load libpkv.so and declare every exported function's signature."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                           "(python -m paged_kv_cache_plan_amd._build)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib
