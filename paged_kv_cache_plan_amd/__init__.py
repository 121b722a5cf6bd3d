"""Paged KV-cache attention for AMD MI355X (gfx950): thin Python binding.

Every call below marshals arguments for one entry point of the C ABI in
``include/pkv.h`` (loaded from the in-tree ``libpkv.so``) and does nothing
else: all computation runs in the library's HIP kernels.  Device buffers are
torch tensors on a ROCm device; host metadata is int32 (numpy arrays, torch
CPU tensors or lists).  Metadata of any other integer type is rejected, never
cast ("FlashInfer 中的 KV-Cache 布局": indptr, page-index and tail arrays are
int32).  The library is required: importing this package without a built
``libpkv.so`` raises.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

from ._abi import (BF16, DECODE, F32, FP8_E4M3, HND, KV_PAGED, KV_RAGGED, MASK_CUSTOM, MASK_NONE, MLA_DECODE, NHD, PREFILL,
                   STATUS_NAMES, CacheDesc, CascadeInfo, CascadeLevel, GraphCaps, PlanInfo, PlanParams,
                   load_library)

_lib = None


def lib():
    """The loaded libpkv.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        _lib = load_library()
    return _lib


from ._abi import LIB_PATH  # noqa: E402  (PKV_LIB_PATH may name another build)


class PkvError(RuntimeError):
    def __init__(self, status: int, message: str, reason: int = 0):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.reason = reason


def _check(status: int):
    if status != 0:
        L = lib()
        raise PkvError(status, L.pkv_last_error().decode(), L.pkv_last_meta_reason())


def last_meta_reason() -> int:
    return lib().pkv_last_meta_reason()


# ---------------------------------------------------------------- helpers --

def _host_i32(x, name):
    """Host int32 array -> (numpy array kept alive, pointer).  None -> (None, None)."""
    if x is None:
        return None, None
    try:
        import torch
        if isinstance(x, torch.Tensor):
            if x.device.type != "cpu":
                raise TypeError(f"{name} must be a host array")
            if x.dtype != torch.int32:
                raise TypeError(f"{name} must be int32, got {x.dtype}")
            x = x.contiguous().numpy()
    except ImportError:
        pass
    if isinstance(x, (list, tuple)):
        x = np.asarray(x, dtype=np.int32)
    if not isinstance(x, np.ndarray) or x.dtype != np.int32:
        raise TypeError(f"{name} must be int32, got {getattr(x, 'dtype', type(x))}")
    x = np.ascontiguousarray(x)
    return x, x.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _check_batch(params, qo, kvp, last):
    """The C ABI reads B+1 / B entries (B = params.batch_size) from these host arrays."""
    b = params.batch_size
    ragged = params.kv_format == KV_RAGGED
    if (kvp is None or len(kvp) != b + 1 or (qo is not None and len(qo) != b + 1)
            or (not ragged and (last is None or len(last) != b))):
        raise ValueError(f"metadata lengths do not match batch_size {b}")


def _dev(t, name, dtype=None):
    """Device tensor -> raw pointer (checks device and dtype)."""
    import torch
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):   # E4M3 codes
        return FP8_E4M3
    raise TypeError(f"unsupported payload dtype {t.dtype}")


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def version() -> str:
    return lib().pkv_version().decode()


def device_num_cus() -> int:
    out = ctypes.c_int32()
    _check(lib().pkv_device_num_cus(ctypes.byref(out)))
    return out.value


def cache_desc(k, v, layout: str, page_size: int, num_kv_heads: int, head_dim: int, k_scale: float = 1.0,
               v_scale: float = 1.0) -> CacheDesc:
    """Descriptor of a paged cache given as two 4-D views (either the tuple
    form or the K/V halves of a 5-D [pages, 2, ...] tensor).  Strides are taken
    from the tensors; the innermost (dim) stride must be 1."""
    if k.dim() != 4 or v.dim() != 4 or k.shape != v.shape or k.stride() != v.stride():
        raise ValueError("k and v must be 4-D views with equal shapes and strides")
    if k.stride(3) != 1:
        raise ValueError("head_dim must be contiguous")
    if layout == "NHD":
        page_st, tok_st, head_st = k.stride(0), k.stride(1), k.stride(2)
        shape = (page_size, num_kv_heads, head_dim)
    elif layout == "HND":
        page_st, tok_st, head_st = k.stride(0), k.stride(2), k.stride(1)
        shape = (num_kv_heads, page_size, head_dim)
    else:
        raise ValueError(layout)
    if tuple(k.shape[1:]) != shape:
        raise ValueError(f"cache shape {tuple(k.shape)} does not match {layout} {shape}")
    d = CacheDesc()
    d.k = k.data_ptr()
    d.v = v.data_ptr()
    d.page_stride, d.token_stride, d.head_stride = page_st, tok_st, head_st
    d.max_num_pages = k.shape[0]
    d.page_size, d.num_kv_heads, d.head_dim = page_size, num_kv_heads, head_dim
    d.dtype = _dtype_code(k)
    d.layout = NHD if layout == "NHD" else HND
    d.k_scale, d.v_scale = k_scale, v_scale
    return d


# -------------------------------------------------------------- validation --

def validate(*, qo_indptr, kv_indptr, kv_indices, kv_last_page_len, page_size, max_num_pages,
             num_qo_heads=1, num_kv_heads=1, decode=False):
    """pkv_validate: returns kv_len per request (numpy int32) or raises PkvError."""
    qo, qo_p = _host_i32(qo_indptr, "qo_indptr")
    kvp, kvp_p = _host_i32(kv_indptr, "kv_indptr")
    idx, idx_p = _host_i32(kv_indices, "kv_indices")
    last, last_p = _host_i32(kv_last_page_len, "kv_last_page_len")
    b = len(last)
    out = np.zeros(max(b, 1), dtype=np.int32)
    _check(lib().pkv_validate(qo_p, kvp_p, idx_p, len(idx), last_p, b, page_size, max_num_pages,
                              num_qo_heads, num_kv_heads, int(decode),
                              out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))))
    return out[:b]


def validate_append(*, append_indptr, kv_indptr, kv_indices, kv_last_page_len, page_size, max_num_pages):
    ap, ap_p = _host_i32(append_indptr, "append_indptr")
    kvp, kvp_p = _host_i32(kv_indptr, "kv_indptr")
    idx, idx_p = _host_i32(kv_indices, "kv_indices")
    last, last_p = _host_i32(kv_last_page_len, "kv_last_page_len")
    _check(lib().pkv_validate_append(ap_p, kvp_p, idx_p, len(idx), last_p, len(last), page_size, max_num_pages))


# ------------------------------------------------------------------- plan --

_MODES = {"decode": DECODE, "prefill": PREFILL, "mla": MLA_DECODE}
_DTYPES = {"f32": F32, "bf16": BF16, "fp8": FP8_E4M3}


def plan_params(*, mode, batch_size, num_qo_heads, num_kv_heads, head_dim_qk, head_dim_vo=None, page_size,
                causal=True, dtype="bf16", num_cus=0, fixed_split_pages=0, target_per_cu=0,
                mla_head_groups=0, max_num_pages=0, tail_split=0, ragged=False, custom_mask=False,
                kv_dtype=None, merge_in_launch=False, row_waves=0) -> PlanParams:
    p = PlanParams()
    p.mode = _MODES[mode] if isinstance(mode, str) else mode
    p.batch_size = batch_size
    p.num_qo_heads, p.num_kv_heads = num_qo_heads, num_kv_heads
    p.head_dim_qk = head_dim_qk
    p.head_dim_vo = head_dim_qk if head_dim_vo is None else head_dim_vo
    p.page_size = page_size
    p.causal = int(causal)
    p.q_dtype = p.kv_dtype = _DTYPES[dtype] if isinstance(dtype, str) else dtype
    if kv_dtype is not None:
        p.kv_dtype = _DTYPES[kv_dtype] if isinstance(kv_dtype, str) else kv_dtype
    p.num_cus, p.fixed_split_pages, p.target_per_cu = num_cus, fixed_split_pages, target_per_cu
    p.mla_head_groups, p.max_num_pages = mla_head_groups, max_num_pages
    p.tail_split = tail_split
    p.kv_format = KV_RAGGED if ragged else KV_PAGED
    p.mask_mode = MASK_CUSTOM if custom_mask else MASK_NONE
    p.merge_in_launch = int(merge_in_launch)
    p.row_waves = row_waves
    return p


def plan_compute(params: PlanParams, *, qo_indptr, kv_indptr, kv_indices, kv_last_page_len):
    """pkv_plan_compute (host only): (info dict, items [n, 8] int32, merges [m, 4] int32)."""
    qo, qo_p = _host_i32(qo_indptr, "qo_indptr")
    kvp, kvp_p = _host_i32(kv_indptr, "kv_indptr")
    idx, idx_p = _host_i32(kv_indices, "kv_indices")
    last, last_p = _host_i32(kv_last_page_len, "kv_last_page_len")
    n_idx = 0 if idx is None else len(idx)
    info = PlanInfo()
    L = lib()
    _check(L.pkv_plan_compute(ctypes.byref(params), qo_p, kvp_p, idx_p, n_idx, last_p, None, 0, None, 0,
                              ctypes.byref(info)))
    items = np.zeros((info.num_items, 8), dtype=np.int32)
    merges = np.zeros((info.num_merges, 4), dtype=np.int32)
    _check(L.pkv_plan_compute(ctypes.byref(params), qo_p, kvp_p, idx_p, n_idx, last_p,
                              items.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), items.size,
                              merges.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), merges.size,
                              ctypes.byref(info)))
    return info.as_dict(), items, merges


class Plan:
    """pkv_plan_create / pkv_run / pkv_plan_destroy with torch-owned buffers.

    The workspace (device) and staging (pinned host) buffers are allocated
    here with torch and kept alive as long as the plan.  ``workspace`` /
    ``staging`` may be passed in to reuse buffers across plans (the library
    waits for the previous upload from a reused staging buffer)."""

    def __init__(self, params: PlanParams, *, kv_indptr, kv_last_page_len, kv_indices=None, qo_indptr=None,
                 workspace=None, staging=None, stream=None):
        import torch
        self.params = params
        self._meta = [_host_i32(x, n) for x, n in ((qo_indptr, "qo_indptr"), (kv_indptr, "kv_indptr"),
                                                    (kv_indices, "kv_indices"),
                                                    (kv_last_page_len, "kv_last_page_len"))]
        (qo, qo_p), (kvp, kvp_p), (idx, idx_p), (last, last_p) = self._meta
        _check_batch(params, qo, kvp, last)
        n_idx = 0 if idx is None else len(idx)
        info = PlanInfo()
        _check(lib().pkv_plan_compute(ctypes.byref(params), qo_p, kvp_p, idx_p, n_idx, last_p, None, 0, None, 0,
                                      ctypes.byref(info)))
        ws_bytes = max(int(info.workspace_bytes), 256)
        st_bytes = max(int(info.staging_bytes), 256)
        if workspace is None or workspace.numel() < ws_bytes:
            workspace = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
        if staging is None or staging.numel() < st_bytes:
            staging = torch.empty(st_bytes, dtype=torch.uint8, pin_memory=True)
        self.workspace, self.staging = workspace, staging
        handle = ctypes.c_void_p()
        _check(lib().pkv_plan_create(ctypes.byref(params), qo_p, kvp_p, idx_p, n_idx, last_p,
                                     ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
                                     ctypes.c_void_p(staging.data_ptr()), staging.numel(), _stream(stream),
                                     ctypes.byref(handle)))
        self._handle = handle

    @property
    def info(self) -> dict:
        out = PlanInfo()
        _check(lib().pkv_plan_get_info(self._handle, ctypes.byref(out)))
        return out.as_dict()

    def check(self, *, kv_indptr, kv_last_page_len, kv_indices=None, qo_indptr=None):
        """pkv_plan_check: raises PkvError(STALE_PLAN) if the metadata changed."""
        qo, qo_p = _host_i32(qo_indptr, "qo_indptr")
        kvp, kvp_p = _host_i32(kv_indptr, "kv_indptr")
        idx, idx_p = _host_i32(kv_indices, "kv_indices")
        last, last_p = _host_i32(kv_last_page_len, "kv_last_page_len")
        _check(lib().pkv_plan_check(self._handle, qo_p, kvp_p, idx_p, 0 if idx is None else len(idx), last_p))

    def run(self, q, k_cache, v_cache, kv_indices, out, lse=None, *, layout, sm_scale=0.0, stream=None,
            _entry="pkv_run", k_scale=1.0, v_scale=1.0):
        """pkv_run.  q [nnz, Hq, D] and out [nnz, Hq, D] device tensors of the plan's dtype;
        k_cache/v_cache 4-D views (see ``cache_desc``); kv_indices device int32; lse float32 [nnz, Hq]."""
        import torch
        p = self.params
        desc = cache_desc(k_cache, v_cache, layout, p.page_size, p.num_kv_heads, p.head_dim_qk, k_scale, v_scale)
        if q.dim() != 3 or out.dim() != 3 or q.stride(2) != 1 or out.stride(2) != 1:
            raise ValueError("q and out must be [tokens, heads, dim] with contiguous dim")
        if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()):
            raise TypeError("lse must be contiguous float32")
        _check(getattr(lib(), _entry)(self._handle, _dev(q, "q"), q.stride(0), q.stride(1), ctypes.byref(desc),
                                      _dev(kv_indices, "kv_indices", torch.int32), _dev(out, "out", q.dtype),
                                      out.stride(0), out.stride(1), None if lse is None else _dev(lse, "lse"),
                                      ctypes.c_float(sm_scale), _stream(stream)))

    def run_attention(self, q, k_cache, v_cache, kv_indices, out, lse=None, *, layout, sm_scale=0.0, stream=None,
                      k_scale=1.0, v_scale=1.0):
        """pkv_run_attention: the attention kernel only (split tiles stay as partial states)."""
        self.run(q, k_cache, v_cache, kv_indices, out, lse, layout=layout, sm_scale=sm_scale, stream=stream,
                 _entry="pkv_run_attention", k_scale=k_scale, v_scale=v_scale)

    def run_append(self, q, k_cache, v_cache, kv_indices, out, lse=None, *, k_new, v_new, append_indptr, kv_indptr,
                   kv_last_page_len, layout, sm_scale=0.0, with_merge=True, stream=None, k_scale=1.0, v_scale=1.0):
        """pkv_run_append: append_paged_kv of k_new/v_new [nnz, Hkv, D] fused into this decode run
        (with_merge False: the attention launch only, like run_attention).  Metadata device int32."""
        import torch
        p = self.params
        desc = cache_desc(k_cache, v_cache, layout, p.page_size, p.num_kv_heads, p.head_dim_qk, k_scale, v_scale)
        if q.dim() != 3 or out.dim() != 3 or q.stride(2) != 1 or out.stride(2) != 1:
            raise ValueError("q and out must be [tokens, heads, dim] with contiguous dim")
        if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()):
            raise TypeError("lse must be contiguous float32")
        if k_new.shape != v_new.shape or k_new.stride() != v_new.stride() or k_new.stride(2) != 1:
            raise ValueError("k_new and v_new must be [nnz, heads, dim] with equal strides")
        i32 = torch.int32
        _check(lib().pkv_run_append(self._handle, _dev(q, "q"), q.stride(0), q.stride(1), ctypes.byref(desc),
                                    _dev(kv_indices, "kv_indices", i32), _dev(k_new, "k_new", k_cache.dtype),
                                    _dev(v_new, "v_new", k_cache.dtype), k_new.stride(0), k_new.stride(1),
                                    _dev(append_indptr, "append_indptr", i32), _dev(kv_indptr, "kv_indptr", i32),
                                    _dev(kv_last_page_len, "kv_last_page_len", i32), k_new.shape[0],
                                    _dev(out, "out", q.dtype), out.stride(0), out.stride(1),
                                    None if lse is None else _dev(lse, "lse"), ctypes.c_float(sm_scale),
                                    1 if with_merge else 0, _stream(stream)))

    def run_merge(self, out, lse=None, *, stream=None):
        """pkv_run_merge: merge the split tiles' partial states into out / lse."""
        _check(lib().pkv_run_merge(self._handle, _dev(out, "out"), out.stride(0), out.stride(1),
                                   None if lse is None else _dev(lse, "lse"), _stream(stream)))

    def run_masked(self, q, k_cache, v_cache, kv_indices, mask_packed, out, lse=None, *, layout, sm_scale=0.0,
                   stream=None, k_scale=1.0, v_scale=1.0):
        """pkv_run_masked: mask_packed is the device bit-packed custom mask (see ``packbits``)."""
        import torch
        p = self.params
        desc = cache_desc(k_cache, v_cache, layout, p.page_size, p.num_kv_heads, p.head_dim_qk, k_scale, v_scale)
        if q.dim() != 3 or out.dim() != 3 or q.stride(2) != 1 or out.stride(2) != 1:
            raise ValueError("q and out must be [tokens, heads, dim] with contiguous dim")
        if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()):
            raise TypeError("lse must be contiguous float32")
        _check(lib().pkv_run_masked(self._handle, _dev(q, "q"), q.stride(0), q.stride(1), ctypes.byref(desc),
                                    _dev(kv_indices, "kv_indices", torch.int32), _dev(mask_packed, "mask", torch.uint8),
                                    _dev(out, "out", q.dtype), out.stride(0), out.stride(1),
                                    None if lse is None else _dev(lse, "lse"), ctypes.c_float(sm_scale),
                                    _stream(stream)))

    def run_ragged(self, q, k, v, kv_indptr, out, lse=None, *, mask_packed=None, sm_scale=0.0, stream=None):
        """pkv_run_ragged: k, v [tokens, Hkv, D] device tensors; kv_indptr device int32 [B+1]."""
        import torch
        if k.dim() != 3 or k.shape != v.shape or k.stride() != v.stride() or k.stride(2) != 1:
            raise ValueError("k and v must be [tokens, heads, dim] with equal strides and contiguous dim")
        if q.dim() != 3 or out.dim() != 3 or q.stride(2) != 1 or out.stride(2) != 1:
            raise ValueError("q and out must be [tokens, heads, dim] with contiguous dim")
        if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()):
            raise TypeError("lse must be contiguous float32")
        kv_dt = torch.uint8 if self.params.kv_dtype == FP8_E4M3 else q.dtype   # fp8: E4M3 codes
        _check(lib().pkv_run_ragged(self._handle, _dev(q, "q"), q.stride(0), q.stride(1), _dev(k, "k", kv_dt),
                                    _dev(v, "v", kv_dt), k.stride(0), k.stride(1),
                                    _dev(kv_indptr, "kv_indptr", torch.int32),
                                    None if mask_packed is None else _dev(mask_packed, "mask", torch.uint8),
                                    _dev(out, "out", q.dtype), out.stride(0), out.stride(1),
                                    None if lse is None else _dev(lse, "lse"), ctypes.c_float(sm_scale),
                                    _stream(stream)))

    def run_mla(self, q_ckv, q_kpe, ckv, kpe, kv_indices, out, lse=None, *, sm_scale=0.0, stream=None):
        """pkv_run_mla.  ckv/kpe are [pages, P, 512] / [pages, P, 64] views (same page/token strides)."""
        import torch
        for t, n in ((q_ckv, "q_ckv"), (q_kpe, "q_kpe"), (out, "out")):
            if not t.is_contiguous() or t.dtype != torch.bfloat16:
                raise TypeError(f"{n} must be contiguous bf16")
        if ckv.stride() != kpe.stride() or ckv.stride(2) != 1:
            raise ValueError("ckv and kpe must share page/token strides with contiguous dims")
        _check(lib().pkv_run_mla(self._handle, _dev(q_ckv, "q_ckv"), _dev(q_kpe, "q_kpe"), _dev(ckv, "ckv"),
                                 _dev(kpe, "kpe"), ckv.stride(0), ckv.stride(1),
                                 _dev(kv_indices, "kv_indices", torch.int32), _dev(out, "out"),
                                 None if lse is None else _dev(lse, "lse", torch.float32),
                                 ctypes.c_float(sm_scale), _stream(stream)))

    def __del__(self):
        h = getattr(self, "_handle", None)
        if h and _lib is not None:
            _lib.pkv_plan_destroy(h)
            self._handle = None


# ---------------------------------------------------- run without allocation --

NOALLOC_SCRATCH_BYTES = 32 << 20


def run_noalloc(params: PlanParams, q, k_cache, v_cache, kv_indices, out, lse=None, *, kv_indptr, kv_last_page_len,
                kv_indices_host=None, qo_indptr=None, layout, sm_scale=0.0, stream=None, k_scale=1.0, v_scale=1.0):
    """pkv_run_noalloc: plan this batch on the host and run it with the work
    list and partial states in the library's per-device array (no workspace,
    staging or plan object).  Host metadata as for ``Plan``; device tensors as
    for ``Plan.run``."""
    import torch
    meta = [_host_i32(x, n) for x, n in ((qo_indptr, "qo_indptr"), (kv_indptr, "kv_indptr"),
                                          (kv_indices_host, "kv_indices_host"),
                                          (kv_last_page_len, "kv_last_page_len"))]
    (qo, qo_p), (kvp, kvp_p), (idx, idx_p), (last, last_p) = meta
    _check_batch(params, qo, kvp, last)
    desc = cache_desc(k_cache, v_cache, layout, params.page_size, params.num_kv_heads, params.head_dim_qk,
                      k_scale, v_scale)
    if q.dim() != 3 or out.dim() != 3 or q.stride(2) != 1 or out.stride(2) != 1:
        raise ValueError("q and out must be [tokens, heads, dim] with contiguous dim")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()):
        raise TypeError("lse must be contiguous float32")
    _check(lib().pkv_run_noalloc(ctypes.byref(params), qo_p, kvp_p, idx_p, 0 if idx is None else len(idx), last_p,
                                 _dev(q, "q"), q.stride(0), q.stride(1), ctypes.byref(desc),
                                 _dev(kv_indices, "kv_indices", torch.int32), _dev(out, "out", q.dtype),
                                 out.stride(0), out.stride(1), None if lse is None else _dev(lse, "lse"),
                                 ctypes.c_float(sm_scale), _stream(stream)))


# --------------------------------------------------- fixed-capacity plans --

def graph_caps(*, max_total_rows=0, max_total_pages, max_items=0, max_merges=0, max_partial_rows=0) -> GraphCaps:
    c = GraphCaps()
    c.max_total_rows, c.max_total_pages = max_total_rows, max_total_pages
    c.max_items, c.max_merges, c.max_partial_rows = max_items, max_merges, max_partial_rows
    return c


def graph_plan_size(params: PlanParams, caps: GraphCaps):
    """pkv_graph_plan_size: (resolved capacities dict, workspace bytes, staging bytes)."""
    out = GraphCaps()
    ws, st = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().pkv_graph_plan_size(ctypes.byref(params), ctypes.byref(caps), ctypes.byref(out), ctypes.byref(ws),
                                     ctypes.byref(st)))
    return out.as_dict(), ws.value, st.value


class GraphPlan(Plan):
    """pkv_graph_plan_create / pkv_plan_update: a fixed-capacity plan whose
    runs launch the same grids with the same pointers after every update, so
    they can be captured once (torch.cuda.graph) and replayed per batch."""

    def __init__(self, params: PlanParams, caps: GraphCaps, *, stream=None):
        import torch
        self.params = params
        self.caps, ws_bytes, st_bytes = graph_plan_size(params, caps)
        self.workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
        self.staging = torch.empty(max(st_bytes, 256), dtype=torch.uint8, pin_memory=True)
        self._meta = []
        handle = ctypes.c_void_p()
        _check(lib().pkv_graph_plan_create(ctypes.byref(params), ctypes.byref(caps),
                                           ctypes.c_void_p(self.workspace.data_ptr()), self.workspace.numel(),
                                           ctypes.c_void_p(self.staging.data_ptr()), self.staging.numel(),
                                           _stream(stream), ctypes.byref(handle)))
        self._handle = handle

    def update(self, *, kv_indptr, kv_last_page_len, kv_indices=None, qo_indptr=None, stream=None):
        """pkv_plan_update (host work + one asynchronous copy; not capturable)."""
        self._meta = [_host_i32(x, n) for x, n in ((qo_indptr, "qo_indptr"), (kv_indptr, "kv_indptr"),
                                                    (kv_indices, "kv_indices"),
                                                    (kv_last_page_len, "kv_last_page_len"))]
        (qo, qo_p), (kvp, kvp_p), (idx, idx_p), (last, last_p) = self._meta
        _check_batch(self.params, qo, kvp, last)
        _check(lib().pkv_plan_update(self._handle, qo_p, kvp_p, idx_p, 0 if idx is None else len(idx), last_p,
                                     _stream(stream)))


# ---------------------------------------------------------------- cascade --

def _cascade_levels(levels):
    """Host level structs (and the int32 arrays they point at, kept alive)."""
    keep = []
    arr = (CascadeLevel * max(1, len(levels)))()
    for i, lv in enumerate(levels):
        qo, qo_p = _host_i32(lv["qo_indptr"], "qo_indptr")
        kvp, kvp_p = _host_i32(lv["kv_indptr"], "kv_indptr")
        idx, idx_p = _host_i32(lv.get("kv_indices"), "kv_indices")
        last, last_p = _host_i32(lv["kv_last_page_len"], "kv_last_page_len")
        keep += [qo, kvp, idx, last]
        arr[i].num_nodes = len(last)
        arr[i].qo_indptr, arr[i].kv_indptr, arr[i].kv_indices, arr[i].kv_last_page_len = qo_p, kvp_p, idx_p, last_p
        arr[i].num_indices = 0 if idx is None else len(idx)
    return arr, keep


def cascade_plan_compute(params: PlanParams, levels):
    """pkv_cascade_plan_compute (host only): (info dict, per-level info dicts, items [n, 8],
    row_ptr [rows + 1], slots [n_slots]), all int32 arrays."""
    arr, keep = _cascade_levels(levels)
    info = CascadeInfo()
    L = lib()
    _check(L.pkv_cascade_plan_compute(ctypes.byref(params), len(levels), arr, ctypes.byref(info), None, None, 0,
                                      None, 0, None, 0))
    lvl = (PlanInfo * max(1, len(levels)))()
    items = np.zeros((info.num_items, 8), dtype=np.int32)
    row_ptr = np.zeros(info.total_rows + 1, dtype=np.int32)
    slots = np.zeros(info.num_merge_slots, dtype=np.int32)
    p32 = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    _check(L.pkv_cascade_plan_compute(ctypes.byref(params), len(levels), arr, ctypes.byref(info), lvl,
                                      p32(items), items.size, p32(row_ptr), row_ptr.size, p32(slots), slots.size))
    return info.as_dict(), [lvl[i].as_dict() for i in range(len(levels))], items, row_ptr, slots


class CascadePlan:
    """pkv_cascade_plan_create / pkv_cascade_run / pkv_cascade_plan_destroy.

    ``levels``: list of dicts with host int32 qo_indptr, kv_indptr, kv_indices
    (optional) and kv_last_page_len, level 0 (the root) first.  Workspace and
    staging are allocated here with torch unless passed in."""

    def __init__(self, params: PlanParams, levels, *, workspace=None, staging=None, stream=None):
        import torch
        self.params = params
        self._levels, self._keep = _cascade_levels(levels)
        info = CascadeInfo()
        _check(lib().pkv_cascade_plan_compute(ctypes.byref(params), len(levels), self._levels, ctypes.byref(info),
                                              None, None, 0, None, 0, None, 0))
        ws_bytes = max(int(info.workspace_bytes), 256)
        st_bytes = max(int(info.staging_bytes), 256)
        if workspace is None or workspace.numel() < ws_bytes:
            workspace = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
        if staging is None or staging.numel() < st_bytes:
            staging = torch.empty(st_bytes, dtype=torch.uint8, pin_memory=True)
        self.workspace, self.staging = workspace, staging
        handle = ctypes.c_void_p()
        _check(lib().pkv_cascade_plan_create(ctypes.byref(params), len(levels), self._levels,
                                             ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
                                             ctypes.c_void_p(staging.data_ptr()), staging.numel(), _stream(stream),
                                             ctypes.byref(handle)))
        self._handle = handle

    @property
    def info(self) -> dict:
        out = CascadeInfo()
        _check(lib().pkv_cascade_plan_get_info(self._handle, ctypes.byref(out)))
        return out.as_dict()

    def run(self, q, k_cache, v_cache, kv_indices, out, lse=None, *, layout, sm_scale=0.0, stream=None,
            k_scale=1.0, v_scale=1.0):
        """pkv_cascade_run.  kv_indices: device int32, the levels' page ids back to back (level 0 first)."""
        import torch
        p = self.params
        desc = cache_desc(k_cache, v_cache, layout, p.page_size, p.num_kv_heads, p.head_dim_qk, k_scale, v_scale)
        if q.dim() != 3 or out.dim() != 3 or q.stride(2) != 1 or out.stride(2) != 1:
            raise ValueError("q and out must be [tokens, heads, dim] with contiguous dim")
        if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()):
            raise TypeError("lse must be contiguous float32")
        _check(lib().pkv_cascade_run(self._handle, _dev(q, "q"), q.stride(0), q.stride(1), ctypes.byref(desc),
                                     _dev(kv_indices, "kv_indices", torch.int32), _dev(out, "out", q.dtype),
                                     out.stride(0), out.stride(1), None if lse is None else _dev(lse, "lse"),
                                     ctypes.c_float(sm_scale), _stream(stream)))

    def __del__(self):
        h = getattr(self, "_handle", None)
        if h and _lib is not None:
            _lib.pkv_cascade_plan_destroy(h)
            self._handle = None


# ------------------------------------------------------ append and merges --

def append_paged_kv(k_new, v_new, append_indptr, kv_indptr, kv_indices, kv_last_page_len, k_cache, v_cache, *,
                    layout, page_size, stream=None):
    """pkv_append_paged_kv.  k_new/v_new [nnz, Hkv, D]; metadata device int32 (post-append lengths)."""
    import torch
    hkv, d = k_new.shape[1], k_new.shape[2]
    desc = cache_desc(k_cache, v_cache, layout, page_size, hkv, d)
    if k_new.shape != v_new.shape or k_new.stride() != v_new.stride() or k_new.stride(2) != 1:
        raise ValueError("k_new and v_new must be [nnz, heads, dim] with equal strides")
    i32 = torch.int32
    _check(lib().pkv_append_paged_kv(_dev(k_new, "k_new", k_cache.dtype), _dev(v_new, "v_new", k_cache.dtype),
                                     k_new.stride(0), k_new.stride(1), _dev(append_indptr, "append_indptr", i32),
                                     _dev(kv_indptr, "kv_indptr", i32), _dev(kv_indices, "kv_indices", i32),
                                     _dev(kv_last_page_len, "kv_last_page_len", i32), kv_last_page_len.numel(),
                                     k_new.shape[0], ctypes.byref(desc), _stream(stream)))


def time_next_attention(start=None, stop=None):
    """pkv_time_next_attention: the next attention kernel launched from this
    thread records the two timing events (torch.cuda.Event(enable_timing=True))
    at its own start and end; ``start.elapsed_time(stop)`` after a
    synchronisation is then that kernel's duration.  No arguments disarm."""
    if (start is None) != (stop is None):
        raise ValueError("pass both events or neither")
    if start is None:
        _check(lib().pkv_time_next_attention(None, None))
        return
    for ev in (start, stop):
        if not ev.cuda_event:          # torch creates the event on its first record
            ev.record()
    _check(lib().pkv_time_next_attention(ctypes.c_void_p(start.cuda_event), ctypes.c_void_p(stop.cuda_event)))


def packbits(mask_bool, stream=None):
    """pkv_packbits: a device bool/uint8 tensor -> device uint8 tensor of
    ceil(n / 32) * 4 + 32 bytes (the tail zeroed; the masked kernels read up
    to 32 bytes past the last mask byte), element e at bit e % 8 of byte e // 8."""
    import torch
    m = mask_bool.contiguous()
    if m.dtype == torch.bool:
        m = m.view(torch.uint8)
    if m.dtype != torch.uint8:
        raise TypeError("mask must be bool or uint8")
    n = m.numel()
    out = torch.zeros((n + 31) // 32 * 4 + 32, dtype=torch.uint8, device=m.device)
    _check(lib().pkv_packbits(_dev(m, "mask"), n, _dev(out, "packed"), _stream(stream)))
    return out


def merge_state(v_a, s_a, v_b, s_b, v_out=None, s_out=None, stream=None):
    """pkv_merge_state on [rows, heads, dim] / [rows, heads] device tensors; returns (v_out, s_out)."""
    import torch
    for t in (v_a, s_a, v_b, s_b):
        if not t.is_contiguous():
            raise ValueError("merge inputs must be contiguous")
    v_out = torch.empty_like(v_a) if v_out is None else v_out
    s_out = torch.empty_like(s_a) if s_out is None else s_out
    n, h, d = v_a.shape
    _check(lib().pkv_merge_state(_dev(v_a, "v_a"), _dev(s_a, "s_a", torch.float32), _dev(v_b, "v_b", v_a.dtype),
                                 _dev(s_b, "s_b", torch.float32), _dev(v_out, "v_out", v_a.dtype),
                                 _dev(s_out, "s_out", torch.float32), n, h, d, _dtype_code(v_a), _stream(stream)))
    return v_out, s_out


def merge_states(v, s, stream=None):
    """pkv_merge_states: v [rows, K, heads, dim], s [rows, K, heads] -> ([rows, heads, dim], [rows, heads])."""
    import torch
    if not v.is_contiguous() or not s.is_contiguous():
        raise ValueError("merge inputs must be contiguous")
    n, k, h, d = v.shape
    v_out = torch.empty((n, h, d), dtype=v.dtype, device=v.device)
    s_out = torch.empty((n, h), dtype=torch.float32, device=v.device)
    _check(lib().pkv_merge_states(_dev(v, "v"), _dev(s, "s", torch.float32), _dev(v_out, "v_out"),
                                  _dev(s_out, "s_out"), n, k, h, d, _dtype_code(v), _stream(stream)))
    return v_out, s_out
