"""GPU parity of multi-level cascade attention: pkv_cascade_run (through the C
ABI) against the float64 oracle cascade on the same seeded, NaN-poisoned
inputs.  New tokens are first appended into the leaves' pages on the GPU."""

import numpy as np
import pytest

import workloads as wl
from oracle import cascade as occ
from oracle import metadata as omd
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    return gu.require_gpu()


@pytest.fixture(scope="module")
def pkv(torch):
    import paged_kv_cache_plan_amd as pkv
    return pkv


def _leaf_append_host(b):
    """Host copies of the caches after the leaves' new tokens are written."""
    k, v = b.k_cache.copy(), b.v_cache.copy()
    targets = omd.append_targets(list(b.append_indptr), list(b.kv_indptr), list(b.kv_indices),
                                 list(b.kv_last_page_len), b.page_size)
    for t, (page, slot) in enumerate(targets):
        if b.layout == "NHD":
            k[page, slot], v[page, slot] = b.k_new[t], b.v_new[t]
        else:
            k[page, :, slot], v[page, :, slot] = b.k_new[t], b.v_new[t]
    return k, v


def _run_cascade(pkv, torch, b, k_dev, v_dev, *, fixed=0, num_cus=0, causal=None, levels=None):
    levels = b.extra["levels"] if levels is None else levels
    causal = b.causal if causal is None else causal
    params = pkv.plan_params(mode="prefill", batch_size=0, num_qo_heads=b.num_qo_heads, num_kv_heads=b.num_kv_heads,
                             head_dim_qk=b.head_dim, page_size=b.page_size, causal=causal, dtype=b.dtype,
                             num_cus=num_cus, fixed_split_pages=fixed, max_num_pages=k_dev.shape[0])
    plan = pkv.CascadePlan(params, levels)
    q = gu.to_dev(b.q, b.dtype)
    out = gu.empty_like_out(q.shape, b.dtype)
    lse = torch.full((q.shape[0], b.num_qo_heads), float("nan"), dtype=torch.float32, device="cuda")
    idx = gu.to_dev(np.concatenate([lv["kv_indices"][:lv["kv_indptr"][-1]] for lv in levels]), "i32")
    plan.run(q, k_dev, v_dev, idx, out, lse, layout=b.layout, sm_scale=b.sm_scale)
    torch.cuda.synchronize()
    return plan, gu.to_host(out, b.dtype), lse.cpu().numpy()


def _oracle(b, k_host, v_host, causal=None, levels=None):
    return occ.cascade_attention(b.q, k_host, v_host, levels=b.extra["levels"] if levels is None else levels,
                                 page_size=b.page_size, layout=b.layout, num_kv_heads=b.num_kv_heads,
                                 causal=b.causal if causal is None else causal, sm_scale=b.sm_scale,
                                 q_dtype=b.dtype, kv_dtype=b.dtype)


def _append(pkv, b, k_dev, v_dev):
    pkv.append_paged_kv(gu.to_dev(b.k_new, b.dtype), gu.to_dev(b.v_new, b.dtype), gu.to_dev(b.append_indptr, "i32"),
                        gu.to_dev(b.kv_indptr, "i32"), gu.to_dev(b.kv_indices, "i32"),
                        gu.to_dev(b.kv_last_page_len, "i32"), k_dev, v_dev, layout=b.layout, page_size=b.page_size)


@pytest.mark.parametrize("layout,causal", [("NHD", True), ("HND", True), ("NHD", False)])
def test_cascade_small_f32_append_then_run(torch, pkv, layout, causal):
    """Three-level tree of 8 requests (nodes 1 / 3,2,3 / 8 leaves), page 4,
    heads 4/2, dim 64, float32: append into the leaves, then the cascade."""
    print("case cascade_small f32", layout, causal, flush=True)
    b = wl.make("cascade_small", poison=True, layout=layout, causal=causal)
    k_dev, v_dev = gu.to_dev(b.k_cache, "f32"), gu.to_dev(b.v_cache, "f32")
    _append(pkv, b, k_dev, v_dev)
    k_exp, v_exp = _leaf_append_host(b)
    plan, o, lse = _run_cascade(pkv, torch, b, k_dev, v_dev)
    ro, rl = _oracle(b, k_exp, v_exp)
    gu.check_close(o, ro, "f32", "cascade o")
    gu.check_lse(lse, rl, "cascade lse", atol=1e-5)
    assert plan.info["num_levels"] == 3


@pytest.mark.parametrize("fixed", [0, 1, 3])
def test_cascade_bf16_mfma_levels_forced_splits(torch, pkv, fixed):
    """bf16, heads 8/2, dim 128 (the MFMA tile kernel runs the multi-row
    levels) with the keys forced into 1- and 3-page chunks."""
    print("case cascade bf16 fixed", fixed, flush=True)
    b = wl.make("cascade_small", seed=21, poison=True, dtype="bf16", hq=8, hkv=2, dim=128, page_size=16,
                tree=[[12], [5, 7], [2, 3, 4, 3], [1] * 12], level_kv=[(300, 300), (40, 200), (1, 90), (1, 70)],
                qo_range=(1, 9))
    k_dev, v_dev = gu.to_dev(b.k_cache, "bf16"), gu.to_dev(b.v_cache, "bf16")
    _append(pkv, b, k_dev, v_dev)
    k_exp, v_exp = _leaf_append_host(b)
    plan, o, lse = _run_cascade(pkv, torch, b, k_dev, v_dev, fixed=fixed, num_cus=8)
    ro, rl = _oracle(b, k_exp, v_exp)
    gu.check_close(gu.as_f64(o, "bf16"), ro, "bf16", f"cascade bf16 fixed={fixed}")
    gu.check_lse(lse, rl, f"cascade bf16 lse fixed={fixed}")


def test_cascade_shared_prefix_decode_full_size(torch, pkv):
    """64 decode requests under a 16384-token shared prefix, 8 branch nodes of
    U[1024, 4096] tokens and per-request leaves of U[128, 1024] tokens; page
    16, heads 32/8, dim 128, bf16.  The new token of each request is appended
    into its leaf first."""
    print("case cascade full size", flush=True)
    b = wl.make("cascade", poison=True)
    k_dev, v_dev = gu.to_dev(b.k_cache, "bf16"), gu.to_dev(b.v_cache, "bf16")
    _append(pkv, b, k_dev, v_dev)
    k_exp, v_exp = _leaf_append_host(b)
    plan, o, lse = _run_cascade(pkv, torch, b, k_dev, v_dev)
    ro, rl = _oracle(b, k_exp, v_exp)
    rep = gu.check_close(gu.as_f64(o, "bf16"), ro, "bf16", "cascade full o")
    gu.check_lse(lse, rl, "cascade full lse")
    print("cascade parity", rep, plan.info)


def test_one_level_cascade_matches_plain_run(torch, pkv):
    """A cascade of the leaf level alone is ordinary batched attention."""
    b = wl.make("cascade_small", seed=5, poison=True, dtype="bf16", hq=8, hkv=2, dim=128, page_size=16,
                level_kv=[(50, 50), (10, 40), (4, 60)], qo_range=(1, 6))
    k_dev, v_dev = gu.to_dev(b.k_cache, "bf16"), gu.to_dev(b.v_cache, "bf16")
    _append(pkv, b, k_dev, v_dev)
    k_exp, v_exp = _leaf_append_host(b)
    leaf = [b.extra["levels"][-1]]
    _, o, lse = _run_cascade(pkv, torch, b, k_dev, v_dev, levels=leaf)
    ro, rl = _oracle(b, k_exp, v_exp, levels=leaf)
    gu.check_close(gu.as_f64(o, "bf16"), ro, "bf16", "one-level cascade o")
    gu.check_lse(lse, rl, "one-level cascade lse")


def test_cascade_over_fp8_cache(torch, pkv):
    """The bf16 tree above with its cache rounded to E4M3 (bf16 queries)."""
    b = wl.make("cascade_small", seed=21, poison=True, dtype="bf16", hq=8, hkv=2, dim=128, page_size=16,
                tree=[[12], [5, 7], [2, 3, 4, 3], [1] * 12], level_kv=[(300, 300), (40, 200), (1, 90), (1, 70)],
                qo_range=(1, 9))
    # Round the bf16 cache values to E4M3 codes (poisoned slots become the fp8 NaN code).
    k8 = wl.to_fp8_codes(gu.as_f64(b.k_cache, "bf16").astype(np.float32))
    v8 = wl.to_fp8_codes(gu.as_f64(b.v_cache, "bf16").astype(np.float32))
    k8[np.isnan(gu.as_f64(b.k_cache, "bf16"))] = wl.FP8_NAN
    v8[np.isnan(gu.as_f64(b.v_cache, "bf16"))] = wl.FP8_NAN
    kn = wl.to_fp8_codes(gu.as_f64(b.k_new, "bf16").astype(np.float32))
    vn = wl.to_fp8_codes(gu.as_f64(b.v_new, "bf16").astype(np.float32))
    k_dev = torch.from_numpy(k8).cuda()
    v_dev = torch.from_numpy(v8).cuda()
    pkv.append_paged_kv(torch.from_numpy(kn).cuda(), torch.from_numpy(vn).cuda(), gu.to_dev(b.append_indptr, "i32"),
                        gu.to_dev(b.kv_indptr, "i32"), gu.to_dev(b.kv_indices, "i32"),
                        gu.to_dev(b.kv_last_page_len, "i32"), k_dev, v_dev, layout=b.layout, page_size=b.page_size)
    b8 = wl.Batch(**{**b.__dict__, "k_cache": k8, "v_cache": v8, "k_new": kn, "v_new": vn, "kv_dtype": "fp8"})
    k_exp, v_exp = _leaf_append_host(b8)
    levels = b.extra["levels"]
    params = pkv.plan_params(mode="prefill", batch_size=0, num_qo_heads=8, num_kv_heads=2, head_dim_qk=128,
                             page_size=16, causal=True, dtype="bf16", kv_dtype="fp8", max_num_pages=k_dev.shape[0])
    plan = pkv.CascadePlan(params, levels)
    q = gu.to_dev(b.q, "bf16")
    out = gu.empty_like_out(q.shape, "bf16")
    lse = torch.full((q.shape[0], 8), float("nan"), dtype=torch.float32, device="cuda")
    idx = gu.to_dev(np.concatenate([lv["kv_indices"][:lv["kv_indptr"][-1]] for lv in levels]), "i32")
    plan.run(q, k_dev, v_dev, idx, out, lse, layout=b.layout, sm_scale=b.sm_scale, k_scale=0.5, v_scale=2.0)
    torch.cuda.synchronize()
    ro, rl = occ.cascade_attention(b.q, k_exp, v_exp, levels=levels, page_size=16, layout=b.layout, num_kv_heads=2,
                                   causal=True, sm_scale=b.sm_scale * 0.5, q_dtype="bf16", kv_dtype="fp8")
    gu.check_close(gu.as_f64(gu.to_host(out, "bf16"), "bf16"), 2.0 * ro, "bf16", "cascade fp8 o")
    gu.check_lse(lse.cpu().numpy(), rl, "cascade fp8 lse")
