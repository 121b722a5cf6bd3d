"""GPU parity with an fp8 (E4M3) K/V cache: bf16 queries and outputs, the
cache read as one byte per element and expanded in registers, the per-tensor
scales applied.  The float64 oracle decodes every code exactly (its decoding
is pinned against torch's float8_e4m3fn for all 256 codes)."""

import numpy as np
import pytest

import workloads as wl
from oracle import attention as oat
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


def _u8(torch, x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _run(pkv, torch, b, k_dev, v_dev, *, k_scale, v_scale, fixed=0, num_cus=0):
    params = pkv.plan_params(mode=b.mode, batch_size=b.batch_size, num_qo_heads=b.num_qo_heads,
                             num_kv_heads=b.num_kv_heads, head_dim_qk=b.head_dim, page_size=b.page_size,
                             causal=b.causal, dtype="bf16", kv_dtype="fp8", fixed_split_pages=fixed,
                             num_cus=num_cus, max_num_pages=k_dev.shape[0])
    plan = pkv.Plan(params, qo_indptr=b.qo_indptr if b.mode == "prefill" else None, kv_indptr=b.kv_indptr,
                    kv_indices=b.kv_indices, kv_last_page_len=b.kv_last_page_len)
    q = gu.to_dev(b.q, "bf16")
    out = gu.empty_like_out(q.shape, "bf16")
    lse = torch.full((q.shape[0], b.num_qo_heads), float("nan"), dtype=torch.float32, device="cuda")
    plan.run(q, k_dev, v_dev, gu.to_dev(b.kv_indices, "i32"), out, lse, layout=b.layout, sm_scale=b.sm_scale,
             k_scale=k_scale, v_scale=v_scale)
    torch.cuda.synchronize()
    return plan, gu.to_host(out, "bf16"), lse.cpu().numpy()


def _oracle(b, k, v, k_scale, v_scale):
    return oat.paged_attention(b.q, k, v, qo_indptr=list(b.qo_indptr), kv_indptr=list(b.kv_indptr),
                               kv_indices=list(b.kv_indices), kv_last_page_len=list(b.kv_last_page_len),
                               page_size=b.page_size, layout=b.layout, num_kv_heads=b.num_kv_heads,
                               causal=b.causal, sm_scale=b.sm_scale, q_dtype="bf16", kv_dtype="fp8",
                               k_scale=k_scale, v_scale=v_scale)


@pytest.mark.parametrize("layout", ["NHD", "HND"])
def test_fp8_decode_full_size(torch, pkv, layout):
    """The decode workload (64 requests, kv U[512, 4096], page 16, 32/8 heads,
    d 128) with its cache rounded to E4M3; NaN codes everywhere no request owns."""
    print("case fp8 decode", layout, flush=True)
    b = wl.make("decode", kv_dtype="fp8", layout=layout, poison=True)
    plan, o, lse = _run(pkv, torch, b, _u8(torch, b.k_cache), _u8(torch, b.v_cache), k_scale=0.5, v_scale=2.0)
    ro, rl = _oracle(b, b.k_cache, b.v_cache, 0.5, 2.0)
    rep = gu.check_close(gu.as_f64(o, "bf16"), ro, "bf16", "fp8 decode o")
    gu.check_lse(lse, rl, "fp8 decode lse")
    grd = gu.check_guard(gu.as_f64(o, "bf16"), ro, lse, rl, "fp8 decode")
    print("fp8 decode parity", rep, grd, plan.info["num_items"])


@pytest.mark.parametrize("fixed", [0, 1, 5])
def test_fp8_every_finite_code(torch, pkv, fixed):
    """Caches drawn uniformly over all 254 finite codes (subnormals, zeros of
    both signs, up to +-448), scaled down so scores stay moderate; forced
    splits merge into bf16 rows."""
    print("case fp8 codes", fixed, flush=True)
    b = wl.make("decode", kv_dtype="fp8", scale=0.25, batch=12)
    rng = np.random.default_rng(31)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    k = rng.choice(finite, size=b.k_cache.shape)
    v = rng.choice(finite, size=b.v_cache.shape)
    ks, vs = 1.0 / 512, 1.0 / 64
    _, o, lse = _run(pkv, torch, b, _u8(torch, k), _u8(torch, v), k_scale=ks, v_scale=vs, fixed=fixed, num_cus=8)
    ro, rl = _oracle(b, k, v, ks, vs)
    gu.check_close(gu.as_f64(o, "bf16"), ro, "bf16", f"fp8 codes o fixed={fixed}")
    gu.check_lse(lse, rl, f"fp8 codes lse fixed={fixed}")


def test_fp8_prefill_append_hnd(torch, pkv):
    """Chunked prefill (a quarter of the prefill workload, HND, causal) over an
    fp8 cache: the new fp8 rows are appended first (byte copies), then the
    MFMA tile kernel runs 64-row tiles, expanding the fp8 tiles to bf16 in
    LDS."""
    print("case fp8 prefill", flush=True)
    b = wl.make("prefill", kv_dtype="fp8", scale=0.25, batch=4, poison=True)
    k_dev, v_dev = _u8(torch, b.k_cache), _u8(torch, b.v_cache)
    pkv.append_paged_kv(_u8(torch, b.k_new), _u8(torch, b.v_new), gu.to_dev(b.append_indptr, "i32"),
                        gu.to_dev(b.kv_indptr, "i32"), gu.to_dev(b.kv_indices, "i32"),
                        gu.to_dev(b.kv_last_page_len, "i32"), k_dev, v_dev, layout="HND", page_size=b.page_size)
    torch.cuda.synchronize()
    k_exp, v_exp = b.k_cache.copy(), b.v_cache.copy()
    targets = omd.append_targets(list(b.append_indptr), list(b.kv_indptr), list(b.kv_indices),
                                 list(b.kv_last_page_len), b.page_size)
    for t, (page, slot) in enumerate(targets):
        k_exp[page, :, slot], v_exp[page, :, slot] = b.k_new[t], b.v_new[t]
    assert np.array_equal(k_dev.cpu().numpy(), k_exp) and np.array_equal(v_dev.cpu().numpy(), v_exp)
    plan, o, lse = _run(pkv, torch, b, k_dev, v_dev, k_scale=1.0, v_scale=1.0)
    assert plan.info["rows_per_tile"] == 64
    ro, rl = _oracle(b, k_exp, v_exp, 1.0, 1.0)
    gu.check_close(gu.as_f64(o, "bf16"), ro, "bf16", "fp8 prefill o")
    gu.check_lse(lse, rl, "fp8 prefill lse")


def test_fp8_odd_page_size(torch, pkv):
    """Page size 3 (no power of two: every key located through the page table)."""
    b = wl.make("decode", kv_dtype="fp8", scale=0.1, batch=9, page_size=3, poison=True)
    _, o, lse = _run(pkv, torch, b, _u8(torch, b.k_cache), _u8(torch, b.v_cache), k_scale=0.25, v_scale=4.0)
    ro, rl = _oracle(b, b.k_cache, b.v_cache, 0.25, 4.0)
    gu.check_close(gu.as_f64(o, "bf16"), ro, "bf16", "fp8 page 3 o")
    gu.check_lse(lse, rl, "fp8 page 3 lse")


@pytest.mark.parametrize("layout,page_size,fixed,group", [
    ("NHD", 3, 0, 4),      # no power of two: every key located through the page table
    ("HND", 8, 2, 4),      # 8-key pages (one page per load instruction); forced splits
    ("NHD", 16, 1, 2),
    ("HND", 1, 0, 8),
    ("NHD", 32, 3, 1),     # 256-row tiles
])
def test_fp8_prefill_mfma_shapes(torch, pkv, layout, page_size, fixed, group):
    """Prefill over an fp8 cache on the MFMA tile kernel across page sizes,
    layouts, head groups and forced splits, with non-unit K and V scales (the
    V scale reaches split rows before their merge)."""
    print("case fp8 prefill", layout, page_size, fixed, group, flush=True)
    b = wl.make("prefill", kv_dtype="fp8", layout=layout, page_size=page_size, batch=4, qo_range=(1, 150),
                prefix_range=(0, 400), hq=2 * group, hkv=2, poison=True)
    k_dev, v_dev = _u8(torch, b.k_cache), _u8(torch, b.v_cache)
    pkv.append_paged_kv(_u8(torch, b.k_new), _u8(torch, b.v_new), gu.to_dev(b.append_indptr, "i32"),
                        gu.to_dev(b.kv_indptr, "i32"), gu.to_dev(b.kv_indices, "i32"),
                        gu.to_dev(b.kv_last_page_len, "i32"), k_dev, v_dev, layout=layout, page_size=page_size)
    torch.cuda.synchronize()
    k_exp, v_exp = k_dev.cpu().numpy(), v_dev.cpu().numpy()
    plan, o, lse = _run(pkv, torch, b, k_dev, v_dev, k_scale=0.5, v_scale=2.0, fixed=fixed, num_cus=8 if fixed else 0)
    assert plan.info["rows_per_tile"] == 256 // group
    if fixed > 1:
        assert plan.info["num_merges"] > 0
    ro, rl = _oracle(b, k_exp, v_exp, 0.5, 2.0)
    gu.check_close(gu.as_f64(o, "bf16"), ro, "bf16", "fp8 prefill o")
    gu.check_lse(lse, rl, "fp8 prefill lse")
