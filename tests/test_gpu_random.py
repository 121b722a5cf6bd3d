"""GPU parity on seeded random small batches: mode, payload and cache dtype,
head_dim, GQA group, page size (powers of two and not), layout, causal flag,
forced split size and lengths are drawn per case, so tile edges, page edges
and chunk edges fall at many offsets.  Every case is checked against the
float64 oracle; caches are NaN-poisoned outside the requests' slots."""

import math

import numpy as np
import pytest

import workloads as wl
from oracle import attention as oat
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

N_CASES = 96


def _case(i):
    rng = np.random.default_rng(9000 + i)
    mode = ["decode", "prefill"][i % 2]
    dtype, kv_dtype = [("bf16", "bf16"), ("f32", "f32"), ("bf16", "fp8")][int(rng.integers(0, 3))]
    dim = 128 if kv_dtype == "fp8" else int(rng.choice([64, 128]))
    groups = [1, 2, 4] if dtype == "f32" else [1, 2, 4, 8]
    group = int(rng.choice(groups))
    page = int(rng.choice([1, 2, 3, 5, 8, 16, 32, 64]))
    layout = str(rng.choice(["NHD", "HND"]))
    fixed = int(rng.choice([0, 0, 1, 3, 7]))
    batch = int(rng.integers(1, 7))
    seed = 7000 + i
    kw = dict(hq=2 * group, hkv=2, dim=dim, dtype=dtype, kv_dtype=kv_dtype, batch=batch, page_size=page,
              layout=layout, seed=seed, poison=True)
    if mode == "decode":
        hi = int(rng.integers(1, 400))
        b = wl.make("decode", kv_range=(1, hi), pool=batch * (hi // page + 2) + 4, **kw)
    else:
        qhi = int(rng.integers(1, 90))
        phi = int(rng.integers(0, 300))
        causal = bool(rng.integers(0, 2))
        b = wl.make("prefill", qo_range=(1, qhi), prefix_range=(0, phi), causal=causal, **kw)
    return b, fixed


@pytest.fixture(scope="module")
def torch():
    return gu.require_gpu()


@pytest.fixture(scope="module")
def pkv(torch):
    import paged_kv_cache_plan_amd as pkv
    return pkv


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_batch(torch, pkv, i):
    b, fixed = _case(i)
    waves = 1 if b.mode == "decode" and i % 2 else 0   # odd decode cases: one-wave row workgroups
    print(f"case random {i}: {b.mode} {b.dtype}/{b.kv_dtype} d{b.head_dim} g{b.num_qo_heads // 2} page {b.page_size} "
          f"{b.layout} causal={b.causal} fixed={fixed} waves={waves} qo={list(b.qo_lens)} kv={list(b.kv_lens)}",
          flush=True)
    fp8 = b.kv_dtype == "fp8"
    to_kv = (lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()) if fp8 else (lambda x: gu.to_dev(x, b.dtype))
    k_dev, v_dev = to_kv(b.k_cache), to_kv(b.v_cache)
    if b.mode == "prefill":   # the new rows go into their slots first
        pkv.append_paged_kv(to_kv(b.k_new), to_kv(b.v_new), gu.to_dev(b.append_indptr, "i32"),
                            gu.to_dev(b.kv_indptr, "i32"), gu.to_dev(b.kv_indices, "i32"),
                            gu.to_dev(b.kv_last_page_len, "i32"), k_dev, v_dev, layout=b.layout,
                            page_size=b.page_size)
        torch.cuda.synchronize()
    k_host = k_dev.cpu().numpy() if fp8 else gu.to_host(k_dev, b.dtype)
    v_host = v_dev.cpu().numpy() if fp8 else gu.to_host(v_dev, b.dtype)
    params = pkv.plan_params(mode=b.mode, batch_size=b.batch_size, num_qo_heads=b.num_qo_heads, num_kv_heads=2,
                             head_dim_qk=b.head_dim, page_size=b.page_size, causal=b.causal, dtype=b.dtype,
                             kv_dtype=b.kv_dtype, fixed_split_pages=fixed, num_cus=8 if fixed else 0,
                             max_num_pages=b.max_num_pages, row_waves=waves)
    plan = pkv.Plan(params, qo_indptr=b.qo_indptr if b.mode == "prefill" else None, kv_indptr=b.kv_indptr,
                    kv_indices=b.kv_indices, kv_last_page_len=b.kv_last_page_len)
    assert plan.info["row_waves"] == waves if waves else plan.info["row_waves"] in (1, 4)
    q = gu.to_dev(b.q, b.dtype)
    out = gu.empty_like_out(q.shape, b.dtype)
    lse = torch.full((q.shape[0], b.num_qo_heads), float("nan"), dtype=torch.float32, device="cuda")
    ks, vs = (0.75, 1.5) if fp8 else (1.0, 1.0)
    plan.run(q, k_dev, v_dev, gu.to_dev(b.kv_indices, "i32"), out, lse, layout=b.layout, sm_scale=b.sm_scale,
             k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    ro, rl = oat.paged_attention(b.q, k_host, v_host, qo_indptr=list(b.qo_indptr), kv_indptr=list(b.kv_indptr),
                                 kv_indices=list(b.kv_indices), kv_last_page_len=list(b.kv_last_page_len),
                                 page_size=b.page_size, layout=b.layout, num_kv_heads=2, causal=b.causal,
                                 sm_scale=b.sm_scale, q_dtype=b.dtype, kv_dtype=b.kv_dtype, k_scale=ks, v_scale=vs)
    got = gu.to_host(out, b.dtype)
    gu.check_close(gu.as_f64(got, "bf16") if b.dtype == "bf16" else got, ro, b.dtype, f"random {i} o")
    gu.check_lse(lse.cpu().numpy(), rl, f"random {i} lse", atol=1e-5 if b.dtype == "f32" else 1e-3)


N_MLA_CASES = 24


def _mla_case(i):
    rng = np.random.default_rng(9500 + i)
    page = int(rng.choice([1, 3, 8, 16, 32, 64, 128]))
    batch = int(rng.integers(1, 9))
    hi = int(rng.integers(1, 600))
    heads = int(rng.choice([64, 128]))
    fixed = int(rng.choice([0, 0, 1, 2, 5]))
    b = wl.make("mla", page_size=page, batch=batch, kv_range=(1, hi), heads=heads, seed=8500 + i, poison=True)
    return b, fixed


@pytest.mark.parametrize("i", range(N_MLA_CASES))
def test_random_mla_batch(torch, pkv, i):
    b, fixed = _mla_case(i)
    heads = b.num_qo_heads
    print(f"case random mla {i}: page {b.page_size} heads {heads} fixed={fixed} kv={list(b.kv_lens)}", flush=True)
    cache = gu.to_dev(b.k_cache, "bf16")
    params = pkv.plan_params(mode="mla", batch_size=b.batch_size, num_qo_heads=heads, num_kv_heads=1,
                             head_dim_qk=576, head_dim_vo=512, page_size=b.page_size, dtype="bf16",
                             fixed_split_pages=fixed, num_cus=16 if fixed else 0, max_num_pages=b.max_num_pages)
    plan = pkv.Plan(params, kv_indptr=b.kv_indptr, kv_indices=b.kv_indices, kv_last_page_len=b.kv_last_page_len)
    out = gu.empty_like_out((b.batch_size, heads, 512), "bf16")
    lse = torch.full((b.batch_size, heads), float("nan"), dtype=torch.float32, device="cuda")
    plan.run_mla(gu.to_dev(b.q, "bf16"), gu.to_dev(b.q_kpe, "bf16"), cache[..., :512], cache[..., 512:],
                 gu.to_dev(b.kv_indices, "i32"), out, lse, sm_scale=b.sm_scale)
    torch.cuda.synchronize()
    ro, rl = oat.mla_decode(b.q, b.q_kpe, b.k_cache[..., :512], b.k_cache[..., 512:], kv_indptr=list(b.kv_indptr),
                            kv_indices=list(b.kv_indices), kv_last_page_len=list(b.kv_last_page_len),
                            page_size=b.page_size, sm_scale=b.sm_scale, dtype="bf16")
    gu.check_close(gu.as_f64(gu.to_host(out, "bf16"), "bf16"), ro, "bf16", f"random mla {i} o")
    gu.check_lse(lse.cpu().numpy(), rl, f"random mla {i} lse")


N_CASCADE_CASES = 16


def _partition(rng, parts):
    """Random refinement of a list of group sizes: every group splits into 1..3 consecutive groups."""
    out = []
    for n in parts:
        k = int(rng.integers(1, min(3, n) + 1))
        cuts = sorted(rng.choice(np.arange(1, n), size=k - 1, replace=False).tolist()) if k > 1 else []
        edges = [0] + cuts + [n]
        out += [edges[j + 1] - edges[j] for j in range(k)]
    return out


def _cascade_case(i):
    rng = np.random.default_rng(9800 + i)
    batch = int(rng.integers(2, 11))
    depth = int(rng.integers(2, 5))
    tree = [[batch]]
    for _ in range(depth - 2):
        tree.append(_partition(rng, tree[-1]))
    tree.append([1] * batch)
    level_kv = [(int(lo), int(lo + rng.integers(0, 60))) for lo in rng.integers(1, 80, size=depth)]
    bf16 = bool(rng.integers(0, 2))
    kw = dict(tree=tree, level_kv=level_kv, qo_range=(1, int(rng.integers(1, 6))),
              page_size=int(rng.choice([1, 4, 16])), layout=str(rng.choice(["NHD", "HND"])),
              causal=bool(rng.integers(0, 2)), seed=8800 + i, poison=True)
    if bf16:
        kw.update(hq=8, hkv=2, dim=128, dtype="bf16")
    b = wl.make("cascade_small", **kw)
    return b, int(rng.choice([0, 0, 1, 3]))


@pytest.mark.parametrize("i", range(N_CASCADE_CASES))
def test_random_cascade(torch, pkv, i):
    from oracle import cascade as occ
    from oracle import metadata as omd
    b, fixed = _cascade_case(i)
    levels = b.extra["levels"]
    print(f"case random cascade {i}: {b.dtype} page {b.page_size} {b.layout} causal={b.causal} fixed={fixed} "
          f"tree={[len(lv['kv_lens']) for lv in levels]} qo={list(b.qo_lens)}", flush=True)
    k_dev, v_dev = gu.to_dev(b.k_cache, b.dtype), gu.to_dev(b.v_cache, b.dtype)
    pkv.append_paged_kv(gu.to_dev(b.k_new, b.dtype), gu.to_dev(b.v_new, b.dtype), gu.to_dev(b.append_indptr, "i32"),
                        gu.to_dev(b.kv_indptr, "i32"), gu.to_dev(b.kv_indices, "i32"),
                        gu.to_dev(b.kv_last_page_len, "i32"), k_dev, v_dev, layout=b.layout, page_size=b.page_size)
    torch.cuda.synchronize()
    k_host, v_host = gu.to_host(k_dev, b.dtype), gu.to_host(v_dev, b.dtype)
    params = pkv.plan_params(mode="prefill", batch_size=0, num_qo_heads=b.num_qo_heads, num_kv_heads=b.num_kv_heads,
                             head_dim_qk=b.head_dim, page_size=b.page_size, causal=b.causal, dtype=b.dtype,
                             num_cus=8 if fixed else 0, fixed_split_pages=fixed, max_num_pages=k_dev.shape[0])
    plan = pkv.CascadePlan(params, levels)
    q = gu.to_dev(b.q, b.dtype)
    out = gu.empty_like_out(q.shape, b.dtype)
    lse = torch.full((q.shape[0], b.num_qo_heads), float("nan"), dtype=torch.float32, device="cuda")
    idx = gu.to_dev(np.concatenate([lv["kv_indices"][:lv["kv_indptr"][-1]] for lv in levels]), "i32")
    plan.run(q, k_dev, v_dev, idx, out, lse, layout=b.layout, sm_scale=b.sm_scale)
    torch.cuda.synchronize()
    ro, rl = occ.cascade_attention(b.q, k_host, v_host, levels=levels, page_size=b.page_size, layout=b.layout,
                                   num_kv_heads=b.num_kv_heads, causal=b.causal, sm_scale=b.sm_scale,
                                   q_dtype=b.dtype, kv_dtype=b.dtype)
    got = gu.to_host(out, b.dtype)
    gu.check_close(gu.as_f64(got, "bf16") if b.dtype == "bf16" else got, ro, b.dtype, f"random cascade {i} o")
    gu.check_lse(lse.cpu().numpy(), rl, f"random cascade {i} lse", atol=1e-5 if b.dtype == "f32" else 1e-3)
