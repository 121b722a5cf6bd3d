"""GPU parity: the HIP path (through the C ABI) against the float64 oracle on
the same seeded inputs.  Caches are NaN-poisoned wherever no request owns a
slot, so a read of a tail, a free page or a not-yet-appended slot shows up as
a non-finite output."""

import math

import numpy as np
import pytest

import workloads as wl
from oracle import attention as oat
from oracle import merge as omg
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


def _expected_after_append(b, k_host, v_host):
    """Host copy of the cache after the append (placement from the oracle's slot map)."""
    k_exp, v_exp = k_host.copy(), v_host.copy()
    targets = omd.append_targets(list(b.append_indptr), list(b.kv_indptr), list(b.kv_indices),
                                 list(b.kv_last_page_len), b.page_size)
    for t, (page, slot) in enumerate(targets):
        if b.layout == "NHD":
            k_exp[page, slot], v_exp[page, slot] = b.k_new[t], b.v_new[t]
        else:
            k_exp[page, :, slot], v_exp[page, :, slot] = b.k_new[t], b.v_new[t]
    return k_exp, v_exp


def _run_gqa(pkv, torch, b, *, k_cache, v_cache, mode=None, fixed_split_pages=0, num_cus=0, layout=None,
             q_dev=None):
    mode = mode or b.mode
    layout = layout or b.layout
    params = pkv.plan_params(mode=mode, batch_size=b.batch_size, num_qo_heads=b.num_qo_heads,
                             num_kv_heads=b.num_kv_heads, head_dim_qk=b.head_dim, page_size=b.page_size,
                             causal=b.causal, dtype=b.dtype, num_cus=num_cus, fixed_split_pages=fixed_split_pages,
                             max_num_pages=k_cache.shape[0])
    plan = pkv.Plan(params, qo_indptr=b.qo_indptr if mode == "prefill" else None, kv_indptr=b.kv_indptr,
                    kv_indices=b.kv_indices, kv_last_page_len=b.kv_last_page_len)
    q = gu.to_dev(b.q, b.dtype) if q_dev is None else q_dev
    out = gu.empty_like_out(q.shape, b.dtype)
    lse = torch.full((q.shape[0], b.num_qo_heads), float("nan"), dtype=torch.float32, device="cuda")
    plan.run(q, k_cache, v_cache, gu.to_dev(b.kv_indices, "i32"), out, lse, layout=layout, sm_scale=b.sm_scale)
    torch.cuda.synchronize()
    return plan, gu.to_host(out, b.dtype), lse.cpu().numpy()


def _oracle(b, k_host, v_host, **kw):
    return oat.paged_attention(b.q, k_host, v_host, qo_indptr=list(b.qo_indptr), kv_indptr=list(b.kv_indptr),
                               kv_indices=list(b.kv_indices), kv_last_page_len=list(b.kv_last_page_len),
                               page_size=b.page_size, layout=b.layout, num_kv_heads=b.num_kv_heads,
                               causal=b.causal, sm_scale=b.sm_scale, q_dtype=b.dtype, kv_dtype=b.dtype, **kw)


def _append_on_gpu(pkv, b, k_dev, v_dev):
    pkv.append_paged_kv(gu.to_dev(b.k_new, b.dtype), gu.to_dev(b.v_new, b.dtype), gu.to_dev(b.append_indptr, "i32"),
                        gu.to_dev(b.kv_indptr, "i32"), gu.to_dev(b.kv_indices, "i32"),
                        gu.to_dev(b.kv_last_page_len, "i32"), k_dev, v_dev, layout=b.layout, page_size=b.page_size)


@pytest.mark.parametrize("literal", [True, False])
def test_worked_example_append_then_prefill_f32(torch, pkv, literal):
    """The pages' three-request batch (qo 3/1/4, kv 6/2/9, page 4), float32:
    append the 8 new tokens, then causal prefill; max-abs error <= 1e-5."""
    b = wl.make("worked", literal_pages=literal, poison=True)
    k_dev, v_dev = gu.to_dev(b.k_cache, "f32"), gu.to_dev(b.v_cache, "f32")
    _append_on_gpu(pkv, b, k_dev, v_dev)
    torch.cuda.synchronize()
    k_exp, v_exp = _expected_after_append(b, b.k_cache, b.v_cache)
    assert np.array_equal(gu.to_host(k_dev, "f32").view(np.uint32), k_exp.view(np.uint32))
    assert np.array_equal(gu.to_host(v_dev, "f32").view(np.uint32), v_exp.view(np.uint32))
    plan, o, lse = _run_gqa(pkv, torch, b, k_cache=k_dev, v_cache=v_dev)
    ro, rl = _oracle(b, k_exp, v_exp)
    gu.check_close(o, ro, "f32", "worked o")
    gu.check_lse(lse, rl, "worked lse", atol=1e-5)


@pytest.mark.parametrize("fixed", [0, 1, 2])
def test_worked_example_forced_splits(torch, pkv, fixed):
    """Same batch with the keys forced into 1- and 2-page chunks (split + merge)."""
    b = wl.make("worked", literal_pages=True, poison=True)
    k_exp, v_exp = _expected_after_append(b, b.k_cache, b.v_cache)
    plan, o, lse = _run_gqa(pkv, torch, b, k_cache=gu.to_dev(k_exp, "f32"), v_cache=gu.to_dev(v_exp, "f32"),
                            fixed_split_pages=fixed, num_cus=4)
    if fixed:
        assert plan.info["split"] == 1
    ro, rl = _oracle(b, k_exp, v_exp)
    gu.check_close(o, ro, "f32", "split o")
    gu.check_lse(lse, rl, "split lse", atol=1e-5)


def test_decode_full_size(torch, pkv):
    """64 requests, kv U[512, 4096], page 16, 20k-page pool, 32/8 heads, bf16 NHD."""
    b = wl.make("decode", poison=True)
    k_dev, v_dev = gu.to_dev(b.k_cache, "bf16"), gu.to_dev(b.v_cache, "bf16")
    plan, o, lse = _run_gqa(pkv, torch, b, k_cache=k_dev, v_cache=v_dev)
    ro, rl = _oracle(b, b.k_cache, b.v_cache)
    rep = gu.check_close(gu.as_f64(o, "bf16"), ro, "bf16", "decode o")
    gu.check_lse(lse, rl, "decode lse")
    grd = gu.check_guard(gu.as_f64(o, "bf16"), ro, lse, rl, "decode")
    print("decode parity", rep, grd, plan.info["num_items"], plan.info["split"])


@pytest.mark.parametrize("fixed", [1, 2, 7])
def test_decode_forced_split_matches_unsplit(torch, pkv, fixed):
    b = wl.make("decode", scale=0.25, poison=True, batch=12)
    k_dev, v_dev = gu.to_dev(b.k_cache, "bf16"), gu.to_dev(b.v_cache, "bf16")
    plan, o, lse = _run_gqa(pkv, torch, b, k_cache=k_dev, v_cache=v_dev, fixed_split_pages=fixed)
    assert plan.info["split"] == 1
    ro, rl = _oracle(b, b.k_cache, b.v_cache)
    gu.check_close(gu.as_f64(o, "bf16"), ro, "bf16", "split decode o")
    gu.check_lse(lse, rl, "split decode lse")


def test_skewed_decode_split_and_merge(torch, pkv):
    """One 32k-token request among 15 short ones, page size 1: the planner
    splits the long history and the merge kernel recombines it."""
    b = wl.make("skewed", poison=True)
    k_dev, v_dev = gu.to_dev(b.k_cache, "bf16"), gu.to_dev(b.v_cache, "bf16")
    plan, o, lse = _run_gqa(pkv, torch, b, k_cache=k_dev, v_cache=v_dev)
    assert plan.info["split"] == 1 and plan.info["num_merges"] >= 1
    ro, rl = _oracle(b, b.k_cache, b.v_cache)
    gu.check_close(gu.as_f64(o, "bf16"), ro, "bf16", "skewed o")
    gu.check_lse(lse, rl, "skewed lse")
    print("skewed guard", gu.check_guard(gu.as_f64(o, "bf16"), ro, lse, rl, "skewed"))


@pytest.mark.parametrize("fixed", [100, 30, 10])
@pytest.mark.parametrize("dtype,dim", [("bf16", 128), ("f32", 64)])
def test_split_merge_chunk_counts(torch, pkv, fixed, dtype, dim):
    """A 4000-token request among short ones (page 1) split into about 40,
    130 and 400 chunks: the merge's one-wave path (up to 64 chunks), its
    prefetching block path (up to 256) and its segmented block path."""
    print("case merge chunks", fixed, dtype, dim, flush=True)
    b = wl.make("skewed", poison=True, long_len=4000, kv_range=(20, 300), dtype=dtype, dim=dim)
    k_dev, v_dev = gu.to_dev(b.k_cache, dtype), gu.to_dev(b.v_cache, dtype)
    plan, o, lse = _run_gqa(pkv, torch, b, k_cache=k_dev, v_cache=v_dev, fixed_split_pages=fixed, num_cus=64)
    assert plan.info["num_merges"] >= 1
    ro, rl = _oracle(b, b.k_cache, b.v_cache)
    got = gu.as_f64(o, "bf16") if dtype == "bf16" else o
    gu.check_close(got, ro, dtype, f"merge chunks {fixed} o")
    gu.check_lse(lse, rl, f"merge chunks {fixed} lse", atol=1e-5 if dtype == "f32" else 1e-3)


@pytest.fixture(scope="module")
def prefill_full():
    """The full-size prefill batch, its cache after the append (host), and the
    oracle over every query head, computed once for the module (one thread per
    kv head's 4 query heads)."""
    b = wl.make("prefill", poison=True)
    k_exp, v_exp = _expected_after_append(b, b.k_cache, b.v_cache)
    print("prefill oracle: 32 heads in threads", flush=True)
    ro, rl = gu.oracle_in_threads(lambda heads: _oracle(b, k_exp, v_exp, heads=heads),
                                  [list(range(g * 4, g * 4 + 4)) for g in range(8)])
    assert not np.isnan(ro).any() and not np.isnan(rl).any()
    return b, k_exp, v_exp, ro, rl


def test_prefill_full_size_append_then_run(torch, pkv, prefill_full):
    """8 requests, 512-2048 new rows after a 0-8192 prefix, page 16, HND,
    causal, bf16: append (bit-exact) then prefill, every output element and
    LSE against the oracle, plus the regression guard."""
    b, k_exp, v_exp, ro, rl = prefill_full
    k_dev, v_dev = gu.to_dev(b.k_cache, "bf16"), gu.to_dev(b.v_cache, "bf16")
    _append_on_gpu(pkv, b, k_dev, v_dev)
    torch.cuda.synchronize()
    assert np.array_equal(gu.to_host(k_dev, "bf16"), k_exp)
    assert np.array_equal(gu.to_host(v_dev, "bf16"), v_exp)
    plan, o, lse = _run_gqa(pkv, torch, b, k_cache=k_dev, v_cache=v_dev)
    got = gu.as_f64(o, "bf16")
    rep = gu.check_close(got, ro, "bf16", "prefill o")
    gu.check_lse(lse, rl, "prefill lse")
    grd = gu.check_guard(got, ro, lse, rl, "prefill")
    assert rep["n"] == b.nnz * b.num_qo_heads * b.head_dim
    print("prefill parity", rep, grd)


@pytest.mark.parametrize("fixed", [4, 12, 64])
def test_prefill_forced_chunk_lengths(torch, pkv, prefill_full, fixed):
    """The full-size prefill batch split into chunks of 4, 12 and 64 pages
    (1, 3 and 16 key tiles): every tile pipeline depth, each chunk's partial
    last tile, and the merge of up to ~40 partial states per row.  Every head
    against the oracle; the guard's LSE bound catches a stale or missing key
    tile that the output tolerance alone can miss."""
    print("case prefill forced chunk", fixed, flush=True)
    b, k_exp, v_exp, ro, rl = prefill_full
    plan, o, lse = _run_gqa(pkv, torch, b, k_cache=gu.to_dev(k_exp, "bf16"), v_cache=gu.to_dev(v_exp, "bf16"),
                            fixed_split_pages=fixed)
    got = gu.as_f64(o, "bf16")
    gu.check_close(got, ro, "bf16", f"prefill o fixed={fixed}")
    gu.check_lse(lse, rl, f"prefill lse fixed={fixed}")
    grd = gu.check_guard(got, ro, lse, rl, f"prefill fixed={fixed}")
    assert plan.info["num_merges"] > 0
    print("prefill forced chunk guard", fixed, grd)


def test_mla_decode_full_size(torch, pkv):
    """32 requests, kv U[1024, 8192], page 64, latent cache [pages, 64, 576],
    128 heads, sm_scale 1/sqrt(576)."""
    b = wl.make("mla", poison=True)
    cache = gu.to_dev(b.k_cache, "bf16")
    params = pkv.plan_params(mode="mla", batch_size=b.batch_size, num_qo_heads=128, num_kv_heads=1,
                             head_dim_qk=576, head_dim_vo=512, page_size=b.page_size, dtype="bf16",
                             max_num_pages=b.max_num_pages)
    plan = pkv.Plan(params, kv_indptr=b.kv_indptr, kv_indices=b.kv_indices, kv_last_page_len=b.kv_last_page_len)
    out = gu.empty_like_out((b.batch_size, 128, 512), "bf16")
    lse = torch.full((b.batch_size, 128), float("nan"), dtype=torch.float32, device="cuda")
    plan.run_mla(gu.to_dev(b.q, "bf16"), gu.to_dev(b.q_kpe, "bf16"), cache[..., :512], cache[..., 512:],
                 gu.to_dev(b.kv_indices, "i32"), out, lse, sm_scale=b.sm_scale)
    torch.cuda.synchronize()
    ro, rl = oat.mla_decode(b.q, b.q_kpe, b.k_cache[..., :512], b.k_cache[..., 512:], kv_indptr=list(b.kv_indptr),
                            kv_indices=list(b.kv_indices), kv_last_page_len=list(b.kv_last_page_len),
                            page_size=b.page_size, sm_scale=b.sm_scale, dtype="bf16")
    got = gu.as_f64(gu.to_host(out, "bf16"), "bf16")
    rep = gu.check_close(got, ro, "bf16", "mla o")
    gu.check_lse(lse.cpu().numpy(), rl, "mla lse")
    grd = gu.check_guard(got, ro, lse.cpu().numpy(), rl, "mla")
    print("mla parity", rep, grd, plan.info)


@pytest.mark.parametrize("page_size,kv_range,batch,fixed,heads", [
    (1, (1, 200), 6, 0, 128),      # one key per page: every key located through the page table
    (3, (5, 300), 5, 7, 128),      # no power of two; forced 21-token chunks end inside tiles
    (16, (30, 700), 4, 5, 64),     # pages shorter than a tile; one head group
    (64, (1, 40), 9, 0, 128),      # requests shorter than one tile
    (64, (32, 32), 3, 1, 128),     # exactly one tile per request; one-page chunks
])
def test_mla_decode_page_shapes_and_splits(torch, pkv, page_size, kv_range, batch, fixed, heads):
    """MLA decode on small batches whose pages, chunk ends and lengths cut the
    key tiles at every offset (NaN-poisoned caches)."""
    print("case mla shapes", page_size, kv_range, batch, fixed, heads, flush=True)
    b = wl.make("mla", poison=True, page_size=page_size, kv_range=kv_range, batch=batch, heads=heads)
    cache = gu.to_dev(b.k_cache, "bf16")
    params = pkv.plan_params(mode="mla", batch_size=b.batch_size, num_qo_heads=heads, num_kv_heads=1,
                             head_dim_qk=576, head_dim_vo=512, page_size=page_size, dtype="bf16",
                             fixed_split_pages=fixed, num_cus=16 if fixed else 0, max_num_pages=b.max_num_pages)
    plan = pkv.Plan(params, kv_indptr=b.kv_indptr, kv_indices=b.kv_indices, kv_last_page_len=b.kv_last_page_len)
    out = gu.empty_like_out((b.batch_size, heads, 512), "bf16")
    lse = torch.full((b.batch_size, heads), float("nan"), dtype=torch.float32, device="cuda")
    plan.run_mla(gu.to_dev(b.q, "bf16"), gu.to_dev(b.q_kpe, "bf16"), cache[..., :512], cache[..., 512:],
                 gu.to_dev(b.kv_indices, "i32"), out, lse, sm_scale=b.sm_scale)
    torch.cuda.synchronize()
    ro, rl = oat.mla_decode(b.q, b.q_kpe, b.k_cache[..., :512], b.k_cache[..., 512:], kv_indptr=list(b.kv_indptr),
                            kv_indices=list(b.kv_indices), kv_last_page_len=list(b.kv_last_page_len),
                            page_size=page_size, sm_scale=b.sm_scale, dtype="bf16")
    gu.check_close(gu.as_f64(gu.to_host(out, "bf16"), "bf16"), ro, "bf16", "mla o")
    gu.check_lse(lse.cpu().numpy(), rl, "mla lse")
    if fixed > 1:
        assert plan.info["num_merges"] > 0


@pytest.mark.parametrize("heads", [128, 64])
def test_mla_decode_score_jump_past_the_first_tile(torch, pkv, heads):
    """A key far into a chunk whose score for some heads exceeds the max of
    the chunk's first tile by far more than the weights may grow (a latent row
    equal to 4x one head's query: a score gap of about 96 for that head), so
    the kernel's second pass with the chunk's largest max runs."""
    print("case mla score jump", heads, flush=True)
    b = wl.make("mla", poison=True, page_size=16, kv_range=(150, 400), batch=3, heads=heads)
    lat = gu.as_f64(b.k_cache, "bf16").astype(np.float32)
    q = gu.as_f64(b.q, "bf16").astype(np.float32)
    qk = gu.as_f64(b.q_kpe, "bf16").astype(np.float32)
    # chunks of 64 keys, tiles of 32: keys 100 and 300 sit in a chunk's second
    # tile (the second pass runs), 140 and 7 in a first tile (it need not)
    for r, j, h in [(0, 100, 0), (0, 300, heads // 2), (1, 140, heads - 1), (2, 7, 5)]:
        page, slot = omd.token_address(list(b.kv_indptr), list(b.kv_indices), b.page_size, r, j)
        lat[page, slot, :512] = 4 * q[r, h]
        lat[page, slot, 512:] = 4 * qk[r, h]
    b.k_cache = wl.to_bf16_bits(lat)
    cache = gu.to_dev(b.k_cache, "bf16")
    params = pkv.plan_params(mode="mla", batch_size=b.batch_size, num_qo_heads=heads, num_kv_heads=1,
                             head_dim_qk=576, head_dim_vo=512, page_size=b.page_size, dtype="bf16",
                             fixed_split_pages=4, num_cus=16, max_num_pages=b.max_num_pages)
    plan = pkv.Plan(params, kv_indptr=b.kv_indptr, kv_indices=b.kv_indices, kv_last_page_len=b.kv_last_page_len)
    out = gu.empty_like_out((b.batch_size, heads, 512), "bf16")
    lse = torch.full((b.batch_size, heads), float("nan"), dtype=torch.float32, device="cuda")
    plan.run_mla(gu.to_dev(b.q, "bf16"), gu.to_dev(b.q_kpe, "bf16"), cache[..., :512], cache[..., 512:],
                 gu.to_dev(b.kv_indices, "i32"), out, lse, sm_scale=b.sm_scale)
    torch.cuda.synchronize()
    ro, rl = oat.mla_decode(b.q, b.q_kpe, b.k_cache[..., :512], b.k_cache[..., 512:], kv_indptr=list(b.kv_indptr),
                            kv_indices=list(b.kv_indices), kv_last_page_len=list(b.kv_last_page_len),
                            page_size=b.page_size, sm_scale=b.sm_scale, dtype="bf16")
    got = gu.as_f64(gu.to_host(out, "bf16"), "bf16")
    gu.check_close(got, ro, "bf16", "mla jump o")
    gu.check_lse(lse.cpu().numpy(), rl, "mla jump lse")
    gu.check_guard(got, ro, lse.cpu().numpy(), rl, "mla jump")
    assert plan.info["num_merges"] > 0
    # the planted keys dominate their heads: those rows are (nearly) 4 q
    assert rl[0, 0] > np.median(rl[0]) + 20


def test_layouts_page_sizes_and_storage_forms_agree(torch, pkv):
    """The same logical decode batch stored NHD and HND, at page sizes 1, 3
    and 16, and as a 5-D [pages, 2, ...] tensor: each matches the oracle."""
    base = wl.make("decode", scale=0.05, batch=6)
    lens = base.kv_lens
    rng = np.random.default_rng(77)
    seq_k = [rng.standard_normal((n, 8, 128)).astype(np.float32) for n in lens]
    seq_v = [rng.standard_normal((n, 8, 128)).astype(np.float32) for n in lens]
    q = wl.to_bf16_bits(rng.standard_normal((len(lens), 32, 128)).astype(np.float32))
    ref = None
    for page_size in (1, 3, 16):
        for layout in ("NHD", "HND"):
            n_pages = [math.ceil(n / page_size) for n in lens]
            pool = sum(n_pages) + 5
            perm = rng.permutation(pool).astype(np.int32)
            kv_indptr = np.array([0] + list(np.cumsum(n_pages)), dtype=np.int32)
            kv_indices = perm[:sum(n_pages)]
            last = np.array([n - (m - 1) * page_size for n, m in zip(lens, n_pages)], dtype=np.int32)
            shape = (pool, page_size, 8, 128) if layout == "NHD" else (pool, 8, page_size, 128)
            kc = np.full(shape, wl.BF16_NAN, dtype=np.uint16)
            vc = np.full(shape, wl.BF16_NAN, dtype=np.uint16)
            for bi, n in enumerate(lens):
                for j in range(n):
                    page, slot = omd.token_address(list(kv_indptr), list(kv_indices), page_size, bi, j)
                    if layout == "NHD":
                        kc[page, slot], vc[page, slot] = wl.to_bf16_bits(seq_k[bi][j]), wl.to_bf16_bits(seq_v[bi][j])
                    else:
                        kc[page, :, slot], vc[page, :, slot] = wl.to_bf16_bits(seq_k[bi][j]), wl.to_bf16_bits(seq_v[bi][j])
            b = wl.Batch(name="x", mode="decode", dtype="bf16", layout=layout, page_size=page_size, num_qo_heads=32,
                         num_kv_heads=8, head_dim=128, causal=True, sm_scale=1 / math.sqrt(128), qo_lens=[1] * len(lens),
                         kv_lens=lens, qo_indptr=np.arange(len(lens) + 1, dtype=np.int32), kv_indptr=kv_indptr,
                         kv_indices=kv_indices, kv_last_page_len=last, max_num_pages=pool, q=q, k_cache=kc, v_cache=vc)
            forms = ["tuple", "single"] if page_size == 16 else ["tuple"]
            for form in forms:
                if form == "tuple":
                    k_dev, v_dev = gu.to_dev(kc, "bf16"), gu.to_dev(vc, "bf16")
                else:
                    both = torch.stack([gu.to_dev(kc, "bf16"), gu.to_dev(vc, "bf16")], dim=1)
                    k_dev, v_dev = both[:, 0], both[:, 1]
                _, o, lse = _run_gqa(pkv, torch, b, k_cache=k_dev, v_cache=v_dev)
                if ref is None:
                    ref = _oracle(b, kc, vc)
                gu.check_close(gu.as_f64(o, "bf16"), ref[0], "bf16", f"{layout} P={page_size} {form}")
                gu.check_lse(lse, ref[1], f"{layout} P={page_size} {form} lse")


def test_prefill_edge_cases(torch, pkv):
    """An empty request (qo_len 0), a one-token history, a non-power-of-two
    page size and non-causal attention, with forced splits."""
    rng = np.random.default_rng(5)
    qo_lens, kv_lens, page_size = [5, 0, 1, 37], [9, 4, 1, 80], 3
    for causal in (True, False):
        for fixed in (0, 1, 4):
            n_pages = [math.ceil(n / page_size) for n in kv_lens]
            pool = sum(n_pages) + 2
            perm = rng.permutation(pool).astype(np.int32)
            kv_indptr = np.array([0] + list(np.cumsum(n_pages)), dtype=np.int32)
            last = np.array([n - (m - 1) * page_size for n, m in zip(kv_lens, n_pages)], dtype=np.int32)
            qo_indptr = np.array([0] + list(np.cumsum(qo_lens)), dtype=np.int32)
            kc = wl.to_bf16_bits(rng.standard_normal((pool, page_size, 2, 128)).astype(np.float32))
            vc = wl.to_bf16_bits(rng.standard_normal((pool, page_size, 2, 128)).astype(np.float32))
            q = wl.to_bf16_bits(rng.standard_normal((int(qo_indptr[-1]), 8, 128)).astype(np.float32))
            b = wl.Batch(name="edge", mode="prefill", dtype="bf16", layout="NHD", page_size=page_size, num_qo_heads=8,
                         num_kv_heads=2, head_dim=128, causal=causal, sm_scale=0.1, qo_lens=qo_lens, kv_lens=kv_lens,
                         qo_indptr=qo_indptr, kv_indptr=kv_indptr, kv_indices=perm[:kv_indptr[-1]],
                         kv_last_page_len=last, max_num_pages=pool, q=q, k_cache=kc, v_cache=vc)
            _, o, lse = _run_gqa(pkv, torch, b, k_cache=gu.to_dev(kc, "bf16"), v_cache=gu.to_dev(vc, "bf16"),
                                 fixed_split_pages=fixed, num_cus=2)
            ro, rl = _oracle(b, kc, vc)
            gu.check_close(gu.as_f64(o, "bf16"), ro, "bf16", f"edge causal={causal} fixed={fixed}")
            gu.check_lse(lse, rl, f"edge lse causal={causal} fixed={fixed}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_merge_state_kernels(torch, pkv, dtype):
    """pkv_merge_state / pkv_merge_states against the oracle merge, including
    empty (-inf) states on either side, both sides, and in-place output."""
    rng = np.random.default_rng(12)
    n, h, d, k = 37, 5, 96, 6
    v = rng.standard_normal((n, k, h, d)).astype(np.float32)
    s = rng.uniform(-40, 40, (n, k, h)).astype(np.float32)
    empty = rng.random((n, k, h)) < 0.2
    s[empty] = -np.inf
    v[empty] = 0.0
    s[0, :, 0] = -np.inf
    v[0, :, 0] = 0.0
    if dtype == "bf16":
        v_store = wl.to_bf16_bits(v)
        v64 = gu.as_f64(v_store, "bf16")
    else:
        v_store, v64 = v, v.astype(np.float64)
    want_v, want_s = omg.merge_states(v64, s.astype(np.float64))
    vd = gu.to_dev(v_store, dtype)
    sd = torch.from_numpy(s).cuda()
    got_v, got_s = pkv.merge_states(vd, sd)
    torch.cuda.synchronize()
    gu.check_close(gu.as_f64(gu.to_host(got_v, dtype), dtype), want_v, dtype, "merge_states")
    gu.check_lse(got_s.cpu().numpy(), want_s, "merge_states lse", atol=1e-5)
    # pairwise, written in place over the first operand
    wa, wsa = omg.merge_state_arrays(v64[:, 0], s[:, 0].astype(np.float64), v64[:, 1], s[:, 1].astype(np.float64))
    va = vd[:, 0].contiguous()
    sa = sd[:, 0].contiguous()
    pkv.merge_state(va, sa, vd[:, 1].contiguous(), sd[:, 1].contiguous(), v_out=va, s_out=sa)
    torch.cuda.synchronize()
    gu.check_close(gu.as_f64(gu.to_host(va, dtype), dtype), wa, dtype, "merge_state in place")
    gu.check_lse(sa.cpu().numpy(), wsa, "merge_state lse", atol=1e-5)


def test_stale_plan_and_int64_rejection(torch, pkv):
    b = wl.make("worked", literal_pages=True)
    params = pkv.plan_params(mode="prefill", batch_size=3, num_qo_heads=4, num_kv_heads=2, head_dim_qk=64,
                             page_size=4, dtype="f32", max_num_pages=16)
    plan = pkv.Plan(params, qo_indptr=b.qo_indptr, kv_indptr=b.kv_indptr, kv_indices=b.kv_indices,
                    kv_last_page_len=b.kv_last_page_len)
    plan.check(qo_indptr=b.qo_indptr, kv_indptr=b.kv_indptr, kv_indices=b.kv_indices,
               kv_last_page_len=b.kv_last_page_len)
    grown = b.kv_last_page_len.copy()
    grown[2] += 1
    with pytest.raises(pkv.PkvError) as e:
        plan.check(qo_indptr=b.qo_indptr, kv_indptr=b.kv_indptr, kv_indices=b.kv_indices, kv_last_page_len=grown)
    assert e.value.status == 5
    with pytest.raises(TypeError):
        pkv.Plan(params, qo_indptr=b.qo_indptr.astype(np.int64), kv_indptr=b.kv_indptr, kv_indices=b.kv_indices,
                 kv_last_page_len=b.kv_last_page_len)


ROW_KERNEL_CASES = [
    ("bf16", "bf16", 128, 1), ("bf16", "bf16", 128, 2), ("bf16", "bf16", 128, 8),
    ("bf16", "bf16", 64, 1), ("bf16", "bf16", 64, 2), ("bf16", "bf16", 64, 4), ("bf16", "bf16", 64, 8),
    ("f32", "f32", 128, 1), ("f32", "f32", 128, 2), ("f32", "f32", 128, 4),
    ("f32", "f32", 64, 1), ("f32", "f32", 64, 4),
    ("bf16", "fp8", 128, 1), ("bf16", "fp8", 128, 2), ("bf16", "fp8", 128, 8),
]


@pytest.mark.parametrize("mode,waves", [("decode", 4), ("decode", 1), ("prefill", 0)])
@pytest.mark.parametrize("dtype,kv_dtype,dim,group", ROW_KERNEL_CASES)
def test_every_dtype_dim_and_group(torch, pkv, mode, waves, dtype, kv_dtype, dim, group):
    """Every (query dtype, cache dtype, head_dim, GQA group) the library builds,
    in decode (row kernel workgroups of 4 waves and of one) and prefill, on
    small batches (2 kv heads; HND for prefill): each kernel instantiation
    against the oracle.  bf16 prefill with head_dim 128 runs the MFMA tile
    kernel, the rest the row kernel."""
    print("case kernel", mode, waves, dtype, kv_dtype, dim, group, flush=True)
    kw = dict(hq=2 * group, hkv=2, dim=dim, dtype=dtype, kv_dtype=kv_dtype, batch=5)
    if mode == "decode":
        b = wl.make("decode", kv_range=(1, 300), pool=128, poison=True, **kw)
    else:
        b = wl.make("prefill", qo_range=(1, 70), prefix_range=(0, 200), **kw)
    fp8 = kv_dtype == "fp8"
    to_kv = (lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()) if fp8 else (lambda x: gu.to_dev(x, dtype))
    k_dev, v_dev = to_kv(b.k_cache), to_kv(b.v_cache)
    params = pkv.plan_params(mode=mode, batch_size=b.batch_size, num_qo_heads=b.num_qo_heads,
                             num_kv_heads=2, head_dim_qk=dim, page_size=b.page_size, causal=b.causal,
                             dtype=dtype, kv_dtype=kv_dtype, max_num_pages=b.max_num_pages, row_waves=waves)
    plan = pkv.Plan(params, qo_indptr=b.qo_indptr if mode == "prefill" else None, kv_indptr=b.kv_indptr,
                    kv_indices=b.kv_indices, kv_last_page_len=b.kv_last_page_len)
    assert plan.info["row_waves"] == (waves or 4)
    q = gu.to_dev(b.q, dtype)
    out = gu.empty_like_out(q.shape, dtype)
    lse = torch.full((q.shape[0], b.num_qo_heads), float("nan"), dtype=torch.float32, device="cuda")
    ks, vs = (0.5, 2.0) if fp8 else (1.0, 1.0)
    plan.run(q, k_dev, v_dev, gu.to_dev(b.kv_indices, "i32"), out, lse, layout=b.layout, sm_scale=b.sm_scale,
             k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    ro, rl = oat.paged_attention(b.q, b.k_cache, b.v_cache, qo_indptr=list(b.qo_indptr), kv_indptr=list(b.kv_indptr),
                                 kv_indices=list(b.kv_indices), kv_last_page_len=list(b.kv_last_page_len),
                                 page_size=b.page_size, layout=b.layout, num_kv_heads=2, causal=b.causal,
                                 sm_scale=b.sm_scale, q_dtype=dtype, kv_dtype=kv_dtype, k_scale=ks, v_scale=vs)
    got = gu.to_host(out, dtype)
    gu.check_close(gu.as_f64(got, "bf16") if dtype == "bf16" else got, ro, dtype, f"{mode} o")
    gu.check_lse(lse.cpu().numpy(), rl, f"{mode} lse", atol=1e-5 if dtype == "f32" else 1e-3)
