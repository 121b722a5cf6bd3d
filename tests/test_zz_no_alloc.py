"""pkv_run_noalloc, the entry point that allocates nothing, against pkv_run:
two calls in a row on one device, the second with a smaller batch (fewer
items and partial states in the shared scratch array), each checked bit for
bit against pkv_run's output and LSE on the same inputs (both run the same
work list through the same kernels) and against the oracle at the bf16
tolerance and the regression guard."""

import numpy as np
import pytest

import workloads as wl
from oracle import attention as oat
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    return gu.require_gpu()


def _run_both(torch, pkv, b, fixed_split_pages=0):
    params = pkv.plan_params(mode=b.mode, batch_size=b.batch_size, num_qo_heads=b.num_qo_heads,
                             num_kv_heads=b.num_kv_heads, head_dim_qk=b.head_dim, page_size=b.page_size,
                             causal=b.causal, dtype=b.dtype, fixed_split_pages=fixed_split_pages,
                             max_num_pages=b.max_num_pages)
    qo = b.qo_indptr if b.mode == "prefill" else None
    q = gu.to_dev(b.q, b.dtype)
    k, v = gu.to_dev(b.k_cache, b.dtype), gu.to_dev(b.v_cache, b.dtype)
    idx = gu.to_dev(b.kv_indices, "i32")
    plan = pkv.Plan(params, qo_indptr=qo, kv_indptr=b.kv_indptr, kv_indices=b.kv_indices,
                    kv_last_page_len=b.kv_last_page_len)
    out_ref = gu.empty_like_out(q.shape, b.dtype)
    lse_ref = torch.full((q.shape[0], b.num_qo_heads), float("nan"), dtype=torch.float32, device="cuda")
    plan.run(q, k, v, idx, out_ref, lse_ref, layout=b.layout, sm_scale=b.sm_scale)
    out = gu.empty_like_out(q.shape, b.dtype)
    lse = torch.full((q.shape[0], b.num_qo_heads), float("nan"), dtype=torch.float32, device="cuda")
    pkv.run_noalloc(params, q, k, v, idx, out, lse, qo_indptr=qo, kv_indptr=b.kv_indptr,
                    kv_indices_host=b.kv_indices, kv_last_page_len=b.kv_last_page_len, layout=b.layout,
                    sm_scale=b.sm_scale)
    torch.cuda.synchronize()
    return plan.info, gu.to_host(out_ref, b.dtype), lse_ref.cpu().numpy(), gu.to_host(out, b.dtype), lse.cpu().numpy()


def _check(b, o_ref, l_ref, o, lse, what):
    assert np.array_equal(o, o_ref), f"{what}: output differs from pkv_run"
    assert np.array_equal(lse, l_ref), f"{what}: LSE differs from pkv_run"
    ro, rl = oat.paged_attention(b.q, b.k_cache, b.v_cache, qo_indptr=list(b.qo_indptr), kv_indptr=list(b.kv_indptr),
                                 kv_indices=list(b.kv_indices), kv_last_page_len=list(b.kv_last_page_len),
                                 page_size=b.page_size, layout=b.layout, num_kv_heads=b.num_kv_heads,
                                 causal=b.causal, sm_scale=b.sm_scale, q_dtype=b.dtype, kv_dtype=b.dtype)
    got = gu.as_f64(o, "bf16")
    gu.check_close(got, ro, "bf16", f"{what} o")
    gu.check_lse(lse, rl, f"{what} lse")
    gu.check_guard(got, ro, lse, rl, what)


def test_noalloc_matches_run_on_two_calls_second_smaller(torch):
    import paged_kv_cache_plan_amd as pkv
    # Call 1: a split prefill on the MFMA tile kernel (partial states and a merge in the array).
    big = wl.make("prefill", batch=3, qo_range=(60, 200), prefix_range=(300, 1500), poison=False)
    print("case noalloc call 1: prefill", list(big.qo_lens), list(big.kv_lens), flush=True)
    info1, o_ref, l_ref, o, lse = _run_both(torch, pkv, big, fixed_split_pages=32)   # ~10.6 MiB of scratch
    assert info1["num_merges"] > 0
    _check(big, o_ref, l_ref, o, lse, "noalloc prefill")
    # Call 2: a smaller decode batch (row kernel, tail-split merge) in the same array.
    small = wl.make("decode", batch=6, kv_range=(100, 900), poison=True)
    print("case noalloc call 2: decode", list(small.kv_lens), flush=True)
    info2, o_ref, l_ref, o, lse = _run_both(torch, pkv, small)
    assert info2["num_merges"] > 0
    assert info2["workspace_bytes"] < info1["workspace_bytes"] and info2["total_rows"] < info1["total_rows"]
    _check(small, o_ref, l_ref, o, lse, "noalloc decode")
