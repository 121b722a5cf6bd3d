"""Kernel timing through pkv_time_next_attention: the armed events are
recorded by the attention kernel's own dispatch, one launch per arming, and
arming changes no result."""

import numpy as np
import pytest

import workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    return gu.require_gpu()


@pytest.fixture(scope="module")
def pkv(torch):
    import paged_kv_cache_plan_amd as pkv
    return pkv


def _gqa(pkv, torch, name, **kw):
    b = wl.make(name, **kw)
    k, v = gu.to_dev(b.k_cache, b.dtype), gu.to_dev(b.v_cache, b.dtype)
    params = pkv.plan_params(mode=b.mode, batch_size=b.batch_size, num_qo_heads=b.num_qo_heads,
                             num_kv_heads=b.num_kv_heads, head_dim_qk=b.head_dim, page_size=b.page_size,
                             causal=b.causal, dtype=b.dtype, max_num_pages=k.shape[0])
    plan = pkv.Plan(params, qo_indptr=b.qo_indptr if b.mode == "prefill" else None, kv_indptr=b.kv_indptr,
                    kv_indices=b.kv_indices, kv_last_page_len=b.kv_last_page_len)
    q = gu.to_dev(b.q, b.dtype)
    idx = gu.to_dev(b.kv_indices, "i32")

    def run():
        out = gu.empty_like_out(q.shape, b.dtype)
        lse = torch.empty((q.shape[0], b.num_qo_heads), dtype=torch.float32, device="cuda")
        plan.run(q, k, v, idx, out, lse, layout=b.layout, sm_scale=b.sm_scale)
        return out, lse
    return run


@pytest.mark.parametrize("name,kw", [("decode", dict(scale=0.25, batch=16)),      # row kernel
                                     ("prefill", dict(scale=0.25, batch=3))])     # MFMA tile kernel
def test_armed_events_time_one_launch(torch, pkv, name, kw):
    print("case timing", name, flush=True)
    run = _gqa(pkv, torch, name, **kw)
    o0, l0 = run()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    pkv.time_next_attention(start, stop)
    o1, l1 = run()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop)
    assert 0.0 < ms < 1000.0
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    # Disarmed by that launch: later runs leave the events as they were.
    o2, _ = run()
    o3, _ = run()
    torch.cuda.synchronize()
    assert start.elapsed_time(stop) == ms
    assert torch.equal(o0, o3)
    print("timed", name, f"{ms * 1e3:.1f} us", flush=True)


def test_armed_events_on_mla(torch, pkv):
    print("case timing mla", flush=True)
    b = wl.make("mla", scale=0.25, batch=8)
    cache = gu.to_dev(b.k_cache, "bf16")
    params = pkv.plan_params(mode="mla", batch_size=b.batch_size, num_qo_heads=128, num_kv_heads=1,
                             head_dim_qk=576, head_dim_vo=512, page_size=b.page_size, dtype="bf16",
                             max_num_pages=b.max_num_pages)
    plan = pkv.Plan(params, kv_indptr=b.kv_indptr, kv_indices=b.kv_indices, kv_last_page_len=b.kv_last_page_len)
    out = gu.empty_like_out((b.batch_size, 128, 512), "bf16")
    lse = torch.empty((b.batch_size, 128), dtype=torch.float32, device="cuda")
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    pkv.time_next_attention(start, stop)
    plan.run_mla(gu.to_dev(b.q, "bf16"), gu.to_dev(b.q_kpe, "bf16"), cache[..., :512], cache[..., 512:],
                 gu.to_dev(b.kv_indices, "i32"), out, lse, sm_scale=b.sm_scale)
    torch.cuda.synchronize()
    assert 0.0 < start.elapsed_time(stop) < 1000.0
    assert np.isfinite(lse.cpu().numpy()).all()
