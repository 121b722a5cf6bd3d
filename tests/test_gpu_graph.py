"""GPU tests of fixed-capacity plans under graph capture: one pkv_run is
captured into a HIP graph (torch.cuda.graph) once; then, batch after batch,
the plan is updated, the inputs are refreshed in their fixed buffers and the
graph is replayed.  Every replay is checked against the float64 oracle, with
eager work and synchronisations between replays."""

import numpy as np
import pytest

import workloads as wl
from oracle import attention as oat
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    return gu.require_gpu()


@pytest.fixture(scope="module")
def pkv(torch):
    import paged_kv_cache_plan_amd as pkv
    return pkv


def _oracle(b):
    return oat.paged_attention(b.q, b.k_cache, b.v_cache, qo_indptr=list(b.qo_indptr), kv_indptr=list(b.kv_indptr),
                               kv_indices=list(b.kv_indices), kv_last_page_len=list(b.kv_last_page_len),
                               page_size=b.page_size, layout=b.layout, num_kv_heads=b.num_kv_heads,
                               causal=b.causal, sm_scale=b.sm_scale, q_dtype=b.dtype, kv_dtype=b.dtype)


def _fill(torch, dst, host, dtype):
    src = gu.to_dev(host, dtype)
    dst.view(-1)[:src.numel()].copy_(src.reshape(-1))


class _Fixed:
    """Fixed-address device buffers sized for the largest batch."""

    def __init__(self, torch, b0, max_rows, max_pages):
        bf = b0.dtype == "bf16"
        dt = torch.bfloat16 if bf else torch.float32
        self.q = torch.zeros((max_rows, b0.num_qo_heads, b0.head_dim), dtype=dt, device="cuda")
        self.out = torch.zeros_like(self.q)
        self.lse = torch.zeros((max_rows, b0.num_qo_heads), dtype=torch.float32, device="cuda")
        self.k = torch.zeros(b0.k_cache.shape, dtype=dt, device="cuda")
        self.v = torch.zeros(b0.v_cache.shape, dtype=dt, device="cuda")
        self.idx = torch.zeros(max_pages, dtype=torch.int32, device="cuda")

    def load(self, torch, b):
        _fill(torch, self.q, b.q, b.dtype)
        _fill(torch, self.k, b.k_cache, b.dtype)
        _fill(torch, self.v, b.v_cache, b.dtype)
        self.idx[:len(b.kv_indices)].copy_(gu.to_dev(b.kv_indices, "i32"))


def _capture(torch, fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                      # eager warm-up on the side stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _check(b, buf, what):
    n = int(b.qo_indptr[-1])
    o = gu.to_host(buf.out[:n], b.dtype)
    lse = buf.lse[:n].cpu().numpy()
    ro, rl = _oracle(b)
    gu.check_close(gu.as_f64(o, b.dtype), ro, b.dtype, what + " o")
    gu.check_lse(lse, rl, what + " lse", atol=1e-5 if b.dtype == "f32" else 1e-3)


@pytest.mark.parametrize("mode", ["decode", "prefill"])
def test_captured_run_replays_across_updates(torch, pkv, mode):
    if mode == "decode":
        mk = lambda seed, lo, hi: wl.make("decode", seed=seed, batch=16, kv_range=(lo, hi), pool=2100)
        ranges = [(64, 2048), (1, 300), (1500, 2000), (64, 2048)]
        max_rows = 16
    else:
        mk = lambda seed, lo, hi: wl.make("prefill", seed=seed, batch=4, qo_range=(lo, hi), prefix_range=(0, 900),
                                          pool=600)
        ranges = [(50, 300), (1, 40), (200, 320), (50, 300)]
        max_rows = 4 * 320
    batches = [mk(500 + i, lo, hi) for i, (lo, hi) in enumerate(ranges)]
    b0 = batches[0]
    params = pkv.plan_params(mode=mode, batch_size=b0.batch_size, num_qo_heads=b0.num_qo_heads,
                             num_kv_heads=b0.num_kv_heads, head_dim_qk=b0.head_dim, page_size=b0.page_size,
                             causal=b0.causal, dtype=b0.dtype, max_num_pages=b0.max_num_pages)
    caps = pkv.graph_caps(max_total_rows=max_rows, max_total_pages=b0.max_num_pages,
                          max_partial_rows=16384 if mode == "prefill" else 0)
    plan = pkv.GraphPlan(params, caps)
    buf = _Fixed(torch, b0, max_rows, b0.max_num_pages)
    qo = lambda b: b.qo_indptr if mode == "prefill" else None
    plan.update(qo_indptr=qo(b0), kv_indptr=b0.kv_indptr, kv_indices=b0.kv_indices,
                kv_last_page_len=b0.kv_last_page_len)
    buf.load(torch, b0)
    nrows = lambda b: int(b.qo_indptr[-1])

    def run():
        plan.run(buf.q[:max_rows], buf.k, buf.v, buf.idx, buf.out[:max_rows], buf.lse[:max_rows],
                 layout=b0.layout, sm_scale=b0.sm_scale)

    g = _capture(torch, run)
    for i, b in enumerate(batches):
        print(f"graph {mode} batch {i} rows {nrows(b)} pages {len(b.kv_indices)}", flush=True)
        plan.update(qo_indptr=qo(b), kv_indptr=b.kv_indptr, kv_indices=b.kv_indices,
                    kv_last_page_len=b.kv_last_page_len)
        buf.load(torch, b)
        buf.out.fill_(float("nan"))
        for rep in range(2):
            g.replay()
            torch.cuda.synchronize()
            _check(b, buf, f"{mode} batch {i} replay {rep}")
            torch.zeros(1 << 20, device="cuda").add_(1.0)      # eager work between replays
            torch.cuda.synchronize()
        assert plan.info["num_items"] <= plan.caps["max_items"]


def test_update_beyond_capacity_keeps_previous_batch(torch, pkv):
    b0 = wl.make("decode", seed=77, batch=8, kv_range=(100, 900), pool=600)
    big = wl.make("decode", seed=78, batch=8, kv_range=(4000, 4500), pool=600 * 4)
    params = pkv.plan_params(mode="decode", batch_size=8, num_qo_heads=32, num_kv_heads=8, head_dim_qk=128,
                             page_size=16, max_num_pages=big.max_num_pages)
    plan = pkv.GraphPlan(params, pkv.graph_caps(max_total_pages=600))
    buf = _Fixed(torch, big, 8, big.max_num_pages)
    b0.k_cache = np.concatenate([b0.k_cache, np.zeros((big.max_num_pages - 600,) + b0.k_cache.shape[1:],
                                                      b0.k_cache.dtype)])
    b0.v_cache = np.concatenate([b0.v_cache, np.zeros((big.max_num_pages - 600,) + b0.v_cache.shape[1:],
                                                      b0.v_cache.dtype)])
    plan.update(kv_indptr=b0.kv_indptr, kv_indices=b0.kv_indices, kv_last_page_len=b0.kv_last_page_len)
    buf.load(torch, b0)
    with pytest.raises(pkv.PkvError) as e:
        plan.update(kv_indptr=big.kv_indptr, kv_indices=big.kv_indices, kv_last_page_len=big.kv_last_page_len)
    assert e.value.status == 4
    with pytest.raises(ValueError):              # another batch size
        plan.update(kv_indptr=b0.kv_indptr[:5], kv_indices=b0.kv_indices, kv_last_page_len=b0.kv_last_page_len[:4])
    plan.run(buf.q[:8], buf.k, buf.v, buf.idx, buf.out[:8], buf.lse[:8], layout="NHD", sm_scale=b0.sm_scale)
    torch.cuda.synchronize()
    _check(b0, buf, "previous batch")


def test_captured_mla_run_replays_across_updates(torch, pkv):
    batches = [wl.make("mla", seed=600 + i, batch=8, kv_range=r, pool=700)
               for i, r in enumerate([(100, 3000), (1, 200), (2500, 4000)])]
    b0 = batches[0]
    params = pkv.plan_params(mode="mla", batch_size=8, num_qo_heads=128, num_kv_heads=1, head_dim_qk=576,
                             head_dim_vo=512, page_size=64, max_num_pages=700)
    plan = pkv.GraphPlan(params, pkv.graph_caps(max_total_pages=700))
    q_ckv = torch.zeros((8, 128, 512), dtype=torch.bfloat16, device="cuda")
    q_kpe = torch.zeros((8, 128, 64), dtype=torch.bfloat16, device="cuda")
    cache = torch.zeros((700, 64, 576), dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros(700, dtype=torch.int32, device="cuda")
    out = torch.zeros((8, 128, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((8, 128), dtype=torch.float32, device="cuda")

    def load(b):
        q_ckv.copy_(gu.to_dev(b.q, "bf16"))
        q_kpe.copy_(gu.to_dev(b.q_kpe, "bf16"))
        cache.copy_(gu.to_dev(b.k_cache, "bf16"))
        idx[:len(b.kv_indices)].copy_(gu.to_dev(b.kv_indices, "i32"))

    plan.update(kv_indptr=b0.kv_indptr, kv_indices=b0.kv_indices, kv_last_page_len=b0.kv_last_page_len)
    load(b0)
    g = _capture(torch, lambda: plan.run_mla(q_ckv, q_kpe, cache[..., :512], cache[..., 512:], idx, out, lse,
                                             sm_scale=b0.sm_scale))
    for i, b in enumerate(batches):
        print(f"graph mla batch {i}", flush=True)
        plan.update(kv_indptr=b.kv_indptr, kv_indices=b.kv_indices, kv_last_page_len=b.kv_last_page_len)
        load(b)
        for rep in range(2):
            g.replay()
            torch.cuda.synchronize()
            ckv = b.k_cache[..., :512]
            kpe = b.k_cache[..., 512:]
            ro, rl = oat.mla_decode(b.q, b.q_kpe, ckv, kpe, kv_indptr=list(b.kv_indptr), kv_indices=list(b.kv_indices),
                                    kv_last_page_len=list(b.kv_last_page_len), page_size=64, sm_scale=b.sm_scale)
            gu.check_close(gu.as_f64(gu.to_host(out, "bf16"), "bf16"), ro, "bf16", f"mla batch {i} o")
            gu.check_lse(lse.cpu().numpy(), rl, f"mla batch {i} lse")
            torch.zeros(1 << 20, device="cuda").add_(1.0)
            torch.cuda.synchronize()


def test_captured_masked_prefill_replays_across_updates(torch, pkv):
    """A fixed-capacity plan with a custom mask (the MFMA kernel's mask tiles)
    captured once and replayed for three batches; the packed mask lives in a
    fixed buffer whose contents change with each batch."""
    rng = np.random.default_rng(77)
    batches = [wl.make("prefill", seed=700 + i, batch=4, qo_range=r, prefix_range=(0, 700), pool=500)
               for i, r in enumerate([(60, 250), (1, 50), (200, 260)])]
    b0 = batches[0]
    max_rows = 4 * 260
    params = pkv.plan_params(mode="prefill", batch_size=4, num_qo_heads=32, num_kv_heads=8, head_dim_qk=128,
                             page_size=16, causal=False, dtype="bf16", custom_mask=True, max_num_pages=500)
    plan = pkv.GraphPlan(params, pkv.graph_caps(max_total_rows=max_rows, max_total_pages=500, max_partial_rows=8192))
    buf = _Fixed(torch, b0, max_rows, 500)
    max_bits = max_rows * 960
    mask_dev = torch.zeros(max_bits // 8 + 64, dtype=torch.uint8, device="cuda")
    masks = []
    for b in batches:
        segs = [(rng.random((q, k)) < 0.6).reshape(-1) for q, k in zip(b.qo_lens, b.kv_lens)]
        masks.append(np.concatenate(segs))
        assert len(masks[-1]) <= max_bits

    def load(i):
        b = batches[i]
        plan.update(qo_indptr=b.qo_indptr, kv_indptr=b.kv_indptr, kv_indices=b.kv_indices,
                    kv_last_page_len=b.kv_last_page_len)
        buf.load(torch, b)
        packed = np.packbits(masks[i], bitorder="little")
        mask_dev.zero_()
        mask_dev[:len(packed)].copy_(torch.from_numpy(packed).cuda())

    def run():
        plan.run_masked(buf.q[:max_rows], buf.k, buf.v, buf.idx, mask_dev, buf.out[:max_rows], buf.lse[:max_rows],
                        layout=b0.layout, sm_scale=b0.sm_scale)

    load(0)
    g = _capture(torch, run)
    for i, b in enumerate(batches):
        print(f"graph masked batch {i}", flush=True)
        load(i)
        buf.out.fill_(float("nan"))
        for rep in range(2):
            g.replay()
            torch.cuda.synchronize()
            n = int(b.qo_indptr[-1])
            ro, rl = oat.paged_attention(b.q, b.k_cache, b.v_cache, qo_indptr=list(b.qo_indptr),
                                         kv_indptr=list(b.kv_indptr), kv_indices=list(b.kv_indices),
                                         kv_last_page_len=list(b.kv_last_page_len), page_size=16, layout=b.layout,
                                         num_kv_heads=8, sm_scale=b.sm_scale, q_dtype="bf16", kv_dtype="bf16",
                                         custom_mask=masks[i])
            gu.check_close(gu.as_f64(gu.to_host(buf.out[:n], "bf16"), "bf16"), ro, "bf16", f"masked batch {i} o")
            gu.check_lse(buf.lse[:n].cpu().numpy(), rl, f"masked batch {i} lse")
            torch.zeros(1 << 20, device="cuda").add_(1.0)
            torch.cuda.synchronize()
