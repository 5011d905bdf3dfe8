"""Expert streaming from a pinned host pool through a device expert cache
("One GPU, three storage tiers"; "Read the experts the router needs"): every
output of moe_layer_streamed must match the CPU oracle on the same inputs
(ids, weights, bucketing exactly; floating outputs within the layer's bar)
and equal moe_layer_mxfp4 on the same layer held in device memory, bit for
bit, over call sequences that hit, miss, evict and bypass; the cache's
counters must agree with the routing.  Needs an MI355X."""
import numpy as np
import pytest

import oracle
import synth
from conftest import assert_close

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _moe():
    import router_top_bucket_amd as moe
    return moe


def _host_pool(shape, seeds):
    rec = shape.n_experts * shape.stride
    pool = torch.empty(len(seeds) * rec, dtype=torch.uint8, pin_memory=True)
    for l, seed in enumerate(seeds):
        for e, r in synth.expert_records(shape, seed, range(shape.n_experts)):
            off = l * rec + e * shape.stride
            pool[off:off + shape.stride].copy_(torch.from_numpy(r))
    return pool


def _outputs(res, M, k, S):
    torch.cuda.synchronize()
    na = int(res["n_active"][0].item())
    return dict(logits=res["logits"][:M].cpu().numpy(), ids=res["topk_ids"][:M].cpu().numpy(),
                w=res["topk_w"][:M].cpu().numpy(), offsets=res["offsets"].cpu().numpy(),
                perm=res["perm"][:M * (k + S)].cpu().numpy(), active=res["active"][:na].cpu().numpy(),
                y=res["y_slots"][:M * (k + S)].cpu().numpy(), out=res["out"][:M].cpu().numpy())


def _x(shape, seed, M, block=False):
    x = synth.block_x(shape, seed, M) if block else synth.rows_x(shape, seed, M)
    t = torch.from_numpy(np.ascontiguousarray(x))
    return (t.view(torch.bfloat16) if shape.x_dtype == "bf16" else t).cuda()


def _against_oracle(b, shape, seed, x_host, rec, what):
    """One streamed call's outputs against the oracle layer.  The logits are
    compared within the bar; ids and everything after them are checked
    against the oracle run on the GPU's own logits, so a near-tie that rounds
    the other way on one side cannot flip the comparison."""
    k, S, E = shape.k, shape.n_shared, shape.n_routed
    wr = synth.router_weight(shape, seed)
    ref = oracle.layer(x_host, k, E, S, shape.d, shape.f, rec, w_r=wr)
    assert_close(b["logits"], ref["logits"], what + " logits")
    ref = oracle.layer(x_host, k, E, S, shape.d, shape.f, rec, logits=b["logits"])
    assert np.array_equal(b["ids"], ref["ids"]), what + " ids"
    assert_close(b["w"], ref["w"], what + " w")
    assert np.array_equal(b["offsets"], ref["offsets"]) and np.array_equal(b["perm"], ref["perm"]), what
    assert np.array_equal(b["active"], ref["active"]), what + " active"
    assert_close(b["y"], ref["y_slots"], what + " y_slots")
    assert_close(b["out"], ref["out"], what + " out")


def _check_sequence(moe, shape, seeds, cache, calls, max_rows, block=False, oracle_rows=None):
    """calls: (layer, M, x seed).  Streamed vs resident, every output bit for
    bit; and the streamed outputs against the oracle for every call with at
    most ``oracle_rows`` rows (None: every call)."""
    k, S, E = shape.k, shape.n_shared, shape.n_routed
    resident = [moe.Experts(synth.device_experts(shape, s), shape.stride, shape.d, shape.f, E, S) for s in seeds]
    routers = [torch.from_numpy(synth.router_weight(shape, s)).cuda() for s in seeds]
    st = moe.MoELayer(cache.descriptor(), k, max_rows)
    routed = 0
    recs = [{} for _ in seeds]

    def rec_of(layer):
        def rec(e):
            if e not in recs[layer]:
                recs[layer][e] = synth.expert_record(shape, seeds[layer], e)
            return recs[layer][e]
        return rec

    for i, (layer, M, xs) in enumerate(calls):
        x = _x(shape, xs, M, block)
        ref = moe.MoELayer(resident[layer], k, M, w_router=routers[layer])
        a = _outputs(ref.forward(x), M, k, S)
        st.w_router = routers[layer]
        for t in (st.y_slots, st.out):
            t.fill_(float("nan"))
        b = _outputs(st.forward_streamed(cache, layer, x), M, k, S)
        for key in a:
            assert np.array_equal(a[key].view(np.uint8), b[key].view(np.uint8)), (i, layer, M, key)
        if oracle_rows is None or M <= oracle_rows:
            x_host = synth.block_x(shape, xs, M) if block else synth.rows_x(shape, xs, M)
            _against_oracle(b, shape, seeds[layer], x_host, rec_of(layer), f"streamed call {i} (layer {layer}, M={M})")
        routed += int(np.sum(a["active"] < E))
    s = cache.stats()
    assert s["calls"] == len(calls)
    assert s["hits"] + s["misses"] == routed
    assert s["bytes_uploaded"] == s["misses"] * shape.stride
    return s


SMALL = synth.LayerShape("s3", 416, 224, 9, 2, 4, -7, -3, 0.05, "bf16")


@pytest.mark.parametrize("streams,groups,admit,transient", [(1, 1, 0, 0), (4, 3, 0, 2), (8, 16, 2, 5),
                                                            (2, 2, 3, 9)])
def test_streamed_equals_resident_small(streams, groups, admit, transient):
    moe = _moe()
    shape = SMALL
    seeds = [51, 52, 53]
    host = _host_pool(shape, seeds)
    n_cache = max(1, shape.n_routed - transient)  # routed slots = E: every call fits
    n_slots = len(seeds) * shape.n_shared + transient + n_cache
    dev_pool = torch.zeros(n_slots * shape.stride, dtype=torch.uint8, device="cuda")
    cache = moe.ExpertCache(dev_pool, host, len(seeds), shape.n_routed, shape.n_shared, shape.d, shape.f,
                            shape.stride, n_upload_streams=streams, upload_groups=groups, admit_min_rows=admit,
                            n_transient=transient)
    g = np.random.default_rng(streams * 100 + groups)
    calls = [(int(g.integers(0, 3)), int(m), 300 + i) for i, m in enumerate(g.choice([1, 2, 3, 5, 16, 40], 14))]
    s = _check_sequence(moe, shape, seeds, cache, calls, 40)
    assert s["misses"] > 0 and s["hits"] > 0
    cache.close()


def test_streamed_rejects_calls_that_cannot_fit():
    moe = _moe()
    shape = SMALL
    host = _host_pool(shape, [61])
    n_slots = shape.n_shared + 3  # 3 routed slots: 2 rows x k=4 can need 8
    dev_pool = torch.zeros(n_slots * shape.stride, dtype=torch.uint8, device="cuda")
    cache = moe.ExpertCache(dev_pool, host, 1, shape.n_routed, shape.n_shared, shape.d, shape.f, shape.stride)
    st = moe.MoELayer(cache.descriptor(), shape.k, 2, w_router=torch.from_numpy(synth.router_weight(shape, 61)).cuda())
    with pytest.raises(moe.MoeError) as ei:
        st.forward_streamed(cache, 0, _x(shape, 1, 2))
    assert ei.value.rc == moe.MOE_EUNSUPPORTED
    # a host pool that is not pinned: refused by the library itself
    import ctypes
    plain = np.zeros(host.numel(), dtype=np.uint8)
    cfg = moe._CacheConfig(dev_pool.data_ptr(), n_slots, plain.ctypes.data, 1, shape.n_routed, shape.n_shared,
                           shape.d, shape.f, shape.stride, 1, 1, 0, 0)
    h = ctypes.c_void_p()
    assert moe.raw_library().moe_cache_create(ctypes.byref(cfg), ctypes.byref(h)) == moe.MOE_EINVAL
    cache.close()


def test_streamed_kimi_decode_and_blocks(kimi_layer_host):
    """Kimi shape: a 1-row and 16-row call sequence through a cache of 300
    routed slots (one layer in the host pool)."""
    moe = _moe()
    shape, host, seed = kimi_layer_host
    n_slots = shape.n_shared + 16 + 284
    dev_pool = torch.zeros(n_slots * shape.stride, dtype=torch.uint8, device="cuda")
    cache = moe.ExpertCache(dev_pool, host, 1, shape.n_routed, shape.n_shared, shape.d, shape.f, shape.stride,
                            n_upload_streams=8, upload_groups=4, admit_min_rows=0, n_transient=16)
    calls = [(0, 1, 700), (0, 1, 700), (0, 16, 701), (0, 1, 702), (0, 16, 701), (0, 16, 703)]
    s = _check_sequence(moe, shape, [seed], cache, calls, 16, block=True, oracle_rows=1)
    assert s["hits"] >= 16  # the repeated 1-row call hits every routed expert
    del dev_pool
    cache.close()


@pytest.fixture(scope="module")
def kimi_layer_host():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    shape = synth.KIMI
    print(f"\n[kimi_layer_host] {shape.n_experts} experts into pinned host memory", flush=True)
    return shape, _host_pool(shape, [0]), 0
