"""GPU parity: every C-ABI call against the CPU oracle on the same seeded
inputs, plus the pages' invariants on the GPU path ("Run Kimi 3.1 locally on
one GPU", section "A drafter that leaves the answer unchanged": a row's
results inside a multi-row block are bit-identical to a one-row call, and do
not depend on the order in which experts are computed).  Needs an MI355X."""
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


def _dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def _host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


# ----------------------------------------------------------------------------- fixtures
@pytest.fixture(scope="session")
def kimi_layer():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe = _moe()
    shp = synth.KIMI
    seed = 0
    print(f"\n[kimi_layer] generating {shp.n_experts} experts ({shp.n_experts * shp.stride / 1e9:.1f} GB)", flush=True)
    base = synth.device_experts(shp, seed)
    ex = moe.Experts(base, shp.stride, shp.d, shp.f, shp.n_routed, shp.n_shared)
    wr = synth.router_weight(shp, seed)
    cache = {}

    def rec(e):
        if e not in cache:
            cache[e] = synth.expert_record(shp, seed, e)
        return cache[e]

    return dict(shape=shp, experts=ex, wr=wr, wr_dev=_dev(wr), rec=rec)


def _small_layer(shape, seed):
    moe = _moe()
    base = synth.device_experts(shape, seed)
    ex = moe.Experts(base, shape.stride, shape.d, shape.f, shape.n_routed, shape.n_shared)
    recs = {e: synth.expert_record(shape, seed, e) for e in range(shape.n_experts)}
    return ex, recs


def _x_dev(shape, x):
    return _dev(x, torch.bfloat16) if shape.x_dtype == "bf16" else _dev(x)


def _compare_layer(res_gpu, ref, what, k, S, exact_ids=True, rerun=None):
    """GPU layer outputs against the oracle's.  With the router computed on
    both sides (``rerun`` given: the oracle layer on given logits), the
    logits agree only to rounding, so where the ids differ the top-k
    decision and everything after it are checked against the oracle run on
    the GPU's own fp32 logits: two experts whose logits tie within rounding
    may rank either way."""
    gpu_logits = _host(res_gpu["logits"])
    assert_close(gpu_logits, ref["logits"], what + " logits")
    ids = _host(res_gpu["topk_ids"])
    if rerun is not None and not np.array_equal(ids, ref["ids"]):
        ref = rerun(gpu_logits)
    if exact_ids:
        assert np.array_equal(ids, ref["ids"]), what + " ids"
    assert_close(_host(res_gpu["topk_w"]), ref["w"], what + " w")
    assert np.array_equal(_host(res_gpu["offsets"]), ref["offsets"]), what + " offsets"
    assert np.array_equal(_host(res_gpu["perm"]), ref["perm"]), what + " perm"
    na = int(_host(res_gpu["n_active"])[0])
    assert na == ref["n_active"]
    assert np.array_equal(_host(res_gpu["active"])[:na], ref["active"]), what + " active"
    assert int(_host(res_gpu["dev_error"])[0]) == 0
    assert_close(_host(res_gpu["y_slots"]), ref["y_slots"], what + " y_slots")
    assert_close(_host(res_gpu["out"]), ref["out"], what + " out")


# ----------------------------------------------------------------------------- tiny layer
@pytest.mark.parametrize("seed", range(20))
def test_tiny_layer_parity(seed):
    moe = _moe()
    shp = synth.TINY
    ex, recs = _small_layer(shp, seed)
    wr = synth.router_weight(shp, seed)
    x = synth.rows_x(shp, seed, 1)
    layer = moe.MoELayer(ex, shp.k, 1, w_router=_dev(wr))
    res = layer.forward(_x_dev(shp, x))
    ref = oracle.layer(x, shp.k, shp.n_routed, shp.n_shared, shp.d, shp.f, recs.__getitem__, w_r=wr)
    _compare_layer(res, ref, f"tiny seed {seed}", shp.k, shp.n_shared,
                   rerun=lambda lg: oracle.layer(x, shp.k, shp.n_routed, shp.n_shared, shp.d, shp.f, recs.__getitem__, logits=lg))


# ----------------------------------------------------------------------------- route
@pytest.mark.parametrize("M,E,k", [(1, 896, 16), (16, 896, 16), (1533, 896, 16), (7, 16, 2), (3, 100, 1),
                                   (5, 64, 64), (2, 4096, 16)])
def test_route_given_logits_exact(M, E, k):
    moe = _moe()
    lg = synth.random_logits(M + E, M, E)
    # ties and NaN: quantise some rows to a coarse grid, poison a few entries
    lg[::3] = np.round(lg[::3] * 2) / 2
    lg[1::5, ::7] = np.nan
    if M > 1:
        lg[-1] = 0.25  # an all-equal row
    ids_ref, w_ref = oracle.topk(lg, k)
    d_lg = _dev(lg)
    ids = torch.empty((M, k), dtype=torch.int32, device="cuda")
    w = torch.empty((M, k), dtype=torch.float32, device="cuda")
    moe.moe_route(None, None, d_lg, k, ids, w)
    assert np.array_equal(_host(ids), ids_ref)
    assert_close(_host(w), w_ref, "topk weights")


def _near_threshold_logits(g, M, E, n_near):
    """Rows of logits in [-1, 0.9) with n_near of them set to 1 + i 2^-20
    (distinct values that share their top 16 order bits), in n_near distinct
    lanes (index mod 64) while n_near <= 64."""
    lg = (g.random((M, E), dtype=np.float32) * np.float32(1.9) - np.float32(1.0)).astype(np.float32)
    near = np.float32(1.0) + np.arange(n_near, dtype=np.float32) * np.float32(2.0 ** -20)
    for m in range(M):
        if n_near <= 64:
            lanes = g.choice(64, n_near, replace=False)
            pos = lanes + 64 * g.integers(0, E // 64, n_near)
        else:
            pos = g.choice(E, n_near, replace=False)
        lg[m, pos] = g.permutation(near)
    return lg


@pytest.mark.parametrize("n_near", [16, 17, 40, 64, 65, 130])
def test_route_threshold_candidates(n_near):
    """The ranking gathers the logits whose top 16 order bits reach those of
    the k-th largest lane maximum and ranks up to 64 of them by counting;
    past 64 it runs the list rounds.  With n_near near-equal top logits in
    distinct lanes exactly n_near are gathered: ids exact and weights within
    the bar against the oracle on both sides of the boundary, for moe_route
    (1, 4 and 16 rows) and for the one-row layer call, whose gate/up launch
    ranks the logits itself (route mode)."""
    moe = _moe()
    E, k = 896, 16
    g = np.random.default_rng(1000 + n_near)
    for M in (1, 4, 16):
        lg = _near_threshold_logits(g, M, E, n_near)
        ids_ref, w_ref = oracle.topk(lg, k)
        ids = torch.empty((M, k), dtype=torch.int32, device="cuda")
        w = torch.empty((M, k), dtype=torch.float32, device="cuda")
        moe.moe_route(None, None, _dev(lg), k, ids, w)
        assert np.array_equal(_host(ids), ids_ref), (n_near, M)
        assert_close(_host(w), w_ref, f"topk weights, {n_near} near the threshold, M={M}")
    shape = synth.LayerShape("e896", 64, 32, E, 1, k, -6, -2, 0.05, "bf16")
    ex, recs = _small_layer(shape, 51)
    layer = moe.MoELayer(ex, k, 1)
    for trial in range(3):
        lg = _near_threshold_logits(g, 1, E, n_near)
        x = synth.rows_x(shape, 52 + trial, 1)
        res = layer.forward(_x_dev(shape, x), logits=_dev(lg))
        ref = oracle.layer(x, k, shape.n_routed, shape.n_shared, shape.d, shape.f, recs.__getitem__, logits=lg)
        _compare_layer(res, ref, f"route mode, {n_near} near the threshold", k, shape.n_shared)


ROUTER_SHAPES = [
    synth.KIMI,
    synth.LayerShape("r3", 416, 224, 9, 2, 4, -7, -3, 0.05, "bf16"),
    synth.LayerShape("f32", 256, 128, 16, 0, 2, -6, -2, 0.05, "f32"),
    synth.LayerShape("odd", 1056, 64, 37, 0, 3, -6, -2, 0.05, "bf16"),
]


@pytest.mark.parametrize("shape", ROUTER_SHAPES, ids=lambda s: s.name)
def test_router_logits_rows_equal_single_rows(shape):
    """Router logits: every row of a call of up to 16 rows equals the same
    row computed alone, bit for bit; above 16 rows (the MFMA form) the rows
    of one call equal the same rows in another call of more than 16 rows
    bit for bit, and the single-row logits within the bar; all agree with
    the oracle within the bar."""
    moe = _moe()
    wr = synth.router_weight(shape, 61)
    dwr = _dev(wr)
    x = synth.rows_x(shape, 62, 150)
    xd = _x_dev(shape, x)
    E, k = shape.n_routed, shape.k

    def logits(rows):
        M = rows.shape[0]
        lg = torch.empty((M, E), dtype=torch.float32, device="cuda")
        ids = torch.empty((M, k), dtype=torch.int32, device="cuda")
        w = torch.empty((M, k), dtype=torch.float32, device="cuda")
        moe.moe_route(rows, dwr, lg, k, ids, w)
        return _host(lg)

    single = np.stack([logits(xd[m:m + 1])[0] for m in range(150)])
    ref = oracle.router_logits(x, wr)
    assert_close(single, ref, f"{shape.name} router logits")
    for M in (2, 3, 5, 9, 16):
        got = logits(xd[:M])
        assert np.array_equal(got.view(np.uint32), single[:M].view(np.uint32)), (shape.name, M)
    big = logits(xd)
    assert_close(big, ref, f"{shape.name} router logits, 150 rows")
    assert_close(big, single, f"{shape.name} 150-row logits against single rows")
    for M in (17, 40, 64, 65):
        got = logits(xd[:M])
        assert np.array_equal(got.view(np.uint32), big[:M].view(np.uint32)), (shape.name, M)
    # larger calls take other tile shapes (1 x 4, 2 x 2 and 2 x 4 router x x
    # tiles per wave, by row count and x type): the same rows, the same bits
    x8 = synth.rows_x(shape, 63, 800)
    xd8 = _x_dev(shape, x8)
    first = logits(xd8[:150])
    for M in (300, 500, 800):
        got = logits(xd8[:M])
        assert np.array_equal(got[:150].view(np.uint32), first.view(np.uint32)), (shape.name, M)
        assert_close(got[M - 40:], oracle.router_logits(x8[M - 40:M], wr), f"{shape.name} {M}-row logits, last rows")


def test_route_zipf_prefill_logits_exact():
    moe = _moe()
    for M in (270, 1533):
        lg = synth.zipf_logits(synth.KIMI, 1, M)
        ids_ref, w_ref = oracle.topk(lg, 16)
        ids = torch.empty((M, 16), dtype=torch.int32, device="cuda")
        w = torch.empty((M, 16), dtype=torch.float32, device="cuda")
        moe.moe_route(None, None, _dev(lg), 16, ids, w)
        assert np.array_equal(_host(ids), ids_ref)
        assert_close(_host(w), w_ref, "zipf weights")


# ----------------------------------------------------------------------------- bucket
def _run_bucket(ids_np, E, S):
    moe = _moe()
    M, k = ids_np.shape
    T = M * (k + S)
    i32 = dict(dtype=torch.int32, device="cuda")
    offsets = torch.full((E + S + 1,), -7, **i32)
    perm = torch.full((max(T, 1),), -7, **i32)
    active = torch.full((E + S,), -7, **i32)
    na = torch.full((1,), -7, **i32)
    err = torch.full((1,), -7, **i32)
    moe.moe_bucket(_dev(ids_np), E, S, offsets, perm, active, na, err)
    return _host(offsets), _host(perm)[:T], _host(active), int(_host(na)[0]), int(_host(err)[0])


# 4000 and 4100 rows at E + S = 898 sit on either side of the general
# kernel's LDS limit for keeping every slot's expert on chip (152 KB)
@pytest.mark.parametrize("M,E,k,S", [(1, 896, 16, 2), (3, 16, 2, 0), (16, 896, 16, 2), (64, 896, 16, 2),
                                     (65, 896, 16, 2), (270, 896, 16, 2), (1533, 896, 16, 2), (5, 4, 4, 1),
                                     (200, 4000, 16, 96), (4000, 896, 16, 2), (4100, 896, 16, 2)])
def test_bucket_exact(M, E, k, S):
    g = synth.rng(3, M, E)
    ids = np.stack([g.permutation(E)[:k] for _ in range(M)]).astype(np.int32)
    off, perm, act, na, err = _run_bucket(ids, E, S)
    r_off, r_perm, r_act, r_na = oracle.bucket(ids, E, S)
    assert err == 0
    assert np.array_equal(off, r_off) and np.array_equal(perm, r_perm)
    assert na == r_na and np.array_equal(act[:na], r_act)


def test_bucket_zipf_exact():
    lg = synth.zipf_logits(synth.KIMI, 2, 1533)
    ids, _ = oracle.topk(lg, 16)
    off, perm, act, na, err = _run_bucket(ids, 896, 2)
    r_off, r_perm, r_act, r_na = oracle.bucket(ids, 896, 2)
    assert err == 0 and np.array_equal(off, r_off) and np.array_equal(perm, r_perm)
    assert na == r_na and np.array_equal(act[:na], r_act)


def test_bucket_flags_bad_ids_in_bounds():
    ids = np.array([[0, 5], [3, 16], [-1, 2], [4, 4]], dtype=np.int32)  # out of range and a repeat
    off, perm, act, na, err = _run_bucket(ids, 16, 1)
    assert err == 1
    assert off[-1] <= 4 * 3  # only valid slots counted, all writes in bounds
    valid = np.array([[0, 5], [3, 1], [6, 2], [7, 8]], dtype=np.int32)
    off, perm, act, na, err = _run_bucket(valid, 16, 1)
    assert err == 0  # the flag is cleared by a clean call


@pytest.mark.parametrize("M", [100, 26000])
def test_bucket_general_kernel_flags_bad_ids(M):
    """The general bucket kernel (more than 64 rows), with the slots' experts
    kept in LDS (100 rows) and read from global memory (26,000 rows: 78,000
    slots are past the LDS limit): an out-of-range id, a negative id and a
    repeated id set the flag, and every write stays in bounds."""
    E, k, S = 16, 2, 1
    g = synth.rng(5, M, E)
    ids = np.stack([g.permutation(E)[:k] for _ in range(M)]).astype(np.int32)
    ids[M // 3, 0] = E + 3
    ids[M // 2, 1] = -1
    ids[M - 1, 1] = ids[M - 1, 0]
    T = M * (k + S)
    off, perm, act, na, err = _run_bucket(ids, E, S)
    assert err == 1
    assert 0 <= off[-1] <= T
    written = perm[perm != -7]
    assert ((written >= 0) & (written < T)).all()
    ok = np.stack([g.permutation(E)[:k] for _ in range(M)]).astype(np.int32)
    off, perm, act, na, err = _run_bucket(ok, E, S)
    r_off, r_perm, r_act, r_na = oracle.bucket(ok, E, S)
    assert err == 0 and np.array_equal(off, r_off) and np.array_equal(perm, r_perm)
    assert na == r_na and np.array_equal(act[:na], r_act)


ROUTE_SHAPES = [
    synth.LayerShape("e896", 64, 32, 896, 2, 16, -6, -2, 0.05, "bf16"),
    synth.LayerShape("e16", 64, 32, 16, 0, 2, -6, -2, 0.05, "f32"),
    synth.LayerShape("e64k64", 64, 32, 64, 0, 64, -6, -2, 0.05, "f32"),
    synth.LayerShape("e100s3", 64, 32, 100, 3, 1, -6, -2, 0.05, "bf16"),
    synth.LayerShape("e2000", 64, 32, 2000, 1, 8, -6, -2, 0.05, "bf16"),
    synth.LayerShape("e4000s40", 64, 32, 4000, 40, 16, -6, -2, 0.05, "bf16"),
    synth.LayerShape("e4090s6", 64, 32, 4090, 6, 8, -6, -2, 0.05, "f32"),
]


@pytest.mark.parametrize("shape", ROUTE_SHAPES, ids=lambda s: s.name)
def test_layer_routing_exact_adversarial_logits(shape):
    """The layer call routes and buckets (for a few rows: one top-k + bucket
    kernel) exactly as the oracle and as moe_route + moe_bucket do, on given
    logits with ties, NaN and an all-equal row."""
    moe = _moe()
    ex, _ = _small_layer(shape, 51)
    E, S, k = shape.n_routed, shape.n_shared, shape.k
    for M in (1, 2, 4, 5, 16):
        lg = synth.random_logits(E + M, M, E)
        lg[::2] = np.round(lg[::2] * 2) / 2
        lg[:, ::11] = np.nan
        lg[-1] = 0.5
        ids_ref, w_ref = oracle.topk(lg, k)
        r_off, r_perm, r_act, r_na = oracle.bucket(ids_ref, E, S)
        x = synth.rows_x(shape, 52 + M, M)
        layer = moe.MoELayer(ex, k, M)
        layer.dev_error.fill_(-7)
        layer.offsets.fill_(-7)
        layer.perm.fill_(-7)
        res = layer.forward(_x_dev(shape, x), logits=_dev(lg))
        got = _layer_outputs(res, M, k, S)
        what = (shape.name, M)
        assert np.array_equal(got["ids"], ids_ref), what
        assert np.array_equal(got["offsets"], r_off) and np.array_equal(got["perm"], r_perm), what
        assert got["n_active"][0] == r_na and np.array_equal(got["active"], r_act), what
        assert int(got["dev_error"][0]) == 0, what
        assert_close(got["w"], w_ref, f"routing weights {what}")
        ids2 = torch.empty((M, k), dtype=torch.int32, device="cuda")
        w2 = torch.empty((M, k), dtype=torch.float32, device="cuda")
        moe.moe_route(None, None, _dev(lg), k, ids2, w2)
        assert np.array_equal(_host(w2).view(np.uint8), got["w"].view(np.uint8)), what


# ----------------------------------------------------------------------------- combine
@pytest.mark.parametrize("M,k,S,d", [(1, 16, 2, 7168), (16, 16, 2, 7168), (5, 2, 0, 256), (3, 4, 3, 8)])
def test_combine_parity(M, k, S, d):
    moe = _moe()
    g = synth.rng(4, M, d)
    y = g.standard_normal((M * (k + S), d)).astype(np.float32)
    w = g.random((M, k)).astype(np.float32)
    out = torch.empty((M, d), dtype=torch.float32, device="cuda")
    moe.moe_combine(_dev(y), _dev(w), k, S, out)
    assert_close(_host(out), oracle.combine(y, w, k, S), "combine")


# ----------------------------------------------------------------------------- FFN, ragged shapes
RAGGED = [
    synth.LayerShape("r1", 160, 96, 5, 1, 3, -6, -2, 0.05, "f32"),
    synth.LayerShape("r2", 160, 96, 5, 1, 3, -6, -2, 0.05, "bf16"),
    synth.LayerShape("r3", 416, 224, 9, 2, 4, -7, -3, 0.05, "bf16"),
    synth.LayerShape("r4", 96, 32, 3, 0, 1, -5, -1, 0.05, "f32"),
    # f = 640: five whole 128-element steps, so the ring-mode down kernels
    # stage B by LDS DMA (staged scales up to 16 rows, d/32 not a multiple
    # of 16; ring scales beyond)
    synth.LayerShape("r5", 160, 640, 7, 1, 3, -6, -2, 0.05, "bf16"),
]


@pytest.mark.parametrize("shape", RAGGED, ids=lambda s: s.name)
@pytest.mark.parametrize("M", [1, 3, 7, 16, 17, 40])
def test_ffn_ragged_parity(shape, M):
    moe = _moe()
    ex, recs = _small_layer(shape, 5)
    wr = synth.router_weight(shape, 5)
    x = synth.rows_x(shape, 6, M)
    layer = moe.MoELayer(ex, shape.k, M, w_router=_dev(wr))
    res = layer.forward(_x_dev(shape, x))
    ref = oracle.layer(x, shape.k, shape.n_routed, shape.n_shared, shape.d, shape.f, recs.__getitem__, w_r=wr)
    _compare_layer(res, ref, f"{shape.name} M={M}", shape.k, shape.n_shared,
                   rerun=lambda lg: oracle.layer(x, shape.k, shape.n_routed, shape.n_shared, shape.d, shape.f, recs.__getitem__, logits=lg))


# d % 128 == 0: with many rows, experts with more than 16 slots are cut into
# groups of up to 64 slots that run on the wide gate/up kernel and on the
# 32- and 64-column down kernels
WIDE = [
    synth.LayerShape("w1", 256, 96, 5, 1, 2, -6, -2, 0.05, "f32"),
    synth.LayerShape("w2", 384, 160, 6, 1, 2, -6, -2, 0.05, "bf16"),
    # f % 128 == 0: the wide down kernels take their scales through the ring
    # (one 128-element step plus three padding steps; three steps)
    synth.LayerShape("w3", 256, 128, 5, 1, 2, -6, -2, 0.05, "bf16"),
    synth.LayerShape("w4", 384, 384, 6, 1, 2, -6, -2, 0.05, "f32"),
    # f >= 512 in whole steps: every ring-mode down kernel stages B by LDS DMA
    synth.LayerShape("w5", 256, 512, 5, 1, 2, -6, -2, 0.05, "bf16"),
    synth.LayerShape("w6", 384, 640, 6, 1, 2, -6, -2, 0.05, "f32"),
    # bf16 x with d >= 512: the wide gate/up kernel stages x by LDS DMA
    # (d = 640: five steps, padded to eight in whole groups of four)
    synth.LayerShape("w7", 640, 512, 5, 1, 2, -6, -2, 0.05, "bf16"),
]


@pytest.mark.parametrize("shape", WIDE, ids=lambda s: s.name)
@pytest.mark.parametrize("M", [40, 90, 150])
def test_ffn_wide_groups_parity_and_row_identity(shape, M):
    """Parity with the oracle, and every sampled row bit-identical to the
    same row run alone (one-row decode path)."""
    moe = _moe()
    ex, recs = _small_layer(shape, 21)
    wr = synth.router_weight(shape, 21)
    x = synth.rows_x(shape, 22, M)
    xd = _x_dev(shape, x)
    layer = moe.MoELayer(ex, shape.k, M, w_router=_dev(wr))
    res = layer.forward(xd)
    ref = oracle.layer(x, shape.k, shape.n_routed, shape.n_shared, shape.d, shape.f, recs.__getitem__, w_r=wr)
    _compare_layer(res, ref, f"{shape.name} M={M}", shape.k, shape.n_shared,
                   rerun=lambda lg: oracle.layer(x, shape.k, shape.n_routed, shape.n_shared, shape.d, shape.f, recs.__getitem__, logits=lg))
    counts = np.diff(ref["offsets"])
    assert counts.max() > 32, "the case must reach the 64-wide groups"
    one = moe.MoELayer(ex, shape.k, 1)
    lg = res["logits"].clone()
    for m in (0, M // 2, M - 1):
        r1 = one.forward(xd[m:m + 1], logits=lg[m:m + 1].contiguous())
        a = _row_outputs(res, m, shape.k, shape.n_shared)
        b = _row_outputs(r1, 0, shape.k, shape.n_shared)
        for key in ("ids", "w", "y", "out"):
            assert np.array_equal(a[key].view(np.uint8), b[key].view(np.uint8)), (m, key)
    _stages_equal_full(moe, ex, shape.k, xd, layer, layer.forward(xd))


def _stages_equal_full(moe, ex, k, xd, layer, res):
    """moe_ffn_gateup_mxfp4 + moe_ffn_down_mxfp4 == moe_expert_ffn_mxfp4, bit for bit."""
    y_full = _host(res["y_slots"]).copy()
    res["y_slots"].fill_(float("nan"))
    M = xd.shape[0]
    moe.moe_ffn_gateup_mxfp4(xd, k, ex, res["offsets"], res["perm"], res["active"], res["n_active"], layer.workspace)
    moe.moe_ffn_down_mxfp4(M, k, ex, res["offsets"], res["perm"], res["active"], res["n_active"], res["y_slots"],
                           layer.workspace)
    assert np.array_equal(_host(res["y_slots"]).view(np.uint8), y_full.view(np.uint8))


@pytest.mark.parametrize("shape", RAGGED[1:3], ids=lambda s: s.name)
@pytest.mark.parametrize("M", [1, 4, 16, 40])
def test_ffn_stages_equal_full_call(shape, M):
    moe = _moe()
    ex, _ = _small_layer(shape, 11)
    wr = synth.router_weight(shape, 11)
    xd = _x_dev(shape, synth.rows_x(shape, 12, M))
    layer = moe.MoELayer(ex, shape.k, M, w_router=_dev(wr))
    _stages_equal_full(moe, ex, shape.k, xd, layer, layer.forward(xd))


def _layer_outputs(res, M, k, S):
    na = int(_host(res["n_active"])[0])
    return dict(logits=_host(res["logits"][:M]), ids=_host(res["topk_ids"][:M]), w=_host(res["topk_w"][:M]),
                offsets=_host(res["offsets"]), perm=_host(res["perm"][:M * (k + S)]), n_active=np.array([na]),
                active=_host(res["active"])[:na], dev_error=_host(res["dev_error"]),
                y=_host(res["y_slots"][:M * (k + S)]), out=_host(res["out"][:M]))


def _fused_equals_calls(moe, ex, k, xd, w_router, what):
    """moe_layer_mxfp4 == moe_route + moe_bucket + moe_expert_ffn_mxfp4 +
    moe_combine, every output bit for bit (fresh buffers for each side, the
    fused side's poisoned first)."""
    M = xd.shape[0]
    S = ex.n_shared
    outs = []
    for fused in (False, True):
        layer = moe.MoELayer(ex, k, M, w_router=w_router)
        for t in (layer.y_slots, layer.out, layer.topk_w, layer.logits):
            t.fill_(float("nan"))
        for t in (layer.perm, layer.offsets, layer.active, layer.topk_ids):
            t.fill_(-7)
        layer.workspace.fill_(0xA5)  # workspace contents on entry do not matter
        outs.append(_layer_outputs(layer.forward(xd, fused=fused), M, k, S))
    a, b = outs
    for key in a:
        assert np.array_equal(a[key].view(np.uint8), b[key].view(np.uint8)), (what, M, key)


@pytest.mark.parametrize("shape", [synth.TINY] + RAGGED + WIDE, ids=lambda s: s.name)
def test_layer_call_equals_four_calls(shape):
    moe = _moe()
    ex, _ = _small_layer(shape, 31)
    wr = _dev(synth.router_weight(shape, 31))
    for M in (1, 2, 3, 5, 16, 17, 40):
        xd = _x_dev(shape, synth.rows_x(shape, 32 + M, M))
        _fused_equals_calls(moe, ex, shape.k, xd, wr, shape.name)


def test_layer_call_back_to_back_and_given_logits():
    """Calls in a row on one set of buffers with M going up and down, and
    with logits given instead of a router."""
    moe = _moe()
    shape = RAGGED[2]
    ex, recs = _small_layer(shape, 41)
    wr = synth.router_weight(shape, 41)
    layer = moe.MoELayer(ex, shape.k, 16, w_router=_dev(wr))
    for M in (16, 9, 1, 16, 4):
        x = synth.rows_x(shape, 42 + M, M)
        res = layer.forward(_x_dev(shape, x))
        ref = oracle.layer(x, shape.k, shape.n_routed, shape.n_shared, shape.d, shape.f, recs.__getitem__, w_r=wr)
        _compare_layer(res, ref, f"back-to-back M={M}", shape.k, shape.n_shared,
                       rerun=lambda lg: oracle.layer(x, shape.k, shape.n_routed, shape.n_shared, shape.d, shape.f, recs.__getitem__, logits=lg))
    lg = synth.random_logits(43, 7, shape.n_routed)
    x = synth.rows_x(shape, 44, 7)
    given = moe.MoELayer(ex, shape.k, 7)
    res = given.forward(_x_dev(shape, x), logits=_dev(lg))
    ref = oracle.layer(x, shape.k, shape.n_routed, shape.n_shared, shape.d, shape.f, recs.__getitem__, logits=lg)
    _compare_layer(res, ref, "given logits", shape.k, shape.n_shared)


def test_wide_groups_scale_bytes_after_the_plane():
    """The wide gate/up kernel reads a scale dword per lane for each step of a
    4-step group; with d/128 not a multiple of 4 the last group has padding
    steps, whose dwords lie past a row's scale bytes.  Codes bytes of 0xFF
    right after the W_gate and W_up scale planes (the first bytes of the
    W_up and W_down codes planes: valid E2M1 data) must not reach the
    arithmetic as scales: the layer still matches the oracle."""
    moe = _moe()
    shape = synth.LayerShape("pad", 384, 32, 3, 1, 2, -6, -2, 0.05, "bf16")
    seed, M = 7, 24  # the shared expert's 24 slots form a 32-wide group
    c, sc = shape.f * shape.d // 2, shape.f * shape.d // 32
    recs = {}
    for e in range(shape.n_experts):
        r = synth.expert_record(shape, seed, e).copy()
        r[c + sc:c + sc + 16] = 0xFF              # first bytes of W_up codes
        r[2 * (c + sc):2 * (c + sc) + 16] = 0xFF  # first bytes of W_down codes
        recs[e] = r
    base = torch.from_numpy(np.concatenate([recs[e] for e in range(shape.n_experts)])).cuda()
    ex = moe.Experts(base, shape.stride, shape.d, shape.f, shape.n_routed, shape.n_shared)
    wr = synth.router_weight(shape, seed)
    x = synth.rows_x(shape, seed, M)
    layer = moe.MoELayer(ex, shape.k, M, w_router=_dev(wr))
    layer.workspace.fill_(0xFF)
    res = layer.forward(_x_dev(shape, x))
    ref = oracle.layer(x, shape.k, shape.n_routed, shape.n_shared, shape.d, shape.f, recs.__getitem__, w_r=wr)
    _compare_layer(res, ref, "scale bytes after the plane", shape.k, shape.n_shared,
                   rerun=lambda lg: oracle.layer(x, shape.k, shape.n_routed, shape.n_shared, shape.d, shape.f, recs.__getitem__, logits=lg))


# ----------------------------------------------------------------------------- Kimi decode
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_kimi_one_row_parity(kimi_layer, seed):
    moe = _moe()
    L = kimi_layer
    shp = L["shape"]
    x = synth.rows_x(shp, 100 + seed, 1)
    layer = moe.MoELayer(L["experts"], shp.k, 1, w_router=L["wr_dev"])
    res = layer.forward(_x_dev(shp, x))
    ref = oracle.layer(x, shp.k, shp.n_routed, shp.n_shared, shp.d, shp.f, L["rec"], w_r=L["wr"])
    _compare_layer(res, ref, f"kimi 1 row seed {seed}", shp.k, shp.n_shared,
                   rerun=lambda lg: oracle.layer(x, shp.k, shp.n_routed, shp.n_shared, shp.d, shp.f, L["rec"], logits=lg))
    # the down pass's two-part h (|h - hi - lo| <= 2^-18 |h|, rounded to
    # nearest) leaves about 2.5e-6 relative L2 at this shape; a split with a
    # truncated hi part would leave about 5e-6
    r, _ = assert_close(_host(res["out"]), ref["out"], f"kimi 1 row seed {seed} out", rel=4e-6, maxabs_frac=1e-5)
    print(f"kimi 1 row seed {seed}: out rel L2 {r:.2e}", flush=True)


def _row_outputs(res, m, k, S):
    kps = k + S
    return dict(logits=_host(res["logits"][m]), ids=_host(res["topk_ids"][m]), w=_host(res["topk_w"][m]),
                y=_host(res["y_slots"][m * kps:(m + 1) * kps]), out=_host(res["out"][m]))


@pytest.mark.parametrize("B", [2, 8, 16])
def test_kimi_block_rows_equal_single_rows(kimi_layer, B):
    """Every row of a block is bit-identical to the same row called alone."""
    moe = _moe()
    L = kimi_layer
    shp = L["shape"]
    blk = moe.MoELayer(L["experts"], shp.k, B, w_router=L["wr_dev"])
    one = moe.MoELayer(L["experts"], shp.k, 1, w_router=L["wr_dev"])
    for seed in range(20):  # 20 seeded blocks per block size
        x = synth.block_x(shp, seed, B)
        xd = _x_dev(shp, x)
        rb = blk.forward(xd)
        for m in range(B):
            r1 = one.forward(xd[m:m + 1])
            a = _row_outputs(rb, m, shp.k, shp.n_shared)
            b = _row_outputs(r1, 0, shp.k, shp.n_shared)
            for key in a:
                assert np.array_equal(a[key].view(np.uint8), b[key].view(np.uint8)), (B, seed, m, key)


@pytest.mark.parametrize("B", [2, 8, 16])
def test_kimi_block_parity_all_seeds(kimi_layer, B):
    """The verification-block workload: 20 seeded blocks per block size (row 0
    x0 ~ N(0,1), rows i > 0 x0 + N(0, 0.3^2)), every output of every block
    against the oracle."""
    moe = _moe()
    L = kimi_layer
    shp = L["shape"]
    layer = moe.MoELayer(L["experts"], shp.k, B, w_router=L["wr_dev"])
    unions = []
    for seed in range(20):
        x = synth.block_x(shp, seed, B)
        res = layer.forward(_x_dev(shp, x))
        ref = oracle.layer(x, shp.k, shp.n_routed, shp.n_shared, shp.d, shp.f, L["rec"], w_r=L["wr"])
        _compare_layer(res, ref, f"kimi block {B} seed {seed}", shp.k, shp.n_shared,
                       rerun=lambda lg: oracle.layer(x, shp.k, shp.n_routed, shp.n_shared, shp.d, shp.f, L["rec"],
                                                     logits=lg))
        unions.append(int(ref["n_active"]))
        print(f"block of {B} seed {seed}: U+S = {unions[-1]}", flush=True)
    print(f"block of {B}: U+S mean {np.mean(unions):.1f}, range {min(unions)}-{max(unions)}", flush=True)


@pytest.mark.parametrize("sigma", [0.5, 1.0])
def test_kimi_block16_wider_unions(kimi_layer, sigma):
    """16-row blocks whose rows spread further from row 0 (sigma 0.5 and 1.0)
    reach the upper end of the pages' block unions (about 40 to 120 experts):
    5 seeded blocks each, every output against the oracle, and every row
    bit-identical to the same row called alone."""
    moe = _moe()
    L = kimi_layer
    shp = L["shape"]
    blk = moe.MoELayer(L["experts"], shp.k, 16, w_router=L["wr_dev"])
    one = moe.MoELayer(L["experts"], shp.k, 1, w_router=L["wr_dev"])
    unions = []
    for seed in range(100, 105):
        x = synth.block_x(shp, seed, 16, sigma=sigma)
        xd = _x_dev(shp, x)
        res = blk.forward(xd)
        ref = oracle.layer(x, shp.k, shp.n_routed, shp.n_shared, shp.d, shp.f, L["rec"], w_r=L["wr"])
        _compare_layer(res, ref, f"kimi block 16 sigma {sigma} seed {seed}", shp.k, shp.n_shared,
                       rerun=lambda lg: oracle.layer(x, shp.k, shp.n_routed, shp.n_shared, shp.d, shp.f, L["rec"],
                                                     logits=lg))
        for m in range(16):
            r1 = one.forward(xd[m:m + 1])
            a = _row_outputs(res, m, shp.k, shp.n_shared)
            b = _row_outputs(r1, 0, shp.k, shp.n_shared)
            for key in a:
                assert np.array_equal(a[key].view(np.uint8), b[key].view(np.uint8)), (sigma, seed, m, key)
        unions.append(int(ref["n_active"]))
        print(f"block of 16, sigma {sigma}, seed {seed}: U+S = {unions[-1]}", flush=True)
    assert max(unions) > 47, "wider spreads must reach larger unions than sigma 0.3"


def test_kimi_expert_order_independence(kimi_layer):
    """Outputs do not depend on the order experts are computed in."""
    moe = _moe()
    L = kimi_layer
    shp = L["shape"]
    x = _x_dev(shp, synth.block_x(shp, 3, 16))
    layer = moe.MoELayer(L["experts"], shp.k, 16, w_router=L["wr_dev"])
    res = layer.forward(x)
    y_ref = _host(res["y_slots"]).copy()
    na = int(_host(res["n_active"])[0])
    act = res["active"]
    g = torch.Generator().manual_seed(0)
    for order in ("reverse", "shuffle"):
        idx = torch.arange(na - 1, -1, -1) if order == "reverse" else torch.randperm(na, generator=g)
        act[:na] = act[:na][idx.cuda()].clone()
        res["y_slots"].zero_()
        moe.moe_expert_ffn_mxfp4(x, shp.k, L["experts"], res["offsets"], res["perm"], act, res["n_active"],
                                 res["y_slots"], layer.workspace)
        assert np.array_equal(_host(res["y_slots"]).view(np.uint8), y_ref.view(np.uint8)), order


@pytest.mark.parametrize("M", [1, 4, 16])
def test_kimi_layer_call_equals_four_calls(kimi_layer, M):
    moe = _moe()
    L = kimi_layer
    shp = L["shape"]
    xd = _x_dev(shp, synth.block_x(shp, 7, M))
    _fused_equals_calls(moe, L["experts"], shp.k, xd, L["wr_dev"], "kimi")


@pytest.mark.parametrize("M", [1, 16])
def test_kimi_stages_equal_full_call(kimi_layer, M):
    moe = _moe()
    L = kimi_layer
    shp = L["shape"]
    xd = _x_dev(shp, synth.block_x(shp, 4, M))
    layer = moe.MoELayer(L["experts"], shp.k, M, w_router=L["wr_dev"])
    _stages_equal_full(moe, L["experts"], shp.k, xd, layer, layer.forward(xd))


@pytest.mark.parametrize("M", [1, 16])
def test_kimi_layer_graph_replay(kimi_layer, M):
    """The whole layer pass captured in a HIP graph: every replay, with eager
    work and synchronisation in between, equals the eager pass bit for bit."""
    moe = _moe()
    L = kimi_layer
    shp = L["shape"]
    xs = [_x_dev(shp, synth.block_x(shp, 20 + i, M)) for i in range(2)]
    layer = moe.MoELayer(L["experts"], shp.k, M, w_router=L["wr_dev"])
    eager = []
    for x in xs:
        r = layer.forward(x)
        eager.append((_host(r["out"]).copy(), _host(r["y_slots"]).copy(), _host(r["topk_ids"]).copy()))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graphs = []
    for x in xs:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            layer.forward(x)
        graphs.append(g)
    torch.cuda.synchronize()
    for rep in range(3):
        for i, g in enumerate(graphs):
            layer.out.fill_(float("nan"))
            layer.y_slots.fill_(float("nan"))
            g.replay()
            torch.cuda.synchronize()
            out, y, ids = eager[i]
            assert np.array_equal(_host(layer.out[:M]).view(np.uint8), out.view(np.uint8)), (rep, i, "out")
            assert np.array_equal(_host(layer.y_slots[:len(y)]).view(np.uint8), y.view(np.uint8)), (rep, i, "y")
            assert np.array_equal(_host(layer.topk_ids[:M]), ids), (rep, i, "ids")
            layer.forward(xs[1 - i])  # eager work between replays
            torch.cuda.synchronize()


# ----------------------------------------------------------------------------- prefill
@pytest.mark.parametrize("M", [270, 1533])
def test_kimi_prefill_parity_sampled(kimi_layer, M):
    moe = _moe()
    L = kimi_layer
    shp = L["shape"]
    kps = shp.k + shp.n_shared
    x = synth.rows_x(shp, 7, M)
    lg = synth.zipf_logits(shp, 7, M)
    layer = moe.MoELayer(L["experts"], shp.k, M)
    res = layer.forward(_x_dev(shp, x), logits=_dev(lg))
    ids_ref, w_ref = oracle.topk(lg, shp.k)
    assert np.array_equal(_host(res["topk_ids"]), ids_ref)
    off_ref, perm_ref, act_ref, na_ref = oracle.bucket(ids_ref, shp.n_routed, shp.n_shared)
    assert np.array_equal(_host(res["offsets"]), off_ref) and np.array_equal(_host(res["perm"]), perm_ref)
    y = _host(res["y_slots"])
    out = _host(res["out"])
    xf = oracle.as_f32_rows(x)
    # sampled rows: every slot of these rows, and their combined output
    g = synth.rng(8, M)
    rows = sorted(set([0, M - 1] + list(g.choice(M, 3, replace=False))))
    for m in rows:
        y_ref = np.zeros((kps, shp.d), np.float32)
        for j in range(kps):
            e = int(ids_ref[m, j]) if j < shp.k else shp.n_routed + j - shp.k
            y_ref[j] = oracle.expert_ffn(xf[m:m + 1], L["rec"](e), shp.d, shp.f)[0]
        assert_close(y[m * kps:(m + 1) * kps], y_ref, f"prefill M={M} row {m} y_slots")
        o_ref = oracle.combine(y_ref, w_ref[m:m + 1], shp.k, shp.n_shared)
        assert_close(out[m:m + 1], o_ref, f"prefill M={M} row {m} out")
    # slots from every kind of group the many-row path forms: an expert with
    # at most 16 slots is one narrow group; a longer segment is cut into
    # groups of 64 slots plus a remainder that is narrow (<= 16), 32-wide
    # (17..32) or 64-wide (33..63); the first, middle and last slot of two
    # groups of each kind (the hottest routed expert's first 64-group among them)
    samples = {"narrow": [], "32-wide": [], "64-wide": []}
    for e in np.argsort(-np.diff(off_ref), kind="stable"):
        seg = perm_ref[off_ref[e]:off_ref[e + 1]]
        n = len(seg)
        if n == 0:
            continue
        if n <= 16:
            groups = [("narrow", seg)]
        else:
            full, rem = n // 64, n % 64
            groups = [("64-wide", seg[64 * j:64 * (j + 1)]) for j in range(full)]
            if rem:
                groups.append(("narrow" if rem <= 16 else "32-wide" if rem <= 32 else "64-wide", seg[64 * full:]))
        for kind, gs in groups:
            if len(samples[kind]) < 2:
                samples[kind].append((int(e), gs))
    for kind, got in samples.items():
        assert got, f"prefill M={M}: no {kind} group to sample"
        for e, gs in got:
            for t in sorted({int(gs[0]), int(gs[len(gs) // 2]), int(gs[-1])}):
                m = t // kps
                y_ref = oracle.expert_ffn(xf[m:m + 1], L["rec"](e), shp.d, shp.f)[0]
                assert_close(y[t], y_ref, f"prefill M={M} {kind} group of expert {e}, slot {t}")
    print(f"prefill M={M}: sampled " + ", ".join(f"{len(v)} {k} groups" for k, v in samples.items()), flush=True)


def test_kimi_prefill_rows_equal_decode_rows(kimi_layer):
    """The >16-row path runs the same per-slot arithmetic as the decode path."""
    moe = _moe()
    L = kimi_layer
    shp = L["shape"]
    M = 270
    x = _x_dev(shp, synth.rows_x(shp, 9, M))
    lg = _dev(synth.zipf_logits(shp, 9, M))
    big = moe.MoELayer(L["experts"], shp.k, M)
    rb = big.forward(x, logits=lg)
    one = moe.MoELayer(L["experts"], shp.k, 1)
    for m in (0, 57, 269):
        r1 = one.forward(x[m:m + 1], logits=lg[m:m + 1].contiguous())
        a = _row_outputs(rb, m, shp.k, shp.n_shared)
        b = _row_outputs(r1, 0, shp.k, shp.n_shared)
        for key in ("ids", "w", "y", "out"):
            assert np.array_equal(a[key].view(np.uint8), b[key].view(np.uint8)), (m, key)


# ----------------------------------------------------------------------------- Q8_0
def _q8(seed, K, N, M):
    wq, ws = synth.q8_0_weight(seed, K, N)
    X = synth.q8_0_x(seed, M, K)
    return X, wq, ws


@pytest.mark.parametrize("K,N,M", [(K, N, M) for (K, N) in [(7168, 7168), (256, 100), (96, 33), (7168, 18432)]
                                    for M in (1, 2, 4, 8)]
                         + [(K, N, M) for (K, N) in [(7168, 7168), (512, 70)] for M in (3, 5, 6, 7)])
def test_q8_0_parity(K, N, M):
    moe = _moe()
    X, wq, ws = _q8(10, K, N, M)
    Y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    moe.q8_0_matmul(_dev(X), _dev(wq), _dev(ws, torch.int16), Y)
    assert_close(_host(Y), oracle.q8_0_matmul(X, wq, ws), f"q8_0 K={K} N={N} M={M}")


def test_q8_0_large_sampled_and_row_invariance():
    moe = _moe()
    K, N = 7168, 163840
    wq, ws = synth.q8_0_weight(11, K, N)
    X = synth.q8_0_x(11, 8, K)
    dwq, dws = _dev(wq), _dev(ws, torch.int16)
    Y8 = torch.empty((8, N), dtype=torch.float32, device="cuda")
    moe.q8_0_matmul(_dev(X), dwq, dws, Y8)
    y8 = _host(Y8)
    cols = np.sort(synth.rng(12).choice(N, 512, replace=False))
    ref = oracle.q8_0_matmul(X, wq[cols], ws[cols])
    assert_close(y8[:, cols], ref, "q8_0 163840 sampled")
    for M in (1, 2, 3, 4, 5, 6, 7):
        YM = torch.empty((M, N), dtype=torch.float32, device="cuda")
        moe.q8_0_matmul(_dev(X[:M]), dwq, dws, YM)
        assert np.array_equal(_host(YM).view(np.uint8), y8[:M].view(np.uint8)), M


def test_q8_0_unaligned_scales():
    """A scale plane that is not 16-byte aligned takes the per-element load
    path; the result is the oracle's, and bit-identical to the aligned call."""
    moe = _moe()
    K, N, M = 7168, 300, 3
    X, wq, ws = _q8(13, K, N, M)
    dwq = _dev(wq)
    flat = torch.zeros(N * (K // 32) + 8, dtype=torch.int16, device="cuda")
    dws_u = flat[1:1 + N * (K // 32)].view(N, K // 32)  # 2 bytes past a 16-byte boundary
    dws_u.copy_(torch.from_numpy(ws.view(np.int16)))
    assert dws_u.data_ptr() % 16 != 0
    Yu = torch.empty((M, N), dtype=torch.float32, device="cuda")
    Ya = torch.empty((M, N), dtype=torch.float32, device="cuda")
    moe.q8_0_matmul(_dev(X), dwq, dws_u, Yu)
    moe.q8_0_matmul(_dev(X), dwq, _dev(ws, torch.int16), Ya)
    assert_close(_host(Yu), oracle.q8_0_matmul(X, wq, ws), "q8_0 unaligned scales")
    assert np.array_equal(_host(Yu).view(np.uint8), _host(Ya).view(np.uint8))
