"""Seeded random layer shapes through the whole layer call on the GPU, each
against the oracle, with row 0 of every block checked bit for bit against
the same row run alone, and the tile-ordered records against row order.
d and f come from sizes the fixed-shape tests already cover; E, k, S, M and
the x dtype vary around them (M on both sides of the 16-row switch to the
grouped prefill path).  MOE_RANDOM_SEED and MOE_RANDOM_CASES (layer cases;
the Q8_0 cases are a third of that) draw another set.  Needs an MI355X."""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from conftest import assert_close

pytestmark = pytest.mark.gpu

SEED = int(os.environ.get("MOE_RANDOM_SEED", "20261202"))
N_CASES = int(os.environ.get("MOE_RANDOM_CASES", "60"))
D_CHOICES = (32, 64, 96, 128, 160, 256, 384, 416, 512, 640, 768, 1024)
F_CHOICES = (32, 64, 96, 128, 160, 224, 256, 288, 352, 512)
E_CHOICES = (1, 2, 3, 4, 5, 9, 16, 33, 64, 100, 300, 896)
M_CHOICES = (1, 2, 3, 4, 5, 6, 8, 13, 15, 16, 17, 24, 33, 40, 64, 65, 130, 200, 333)


def _moe():
    import router_top_bucket_amd as moe
    return moe


def _cases():
    g = np.random.default_rng(SEED)
    out = []
    for i in range(N_CASES):
        d = int(g.choice(D_CHOICES))
        f = int(g.choice(F_CHOICES))
        E = int(g.choice(E_CHOICES))
        k = int(g.integers(1, min(E, 16) + 1))
        S = int(g.integers(0, 4))
        M = int(g.choice(M_CHOICES))
        dt = "bf16" if g.integers(0, 2) else "f32"
        out.append((synth.LayerShape(f"rnd{i}", d, f, E, S, k, -6, -2, 0.05, dt), M, 1000 + i))
    return out


def _host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _x_dev(shape, x):
    t = torch.from_numpy(np.ascontiguousarray(x))
    return (t.view(torch.bfloat16) if shape.x_dtype == "bf16" else t).cuda()


def _outputs(res, M, k, S):
    kps = k + S
    na = int(_host(res["n_active"])[0])
    return dict(logits=_host(res["logits"][:M]), ids=_host(res["topk_ids"][:M]), w=_host(res["topk_w"][:M]),
                offsets=_host(res["offsets"]), perm=_host(res["perm"][:M * kps]), active=_host(res["active"])[:na],
                y=_host(res["y_slots"][:M * kps]), out=_host(res["out"][:M]), dev_error=_host(res["dev_error"]))


@pytest.mark.parametrize("shape,M,seed", _cases(), ids=lambda v: v.name if hasattr(v, "name") else str(v))
def test_random_shape_layer(shape, M, seed):
    moe = _moe()
    k, S = shape.k, shape.n_shared
    base = synth.device_experts(shape, seed)
    ex = moe.Experts(base, shape.stride, shape.d, shape.f, shape.n_routed, shape.n_shared)
    recs = {e: synth.expert_record(shape, seed, e) for e in range(shape.n_experts)}
    wr = synth.router_weight(shape, seed)
    wr_d = torch.from_numpy(wr).cuda()
    x = synth.rows_x(shape, seed, M)
    what = f"{shape} M={M}"

    res = moe.MoELayer(ex, k, M, w_router=wr_d).forward(_x_dev(shape, x))
    got = _outputs(res, M, k, S)
    assert_close(got["logits"], oracle.router_logits(x, wr), what + " logits")
    # The top-k decision and everything after it against the oracle on the
    # same fp32 logits the GPU decided on: the two logit sums agree only to
    # rounding, and two experts whose logits tie within it may rank either way.
    ref = oracle.layer(x, k, shape.n_routed, S, shape.d, shape.f, recs.__getitem__, logits=got["logits"])
    assert np.array_equal(got["ids"], ref["ids"]), what + " ids"
    assert_close(got["w"], ref["w"], what + " w")
    assert np.array_equal(got["offsets"], ref["offsets"]) and np.array_equal(got["perm"], ref["perm"]), what
    assert np.array_equal(got["active"], ref["active"]) and int(got["dev_error"][0]) == 0, what
    assert_close(got["y"], ref["y_slots"], what + " y_slots")
    assert_close(got["out"], ref["out"], what + " out")

    if M > 1:  # row 0 of the block against the row alone, bit for bit
        # (above 16 rows the router's MFMA form agrees with the one-row logits
        # within rounding only: there the row alone is routed on the block's
        # logits, and everything after the router must match bit for bit)
        given = None if M <= 16 else res["logits"][:1].clone()
        one_layer = moe.MoELayer(ex, k, 1, w_router=None if given is not None else wr_d)
        one = _outputs(one_layer.forward(_x_dev(shape, x[:1]), logits=given), 1, k, S)
        for key in ("logits", "ids", "w", "out"):
            assert np.array_equal(got[key][:1].view(np.uint8), one[key].view(np.uint8)), (what, key)
        assert np.array_equal(got["y"][:k + S].view(np.uint8), one["y"].view(np.uint8)), (what, "y")

    # tile-ordered records give the same bits
    tiles = moe.tile_experts(ex)
    got_t = _outputs(moe.MoELayer(tiles, k, M, w_router=wr_d).forward(_x_dev(shape, x)), M, k, S)
    for key in ("y", "out"):
        assert np.array_equal(got_t[key].view(np.uint8), got[key].view(np.uint8)), (what, "tiles", key)


# ----------------------------------------------------------------------------- Q8_0
def _q8_cases():
    g = np.random.default_rng(SEED + 1)
    out = []
    for i in range(max(1, N_CASES // 3)):
        K = int(g.choice((32, 64, 96, 128, 160, 224, 512, 1024, 2048, 2080, 4096, 7168)))
        N = int(g.choice((1, 2, 5, 15, 16, 17, 31, 48, 100, 256, 1000, 4096, 8192)))
        M = int(g.integers(1, 9))
        out.append((K, N, M, 7000 + i))
    return out


@pytest.mark.parametrize("K,N,M,seed", _q8_cases())
def test_random_shape_q8_0(K, N, M, seed):
    """Q8_0 against the oracle; row 0 of M rows equals the row alone bit for
    bit; the tile-ordered plane (N % 16 == 0) gives the same bits."""
    moe = _moe()
    wq, ws = synth.q8_0_weight(seed, K, N)
    X = synth.q8_0_x(seed, M, K)
    dwq = torch.from_numpy(wq).cuda()
    dws = torch.from_numpy(ws.view(np.int16)).cuda()
    Y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    moe.q8_0_matmul(torch.from_numpy(X).cuda(), dwq, dws, Y)
    got = _host(Y)
    assert_close(got, oracle.q8_0_matmul(X, wq, ws), f"q8_0 K={K} N={N} M={M}")
    Y1 = torch.empty((1, N), dtype=torch.float32, device="cuda")
    moe.q8_0_matmul(torch.from_numpy(X[:1].copy()).cuda(), dwq, dws, Y1)
    assert np.array_equal(_host(Y1).view(np.uint32), got[:1].view(np.uint32)), (K, N, M)
    if N % 16 == 0:
        tq = torch.empty_like(dwq)
        moe.q8_0_pack(dwq, tq, moe.MOE_LAYOUT_TILES)
        Yt = torch.empty_like(Y)
        moe.q8_0_matmul(torch.from_numpy(X).cuda(), tq, dws, Yt, layout=moe.MOE_LAYOUT_TILES)
        assert np.array_equal(_host(Yt).view(np.uint32), got.view(np.uint32)), (K, N, M, "tiles")
