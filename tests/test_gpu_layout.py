"""Tile-ordered codes planes (MOE_LAYOUT_TILES): the packer against the
header's placement formula, packing back restores every byte, and every
output of the layer is bit-identical for the two orders (small, ragged, wide
and Kimi shapes; decode, blocks, prefill; streamed).  Needs an MI355X."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _moe():
    import router_top_bucket_amd as moe
    return moe


def _tiles_ref(rec: np.ndarray, d: int, f: int) -> np.ndarray:
    """The tile order of one record, from the placement rule: block kb of row
    `row` of a codes plane with K columns goes to ((row/16)*(K/32)+kb)*256 +
    (row%16)*16; everything else stays."""
    out = rec.copy()
    pc, ps = f * d // 2, f * d // 32
    for base, rows, K in ((0, f, d), (pc + ps, f, d), (2 * (pc + ps), d, f)):
        nb = K // 32
        blocks = rec[base:base + pc].reshape(rows, nb, 16)
        tiled = blocks.reshape(rows // 16, 16, nb, 16).transpose(0, 2, 1, 3)  # [tile][kb][row%16][16]
        out[base:base + pc] = tiled.reshape(-1)
    return out


SHAPES = [synth.TINY,
          synth.LayerShape("r2", 160, 96, 5, 1, 3, -6, -2, 0.05, "bf16"),
          synth.LayerShape("r3", 416, 224, 9, 2, 4, -7, -3, 0.05, "bf16"),
          synth.LayerShape("w1", 256, 96, 5, 1, 2, -6, -2, 0.05, "f32")]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: s.name)
def test_pack_matches_rule_and_round_trips(shape):
    moe = _moe()
    base = synth.device_experts(shape, 61)
    n = shape.n_experts
    tiled = torch.empty_like(base)
    back = torch.empty_like(base)
    moe.moe_pack_experts(base, tiled, n, shape.stride, shape.d, shape.f, moe.MOE_LAYOUT_TILES)
    moe.moe_pack_experts(tiled, back, n, shape.stride, shape.d, shape.f, moe.MOE_LAYOUT_ROWS)
    torch.cuda.synchronize()
    assert torch.equal(back, base)
    host = base.cpu().numpy()
    got = tiled.cpu().numpy()
    for e in range(n):
        rec = host[e * shape.stride:(e + 1) * shape.stride]
        assert np.array_equal(got[e * shape.stride:(e + 1) * shape.stride], _tiles_ref(rec, shape.d, shape.f)), e
    assert not torch.equal(tiled, base)


def _outputs(res, M, k, S):
    torch.cuda.synchronize()
    na = int(res["n_active"][0].item())
    return dict(ids=res["topk_ids"][:M].cpu().numpy(), w=res["topk_w"][:M].cpu().numpy(),
                perm=res["perm"][:M * (k + S)].cpu().numpy(), active=res["active"][:na].cpu().numpy(),
                y=res["y_slots"][:M * (k + S)].cpu().numpy(), out=res["out"][:M].cpu().numpy())


def _x(shape, seed, M):
    t = torch.from_numpy(np.ascontiguousarray(synth.rows_x(shape, seed, M)))
    return (t.view(torch.bfloat16) if shape.x_dtype == "bf16" else t).cuda()


def _same(a, b, what):
    for key in a:
        assert np.array_equal(a[key].view(np.uint8), b[key].view(np.uint8)), (what, key)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: s.name)
def test_layer_tiles_equal_rows(shape):
    moe = _moe()
    rows = moe.Experts(synth.device_experts(shape, 62), shape.stride, shape.d, shape.f, shape.n_routed,
                       shape.n_shared)
    tiles = moe.tile_experts(rows)
    wr = torch.from_numpy(synth.router_weight(shape, 62)).cuda()
    for M in (1, 2, 3, 5, 16, 17, 40, 90, 150):
        x = _x(shape, 63 + M, M)
        a = _outputs(moe.MoELayer(rows, shape.k, M, w_router=wr).forward(x), M, shape.k, shape.n_shared)
        b = _outputs(moe.MoELayer(tiles, shape.k, M, w_router=wr).forward(x), M, shape.k, shape.n_shared)
        _same(a, b, f"{shape.name} M={M}")


@pytest.fixture(scope="module")
def kimi_rows_tiles():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe = _moe()
    shp = synth.KIMI
    rows = moe.Experts(synth.device_experts(shp, 0), shp.stride, shp.d, shp.f, shp.n_routed, shp.n_shared)
    return shp, rows, moe.tile_experts(rows), torch.from_numpy(synth.router_weight(shp, 0)).cuda()


@pytest.mark.parametrize("M", [1, 2, 16])
def test_kimi_tiles_equal_rows_decode(kimi_rows_tiles, M):
    moe = _moe()
    shp, rows, tiles, wr = kimi_rows_tiles
    x = torch.from_numpy(synth.block_x(shp, 70 + M, M)).view(torch.bfloat16).cuda()
    a = _outputs(moe.MoELayer(rows, shp.k, M, w_router=wr).forward(x), M, shp.k, shp.n_shared)
    b = _outputs(moe.MoELayer(tiles, shp.k, M, w_router=wr).forward(x), M, shp.k, shp.n_shared)
    _same(a, b, f"kimi M={M}")


def test_kimi_tiles_equal_rows_prefill(kimi_rows_tiles):
    moe = _moe()
    shp, rows, tiles, _ = kimi_rows_tiles
    M = 270
    x = torch.from_numpy(synth.rows_x(shp, 71, M)).view(torch.bfloat16).cuda()
    lg = torch.from_numpy(synth.zipf_logits(shp, 71, M)).cuda()
    a = _outputs(moe.MoELayer(rows, shp.k, M).forward(x, logits=lg), M, shp.k, shp.n_shared)
    b = _outputs(moe.MoELayer(tiles, shp.k, M).forward(x, logits=lg), M, shp.k, shp.n_shared)
    _same(a, b, "kimi prefill 270")


def test_streamed_tiles_equal_resident_rows():
    moe = _moe()
    shape = SHAPES[2]
    k, E, S = shape.k, shape.n_routed, shape.n_shared
    rec = shape.n_experts * shape.stride
    seeds = [81, 82]
    host = torch.empty(len(seeds) * rec, dtype=torch.uint8, pin_memory=True)
    resident = []
    for l, s in enumerate(seeds):
        rows = moe.Experts(synth.device_experts(shape, s), shape.stride, shape.d, shape.f, E, S)
        resident.append(rows)
        host[l * rec:(l + 1) * rec].copy_(moe.tile_experts(rows).base)
    routers = [torch.from_numpy(synth.router_weight(shape, s)).cuda() for s in seeds]
    n_slots = len(seeds) * S + 2 + (E - 2)
    pool = torch.zeros(n_slots * shape.stride, dtype=torch.uint8, device="cuda")
    cache = moe.ExpertCache(pool, host, len(seeds), E, S, shape.d, shape.f, shape.stride, n_upload_streams=2,
                            upload_groups=3, n_transient=2, layout=moe.MOE_LAYOUT_TILES)
    st = moe.MoELayer(cache.descriptor(), k, 16)
    for i, (layer, M) in enumerate([(0, 1), (1, 5), (0, 16), (1, 1), (0, 3)]):
        x = _x(shape, 90 + i, M)
        a = _outputs(moe.MoELayer(resident[layer], k, M, w_router=routers[layer]).forward(x), M, k, S)
        st.w_router = routers[layer]
        b = _outputs(st.forward_streamed(cache, layer, x), M, k, S)
        _same(a, b, f"streamed call {i}")
    cache.close()


# ----------------------------------------------------------------------------- Q8_0 weights
def _q8_tiles_ref(wq: np.ndarray) -> np.ndarray:
    """Tile order of an int8 plane [N x K]: block b of row n goes to
    ((n/16)*(K/32) + b)*512 + (n%16)*32."""
    N, K = wq.shape
    return wq.reshape(N // 16, 16, K // 32, 32).transpose(0, 2, 1, 3).reshape(-1)


@pytest.mark.parametrize("N,K", [(48, 96), (7168, 7168), (160, 416)])
def test_q8_0_pack_rule_and_round_trip(N, K):
    moe = _moe()
    wq, _ = synth.q8_0_weight(5, K, N)
    src = torch.from_numpy(wq).cuda()
    t = torch.empty_like(src)
    back = torch.empty_like(src)
    moe.q8_0_pack(src, t, moe.MOE_LAYOUT_TILES)
    moe.q8_0_pack(t, back, moe.MOE_LAYOUT_ROWS)
    torch.cuda.synchronize()
    assert torch.equal(back, src)
    assert np.array_equal(t.cpu().numpy().reshape(-1), _q8_tiles_ref(wq))


@pytest.mark.parametrize("K,N", [(7168, 7168), (7168, 18432), (256, 96), (96, 48), (416, 160)])
def test_q8_0_tiles_equal_rows(K, N):
    moe = _moe()
    wq, ws = synth.q8_0_weight(6, K, N)
    dwq = torch.from_numpy(wq).cuda()
    tiles = torch.empty_like(dwq)
    moe.q8_0_pack(dwq, tiles, moe.MOE_LAYOUT_TILES)
    # aligned scales (fast path where K allows) and scales one element off
    # 16-byte alignment (the masked path)
    sbuf = torch.from_numpy(np.concatenate([np.zeros(1, np.uint16), ws.reshape(-1)]).view(np.int16)).cuda()
    for dws in (torch.from_numpy(ws.view(np.int16)).cuda(), sbuf[1:].view(N, K // 32)):
        for M in range(1, 9):
            X = torch.from_numpy(synth.q8_0_x(7, M, K)).cuda()
            Ya = torch.empty((M, N), dtype=torch.float32, device="cuda")
            Yb = torch.empty_like(Ya)
            moe.q8_0_matmul(X, dwq, dws, Ya)
            moe.q8_0_matmul(X, tiles, dws, Yb, layout=moe.MOE_LAYOUT_TILES)
            torch.cuda.synchronize()
            assert torch.equal(Ya.view(torch.int32), Yb.view(torch.int32)), (K, N, M)
