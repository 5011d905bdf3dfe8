"""moe_layer_mxfp4_noalloc, the layer call whose scratch is the library's
static device array, against moe_layer_mxfp4 with a caller workspace: every
output bit for bit, over two calls in a row on one set of buffers, the second
with fewer rows.  Needs an MI355X."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SHAPES = [
    (synth.TINY, (16, 3), False),
    (synth.LayerShape("r3", 416, 224, 9, 2, 4, -7, -3, 0.05, "bf16"), (40, 5), False),
    # d % 128 == 0: above 16 rows the group plan and the wide groups use the scratch too
    (synth.LayerShape("w2", 384, 160, 6, 1, 2, -6, -2, 0.05, "bf16"), (150, 17), False),
    # the Kimi widths with few experts, tile-ordered records
    (synth.LayerShape("kd", 7168, 1536, 24, 2, 16, -8, -4, 0.02, "bf16"), (16, 1), True),
]


def _moe():
    import router_top_bucket_amd as moe
    return moe


def _buffers(M, k, E, S, d):
    i32 = dict(dtype=torch.int32, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    T = M * (k + S)
    b = dict(logits=torch.empty((M, E), **f32), topk_ids=torch.empty((M, k), **i32),
             topk_w=torch.empty((M, k), **f32), offsets=torch.empty(E + S + 1, **i32), perm=torch.empty(T, **i32),
             active=torch.empty(E + S, **i32), n_active=torch.empty(1, **i32), dev_error=torch.empty(1, **i32),
             y_slots=torch.empty((T, d), **f32), out=torch.empty((M, d), **f32))
    for key, t in b.items():
        t.fill_(float("nan") if t.dtype == torch.float32 else -7)
    return b


def _call(moe, noalloc, x, wr, k, ex, b):
    M = x.shape[0]
    S = ex.n_shared
    T = M * (k + S)
    args = (x, wr, b["logits"][:M], k, ex, b["topk_ids"][:M], b["topk_w"][:M], b["offsets"], b["perm"][:T],
            b["active"], b["n_active"], b["dev_error"], b["y_slots"][:T], b["out"][:M])
    if noalloc:
        moe.moe_layer_mxfp4_noalloc(*args)
    else:
        ws = torch.full((moe.moe_workspace_bytes(M, k, ex),), 0xA5, dtype=torch.uint8, device="cuda")
        moe.moe_layer_mxfp4(*args, ws)
    torch.cuda.synchronize()
    na = int(b["n_active"][0].item())
    return dict(logits=b["logits"][:M].cpu().numpy(), ids=b["topk_ids"][:M].cpu().numpy(),
                w=b["topk_w"][:M].cpu().numpy(), offsets=b["offsets"].cpu().numpy(),
                perm=b["perm"][:T].cpu().numpy(), active=b["active"][:na].cpu().numpy(), n_active=np.array([na]),
                dev_error=b["dev_error"].cpu().numpy(), y=b["y_slots"][:T].cpu().numpy(),
                out=b["out"][:M].cpu().numpy())


@pytest.mark.parametrize("shape,rows,tiles", SHAPES, ids=[s[0].name for s in SHAPES])
def test_noalloc_equals_layer_call(shape, rows, tiles):
    moe = _moe()
    seed = 71
    print(f"\n[noalloc] {shape.name}: rows {rows}, tile order {tiles}", flush=True)
    ex = moe.Experts(synth.device_experts(shape, seed), shape.stride, shape.d, shape.f, shape.n_routed,
                     shape.n_shared)
    if tiles:
        ex = moe.tile_experts(ex)
    wr = torch.from_numpy(synth.router_weight(shape, seed)).cuda()
    M1 = rows[0]
    ref_b = _buffers(M1, shape.k, shape.n_routed, shape.n_shared, shape.d)
    na_b = _buffers(M1, shape.k, shape.n_routed, shape.n_shared, shape.d)
    for i, M in enumerate(rows):  # the second call has fewer rows than the first
        x = synth.block_x(shape, seed + i, M) if M <= 16 else synth.rows_x(shape, seed + i, M)
        xt = torch.from_numpy(np.ascontiguousarray(x))
        xd = (xt.view(torch.bfloat16) if shape.x_dtype == "bf16" else xt).cuda()
        a = _call(moe, False, xd, wr, shape.k, ex, ref_b)
        b = _call(moe, True, xd, wr, shape.k, ex, na_b)
        assert int(a["dev_error"][0]) == 0
        for key in a:
            assert np.array_equal(a[key].view(np.uint8), b[key].view(np.uint8)), (shape.name, M, key)


def test_noalloc_refuses_more_rows_than_its_scratch():
    """76 rows of the Kimi widths need more than the 8 MiB array: refused on
    the host, nothing enqueued, every output left as it was."""
    moe = _moe()
    shape = synth.LayerShape("kd", 7168, 1536, 24, 2, 16, -8, -4, 0.02, "bf16")
    ex = moe.Experts(torch.zeros(shape.n_experts * shape.stride, dtype=torch.uint8, device="cuda"), shape.stride,
                     shape.d, shape.f, shape.n_routed, shape.n_shared)
    M = 76
    assert moe.moe_workspace_bytes(M, shape.k, ex) > moe.moe_noalloc_scratch_bytes()
    b = _buffers(M, shape.k, shape.n_routed, shape.n_shared, shape.d)
    x = torch.zeros((M, shape.d), dtype=torch.bfloat16, device="cuda")
    wr = torch.zeros((shape.n_routed, shape.d), dtype=torch.float32, device="cuda")
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_layer_mxfp4_noalloc(x, wr, b["logits"], shape.k, ex, b["topk_ids"], b["topk_w"], b["offsets"],
                                    b["perm"], b["active"], b["n_active"], b["dev_error"], b["y_slots"], b["out"])
    assert ei.value.rc == moe.MOE_ESCRATCH
    torch.cuda.synchronize()
    assert int(b["n_active"][0].item()) == -7 and torch.isnan(b["out"]).all()
