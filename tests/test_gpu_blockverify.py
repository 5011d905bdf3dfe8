"""Block verification ("A drafter that leaves the answer unchanged"): the
harness kernels against exact references, a layer stack whose 16-row block
equals 16 plain steps in every logits bit (FNV-1a per position, as the pages'
run record compares), greedy acceptance with a wrong draft planted at the
start, in the middle and at the end, short proposals, and the stack's composition
checked layer by layer against the oracle.  Needs an MI355X."""
import numpy as np
import pytest

import oracle
import synth
from conftest import assert_close
from oracle.hashes import fnv1a64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _moe():
    import router_top_bucket_amd as moe
    return moe


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


# ----------------------------------------------------------------------------- kernels
@pytest.mark.parametrize("tiles", [False, True])
def test_q8_0_rows_exact(tiles):
    moe = _moe()
    K, N = 416, 304
    wq, ws = synth.q8_0_weight(9, K, N)
    ids = np.array([0, 303, 17, 17, -1, 304, 5], dtype=np.int32)
    X = torch.empty((len(ids), K), dtype=torch.float32, device="cuda")
    dwq = _dev(wq)
    if tiles:
        t = torch.empty_like(dwq)
        moe.q8_0_pack(dwq, t, moe.MOE_LAYOUT_TILES)
        dwq = t
    moe.q8_0_rows(_dev(ids), dwq, _dev(ws.view(np.int16)), X,
                  layout=moe.MOE_LAYOUT_TILES if tiles else moe.MOE_LAYOUT_ROWS)
    sc = ws.view(np.float16).astype(np.float32)
    ref = np.zeros((len(ids), K), dtype=np.float32)
    for m, i in enumerate(ids):
        if 0 <= i < N:
            ref[m] = wq[i].astype(np.float32) * np.repeat(sc[i], 32)
    assert np.array_equal(X.cpu().numpy().view(np.uint32), ref.view(np.uint32))


def test_residual_and_bf16_exact():
    moe = _moe()
    g = synth.rng(3, 77)
    h = g.standard_normal(5000).astype(np.float32) * 10
    a = g.standard_normal(5000).astype(np.float32)
    dh, da = _dev(h), _dev(a)
    hb = torch.empty(5000, dtype=torch.int16, device="cuda")
    moe.moe_residual_bf16(dh, da, hb)
    s = (h + a).astype(np.float32)
    assert np.array_equal(dh.cpu().numpy().view(np.uint32), s.view(np.uint32))
    assert np.array_equal(hb.cpu().numpy().view(np.uint16), synth.bf16_bits(s))


@pytest.mark.parametrize("d", [7168, 416, 418, 9000])
def test_rmsnorm_close_and_row_independent(d):
    moe = _moe()
    g = synth.rng(3, 78, d)
    h = (g.standard_normal((9, d)) * np.arange(1, 10)[:, None]).astype(np.float32)
    out = torch.empty_like(_dev(h))
    outb = torch.empty((9, d), dtype=torch.int16, device="cuda")
    moe.moe_rmsnorm(_dev(h), out, outb, 1e-6)
    h64 = h.astype(np.float64)
    ref = h64 / np.sqrt((h64 ** 2).mean(axis=1, keepdims=True) + 1e-6)
    o = out.cpu().numpy()
    assert_close(o, ref.astype(np.float32), "rmsnorm")
    assert np.array_equal(outb.cpu().numpy().view(np.uint16), synth.bf16_bits(o))
    # a row alone gives the same bits
    one = torch.empty((1, d), dtype=torch.float32, device="cuda")
    moe.moe_rmsnorm(_dev(h[4:5]), one, None, 1e-6)
    assert np.array_equal(one.cpu().numpy().view(np.uint32), o[4:5].view(np.uint32))


def test_argmax_rows_exact_with_ties_and_nan():
    moe = _moe()
    g = synth.rng(3, 79)
    X = g.standard_normal((6, 163840)).astype(np.float32)
    X[1, [10, 5000, 70000]] = 99.0          # ties: the lowest index
    X[2, :] = np.nan
    X[2, 123] = -5.0                        # NaN below every number
    X[3, :] = -np.inf
    X[4, 163839] = 1e30                     # the last element
    idx = torch.empty(6, dtype=torch.int32, device="cuda")
    moe.moe_argmax_rows(_dev(X), idx)
    Xr = np.where(np.isnan(X), -np.inf, X)
    ref = Xr.argmax(axis=1)
    assert idx.cpu().numpy().tolist() == ref.tolist()
    assert ref[1] == 10 and ref[2] == 123 and ref[3] == 0 and ref[4] == 163839
    # a length that is not a multiple of 4, and one shorter than a round
    for N in (1003, 37):
        Y = g.standard_normal((3, N)).astype(np.float32)
        Y[1, [N - 1, 2]] = 50.0
        idx = torch.empty(3, dtype=torch.int32, device="cuda")
        moe.moe_argmax_rows(_dev(Y), idx)
        assert idx.cpu().numpy().tolist() == Y.argmax(axis=1).tolist()


def test_fnv1a_rows_match_reference():
    moe = _moe()
    g = synth.rng(3, 80)
    X = g.standard_normal((5, 777)).astype(np.float32)
    X[3] = 0.0
    hs = torch.empty(5, dtype=torch.int64, device="cuda")
    moe.moe_fnv1a_rows(_dev(X), hs)
    got = [int(v) & 0xFFFFFFFFFFFFFFFF for v in hs.cpu().tolist()]
    assert got == [fnv1a64(X[m].tobytes()) for m in range(5)]


# ----------------------------------------------------------------------------- the stack
SMALL = synth.LayerShape("s3", 416, 224, 9, 2, 4, -7, -3, 0.05, "bf16")
VOCAB = 1008  # a multiple of 16, so the head can be tile-ordered


def _small_stack(moe, n_layers=3):
    from router_top_bucket_amd.blockverify import Q8Matrix, Stack
    shape = SMALL
    layers, spines, host = [], [], []
    for l in range(n_layers):
        base = synth.device_experts(shape, 90 + l)
        wr = synth.router_weight(shape, 90 + l)
        layers.append((moe.Experts(base, shape.stride, shape.d, shape.f, shape.n_routed, shape.n_shared), _dev(wr)))
        wq, ws = synth.q8_0_weight(190 + l, shape.d, shape.d)
        spines.append(Q8Matrix(_dev(wq), _dev(ws.view(np.int16))))
        host.append(dict(wr=wr, wq=wq, ws=ws,
                         rec={e: synth.expert_record(shape, 90 + l, e) for e in range(shape.n_experts)}))
    hq, hs = synth.q8_0_weight(290, shape.d, VOCAB)
    head = Q8Matrix(_dev(hq), _dev(hs.view(np.int16)))
    return Stack(layers, spines, head, shape.k, 16), host, (hq, hs)


def test_block_equals_plain_steps_and_greedy_acceptance():
    moe = _moe()
    from router_top_bucket_amd.blockverify import plain_steps, verify_block
    stack, _, _ = _small_stack(moe)
    t0 = 7
    plain, ph = plain_steps(stack, t0, 16)
    seq = [t0] + plain                       # seq[i+1] = the model's token after seq[i]
    # a perfect 15-token proposal: every draft kept, 16 tokens emitted, and
    # every row's logits bit-identical to the plain step fed the same token
    emitted, kept, bh = verify_block(stack, t0, seq[1:16])
    assert kept == 15 and emitted == plain[:16]
    assert bh == ph[:16]
    # a wrong draft planted at position 1, in the middle and at the end
    for j in (1, 8, 15):
        drafts = list(seq[1:16])
        drafts[j - 1] = (drafts[j - 1] + 1) % VOCAB
        emitted, kept, bh = verify_block(stack, t0, drafts)
        assert kept == j - 1 and emitted == plain[:j], j
        assert bh[:j] == ph[:j]            # rows before the bad draft are the plain steps
    # short proposals
    for n in (0, 1, 3):
        emitted, kept, bh = verify_block(stack, t0, seq[1:1 + n])
        assert kept == n and emitted == plain[:n + 1] and bh == ph[:n + 1]


def test_stack_composition_against_oracle():
    """Each stage of Stack.run, fed the GPU's own input to that stage, against
    the oracle's arithmetic (so a difference cannot compound)."""
    moe = _moe()
    from router_top_bucket_amd.blockverify import EPS
    stack, host, (hq, hs) = _small_stack(moe)
    shape = SMALL
    tokens = np.array([3, 999, 41], dtype=np.int32)
    M = len(tokens)
    stack.run(_dev(tokens))
    logits = stack.logits[:M].cpu().numpy()
    # replay on the GPU stage by stage, checking each against the oracle
    h = torch.empty((M, shape.d), dtype=torch.float32, device="cuda")
    moe.q8_0_rows(_dev(tokens), stack.head.wq, stack.head.ws, h, layout=stack.head.layout)
    emb = hq[tokens].astype(np.float32) * np.repeat(hs.view(np.float16).astype(np.float32)[tokens], 32, axis=1)
    assert np.array_equal(h.cpu().numpy(), emb)

    def norm(x):
        x64 = x.astype(np.float64)
        return (x64 / np.sqrt((x64 ** 2).mean(axis=1, keepdims=True) + EPS)).astype(np.float32)

    n = torch.empty_like(h)
    a = torch.empty_like(h)
    hb = torch.empty((M, shape.d), dtype=torch.bfloat16, device="cuda")
    for l, ml in enumerate(stack.mls):
        hh = h.cpu().numpy()
        moe.moe_rmsnorm(h, n, None, EPS)
        assert_close(n.cpu().numpy(), norm(hh), f"layer {l} norm 1")
        moe.q8_0_matmul(n, stack.spines[l].wq, stack.spines[l].ws, a, layout=stack.spines[l].layout)
        assert_close(a.cpu().numpy(), oracle.q8_0_matmul(n.cpu().numpy(), host[l]["wq"], host[l]["ws"]),
                     f"layer {l} spine")
        a_h = a.cpu().numpy()
        moe.moe_residual_bf16(h, a, None)
        assert np.array_equal(h.cpu().numpy(), (hh + a_h).astype(np.float32))
        moe.moe_rmsnorm(h, None, hb, EPS)
        xb = hb.view(torch.int16).cpu().numpy().view(np.uint16)
        v = ml.forward(hb)
        ref = oracle.layer(xb, shape.k, shape.n_routed, shape.n_shared, shape.d, shape.f, host[l]["rec"].__getitem__,
                           w_r=host[l]["wr"])
        assert np.array_equal(v["topk_ids"][:M].cpu().numpy(), ref["ids"]), l
        assert_close(v["out"][:M].cpu().numpy(), ref["out"], f"layer {l} moe")
        hh = h.cpu().numpy()
        moe.moe_residual_bf16(h, v["out"][:M], None)
        assert np.array_equal(h.cpu().numpy(), (hh + v["out"][:M].cpu().numpy()).astype(np.float32))
    moe.moe_rmsnorm(h, n, None, EPS)
    assert_close(logits, oracle.q8_0_matmul(n.cpu().numpy(), hq, hs), "head logits")
    assert np.array_equal(stack.next[:M].cpu().numpy(), logits.argmax(axis=1))


def test_stack_with_tiled_weights_equals_row_order():
    """Tile-ordered expert records and Q8_0 spines/head: the same logits bits."""
    moe = _moe()
    from router_top_bucket_amd.blockverify import Stack, plain_steps
    stack, _, _ = _small_stack(moe)
    tiled = Stack([(moe.tile_experts(ml.experts), ml.w_router) for ml in stack.mls],
                  [sp.tiled() for sp in stack.spines], stack.head.tiled(), stack.k, 16)
    a_tok, a_hash = plain_steps(stack, 11, 6)
    b_tok, b_hash = plain_steps(tiled, 11, 6)
    assert a_tok == b_tok and a_hash == b_hash
