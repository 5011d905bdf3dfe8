"""Pins for the CPU oracle, each against something other than the oracle itself:
published format tables, the pages' stated sizes, closed forms, brute force on
tiny inputs, exact integer special cases, and invariants.  CPU only."""
import itertools
import math
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
import synth
from conftest import ROOT, make_expert, read_golden, rel_l2


# ----------------------------------------------------------------------------- formats
def test_e2m1_table_matches_ocp_mx():
    for code, val in read_golden("e2m1_values.txt"):
        got = oracle.e2m1(int(code))
        assert got == float(val)
        assert math.copysign(1.0, got) == math.copysign(1.0, float(val)), f"sign of code {code}"


def test_e8m0_values():
    for b, val in read_golden("e8m0_values.txt"):
        got = oracle.e8m0(int(b))
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val), (b, got, val)


def test_mxfp4_elements_exact_in_fp32_and_bf16():
    # 2 significant bits times a power of two: exact in both formats for the
    # scale range the workloads draw (2^-8..2^-2) and far beyond it
    for code in range(16):
        for b in range(100, 160):
            v = oracle.e2m1(code) * oracle.e8m0(b)
            f32 = np.float32(v)
            assert float(f32) == v
            bits = f32.view(np.uint32)
            assert bits & 0xFFFF == 0, "not representable in bf16"


def test_fp16_decode_all_bit_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.fp16(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_bf16_widen_and_round():
    rng = np.random.default_rng(0)
    a = rng.standard_normal(10000).astype(np.float32)
    b = synth.bf16_bits(a)
    w = oracle.widen_bf16(b)
    # widening is exact: the upper 16 bits of binary32
    assert np.array_equal(w.view(np.uint32), b.astype(np.uint32) << 16)
    # rounding is to nearest: error at most half a bf16 ulp (2^-8 relative)
    assert np.all(np.abs(w - a) <= np.abs(a) * 2.0 ** -8 + 1e-30)


def test_expert_record_size_from_the_pages():
    g = dict((k, v) for k, v in read_golden("expert_record_kimi.txt"))
    off = oracle.expert_layout(int(g["d"]), int(g["f"]))
    assert off[6] == int(g["record_bytes"]) == 17547264
    assert synth.KIMI.stride == off[6]
    assert int(g["moe_layers"]) * int(g["experts_per_layer"]) == int(g["experts_total"])
    total_tb = int(g["experts_total"]) * off[6] / 1e12
    assert abs(total_tb - float(g["payload_tb_approx"])) < 0.005
    # one layer's 896 routed experts: about 15.7 GB
    assert abs(896 * off[6] / 1e9 - 15.72) < 0.01
    # sections: gate codes, gate scales, up codes, up scales, down codes, down scales
    d, f = 7168, 1536
    sizes = np.diff(off)
    assert list(sizes) == [f * d // 2, f * d // 32] * 3
    assert all(o % 16 == 0 for o in off)


def test_tiny_record_size():
    off = oracle.expert_layout(256, 128)
    assert off[6] == 52224 == synth.TINY.stride


def test_mxfp4_handmade_block():
    rows, K = 2, 64
    codes = np.zeros((rows, K // 2), dtype=np.uint8)
    scales = np.full((rows, K // 32), 127, dtype=np.uint8)
    expect = {}
    for line in read_golden("mxfp4_handmade.txt"):
        kind = line[0]
        if kind == "scale":
            scales[int(line[1]), int(line[2])] = int(line[3])
        elif kind == "byte":
            codes[int(line[1]), int(line[2])] = int(line[3], 16)
        elif kind == "value":
            expect[(int(line[1]), int(line[2]))] = float(line[3])
    W = oracle.mxfp4_dequant(codes.ravel(), scales.ravel(), rows, K)
    for (r, c), v in expect.items():
        assert W[r, c] == v, (r, c, W[r, c], v)
        assert math.copysign(1, W[r, c]) == math.copysign(1, v), (r, c)
    nz = {(r, c) for r in range(rows) for c in range(K) if W[r, c] != 0}
    assert nz == {rc for rc, v in expect.items() if v != 0}


def test_mxfp4_one_hot_positions():
    # a single nonzero code at (r, c) decodes at (r, c) only: catches a
    # transposed or shifted index anywhere in the matrix, first and last
    rows, K = 5, 96
    for (r, c) in [(0, 0), (0, K - 1), (rows - 1, 0), (rows - 1, K - 1), (2, 33), (3, 62)]:
        codes = np.zeros((rows, K // 2), dtype=np.uint8)
        scales = np.full((rows, K // 32), 127, dtype=np.uint8)
        codes[r, c // 2] = (5 << 4) if c % 2 else 5  # code 5 = 3.0
        scales[r, c // 32] = 125  # 2^-2
        W = oracle.mxfp4_dequant(codes.ravel(), scales.ravel(), rows, K)
        assert W[r, c] == 0.75
        assert np.count_nonzero(W) == 1


# ----------------------------------------------------------------------------- router
def test_router_logits_one_hot_rows():
    # W_r[e] = unit vector at column 3e+1: logits[m,e] = x[m, 3e+1]
    E, d, M = 7, 32, 3
    w = np.zeros((E, d), dtype=np.float32)
    for e in range(E):
        w[e, 3 * e + 1] = 1.0
    x = synth.rng(1, 1).standard_normal((M, d)).astype(np.float32)
    lg = oracle.router_logits(x, w)
    assert np.array_equal(lg, x[:, 1::3][:, :E])


def test_router_logits_integer_exact():
    g = synth.rng(2, 2)
    M, d, E = 4, 96, 9
    x = g.integers(-8, 9, size=(M, d)).astype(np.float32)
    w = g.integers(-8, 9, size=(E, d)).astype(np.float32)
    ref = x.astype(np.int64) @ w.astype(np.int64).T
    assert np.array_equal(oracle.router_logits(x, w), ref.astype(np.float32))


def test_router_logits_bf16_input_is_widened():
    g = synth.rng(3, 3)
    x = g.integers(-4, 5, size=(2, 64)).astype(np.float32)
    w = g.integers(-4, 5, size=(5, 64)).astype(np.float32)
    assert np.array_equal(oracle.router_logits(synth.bf16_bits(x), w), oracle.router_logits(x, w))


def _brute_topk_sets(row, k):
    """All index sets a correct top-k may return, by brute force."""
    key = [(-np.inf if np.isnan(v) else float(v)) for v in row]
    best = None
    for comb in itertools.combinations(range(len(row)), k):
        # a valid top-k: every chosen beats every unchosen (ties: lower index)
        chosen = set(comb)
        ok = all((key[a] > key[b]) or (key[a] == key[b] and a < b)
                 for a in chosen for b in range(len(row)) if b not in chosen)
        if ok:
            assert best is None, "tie rule must make the set unique"
            best = comb
    return best


@pytest.mark.parametrize("k", [1, 2, 3, 5])
def test_topk_brute_force_tiny(k):
    E = 9
    g = synth.rng(4, k)
    for trial in range(30):
        row = g.integers(-3, 4, size=E).astype(np.float32)  # many ties
        if trial % 5 == 0:
            row[g.integers(0, E)] = np.nan
        ids, w = oracle.topk(row[None, :], k)
        assert tuple(sorted(ids[0])) == _brute_topk_sets(row, k)
        # rank order: descending logit, ties by index
        keys = [(-(-np.inf if np.isnan(row[i]) else row[i]), i) for i in ids[0]]
        assert keys == sorted(keys)


def test_topk_ties_all_equal():
    ids, w = oracle.topk(np.zeros((1, 16), dtype=np.float32), 4)
    assert list(ids[0]) == [0, 1, 2, 3]
    assert np.all(w == np.float32(0.25))


def test_topk_weights_closed_forms():
    # k = 1: weight exactly 1
    lg = synth.random_logits(5, 20, 16)
    _, w1 = oracle.topk(lg, 1)
    assert np.all(w1 == 1.0)
    # k = 2: w0 = sigmoid(l0 - l1) = (1 + tanh((l0-l1)/2)) / 2
    ids, w2 = oracle.topk(lg, 2)
    for m in range(lg.shape[0]):
        a, b = float(lg[m, ids[m, 0]]), float(lg[m, ids[m, 1]])
        ref0 = 0.5 * (1.0 + math.tanh(0.5 * (a - b)))
        assert abs(float(w2[m, 0]) - ref0) <= 2 ** -23
        assert abs(float(w2[m, 1]) - (1 - ref0)) <= 2 ** -23
    # weights sum to one and are nonincreasing
    ids, w = oracle.topk(lg, 5)
    assert np.all(np.abs(w.astype(np.float64).sum(1) - 1) < 5 * 2 ** -24)
    assert np.all(np.diff(w, axis=1) <= 0)


def test_topk_weights_ignore_unselected_logits():
    # renormalised softmax over the selected set does not depend on the others
    lg = synth.random_logits(6, 8, 32)
    ids, w = oracle.topk(lg, 4)
    lg2 = lg.copy()
    for m in range(8):
        mask = np.ones(32, bool)
        mask[ids[m]] = False
        lg2[m, mask] -= 5.0
    ids2, w2 = oracle.topk(lg2, 4)
    assert np.array_equal(ids, ids2)
    assert np.max(np.abs(w - w2)) <= 2 ** -23


# ----------------------------------------------------------------------------- bucket
def _brute_bucket(ids, E, S):
    M, k = ids.shape
    ex = []
    for m in range(M):
        ex += list(ids[m]) + [E + s for s in range(S)]
    order = sorted(range(len(ex)), key=lambda t: (ex[t], t))
    offsets = [0] * (E + S + 1)
    for e in ex:
        offsets[e + 1] += 1
    for e in range(E + S):
        offsets[e + 1] += offsets[e]
    active = sorted(set(ex))
    return offsets, order, active


@pytest.mark.parametrize("M,E,k,S", [(1, 16, 2, 0), (5, 16, 2, 0), (16, 896, 16, 2), (270, 896, 16, 2),
                                     (0, 16, 2, 0), (3, 4, 4, 1)])
def test_bucket_brute_force(M, E, k, S):
    g = synth.rng(7, M, E)
    if M:
        ids = np.stack([g.permutation(E)[:k] for _ in range(M)]).astype(np.int32)
    else:
        ids = np.zeros((0, k), dtype=np.int32)
    offsets, perm, active, n = oracle.bucket(ids, E, S)
    bo, bp, ba = _brute_bucket(ids, E, S)
    assert list(offsets) == bo
    assert list(perm) == bp
    assert list(active) == ba and n == len(ba)


def test_bucket_zipf_prefill_shape():
    lg = synth.zipf_logits(synth.KIMI, 0, 1533)
    ids, _ = oracle.topk(lg, 16)
    offsets, perm, active, n = oracle.bucket(ids, 896, 2)
    bo, bp, ba = _brute_bucket(ids, 896, 2)
    assert list(offsets) == bo and list(perm) == bp and list(active) == ba
    counts = np.diff(offsets)[:896]
    # Zipf(1.1) popularity: heavy skew, ~27 rows per expert on average
    assert abs(counts.mean() - 1533 * 16 / 896) < 1e-9
    assert counts.max() > 20 * np.median(counts)


def test_bucket_rejects_out_of_range_ids():
    with pytest.raises(ValueError):
        oracle.bucket(np.array([[0, 16]], dtype=np.int32), 16, 0)
    with pytest.raises(ValueError):
        oracle.bucket(np.array([[-1, 2]], dtype=np.int32), 16, 0)


# ----------------------------------------------------------------------------- expert FFN
def _sigmoid(z):
    return 0.5 * (1.0 + math.tanh(0.5 * z))


D, F = 64, 32


def test_ffn_zero_cases():
    g = synth.rng(8, 8)
    x = g.standard_normal((2, D)).astype(np.float32)
    # all-zero codes (including -0 codes) give y = 0
    rec = make_expert(D, F)
    assert np.all(oracle.expert_ffn(x, rec, D, F) == 0)
    rec = np.frombuffer(bytes(rec), dtype=np.uint8).copy()
    # random expert, x = 0 gives y = 0
    rec = synth.expert_record(synth.LayerShape("t", D, F, 1, 0, 1, -6, -2, 0.05, "f32"), 1, 0)
    assert np.all(oracle.expert_ffn(np.zeros((1, D), np.float32), rec, D, F) == 0)


@pytest.mark.parametrize("i0,c0,c1,r0", [(0, 0, 1, 0), (F - 1, D - 1, D - 2, D - 1), (5, 33, 40, 17), (17, 2, 63, 60)])
def test_ffn_one_hot_closed_form(i0, c0, c1, r0):
    # gate (i0,c0), up (i0,c1), down (r0,i0) single nonzero codes:
    #   y[r0] = wd * silu(wg * x[c0]) * (wu * x[c1]), every other y = 0
    cg, sg, cu, su, cd, sd = 5, 126, 11, 128, 7, 125  # 3*2^-1, -1.5*2^1, 6*2^-2
    rec = make_expert(D, F, gate=[(i0, c0, cg, sg)], up=[(i0, c1, cu, su)], down=[(r0, i0, cd, sd)])
    x = synth.rng(9, i0).standard_normal((1, D)).astype(np.float32)
    y = oracle.expert_ffn(x, rec, D, F)
    g_ = 1.5 * float(x[0, c0])
    u_ = -3.0 * float(x[0, c1])
    ref = 1.5 * (g_ * _sigmoid(g_)) * u_
    assert abs(float(y[0, r0]) - ref) <= abs(ref) * 2 ** -23
    mask = np.ones(D, bool)
    mask[r0] = False
    assert np.all(y[0, mask] == 0)


def test_ffn_gate_and_up_are_not_interchangeable():
    # silu acts on the gate only: with gate 0 the output is 0 whatever up is
    rec = make_expert(D, F, up=[(3, 4, 7, 127)], down=[(9, 3, 2, 127)])
    x = np.ones((1, D), np.float32)
    assert np.all(oracle.expert_ffn(x, rec, D, F) == 0)
    rec2 = make_expert(D, F, gate=[(3, 4, 7, 127)], down=[(9, 3, 2, 127)])
    assert np.all(oracle.expert_ffn(x, rec2, D, F) == 0)


def test_ffn_down_scale_linearity():
    shp = synth.LayerShape("t", D, F, 1, 0, 1, -6, -2, 0.05, "f32")
    rec = synth.expert_record(shp, 3, 0)
    x = synth.rng(10, 1).standard_normal((3, D)).astype(np.float32)
    y = oracle.expert_ffn(x, rec, D, F)
    rec2 = rec.copy()
    off = oracle.expert_layout(D, F)
    rec2[off[5]:off[6]] += 1  # every down scale doubles
    y2 = oracle.expert_ffn(x, rec2, D, F)
    assert np.array_equal(y2, 2 * y)


def test_ffn_rows_are_independent():
    shp = synth.LayerShape("t", D, F, 1, 0, 1, -6, -2, 0.05, "f32")
    rec = synth.expert_record(shp, 4, 0)
    x = synth.rng(11, 1).standard_normal((5, D)).astype(np.float32)
    y = oracle.expert_ffn(x, rec, D, F)
    for m in range(5):
        assert np.array_equal(oracle.expert_ffn(x[m:m + 1], rec, D, F)[0], y[m])


# ----------------------------------------------------------------------------- combine
def test_combine_one_hot_and_shared():
    M, k, S, d = 3, 4, 2, 16
    g = synth.rng(12, 1)
    y = g.standard_normal((M * (k + S), d)).astype(np.float32)
    w = np.zeros((M, k), np.float32)
    w[:, 2] = 1.0
    out = oracle.combine(y, w, k, S)
    for m in range(M):
        ref = y[m * (k + S) + 2].astype(np.float64) + y[m * (k + S) + k] + y[m * (k + S) + k + 1]
        assert np.array_equal(out[m], ref.astype(np.float32))
    y0 = y.reshape(M, k + S, d)[:, :k].reshape(M * k, d)
    assert np.all(oracle.combine(y0, np.zeros((M, k), np.float32), k, 0) == 0)


def test_combine_integer_exact():
    M, k, S, d = 4, 16, 2, 32
    g = synth.rng(13, 1)
    y = g.integers(-50, 51, size=(M * (k + S), d)).astype(np.float32)
    w = (2.0 ** -g.integers(0, 6, size=(M, k))).astype(np.float32)
    out = oracle.combine(y, w, k, S)
    yy = y.reshape(M, k + S, d).astype(np.float64)
    ref = (yy[:, :k] * w[:, :, None]).sum(1) + yy[:, k:].sum(1)
    assert np.array_equal(out, ref.astype(np.float32))


# ----------------------------------------------------------------------------- Q8_0
def test_q8_0_integer_exact():
    g = synth.rng(14, 1)
    M, K, N = 4, 128, 24
    X = g.integers(-20, 21, size=(M, K)).astype(np.float32)
    wq = g.integers(-127, 128, size=(N, K), dtype=np.int8)
    e = g.integers(-6, 1, size=(N, K // 32))
    ws = (2.0 ** e).astype(np.float16).view(np.uint16)
    Y = oracle.q8_0_matmul(X, wq, ws)
    scale = np.repeat(2.0 ** e, 32, axis=1)  # [N x K]
    # integers times powers of two >= 2^-6: exact as integer sums scaled by 2^6
    Wint = (wq.astype(np.int64) * (scale * 64).astype(np.int64))
    ref = (X.astype(np.int64) @ Wint.T).astype(np.float64) / 64
    assert np.array_equal(Y, ref.astype(np.float32))


def test_q8_0_block_scale_applies_to_its_32_columns():
    M, K, N = 1, 96, 3
    X = np.zeros((M, K), np.float32)
    wq = np.ones((N, K), np.int8)
    ws = np.full((N, K // 32), np.float16(1.0).view(np.uint16), dtype=np.uint16)
    ws[1, 2] = np.float16(0.5).view(np.uint16)
    for c, ref in [(63, 1.0), (64, 0.5), (95, 0.5), (31, 1.0)]:
        X[:] = 0
        X[0, c] = 1.0
        Y = oracle.q8_0_matmul(X, wq, ws)
        assert Y[0, 1] == ref and Y[0, 0] == 1.0 and Y[0, 2] == 1.0


# ----------------------------------------------------------------------------- layer
def test_layer_block_rows_equal_single_rows():
    shp = synth.TINY
    recs = {e: synth.expert_record(shp, 0, e) for e in range(shp.n_experts)}
    wr = synth.router_weight(shp, 0)
    x = synth.block_x(shp, 1, 4)
    blk = oracle.layer(x, shp.k, shp.n_routed, shp.n_shared, shp.d, shp.f, recs.__getitem__, w_r=wr)
    for m in range(4):
        one = oracle.layer(x[m:m + 1], shp.k, shp.n_routed, shp.n_shared, shp.d, shp.f, recs.__getitem__, w_r=wr)
        assert np.array_equal(one["out"][0], blk["out"][m])
        assert np.array_equal(one["ids"][0], blk["ids"][m])


def test_layer_matches_per_slot_definition():
    # layer() bookkeeping (perm -> rows) against a direct per-slot evaluation
    shp = synth.TINY
    recs = {e: synth.expert_record(shp, 2, e) for e in range(shp.n_experts)}
    wr = synth.router_weight(shp, 2)
    x = synth.rows_x(shp, 3, 3)
    res = oracle.layer(x, shp.k, shp.n_routed, shp.n_shared, shp.d, shp.f, recs.__getitem__, w_r=wr)
    for m in range(3):
        for j in range(shp.k):
            e = int(res["ids"][m, j])
            y = oracle.expert_ffn(x[m:m + 1], recs[e], shp.d, shp.f)[0]
            assert np.array_equal(res["y_slots"][m * shp.k + j], y)


def test_oracle_thread_count_invariance():
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "import numpy as np, oracle, synth\n"
        "shp = synth.TINY\n"
        "recs = {e: synth.expert_record(shp, 5, e) for e in range(shp.n_experts)}\n"
        "x = synth.rows_x(shp, 5, 3); wr = synth.router_weight(shp, 5)\n"
        "r = oracle.layer(x, shp.k, shp.n_routed, 0, shp.d, shp.f, recs.__getitem__, w_r=wr)\n"
        "sys.stdout.write(r['out'].tobytes().hex())\n" % ROOT)
    outs = []
    for n in ("1", "7"):
        env = dict(os.environ, OMP_NUM_THREADS=n)
        outs.append(subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                                   check=True).stdout)
    assert outs[0] == outs[1] and len(outs[0]) > 0


# ----------------------------------------------------------------------------- fp32-accumulation reading
# The oracle's second reading keeps every sum in fp32: a K reduction is cut
# into ascending 32-element blocks, terms added one by one inside a block and
# the block partials then added in order.  Pinned by closed forms that hold in
# any fp32 order, by cases whose result only that order produces, and by its
# agreement with the fp64 reading at the Kimi shape.
def test_f32_router_closed_forms():
    E, d, M = 7, 64, 3
    w = np.zeros((E, d), dtype=np.float32)
    for e in range(E):
        w[e, 3 * e + 1] = 1.0
    x = synth.rng(21, 1).standard_normal((M, d)).astype(np.float32)
    assert np.array_equal(oracle.router_logits(x, w, accum="f32"), x[:, 1::3][:, :E])
    g = synth.rng(21, 2)
    xi = g.integers(-8, 9, size=(4, 96)).astype(np.float32)
    wi = g.integers(-8, 9, size=(9, 96)).astype(np.float32)
    ref = xi.astype(np.int64) @ wi.astype(np.int64).T
    assert np.array_equal(oracle.router_logits(xi, wi, accum="f32"), ref.astype(np.float32))


def test_f32_router_block_order():
    # 2^24 + 1 rounds back to 2^24 in fp32 (ties to even).  One big term ahead
    # of 31 ones inside a block swallows them one by one; the same ones
    # summed in an earlier block arrive as one partial of 31 and survive.
    d = 64
    w = np.ones((2, d), np.float32)
    x = np.zeros((2, d), np.float32)
    x[0, 0], x[0, 1:32] = 2.0 ** 24, 1.0      # big term first, in block 0
    x[1, 0:31], x[1, 32] = 1.0, 2.0 ** 24     # ones in block 0, big term in block 1
    lg = oracle.router_logits(x, w[:1], accum="f32")
    assert lg[0, 0] == np.float32(2.0 ** 24)
    assert lg[1, 0] == np.float32(2.0 ** 24 + 32)    # 2^24 + 31 rounds to even
    lg64 = oracle.router_logits(x, w[:1])
    assert lg64[0, 0] == np.float32(2.0 ** 24 + 32)  # fp64 reading: exact sum, rounded once


def test_f32_topk_weights_closed_forms():
    g = synth.rng(22, 1)
    lg = g.standard_normal((5, 40)).astype(np.float32)
    ids, w = oracle.topk(lg, 1, accum="f32")
    assert np.all(w == 1.0)
    eq = np.full((2, 12), 0.375, np.float32)
    ids, w = oracle.topk(eq, 4, accum="f32")
    assert np.array_equal(ids, [[0, 1, 2, 3]] * 2) and np.all(w == np.float32(0.25))
    ids64, _ = oracle.topk(lg, 6)
    ids32, w32 = oracle.topk(lg, 6, accum="f32")
    assert np.array_equal(ids32, ids64)  # the selection does not depend on the reading
    assert np.allclose(w32.sum(1), 1.0, rtol=0, atol=6 * 2.0 ** -23)


def test_f32_ffn_closed_forms():
    x = synth.rng(23, 1).standard_normal((2, D)).astype(np.float32)
    assert np.all(oracle.expert_ffn(x, make_expert(D, F), D, F, accum="f32") == 0)
    for (i0, c0, c1, r0) in [(0, 0, 1, 0), (F - 1, D - 1, D - 2, D - 1), (5, 33, 40, 17)]:
        rec = make_expert(D, F, gate=[(i0, c0, 5, 126)], up=[(i0, c1, 11, 128)], down=[(r0, i0, 7, 125)])
        xx = synth.rng(24, i0).standard_normal((1, D)).astype(np.float32)
        y = oracle.expert_ffn(xx, rec, D, F, accum="f32")
        g_, u_ = 1.5 * float(xx[0, c0]), -3.0 * float(xx[0, c1])
        ref = 1.5 * (g_ * _sigmoid(g_)) * u_
        assert abs(float(y[0, r0]) - ref) <= abs(ref) * 2 ** -20  # fp32 expf, divide and products
        mask = np.ones(D, bool)
        mask[r0] = False
        assert np.all(y[0, mask] == 0)
    # gate and up are not interchangeable; down scales are linear
    rec = make_expert(D, F, up=[(3, 4, 7, 127)], down=[(9, 3, 2, 127)])
    assert np.all(oracle.expert_ffn(np.ones((1, D), np.float32), rec, D, F, accum="f32") == 0)
    shp = synth.LayerShape("t", D, F, 1, 0, 1, -6, -2, 0.05, "f32")
    rec = synth.expert_record(shp, 3, 0)
    y = oracle.expert_ffn(x, rec, D, F, accum="f32")
    rec2 = rec.copy()
    off = oracle.expert_layout(D, F)
    rec2[off[5]:off[6]] += 1
    assert np.array_equal(oracle.expert_ffn(x, rec2, D, F, accum="f32"), 2 * y)


def test_f32_combine_and_q8_0_closed_forms():
    M, k, S, d = 4, 16, 2, 32
    g = synth.rng(25, 1)
    y = g.integers(-50, 51, size=(M * (k + S), d)).astype(np.float32)
    w = (2.0 ** -g.integers(0, 6, size=(M, k))).astype(np.float32)
    yy = y.reshape(M, k + S, d).astype(np.float64)
    ref = (yy[:, :k] * w[:, :, None]).sum(1) + yy[:, k:].sum(1)
    assert np.array_equal(oracle.combine(y, w, k, S, accum="f32"), ref.astype(np.float32))
    Mq, K, N = 4, 128, 24
    X = g.integers(-20, 21, size=(Mq, K)).astype(np.float32)
    wq = g.integers(-127, 128, size=(N, K), dtype=np.int8)
    e = g.integers(-6, 1, size=(N, K // 32))
    ws = (2.0 ** e).astype(np.float16).view(np.uint16)
    scale = np.repeat(2.0 ** e, 32, axis=1)
    Wint = (wq.astype(np.int64) * (scale * 64).astype(np.int64))
    refq = (X.astype(np.int64) @ Wint.T).astype(np.float64) / 64
    assert np.array_equal(oracle.q8_0_matmul(X, wq, ws, accum="f32"), refq.astype(np.float32))
    # block order: a scaled partial of 2^24 ahead of a block of small terms
    X2 = np.zeros((1, 64), np.float32)
    X2[0, 0] = 2.0 ** 17          # 127 * 2^17 = 16,646,144 in block 0
    X2[0, 32:63] = 1.0            # 31 ones in block 1
    wq2 = np.ones((1, 64), np.int8)
    wq2[0, 0] = 127
    ws2 = np.full((1, 2), np.float16(1.0).view(np.uint16), np.uint16)
    assert oracle.q8_0_matmul(X2, wq2, ws2, accum="f32")[0, 0] == np.float32(127 * 2 ** 17 + 31)


def test_f32_and_f64_readings_agree_at_kimi_shape():
    """The two readings differ far below the layer's 1e-5 bar: the fp64 one
    may serve as the reference for a tolerance stated against fp32."""
    shp = synth.KIMI
    x = synth.block_x(shp, 3, 2)
    xf = oracle.as_f32_rows(x)
    wr = synth.router_weight(shp, 0)
    l64, l32 = oracle.router_logits(xf, wr), oracle.router_logits(xf, wr, accum="f32")
    assert rel_l2(l32, l64) <= 1e-6
    ids, w64 = oracle.topk(l64, shp.k)
    assert rel_l2(oracle.topk(l64, shp.k, accum="f32")[1], w64) <= 1e-6
    ys64, ys32 = [], []
    for e in (int(ids[0, 0]), shp.n_routed):  # one routed and one shared expert
        rec = synth.expert_record(shp, 0, e)
        y64, y32 = oracle.expert_ffn(xf, rec, shp.d, shp.f), oracle.expert_ffn(xf, rec, shp.d, shp.f, accum="f32")
        assert rel_l2(y32, y64) <= 1e-6, e
        ys64.append(y64)
        ys32.append(y32)
    X, (wq, ws) = synth.q8_0_x(4, 1, 7168), synth.q8_0_weight(4, 7168, 2048)
    assert rel_l2(oracle.q8_0_matmul(X, wq, ws, accum="f32"), oracle.q8_0_matmul(X, wq, ws)) <= 1e-6


# ----------------------------------------------------------------------------- MX-scaled tile
def test_e4m3_values_from_the_format():
    """OCP FP8 E4M3: bias 7, 3 mantissa bits, subnormals m * 2^-9, no
    infinities, 0x7F/0xFF NaN, largest 448."""
    assert oracle.e4m3(0x38) == 1.0 and oracle.e4m3(0xB8) == -1.0
    assert oracle.e4m3(0x7E) == 448.0 and oracle.e4m3(0xFE) == -448.0
    assert oracle.e4m3(0x08) == 2.0 ** -6 and oracle.e4m3(0x07) == 7 * 2.0 ** -9 and oracle.e4m3(0x01) == 2.0 ** -9
    assert oracle.e4m3(0x00) == 0.0 and math.copysign(1.0, oracle.e4m3(0x80)) == -1.0
    assert math.isnan(oracle.e4m3(0x7F)) and math.isnan(oracle.e4m3(0xFF))
    pos = [oracle.e4m3(c) for c in range(0x7F)]
    assert all(a < b for a, b in zip(pos, pos[1:]))  # positive codes are ordered by value
    assert all(oracle.e4m3(c | 0x80) == -oracle.e4m3(c) for c in range(0x7F))
    # 4 significant bits: every value is an integer multiple of its binade's step
    for c in range(1, 0x7F):
        v = pos[c]
        step = 2.0 ** (max(math.floor(math.log2(v)), -6) - 3)
        assert v / step == int(v / step)


def _mx_ops(seed):
    g = np.random.default_rng(seed)
    return (np.zeros((16, 64), np.uint8), np.full((16, 4), 127, np.uint8),
            g.integers(0, 0x7F, (16, 128)).astype(np.uint8), np.full((16, 4), 127, np.uint8))


def test_mx_tile_one_hot_rows_and_column_scales():
    """A row i = 1.0 at k = i (E2M1 code 2 in the low nibble for even k, the
    high one for odd k): D[i][j] = B[i][j] * sB[j][0]."""
    a, sa, b, sb = _mx_ops(1)
    for i in range(16):
        a[i, i // 2] = 2 << (4 * (i & 1))
    sb[:, 0] = 127 + (np.arange(16) % 3)
    d = oracle.mx_tile(a, sa, b, sb)
    for i in range(16):
        for j in range(16):
            assert d[i, j] == oracle.e4m3(b[j, i]) * 2.0 ** (j % 3), (i, j)


def test_mx_tile_block_scales_cover_their_32_elements():
    """A row i = 1.0 at k = 32 (i % 4) + i // 4 with sA[i][blk] = 2^blk and
    sB[j][blk] = 2^-blk: D[i][j] = B[k][j] (the two scales of that block)."""
    a, sa, b, sb = _mx_ops(2)
    for i in range(16):
        k = 32 * (i % 4) + i // 4
        a[i, k // 2] = 2 << (4 * (k & 1))
    sa[:] = 127 + np.arange(4)[None, :]
    sb[:] = 127 - np.arange(4)[None, :]
    d = oracle.mx_tile(a, sa, b, sb)
    for i in range(16):
        k = 32 * (i % 4) + i // 4
        for j in range(16):
            assert d[i, j] == oracle.e4m3(b[j, k]), (i, j)


def test_mx_tile_nibble_order_and_sum():
    """Byte c of an A row holds element 2c (low nibble) and 2c+1 (high):
    codes 2 (1.0) low and 4 (2.0) high in byte 0 give B[0] + 2 B[1]."""
    a, sa, b, sb = _mx_ops(3)
    a[:, 0] = 2 | (4 << 4)
    d = oracle.mx_tile(a, sa, b, sb)
    for j in range(16):
        assert d[0, j] == oracle.e4m3(b[j, 0]) + 2 * oracle.e4m3(b[j, 1])
