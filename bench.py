"""Benchmark of the MXFP4 mixture-of-experts layer on one MI355X.

One step = one whole MoE layer pass (router GEMV + top-k, bucketing, expert
FFN, combine) over one batch of rows, through the C ABI, with every input
already resident in HBM.  The headline workload is the Kimi-K3.1-shaped
decode layer at 1 row: d=7168, f=1536, 896 routed experts (top-16) plus 2
shared, MXFP4 experts (17,547,264 bytes each), bf16 x, fp32 router.  The
16-row verification block, the 1,533-row prefill and the Q8_0 spine matmul
are reported in "results".

Prints ONE JSON line (see the keys below).  --gpus N > 1 is refused: this
path runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA, published


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--no-extra", action="store_true", help="skip the 16-row, prefill and Q8_0 results")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-rows", type=int, default=6)
    p.add_argument("--only", default="", help="comma list of workloads to run: decode1,block16,prefill,q8_0")
    return p.parse_args()


class Timer:
    """HIP events recorded on the stream the kernels run on."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream
        self.pairs = []

    def start(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record(self.stream)
        self.pairs.append([e, None])

    def stop(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record(self.stream)
        self.pairs[-1][1] = e

    def ms(self):
        self.stream.synchronize()
        return [a.elapsed_time(b) for a, b in self.pairs]


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU; --gpus must be 1", "n_gpus": args.gpus}))
        sys.exit(2)
    import numpy as np
    import torch

    import router_top_bucket_amd as moe
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream(device=dev)
    only = set(args.only.split(",")) if args.only else {"decode1", "block16", "prefill", "q8_0"}
    if args.no_extra:
        only = {"decode1"}

    shp = synth.KIMI
    seed = 0
    t0 = time.time()
    base = synth.device_experts(shp, seed, device=dev)
    experts = moe.Experts(base, shp.stride, shp.d, shp.f, shp.n_routed, shp.n_shared)
    wr = torch.from_numpy(synth.router_weight(shp, seed)).to(dev)
    log(f"[bench] layer resident: {shp.n_experts} experts, {base.numel() / 1e9:.2f} GB in {time.time() - t0:.1f}s")
    results = {}

    def run_layer(layer, xs, logits=None, steps=args.steps, warmup=args.warmup, ffn_timer=None):
        """Time `steps` layer passes cycling through the row batches xs."""
        n = len(xs)
        with torch.cuda.stream(stream):
            for i in range(warmup):
                layer.forward(xs[i % n], None if logits is None else logits[i % n], stream=stream)
            stream.synchronize()
            t_all = Timer(torch, stream)
            t_all.start()
            for i in range(steps):
                layer.forward(xs[i % n], None if logits is None else logits[i % n], stream=stream)
            t_all.stop()
            total_ms = t_all.ms()[0]
            # the expert-FFN call bracketed alone (same inputs), for the roofline
            ffn = Timer(torch, stream)
            na = []
            for i in range(min(steps, 4 * n)):
                v = layer.forward(xs[i % n], None if logits is None else logits[i % n], stream=stream)
                M = xs[i % n].shape[0]
                ffn.start()
                moe.moe_expert_ffn_mxfp4(xs[i % n], layer.k, layer.experts, v["offsets"], v["perm"], v["active"],
                                         v["n_active"], v["y_slots"], layer.workspace, stream=stream)
                ffn.stop()
            ffn_ms = ffn.ms()
            for i in range(n):
                v = layer.forward(xs[i], None if logits is None else logits[i], stream=stream)
                stream.synchronize()
                na.append(int(v["n_active"].item()))
        return total_ms / steps, float(np.mean(ffn_ms)), float(np.mean(na))

    # ------------------------------------------------------------ headline: 1 row
    M = 1
    pool = 64
    xs = [torch.from_numpy(synth.rows_x(shp, 1000 + i, M)).view(torch.bfloat16).to(dev) for i in range(pool)]
    layer1 = moe.MoELayer(experts, shp.k, M, w_router=wr)
    ms_step, ffn_ms, n_act = run_layer(layer1, xs)
    rows_s = M / (ms_step / 1e3)
    eff_gbs = n_act * shp.stride / (ms_step / 1e3) / 1e9
    x_bytes = M * shp.d * 2
    y_bytes = M * (shp.k + shp.n_shared) * shp.d * 4
    ffn_alg_bytes = n_act * shp.stride + x_bytes + y_bytes
    ffn_gbs = ffn_alg_bytes / (ffn_ms / 1e3) / 1e9
    results["decode_1row"] = dict(rows=M, ms_per_layer=ms_step, rows_per_s=rows_s, experts_read=n_act,
                                  effective_weight_GBps=eff_gbs, hbm_frac_effective=eff_gbs / HBM_PEAK_GBS,
                                  ffn_ms=ffn_ms, ffn_GBps=ffn_gbs)
    log(f"[bench] 1 row: {ms_step * 1e3:.1f} us/layer, {rows_s:.0f} rows/s, eff {eff_gbs:.0f} GB/s, "
        f"ffn {ffn_ms * 1e3:.1f} us ({ffn_gbs:.0f} GB/s)")

    # ------------------------------------------------------------ 16-row verification blocks
    if "block16" in only:
        B = 16
        xs16 = [torch.from_numpy(synth.block_x(shp, s, B)).view(torch.bfloat16).to(dev) for s in range(20)]
        layer16 = moe.MoELayer(experts, shp.k, B, w_router=wr)
        ms16, ffn16, na16 = run_layer(layer16, xs16, steps=max(20, args.steps // 4), warmup=5)
        results["block_16rows"] = dict(rows=B, ms_per_layer=ms16, rows_per_s=B / (ms16 / 1e3), experts_read=na16,
                                       effective_weight_GBps=na16 * shp.stride / (ms16 / 1e3) / 1e9,
                                       hbm_frac_effective=na16 * shp.stride / (ms16 / 1e3) / 1e9 / HBM_PEAK_GBS,
                                       ffn_ms=ffn16)
        log(f"[bench] 16 rows: {ms16 * 1e3:.1f} us/layer, {B / (ms16 / 1e3):.0f} rows/s, U+S={na16:.1f}")
        del layer16

    # ------------------------------------------------------------ prefill 1533 rows
    if "prefill" in only:
        Mp = 1533
        xs_p = [torch.from_numpy(synth.rows_x(shp, 2000 + s, Mp)).view(torch.bfloat16).to(dev) for s in range(3)]
        lg_p = [torch.from_numpy(synth.zipf_logits(shp, 2000 + s, Mp)).to(dev) for s in range(3)]
        layerp = moe.MoELayer(experts, shp.k, Mp)
        msp, ffnp, nap = run_layer(layerp, xs_p, logits=lg_p, steps=10, warmup=2)
        flops = 2.0 * Mp * (shp.k + shp.n_shared) * 3 * shp.d * shp.f
        results["prefill_1533rows"] = dict(rows=Mp, ms_per_layer=msp, rows_per_s=Mp / (msp / 1e3),
                                           experts_read=nap,
                                           effective_weight_GBps=nap * shp.stride / (msp / 1e3) / 1e9,
                                           hbm_frac_effective=nap * shp.stride / (msp / 1e3) / 1e9 / HBM_PEAK_GBS,
                                           useful_TFLOPs=flops / (msp / 1e3) / 1e12,
                                           mfma_frac=flops / (msp / 1e3) / 1e12 / MFMA_BF16_PEAK_TFS,
                                           routing="given Zipf(1.1) logits", ffn_ms=ffnp)
        log(f"[bench] prefill 1533: {msp:.3f} ms/layer, {Mp / (msp / 1e3):.0f} rows/s, experts {nap:.0f}, "
            f"{flops / (msp / 1e3) / 1e12:.1f} TFLOP/s")
        del layerp

    # ------------------------------------------------------------ Q8_0 spine matmul
    if "q8_0" in only:
        q8 = {}
        for (K, N) in synth.Q8_0_SHAPES:
            wq, ws = synth.q8_0_weight(3, K, N)
            dwq = torch.from_numpy(wq).to(dev)
            dws = torch.from_numpy(ws.view(np.int16)).to(dev)
            del wq, ws
            for Mq in (1, 2, 4, 8):
                X = torch.from_numpy(synth.q8_0_x(3, Mq, K)).to(dev)
                Y = torch.empty((Mq, N), dtype=torch.float32, device=dev)
                with torch.cuda.stream(stream):
                    for _ in range(5):
                        moe.q8_0_matmul(X, dwq, dws, Y, stream=stream)
                    t = Timer(torch, stream)
                    reps = 50
                    t.start()
                    for _ in range(reps):
                        moe.q8_0_matmul(X, dwq, dws, Y, stream=stream)
                    t.stop()
                    ms = t.ms()[0] / reps
                wbytes = N * K * 34 / 32
                gbs = (wbytes + Mq * (K + N) * 4) / (ms / 1e3) / 1e9
                q8[f"K{K}_N{N}_M{Mq}"] = dict(us=ms * 1e3, GBps=gbs, hbm_frac=gbs / HBM_PEAK_GBS)
                log(f"[bench] q8_0 K={K} N={N} M={Mq}: {ms * 1e3:.1f} us, {gbs:.0f} GB/s")
            del dwq, dws
        results["q8_0"] = q8

    # ------------------------------------------------------------ CPU baseline: the oracle
    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        nrows = args.cpu_sample_rows
        xh = synth.rows_x(shp, 1000, nrows)
        wr_h = synth.router_weight(shp, seed)
        cache = {}

        def rec(e):
            if e not in cache:
                cache[e] = synth.expert_record(shp, seed, e)
            return cache[e]

        # records are generated before the clock starts: input preparation, not oracle work
        lg = oracle.router_logits(xh, wr_h)
        ids, _ = oracle.topk(lg, shp.k)
        for e in set(ids.ravel().tolist()) | {shp.n_routed + s for s in range(shp.n_shared)}:
            rec(e)
        t1 = time.time()
        for m in range(nrows):
            oracle.layer(xh[m:m + 1], shp.k, shp.n_routed, shp.n_shared, shp.d, shp.f, rec, w_r=wr_h)
        dt = time.time() - t1
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
        cpu = dict(value=nrows / dt, unit="rows/s", cores=threads, kind="oracle",
                   sample=f"{nrows} rows of the 1-row Kimi layer, one layer call per row (router + top-16 + "
                          f"18 expert FFNs + combine), fp64 C oracle, {dt:.1f} s")
        log(f"[bench] cpu oracle: {nrows / dt:.3f} rows/s on {threads} threads")

    line = {
        "metric": "MoE-layer rows/s + effective MXFP4 weight GB/s at 1, 16, 1533 rows",
        "value": rows_s,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "kimi_moe_layer_decode_1row", "d": shp.d, "f": shp.f, "routed_experts": shp.n_routed,
                   "shared_experts": shp.n_shared, "top_k": shp.k, "rows": 1, "weights": "mxfp4",
                   "x": "bf16", "router": "fp32", "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "kernel": "moe_expert_ffn_mxfp4 (ffn_gateup + ffn_down)",
                     "achieved": ffn_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ffn_gbs / HBM_PEAK_GBS,
                     "traffic": None},
        "effective_weight_GBps": eff_gbs,
        "cpu_baseline": cpu,
        "results": results,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
