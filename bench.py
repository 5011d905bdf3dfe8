"""Benchmark of the MXFP4 mixture-of-experts layer on one MI355X.

One step = one whole MoE layer pass (router GEMV + top-k, bucketing, expert
FFN, combine) over one batch of rows, through the C ABI, with every input
already resident in HBM.  The headline workload is the Kimi-K3.1-shaped
decode layer at 1 row: d=7168, f=1536, 896 routed experts (top-16) plus 2
shared, MXFP4 experts (17,547,264 bytes each), bf16 x, fp32 router.  The
16-row verification block, the 1,533-row prefill, the Q8_0 spine matmul, the
experts streamed from a pinned host pool through a device cache, and block
verification over a stack of the resident layers are reported in "results".

Timing: four distinct layers are resident (63 GB) and consecutive steps run
consecutive layers, as a model's decode pass does, with input batches
rotating too; so no expert, router matrix or Q8_0 weight is read again
within 1 GB of other traffic and none can be served from L2 or the 256 MB
memory-side cache.  One pair of HIP events on the kernels' stream brackets
K back-to-back steps.  The layer is timed eagerly (one C-ABI call after
another) and replayed from HIP graphs captured per (layer, batch); the
headline value is the faster of the two.

Prints ONE JSON line.  --gpus N > 1 is refused: this path runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA, published
N_LAYERS = 4  # distinct resident layers the steps rotate through
BLOCK_SIGMA = 0.3  # spread of a verification block's rows around row 0
# rocprofv3 counter summary of the gate/up kernel on the 1-row workload; its
# traffic figure is used only while the kernel sources are the ones it was
# measured on
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "ffn_gateup_kimi_decode_1row_traffic.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "router_top_bucket_amd", "csrc", n) for n in ("ffn.hip", "common.h")]
# every kernel source of a layer pass (the layer traffic figure's validity)
LAYER_SOURCES = [os.path.join(ROOT, "router_top_bucket_amd", "csrc", n)
                 for n in ("ffn.hip", "common.h", "route.hip", "bucket.hip", "topk.h")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--no-extra", action="store_true", help="skip the 16-row, prefill and Q8_0 results")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-rows", type=int, default=25)
    p.add_argument("--only", default="",
                   help="comma list of workloads: decode1,block16,prefill,q8_0,stream,verify (copy = the copy "
                        "kernel that calibrates the HBM counters, run alone)")
    return p.parse_args()


def kernel_sources_sha(paths=None) -> str:
    h = hashlib.sha256()
    for p in (KERNEL_SOURCES if paths is None else paths):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_layer():
    """HBM bytes per 1-row layer pass from the committed counter summary of
    every kernel of the pass, or None when absent or taken on other sources."""
    path = os.path.join(ROOT, "profiles", "moe_kernels_kimi_decode_1row_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_sources_sha256") != kernel_sources_sha(LAYER_SOURCES):
        return None
    try:
        return float(kv["layer_traffic_bytes"])
    except (KeyError, ValueError):
        return None


def measured_traffic():
    """Bytes per launch of the gate/up kernel from the committed counter
    summary, or None when it is absent or was taken on other sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_sources_sha256") != kernel_sources_sha():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def layer_bytes(shp, M, n_active, router):
    """Algorithmic HBM bytes of one layer pass over M rows: every distinct
    expert record read once, the fp32 router matrix once (when the logits are
    computed), bf16 x in and fp32 output rows out."""
    return n_active * shp.stride + (shp.n_routed * shp.d * 4 if router else 0) + M * shp.d * 2 + M * shp.d * 4


class Timer:
    """HIP events on one stream around a region of back-to-back launches."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream

    def region(self, fn, n):
        a = self.torch.cuda.Event(enable_timing=True)
        b = self.torch.cuda.Event(enable_timing=True)
        a.record(self.stream)
        for i in range(n):
            fn(i)
        b.record(self.stream)
        self.stream.synchronize()
        return a.elapsed_time(b) / n  # ms per launch


def run_verify(torch, moe, synth, shp, layers, stream, dev, timer):
    """The resident layers as a stack (Q8_0 spine 7168 x 7168 per layer, Q8_0
    head 163,840 x 7168 tied to the embedding): 16 plain greedy steps against
    one 16-row block whose drafts are those steps' tokens (all kept), timed
    without hashing; then both paths again with every position's logits
    hashed (FNV-1a) and compared."""
    import numpy as np
    from router_top_bucket_amd.blockverify import Q8Matrix, Stack, plain_steps, verify_block
    V = 163840
    spines = []
    for l in range(len(layers)):
        wq, ws = synth.q8_0_weight(400 + l, shp.d, shp.d)
        # the spine and head weights in tile order (q8_0_pack), as the experts
        spines.append(Q8Matrix(torch.from_numpy(wq).to(dev), torch.from_numpy(ws.view(np.int16)).to(dev)).tiled())
    hq, hs = synth.q8_0_weight(500, shp.d, V)
    head = Q8Matrix(torch.from_numpy(hq).to(dev), torch.from_numpy(hs.view(np.int16)).to(dev)).tiled()
    del hq, hs
    torch.cuda.synchronize()
    stack = Stack(layers, spines, head, shp.k, 16, device=dev)
    t0 = 1234
    with torch.cuda.stream(stream):
        plain, _ = plain_steps(stack, t0, 16, hashes=False)  # the drafts, and a warm-up
        drafts = plain[:15]
        verify_block(stack, t0, drafts, hashes=False)
        reps = 5
        stream.synchronize()
        t1 = time.perf_counter()
        for _ in range(reps):
            plain_steps(stack, t0, 16, hashes=False)
        stream.synchronize()
        plain_ms = (time.perf_counter() - t1) / reps * 1e3
        t1 = time.perf_counter()
        for _ in range(reps):
            emitted, kept, _ = verify_block(stack, t0, drafts, hashes=False)
        stream.synchronize()
        block_ms = (time.perf_counter() - t1) / reps * 1e3
        p_tok, p_hash = plain_steps(stack, t0, 16)
        b_tok, b_kept, b_hash = verify_block(stack, t0, drafts)
    differ = sum(int(a != b) for a, b in zip(p_hash, b_hash))
    # the same two paths replayed from HIP graphs (no host launch overhead):
    # one plain step fed the previous step's choice, and the 16-row block
    blk = torch.tensor([t0] + drafts, dtype=torch.int32, device=dev)
    cap = torch.cuda.Stream(device=dev)
    cap.wait_stream(stream)
    g1, gb = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g1, stream=cap):
        stack.run(stack.next[:1])
    with torch.cuda.graph(gb, stream=cap):
        stack.run(blk)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        def plain_graph(i):
            if i % 16 == 0:
                stack.next[:1].fill_(t0)
            g1.replay()

        for i in range(16):
            plain_graph(i)
        plain_g_ms = timer.region(plain_graph, 16 * reps) * 16
        plain_graph(0)
        for i in range(1, 16):
            plain_graph(i)
        chain_ok = int(stack.next[0].item()) == p_tok[15]
        gb.replay()
        block_g_ms = timer.region(lambda i: gb.replay(), reps)
        block_ok = stack.next[:16].cpu().tolist() == p_tok[:16]
    del g1, gb
    r = dict(layers=len(layers), vocab=V, plain_16_steps_ms=plain_ms, block_16rows_ms=block_ms,
             block_speedup=plain_ms / block_ms, plain_16_steps_graph_ms=plain_g_ms, block_16rows_graph_ms=block_g_ms,
             block_speedup_graph=plain_g_ms / block_g_ms, graph_paths_match=bool(chain_ok and block_ok),
             drafts_kept=b_kept, tokens_equal=(b_tok == p_tok), positions_hashed=len(b_hash),
             hashes_differing=differ)
    log(f"[bench] verify: {len(layers)} layers + head, 16 plain steps {plain_ms:.2f} ms, one 16-row block "
        f"{block_ms:.2f} ms ({plain_ms / block_ms:.1f}x); from graphs {plain_g_ms:.2f} vs {block_g_ms:.2f} ms "
        f"({plain_g_ms / block_g_ms:.1f}x, tokens match {chain_ok and block_ok}); {b_kept} drafts kept, tokens "
        f"equal {b_tok == p_tok}, {differ} of {len(b_hash)} logits hashes differ")
    del stack, spines, head
    return {"verify_block_vs_plain": r}


def run_stream(torch, moe, synth, shp, layers, stream, dev):
    """Experts streamed from a pinned host pool of 2 layers through a device
    cache holding 272 routed experts (15% of the pool's): 1-row decode steps
    and 16-row blocks (LRU, then admission of experts used by >= 2 rows).
    Each call synchronises its stream once (the host learns the routing), so
    the wall clock between two synchronisations times a run of calls."""
    L, E, S = 2, shp.n_routed, shp.n_shared
    rec = shp.n_experts * shp.stride
    t0 = time.time()
    host = torch.empty(L * rec, dtype=torch.uint8, pin_memory=True)
    for l in range(L):
        host[l * rec:(l + 1) * rec].copy_(layers[l][0].base)
    n_transient, n_cache = 32, 240
    n_slots = L * S + n_transient + n_cache
    pool = torch.empty(n_slots * shp.stride, dtype=torch.uint8, device=dev)
    log(f"[bench] stream: {L} layers in pinned host memory ({L * rec / 1e9:.1f} GB) in {time.time() - t0:.1f}s, "
        f"device cache {n_slots} slots ({n_slots * shp.stride / 1e9:.1f} GB)")
    # host -> device ceiling: 64 records (1.1 GB) as one copy, and as 8
    # contiguous pieces on 8 streams; the faster of the two
    ups = [torch.cuda.Stream(device=dev) for _ in range(8)]
    nb = 64 * shp.stride
    pcie = 0.0
    for pieces in (1, 8, 1, 8):
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for j in range(pieces):
            a, b = nb * j // pieces, nb * (j + 1) // pieces
            with torch.cuda.stream(ups[j]):
                pool[a:b].copy_(host[a:b], non_blocking=True)
        torch.cuda.synchronize()
        pcie = max(pcie, nb / (time.perf_counter() - t1) / 1e9)
    log(f"[bench] stream: host->device copies {pcie:.1f} GB/s")
    out = {"stream_pcie_h2d_GBps": pcie}

    def run(name, M, xfn, admit, warm, n):
        cache = moe.ExpertCache(pool, host, L, E, S, shp.d, shp.f, shp.stride, n_upload_streams=8, upload_groups=4,
                                admit_min_rows=admit, n_transient=n_transient, layout=layers[0][0].layout)
        ml = moe.MoELayer(cache.descriptor(), shp.k, M)
        xs = [xfn(i) for i in range(warm + n)]

        def call(i):
            ml.w_router = layers[i % L][1]
            ml.forward_streamed(cache, i % L, xs[i], stream=stream)

        for i in range(warm):
            call(i)
        stream.synchronize()
        s0 = cache.stats()
        t1 = time.perf_counter()
        for i in range(warm, warm + n):
            call(i)
        stream.synchronize()
        dt = (time.perf_counter() - t1) / n
        s1 = cache.stats()
        cache.close()
        hits, misses = s1["hits"] - s0["hits"], s1["misses"] - s0["misses"]
        up = (s1["bytes_uploaded"] - s0["bytes_uploaded"]) / n
        r = dict(rows=M, ms_per_layer=dt * 1e3, rows_per_s=M / dt, hit_rate=hits / max(hits + misses, 1),
                 misses_per_layer=misses / n, upload_GBps=up / dt / 1e9, upload_frac_of_h2d=up / dt / 1e9 / pcie,
                 admit_min_rows=admit, layers_in_host_pool=L, cached_slots=n_cache, transient_slots=n_transient)
        log(f"[bench] stream {name}: {dt * 1e3:.2f} ms/layer ({M / dt:.1f} rows/s), hit rate "
            f"{r['hit_rate']:.2f}, {r['misses_per_layer']:.1f} misses/layer, uploads {r['upload_GBps']:.1f} GB/s")
        out[f"stream_{name}"] = r

    def x1(i):
        return torch.from_numpy(synth.rows_x(shp, 5000 + i // L, 1)).view(torch.bfloat16).to(dev)

    def x16(i):
        return torch.from_numpy(synth.block_x(shp, 6000 + i // L, 16)).view(torch.bfloat16).to(dev)

    run("decode_1row", 1, x1, 0, 20, 60)
    run("block_16rows_lru", 16, x16, 0, 8, 24)
    run("block_16rows_admit2", 16, x16, 2, 8, 24)
    del pool, host
    return out


# The pages' own end-to-end figures: the whole Kimi K3.1 model (92 MoE
# layers plus attention, spine and head) on a single RTX PRO 6000 Blackwell
# (96 GB), experts streamed from NVMe ("A drafter that leaves the answer
# unchanged" and the published run record).  Context only: another machine,
# another scope.
PAGE_BLOCK_16ROWS_S = 3.8
PAGE_PLAIN_16_STEPS_S = 8.0
PAGE_STEADY_DECODE_TOK_S = (1.92, 2.61)
MOE_LAYERS = 92


def page_context(results):
    """The pages' figures next to the time this GPU spends in the MoE layers
    alone for the same work (92 resident layers, nothing else of the model)."""
    out = {"note": "pages: whole model, one RTX PRO 6000 96 GB, experts streamed from NVMe; ours: the MoE "
                   "layers only (92 x this layer, experts resident in HBM), no attention, spine or head",
           "pages_block_16rows_s": PAGE_BLOCK_16ROWS_S, "pages_plain_16_steps_s": PAGE_PLAIN_16_STEPS_S,
           "pages_steady_decode_tok_s": list(PAGE_STEADY_DECODE_TOK_S)}
    d1, b16 = results.get("decode_1row"), results.get("block_16rows")
    if d1:
        out["ours_moe_layers_plain_16_steps_s"] = 16 * MOE_LAYERS * d1["ms_per_layer"] / 1e3
        out["ours_moe_layers_decode_tok_s"] = 1e3 / (MOE_LAYERS * d1["ms_per_layer"])
    if b16:
        out["ours_moe_layers_block_16rows_s"] = MOE_LAYERS * b16["ms_per_layer"] / 1e3
    return out


def cpu_info():
    """The host's CPU model and the CPUs this process may run on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count()
    return {"cpu_model": model, "cpus_available": avail, "logical_cpus": os.cpu_count()}


def run_cpu_baseline(args, synth, shp, results):
    """The oracle (the plain C reference, fp64 accumulation, OpenMP over
    output elements) timed on this host's cores on bounded samples of each
    workload, each figure placed beside the GPU figure it matches; the
    headline object is the 1-row layer.  Expert records are generated before
    any clock starts."""
    import numpy as np

    import oracle

    threads = oracle.max_threads()
    info = cpu_info()
    seed = 0
    wr_h = synth.router_weight(shp, seed)
    cache = {}

    def rec(e):
        if e not in cache:
            cache[e] = synth.expert_record(shp, seed, e)
        return cache[e]

    def prepare(x, logits=None):
        lg = oracle.router_logits(x, wr_h) if logits is None else logits
        ids, _ = oracle.topk(lg, shp.k)
        for e in set(ids.ravel().tolist()) | {shp.n_routed + s for s in range(shp.n_shared)}:
            rec(e)

    def layer(x, logits=None):
        if logits is None:
            return oracle.layer(x, shp.k, shp.n_routed, shp.n_shared, shp.d, shp.f, rec, w_r=wr_h)
        return oracle.layer(x, shp.k, shp.n_routed, shp.n_shared, shp.d, shp.f, rec, logits=logits)

    def clock(fn, nthreads=threads):
        oracle.set_threads(nthreads)
        t = time.perf_counter()
        fn()
        dt = time.perf_counter() - t
        oracle.set_threads(threads)
        return dt

    def attach(name, fig):
        if name in results:
            results[name]["cpu_oracle"] = fig

    # headline: rows of the 1-row layer, one layer call per row
    nrows = args.cpu_sample_rows
    xh = synth.rows_x(shp, 1000, nrows)
    prepare(xh)
    dt = clock(lambda: [layer(xh[m:m + 1]) for m in range(nrows)])
    dt1 = clock(lambda: layer(xh[:1]), 1)
    attach("decode_1row", {"rows_per_s": nrows / dt, "threads": threads, "seconds": dt, "sample": f"{nrows} rows",
                           "rows_per_s_1thread": 1 / dt1})
    log(f"[bench] cpu oracle 1-row layer: {nrows / dt:.3f} rows/s on {threads} threads, {1 / dt1:.3f} on 1")
    headline = {"value": nrows / dt, "unit": "rows/s", "cores": threads, "kind": "oracle",
                "sample": f"{nrows} rows of the 1-row Kimi layer, one layer call per row (router + top-16 + 18 expert "
                          f"FFNs + combine), C oracle with fp64 accumulation, {dt:.1f} s on {threads} OpenMP threads",
                "cpu": info, "rows_per_s_1thread": 1 / dt1}

    # the tiny layer (20 rows, one call per row), N threads and 1 thread
    tshp = synth.TINY
    trecs = {e: synth.expert_record(tshp, 0, e) for e in range(tshp.n_experts)}
    twr = synth.router_weight(tshp, 0)
    tx = synth.rows_x(tshp, 0, 20)

    def tiny():
        for m in range(20):
            oracle.layer(tx[m:m + 1], tshp.k, tshp.n_routed, 0, tshp.d, tshp.f, trecs.__getitem__, w_r=twr)

    tn, t1 = clock(tiny), clock(tiny, 1)
    headline["tiny_layer_rows_per_s"] = 20 / tn
    headline["tiny_layer_rows_per_s_1thread"] = 20 / t1

    # verification blocks: one block per workload
    for name, B, sigma in (("block_16rows", 16, BLOCK_SIGMA), ("block_2rows", 2, BLOCK_SIGMA),
                           ("block_8rows", 8, BLOCK_SIGMA), ("block_16rows_sigma0.5", 16, 0.5),
                           ("block_16rows_sigma1", 16, 1.0)):
        if name not in results:
            continue
        xb = synth.block_x(shp, 0, B, sigma=sigma)
        prepare(xb)
        dtb = clock(lambda: layer(xb))
        attach(name, {"rows_per_s": B / dtb, "threads": threads, "seconds": dtb, "sample": "1 block (seed 0)"})
        log(f"[bench] cpu oracle {name}: {B / dtb:.2f} rows/s")

    # prefill: routing, bucketing and combine in full; the expert FFNs timed
    # on 8 experts spread over the popularity range, each with all its rows,
    # and extrapolated to every active expert with t = a + b * rows
    for Mp in (1533, 270):
        name = f"prefill_{Mp}rows"
        if name not in results:
            continue
        xp = oracle.as_f32_rows(synth.rows_x(shp, 2000, Mp))
        lgp = synth.zipf_logits(shp, 2000, Mp)
        kps = shp.k + shp.n_shared
        t0 = time.perf_counter()
        ids, wts = oracle.topk(lgp, shp.k)
        off, perm, act, na = oracle.bucket(ids, shp.n_routed, shp.n_shared)
        t_route = time.perf_counter() - t0
        counts = np.diff(off)[act]
        order = act[np.argsort(counts, kind="stable")]
        pick = sorted(set(order[np.linspace(0, len(order) - 1, 8).astype(int)].tolist()))
        xs_, ts_ = [], []
        for e in pick:
            seg = perm[off[e]:off[e + 1]]
            rows = xp[seg // kps]
            rec(int(e))
            xs_.append(len(seg))
            ts_.append(clock(lambda: oracle.expert_ffn(rows, rec(int(e)), shp.d, shp.f)))
        b, a = np.polyfit(np.array(xs_, float), np.array(ts_, float), 1)
        t_ffn = float(np.sum(a + b * counts))
        y0 = np.zeros((Mp * kps, shp.d), np.float32)
        t_comb = clock(lambda: oracle.combine(y0, wts, shp.k, shp.n_shared))
        tot = t_route + t_ffn + t_comb
        attach(name, {"rows_per_s": Mp / tot, "threads": threads, "seconds_estimated": tot,
                      "sample": f"routing, bucketing and combine timed in full; the FFNs of 8 of the {na} active "
                                f"experts timed with all their rows ({sum(xs_)} slots) and extrapolated linearly "
                                f"in rows to all {int(counts.sum())} slots"})
        log(f"[bench] cpu oracle {name}: {Mp / tot:.2f} rows/s (estimated {tot:.1f} s per layer)")

    # Q8_0: up to 4096 output columns per shape, scaled to N (the work is
    # linear in N); 1 thread at M = 1
    if "q8_0" in results:
        for (K, N) in synth.Q8_0_SHAPES:
            ncol = min(N, 4096)
            wq, ws = synth.q8_0_weight(3, K, ncol)
            for Mq in (1, 2, 4, 8):
                X = synth.q8_0_x(3, Mq, K)
                dtq = clock(lambda: oracle.q8_0_matmul(X, wq, ws)) * N / ncol
                fig = {"us": dtq * 1e6, "threads": threads, "sample": f"{ncol} of {N} columns, scaled"}
                if Mq == 1:
                    fig["us_1thread"] = clock(lambda: oracle.q8_0_matmul(X, wq, ws), 1) * N / ncol * 1e6
                key = f"K{K}_N{N}_M{Mq}"
                if key in results["q8_0"]:
                    results["q8_0"][key]["cpu_oracle"] = fig
        log("[bench] cpu oracle q8_0: done")
    return headline


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
    timer = Timer(torch, stream)
    only = (set(args.only.split(",")) if args.only else
            {"decode1", "block16", "prefill", "q8_0", "stream", "verify"})
    if args.no_extra:
        only = {"decode1"}

    if only == {"copy"}:
        # a plain device copy of known size: the reference the HBM byte
        # counters of the kernels are scaled by
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        with torch.cuda.stream(stream):
            for _ in range(5):
                dst.copy_(src)
        stream.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel() * 4, "copy_bytes_written": dst.numel() * 4,
                          "launches": 5}), flush=True)
        return

    shp = synth.KIMI
    L = N_LAYERS
    t0 = time.time()
    layers = []
    for seed in range(L):
        # records are generated in row order, then packed to tile order (the
        # order the kernels read fastest; outputs are the same bits)
        rows = moe.Experts(synth.device_experts(shp, seed, device=dev), shp.stride, shp.d, shp.f, shp.n_routed,
                           shp.n_shared)
        layers.append((moe.tile_experts(rows), torch.from_numpy(synth.router_weight(shp, seed)).to(dev)))
        del rows
    log(f"[bench] {L} layers resident: {L * shp.n_experts} experts, {L * shp.n_experts * shp.stride / 1e9:.1f} GB "
        f"in {time.time() - t0:.1f}s (codes planes in tile order)")
    results = {}
    gu_bytes_per_expert = 2 * shp.f * shp.d * 17 // 32  # gate + up, codes and scales

    def run_workload(M, xs, logits, steps, warmup, graphs=True):
        """Eager (and, with ``graphs``, graph-replayed) layer passes plus the
        gate/up stage alone and the whole FFN call, step i on layer i % L with
        batch i % len(xs)."""
        n = len(xs)
        P = int(np.lcm(n, L))
        mls = [moe.MoELayer(ex, shp.k, M, w_router=None if logits is not None else wr) for ex, wr in layers]

        def pair(i):
            return mls[i % L], xs[i % n], (None if logits is None else logits[i % n])

        def fwd(i, s=stream):
            ml, x, lg = pair(i)
            return ml.forward(x, lg, stream=s)

        for i in range(warmup):
            fwd(i)
        eager_ms = timer.region(fwd, steps)
        graph_ms = None
        if graphs:
            cap = torch.cuda.Stream(device=dev)
            cap.wait_stream(stream)
            gs = []
            for i in range(P):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=cap):
                    fwd(i, None)
                gs.append(g)
            torch.cuda.synchronize()

            def rep(i):
                with torch.cuda.stream(stream):
                    gs[i % P].replay()

            for i in range(warmup):
                rep(i)
            graph_ms = timer.region(rep, steps)
            del gs
        # each (layer, batch) pair's routing, kept for timing the FFN stages
        routes = []
        for i in range(P):
            v = fwd(i)
            # the copies go on the layer's stream, after the pass that writes them
            with torch.cuda.stream(stream):
                routes.append({k: v[k].clone() for k in ("offsets", "perm", "active", "n_active")})
        stream.synchronize()
        na = np.array([int(r["n_active"].item()) for r in routes], dtype=np.float64)

        def gu(i):
            ml, x, _ = pair(i)
            r = routes[i % P]
            moe.moe_ffn_gateup_mxfp4(x, shp.k, ml.experts, r["offsets"], r["perm"], r["active"], r["n_active"],
                                     ml.workspace, stream=stream)

        def ffn(i):
            ml, x, _ = pair(i)
            r = routes[i % P]
            moe.moe_expert_ffn_mxfp4(x, shp.k, ml.experts, r["offsets"], r["perm"], r["active"], r["n_active"],
                                     ml.y_slots[:M * (shp.k + shp.n_shared)], ml.workspace, stream=stream)

        for i in range(warmup):
            ffn(i)
        gu_ms = timer.region(gu, steps)
        ffn_ms = timer.region(ffn, steps)
        # mean experts read per step over the steps timed
        na_mean = float(np.mean([na[i % P] for i in range(steps)]))
        del mls
        return dict(eager_ms=eager_ms, graph_ms=graph_ms, gu_ms=gu_ms, ffn_ms=ffn_ms, n_active=na_mean,
                    router=logits is None)

    def layer_result(M, r):
        ms = min(r["eager_ms"], r["graph_ms"]) if r["graph_ms"] is not None else r["eager_ms"]
        T = M * (shp.k + shp.n_shared)
        # algorithmic bytes of the gate/up stage: each expert's gate and up
        # weights once, x in (bf16), h out (fp32)
        gu_alg = r["n_active"] * gu_bytes_per_expert + M * shp.d * 2 + T * shp.f * 4
        eff = r["n_active"] * shp.stride / (ms / 1e3) / 1e9
        # the layer's algorithmic bytes: each distinct expert's record once,
        # the router matrix once when the logits are computed, x in and the
        # output rows out
        lay = layer_bytes(shp, M, r["n_active"], r["router"])
        return dict(rows=M, ms_per_layer=ms, ms_per_layer_eager=r["eager_ms"], ms_per_layer_graph=r["graph_ms"],
                    rows_per_s=M / (ms / 1e3), experts_read=r["n_active"], effective_weight_GBps=eff,
                    hbm_frac_effective=eff / HBM_PEAK_GBS, layer_alg_bytes=lay,
                    layer_GBps=lay / (ms / 1e3) / 1e9, layer_hbm_frac=lay / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
                    gateup_us=r["gu_ms"] * 1e3,
                    gateup_GBps=gu_alg / (r["gu_ms"] / 1e3) / 1e9, gateup_alg_bytes=gu_alg,
                    down_us_derived=(r["ffn_ms"] - r["gu_ms"]) * 1e3, ffn_us=r["ffn_ms"] * 1e3)

    # ------------------------------------------------------------ headline: 1 row
    if "decode1" in only:
        M = 1
        xs = [torch.from_numpy(synth.rows_x(shp, 1000 + i, M)).view(torch.bfloat16).to(dev) for i in range(64)]
        res = layer_result(M, run_workload(M, xs, None, args.steps, args.warmup))
        results["decode_1row"] = res
        log(f"[bench] 1 row: {res['ms_per_layer'] * 1e3:.1f} us/layer ({res['rows_per_s']:.0f} rows/s; eager "
            f"{res['ms_per_layer_eager'] * 1e3:.1f} us, graph {res['ms_per_layer_graph'] * 1e3:.1f} us); gate/up "
            f"{res['gateup_us']:.1f} us ({res['gateup_GBps']:.0f} GB/s), ffn {res['ffn_us']:.1f} us")

    # ------------------------------------------------------------ 16-row verification blocks
    if "block16" in only:
        # blocks of 16 (the reported block) and of 2 and 8 rows, rows spread
        # around row 0 with sigma 0.3; then 16-row blocks with sigma 0.5 and
        # 1.0, whose unions reach the upper end of the pages' 40-120 experts
        for B, sigma in ((16, BLOCK_SIGMA), (2, BLOCK_SIGMA), (8, BLOCK_SIGMA), (16, 0.5), (16, 1.0)):
            xsb = [torch.from_numpy(synth.block_x(shp, s, B, sigma=sigma)).view(torch.bfloat16).to(dev)
                   for s in range(20)]
            res = layer_result(B, run_workload(B, xsb, None, max(40, args.steps // 4), 5,
                                               graphs=(B == 16 and sigma == BLOCK_SIGMA)))
            res["sigma"] = sigma
            name = f"block_{B}rows" + ("" if sigma == BLOCK_SIGMA else f"_sigma{sigma:g}")
            results[name] = res
            log(f"[bench] {B} rows, sigma {sigma:g}: {res['ms_per_layer'] * 1e3:.1f} us/layer "
                f"({res['rows_per_s']:.0f} rows/s; eager {res['ms_per_layer_eager'] * 1e3:.1f} us), "
                f"U+S={res['experts_read']:.1f}, gate/up {res['gateup_us']:.1f} us, ffn {res['ffn_us']:.1f} us")

    # ------------------------------------------------------------ prefill 1533 (and 270) rows
    if "prefill" in only:
        for Mp in (1533, 270):
            xs_p = [torch.from_numpy(synth.rows_x(shp, 2000 + s, Mp)).view(torch.bfloat16).to(dev) for s in range(3)]
            lg_p = [torch.from_numpy(synth.zipf_logits(shp, 2000 + s, Mp)).to(dev) for s in range(3)]
            r = run_workload(Mp, xs_p, lg_p, 12, 2, graphs=False)
            res = layer_result(Mp, r)
            # the router on the same rows (the workload gives logits; a prompt
            # pass computes them): logits, top-k and weights
            lgo = torch.empty((Mp, shp.n_routed), dtype=torch.float32, device=dev)
            ids_o = torch.empty((Mp, shp.k), dtype=torch.int32, device=dev)
            w_o = torch.empty((Mp, shp.k), dtype=torch.float32, device=dev)

            def route(i):
                moe.moe_route(xs_p[i % len(xs_p)], layers[i % L][1], lgo, shp.k, ids_o, w_o, stream=stream)

            for i in range(2):
                route(i)
            res["router_us"] = timer.region(route, 12) * 1e3
            flops = 2.0 * Mp * (shp.k + shp.n_shared) * 3 * shp.d * shp.f
            res.update(useful_TFLOPs=flops / (res["ms_per_layer"] / 1e3) / 1e12,
                       mfma_frac=flops / (res["ms_per_layer"] / 1e3) / 1e12 / MFMA_BF16_PEAK_TFS,
                       routing="given Zipf(1.1) logits")
            results[f"prefill_{Mp}rows"] = res
            log(f"[bench] prefill {Mp}: {res['ms_per_layer']:.3f} ms/layer, experts {res['experts_read']:.0f}, "
                f"{res['useful_TFLOPs']:.1f} TFLOP/s, gate/up {res['gateup_us'] / 1e3:.3f} ms, "
                f"ffn {res['ffn_us'] / 1e3:.3f} ms; router on these rows {res['router_us']:.1f} us")

    # ------------------------------------------------------------ Q8_0 spine matmul
    if "q8_0" in only:
        q8 = {}
        for (K, N) in synth.Q8_0_SHAPES:
            wq, ws = synth.q8_0_weight(3, K, N)
            dwq = torch.from_numpy(wq).to(dev)
            dws = torch.from_numpy(ws.view(np.int16)).to(dev)
            del wq, ws
            # int8 plane in tile order (q8_0_pack; the same bits as row order)
            twq = torch.empty_like(dwq)
            moe.q8_0_pack(dwq, twq, moe.MOE_LAYOUT_TILES)
            del dwq
            # copies at distinct addresses so the rotation spans >= 1 GB
            ncopy = max(2, -(-(1 << 30) // twq.numel()))
            copies = [(twq, dws)] + [(twq.clone(), dws.clone()) for _ in range(ncopy - 1)]
            torch.cuda.synchronize()  # the copies are made on torch's stream, read on `stream`
            for Mq in (1, 2, 4, 8):
                X = torch.from_numpy(synth.q8_0_x(3, Mq, K)).to(dev)
                Y = torch.empty((Mq, N), dtype=torch.float32, device=dev)

                def q(i):
                    a, b = copies[i % ncopy]
                    moe.q8_0_matmul(X, a, b, Y, stream=stream, layout=moe.MOE_LAYOUT_TILES)

                for i in range(5):
                    q(i)
                ms = timer.region(q, max(40, 2 * ncopy))
                wbytes = N * K * 34 / 32
                gbs = (wbytes + Mq * (K + N) * 4) / (ms / 1e3) / 1e9
                q8[f"K{K}_N{N}_M{Mq}"] = dict(us=ms * 1e3, GBps=gbs, hbm_frac=gbs / HBM_PEAK_GBS)
                log(f"[bench] q8_0 K={K} N={N} M={Mq}: {ms * 1e3:.1f} us, {gbs:.0f} GB/s")
            del twq, dws, copies
        results["q8_0"] = q8

    # ------------------------------------------------------------ block verification over a layer stack
    if "verify" in only:
        results.update(run_verify(torch, moe, synth, shp, layers, stream, dev, timer))

    # ------------------------------------------------------------ host-tier expert streaming
    if "stream" in only:
        results.update(run_stream(torch, moe, synth, shp, layers, stream, dev))

    # ------------------------------------------------------------ CPU baseline: the oracle
    cpu = None
    if not args.no_cpu_baseline:
        cpu = run_cpu_baseline(args, synth, shp, results)

    dec = results.get("decode_1row", {})
    roof = None
    traffic = measured_traffic()
    if dec:
        # the layer pass is the unit of the metric: its algorithmic bytes over
        # its measured time; the dominant kernel's own figure is a sub-field
        per = {}
        for name in ("decode_1row", "block_16rows", "prefill_1533rows"):
            r = results.get(name)
            if r:
                per[name] = {"rows": r["rows"], "us": r["ms_per_layer"] * 1e3, "alg_bytes": r["layer_alg_bytes"],
                             "GBps": r["layer_GBps"], "hbm_frac": r["layer_hbm_frac"]}
                if "mfma_frac" in r:
                    per[name]["mfma_frac"] = r["mfma_frac"]
        roof = {"bound": "hbm", "achieved": dec["layer_GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": dec["layer_hbm_frac"], "traffic": traffic_layer(),
                "scope": "whole 1-row layer pass (router, top-k + bucket, expert FFN, combine): 18 expert records, "
                         "the fp32 router matrix, x in and the output row out, over the layer's measured time",
                "algorithmic_bytes_per_step": dec["layer_alg_bytes"], "target_frac": 0.70,
                "per_workload": per,
                "kernel": {"name": "ffn_gateup_kernel (moe_ffn_gateup_mxfp4, 1 row)", "achieved": dec["gateup_GBps"],
                           "frac": dec["gateup_GBps"] / HBM_PEAK_GBS, "traffic": traffic,
                           "algorithmic_bytes_per_launch": dec["gateup_alg_bytes"], "launch_us": dec["gateup_us"]}}
    line = {
        "metric": "MoE-layer rows/s + effective MXFP4 weight GB/s at 1, 16, 1533 rows",
        "value": dec.get("rows_per_s"),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": dec.get("ms_per_layer"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "kimi_moe_layer_decode_1row", "d": shp.d, "f": shp.f, "routed_experts": shp.n_routed,
                   "shared_experts": shp.n_shared, "top_k": shp.k, "rows": 1,
                   "weights": "mxfp4, codes planes in tile order (moe_pack_experts)",
                   "x": "bf16", "router": "fp32",
                   "arithmetic": "bf16 MFMA operands with fp32 accumulation: FP4 weights decoded exactly to bf16, "
                                 "bf16 x exact, the fp32 hidden h as two bf16 parts (hi + lo, |h - hi - lo| <= "
                                 "2^-18 |h|); router logits and combine in fp32",
                   "timing": f"{N_LAYERS} resident layers in rotation, back-to-back steps between two HIP events"},
        "roofline": roof,
        "effective_weight_GBps": dec.get("effective_weight_GBps"),
        "cpu_baseline": cpu,
        "context": page_context(results),
        "results": results,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
