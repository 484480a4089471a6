"""Benchmark of the dual-flow decode step on one MI355X.

python bench.py [--steps K] [--warmup W]
                [--workload layer|attn-b16|attn-ragged|attn-long|attn-fp32|step|head|moe|prefill|read-floor]

A step of the default workload is one full dual-flow decode layer (both flows, batch
32, context 8192, hidden 4096, 32/8 heads x 128, SwiGLU 14336, paged bf16 cache of
16-token blocks): RMSNorm, grouped Wqkv, primary K/V append, dual-query attention,
grouped Wo + residual, RMSNorm, grouped gate/up, SwiGLU + b coupling, grouped down +
c coupling + residual. Inputs are seeded synthetic tensors already resident in HBM.
Prints one JSON line; `value` is decode steps/s (one layer step = one generated
position for all 32 sequences of both flows).

Also measured in the same run: the dominant kernel (the dual-query attention call)
timed with HIP events on the stream it runs on, its algorithmic HBM bytes, and the
CPU oracle timed on the host cores (a reported baseline, not a target).

`step` times a whole decode step of a layer stack (token ids -> embeddings -> layers ->
shared output head -> next token), eagerly and as a HIP-graph replay (value: the faster);
`head` the output head alone (final norm, shared vocabulary projection, mixture, greedy
token); `moe` the mixture-of-experts MLP block with router replay; `prefill` one layer of
primary-only prefill over a prompt chunk and its causal attention alone.
"""
import argparse
import hashlib
import itertools
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0   # MI355X published HBM3E bandwidth


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="layer",
                   choices=["layer", "attn-b16", "attn-ragged", "attn-long", "attn-fp32", "step", "head", "moe",
                            "prefill", "read-floor"])
    p.add_argument("--prompt", type=int, default=2048, help="prompt chunk of the 'prefill' workload")
    p.add_argument("--prefill-batch", type=int, default=2, help="sequences of the 'prefill' workload")
    p.add_argument("--layers", type=int, default=8, help="layers of the 'step' workload")
    p.add_argument("--vocab", type=int, default=128256,
                   help="vocabulary of the 'step' and 'head' workloads (0: the step ends at the last layer)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--splits", type=int, default=0, help="attention context splits (0 = plan)")
    p.add_argument("--kernel-reps", type=int, default=20)
    p.add_argument("--no-attention-workloads", action="store_true",
                   help="skip timing the four attention-only workloads in the layer line")
    p.add_argument("--no-split-sweep", action="store_true",
                   help="skip timing dual and single flow at each split count (own-best-split ratio)")
    p.add_argument("--library-gemms", action="store_true",
                   help="'prefill' workload: also time torch's bf16 linear (the ROCm BLAS library) on the "
                        "layer's four projection shapes, for context")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                   help="only run the plain copy kernel on BYTES (5 launches): the reference "
                        "for scaling hardware traffic counters")
    return p.parse_args()


def dev(a):
    import numpy as np
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def attn_bytes(case_like, ctx, F, q_bytes):
    """Algorithmic HBM bytes of one dual-query attention call: every attended K and V
    row once, the query rows (q1, q2), the coupling vector, the outputs and LSE, the
    context lengths and the block-table entries that are read."""
    import numpy as np
    Hkv, D, Hq, B = case_like["Hkv"], case_like["D"], case_like["Hq"], case_like["B"]
    el = case_like["kv_el"]
    tot = int(np.sum(ctx))
    kv = 2 * tot * Hkv * D * el
    q = F * B * Hq * D * q_bytes
    a = D * 4
    out = F * B * Hq * D * 4 + F * B * Hq * 4
    table = int(np.sum(-(-np.asarray(ctx) // case_like["bs"]))) * 4 if case_like["paged"] else 0
    return kv + q + a + out + B * 4 + table


REPLICA_BYTES = 1 << 30


def timed(fn, reps, stream):
    """Average duration (ms) of fn() over reps launches, HIP events on `stream`."""
    import torch
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        fn()
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(reps):
            fn()
        end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / reps


def stream_read(dfx, stream, nbytes=4 << 30, reps=10):
    """Achievable HBM read bandwidth next to the 8 TB/s published figure: the library's read
    helper (contiguous non-temporal 1 KiB loads) over a 4 GiB buffer, HIP events."""
    import torch
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda")
    dfx.fill_bytes(buf, 0x01010101)
    sink = torch.empty(4096 * 256, dtype=torch.int32, device="cuda")
    ms = timed(lambda: dfx.read_bytes(buf, sink), reps, stream)
    del buf
    gbps = nbytes / (ms * 1e-3) / 1e9
    return {"bytes": nbytes, "gbps": round(gbps, 1), "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4)}


def best_split_ratio(dfx, kv, B, Hq, F, mc, q1, q2, a, caches, turn, ctx_t, aws, reps, stream):
    """Dual and single flow, each timed at every split count the planner runs for a range of
    requests and reported at its own best (the plan's ratio is reported beside it)."""
    max_s = max(1, -(-mc // 32))
    cands = sorted({dfx.decode_attn_plan(kv, B, Hq, F, mc, r)[0]
                    for r in (0, 1, 2, 3, 4, 6, 8, 12, 16, 32) if r <= max_s})
    best = {}
    for name, (qq, aa) in (("dual", (q2, a)), ("single", (None, None))):
        def call(n, qq=qq, aa=aa):
            dfx.decode_attn(q1, qq, aa, cache=caches[next(turn)], context_lens=ctx_t, max_context=mc,
                            num_splits=n, want_lse=False, workspace=aws)
        t = {n: timed(lambda n=n: call(n), reps, stream) for n in cands}
        n_best = min(t, key=t.get)
        best[name] = {"splits": n_best, "ms": round(t[n_best], 4)}
    best["ratio"] = round(best["dual"]["ms"] / best["single"]["ms"], 3)
    return best


# The four attention-only workloads (dual-query decode attention alone), with the shapes,
# context lengths and cache layouts of the parity tests; the values are drawn on the GPU
# (timing needs the shapes, not the seeded values).
ATTN_WORKLOADS = {
    1: dict(B=1, Hq=8, Hkv=8, D=64, ctx=("fixed", 512), kv="f32", paged=False, pool=None),
    2: dict(B=16, Hq=32, Hkv=8, D=128, ctx=("fixed", 4096), kv="bf16", paged=False, pool=None),
    3: dict(B=64, Hq=32, Hkv=8, D=128, ctx=("ragged", 303, 1024, 16384), kv="bf16", paged=True, pool=70000),
    4: dict(B=8, Hq=64, Hkv=8, D=128, ctx=("fixed", 131072), kv="bf16", paged=True, pool=65536),
}


def attention_workloads(dfx, gen, stream, reps, which=(1, 2, 3, 4)):
    """Dual-query attention of each attention workload at the planned split count: dual-flow
    and primary-only time (HIP events on the launch stream, back-to-back calls rotating cache
    replicas of >= 1 GB in total), algorithmic bytes, GB/s and the fraction of 8 TB/s."""
    import numpy as np
    import torch
    g = torch.Generator(device="cuda").manual_seed(4242)
    out = []
    for idx in which:
        w = ATTN_WORKLOADS[idx]
        B, Hq, Hkv, D = w["B"], w["Hq"], w["Hkv"], w["D"]
        ctx_np = (np.full(B, w["ctx"][1], np.int32) if w["ctx"][0] == "fixed"
                  else gen.ragged_lengths(w["ctx"][1], B, w["ctx"][2], w["ctx"][3]))
        el = 4 if w["kv"] == "f32" else 2
        kdt = torch.float32 if el == 4 else torch.bfloat16
        if w["paged"]:
            bs = 16
            nblk = w["pool"]
            mb = -(-int(ctx_np.max()) // bs)
            perm = torch.randperm(nblk, generator=g, device="cuda").to(torch.int32)
            need = -(-ctx_np // bs)
            table = torch.zeros(B, mb, dtype=torch.int32, device="cuda")
            off = 0
            for b in range(B):
                table[b, : need[b]] = perm[off: off + need[b]]
                off += int(need[b])
            shape = (nblk, Hkv, bs, D)
        else:
            bs, table = int(ctx_np.max()), None
            shape = (B, Hkv, bs, D)
        pool_bytes = 2 * int(np.prod(shape)) * el
        n_rep = -(-REPLICA_BYTES // pool_bytes) if pool_bytes < REPLICA_BYTES else 1
        caches = [dfx.KVCache(torch.randn(*shape, generator=g, device="cuda", dtype=kdt),
                              torch.randn(*shape, generator=g, device="cuda", dtype=kdt), table)
                  for _ in range(n_rep)]
        qdt = kdt
        q1 = torch.randn(B, Hq, D, generator=g, device="cuda", dtype=qdt)
        q2 = torch.randn(B, Hq, D, generator=g, device="cuda", dtype=qdt)
        a = torch.rand(D, generator=g, device="cuda") * 2 - 1
        ctx_t = torch.from_numpy(ctx_np).cuda()
        mc = int(ctx_np.max())
        aws = dfx.Workspace()
        turn = itertools.cycle(range(n_rep))

        def call(qq, aa):
            dfx.decode_attn(q1, qq, aa, cache=caches[next(turn)], context_lens=ctx_t, max_context=mc,
                            want_lse=False, workspace=aws)

        # one pass over the replicas with each flow count first (first touch of every replica),
        # then dual and single flow timed twice each, interleaved; the mean of the two
        for _ in range(min(n_rep, 64)):
            call(q2, a)
            call(None, None)
        # calls of a few microseconds are timed in longer runs (at least ~4 ms each)
        n = reps if pool_bytes * n_rep >= REPLICA_BYTES and pool_bytes >= (1 << 28) else max(reps, 200)
        t = {"dual": [], "single": []}
        for _ in range(2):
            t["dual"].append(timed(lambda: call(q2, a), n, stream))
            t["single"].append(timed(lambda: call(None, None), n, stream))
        dual, single = sum(t["dual"]) / 2, sum(t["single"]) / 2
        case_like = dict(Hkv=Hkv, D=D, Hq=Hq, B=B, kv_el=el, bs=16, paged=w["paged"])
        nbytes = attn_bytes(case_like, ctx_np, 2, el)
        gbps = nbytes / (dual * 1e-3) / 1e9
        splits, _ = dfx.decode_attn_plan(caches[0], B, Hq, 2, mc, 0)
        rec = {"config": idx,
               "workload": (f"batch {B}, {Hq}/{Hkv} heads x {D}, context "
                            + (f"{mc}" if w["ctx"][0] == "fixed" else f"ragged {int(ctx_np.min())}-{mc}")
                            + f", {'paged (16-token blocks)' if w['paged'] else 'contiguous'} {w['kv']} KV"),
               "ms": round(dual, 4), "single_flow_ms": round(single, 4),
               "dual_single_ratio": round(dual / single, 3), "splits": splits, "bytes": int(nbytes),
               "gbps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4), "kv_replicas": n_rep,
               "steps_per_s": round(1000.0 / dual, 1)}
        if idx == 1:
            rec["target"] = "none: 2 MB per call, launch-latency bound"
        else:
            rec["target_0.70"] = "met" if gbps / HBM_PEAK_GBPS >= 0.70 else "missed"
        out.append(rec)
        del caches, q1, q2
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


def timed_each(fn, reps, stream, flush=None):
    """Per-call durations (ms) of reps calls, an event pair around each; flush(), if given,
    runs between the calls outside the event pairs."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    with torch.cuda.stream(stream):
        fn()
        torch.cuda.synchronize()
        for a, b in ev:
            if flush is not None:
                flush()
            a.record(stream)
            fn()
            b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def hbm_flush(dfx, nbytes=512 << 20):
    """A callable that writes nbytes (the library's fill) so that the next call finds none of
    its inputs in the last-level cache."""
    import torch
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda")
    return lambda: dfx.fill_bytes(buf, 0)


# the headers a kernel source includes: a change in any of them is a change of the kernel
KERNEL_HEADERS = {"attn_mfma.hip": ("attn_tiles.h", "common.h")}


def source_sha(name):
    """Hash of a kernel source together with the headers it includes."""
    h = hashlib.sha256()
    for f in (name,) + KERNEL_HEADERS.get(name, ()):
        h.update(open(os.path.join(ROOT, "dual_flow_shared_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel_file, workload):
    """HBM bytes per launch from the committed counter summary, if it was taken on the
    current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(workload)
    except (ValueError, OSError):
        return None
    if not rec or rec.get("source_sha") != source_sha(kernel_file):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return os.cpu_count() or 1


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import dfx_inputs as gen
    import dual_flow_shared_amd as dfx

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    extra = {}
    if args.workload == "step":
        return bench_step(args)
    if args.workload == "head":
        return bench_head(args)
    if args.workload == "moe":
        return bench_moe(args)
    if args.workload == "prefill":
        return bench_prefill(args)
    if args.workload == "read-floor":
        return bench_read_floor(args)
    if args.copy_calibration:
        n = args.copy_calibration - args.copy_calibration % 16
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dfx.copy_bytes(dst, src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 5}))
        return

    if args.workload == "layer":
        c = gen.config_layer()
        B, F, H = c.batch, 2, c.hidden
        kv = dfx.KVCache(dev(c.cache.k_pool), dev(c.cache.v_pool), dev(c.cache.block_table))
        w = dfx.LayerWeights.from_row_major(dev(c.g_attn), dev(c.w_qkv), dev(c.w_o), dev(c.g_mlp), dev(c.w_gate_up),
                             dev(c.w_down), c.num_q_heads, c.num_kv_heads, c.head_dim, c.eps,
                             dev(c.a), dev(c.b), dev(c.c))
        ctx_np = c.cache.context_lens + 1
        ctx = dev(ctx_np)
        max_ctx = int(ctx_np.max())
        x0 = dev(c.x.copy())
        x = x0.clone()
        ws = dfx.Workspace()

        def step():
            dfx.dual_flow_decode_layer(x, w, kv, ctx, max_ctx, workspace=ws)

        # dominant kernel: the attention call of the layer, on the same cache, queries taken
        # from a Wqkv-shaped fp32 buffer (row stride 6144) as inside the layer
        Nqkv = (c.num_q_heads + 2 * c.num_kv_heads) * c.head_dim
        qkv = torch.randn(F, B, Nqkv, device="cuda", dtype=torch.float32)
        q1 = qkv[0, :, : c.num_q_heads * c.head_dim].view(B, c.num_q_heads, c.head_dim)
        q2 = qkv[1, :, : c.num_q_heads * c.head_dim].view(B, c.num_q_heads, c.head_dim)
        a = dev(c.a)
        aws = dfx.Workspace()
        shape = dict(Hkv=c.num_kv_heads, D=c.head_dim, Hq=c.num_q_heads, B=B, kv_el=2, bs=16, paged=True)
        weights_bytes = 2 * (c.w_qkv.size + c.w_o.size + c.w_gate_up.size + c.w_down.size)
        step_bytes = (weights_bytes + attn_bytes(shape, ctx_np, F, 4)
                      + 2 * B * c.num_kv_heads * c.head_dim * 2      # appended K/V rows
                      + 2 * F * B * H * 4                            # residual rows in and out
                      + 4 * (2 * H + c.head_dim + c.intermediate + H))  # gains, a, b, c
        workload = (f"dual-flow decode layer: batch {B} x context {max_ctx}, hidden {H}, "
                    f"{c.num_q_heads}/{c.num_kv_heads} heads x {c.head_dim}, SwiGLU {c.intermediate}, "
                    f"paged bf16 KV (16-token blocks), both flows")
        cfg = {"workload": workload, "batch": B, "context": max_ctx, "hidden": H,
               "q_heads": c.num_q_heads, "kv_heads": c.num_kv_heads, "head_dim": c.head_dim,
               "intermediate": c.intermediate, "flows": F, "kv_block": 16}
        attn_ctx = (ctx, max_ctx)
        caches, turn = [kv], itertools.cycle([0])
    else:
        idx = {"attn-fp32": 1, "attn-b16": 2, "attn-ragged": 3, "attn-long": 4}[args.workload]
        case = gen.config_attention(idx)
        B, F = case.batch, 2
        kv = dfx.KVCache(dev(case.k_pool), dev(case.v_pool),
                         None if case.block_table is None else dev(case.block_table))
        ctx_np = case.context_lens
        ctx = dev(ctx_np)
        max_ctx = int(ctx_np.max())
        q1, q2, a = dev(case.q1), dev(case.q2), dev(case.a)
        aws = dfx.Workspace()
        el = 4 if case.dtype == "f32" else 2
        shape = dict(Hkv=case.num_kv_heads, D=case.head_dim, Hq=case.num_q_heads, B=B, kv_el=el,
                     bs=case.block_size, paged=case.paged)
        step_bytes = attn_bytes(shape, ctx_np, F, el)

        # Back-to-back calls on a cache smaller than the 256 MB last-level cache (or not much
        # larger) would be partly served from it: rotate replicas of the pools totalling at
        # least 1 GB, so every timed call reads its K/V from HBM.
        kv_bytes = case.k_pool.nbytes + case.v_pool.nbytes
        n_rep = -(-REPLICA_BYTES // kv_bytes) if kv_bytes < REPLICA_BYTES else 1
        caches = [kv] + [dfx.KVCache(kv.k.clone(), kv.v.clone(), kv.block_table) for _ in range(n_rep - 1)]
        extra["kv_replicas"] = n_rep
        turn = itertools.cycle(range(n_rep))

        def step():
            dfx.decode_attn(q1, q2, a, cache=caches[next(turn)], context_lens=ctx, max_context=max_ctx,
                            num_splits=args.splits, workspace=aws)

        workload = (f"dual-query decode attention: batch {B}, {case.num_q_heads}/{case.num_kv_heads} heads x "
                    f"{case.head_dim}, context {'ragged' if idx == 3 else max_ctx}, "
                    f"{'paged' if case.paged else 'contiguous'} {case.dtype} KV")
        cfg = {"workload": workload, "batch": B, "context_max": max_ctx, "context_sum": int(ctx_np.sum()),
               "q_heads": case.num_q_heads, "kv_heads": case.num_kv_heads, "head_dim": case.head_dim,
               "flows": F, "dtype": case.dtype}
        attn_ctx = (ctx, max_ctx)

    # ---- timed steps
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(end) / args.steps
    steps_per_s = 1000.0 / ms

    if args.workload == "layer":
        # the same step with the primary flow alone (the auxiliary flow's cost), and each step
        # timed alone with 512 MB written between steps (outside the event pairs)
        x1 = x0[:1].clone()
        single_step_ms = timed(lambda: dfx.dual_flow_decode_layer(x1, w, kv, ctx, max_ctx, workspace=ws),
                               args.steps, stream)
        each_step = np.array(timed_each(step, args.steps, stream, flush=hbm_flush(dfx)))
        extra.update({"layer_single_flow_ms": round(single_step_ms, 4),
                      "layer_dual_single_ratio": round(ms / single_step_ms, 3),
                      "ms_per_step_flushed": {"median": round(float(np.median(each_step)), 4),
                                              "p10": round(float(np.percentile(each_step, 10)), 4),
                                              "p90": round(float(np.percentile(each_step, 90)), 4),
                                              "steps": int(each_step.size), "flush_bytes_between": 512 << 20}})

    # ---- dominant kernel: dual-query attention, events on its stream
    ctx_t, mc = attn_ctx

    def attn_call(q2_=q2, a_=a):
        dfx.decode_attn(q1, q2_, a_, cache=caches[next(turn)], context_lens=ctx_t, max_context=mc,
                        num_splits=args.splits, want_lse=False, workspace=aws)

    attn_ms = timed(attn_call, args.kernel_reps, stream)
    single_ms = timed(lambda: attn_call(None, None), args.kernel_reps, stream)
    # per call, with 512 MB written between the calls (outside the event pairs)
    each = np.array(timed_each(attn_call, args.kernel_reps, stream, flush=hbm_flush(dfx)))
    extra["attn_ms_each"] = {"median": round(float(np.median(each)), 4), "p10": round(float(np.percentile(each, 10)), 4),
                             "p90": round(float(np.percentile(each, 90)), 4), "calls": int(each.size),
                             "flush_bytes_between": 512 << 20}
    if not args.no_split_sweep:
        extra["attn_best_split"] = best_split_ratio(dfx, kv, B, shape["Hq"], F, mc, q1, q2, a, caches, turn, ctx_t,
                                                    aws, args.kernel_reps, stream)
    abytes = attn_bytes(shape, ctx_np, F, 4 if args.workload == "layer" else shape["kv_el"])
    achieved = abytes / (attn_ms * 1e-3) / 1e9
    splits, _ = dfx.decode_attn_plan(kv, B, shape["Hq"], F, mc, args.splits)
    extra.update({"attn_ms": round(attn_ms, 4), "attn_single_flow_ms": round(single_ms, 4),
                  "dual_single_ratio": round(attn_ms / single_ms, 3), "attn_splits": splits,
                  "step_gbps": round(step_bytes / (ms * 1e-3) / 1e9, 1),
                  "step_bytes": int(step_bytes), "wall_s": round(wall, 3)})

    extra["stream_read"] = stream_read(dfx, stream)
    if args.workload == "layer" and not args.no_attention_workloads:
        extra["attention_workloads"] = attention_workloads(dfx, gen, stream, args.kernel_reps)
    # the layer's attention takes fp32 queries (three bf16 terms); the attention workloads bf16
    kname = "attn_mfma_f32q_kernel" if args.workload == "layer" else "attn_mfma_kernel"
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": traffic_from_profiles("attn_mfma.hip", args.workload),
                "kernel": (kname if splits == 1 else f"{kname} + attn_merge_kernel ({splits} splits)")
                if shape["kv_el"] == 2 else "attn_valu_kernel",
                "bytes_per_launch": int(abytes)}

    # ---- CPU oracle on the host cores (reported baseline only)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.workload, locals())

    line = {"metric": "dual-flow decode attn HBM GB/s (% of peak) and decode steps/s at batch x ctx",
            "value": round(steps_per_s, 2), "unit": "steps/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": cfg, "roofline": roofline, "cpu_baseline": cpu, **extra}
    print(json.dumps(line))


def bench_read_floor(args):
    """The floor a streaming kernel of the step can reach: the library's read helper (contiguous
    non-temporal 1 KiB loads) over the byte counts of the step's kernels, each call alone after
    512 MB were written (per-call events, median of 9) and back to back; and the per-launch time
    of a kernel that writes 16 bytes, back to back."""
    import numpy as np
    import torch

    import dual_flow_shared_amd as dfx
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    sink = torch.empty(4096 * 256, dtype=torch.int32, device="cuda")
    flush = hbm_flush(dfx)
    sizes = {"1 MB": 1e6, "8 MB": 8e6, "W_o 33.5 MB": 33554432, "W_qkv 50.3 MB": 50331648,
             "W_down 117.4 MB": 117440512, "W_gate_up 234.9 MB": 234881024, "layer KV 1076 MB": 1075838976}
    out = {}
    for name, nb in sizes.items():
        n = int(nb) // 16384 * 16384
        buf = torch.empty(n // 4, dtype=torch.int32, device="cuda")
        dfx.fill_bytes(buf, 0x01010101)
        call = lambda: dfx.read_bytes(buf, sink)
        each = np.array(timed_each(call, 9, stream, flush=flush))
        b2b = timed(call, 20, stream)
        out[name] = {"bytes": n, "flushed_us": round(float(np.median(each)) * 1e3, 2),
                     "flushed_gbps": round(n / (float(np.median(each)) * 1e-3) / 1e9, 1),
                     "back_to_back_us": round(b2b * 1e3, 2)}
        del buf
    tiny = torch.empty(4, dtype=torch.int32, device="cuda")
    out["16-byte fill, back to back (us per launch)"] = round(timed(lambda: dfx.fill_bytes(tiny, 0), 200, stream) * 1e3, 2)
    print(json.dumps({"metric": "read helper time at the step's byte counts", "unit": "us", "n_gpus": 1,
                      "results": out}))


def bench_step(args):
    """A decode step of a stack of args.layers dual-flow layers of the one-layer workload's shape
    (batch 32, context 8192, hidden 4096, 32/8 heads x 128, SwiGLU 14336, paged bf16 caches),
    from token ids through both flows' embeddings: eager launches and one HIP-graph replay per
    step. Weights, caches and embeddings are drawn on the GPU (synthetic: the timing needs
    shapes, not values; parity is the GPU tests' job)."""
    import torch

    import dual_flow_shared_amd as dfx
    torch.cuda.set_device(0)
    gen_ = torch.Generator(device="cuda").manual_seed(2024)
    B, H, Hq, Hkv, D, I, ctx_len, bs = 32, 4096, 32, 8, 128, 14336, 8192, 16
    vocab = args.vocab if args.vocab > 0 else 32000
    with_head = args.vocab > 0
    nl = args.layers

    def randn(*shape, std=1.0):
        return (torch.randn(*shape, generator=gen_, device="cuda") * std).to(torch.bfloat16)

    def gains(n):
        return torch.rand(n, generator=gen_, device="cuda") * 0.2 + 0.9

    def unif(n):
        return torch.rand(n, generator=gen_, device="cuda") * 2 - 1

    layers, caches = [], []
    nblk = B * ctx_len // bs
    rm0 = None  # layer 0's row-major matrices and vectors (the CPU baseline's sample)
    for l in range(nl):
        rm = dict(g_attn=gains(H), w_qkv=randn((Hq + 2 * Hkv) * D, H, std=0.02), w_o=randn(H, Hq * D, std=0.02),
                  g_mlp=gains(H), w_gate_up=randn(2 * I, H, std=0.02), w_down=randn(H, I, std=0.02),
                  a=unif(D), b=unif(I), c=unif(H))
        w = dfx.LayerWeights.from_row_major(rm["g_attn"], rm["w_qkv"], rm["w_o"], rm["g_mlp"], rm["w_gate_up"],
                                            rm["w_down"], Hq, Hkv, D, 1e-5, rm["a"], rm["b"], rm["c"])
        rm0 = rm if l == 0 else rm0
        table = torch.randperm(nblk, generator=gen_, device="cuda").to(torch.int32).view(B, ctx_len // bs)
        caches.append(dfx.KVCache(randn(nblk, Hkv, bs, D), randn(nblk, Hkv, bs, D), table))
        layers.append(w)
        torch.cuda.synchronize()
    e1, e2 = randn(vocab, H), randn(vocab, H)
    tokens = torch.randint(0, vocab, (B,), generator=gen_, device="cuda", dtype=torch.int32)
    ctx = torch.full((B,), ctx_len, dtype=torch.int32, device="cuda")
    out = torch.empty(2, B, H, dtype=torch.float32, device="cuda")
    ws = dfx.Workspace()
    ws.get(dfx.step_workspace_size(layers, caches, B, 2, ctx_len))
    hws = dfx.Workspace()
    if with_head:
        w_out_rm = randn(vocab, H, std=0.02)
        w_out = dfx.pack_weight(w_out_rm)
        g_out = gains(H)
        hws.get(dfx.output_head_workspace_size(2, B, H, vocab))

    def step():
        dfx.dual_flow_decode_step(tokens, e1, e2, layers, caches, ctx, ctx_len, out=out, workspace=ws)
        if with_head:
            # greedy next token of the mixture, fed back as the next step's input
            nxt, _, _ = dfx.output_head(out, g_out, 1e-5, w_out, workspace=hws)
            tokens.copy_(nxt)

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    eager_ms = timed(step, args.steps, stream)
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        step()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    graph_ms = timed(graph.replay, args.steps, stream)
    cpu = None
    if not args.no_cpu_baseline:
        import numpy as np
        from oracle.head import output_head
        from oracle.layer import dual_flow_layer
        wts = {k: (v.cpu().numpy() if v.dtype == torch.float32 else host_bits(v)) for k, v in rm0.items()}
        kpool, vpool, tbl = host_bits(caches[0].k), host_bits(caches[0].v), caches[0].block_table.cpu().numpy()
        xs = np.random.default_rng(0).standard_normal((2, B, H)).astype(np.float32)
        before = np.full(B, ctx_len - 1)
        sec_l, n_l, tot_l = oracle_seconds(lambda: dual_flow_layer(
            xs, wts["g_attn"], wts["g_mlp"], wts["w_qkv"], wts["w_o"], wts["w_gate_up"], wts["w_down"], wts["a"],
            wts["b"], wts["c"], 1e-5, kpool, vpool, tbl, before, Hq, Hkv, D), budget=1.0)
        sec_h, n_h = 0.0, 0
        if with_head:
            wo, go = host_bits(w_out_rm), g_out.cpu().numpy()
            sec_h, n_h, _ = oracle_seconds(lambda: output_head(xs, go, 1e-5, wo), budget=1.0)
        cpu = baseline_line(1.0 / (nl * sec_l + sec_h), "steps/s",
                            f"layer 0 of the {nl} identical-shape layers timed whole ({n_l} run(s), {sec_l:.1f} s) and "
                            f"counted {nl} times" + (f", plus the output head ({n_h} run(s), {sec_h:.1f} s)"
                                                    if with_head else ""))
    w_bytes = 2 * (Hq + 2 * Hkv) * D * H + 2 * H * Hq * D + 2 * 2 * I * H + 2 * H * I
    kv_bytes = 2 * B * ctx_len * Hkv * D * 2
    step_bytes = nl * (w_bytes + kv_bytes) + 2 * B * H * 2 + (2 * vocab * H if with_head else 0)
    # value: the faster of the two ways of launching the same step (both are timed and reported)
    ms = min(eager_ms, graph_ms)
    mode = "eager launches" if eager_ms <= graph_ms else "HIP-graph replay"
    line = {"metric": "dual-flow multi-layer decode steps/s at batch x ctx", "value": round(1000.0 / ms, 2),
            "unit": "steps/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": f"dual-flow decode step: {nl} layers, batch {B} x context {ctx_len}, hidden {H}, "
                                   f"{Hq}/{Hkv} heads x {D}, SwiGLU {I}, vocab {vocab}, both flows"
                                   + (", shared output head + mixture + greedy token" if with_head else "")
                                   + f", {mode}",
                       "layers": nl, "batch": B, "context": ctx_len, "hidden": H, "flows": 2,
                       "vocab": vocab, "output_head": with_head},
            "roofline": {"bound": "hbm", "achieved": round(step_bytes / (ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                         "traffic": None,
                         "kernel": "whole step (weights + KV of every layer, and the output matrix, read once)",
                         "bytes_per_launch": int(step_bytes)},
            "cpu_baseline": cpu, "eager_ms_per_step": round(eager_ms, 4), "graph_ms_per_step": round(graph_ms, 4),
            "tokens_per_s": round(B * 1000.0 / ms, 1), "ms_per_layer": round(ms / nl, 4)}
    print(json.dumps(line))


def bench_head(args):
    """The shared output head alone: final norm, one pass over a [vocab][4096] bf16 matrix for
    both flows' rows at batch 32, the mixture and the greedy token (synthetic GPU-drawn inputs:
    W_out ~ N(0, 0.02), rows ~ N(0, 1)). The timed launches read the whole matrix each time; at
    1 GiB it is four times the last-level cache, so no launch finds it cached."""
    import torch

    import dual_flow_shared_amd as dfx
    torch.cuda.set_device(0)
    g = torch.Generator(device="cuda").manual_seed(77)
    B, F, H, V = 32, 2, 4096, args.vocab
    x = torch.randn(F, B, H, generator=g, device="cuda")
    gain = torch.rand(H, generator=g, device="cuda") * 0.2 + 0.9
    w_rm = (torch.randn(V, H, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    w = dfx.pack_weight(w_rm)
    ws = dfx.Workspace()
    ws.get(dfx.output_head_workspace_size(F, B, H, V))
    stream = torch.cuda.current_stream()

    def call():
        dfx.output_head(x, gain, 1e-5, w, workspace=ws)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    ms = timed(call, args.steps, stream)
    alg = 2 * V * H + F * B * H * 4 + 4 * H + B * 8     # W_out, rows, gain, token + alpha
    gbps = alg / (ms * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        from oracle.head import output_head
        xs, gs, wb = x.cpu().numpy(), gain.cpu().numpy(), host_bits(w_rm)
        sec, n, tot = oracle_seconds(lambda: output_head(xs, gs, 1e-5, wb))
        cpu = baseline_line(B / sec, "tokens/s", f"the whole head call (batch {B}, both flows, vocab {V}), "
                                                 f"median of {n} runs, {tot:.1f} s in total")
    line = {"metric": "dual-flow output head (shared vocab projection + mixture) tokens/s", "value": round(B * 1000.0 / ms, 1),
            "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": f"shared output head: batch {B}, both flows, hidden {H}, vocab {V}, "
                                   "final RMSNorm + projection + softmax mixture + greedy token",
                       "batch": B, "hidden": H, "vocab": V, "flows": F},
            "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                         "kernel": "whole head call (4 launches; 5 when the projection splits K); algorithmic bytes = W_out + rows + gain + outputs",
                         "bytes_per_launch": int(alg)},
            "cpu_baseline": cpu}
    print(json.dumps(line))


def bench_moe(args):
    """The mixture-of-experts MLP block with router replay: batch 32, both flows, hidden 4096,
    8 experts of intermediate 14336 (a SwiGLU expert of the one-layer workload's MLP shape),
    primary fan-out 2, auxiliary fan-out 2 (and 4 as a second reading: more decode experts at
    the same prefill cost), synthetic GPU-drawn weights. Algorithmic bytes: the router, the
    matrices of every expert some row uses (each read once), the residual rows in and out."""
    import torch

    import dual_flow_shared_amd as dfx
    torch.cuda.set_device(0)
    g = torch.Generator(device="cuda").manual_seed(91)
    B, H, E, I = 32, 4096, 8, 14336

    def randn(*shape, std=0.02):
        return (torch.randn(*shape, generator=g, device="cuda") * std).to(torch.bfloat16)

    gain = torch.rand(H, generator=g, device="cuda") * 0.2 + 0.9
    wr = randn(E, H)
    gu_rm = [randn(2 * I, H) for _ in range(E)]
    dn_rm = [randn(H, I) for _ in range(E)]
    gu = torch.stack([dfx.pack_weight(t) for t in gu_rm])
    dn = torch.stack([dfx.pack_weight(t) for t in dn_rm])
    bvec = torch.rand(I, generator=g, device="cuda") * 2 - 1
    cvec = torch.rand(H, generator=g, device="cuda") * 2 - 1
    x0 = torch.randn(2, B, H, generator=g, device="cuda")
    stream = torch.cuda.current_stream()
    res = {}
    for F, k2 in ((2, 2), (2, 4), (1, 2)):
        w = dfx.MoeWeights(gain, wr, gu, dn, 2, k2, 1e-5, bvec, cvec)
        ws = dfx.Workspace()
        x = x0[:F].clone()
        dfx.moe_mlp(x, w, workspace=ws)
        torch.cuda.synchronize()
        t = dfx.moe_taps(w, B, F)
        counts = ws.buf[t["counts"]: t["counts"] + 4 * E].view(torch.int32).cpu()
        used = int((counts > 0).sum())

        def call():
            x.copy_(x0[:F])
            dfx.moe_mlp(x, w, workspace=ws)

        for _ in range(args.warmup):
            call()
        torch.cuda.synchronize()
        ms = timed(call, args.steps, stream)
        alg = used * 3 * I * H * 2 + E * H * 2 + 2 * F * B * H * 4 + 4 * H
        res[(F, k2)] = (ms, alg, used)
    ms, alg, used = res[(2, 2)]
    gbps = alg / (ms * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        from oracle.moe import moe_mlp
        import numpy as np
        args_np = (x0.cpu().numpy(), gain.cpu().numpy(), 1e-5, host_bits(wr),
                   np.stack([host_bits(t) for t in gu_rm]), np.stack([host_bits(t) for t in dn_rm]), 2, 2,
                   bvec.cpu().numpy(), cvec.cpu().numpy())
        sec, n, tot = oracle_seconds(lambda: moe_mlp(*args_np))
        cpu = baseline_line(B / sec, "tokens/s", f"the whole block (batch {B}, both flows, fan-outs 2 / 2), "
                                                 f"median of {n} runs, {tot:.1f} s in total")
    line = {"metric": "dual-flow MoE block (router replay) tokens/s", "value": round(B * 1000.0 / ms, 1),
            "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": f"MoE MLP block with router replay: batch {B}, both flows, hidden {H}, {E} experts "
                                   f"x SwiGLU {I}, fan-out primary 2 / auxiliary 2",
                       "batch": B, "hidden": H, "experts": E, "intermediate": I, "top_k_primary": 2, "top_k_aux": 2},
            "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                         "kernel": "whole block call (7 launches, timed with the residual reset copy); algorithmic "
                                   "bytes = router + used experts' matrices once + rows",
                         "bytes_per_launch": int(alg), "experts_used": used},
            "cpu_baseline": cpu,
            "aux_fanout_4": {"ms": round(res[(2, 4)][0], 4), "experts_used": res[(2, 4)][2]},
            "primary_only": {"ms": round(res[(1, 2)][0], 4), "experts_used": res[(1, 2)][2]},
            "dual_over_single": round(ms / res[(1, 2)][0], 3)}
    print(json.dumps(line))


def bench_prefill(args):
    """Primary-only prefill of a prompt chunk through one layer of the one-layer workload's shape
    (hidden 4096, 32/8 heads x 128, SwiGLU 14336, paged bf16 cache of 16-token blocks), and its
    causal attention alone; synthetic GPU-drawn weights and queries. Algorithmic flops: 2 per
    weight per row for the projections, 4 * head_dim per (query head, query, attended key) for
    attention (the hi/lo split the kernel uses for accuracy is not counted)."""
    import torch

    import dual_flow_shared_amd as dfx
    torch.cuda.set_device(0)
    gen_ = torch.Generator(device="cuda").manual_seed(55)
    B, T, H, Hq, Hkv, D, I, bs = args.prefill_batch, args.prompt, 4096, 32, 8, 128, 14336, 16

    def randn(*shape, std=0.02):
        return (torch.randn(*shape, generator=gen_, device="cuda") * std).to(torch.bfloat16)

    gains = lambda n: torch.rand(n, generator=gen_, device="cuda") * 0.2 + 0.9
    rm = dict(g_attn=gains(H), w_qkv=randn((Hq + 2 * Hkv) * D, H), w_o=randn(H, Hq * D), g_mlp=gains(H),
              w_gate_up=randn(2 * I, H), w_down=randn(H, I))
    w = dfx.LayerWeights.from_row_major(rm["g_attn"], rm["w_qkv"], rm["w_o"], rm["g_mlp"], rm["w_gate_up"],
                                        rm["w_down"], Hq, Hkv, D, 1e-5)
    nblk = B * (T // bs + 1)
    table = torch.randperm(nblk, generator=gen_, device="cuda").to(torch.int32).view(B, -1)
    cache = dfx.KVCache(randn(nblk, Hkv, bs, D, std=1.0), randn(nblk, Hkv, bs, D, std=1.0), table)
    cap = table.shape[1] * bs
    start = torch.zeros(B, dtype=torch.int32, device="cuda")
    x0 = torch.randn(B, T, H, generator=gen_, device="cuda")
    x = x0.clone()
    ws = dfx.Workspace()
    stream = torch.cuda.current_stream()

    def layer():
        x.copy_(x0)
        dfx.prefill_layer(x, w, cache, start, cap, workspace=ws)

    q = torch.randn(B, T, Hq, D, generator=gen_, device="cuda")
    q2 = torch.randn(B, T, Hq, D, generator=gen_, device="cuda")
    av = torch.rand(D, generator=gen_, device="cuda") * 2 - 1
    attn = lambda: dfx.prefill_attn(q, cache, start, cap)
    dual = lambda: dfx.prefill_dual_attn(q, q2, av, cache, start, cap)   # both flows (training-time forward)
    for _ in range(args.warmup):
        layer()
        attn()
        dual()
    torch.cuda.synchronize()
    ms = timed(layer, args.steps, stream)
    attn_ms = timed(attn, args.steps, stream)
    dual_ms = timed(dual, args.steps, stream)
    rows = B * T
    wparams = (Hq + 2 * Hkv) * D * H + H * Hq * D + 2 * I * H + H * I
    attn_flops = 4.0 * D * Hq * B * T * (T + 1) / 2
    flops = 2.0 * rows * wparams + attn_flops
    tf = flops / (ms * 1e-3) / 1e12
    atf = attn_flops / (attn_ms * 1e-3) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        import numpy as np
        from oracle.prefill import prefill_layer
        xs, kpool, vpool, tbl = x0.cpu().numpy(), host_bits(cache.k), host_bits(cache.v), table.cpu().numpy()
        wts = {k: (v.cpu().numpy() if v.dtype == torch.float32 else host_bits(v)) for k, v in rm.items()}
        sec, n, tot = oracle_seconds(lambda: prefill_layer(xs, wts["g_attn"], wts["g_mlp"], wts["w_qkv"], wts["w_o"],
                                                           wts["w_gate_up"], wts["w_down"], 1e-5, kpool, vpool, tbl,
                                                           np.zeros(B, np.int64), Hq, Hkv, D), budget=1.0)
        cpu = baseline_line(rows / sec, "tokens/s", f"the whole layer over the {B} x {T}-token chunk, "
                                                    f"{n} run(s), {tot:.1f} s in total")
    line = {"metric": "dual-flow prefill (primary only) tokens/s, one layer", "value": round(rows * 1000.0 / ms, 1),
            "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": f"primary-only prefill: {B} sequences x {T}-token prompt chunk from position 0, "
                                   f"one layer, hidden {H}, {Hq}/{Hkv} heads x {D}, SwiGLU {I}, paged bf16 cache",
                       "batch": B, "prompt": T, "hidden": H},
            "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": 2500.0, "unit": "TFLOP/s",
                         "frac": round(tf / 2500.0, 4), "traffic": None,
                         "kernel": "whole prefill layer (8 launches); algorithmic flops of projections + causal attention",
                         "flops_per_launch": flops},
            "cpu_baseline": cpu,
            "attention": {"ms": round(attn_ms, 4), "tflops": round(atf, 1), "frac_of_bf16_peak": round(atf / 2500.0, 4)},
            "dual_attention": {"ms": round(dual_ms, 4), "tflops": round(2 * attn_flops / (dual_ms * 1e-3) / 1e12, 1),
                               "dual_over_single": round(dual_ms / attn_ms, 3)}}
    if args.library_gemms:
        # context only: the vendor library's bf16 GEMM (bf16 out, no residual) on the same shapes
        xa, xi = randn(rows, H, std=1.0), randn(rows, I, std=1.0)
        lib = {}
        for name, (a_, w_) in {"qkv": (xa, rm["w_qkv"]), "o": (xa, rm["w_o"]), "gate_up": (xa, rm["w_gate_up"]),
                               "down": (xi, rm["w_down"])}.items():
            f = lambda: torch.nn.functional.linear(a_, w_)
            f()
            torch.cuda.synchronize()
            lib[name] = round(timed(f, args.steps, stream) * 1e3, 1)
        line["library_gemms_us"] = lib
    print(json.dumps(line))


def host_cores():
    """Host cores this process may run on (the CPU share this process is given, not the machine's count)."""
    try:
        return len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        return os.cpu_count() or 1


def parallel_oracle(fn, parts, workers):
    """Runs fn(part) for every part on `workers` threads, each with one BLAS thread (numpy
    releases the GIL in its array kernels); returns the wall seconds of the whole set."""
    from concurrent.futures import ThreadPoolExecutor
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:
        threadpool_limits = None
    t0 = time.perf_counter()
    if threadpool_limits is not None:
        with threadpool_limits(limits=1, user_api="blas"):
            with ThreadPoolExecutor(workers) as ex:
                list(ex.map(fn, parts))
    else:
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(fn, parts))
    return time.perf_counter() - t0


def cpu_baseline(workload, env):
    """Time the oracle as it stands on a bounded sample of the workload and scale to steps/s
    of the full workload. The layer and attention workloads time the oracle's fp32 evaluation
    (the same definition in single precision), spread over the host's cores by sequence; the
    layer also reports the fp64 oracle on the BLAS threads alone."""
    import numpy as np
    from oracle.attention import decode_attention
    from oracle.layer import dual_flow_layer
    cores = host_cores()
    if workload == "layer":
        c = env["c"]
        kv = c.cache
        B = c.batch
        chunks = [list(range(i, B, cores)) for i in range(min(cores, B))]

        def rows(idx, dtype):
            return dual_flow_layer(c.x[:, idx], c.g_attn, c.g_mlp, c.w_qkv, c.w_o, c.w_gate_up, c.w_down, c.a,
                                   c.b, c.c, c.eps, kv.k_pool, kv.v_pool, kv.block_table[idx], kv.context_lens[idx],
                                   c.num_q_heads, c.num_kv_heads, c.head_dim, dtype=dtype)

        times = []
        while len(times) < 12 and sum(times) < 10.0:
            times.append(parallel_oracle(lambda idx: rows(idx, np.float32), chunks, len(chunks)))
        full = float(np.median(times))
        sample = (f"the oracle's fp32 evaluation of the whole layer step (all {B} sequences, both flows), "
                  f"the sequences spread over {len(chunks)} threads, median of {len(times)} runs, "
                  f"{sum(times):.1f} s in total")
        t64 = []
        while len(t64) < 6 and sum(t64) < 8.0:
            t0 = time.perf_counter()
            rows(list(range(B)), np.float64)
            t64.append(time.perf_counter() - t0)
        return {"value": round(1.0 / full, 4), "unit": "steps/s", "cores": len(chunks), "kind": "oracle",
                "sample": sample, "cpu_model": cpu_model(),
                "fp64": {"value": round(1.0 / float(np.median(t64)), 4), "unit": "steps/s",
                         "threads": cpu_threads(), "runs": len(t64),
                         "sample": "the fp64 oracle, the whole layer step in one call on the BLAS threads"}}
    case = env["case"]
    # whole sequences, cycling through the batch, the calls spread over the host cores until
    # about 10 s of oracle work; scaled to the full batch by the share of context tokens done
    ctx = case.context_lens.astype(np.int64)
    dtype = np.float32
    t, tokens, calls = 0.0, 0, 0
    while (t < 10.0 or calls == 0) and calls < 1_000_000:
        part = [(calls + i) % case.batch for i in range(cores)]
        t += parallel_oracle(lambda b: decode_attention(case.q1, case.q2, case.a, case.a_head_stride, case.k_pool,
                                                        case.v_pool, case.block_table, case.context_lens,
                                                        batches=[b], dtype=dtype), part, cores)
        tokens += int(ctx[part].sum())
        calls += len(part)
    full = t * float(ctx.sum()) / max(tokens, 1)
    sample = (f"the oracle's fp32 attention, one sequence per call on {cores} threads, {calls} calls "
              f"({tokens / float(ctx.sum()):.2f} passes over the batch, {t:.1f} s), scaled by the share "
              f"of context tokens")
    return {"value": round(1.0 / full, 4), "unit": "steps/s", "cores": cores, "kind": "oracle",
            "sample": sample, "cpu_model": cpu_model()}


def oracle_seconds(fn, budget=10.0, max_runs=50):
    """Median wall seconds of an oracle call, repeated until about `budget` seconds have
    passed (at least once); also the number of runs and their total."""
    import numpy as np
    times = []
    while not times or (sum(times) < budget and len(times) < max_runs):
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
    return float(np.median(times)), len(times), float(sum(times))


def host_bits(t):
    """A bf16 device tensor's bit patterns as a host uint16 array."""
    import numpy as np
    import torch
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def baseline_line(value, unit, sample):
    return {"value": round(value, 4), "unit": unit, "cores": cpu_threads(), "kind": "oracle", "sample": sample,
            "cpu_model": cpu_model()}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


if __name__ == "__main__":
    main()
