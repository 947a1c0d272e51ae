#!/usr/bin/env python3
"""Decode-step benchmark of the NVFP4 sparse-MLA path on one MI355X.

One step = the whole hot path for one batch: quantize-append the step's new
tokens (one per query row) into the paged NVFP4 cache, then the sparse decode
(gather + dequant + QK + online softmax with sink + PV, and the split-KV
combine kernel when the planner splits).  The headline workload is h_q 64 /
batch 32 / top-k 2048.  Reported alongside: the h_q 16 MTP decode (one cache
and the dual-cache layout), the h_q 128 varlen decode, the h_q 64 decode over
432-byte records, a 4096-token sparse prefill at h_q 64, and the 16384-token
quantize-append from bf16 and fp16.  --prefill-sweep times the prefill over
the pages' operator grid instead.

Inputs are resident in HBM before timing starts: each pool is filled with
NVFP4 records by the HIP quantize-append, and the timed loop rotates over R
independent index/query sets on that pool so successive steps do not simply
re-read one step's records out of the 256 MB MALL.  Steps are launched
eagerly (--graph times HIP-graph replays instead; the graphs are always
captured and checked against the eager results); HIP events bracket every
decode on the stream it runs on.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
FLOP_PER_TOKEN_HEAD = 2 * (576 + 512)
HEADLINE = "decode_h64"
METRIC = "sparse decode TFLOP/s + KV GB/s, h_q 16/64/128, topk 2048; % of roofline"
DECODE_SRC = os.path.join(ROOT, "sparse_mla_decode_nvfp4_amd", "csrc", "decode.hip")
FLUSH_BYTES = 1 << 30          # scratch written before each cold-timed decode
COLD_LAUNCHES = 50


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--sets", type=int, default=8, help="index/query sets rotated over one pool")
    p.add_argument("--workload", default=HEADLINE)
    p.add_argument("--no-extra", action="store_true", help="skip the other workloads")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--graph", action="store_true",
                   help="time HIP-graph replays instead of eager launches (graphs are always "
                        "captured and checked against the eager results)")
    p.add_argument("--only", default=None, help="run just this workload (profiling)")
    p.add_argument("--splits", type=int, default=0, help="override the planner's split count")
    p.add_argument("--prefill-sweep", action="store_true",
                   help="time the sparse prefill over the pages' operator grid (heads per rank "
                        "x query tokens) and print one JSON line with the table")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="run only a plain 1 GiB device copy (HBM counter calibration)")
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_hash():
    h = hashlib.sha256()
    for name in sorted(os.listdir(os.path.dirname(DECODE_SRC))):
        with open(os.path.join(os.path.dirname(DECODE_SRC), name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per decode launch from the committed rocprofv3 counter
    summary, or None when it is missing or was taken on other kernel code."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != source_hash():
        return None
    return t.get("bytes_per_launch")


# --------------------------------------------------------------------------- decode
def index_lists(s):
    """(index array, slot count of its cache) of each list of a decode step:
    one for the plain decode, primary and extra for the dual-cache decode."""
    if hasattr(s, "extra_indices"):
        return [(s.indices, s.primary.num_slots), (s.extra_indices, s.extra_pool.num_slots)]
    return [(s.indices, s.num_slots)]


def decode_accounting(sets, wl):
    """Algorithmic flops and bytes per step (averaged over the sets)."""
    fl, kv, uniq = [], [], []
    for s in sets:
        nv = nu = 0
        for idx, n_slots in index_lists(s):
            valid = (idx >= 0) & (idx < n_slots)
            nv += int(valid.sum())
            nu += len(np.unique(idx[valid]))
        rb = getattr(wl, "record_bytes", 352)
        fl.append(nv * FLOP_PER_TOKEN_HEAD * wl.h_q)
        kv.append(nv * rb)
        uniq.append(nu * rb)
    rows = wl.batch * wl.s_q
    other = (rows * wl.h_q * 576 * 2 + rows * wl.h_q * 512 * 2 + rows * wl.h_q * 4
             + rows * wl.topk * 4 + wl.h_q * 4)
    return dict(flops=float(np.mean(fl)), kv_bytes=float(np.mean(kv)),
                unique_bytes=float(np.mean(uniq)) + other, other_bytes=other)


def fill_pool(lib, W, config_id, num_blocks, block_size, seed, dev, record_bytes=352):
    """A paged cache with every slot holding a record quantized (by the HIP
    append) from seeded random latents of the workload's distribution."""
    import torch
    cache = lib.new_cache(num_blocks, block_size, dev, record_bytes=record_bytes)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    chunk = 1 << 20
    num_slots = num_blocks * block_size
    for start in range(0, num_slots, chunk):
        n = min(chunk, num_slots - start)
        lat, rope = W.latents_torch(config_id, n, gen, dev)
        sm = torch.arange(start, start + n, dtype=torch.int64, device=dev)
        lib.quantize_append(lat, rope, sm, cache)
        del lat, rope, sm
    torch.cuda.synchronize()
    return cache


def decode_kernel_name(h_q):
    """The decode kernel the library picks for h_q heads (32- or 16-head
    workgroups)."""
    return "decode_w32_kernel" if h_q % 32 == 0 else "decode_tile16_kernel"


def bench_decode(lib, W, name, steps, warmup, nsets, time_graph, dev, force_splits=0):
    import torch
    t_gen = time.time()
    dual = W.dual_workload(name) is not None
    gen = W.dual_workload(name) if dual else W.DECODE_WORKLOADS[name]
    sets = [gen(rep=r, with_latents=False) for r in range(nsets)]
    wl = sets[0]
    pools = [wl.primary, wl.extra_pool] if dual else [wl]
    log(f"{name}: {nsets} sets generated in {time.time() - t_gen:.1f}s; pools "
        + ", ".join(f"{p.num_slots} slots in {p.block_size}-token pages = "
                    f"{p.num_slots * getattr(wl, 'record_bytes', 352) / 1e9:.2f} GB" for p in pools))
    rb = getattr(wl, "record_bytes", 352)
    caches = [fill_pool(lib, W, wl.config_id, p.num_blocks, p.block_size,
                        1000 * (i + 1) + wl.config_id, dev, rb) for i, p in enumerate(pools)]
    cache = caches[0]
    rows = wl.batch * wl.s_q
    splits = force_splits or lib.plan(wl.batch, wl.s_q, wl.h_q, wl.topk)
    ws_bytes = lib.workspace_size(wl.batch, wl.s_q, wl.h_q, wl.topk, splits)
    ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    out = torch.empty((wl.batch, wl.s_q, wl.h_q, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((wl.batch, wl.s_q, wl.h_q), dtype=torch.float32, device=dev)
    sink = torch.from_numpy(wl.sink).to(dev) if wl.sink is not None else None
    new_slots = torch.from_numpy(wl.new_slots).to(dev)
    inp = []
    for r, s in enumerate(sets):
        nl, nr = W.latents(wl.config_id, rows, rep=100 + r)
        inp.append(dict(q=s.q.to(dev), idx=torch.from_numpy(s.indices).to(dev),
                        lat=nl.to(dev), rope=nr.to(dev)))
        if dual:
            inp[-1]["idx1"] = torch.from_numpy(s.extra_indices).to(dev)

    def append(r):
        lib.quantize_append(inp[r]["lat"], inp[r]["rope"], new_slots, cache)

    def decode(r):
        if dual:
            lib.sparse_decode_dual(inp[r]["q"], caches[0], inp[r]["idx"], caches[1],
                                   inp[r]["idx1"], wl.softmax_scale, sink=sink,
                                   num_splits=splits, workspace=ws, out=out, lse=lse)
        else:
            lib.sparse_decode(inp[r]["q"], cache, inp[r]["idx"], wl.softmax_scale, sink=sink,
                              num_splits=splits, workspace=ws, out=out, lse=lse)

    # eager reference outputs, then graphs checked against them
    ref = []
    for r in range(nsets):
        append(r)
        decode(r)
        torch.cuda.synchronize()
        ref.append(out.clone())
    # every call is capture-safe: capture each step's append and decode as HIP
    # graphs and check that replays reproduce the eager results bit for bit
    # one graph per step (append, then decode) for the step time; the append
    # and decode on their own for the decode's event timing
    g_app, g_dec, g_step = [], [], []
    if True:
        for r in range(nsets):
            ga, gd, gs = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
            with torch.cuda.graph(ga):
                append(r)
            with torch.cuda.graph(gd):
                decode(r)
            with torch.cuda.graph(gs):
                append(r)
                decode(r)
            g_app.append(ga)
            g_dec.append(gd)
            g_step.append(gs)
        for rnd in range(2):
            for r in range(nsets):
                g_app[r].replay()
                g_dec[r].replay()
                torch.cuda.synchronize()
                assert torch.equal(out, ref[r]), f"{name}: graph replay {rnd} set {r} differs"
                g_step[r].replay()
                torch.cuda.synchronize()
                assert torch.equal(out, ref[r]), f"{name}: step graph replay {rnd} set {r} differs"
    if time_graph:
        run_app = lambda r: g_app[r].replay()
        run_dec = lambda r: g_dec[r].replay()
        run_step = lambda r: g_step[r].replay()
    else:
        run_app, run_dec = append, decode

        def run_step(r):
            append(r)
            decode(r)

    for k in range(warmup):
        run_step(k % nsets)
    # the step: wall time over `steps` back-to-back steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        run_step(k % nsets)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_ms = (t1 - t0) * 1e3 / steps
    # the decode alone: HIP events on the launching stream around each decode
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for k in range(steps):
        r = k % nsets
        run_app(r)
        ev[k][0].record()
        run_dec(r)
        ev[k][1].record()
    torch.cuda.synchronize()
    dec_ms = np.array([a.elapsed_time(b) for a, b in ev])
    # cold: before each decode a 1 GiB scratch write evicts the 256 MB MALL
    # and the L2s, so the decode's records come from HBM (median of the
    # event-timed decodes).  The write leaves dirty lines that are written
    # back while the decode runs; a second pass evicts with a 1 GiB read
    # (clean lines) instead.
    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.int32, device=dev)
    n_cold = min(steps, COLD_LAUNCHES)

    def timed_after(evict):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n_cold)]
        sink_acc = torch.zeros((), dtype=torch.int64, device=dev)
        for k in range(n_cold):
            r = k % nsets
            run_app(r)
            evict(k, sink_acc)
            evs[k][0].record()
            run_dec(r)
            evs[k][1].record()
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in evs])

    cold_ms = timed_after(lambda k, acc: flush.fill_(k + 1))
    cold_read_ms = timed_after(lambda k, acc: acc.add_(flush.sum()))
    del flush
    acc = decode_accounting(sets, wl)
    dec_avg = float(dec_ms.mean())
    res = dict(
        workload=name, description=wl.description, rows=rows, h_q=wl.h_q, topk=wl.topk,
        kernel=decode_kernel_name(wl.h_q),
        splits=splits, sets=nsets, ms_per_step=step_ms,
        decode_ms_mean=dec_avg, decode_ms_median=float(np.median(dec_ms)),
        decode_ms_min=float(dec_ms.min()),
        cold_decode_ms_median=float(np.median(cold_ms)), cold_launches=n_cold,
        cold_read_decode_ms_median=float(np.median(cold_read_ms)),
        flops_per_step=acc["flops"], kv_bytes_per_step=acc["kv_bytes"],
        compulsory_bytes_per_step=acc["unique_bytes"],
        step_tflops=acc["flops"] / (step_ms * 1e-3) / 1e12,
        decode_tflops=acc["flops"] / (dec_avg * 1e-3) / 1e12,
        decode_kv_gbps=acc["kv_bytes"] / (dec_avg * 1e-3) / 1e9,
        decode_hbm_gbps=acc["unique_bytes"] / (dec_avg * 1e-3) / 1e9,
    )
    res["mfma_frac"] = res["decode_tflops"] / PEAK_BF16_TFLOPS
    res["hbm_frac"] = res["decode_hbm_gbps"] / PEAK_HBM_GBS
    res["cold_decode_tflops"] = acc["flops"] / (res["cold_decode_ms_median"] * 1e-3) / 1e12
    res["cold_decode_hbm_gbps"] = acc["unique_bytes"] / (res["cold_decode_ms_median"] * 1e-3) / 1e9
    res["cold_mfma_frac"] = res["cold_decode_tflops"] / PEAK_BF16_TFLOPS
    res["cold_hbm_frac"] = res["cold_decode_hbm_gbps"] / PEAK_HBM_GBS
    res["invalid_frac"] = float(np.mean([np.mean(idx < 0) for s in sets
                                         for idx, _ in index_lists(s)]))
    res["block_size"] = ([p.block_size for p in pools] if dual else wl.block_size)
    res["record_bytes"] = getattr(wl, "record_bytes", 352)
    res["batch"], res["s_q"] = wl.batch, wl.s_q
    res["sink"] = wl.sink is not None
    intensity = acc["flops"] / acc["unique_bytes"]
    res["bound"] = "mfma" if intensity > PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9) else "hbm"
    log(f"{name}: step {step_ms * 1e3:.1f} us, decode {dec_avg * 1e3:.1f} us (median "
        f"{res['decode_ms_median'] * 1e3:.1f}), {res['decode_tflops']:.0f} TFLOP/s "
        f"({100 * res['mfma_frac']:.1f}% MFMA), KV {res['decode_kv_gbps']:.0f} GB/s, "
        f"compulsory {res['decode_hbm_gbps']:.0f} GB/s ({100 * res['hbm_frac']:.1f}% HBM), "
        f"splits {splits}; cold median {res['cold_decode_ms_median'] * 1e3:.1f} us after a "
        f"1 GiB write, {res['cold_read_decode_ms_median'] * 1e3:.1f} us after a 1 GiB read")
    del cache, caches, ws, inp, g_app, g_dec
    torch.cuda.empty_cache()
    return res


def bench_append(lib, W, steps, warmup, dev, fp16=False, fused=False):
    """The append_write workload through the bf16 export, with the same
    latents cast to fp16 through the fp16 export, or through the fused
    norm + rotary + quantize export (un-normalised latents, a weight, a
    rotary table and positions)."""
    import torch
    wl = W.append_write()
    name = "append_write_fp16" if fp16 else ("append_write_fused" if fused else "append_write")
    cache = torch.from_numpy(wl.sentinel.reshape(wl.num_blocks, wl.block_size, 352)).to(dev)
    lat, rope = wl.latent.to(dev), wl.rope.to(dev)
    if fp16:
        lat, rope = lat.to(torch.float16), rope.to(torch.float16)
    sm = torch.from_numpy(wl.slot_mapping).to(dev)
    if fused:
        nr = W.norm_rope_inputs(wl.num_tokens)
        w, cs = nr.norm_weight.to(dev), nr.cos_sin.to(dev)
        pos = torch.from_numpy(nr.positions).to(dev)

        def run():
            lib.norm_rope_quantize_append(lat, rope, w, nr.eps, cs, pos, sm, cache)
    else:
        def run():
            lib.quantize_append(lat, rope, sm, cache)
    for _ in range(warmup):
        run()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    for k in range(steps):
        ev[k][0].record()
        run()
        ev[k][1].record()
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    mapped = int((wl.slot_mapping >= 0).sum())
    # compulsory: each mapped token's inputs and record, every slot id (and,
    # fused, its position; the weight and the table rows are cache-resident)
    nbytes = mapped * (512 * 2 + 64 * 2 + 352) + wl.num_tokens * 8 * (2 if fused else 1)
    res = dict(workload=name, tokens=wl.num_tokens, mapped=mapped, ms=ms,
               bytes=nbytes, gbps=nbytes / (ms * 1e-3) / 1e9,
               tokens_per_s=mapped / (ms * 1e-3))
    res["hbm_frac"] = res["gbps"] / PEAK_HBM_GBS
    log(f"{name}: {ms * 1e3:.1f} us, {res['gbps']:.0f} GB/s ({100 * res['hbm_frac']:.1f}% HBM)")
    del cache
    torch.cuda.empty_cache()
    return res


# --------------------------------------------------------------------------- cpu
def cpu_model():
    """The host CPU's model name (as lscpu reports it, from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def numpy_blas():
    """The BLAS numpy was built against (name and version)."""
    try:
        cfg = np.__config__.CONFIG["Build Dependencies"]["blas"]
        return f"{cfg.get('name')} {cfg.get('version')}"
    except (AttributeError, KeyError, TypeError):
        return None


def cpu_baseline(W, name, budget_s=12.0):
    """The oracle (numpy fp64) timed on this host: the step's quantize-append
    of its new tokens plus the decode of a bounded sample of query rows."""
    import torch
    from oracle import attention as OA
    from oracle import codec as OC
    wl = W.DECODE_WORKLOADS[name](rep=0, with_latents=False)
    rows = wl.batch * wl.s_q
    idx = wl.indices.reshape(rows, wl.topk).astype(np.int64)
    q = wl.q.reshape(rows, wl.h_q, 576).to(torch.float64).numpy()
    nl, nr = W.latents(wl.config_id, rows, rep=100)
    nl64, nr64 = nl.to(torch.float64).numpy(), nr.to(torch.float64).numpy()

    def prepare(r):
        ids = idx[r]
        uniq = np.unique(ids[ids >= 0])
        lat, rope = W.latents(wl.config_id, len(uniq), rep=200 + r)
        recs = OC.quantize_records(lat.to(torch.float64).numpy(), rope.to(torch.float64).numpy())
        local = np.where(ids >= 0, np.searchsorted(uniq, np.maximum(ids, 0)), -1)
        return recs, local

    sink = None if wl.sink is None else wl.sink.astype(np.float64)
    t0 = time.perf_counter()
    OC.quantize_records(nl64, nr64)                       # the step's append
    t_app = time.perf_counter() - t0
    # row decodes until the budget is spent, cycling over the workload's rows
    # (each row's cache contents are prepared once, untimed)
    done, t_dec, flops, prepared = 0, 0.0, 0.0, {}
    while t_dec + t_app < budget_s and done < 64 * rows:
        r = done % rows
        if r not in prepared:
            prepared[r] = prepare(r)
        recs, local = prepared[r]
        t0 = time.perf_counter()
        OA.sparse_decode(q[r][None, None], recs, local[None, None], wl.softmax_scale, sink=sink)
        t_dec += time.perf_counter() - t0
        flops += int((local >= 0).sum()) * FLOP_PER_TOKEN_HEAD * wl.h_q
        done += 1
    cores = len(os.sched_getaffinity(0))
    return dict(value=flops / (t_app + t_dec) / 1e12, unit="TFLOP/s", cores=cores, kind="oracle",
                cpu_model=cpu_model(), blas=numpy_blas(),
                sample=f"{done} query-row decodes of {name} (its {rows} rows cycled; float64 numpy) "
                       f"plus the step's {rows}-token quantize-append; {t_app + t_dec:.1f} s",
                seconds=t_app + t_dec)


# --------------------------------------------------------------------------- main
def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (--gpus {args.gpus} "
              "requested): the decode would shard by rows, by heads, or by context with the combine "
              "export merging the slices.", file=sys.stderr)
        sys.exit(2)
    import torch
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        # a plain copy of known size: FETCH_SIZE / WRITE_SIZE of its dispatches
        # give the counters' bytes per real byte moved
        src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": 1 << 30, "dispatches": 3}))
        return
    import sparse_mla_decode_nvfp4_amd as lib
    from sparse_mla_decode_nvfp4_amd import workloads as W
    lib.lib()                      # fails loudly when the HIP library is missing
    use_graph = args.graph

    if args.prefill_sweep:
        table = []
        for h in W.PREFILL_HEADS:
            for t in W.PREFILL_TOKENS:
                r = bench_decode(lib, W, f"prefill_dual_h{h}_t{t}", args.steps, args.warmup, 1,
                                 use_graph, dev)
                table.append({k: r[k] for k in ("workload", "h_q", "rows", "splits", "kernel",
                                                "decode_ms_mean", "decode_tflops", "mfma_frac",
                                                "decode_hbm_gbps")})
        print(json.dumps({"prefill_sweep": table, "steps": args.steps, "warmup": args.warmup}))
        return

    if args.only:
        if args.only in ("append_write", "append_write_fp16", "append_write_fused"):
            res = bench_append(lib, W, args.steps, args.warmup, dev, fp16=args.only.endswith("fp16"),
                               fused=args.only.endswith("fused"))
        else:
            # a prefill's query rows already span its pool: one index set
            nsets = 1 if args.only.startswith("prefill") else args.sets
            res = bench_decode(lib, W, args.only, args.steps, args.warmup, nsets, use_graph, dev,
                               args.splits)
        print(json.dumps(res))
        return

    head = bench_decode(lib, W, args.workload, args.steps, args.warmup, args.sets, use_graph, dev)
    extra = {}
    if not args.no_extra:
        for name in ("decode_h16_mtp", "decode_h16_mtp_dual", "decode_h128_varlen",
                     "decode_h64_ds_mla"):
            if name != args.workload:
                extra[name] = bench_decode(lib, W, name, max(20, args.steps // 2),
                                           max(5, args.warmup // 2), args.sets, use_graph, dev)
        # the prefill's 4096 query rows already span the pool: one index set
        extra["prefill_dual_h64_t4096"] = bench_decode(lib, W, "prefill_dual_h64_t4096",
                                                       max(20, args.steps // 4),
                                                       max(5, args.warmup // 4), 1, use_graph, dev)
        extra["append_write"] = bench_append(lib, W, max(20, args.steps // 2),
                                             max(5, args.warmup // 2), dev)
        extra["append_write_fp16"] = bench_append(lib, W, max(20, args.steps // 2),
                                                  max(5, args.warmup // 2), dev, fp16=True)
        extra["append_write_fused"] = bench_append(lib, W, max(20, args.steps // 2),
                                                   max(5, args.warmup // 2), dev, fused=True)
    cpu = None if args.no_cpu else cpu_baseline(W, args.workload)

    bound = head["bound"]
    if bound == "mfma":
        achieved, peak, unit = head["decode_tflops"], PEAK_BF16_TFLOPS, "TFLOP/s"
    else:
        achieved, peak, unit = head["decode_hbm_gbps"], PEAK_HBM_GBS, "GB/s"
    line = {
        "metric": METRIC,
        "value": head["step_tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": head["batch"], "s_q": head["s_q"],
                   "h_q": head["h_q"], "topk": head["topk"], "d_qk": 576, "d_v": 512,
                   "record_bytes": head["record_bytes"], "block_size": head["block_size"],
                   "invalid_frac": round(head["invalid_frac"], 4), "sink": head["sink"],
                   "splits": head["splits"], "index_sets": args.sets,
                   "timed_launches": "graph" if use_graph else "eager"},
        "kv_gbps": head["kv_bytes_per_step"] / (head["ms_per_step"] * 1e-3) / 1e9,
        "roofline": {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
                     "frac": achieved / peak, "traffic": measured_traffic(args.workload),
                     "kernel": head["kernel"] + ("+combine_kernel" if head["splits"] > 1 and
                                                 head["kernel"] != "decode_tile16_kernel" else ""),
                     "kernel_us_mean": head["decode_ms_mean"] * 1e3,
                     "cold_kernel_us_median": head["cold_decode_ms_median"] * 1e3,
                     "cold_read_kernel_us_median": head["cold_read_decode_ms_median"] * 1e3,
                     "cold_frac": (head["cold_mfma_frac"] if bound == "mfma"
                                   else head["cold_hbm_frac"]),
                     "other_resource_frac": head["hbm_frac"] if bound == "mfma" else head["mfma_frac"]},
        "cpu_baseline": cpu,
        "workloads": {args.workload: head, **extra},
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
