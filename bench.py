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
    p.add_argument("--no-cold", action="store_true",
                   help="skip the cold (flushed) timing passes (profiling runs)")
    p.add_argument("--profile-commands", metavar="OUT_DIR",
                   help="print the rocprofv3 commands whose output --summarize-profiles reads")
    p.add_argument("--summarize-profiles", metavar="OUT_DIR",
                   help="turn the rocprofv3 CSV output under OUT_DIR into the summaries in profiles/")
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


def bench_decode(lib, W, name, steps, warmup, nsets, time_graph, dev, force_splits=0,
                 no_cold=False):
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
    n_cold = 0 if no_cold else min(steps, COLD_LAUNCHES)

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

    cold_ms = timed_after(lambda k, acc: flush.fill_(k + 1)) if n_cold else np.array([np.nan])
    cold_read_ms = timed_after(lambda k, acc: acc.add_(flush.sum())) if n_cold else np.array([np.nan])
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
    # the same launches back to back, replayed from one HIP graph between one
    # event pair: the kernel's throughput when appends queue up, without the
    # host's per-call time between launches
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(steps):
            run()
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    b2b_ms = e0.elapsed_time(e1) / steps
    del graph
    mapped = int((wl.slot_mapping >= 0).sum())
    # compulsory: each mapped token's inputs and record, every slot id (and,
    # fused, its position; the weight and the table rows are cache-resident)
    nbytes = mapped * (512 * 2 + 64 * 2 + 352) + wl.num_tokens * 8 * (2 if fused else 1)
    res = dict(workload=name, tokens=wl.num_tokens, mapped=mapped, ms=ms,
               bytes=nbytes, gbps=nbytes / (ms * 1e-3) / 1e9,
               tokens_per_s=mapped / (ms * 1e-3))
    res["hbm_frac"] = res["gbps"] / PEAK_HBM_GBS
    res["b2b_ms"] = b2b_ms
    res["b2b_gbps"] = nbytes / (b2b_ms * 1e-3) / 1e9
    res["b2b_hbm_frac"] = res["b2b_gbps"] / PEAK_HBM_GBS
    log(f"{name}: {ms * 1e3:.1f} us per launch ({res['gbps']:.0f} GB/s, {100 * res['hbm_frac']:.1f}% HBM); "
        f"back to back {b2b_ms * 1e3:.1f} us ({res['b2b_gbps']:.0f} GB/s, {100 * res['b2b_hbm_frac']:.1f}% HBM)")
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


# --------------------------------------------------------------------------- profiles
# rocprofv3 runs behind the summaries in profiles/: a kernel trace per
# workload, counter passes (each within one pass's per-block counter limits)
# for the decode workloads, and a plain 1 GiB copy that calibrates the HBM
# byte counters.
PROFILE_TRACE = ["decode_h64", "decode_h128_varlen", "decode_h16_mtp", "decode_h16_mtp_dual",
                 "decode_h64_ds_mla", "prefill_dual_h64_t4096", "append_write", "append_write_fp16",
                 "append_write_fused"]
PROFILE_COUNTERS = ["decode_h64", "decode_h128_varlen", "decode_h16_mtp"]
COUNTER_PASSES = {
    "util": "SQ_VALU_MFMA_BUSY_CYCLES SQ_ACTIVE_INST_VALU SQ_LDS_IDX_ACTIVE SQ_BUSY_CU_CYCLES GRBM_GUI_ACTIVE",
    "insts": ("SQ_INSTS_VALU_MFMA_MOPS_F16 SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_MFMA SQ_INSTS_VALU "
              "SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_INSTS_VMEM_RD SQ_WAVES"),
    "mem": "TA_TA_BUSY SQ_ACTIVE_INST_VMEM SQ_WAIT_INST_ANY GRBM_GUI_ACTIVE",
    "fetch": "FETCH_SIZE",
    "write": "WRITE_SIZE",
}
SIMD_NUM = 1024                # MI355X: 256 CUs x 4 SIMDs
CU_NUM = 256


def profile_bench_args(w, trace):
    if w.startswith("append"):
        return f"--only {w} --steps 50 --warmup 5"
    sets = "" if trace else " --sets 2"
    steps = "--steps 100 --warmup 10" if trace else "--steps 6 --warmup 1"
    if w.startswith("prefill"):
        steps = "--steps 20 --warmup 2" if trace else "--steps 2 --warmup 1"
    return f"--only {w} {steps}{sets} --no-cold"


def profile_commands(out):
    """(name, command) of every rocprofv3 run, each run from the repository
    root with TMPDIR=/tmp."""
    cmds = []
    for w in PROFILE_TRACE:
        cmds.append((f"kt_{w}", f"rocprofv3 --kernel-trace --stats --output-format csv -d {out}/kt_{w} "
                                f"-o run -- python3 bench.py {profile_bench_args(w, True)}"))
    for w in PROFILE_COUNTERS:
        for tag, ctrs in COUNTER_PASSES.items():
            cmds.append((f"pmc_{tag}_{w}", f"rocprofv3 --pmc {ctrs} --output-format csv -d "
                                           f"{out}/pmc_{tag}_{w} -o run -- python3 bench.py "
                                           f"{profile_bench_args(w, False)}"))
    for tag in ("fetch", "write"):
        cmds.append((f"pmc_{tag}_copy", f"rocprofv3 --pmc {COUNTER_PASSES[tag]} --output-format csv -d "
                                        f"{out}/pmc_{tag}_copy -o run -- python3 bench.py --calibrate-copy"))
    return cmds


def _csv_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _find(d, suffix):
    for root, _, files in os.walk(d):
        for f in files:
            if f.endswith(suffix):
                return os.path.join(root, f)
    return None


def _short(name):
    return name.split("(")[0].replace("void ", "").strip()


def _per_dispatch(d, library_only=True):
    """{kernel: {counter: [value per dispatch]}} from a counter-collection CSV
    (rows of one dispatch and counter summed over instances); the library's
    kernels only, unless library_only is false (the copy calibration)."""
    import collections
    path = _find(d, "counter_collection.csv")
    acc = collections.defaultdict(float)
    for r in _csv_rows(path):
        if library_only and "nvfp4::" not in r["Kernel_Name"]:
            continue
        acc[(_short(r["Kernel_Name"]), r["Counter_Name"], r["Dispatch_Id"])] += float(r["Counter_Value"])
    out = collections.defaultdict(lambda: collections.defaultdict(list))
    for (k, c, _), v in acc.items():
        out[k][c].append(v)
    return out


def summarize_profiles(out):
    """Writes profiles/<w>_kernel_trace.txt, profiles/<w>_counters.txt and
    profiles/traffic_<w>.json from the runs of profile_commands(out)."""
    cmds = dict(profile_commands(out))
    pdir = os.path.join(ROOT, "profiles")
    os.makedirs(pdir, exist_ok=True)
    h = source_hash()
    # kernel traces: per-dispatch durations
    for w in PROFILE_TRACE:
        path = _find(os.path.join(out, f"kt_{w}"), "kernel_trace.csv")
        if path is None:
            continue
        durs = {}
        for r in _csv_rows(path):
            k = _short(r["Kernel_Name"])
            if "nvfp4" not in k:
                continue
            durs.setdefault(k, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        lines = [f"# rocprofv3 kernel trace, workload {w} (library source hash {h})",
                 f"# command (repository root, TMPDIR=/tmp): {cmds['kt_' + w]}",
                 "# every dispatch of the run: eager reference, graph checks, warmup and timed steps;",
                 "# for the append workloads the pool fill is included (min/median are the steps)",
                 f"{'kernel':58s} {'calls':>6s} {'median_us':>10s} {'mean_us':>9s} {'min_us':>8s} {'max_us':>8s}"]
        for k, v in sorted(durs.items()):
            a = np.array(v)
            lines.append(f"{k:58s} {len(a):6d} {np.median(a):10.2f} {a.mean():9.2f} {a.min():8.2f} {a.max():8.2f}")
        with open(os.path.join(pdir, f"{w}_kernel_trace.txt"), "w") as f:
            f.write("\n".join(lines) + "\n")
    # HBM byte calibration: a plain copy of 1 GiB
    try:
        cf = _per_dispatch(os.path.join(out, "pmc_fetch_copy"), library_only=False)
        cw = _per_dispatch(os.path.join(out, "pmc_write_copy"), library_only=False)
        kf = max(cf, key=lambda k: np.mean(cf[k]["FETCH_SIZE"]))
        kw = max(cw, key=lambda k: np.mean(cw[k]["WRITE_SIZE"]))
        fetch_kib, write_kib = float(np.mean(cf[kf]["FETCH_SIZE"])), float(np.mean(cw[kw]["WRITE_SIZE"]))
        fscale, wscale = (1 << 30) / (fetch_kib * 1024), (1 << 30) / (write_kib * 1024)
    except (OSError, TypeError, ValueError):
        fscale = wscale = None
    for w in PROFILE_COUNTERS:
        per = {}
        for tag in COUNTER_PASSES:
            d = os.path.join(out, f"pmc_{tag}_{w}")
            if os.path.isdir(d):
                for k, cs in _per_dispatch(d).items():
                    for c, vals in cs.items():
                        per.setdefault(k, {})[c] = float(np.mean(vals))
        if not per:
            continue
        lines = [f"# rocprofv3 counters, workload {w} (library source hash {h}); mean per dispatch",
                 "# commands (repository root, TMPDIR=/tmp):"]
        lines += [f"#   {cmds[f'pmc_{t}_{w}']}" for t in COUNTER_PASSES]
        lines += [f"#   {cmds['pmc_fetch_copy']}", f"#   {cmds['pmc_write_copy']}",
                  "# derived: mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE/8 * 1024 SIMDs)",
                  "#   (GRBM_GUI_ACTIVE is summed over the 8 XCDs); valu_busy = SQ_ACTIVE_INST_VALU /",
                  "#   (GRBM_GUI_ACTIVE/8 * 256 CUs); mfma_tflop = SQ_INSTS_VALU_MFMA_MOPS_F16+BF16 * 512;",
                  "#   HBM bytes = FETCH_SIZE * fetch_scale + WRITE_SIZE * write_scale (KiB, copy-calibrated)"]
        traffic = {}
        for k, c in sorted(per.items()):
            lines.append(f"[{k}]")
            for name in sorted(c):
                lines.append(f"  {name:32s} {c[name]:18.1f}")
            gui = c.get("GRBM_GUI_ACTIVE")
            if gui:
                cyc = gui / 8
                if "SQ_VALU_MFMA_BUSY_CYCLES" in c:
                    lines.append(f"  {'mfma_busy':32s} {c['SQ_VALU_MFMA_BUSY_CYCLES'] / (cyc * SIMD_NUM):18.3f}")
                if "SQ_ACTIVE_INST_VALU" in c:
                    lines.append(f"  {'valu_busy':32s} {c['SQ_ACTIVE_INST_VALU'] / (cyc * CU_NUM):18.3f}")
                if "SQ_LDS_IDX_ACTIVE" in c:
                    lines.append(f"  {'lds_active':32s} {c['SQ_LDS_IDX_ACTIVE'] / (cyc * CU_NUM):18.3f}")
                lines.append(f"  {'gpu_busy_cycles_per_xcd':32s} {cyc:18.1f}")
            mops = c.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0.0) + c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0)
            if mops:
                lines.append(f"  {'mfma_gflop':32s} {mops * 512 / 1e9:18.3f}")
            if fscale and "FETCH_SIZE" in c and "WRITE_SIZE" in c:
                rb, wb = c["FETCH_SIZE"] * 1024 * fscale, c["WRITE_SIZE"] * 1024 * wscale
                lines.append(f"  {'hbm_read_mb':32s} {rb / 1e6:18.3f}")
                lines.append(f"  {'hbm_write_mb':32s} {wb / 1e6:18.3f}")
                traffic[k] = {"read_bytes": rb, "write_bytes": wb, "fetch_kib_raw": c["FETCH_SIZE"],
                              "write_kib_raw": c["WRITE_SIZE"]}
        if fscale:
            lines.append(f"# calibration: the 1 GiB copy reads FETCH_SIZE {fetch_kib:.0f} KiB and WRITE_SIZE "
                         f"{write_kib:.0f} KiB per dispatch: fetch_scale {fscale:.4f}, write_scale {wscale:.4f}")
        with open(os.path.join(pdir, f"{w}_counters.txt"), "w") as f:
            f.write("\n".join(lines) + "\n")
        # the decode call's kernels: the decode and, with splits, the combine
        dec = {k: v for k, v in traffic.items() if "decode" in k or "combine" in k}
        if dec:
            doc = {"workload": w, "source_hash": h,
                   "bytes_per_launch": sum(v["read_bytes"] + v["write_bytes"] for v in dec.values()),
                   "kernels": dec, "fetch_scale": fscale, "write_scale": wscale,
                   "calibration": f"plain 1 GiB device copy: FETCH_SIZE {fetch_kib:.0f} KiB, "
                                  f"WRITE_SIZE {write_kib:.0f} KiB per dispatch",
                   "commands": [cmds[f"pmc_fetch_{w}"], cmds[f"pmc_write_{w}"], cmds["pmc_fetch_copy"],
                                cmds["pmc_write_copy"]]}
            with open(os.path.join(pdir, f"traffic_{w}.json"), "w") as f:
                json.dump(doc, f, indent=1)
    print(f"profiles written for source hash {h}")


# --------------------------------------------------------------------------- main
def main():
    args = parse()
    if args.profile_commands:
        for _, c in profile_commands(args.profile_commands):
            print(c)
        return
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles)
        return
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
                               args.splits, no_cold=args.no_cold)
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
