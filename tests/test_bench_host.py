"""Host-side checks of bench.py (no GPU): it parses, refuses more than one
GPU before touching the device, and its algorithmic accounting counts what
the workloads hold."""

import subprocess
import sys

import numpy as np

import bench
from sparse_mla_decode_nvfp4_amd import workloads as W


def test_more_than_one_gpu_is_refused_before_any_device_work():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=bench.ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_accounting_counts_valid_tokens_of_every_list():
    wl = W.tiny()
    acc = bench.decode_accounting([wl], wl)
    nv = int(((wl.indices >= 0) & (wl.indices < wl.num_slots)).sum())
    assert acc["flops"] == nv * 2 * (576 + 512) * wl.h_q
    assert acc["kv_bytes"] == nv * 352
    d = W.prefill_dual(tokens=8, h_q=16, seq=1024, with_latents=False)
    acc = bench.decode_accounting([d], d)
    nv = int((d.indices >= 0).sum() + (d.extra_indices >= 0).sum())
    assert acc["flops"] == nv * 2 * (576 + 512) * 16
    uniq = len(np.unique(d.indices[d.indices >= 0])) + len(np.unique(d.extra_indices[d.extra_indices >= 0]))
    assert acc["unique_bytes"] - acc["other_bytes"] == uniq * 352


def test_432_byte_workload_counts_its_record_size():
    wl = W.decode_h64_ds_mla(batch=2, with_latents=False)
    acc = bench.decode_accounting([wl], wl)
    nv = int(((wl.indices >= 0) & (wl.indices < wl.num_slots)).sum())
    assert acc["kv_bytes"] == nv * 432


def test_named_prefill_workloads_resolve():
    gen = W.dual_workload("prefill_dual_h32_t16")
    wl = gen(with_latents=False)
    assert (wl.h_q, wl.s_q, wl.batch, wl.topk) == (32, 16, 1, 640)
    assert W.dual_workload("decode_h64") is None
    assert len(bench.source_hash()) == 16
