"""GPU parity at the limits the C ABI accepts: the largest head count (256,
both kernels: 256 runs the 32-head kernel, 240 the 16-head one), the
largest top-k (65536, drawn with repeats from a small pool so the oracle
stays quick), the largest split count (64), very large and one-token pages,
and empty batches.  Same tolerance as every decode test."""

import numpy as np
import pytest
import torch

from oracle import attention as OA
from oracle import codec as OC
from sparse_mla_decode_nvfp4_amd import workloads as W
from tests._gpu_util import assert_decode_close, f64, note

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def pool(n, rep):
    lat, rope = W.latents(0, n, rep=rep)
    return OC.quantize_records(f64(lat), f64(rope))


def run(lib, recs, bs, q, idx, sink, splits, scale=1.0 / 24):
    cache = torch.from_numpy(recs.reshape(-1, bs, 352)).to(DEV)
    o, lse = lib.sparse_decode(q.to(DEV), cache, torch.from_numpy(idx).to(DEV), scale,
                               sink=torch.from_numpy(sink).to(DEV), num_splits=splits)
    torch.cuda.synchronize()
    o_ref, l_ref = OA.sparse_decode(f64(q), recs, idx, scale, sink=sink.astype(np.float64))
    return o, lse, o_ref, l_ref


@pytest.mark.parametrize("h", [256, 240])
def test_largest_heads_and_topk(lib, h):
    note(f"limits: h={h} topk=65536")
    rng = np.random.default_rng(h)
    recs = pool(4096, 1)
    q = torch.from_numpy(rng.standard_normal((1, 1, h, 576)).astype(np.float32)).to(torch.bfloat16)
    idx = rng.integers(0, 4096, size=(1, 1, 65536)).astype(np.int32)
    idx[rng.random(idx.shape) < 0.05] = -1
    sink = rng.standard_normal(h).astype(np.float32)
    o, lse, o_ref, l_ref = run(lib, recs, 64, q, idx, sink, 0)
    assert_decode_close(o, lse, o_ref, l_ref, f"h{h} topk65536")


@pytest.mark.parametrize("h", [16, 32])
def test_largest_split_count(lib, h):
    note(f"limits: 64 splits h={h}")
    rng = np.random.default_rng(64 + h)
    recs = pool(2048, 2)
    q = torch.from_numpy(rng.standard_normal((2, 1, h, 576)).astype(np.float32)).to(torch.bfloat16)
    idx = rng.integers(0, 2048, size=(2, 1, 3000)).astype(np.int32)
    idx[rng.random(idx.shape) < 0.1] = -1
    idx[1, 0, :1500] = -1                 # many empty splits in row 1
    sink = rng.standard_normal(h).astype(np.float32)
    o, lse, o_ref, l_ref = run(lib, recs, 64, q, idx, sink, 64)
    assert_decode_close(o, lse, o_ref, l_ref, f"64 splits h{h}")


@pytest.mark.parametrize("bs", [1, 1024])
def test_one_token_and_large_pages(lib, bs):
    note(f"limits: block_size={bs}")
    rng = np.random.default_rng(bs)
    recs = pool(2048, 3)
    q = torch.from_numpy(rng.standard_normal((3, 1, 32, 576)).astype(np.float32)).to(torch.bfloat16)
    idx = rng.integers(-1, 2048, size=(3, 1, 700)).astype(np.int32)
    sink = rng.standard_normal(32).astype(np.float32)
    o, lse, o_ref, l_ref = run(lib, recs, bs, q, idx, sink, 0)
    assert_decode_close(o, lse, o_ref, l_ref, f"block_size {bs}")


def test_empty_batch_is_a_no_op(lib):
    cache = lib.new_cache(2, 64, DEV)
    q = torch.zeros((0, 1, 16, 576), dtype=torch.bfloat16, device=DEV)
    idx = torch.zeros((0, 1, 8), dtype=torch.int32, device=DEV)
    o, lse = lib.sparse_decode(q, cache, idx, 0.04)
    torch.cuda.synchronize()
    assert o.shape == (0, 1, 16, 512) and lse.shape == (0, 1, 16)
