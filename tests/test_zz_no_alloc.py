"""GPU check of the allocation-free decode entry point
(nvfp4_mla_sparse_decode_noalloc): its split partials live in the library's
static per-GPU scratch array instead of a caller workspace.  Called through
the C ABI, it must give the same O and LSE bits as nvfp4_mla_sparse_decode
with the same split count (the same kernels), and both must meet the fp64
oracle's tolerance.  Two calls run back to back, the second on a smaller
input, so the second reads nothing the first left in the array.  A split
count whose partials exceed the array is refused before any launch.
"""

import numpy as np
import pytest
import torch

import sparse_mla_decode_nvfp4_amd as M
from oracle import attention as OA
from oracle import codec as OC
from sparse_mla_decode_nvfp4_amd import workloads as W
from tests._gpu_util import assert_decode_close, f64, note

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SCALE = 1.0 / 24


def case(seed, b, h, topk, nblocks=24, bs=64):
    rng = np.random.default_rng(seed)
    n = nblocks * bs
    lat, rope = W.latents(0, n, rep=seed)
    recs = OC.quantize_records(f64(lat), f64(rope))
    q = torch.from_numpy(rng.standard_normal((b, 1, h, 576)).astype(np.float32)).to(torch.bfloat16)
    idx = rng.integers(0, n, size=(b, 1, topk)).astype(np.int32)
    idx[rng.random(idx.shape) < 0.1] = -1
    sink = rng.standard_normal(h).astype(np.float32)
    return recs, q, idx, sink, nblocks, bs


@pytest.mark.parametrize("h,splits", [(16, 3), (64, 4), (128, 0)])
def test_noalloc_matches_the_workspace_decode_on_two_calls(lib, h, splits):
    for k, (b, topk) in enumerate([(6, 700), (2, 300)]):        # second call smaller
        note(f"noalloc h={h} splits={splits} call {k}: b={b} topk={topk}")
        recs, q, idx, sink, nb, bs = case(100 * h + k, b, h, topk)
        cache = torch.from_numpy(recs.reshape(nb, bs, 352)).to(DEV)
        qd, idd, sk = q.to(DEV), torch.from_numpy(idx).to(DEV), torch.from_numpy(sink).to(DEV)
        o1, l1 = lib.sparse_decode_noalloc(qd, cache, idd, SCALE, sink=sk, num_splits=splits)
        o2, l2 = lib.sparse_decode(qd, cache, idd, SCALE, sink=sk, num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), "differs from the workspace decode"
        o_ref, l_ref = OA.sparse_decode(f64(q), recs, idx, SCALE, sink=sink.astype(np.float64))
        assert_decode_close(o1, l1, o_ref, l_ref, f"noalloc h{h} call {k}")


def test_noalloc_refuses_partials_beyond_its_array(lib):
    # 64 rows x 128 heads x 64 splits of partials: far beyond the array
    recs, q, idx, sink, nb, bs = case(7, 64, 128, 1024)
    cache = torch.from_numpy(recs.reshape(nb, bs, 352)).to(DEV)
    with pytest.raises(M.Nvfp4MlaError) as e:
        lib.sparse_decode_noalloc(q.to(DEV), cache, torch.from_numpy(idx).to(DEV), SCALE,
                                  num_splits=64)
    assert e.value.code == M.ERR_WORKSPACE_TOO_SMALL
    assert "allocation-free" in str(e.value)
