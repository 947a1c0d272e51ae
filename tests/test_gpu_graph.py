"""HIP-graph capture of the library calls: the quantize-append and the decode
(both kernels, with and without splits, one cache and two, 352- and 432-byte
records) are captured once and replayed several times, with other eager work
and synchronisations between the replays; every replay must reproduce the
eager result bit for bit.  The calls allocate nothing and issue no memsets,
so the captured graphs hold kernel nodes only."""

import numpy as np
import pytest
import torch

from oracle import codec as OC
from sparse_mla_decode_nvfp4_amd import workloads as W
from tests._gpu_util import f64, note

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def records(n, rb, rep):
    lat, rope = W.latents(0, n, rep=rep)
    return OC.quantize_records(f64(lat), f64(rope), rb)


@pytest.mark.parametrize("h,splits,dual,rb,b", [
    (16, 1, False, 352, 3), (16, 3, False, 352, 3), (32, 1, False, 352, 3), (64, 4, False, 352, 3),
    (16, 2, True, 352, 3), (64, 2, True, 352, 3), (32, 3, False, 432, 3), (16, 1, True, 432, 3),
    # 1024 and 2048 workgroups: the 32-head kernel's two-pair shape
    (64, 1, False, 352, 256), (64, 2, True, 352, 256),
])
def test_captured_append_and_decode_replay_bit_exact(lib, h, splits, dual, rb, b):
    note(f"graph h={h} splits={splits} dual={dual} record={rb} batch={b}")
    rng = np.random.default_rng(h * 7 + splits + rb + b)
    s_q, k0, k1 = 2, 300, 200
    c0 = torch.from_numpy(records(1024, rb, 1).reshape(16, 64, rb)).to(DEV)
    c1 = torch.from_numpy(records(512, rb, 2).reshape(256, 2, rb)).to(DEV)
    q = torch.from_numpy(rng.standard_normal((b, s_q, h, 576)).astype(np.float32)).to(torch.bfloat16).to(DEV)
    i0 = torch.from_numpy(rng.integers(-1, 1024, size=(b, s_q, k0)).astype(np.int32)).to(DEV)
    i1 = torch.from_numpy(rng.integers(-1, 512, size=(b, s_q, k1)).astype(np.int32)).to(DEV)
    sink = torch.from_numpy(rng.standard_normal(h).astype(np.float32)).to(DEV)
    lat, rope = W.latents(0, b * s_q, rep=9)
    lat, rope = lat.to(DEV), rope.to(DEV)
    slots = torch.from_numpy(rng.choice(1024, size=b * s_q, replace=False).astype(np.int64)).to(DEV)
    topk = k0 + (k1 if dual else 0)
    ws = torch.empty(max(lib.workspace_size(b, s_q, h, topk, splits), 256), dtype=torch.uint8, device=DEV)
    out = torch.empty((b, s_q, h, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((b, s_q, h), dtype=torch.float32, device=DEV)

    def step():
        lib.quantize_append(lat, rope, slots, c0)
        if dual:
            lib.sparse_decode_dual(q, c0, i0, c1, i1, 1.0 / 24, sink=sink, num_splits=splits,
                                   workspace=ws, out=out, lse=lse)
        else:
            lib.sparse_decode(q, c0, i0, 1.0 / 24, sink=sink, num_splits=splits, workspace=ws,
                              out=out, lse=lse)

    step()
    torch.cuda.synchronize()
    ref_o, ref_l, ref_c = out.clone(), lse.clone(), c0.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                      # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(0)
        lse.fill_(float("nan"))
        junk = torch.randn(1 << 16, device=DEV).sum()         # other eager work in between
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o), f"replay {rep}: O differs"
        assert torch.equal(lse, ref_l), f"replay {rep}: LSE differs"
        assert torch.equal(c0, ref_c), f"replay {rep}: cache differs"
        assert bool(torch.isfinite(junk))
