"""GPU parity of the decodes on padded page layouts, and canaries around every
buffer the kernels write.

Padded pages: the paged-cache convention lets a page start
block_stride_bytes after the previous one with block_stride_bytes larger
than block_size * R (vLLM PR #82, review thread on the block and entry
strides).  Caches here are as_strided views over random backing bytes, with
pads of 16 bytes to over 4 KB, page sizes that are and are not powers of
two, both record widths, both decode kernels, splits, and dual-cache decodes
whose two caches have different page sizes and strides.  O and LSE must meet
the fp64 oracle's tolerance (|d| <= 1e-2 + 2e-2 |ref|, LSE 1e-3) and the
backing bytes must be unchanged.

Canaries: O, LSE, the decode workspace, the combine's outputs and the
gather's output are placed between two 4 KB regions of a known byte; after
the call every canary byte must be intact and the results correct (an
out-of-bounds write that lands next to a buffer shows up here).
"""

import numpy as np
import pytest
import torch

from oracle import attention as OA
from oracle import codec as OC
from sparse_mla_decode_nvfp4_amd import workloads as W
from tests._gpu_util import Guarded, assert_decode_close, f64, note, padded_cache

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SCALE = 1.0 / 24


def records(seed, n, rb, pool=0):
    lat, rope = W.latents(0, n, rep=seed, pool=pool)
    return OC.quantize_records(f64(lat), f64(rope), rb)


def query(rng, b, s_q, h):
    return torch.from_numpy(rng.standard_normal((b, s_q, h, 576)).astype(np.float32)).to(torch.bfloat16)


def index_list(rng, n, shape, p_inval=0.1):
    idx = rng.integers(0, n, size=shape).astype(np.int32)
    idx[rng.random(shape) < p_inval] = -1
    return idx


# b, s_q, h, topk, block_size, pad bytes, record bytes, splits
PADDED = [
    (2, 1, 16, 300, 48, 16, 352, 1),
    (2, 2, 16, 700, 48, 48, 352, 3),
    (1, 1, 32, 333, 64, 32, 352, 1),
    (2, 1, 64, 900, 64, 4112, 352, 4),
    (1, 2, 128, 200, 3, 16, 352, 1),
    (3, 1, 48, 129, 7, 80, 352, 2),
    (2, 1, 16, 257, 48, 16, 432, 2),
    (2, 1, 64, 500, 64, 80, 432, 1),
    (1, 1, 128, 300, 5, 32, 432, 3),
]


@pytest.mark.parametrize("b,s_q,h,topk,bs,pad,rb,splits", PADDED)
def test_decode_on_padded_pages(lib, b, s_q, h, topk, bs, pad, rb, splits):
    what = f"padded pages b{b} s{s_q} h{h} k{topk} bs{bs} pad{pad} R{rb} sp{splits}"
    note(what)
    rng = np.random.default_rng(b * 131 + h + bs + pad)
    n = max(20 * bs, 2 * topk)
    recs = records(7 + bs + pad, n, rb)
    cache, back, backing = padded_cache(recs, bs, pad, seed=bs + pad, device=DEV)
    assert cache.stride(0) == bs * rb + pad
    q = query(rng, b, s_q, h)
    idx = index_list(rng, n, (b, s_q, topk))
    sink = rng.standard_normal(h).astype(np.float32)
    o, lse = lib.sparse_decode(q.to(DEV), cache, torch.from_numpy(idx).to(DEV), SCALE,
                               sink=torch.from_numpy(sink).to(DEV), num_splits=splits)
    torch.cuda.synchronize()
    o_ref, l_ref = OA.sparse_decode(f64(q), recs, idx, SCALE, sink=sink.astype(np.float64))
    assert_decode_close(o, lse, o_ref, l_ref, what)
    assert np.array_equal(back.cpu().numpy(), backing), "the decode wrote into the cache"


# b, s_q, h, topk0, topk1, (bs0, pad0), (bs1, pad1), record bytes, splits
PADDED_DUAL = [
    (2, 2, 16, 128, 512, (64, 16), (2, 48), 352, 1),
    (1, 1, 64, 100, 300, (48, 32), (3, 16), 352, 3),
    (2, 1, 32, 150, 90, (64, 4096), (1, 16), 352, 2),
    (1, 1, 16, 70, 200, (64, 16), (2, 32), 432, 2),
    (1, 2, 64, 128, 256, (48, 48), (64, 80), 432, 1),
]


@pytest.mark.parametrize("b,s_q,h,k0,k1,g0,g1,rb,splits", PADDED_DUAL)
def test_dual_decode_on_padded_pages_of_two_geometries(lib, b, s_q, h, k0, k1, g0, g1, rb, splits):
    (bs0, pad0), (bs1, pad1) = g0, g1
    what = f"dual padded b{b} s{s_q} h{h} k{k0}+{k1} pages {bs0}+{pad0}/{bs1}+{pad1} R{rb} sp{splits}"
    note(what)
    rng = np.random.default_rng(b * 71 + h + k0 + k1)
    n0, n1 = 6 * bs0 + 3, 150 * bs1 + 1
    r0 = records(11 + bs0, n0, rb)
    r1 = records(12 + bs1, n1, rb, pool=1)
    c0, back0, bytes0 = padded_cache(r0, bs0, pad0, seed=pad0, device=DEV)
    c1, back1, bytes1 = padded_cache(r1, bs1, pad1, seed=pad1 + 1, device=DEV)
    q = query(rng, b, s_q, h)
    i0 = index_list(rng, n0, (b, s_q, k0))
    i1 = index_list(rng, n1, (b, s_q, k1))
    sink = rng.standard_normal(h).astype(np.float32)
    o, lse = lib.sparse_decode_dual(q.to(DEV), c0, torch.from_numpy(i0).to(DEV), c1,
                                    torch.from_numpy(i1).to(DEV), SCALE,
                                    sink=torch.from_numpy(sink).to(DEV), num_splits=splits)
    torch.cuda.synchronize()
    o_ref, l_ref = OA.sparse_decode_dual(f64(q), r0, i0, r1, i1, SCALE, sink=sink.astype(np.float64))
    assert_decode_close(o, lse, o_ref, l_ref, what)
    assert np.array_equal(back0.cpu().numpy(), bytes0) and np.array_equal(back1.cpu().numpy(), bytes1)


# ---------------------------------------------------------------- canaries
def guarded_outputs(b, s_q, h):
    go = Guarded(b * s_q * h * 512 * 2, DEV, fill=0x7F)
    gl = Guarded(b * s_q * h * 4, DEV, fill=0x7F)
    return go, gl, go.view(torch.bfloat16, (b, s_q, h, 512)), gl.view(torch.float32, (b, s_q, h))


@pytest.mark.parametrize("b,s_q,h,topk,splits,rb", [
    (3, 1, 16, 500, 1, 352), (2, 2, 16, 700, 4, 352), (2, 1, 64, 900, 1, 352),
    (3, 1, 64, 1000, 5, 352), (1, 1, 128, 600, 3, 352), (2, 1, 48, 300, 2, 432),
    (2, 1, 32, 777, 6, 432),
])
def test_decode_writes_nothing_outside_o_lse_and_its_workspace(lib, b, s_q, h, topk, splits, rb):
    what = f"canaries b{b} s{s_q} h{h} k{topk} sp{splits} R{rb}"
    note(what)
    rng = np.random.default_rng(h * 7 + splits + rb)
    n = 40 * 64
    recs = records(3 + h, n, rb)
    cache = torch.from_numpy(recs.reshape(40, 64, rb)).to(DEV)
    q = query(rng, b, s_q, h)
    idx = index_list(rng, n, (b, s_q, topk))
    idx[0, 0, :] = -1                                  # an empty row
    sink = rng.standard_normal(h).astype(np.float32)
    go, gl, o, lse = guarded_outputs(b, s_q, h)
    need = lib.workspace_size(b, s_q, h, topk, splits)
    gw = Guarded(max(need, 256), DEV, fill=0xC3)
    ws = gw.inner if need else None
    lib.sparse_decode(q.to(DEV), cache, torch.from_numpy(idx).to(DEV), SCALE,
                      sink=torch.from_numpy(sink).to(DEV), num_splits=splits, workspace=ws,
                      out=o, lse=lse)
    torch.cuda.synchronize()
    for g, name in ((go, "O"), (gl, "LSE"), (gw, "workspace")):
        g.check(f"{what} {name}")
    o_ref, l_ref = OA.sparse_decode(f64(q), recs, idx, SCALE, sink=sink.astype(np.float64))
    assert_decode_close(o, lse, o_ref, l_ref, what)


@pytest.mark.parametrize("h,splits", [(16, 3), (64, 2)])
def test_dual_decode_writes_nothing_outside_its_buffers(lib, h, splits):
    what = f"dual canaries h{h} sp{splits}"
    note(what)
    rng = np.random.default_rng(h + splits)
    n0, n1 = 4 * 64, 300 * 2
    r0, r1 = records(21, n0, 352), records(22, n1, 352, pool=1)
    c0 = torch.from_numpy(r0.reshape(4, 64, 352)).to(DEV)
    c1 = torch.from_numpy(r1.reshape(300, 2, 352)).to(DEV)
    b, s_q = 2, 2
    q = query(rng, b, s_q, h)
    i0, i1 = index_list(rng, n0, (b, s_q, 128)), index_list(rng, n1, (b, s_q, 512))
    sink = rng.standard_normal(h).astype(np.float32)
    go, gl, o, lse = guarded_outputs(b, s_q, h)
    need = lib.workspace_size(b, s_q, h, 640, splits)
    gw = Guarded(need, DEV, fill=0x3C)
    lib.sparse_decode_dual(q.to(DEV), c0, torch.from_numpy(i0).to(DEV), c1,
                           torch.from_numpy(i1).to(DEV), SCALE,
                           sink=torch.from_numpy(sink).to(DEV), num_splits=splits,
                           workspace=gw.inner, out=o, lse=lse)
    torch.cuda.synchronize()
    for g, name in ((go, "O"), (gl, "LSE"), (gw, "workspace")):
        g.check(f"{what} {name}")
    o_ref, l_ref = OA.sparse_decode_dual(f64(q), r0, i0, r1, i1, SCALE, sink=sink.astype(np.float64))
    assert_decode_close(o, lse, o_ref, l_ref, what)


def test_combine_and_gather_write_nothing_outside_their_outputs(lib):
    rng = np.random.default_rng(5)
    p, r, h = 3, 5, 32
    o_part = rng.standard_normal((p, r, h, 512)).astype(np.float32)
    lse_part = rng.standard_normal((p, r, h)).astype(np.float32)
    sink = rng.standard_normal(h).astype(np.float32)
    go, gl = Guarded(r * h * 512 * 2, DEV), Guarded(r * h * 4, DEV)
    o = go.view(torch.bfloat16, (r, h, 512))
    lse = gl.view(torch.float32, (r, h))
    lib.combine(torch.from_numpy(o_part).to(DEV), torch.from_numpy(lse_part).to(DEV),
                sink=torch.from_numpy(sink).to(DEV), out=o, lse=lse)
    torch.cuda.synchronize()
    go.check("combine O")
    gl.check("combine LSE")
    o_ref, l_ref = OA.combine(o_part.astype(np.float64), lse_part.astype(np.float64),
                              sink=sink.astype(np.float64))
    assert_decode_close(o, lse, o_ref, l_ref, "combine")
    # the gather: 37 rows (a ragged count of 4-row blocks)
    recs = records(9, 4 * 64, 352)
    cache = torch.from_numpy(recs.reshape(4, 64, 352)).to(DEV)
    slots = rng.integers(-1, 4 * 64, size=37).astype(np.int32)
    gg = Guarded(37 * 576 * 2, DEV)
    out = gg.view(torch.bfloat16, (37, 576))
    lib.dequantize_gather(cache, torch.from_numpy(slots).to(DEV), out=out)
    torch.cuda.synchronize()
    gg.check("gather")
    ref = OC.dequantize_records(recs)[np.maximum(slots, 0)]
    ref[slots < 0] = 0
    assert np.array_equal(out.to(torch.float64).cpu().numpy(), ref)
