"""A seeded random sweep of decode configurations against the fp64 oracle.

Each case draws, from one fixed seed, a combination the hand-picked cases
elsewhere do not enumerate: head count (every multiple of 16 kernel path up
to 256), batch and query rows, top-k from 1 to a few thousand, split count
(planner or explicit), page size (1 to 256 tokens, powers of two and not),
page padding, record width (352 or 432 bytes), one cache or two (each list
with its own page geometry, either list possibly empty), invalid and
out-of-range indices, duplicates, sink on or off, and the sign and size of
the softmax scale.  Outputs start as NaN; O and LSE must meet the oracle's
tolerance on every element (|d| <= 1e-2 + 2e-2 |ref|, LSE 1e-3, -inf rows
exact).
"""

import numpy as np
import pytest
import torch

from oracle import attention as OA
from oracle import codec as OC
from sparse_mla_decode_nvfp4_amd import workloads as W
from tests._gpu_util import assert_decode_close, f64, nan_outputs, note, padded_cache

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
HEADS = [16, 32, 48, 64, 80, 96, 112, 128, 144, 160, 192, 224, 240, 256]
PAGES = [1, 2, 3, 7, 16, 48, 64, 256]
PADS = [0, 0, 16, 48, 208]
SCALES = [1.0 / 24, 1.0 / 24, 0.1, 0.02, -1.0 / 24]


def draw_cases(n_cases=80, seed=20240611):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n_cases):
        h = int(rng.choice(HEADS))
        b, s_q = int(rng.integers(1, 5)), int(rng.integers(1, 4))
        dual = bool(rng.random() < 0.35)
        if dual:
            k0, k1 = int(rng.integers(0, 300)), int(rng.integers(0, 800))
            empty = rng.random()          # either list may be empty
            if empty < 0.15:
                k0 = 0
            elif empty < 0.3:
                k1 = 0
            if k0 + k1 == 0:
                k1 = 1
        else:
            k0, k1 = int(np.exp(rng.uniform(0, np.log(2600)))), 0
        topk = k0 + k1
        splits = int(rng.choice([0, 0, 1, 2, 3, 5, 8]))
        splits = min(splits, max(1, topk // 16)) if splits else 0
        cases.append(dict(
            i=i, h=h, b=b, s_q=s_q, dual=dual, k0=k0, k1=k1, splits=splits,
            rb=int(rng.choice([352, 432])),
            g0=(int(rng.choice(PAGES)), int(rng.choice(PADS))),
            g1=(int(rng.choice(PAGES)), int(rng.choice(PADS))),
            p_inval=float(rng.choice([0.0, 0.05, 0.3, 0.9])),
            oob=bool(rng.random() < 0.3), sink=bool(rng.random() < 0.7),
            scale=float(rng.choice(SCALES)), seed=int(rng.integers(1 << 30))))
    return cases


CASES = draw_cases()


def index_list(rng, n, num_slots, shape, p_inval, oob):
    """Slot ids of the n records (duplicates allowed), a fraction invalid
    (-1), and (oob) some at or beyond the cache's num_slots (num_blocks *
    block_size, which may exceed n: the last page's unused slots hold zero
    bytes and are valid slots).  Returns (list for the GPU, list for the
    oracle with the out-of-range ids marked invalid, which is how the GPU
    must treat them)."""
    idx = rng.integers(0, n, size=shape).astype(np.int32)
    idx[rng.random(shape) < p_inval] = -1
    if oob and idx.size:
        sel = rng.random(shape) < 0.05
        idx[sel] = num_slots + rng.integers(0, 1000, size=int(sel.sum()))
    return idx, np.where(idx >= num_slots, -1, idx).astype(np.int32)


def cache_of(rng_seed, n, rb, geometry, pool):
    """n records in pages of `geometry` = (block_size, pad bytes); returns
    (the records, the paged cache, its slot count)."""
    bs, pad = geometry
    lat, rope = W.latents(0, n, rep=rng_seed % 1000, pool=pool)
    recs = OC.quantize_records(f64(lat), f64(rope), rb)
    nb = -(-n // bs)
    if pad == 0:
        full = np.zeros((nb * bs, rb), np.uint8)
        full[:n] = recs
        return recs, torch.from_numpy(full.reshape(nb, bs, rb)).to(DEV), nb * bs
    cache, _, _ = padded_cache(recs, bs, pad, seed=rng_seed % 997, device=DEV)
    assert cache.shape[0] * cache.shape[1] == nb * bs
    return recs, cache, nb * bs


@pytest.mark.parametrize("case", CASES, ids=[f"c{c['i']}" for c in CASES])
def test_random_configuration_matches_oracle(lib, case):
    c = case
    what = (f"sweep c{c['i']}: b{c['b']} s{c['s_q']} h{c['h']} k{c['k0']}+{c['k1']} "
            f"{'dual' if c['dual'] else 'single'} R{c['rb']} pages {c['g0']}/{c['g1']} "
            f"sp{c['splits']} inval{c['p_inval']} oob{c['oob']} sink{c['sink']} scale{c['scale']:.4f}")
    note(what)
    rng = np.random.default_rng(c["seed"])
    b, s_q, h = c["b"], c["s_q"], c["h"]
    q = torch.from_numpy(rng.standard_normal((b, s_q, h, 576)).astype(np.float32)).to(torch.bfloat16)
    sink = rng.standard_normal(h).astype(np.float32) if c["sink"] else None
    sink_d = None if sink is None else torch.from_numpy(sink).to(DEV)
    sink_o = None if sink is None else sink.astype(np.float64)
    out, lse = nan_outputs((b, s_q, h), DEV)
    n0 = max(2 * c["k0"], 3 * c["g0"][0] + 5, 8)
    r0, c0, ns0 = cache_of(c["seed"], n0, c["rb"], c["g0"], pool=0)
    i0, i0_ref = index_list(rng, n0, ns0, (b, s_q, c["k0"]), c["p_inval"], c["oob"])
    if c["dual"]:
        n1 = max(2 * c["k1"], 3 * c["g1"][0] + 5, 8)
        r1, c1, ns1 = cache_of(c["seed"] + 1, n1, c["rb"], c["g1"], pool=1)
        i1, i1_ref = index_list(rng, n1, ns1, (b, s_q, c["k1"]), c["p_inval"], c["oob"])
        lib.sparse_decode_dual(q.to(DEV), c0, torch.from_numpy(i0).to(DEV), c1,
                               torch.from_numpy(i1).to(DEV), c["scale"], sink=sink_d,
                               num_splits=c["splits"], out=out, lse=lse)
        torch.cuda.synchronize()
        o_ref, l_ref = OA.sparse_decode_dual(f64(q), r0, i0_ref, r1, i1_ref, c["scale"], sink=sink_o)
    else:
        lib.sparse_decode(q.to(DEV), c0, torch.from_numpy(i0).to(DEV), c["scale"], sink=sink_d,
                          num_splits=c["splits"], out=out, lse=lse)
        torch.cuda.synchronize()
        o_ref, l_ref = OA.sparse_decode(f64(q), r0, i0_ref, c["scale"], sink=sink_o)
    assert_decode_close(out, lse, o_ref, l_ref, what)
