"""C-ABI tests that need no GPU: the library loads, exports every function
include/nvfp4_mla.h declares, and rejects every invalid argument with its own
status code before making any HIP call.

None of these calls reaches a kernel launch: each one fails argument
validation first (or, on a machine without a GPU, the device gate), so the
placeholder pointers below are never dereferenced.
"""

import ctypes
import os
import re

import pytest
import torch

import sparse_mla_decode_nvfp4_amd as m

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4_mla.h")

# placeholder "device pointers": aligned, never dereferenced by these tests
P16 = ctypes.c_void_p(0x100000)
P256 = ctypes.c_void_p(0x200000)
NULL = ctypes.c_void_p(0)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_mla_\w+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = m.lib()
    names = declared_functions()
    assert len(names) == 19
    for name in names:
        assert hasattr(lib, name), name
        assert name in m.SIGNATURES, name
    assert m.abi_version() == 1


def test_check_format_accepts_the_352_and_432_byte_records():
    m.check_format()
    m.check_format(record_bytes=432)
    lib = m.lib()
    for args in [(656, 512, 64, 512), (584, 512, 64, 512), (384, 512, 64, 512),
                 (352, 448, 64, 512), (352, 512, 128, 512), (352, 512, 64, 576),
                 (432, 512, 64, 576)]:
        assert lib.nvfp4_mla_check_format(*args) == m.ERR_UNSUPPORTED_FORMAT
        assert "unsupported format" in m.last_error()


def qa(fn="nvfp4_mla_quantize_append", **kw):
    rb = 432 if fn.endswith("ds_mla") else 352
    a = dict(latent=P16, lstride=512, rope=P16, rstride=64, slots=P16, n=4, cache=P16,
             nblocks=4, bs=64, stride=64 * rb, stream=NULL)
    a.update(kw)
    return getattr(m.lib(), fn)(a["latent"], a["lstride"], a["rope"], a["rstride"],
                                a["slots"], a["n"], a["cache"], a["nblocks"],
                                a["bs"], a["stride"], a["stream"])


@pytest.mark.parametrize("kw, needle", [
    (dict(n=-1), "num_tokens"),
    (dict(cache=NULL), "kv_cache is NULL"),
    (dict(cache=ctypes.c_void_p(0x100008)), "16-byte aligned"),
    (dict(nblocks=0), "num_blocks"),
    (dict(bs=0), "block_size"),
    (dict(stride=64 * 352 + 8), "multiple of 16"),
    (dict(stride=63 * 352), "block_stride_bytes"),
    (dict(nblocks=1 << 26, bs=64), "2^31-1"),
    (dict(latent=NULL), "non-NULL"),
    (dict(slots=NULL), "non-NULL"),
    (dict(lstride=511), "row strides"),
    (dict(rstride=32), "row strides"),
    (dict(lstride=520 + 4), "16-byte aligned"),
    (dict(latent=ctypes.c_void_p(0x100004)), "16-byte aligned"),
])
@pytest.mark.parametrize("fn", ["nvfp4_mla_quantize_append", "nvfp4_mla_quantize_append_fp16",
                                "nvfp4_mla_quantize_append_ds_mla"])
def test_quantize_append_rejects_bad_arguments(fn, kw, needle):
    if fn.endswith("ds_mla") and "stride" in kw:
        kw = dict(stride=kw["stride"] // 352 * 432 + kw["stride"] % 352)
    assert qa(fn, **kw) == m.ERR_INVALID_ARGUMENT
    assert needle in m.last_error()


def test_ds_mla_exports_check_the_432_byte_page_stride():
    # a stride that holds 64 records of 352 bytes but not of 432
    assert qa("nvfp4_mla_quantize_append_ds_mla", stride=64 * 352) == m.ERR_INVALID_ARGUMENT
    assert "block_size * 432" in m.last_error()
    assert m.lib().nvfp4_mla_dequantize_gather_ds_mla(P16, 4, 64, 64 * 352, P16, 3, P16,
                                                      NULL) == m.ERR_INVALID_ARGUMENT
    assert "block_size * 432" in m.last_error()
    assert m.lib().nvfp4_mla_sparse_decode_ds_mla(
        P16, P16, 4, 64, 64 * 352, P16, 2, 1, 16, 64, NULL, 0.04, P16, P16, NULL, 0, 1,
        NULL) == m.ERR_INVALID_ARGUMENT
    assert "block_size * 432" in m.last_error()


def dec(**kw):
    a = dict(q=P16, cache=P16, nblocks=4, bs=64, stride=64 * 352, idx=P16, batch=2, s_q=1,
             h_q=16, topk=64, sink=NULL, scale=0.04, out=P16, lse=P16, ws=NULL, ws_bytes=0,
             splits=1, stream=NULL)
    a.update(kw)
    return m.lib().nvfp4_mla_sparse_decode(a["q"], a["cache"], a["nblocks"], a["bs"], a["stride"],
                                           a["idx"], a["batch"], a["s_q"], a["h_q"], a["topk"],
                                           a["sink"], a["scale"], a["out"], a["lse"], a["ws"],
                                           a["ws_bytes"], a["splits"], a["stream"])


@pytest.mark.parametrize("kw, needle", [
    (dict(h_q=8), "multiple of 16"),
    (dict(h_q=24), "multiple of 16"),
    (dict(h_q=272), "multiple of 16"),
    (dict(topk=0), "topk"),
    (dict(topk=65537), "topk"),
    (dict(batch=-1), "batch"),
    (dict(cache=NULL), "kv_cache"),
    (dict(stride=100), "multiple of 16"),
    (dict(splits=-1), "num_splits"),
    (dict(splits=65), "num_splits"),
    (dict(scale=float("nan")), "softmax_scale"),
    (dict(scale=float("inf")), "softmax_scale"),
    (dict(q=NULL), "non-NULL"),
    (dict(idx=NULL), "non-NULL"),
    (dict(out=NULL), "non-NULL"),
    (dict(lse=NULL), "non-NULL"),
    (dict(q=ctypes.c_void_p(0x100008)), "aligned"),
    (dict(out=ctypes.c_void_p(0x100004)), "aligned"),
    (dict(sink=ctypes.c_void_p(0x100002)), "aligned"),
    # one launch's work-items must fit HIP's 32-bit grid size: the 32-head
    # kernel (8 groups x 2^21 rows x 512), the 16-head kernel (15 groups x
    # 2^20 rows x 64 splits x 256) and the combine alone (96 x 2^20 x 64)
    (dict(batch=2 ** 21, h_q=256), "work-items"),
    (dict(batch=2 ** 20, h_q=240, splits=64), "work-items"),
    (dict(batch=2 ** 20, h_q=96, splits=2), "work-items"),
])
def test_sparse_decode_rejects_bad_arguments(kw, needle):
    assert dec(**kw) == m.ERR_INVALID_ARGUMENT
    assert needle in m.last_error()


def dec_noalloc(**kw):
    a = dict(q=P16, cache=P16, nblocks=4, bs=64, stride=64 * 352, idx=P16, batch=2, s_q=1,
             h_q=16, topk=64, sink=NULL, scale=0.04, out=P16, lse=P16, splits=1, stream=NULL)
    a.update(kw)
    return m.lib().nvfp4_mla_sparse_decode_noalloc(
        a["q"], a["cache"], a["nblocks"], a["bs"], a["stride"], a["idx"], a["batch"], a["s_q"],
        a["h_q"], a["topk"], a["sink"], a["scale"], a["out"], a["lse"], a["splits"], a["stream"])


@pytest.mark.parametrize("kw, needle", [
    (dict(h_q=24), "multiple of 16"),
    (dict(topk=0), "topk"),
    (dict(cache=NULL), "kv_cache"),
    (dict(stride=64 * 352 - 16), "block_size * 352"),
    (dict(splits=65), "num_splits"),
    (dict(q=NULL), "non-NULL"),
    (dict(lse=ctypes.c_void_p(0x100002)), "aligned"),
])
def test_sparse_decode_noalloc_rejects_bad_arguments(kw, needle):
    assert dec_noalloc(**kw) == m.ERR_INVALID_ARGUMENT
    assert needle in m.last_error()


def test_sparse_decode_noalloc_without_a_gpu_reports_the_device_gate():
    if torch.cuda.device_count() > 0:
        pytest.skip("device-gate check is for GPU-less hosts")
    assert dec_noalloc() == m.ERR_UNSUPPORTED_DEVICE
    assert dec_noalloc(splits=4) == m.ERR_UNSUPPORTED_DEVICE


def fused(fn="nvfp4_mla_norm_rope_quantize_append", **kw):
    rb = 432 if fn.endswith("ds_mla") else 352
    a = dict(latent=P16, lstride=512, rope=P16, rstride=64, weight=P16, eps=1e-6, cs=P16,
             maxpos=128, pos=P16, neox=0, slots=P16, n=4, cache=P16, nblocks=4, bs=64,
             stride=64 * rb, stream=NULL)
    a.update(kw)
    return getattr(m.lib(), fn)(a["latent"], a["lstride"], a["rope"], a["rstride"], a["weight"],
                                a["eps"], a["cs"], a["maxpos"], a["pos"], a["neox"], a["slots"],
                                a["n"], a["cache"], a["nblocks"], a["bs"], a["stride"],
                                a["stream"])


@pytest.mark.parametrize("fn", ["nvfp4_mla_norm_rope_quantize_append",
                                "nvfp4_mla_norm_rope_quantize_append_ds_mla"])
@pytest.mark.parametrize("kw, needle", [
    (dict(eps=float("nan")), "eps"),
    (dict(eps=-1e-6), "eps"),
    (dict(eps=float("inf")), "eps"),
    (dict(neox=2), "rope_neox"),
    (dict(maxpos=0), "max_position"),
    (dict(weight=NULL), "non-NULL"),
    (dict(cs=NULL), "non-NULL"),
    (dict(pos=NULL), "non-NULL"),
    (dict(weight=ctypes.c_void_p(0x100008)), "aligned"),
    (dict(pos=ctypes.c_void_p(0x100004)), "aligned"),
    (dict(lstride=500), "row strides"),
    (dict(cache=NULL), "kv_cache"),
    (dict(stride=64 * 352 - 16), "block_size"),
])
def test_fused_write_rejects_bad_arguments(fn, kw, needle):
    if fn.endswith("ds_mla") and kw.get("stride") == 64 * 352 - 16:
        kw = dict(stride=64 * 432 - 16)
    assert fused(fn, **kw) == m.ERR_INVALID_ARGUMENT
    assert needle in m.last_error()


def test_fused_f32_export_rejects_bad_arguments():
    lib = m.lib()
    call = lambda **kw: lib.nvfp4_mla_norm_rope_f32(
        kw.get("latent", P16), 512, P16, 64, kw.get("weight", P16), kw.get("eps", 0.0), P16,
        kw.get("maxpos", 16), P16, 0, kw.get("n", 3), kw.get("out", P16), NULL)
    assert call(n=-1) == m.ERR_INVALID_ARGUMENT
    assert call(eps=float("nan")) == m.ERR_INVALID_ARGUMENT
    assert call(out=NULL) == m.ERR_INVALID_ARGUMENT
    assert call(out=ctypes.c_void_p(0x100004)) == m.ERR_INVALID_ARGUMENT
    assert "aligned" in m.last_error()
    assert call(maxpos=0) == m.ERR_INVALID_ARGUMENT


def test_header_compiles_as_c_and_cxx():
    """The header is plain C (its own hipStream_t declaration, no HIP
    include needed) and sits beside hip_runtime_api.h in C++."""
    import shutil
    import subprocess
    import tempfile
    cc, cxx = shutil.which("gcc"), shutil.which("g++")
    if cc is None or cxx is None:
        pytest.skip("no host compiler")
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "t.c")
        with open(c, "w") as f:
            f.write('#include "nvfp4_mla.h"\nint main(void) { hipStream_t s = 0; (void)s; '
                    'int (*f)(void) = nvfp4_mla_abi_version; return f == 0; }\n')
        r = subprocess.run([cc, "-std=c11", "-Wall", "-Werror", "-fsyntax-only", "-I",
                            os.path.dirname(HEADER), c], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        cpp = os.path.join(d, "t.cpp")
        with open(cpp, "w") as f:
            f.write('#include "nvfp4_mla.h"\n#include <hip/hip_runtime_api.h>\n'
                    'int main() { hipStream_t s = nullptr; return s ? 1 : 0; }\n')
        r = subprocess.run([cxx, "-std=c++17", "-Wall", "-Werror", "-fsyntax-only",
                            "-D__HIP_PLATFORM_AMD__", "-I", os.path.dirname(HEADER), "-I",
                            "/opt/rocm/include", cpp], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr


def dual(**kw):
    a = dict(q=P16, cache=P16, nblocks=4, bs=64, stride=64 * 352, idx=P16, topk=128,
             xcache=P256, xnblocks=100, xbs=2, xstride=2 * 352, xidx=P16, xtopk=512,
             batch=2, s_q=1, h_q=16, sink=NULL, scale=0.04, out=P16, lse=P16, ws=NULL,
             ws_bytes=0, splits=1, stream=NULL)
    a.update(kw)
    return m.lib().nvfp4_mla_sparse_decode_dual(
        a["q"], a["cache"], a["nblocks"], a["bs"], a["stride"], a["idx"], a["topk"],
        a["xcache"], a["xnblocks"], a["xbs"], a["xstride"], a["xidx"], a["xtopk"],
        a["batch"], a["s_q"], a["h_q"], a["sink"], a["scale"], a["out"], a["lse"], a["ws"],
        a["ws_bytes"], a["splits"], a["stream"])


@pytest.mark.parametrize("kw, needle", [
    (dict(topk=-1), "[0, 65536]"),
    (dict(xtopk=-5), "[0, 65536]"),
    (dict(xtopk=70000), "[0, 65536]"),
    (dict(topk=0, xtopk=0), "topk"),
    (dict(topk=60000, xtopk=6000), "topk"),
    (dict(xcache=NULL), "extra cache: kv_cache is NULL"),
    (dict(xstride=2 * 352 + 8), "extra cache"),
    (dict(xstride=352), "extra cache"),
    (dict(xbs=0), "extra cache"),
    (dict(cache=NULL), "kv_cache is NULL"),
    (dict(idx=NULL), "non-NULL"),
    (dict(xidx=NULL), "non-NULL"),
    (dict(xidx=ctypes.c_void_p(0x100002)), "aligned"),
    (dict(h_q=24), "multiple of 16"),
    (dict(splits=65), "num_splits"),
])
def test_sparse_decode_dual_rejects_bad_arguments(kw, needle):
    assert dual(**kw) == m.ERR_INVALID_ARGUMENT
    assert needle in m.last_error()


def test_sparse_decode_dual_accepts_an_empty_list_with_a_null_pointer():
    if torch.cuda.device_count() > 0:
        pytest.skip("device-gate check is for GPU-less hosts")
    assert dual(topk=0, idx=NULL) == m.ERR_UNSUPPORTED_DEVICE
    assert dual(xtopk=0, xidx=NULL) == m.ERR_UNSUPPORTED_DEVICE


def test_combine_and_gather_reject_bad_arguments():
    lib = m.lib()
    assert lib.nvfp4_mla_combine(P16, P16, 0, 4, 16, NULL, P16, P16, NULL) == m.ERR_INVALID_ARGUMENT
    assert lib.nvfp4_mla_combine(P16, P16, 2, -1, 16, NULL, P16, P16, NULL) == m.ERR_INVALID_ARGUMENT
    assert lib.nvfp4_mla_combine(NULL, P16, 2, 4, 16, NULL, P16, P16, NULL) == m.ERR_INVALID_ARGUMENT
    # 2^20 rows x 64 heads x 64 work-items exceeds one launch
    assert lib.nvfp4_mla_combine(P16, P16, 2, 2 ** 20, 64, NULL, P16, P16, NULL) == m.ERR_INVALID_ARGUMENT
    assert "too large" in m.last_error()
    assert lib.nvfp4_mla_dequantize_gather(P16, 4, 64, 64 * 352, P16, -1, P16, NULL) == m.ERR_INVALID_ARGUMENT
    assert lib.nvfp4_mla_dequantize_gather(P16, 4, 64, 64 * 352, NULL, 3, P16, NULL) == m.ERR_INVALID_ARGUMENT
    assert lib.nvfp4_mla_dequantize_gather(P16, 4, 64, 64 * 352, P16, 3,
                                           ctypes.c_void_p(0x100008), NULL) == m.ERR_INVALID_ARGUMENT
    assert lib.nvfp4_mla_dequantize_gather(P16, 4, 64, 64 * 352, ctypes.c_void_p(0x100002), 3,
                                           P16, NULL) == m.ERR_INVALID_ARGUMENT
    assert "slots 4-byte aligned" in m.last_error()
    out = ctypes.c_int32(0)
    assert lib.nvfp4_mla_sparse_decode_plan(1, 1, 12, 64, ctypes.byref(out)) == m.ERR_INVALID_ARGUMENT
    assert lib.nvfp4_mla_sparse_decode_plan(1, 1, 16, 64, None) == m.ERR_INVALID_ARGUMENT
    assert lib.nvfp4_mla_sparse_decode_workspace_size(1, 1, 16, 64, 99) == 0
    assert "num_splits" in m.last_error()


def test_workspace_size_for_explicit_splits():
    lib = m.lib()
    assert lib.nvfp4_mla_sparse_decode_workspace_size(4, 2, 16, 640, 1) == 0
    rows, h, s = 8, 16, 3
    al = lambda x: ((x + 255) // 256) * 256
    o = s * rows * h * 512 * 4                 # partial O
    lse = s * rows * h * 4                     # partial LSE
    assert lib.nvfp4_mla_sparse_decode_workspace_size(4, 2, 16, 640, s) == al(o) + al(lse)


def test_empty_inputs_are_no_ops_after_validation():
    # zero tokens / zero rows are valid; without a GPU the device gate answers
    if torch.cuda.device_count() > 0:
        pytest.skip("device-gate check is for GPU-less hosts")
    assert qa(n=0) == m.ERR_UNSUPPORTED_DEVICE
    assert "device" in m.last_error()


def test_valid_calls_without_a_gpu_report_the_device_gate():
    if torch.cuda.device_count() > 0:
        pytest.skip("device-gate check is for GPU-less hosts")
    assert qa() == m.ERR_UNSUPPORTED_DEVICE
    assert dec() == m.ERR_UNSUPPORTED_DEVICE
    out = ctypes.c_int32(0)
    assert m.lib().nvfp4_mla_sparse_decode_plan(1, 1, 16, 64, ctypes.byref(out)) == m.ERR_UNSUPPORTED_DEVICE


def test_workspace_too_small_is_its_own_error():
    if torch.cuda.device_count() > 0:
        pytest.skip("uses placeholder pointers; GPU-less hosts only")
    # the device gate comes before the workspace check, so on a GPU-less host
    # this reports the gate; the dedicated code is exercised in the GPU tests
    assert dec(splits=4, ws=NULL, ws_bytes=0) == m.ERR_UNSUPPORTED_DEVICE


def _decode_args():
    q = torch.zeros((2, 1, 16, 576), dtype=torch.bfloat16)
    cache = torch.zeros((4, 64, 352), dtype=torch.uint8)
    idx = torch.zeros((2, 1, 8), dtype=torch.int32)
    return q, cache, idx


META = torch.device("meta")


@pytest.mark.parametrize("change, needle", [
    (dict(out=torch.zeros((2, 1, 16, 256), dtype=torch.bfloat16)), "out must be"),
    (dict(out=torch.zeros((2, 1, 16, 512), dtype=torch.float32)), "out must be"),
    (dict(lse=torch.zeros((2, 1, 16), dtype=torch.float16)), "lse must be"),
    (dict(lse=torch.zeros((2, 16), dtype=torch.float32)), "lse must be"),
    (dict(kv_cache=torch.zeros((4, 64, 352), dtype=torch.uint8, device=META)), "kv_cache is on meta"),
    (dict(indices=torch.zeros((2, 1, 8), dtype=torch.int32, device=META)), "indices is on meta"),
    (dict(sink=torch.zeros(16, dtype=torch.float32, device=META)), "sink is on meta"),
    (dict(workspace=torch.zeros(1024, dtype=torch.uint8, device=META)), "workspace is on meta"),
    # a strided view: the kernels read sink[h] as consecutive floats
    (dict(sink=torch.zeros((16, 2), dtype=torch.float32)[:, 0]), "contiguous float32"),
])
def test_binding_checks_caller_tensors_before_any_library_call(change, needle):
    """The library takes raw pointers, so a tensor of the wrong shape, dtype
    or device would be read or written out of bounds; the binding refuses it
    first (on a machine without a GPU too: no library call is reached)."""
    q, cache, idx = _decode_args()
    kw = dict(q=q, kv_cache=cache, indices=idx, softmax_scale=0.1)
    kw.update(change)
    with pytest.raises(ValueError, match=needle):
        m.sparse_decode(**kw)


def test_binding_checks_dual_combine_append_and_gather_tensors():
    q, cache, idx = _decode_args()
    with pytest.raises(ValueError, match="extra_indices is on meta"):
        m.sparse_decode_dual(q, cache, idx, cache, idx.to(META), 0.1)
    with pytest.raises(ValueError, match="extra_kv_cache is on meta"):
        m.sparse_decode_dual(q, cache, idx, cache.to(META), idx, 0.1)
    o = torch.zeros((2, 3, 16, 512), dtype=torch.float32)
    with pytest.raises(ValueError, match="lse_partial"):
        m.combine(o, torch.zeros((2, 3, 8), dtype=torch.float32))
    with pytest.raises(ValueError, match="o_partial"):
        m.combine(o.half(), torch.zeros((2, 3, 16), dtype=torch.float32))
    with pytest.raises(ValueError, match="out must be"):
        m.combine(o, torch.zeros((2, 3, 16)), out=torch.zeros((3, 16, 512), dtype=torch.float32))
    with pytest.raises(ValueError, match="sink"):
        m.combine(o, torch.zeros((2, 3, 16)), sink=torch.zeros(8))
    with pytest.raises(ValueError, match="contiguous float32"):
        m.combine(o, torch.zeros((2, 3, 16)), sink=torch.zeros((16, 2))[:, 1])
    with pytest.raises(ValueError, match="contiguous float32"):
        m.sparse_decode_dual(q, cache, idx, cache, idx, 0.1,
                             sink=torch.zeros((16, 3), dtype=torch.float32)[:, 2])
    lat = torch.zeros((4, 512), dtype=torch.bfloat16)
    rope = torch.zeros((4, 64), dtype=torch.bfloat16)
    slots = torch.zeros(4, dtype=torch.int64)
    with pytest.raises(ValueError, match=r"\[N, >=512\]"):
        m.quantize_append(lat[:, :256], rope, slots, cache)
    with pytest.raises(ValueError, match="slot_mapping is on meta"):
        m.quantize_append(lat, rope, slots.to(META), cache)
    with pytest.raises(ValueError, match="out must be"):
        m.dequantize_gather(cache, torch.zeros(4, dtype=torch.int32),
                            out=torch.zeros((4, 512), dtype=torch.bfloat16))


def test_the_package_never_imports_the_oracle():
    # the product path (package import, library load, argument checks) runs
    # with no oracle module loaded, and no package source names one
    import subprocess
    import sys
    code = ("import sys, sparse_mla_decode_nvfp4_amd as m; m.lib(); m.check_format(); "
            "import sparse_mla_decode_nvfp4_amd.workloads; "
            "bad = [k for k in sys.modules if k == 'oracle' or k.startswith('oracle.')]; "
            "assert not bad, bad")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    pkg = os.path.join(ROOT, "sparse_mla_decode_nvfp4_amd")
    for name in os.listdir(pkg):
        if name.endswith(".py"):
            text = open(os.path.join(pkg, name)).read()
            assert not re.search(r"^\s*(import|from)\s+oracle\b", text, flags=re.M), name


def test_a_missing_library_fails_loudly():
    # no fallback: with the shared library absent every call raises
    import subprocess
    import sys
    code = ("import sparse_mla_decode_nvfp4_amd as m; m.LIB_PATH = '/nonexistent/libnvfp4_mla.so'\n"
            "try:\n    m.abi_version()\nexcept m.NativeLibraryMissing as e:\n    print('raised', e)\n"
            "else:\n    raise SystemExit('no error')")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True)
    assert r.returncode == 0 and "raised" in r.stdout, r.stdout + r.stderr
