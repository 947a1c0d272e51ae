"""MI355X (gfx950) NVFP4 sparse-MLA decode: thin Python binding.

Every step of the path runs in the HIP kernels of libnvfp4_mla.so behind the C
ABI declared in include/nvfp4_mla.h; this module only marshals torch tensors
(device memory and the current stream) into those calls and turns error codes
into exceptions.  There is no fallback: if the library is not built, or the
device is not gfx950, every call raises.

Build the library with ``python -m sparse_mla_decode_nvfp4_amd.build``.
"""

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libnvfp4_mla.so")

RECORD_BYTES = 352            # "nvfp4.fp8rope" record
DS_MLA_RECORD_BYTES = 432     # "nvfp4_ds_mla" record (the *_ds_mla exports)
NOPE_DIM = 512
ROPE_DIM = 64
QK_DIM = 576
V_DIM = 512
MAX_SPLITS = 64

OK = 0
ERR_INVALID_ARGUMENT = -1
ERR_UNSUPPORTED_FORMAT = -2
ERR_UNSUPPORTED_DEVICE = -3
ERR_WORKSPACE_TOO_SMALL = -4
ERR_HIP = -5

# exported symbol -> (restype, argtypes)
_P, _I32, _I64, _SZ, _F32 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                             ctypes.c_size_t, ctypes.c_float)
SIGNATURES = {
    "nvfp4_mla_abi_version": (ctypes.c_int, []),
    "nvfp4_mla_last_error": (ctypes.c_char_p, []),
    "nvfp4_mla_check_format": (ctypes.c_int, [_I32, _I32, _I32, _I32]),
    "nvfp4_mla_quantize_append": (ctypes.c_int, [_P, _I64, _P, _I64, _P, _I64, _P, _I64, _I32,
                                                 _I64, _P]),
    "nvfp4_mla_quantize_append_fp16": (ctypes.c_int, [_P, _I64, _P, _I64, _P, _I64, _P, _I64,
                                                      _I32, _I64, _P]),
    "nvfp4_mla_dequantize_gather": (ctypes.c_int, [_P, _I64, _I32, _I64, _P, _I64, _P, _P]),
    "nvfp4_mla_sparse_decode_plan": (ctypes.c_int, [_I32, _I32, _I32, _I32,
                                                    ctypes.POINTER(ctypes.c_int32)]),
    "nvfp4_mla_sparse_decode_workspace_size": (_SZ, [_I32, _I32, _I32, _I32, _I32]),
    "nvfp4_mla_sparse_decode": (ctypes.c_int, [_P, _P, _I64, _I32, _I64, _P, _I32, _I32, _I32,
                                               _I32, _P, _F32, _P, _P, _P, _SZ, _I32, _P]),
    "nvfp4_mla_sparse_decode_dual": (ctypes.c_int, [_P, _P, _I64, _I32, _I64, _P, _I32,
                                                    _P, _I64, _I32, _I64, _P, _I32,
                                                    _I32, _I32, _I32, _P, _F32, _P, _P, _P, _SZ,
                                                    _I32, _P]),
    "nvfp4_mla_sparse_decode_noalloc": (ctypes.c_int, [_P, _P, _I64, _I32, _I64, _P, _I32, _I32,
                                                       _I32, _I32, _P, _F32, _P, _P, _I32, _P]),
    "nvfp4_mla_norm_rope_quantize_append": (ctypes.c_int, [_P, _I64, _P, _I64, _P, _F32, _P, _I64,
                                                           _P, _I32, _P, _I64, _P, _I64, _I32,
                                                           _I64, _P]),
    "nvfp4_mla_norm_rope_quantize_append_ds_mla": (ctypes.c_int, [_P, _I64, _P, _I64, _P, _F32, _P,
                                                                  _I64, _P, _I32, _P, _I64, _P,
                                                                  _I64, _I32, _I64, _P]),
    "nvfp4_mla_norm_rope_f32": (ctypes.c_int, [_P, _I64, _P, _I64, _P, _F32, _P, _I64, _P, _I32,
                                               _I64, _P, _P]),
    "nvfp4_mla_quantize_append_ds_mla": (ctypes.c_int, [_P, _I64, _P, _I64, _P, _I64, _P,
                                                        _I64, _I32, _I64, _P]),
    "nvfp4_mla_dequantize_gather_ds_mla": (ctypes.c_int, [_P, _I64, _I32, _I64, _P, _I64, _P,
                                                          _P]),
    "nvfp4_mla_sparse_decode_ds_mla": (ctypes.c_int, [_P, _P, _I64, _I32, _I64, _P, _I32, _I32,
                                                      _I32, _I32, _P, _F32, _P, _P, _P, _SZ,
                                                      _I32, _P]),
    "nvfp4_mla_sparse_decode_dual_ds_mla": (ctypes.c_int, [_P, _P, _I64, _I32, _I64, _P, _I32,
                                                           _P, _I64, _I32, _I64, _P, _I32,
                                                           _I32, _I32, _I32, _P, _F32, _P, _P,
                                                           _P, _SZ, _I32, _P]),
    "nvfp4_mla_combine": (ctypes.c_int, [_P, _P, _I32, _I64, _I32, _P, _P, _P, _P]),
}

_lib_handle = None


class NativeLibraryMissing(ImportError):
    pass


class Nvfp4MlaError(RuntimeError):
    def __init__(self, fn, code, msg):
        super().__init__(f"{fn} failed with status {code}: {msg}")
        self.code = code


def lib():
    """The loaded C library (loads it on first use; raises if not built)."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise NativeLibraryMissing(
                f"{LIB_PATH} is not built; run python -m sparse_mla_decode_nvfp4_amd.build")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _lib_handle = h
    return _lib_handle


def last_error():
    return lib().nvfp4_mla_last_error().decode()


def _check(fn, code):
    if code != OK:
        raise Nvfp4MlaError(fn, code, last_error())


def abi_version():
    return lib().nvfp4_mla_abi_version()


def check_format(record_bytes=RECORD_BYTES, nope_dim=NOPE_DIM, rope_dim=ROPE_DIM, v_dim=V_DIM):
    _check("nvfp4_mla_check_format",
           lib().nvfp4_mla_check_format(record_bytes, nope_dim, rope_dim, v_dim))


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _same_device(device, **tensors):
    """Raises unless every given tensor (None skipped) is on `device`: the
    library receives raw pointers and cannot tell host from device memory."""
    for name, t in tensors.items():
        if t is not None and t.device != device:
            raise ValueError(f"{name} is on {t.device}; expected {device}")


def _check_sink(sink, h):
    """The sink is read as h_q consecutive floats: a strided view would hand
    the kernels the wrong values."""
    if sink is not None and (sink.dtype != torch.float32 or sink.numel() != h
                             or not sink.is_contiguous()):
        raise ValueError("sink must be a contiguous float32 [H] tensor")


def _outputs(out, lse, shape, device):
    """Caller-supplied or new O (bf16 [*shape, 512]) and LSE (float32 shape)."""
    if out is None:
        out = torch.empty((*shape, V_DIM), dtype=torch.bfloat16, device=device)
    elif (out.dtype != torch.bfloat16 or tuple(out.shape) != (*shape, V_DIM)
          or not out.is_contiguous()):
        raise ValueError(f"out must be a contiguous bf16 {[*shape, V_DIM]} tensor")
    if lse is None:
        lse = torch.empty(shape, dtype=torch.float32, device=device)
    elif lse.dtype != torch.float32 or tuple(lse.shape) != tuple(shape) or not lse.is_contiguous():
        raise ValueError(f"lse must be a contiguous float32 {list(shape)} tensor")
    return out, lse


def _workspace_bytes(workspace):
    if workspace is None:
        return 0
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    return workspace.numel() * workspace.element_size()


def _cache_geometry(kv_cache):
    """(num_blocks, block_size, block_stride_bytes) of a [blocks, block_size,
    R] uint8 cache tensor, R = 352 or 432 (pages may be padded: stride(0) >=
    block_size * R)."""
    if (kv_cache.dtype != torch.uint8 or kv_cache.dim() != 3
            or kv_cache.shape[2] not in (RECORD_BYTES, DS_MLA_RECORD_BYTES)):
        raise ValueError("kv_cache must be a uint8 tensor [num_blocks, block_size, 352 or 432]")
    r = kv_cache.shape[2]
    if kv_cache.stride(2) != 1 or kv_cache.stride(1) != r:
        raise ValueError(f"records within a page must be contiguous {r}-byte rows")
    return kv_cache.shape[0], kv_cache.shape[1], kv_cache.stride(0)


def _ds(kv_cache):
    """Export-name suffix for the cache's record: '' or '_ds_mla'."""
    return "_ds_mla" if kv_cache.shape[2] == DS_MLA_RECORD_BYTES else ""


def new_cache(num_blocks, block_size, device="cuda", fill=0, record_bytes=RECORD_BYTES):
    """A zero-filled (or `fill`-filled) paged cache [num_blocks, block_size,
    record_bytes] (352 or 432)."""
    if record_bytes not in (RECORD_BYTES, DS_MLA_RECORD_BYTES):
        raise ValueError("record_bytes must be 352 or 432")
    return torch.full((num_blocks, block_size, record_bytes), fill, dtype=torch.uint8,
                      device=device)


def quantize_append(latent, rope, slot_mapping, kv_cache):
    """Writes NVFP4 records for each token with slot_mapping >= 0, in place.

    latent: bf16 or fp16 [N, >=512] (rows 16-byte aligned), rope: the same
    dtype [N, >=64], slot_mapping: int64 [N], kv_cache: uint8 [num_blocks,
    block_size, 352 or 432].  The 432-byte record takes bf16 only.
    """
    n = latent.shape[0]
    if latent.dtype not in (torch.bfloat16, torch.float16) or rope.dtype != latent.dtype:
        raise ValueError("latent and rope must both be bfloat16 or both float16")
    if slot_mapping.dtype != torch.int64 or slot_mapping.numel() != n or rope.shape[0] != n:
        raise ValueError("slot_mapping must be int64 [N] matching latent/rope rows")
    if latent.stride(-1) != 1 or rope.stride(-1) != 1 or not slot_mapping.is_contiguous():
        raise ValueError("inner dimensions must be contiguous")
    if latent.dim() != 2 or rope.dim() != 2 or latent.shape[1] < NOPE_DIM or rope.shape[1] < ROPE_DIM:
        raise ValueError("latent must be [N, >=512] and rope [N, >=64]")
    _same_device(kv_cache.device, latent=latent, rope=rope, slot_mapping=slot_mapping)
    nb, bs, stride = _cache_geometry(kv_cache)
    if _ds(kv_cache):
        if latent.dtype != torch.bfloat16:
            raise ValueError("the 432-byte record stores bf16 RoPE: inputs must be bfloat16")
        fn = "nvfp4_mla_quantize_append_ds_mla"
    else:
        fn = "nvfp4_mla_quantize_append" + ("_fp16" if latent.dtype == torch.float16 else "")
    code = getattr(lib(), fn)(
        _ptr(latent), latent.stride(0), _ptr(rope), rope.stride(0), _ptr(slot_mapping), n,
        _ptr(kv_cache), nb, bs, stride, _stream(kv_cache.device))
    _check(fn, code)
    return kv_cache


def _norm_rope_inputs(latent, rope, norm_weight, cos_sin, positions, device):
    """Checks the fused write path's tensors; returns the token count."""
    n = latent.shape[0]
    if latent.dtype != torch.bfloat16 or rope.dtype != torch.bfloat16:
        raise ValueError("latent and rope must be bfloat16")
    if latent.dim() != 2 or rope.dim() != 2 or latent.shape[1] < NOPE_DIM or rope.shape[1] < ROPE_DIM:
        raise ValueError("latent must be [N, >=512] and rope [N, >=64]")
    if rope.shape[0] != n or latent.stride(-1) != 1 or rope.stride(-1) != 1:
        raise ValueError("latent and rope need N rows with contiguous inner dimensions")
    if (norm_weight.dtype != torch.bfloat16 or norm_weight.numel() != NOPE_DIM
            or not norm_weight.is_contiguous()):
        raise ValueError("norm_weight must be a contiguous bfloat16 [512] tensor")
    if (cos_sin.dtype != torch.float32 or cos_sin.dim() != 2 or cos_sin.shape[1] != ROPE_DIM
            or not cos_sin.is_contiguous()):
        raise ValueError("cos_sin must be a contiguous float32 [max_position, 64] tensor")
    if positions.dtype != torch.int64 or positions.numel() != n or not positions.is_contiguous():
        raise ValueError("positions must be a contiguous int64 [N] tensor")
    _same_device(device, latent=latent, rope=rope, norm_weight=norm_weight, cos_sin=cos_sin,
                 positions=positions)
    return n


def norm_rope_quantize_append(latent, rope, norm_weight, eps, cos_sin, positions, slot_mapping,
                              kv_cache, neox=False):
    """Fused write path, in place: RMSNorm(latent) * norm_weight and the
    rotary turn of `rope` by the rows positions[n] of cos_sin ([max_position,
    64] float32: 32 cosines, then 32 sines; pairs (2i, 2i+1), or (i, i+32)
    when neox), both rounded to bf16, then quantized into the records at
    slot_mapping.  Tokens with slot -1 or a position outside the table are
    skipped."""
    n = _norm_rope_inputs(latent, rope, norm_weight, cos_sin, positions, kv_cache.device)
    if slot_mapping.dtype != torch.int64 or slot_mapping.numel() != n or not slot_mapping.is_contiguous():
        raise ValueError("slot_mapping must be a contiguous int64 [N] tensor")
    _same_device(kv_cache.device, slot_mapping=slot_mapping)
    nb, bs, stride = _cache_geometry(kv_cache)
    fn = "nvfp4_mla_norm_rope_quantize_append" + _ds(kv_cache)
    code = getattr(lib(), fn)(
        _ptr(latent), latent.stride(0), _ptr(rope), rope.stride(0), _ptr(norm_weight),
        float(eps), _ptr(cos_sin), cos_sin.shape[0], _ptr(positions), int(bool(neox)),
        _ptr(slot_mapping), n, _ptr(kv_cache), nb, bs, stride, _stream(kv_cache.device))
    _check(fn, code)
    return kv_cache


def norm_rope_f32(latent, rope, norm_weight, eps, cos_sin, positions, neox=False, out=None):
    """float32 [N, 576]: the fused path's normalised latent and turned RoPE
    before their bf16 rounding (test export)."""
    n = _norm_rope_inputs(latent, rope, norm_weight, cos_sin, positions, latent.device)
    if out is None:
        out = torch.empty((n, QK_DIM), dtype=torch.float32, device=latent.device)
    elif out.dtype != torch.float32 or tuple(out.shape) != (n, QK_DIM) or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous float32 [{n}, {QK_DIM}] tensor")
    _same_device(latent.device, out=out)
    code = lib().nvfp4_mla_norm_rope_f32(
        _ptr(latent), latent.stride(0), _ptr(rope), rope.stride(0), _ptr(norm_weight),
        float(eps), _ptr(cos_sin), cos_sin.shape[0], _ptr(positions), int(bool(neox)), n,
        _ptr(out), _stream(latent.device))
    _check("nvfp4_mla_norm_rope_f32", code)
    return out


def dequantize_gather(kv_cache, slots, out=None):
    """bf16 [n, 576] dequantized keys of the records at `slots` (int32)."""
    if slots.dtype != torch.int32 or not slots.is_contiguous():
        raise ValueError("slots must be a contiguous int32 tensor")
    n = slots.numel()
    if out is None:
        out = torch.empty((n, QK_DIM), dtype=torch.bfloat16, device=kv_cache.device)
    elif out.dtype != torch.bfloat16 or tuple(out.shape) != (n, QK_DIM) or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous bf16 [{n}, {QK_DIM}] tensor")
    _same_device(kv_cache.device, slots=slots, out=out)
    nb, bs, stride = _cache_geometry(kv_cache)
    fn = "nvfp4_mla_dequantize_gather" + _ds(kv_cache)
    code = getattr(lib(), fn)(_ptr(kv_cache), nb, bs, stride, _ptr(slots), n,
                              _ptr(out), _stream(kv_cache.device))
    _check(fn, code)
    return out


def plan(batch, s_q, h_q, topk):
    out = ctypes.c_int32(0)
    _check("nvfp4_mla_sparse_decode_plan",
           lib().nvfp4_mla_sparse_decode_plan(batch, s_q, h_q, topk, ctypes.byref(out)))
    return out.value


def workspace_size(batch, s_q, h_q, topk, num_splits=0):
    """Bytes of decode workspace (no initialisation needed; reusable)."""
    n = lib().nvfp4_mla_sparse_decode_workspace_size(batch, s_q, h_q, topk, num_splits)
    err = last_error()
    if err:
        raise Nvfp4MlaError("nvfp4_mla_sparse_decode_workspace_size", ERR_INVALID_ARGUMENT, err)
    return n


def sparse_decode(q, kv_cache, indices, softmax_scale, sink=None, num_splits=0,
                  workspace=None, out=None, lse=None):
    """Sparse MLA decode.  q: bf16 [B, S_q, H, 576]; indices: int32 [B, S_q, topk]
    slot ids (< 0 invalid); sink: float32 [H] or None.  Returns (O bf16
    [B, S_q, H, 512], LSE float32 [B, S_q, H])."""
    if q.dtype != torch.bfloat16 or q.dim() != 4 or q.shape[-1] != QK_DIM or not q.is_contiguous():
        raise ValueError("q must be a contiguous bf16 [B, S_q, H, 576] tensor")
    b, s, h, _ = q.shape
    if (indices.dtype != torch.int32 or indices.dim() != 3 or tuple(indices.shape[:2]) != (b, s)
            or not indices.is_contiguous()):
        raise ValueError("indices must be a contiguous int32 [B, S_q, topk] tensor")
    topk = indices.shape[2]
    _check_sink(sink, h)
    out, lse = _outputs(out, lse, (b, s, h), q.device)
    _same_device(q.device, kv_cache=kv_cache, indices=indices, sink=sink, workspace=workspace,
                 out=out, lse=lse)
    if num_splits == 0:
        num_splits = plan(b, s, h, topk)
    need = workspace_size(b, s, h, topk, num_splits)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    nb, bs, stride = _cache_geometry(kv_cache)
    fn = "nvfp4_mla_sparse_decode" + _ds(kv_cache)
    code = getattr(lib(), fn)(
        _ptr(q), _ptr(kv_cache), nb, bs, stride, _ptr(indices), b, s, h, topk, _ptr(sink),
        float(softmax_scale), _ptr(out), _ptr(lse), _ptr(workspace),
        _workspace_bytes(workspace), num_splits, _stream(q.device))
    _check(fn, code)
    return out, lse


def sparse_decode_noalloc(q, kv_cache, indices, softmax_scale, sink=None, num_splits=0,
                          out=None, lse=None):
    """The decode of sparse_decode through the allocation-free entry point:
    split partials live in the library's static per-GPU scratch array, so no
    workspace is passed (or allocated here when out and lse are given).
    352-byte records only.  Calls that may overlap on one GPU race on that
    array.  Returns (O, LSE) as sparse_decode does."""
    if q.dtype != torch.bfloat16 or q.dim() != 4 or q.shape[-1] != QK_DIM or not q.is_contiguous():
        raise ValueError("q must be a contiguous bf16 [B, S_q, H, 576] tensor")
    b, s, h, _ = q.shape
    topk = _index_list(indices, b, s, "indices")
    _check_sink(sink, h)
    out, lse = _outputs(out, lse, (b, s, h), q.device)
    _same_device(q.device, kv_cache=kv_cache, indices=indices, sink=sink, out=out, lse=lse)
    nb, bs, stride = _cache_geometry(kv_cache)
    if _ds(kv_cache):
        raise ValueError("the allocation-free entry point reads 352-byte records")
    code = lib().nvfp4_mla_sparse_decode_noalloc(
        _ptr(q), _ptr(kv_cache), nb, bs, stride, _ptr(indices), b, s, h, topk, _ptr(sink),
        float(softmax_scale), _ptr(out), _ptr(lse), num_splits, _stream(q.device))
    _check("nvfp4_mla_sparse_decode_noalloc", code)
    return out, lse


def _index_list(indices, b, s, what):
    if (indices.dtype != torch.int32 or indices.dim() != 3 or tuple(indices.shape[:2]) != (b, s)
            or not indices.is_contiguous()):
        raise ValueError(f"{what} must be a contiguous int32 [B, S_q, topk] tensor")
    return indices.shape[2]


def sparse_decode_dual(q, kv_cache, indices, extra_kv_cache, extra_indices, softmax_scale,
                       sink=None, num_splits=0, workspace=None, out=None, lse=None):
    """Dual-cache sparse MLA decode: one softmax over `indices` (slot ids of
    kv_cache) and `extra_indices` (slot ids of extra_kv_cache), each cache
    with its own page size.  Shapes as for sparse_decode; either list may have
    top-k 0.  Returns (O bf16 [B, S_q, H, 512], LSE float32 [B, S_q, H])."""
    if q.dtype != torch.bfloat16 or q.dim() != 4 or q.shape[-1] != QK_DIM or not q.is_contiguous():
        raise ValueError("q must be a contiguous bf16 [B, S_q, H, 576] tensor")
    b, s, h, _ = q.shape
    topk0 = _index_list(indices, b, s, "indices")
    topk1 = _index_list(extra_indices, b, s, "extra_indices")
    _check_sink(sink, h)
    out, lse = _outputs(out, lse, (b, s, h), q.device)
    _same_device(q.device, kv_cache=kv_cache, indices=indices, extra_kv_cache=extra_kv_cache,
                 extra_indices=extra_indices, sink=sink, workspace=workspace, out=out, lse=lse)
    if num_splits == 0:
        num_splits = plan(b, s, h, topk0 + topk1)
    need = workspace_size(b, s, h, topk0 + topk1, num_splits)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    nb0, bs0, st0 = _cache_geometry(kv_cache)
    nb1, bs1, st1 = _cache_geometry(extra_kv_cache)
    if kv_cache.shape[2] != extra_kv_cache.shape[2]:
        raise ValueError("both caches must hold the same record (352 or 432 bytes)")
    fn = "nvfp4_mla_sparse_decode_dual" + _ds(kv_cache)
    code = getattr(lib(), fn)(
        _ptr(q), _ptr(kv_cache), nb0, bs0, st0, _ptr(indices) if topk0 else None, topk0,
        _ptr(extra_kv_cache), nb1, bs1, st1, _ptr(extra_indices) if topk1 else None, topk1,
        b, s, h, _ptr(sink), float(softmax_scale), _ptr(out), _ptr(lse), _ptr(workspace),
        _workspace_bytes(workspace), num_splits, _stream(q.device))
    _check(fn, code)
    return out, lse


def combine(o_partial, lse_partial, sink=None, out=None, lse=None):
    """LSE-weighted merge.  o_partial float32 [P, R, H, 512], lse_partial float32
    [P, R, H].  Returns (O bf16 [R, H, 512], LSE float32 [R, H])."""
    if o_partial.dtype != torch.float32 or o_partial.dim() != 4 or o_partial.shape[-1] != V_DIM:
        raise ValueError("o_partial must be float32 [P, R, H, 512]")
    p, r, h, _ = o_partial.shape
    if lse_partial.dtype != torch.float32 or tuple(lse_partial.shape) != (p, r, h):
        raise ValueError("lse_partial must be float32 [P, R, H] matching o_partial")
    _check_sink(sink, h)
    o_partial = o_partial.contiguous()
    lse_partial = lse_partial.contiguous()
    out, lse = _outputs(out, lse, (r, h), o_partial.device)
    _same_device(o_partial.device, lse_partial=lse_partial, sink=sink, out=out, lse=lse)
    code = lib().nvfp4_mla_combine(_ptr(o_partial), _ptr(lse_partial),
                                   p, r, h, _ptr(sink), _ptr(out), _ptr(lse),
                                   _stream(o_partial.device))
    _check("nvfp4_mla_combine", code)
    return out, lse
