"""fp8_e4m3_paged_kv_amd -- FP8 E4M3 paged KV cache for MI355X (gfx950).

A thin ctypes binding over ``libfp8kv.so`` (C ABI: ``include/fp8kv.h``).
It only marshals arguments -- pointers, strides, the current HIP stream --
and raises on a nonzero status; every step of the computation runs in the
library's HIP kernels. There is no fallback: if the library is missing the
import of any entry point raises.

Cache layout used by the helpers here:
  k_cache, v_cache   uint8  [num_slots, Hkv, D]  (or [num_blocks, bs, Hkv, D])
  k_scale, v_scale   fp32   any 2-D view [num_slots, Hkv] -- including a
                     transposed view of a head-major [Hkv, num_slots] plane
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfp8kv.so")

DTYPE_BF16 = 1
DTYPE_FP16 = 2
DTYPE_FP32 = 3

KEYS_MXFP4 = 0
KEYS_E4M3 = 1
KEYS_BF16 = 2

_TORCH_DTYPE = {torch.bfloat16: DTYPE_BF16, torch.float16: DTYPE_FP16,
                torch.float32: DTYPE_FP32}

_lib = None


class Fp8KvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"fp8kv status {status}: {message}")
        self.status = status


def lib():
    """Load libfp8kv.so (built in-tree by ``python -m
    fp8_e4m3_paged_kv_amd.build``); raises if it is not there."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m fp8_e4m3_paged_kv_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    SZ = ctypes.c_size_t
    L.fp8kv_abi_version.restype = ctypes.c_int
    L.fp8kv_status_string.argtypes = [ctypes.c_int]
    L.fp8kv_status_string.restype = ctypes.c_char_p
    L.fp8kv_last_error.restype = ctypes.c_char_p
    L.fp8kv_set_checked.argtypes = [ctypes.c_int]
    L.fp8kv_set_checked.restype = ctypes.c_int
    L.fp8kv_kv_quant_scatter.argtypes = [P, I64, I64, P, I64, I64, I32, I32,
                                         I32, I32, P, P, P, I64, I64, P, P,
                                         I64, I64, I64, P]
    L.fp8kv_kv_quant_scatter.restype = ctypes.c_int
    dec = [P, I64, I64, I64, I32, P, P, I64, I64, P, P, I64, I64, I64, P, I64,
           P, I32, I32, I32, I32, I32, I32, F, I32, I32, P, SZ]
    L.fp8kv_paged_decode_attn_fp8.argtypes = dec + [P, I64, I64, I64, I32, P]
    L.fp8kv_paged_decode_attn_fp8.restype = ctypes.c_int
    L.fp8kv_paged_decode_append_attn_fp8.argtypes = (dec[:5] + [P, I64, I64, I64, P, I64, I64, I64, I32]
                                                      + dec[5:] + [P, I64, I64, I64, I32, P])
    L.fp8kv_paged_decode_append_attn_fp8.restype = ctypes.c_int
    L.fp8kv_paged_decode_append_partials.argtypes = (dec[:5] + [P, I64, I64, I64, P, I64, I64, I64, I32]
                                                      + dec[5:] + [P])
    L.fp8kv_paged_decode_append_partials.restype = ctypes.c_int
    L.fp8kv_paged_decode_attn_fp8_noalloc.argtypes = dec[:-2] + [P, I64, I64, I64, I32, P]
    L.fp8kv_paged_decode_attn_fp8_noalloc.restype = ctypes.c_int
    L.fp8kv_paged_decode_partials.argtypes = dec + [P]
    L.fp8kv_paged_decode_partials.restype = ctypes.c_int
    L.fp8kv_kv_quant_scatter_unscaled.argtypes = [P, I64, I64, P, I64, I64, I32, I32,
                                                  I32, I32, P, P, P, I64, I64, I64, I32, P]
    L.fp8kv_kv_quant_scatter_unscaled.restype = ctypes.c_int
    udec = dec[:9] + dec[13:]                 # no scale planes
    L.fp8kv_paged_decode_attn_unscaled.argtypes = udec + [P, I64, I64, I64, I32, I32, P]
    L.fp8kv_paged_decode_attn_unscaled.restype = ctypes.c_int
    L.fp8kv_paged_decode_partials_unscaled.argtypes = udec + [I32, P]
    L.fp8kv_paged_decode_partials_unscaled.restype = ctypes.c_int
    sdec = dec[:16] + [P, I64] + dec[16:]
    L.fp8kv_sparse_decode_attn_fp8.argtypes = sdec + [P, I64, I64, I64, I32, P]
    L.fp8kv_sparse_decode_attn_fp8.restype = ctypes.c_int
    L.fp8kv_sparse_decode_partials.argtypes = sdec + [P]
    L.fp8kv_sparse_decode_partials.restype = ctypes.c_int
    L.fp8kv_prefill_attn_fp8.argtypes = [P, I64, I64, I64, I32, P, P, I64, I64,
                                         P, P, I64, I64, I64, P, I64, P, P,
                                         I32, I32, I32, I32, I32, I32, F, I32,
                                         P, I64, I64, I64, I32, P]
    L.fp8kv_prefill_attn_fp8.restype = ctypes.c_int
    pre = L.fp8kv_prefill_attn_fp8.argtypes
    L.fp8kv_sparse_prefill_attn_fp8.argtypes = pre[:16] + [P, I64] + pre[16:]
    L.fp8kv_sparse_prefill_attn_fp8.restype = ctypes.c_int
    L.fp8kv_paged_decode_merge.argtypes = [I32, I32, I32, I32, I32, I32, P,
                                           SZ, P, I64, I64, I64, I32, P]
    L.fp8kv_paged_decode_merge.restype = ctypes.c_int
    L.fp8kv_paged_decode_workspace_bytes.argtypes = [I32] * 6
    L.fp8kv_paged_decode_workspace_bytes.restype = I64
    L.fp8kv_paged_decode_num_ranges.argtypes = [I32, I32]
    L.fp8kv_paged_decode_num_ranges.restype = I32
    L.fp8kv_index_keys_quantize.argtypes = [P, I64, I64, I32, I32, P, I64, P,
                                            I64, P]
    L.fp8kv_index_keys_quantize.restype = ctypes.c_int
    L.fp8kv_index_keys_build.argtypes = [P, I64, I64, I32, I64, I64, I32, I32,
                                         P, I64, I64, P, I64, I64, P]
    L.fp8kv_index_keys_build.restype = ctypes.c_int
    L.fp8kv_index_score_mxfp4.argtypes = [P, I64, I64, I64, I32, P, I64, I64,
                                          I64, I32, P, I64, I64, P, I64, I64,
                                          I32, I32, I32, I32, I32, I32, P,
                                          I64, I64, P]
    L.fp8kv_index_score_mxfp4.restype = ctypes.c_int
    _lib = L
    return L


def _check(status: int):
    if status != 0:
        L = lib()
        raise Fp8KvError(status, L.fp8kv_last_error().decode() or
                         L.fp8kv_status_string(status).decode())


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _dev(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("fp8kv: every tensor must live on the GPU")


def _cache_strides(cache: torch.Tensor):
    """(stride_slot, stride_head, S, H, D) of a uint8 [S, H, D] or
    [NB, bs, H, D] code buffer whose head_dim is contiguous."""
    if cache.dtype != torch.uint8:
        raise ValueError("code buffers are uint8")
    if cache.dim() == 4:
        nb, bs, H, D = cache.shape
        if cache.stride(0) != bs * cache.stride(1):
            raise ValueError("4-D cache: blocks must be evenly spaced slots")
        css, csh, S = cache.stride(1), cache.stride(2), nb * bs
    elif cache.dim() == 3:
        S, H, D = cache.shape
        css, csh = cache.stride(0), cache.stride(1)
    else:
        raise ValueError("cache must be [S, H, D] or [NB, bs, H, D]")
    if D > 1 and cache.stride(-1) != 1:
        raise ValueError("cache: head_dim must be the contiguous dimension")
    return css, csh, S, H, D


def _kv_caches(k_cache: torch.Tensor, v_cache: torch.Tensor):
    """Geometry of a K/V code-buffer pair: same shape and strides."""
    geom = _cache_strides(k_cache)
    if v_cache.shape != k_cache.shape or _cache_strides(v_cache)[:2] != geom[:2]:
        raise ValueError("k_cache and v_cache must share shape and strides")
    return geom


def _scale_strides(scale: torch.Tensor, S=None, H=None):
    """(stride_slot, stride_head) of an fp32 scale plane viewed as [S, H]
    or [NB, bs, H]; with S and H given, the plane must cover exactly the
    cache's S slots and H heads."""
    if scale.dtype != torch.float32:
        raise ValueError("scale planes are float32")
    if scale.dim() == 3:          # [NB, bs, H]
        nb, bs, h = scale.shape
        if nb > 1 and scale.stride(0) != bs * scale.stride(1):
            raise ValueError("3-D scale plane: blocks must be evenly spaced slots")
        shape, strides = (nb * bs, h), (scale.stride(1), scale.stride(2))
    elif scale.dim() == 2:        # [S, H]
        shape, strides = tuple(scale.shape), (scale.stride(0), scale.stride(1))
    else:
        raise ValueError("scale plane must be [S, H] or [NB, bs, H]")
    if S is not None and shape != (S, H):
        raise ValueError(f"scale plane covers {shape} (slots, heads), the cache ({S}, {H})")
    return strides


def _scale_pair(k_scale, v_scale, S, H):
    sss, ssh = _scale_strides(k_scale, S, H)
    if _scale_strides(v_scale, S, H) != (sss, ssh):
        raise ValueError("k_scale and v_scale must share strides")
    return sss, ssh


def _tables(block_tables, context_lens, B, block_size, max_context, extra=()):
    """Page tables and per-request lengths of B requests: every length the
    kernels use is clamped to max_context, so the tables must hold
    ceil(max_context / block_size) entries per request."""
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or \
            (block_tables.shape[1] > 1 and block_tables.stride(1) != 1):
        raise ValueError("block_tables must be int32 [B, max_blocks], rows contiguous")
    for t in (context_lens,) + tuple(extra):
        if t.dtype != torch.int32 or t.dim() != 1 or not t.is_contiguous():
            raise ValueError("context_lens / q_lens must be contiguous int32 [B]")
        if t.shape[0] != B:
            raise ValueError(f"context_lens / q_lens hold {t.shape[0]} entries for {B} requests")
    if block_size <= 0 or max_context < 0:
        raise ValueError("block_size must be positive and max_context >= 0")
    if B > 0 and block_tables.shape[0] < B:
        raise ValueError(f"block_tables has {block_tables.shape[0]} rows for {B} requests")
    if B > 0 and block_tables.shape[1] * block_size < max_context:
        raise ValueError(f"block_tables rows cover {block_tables.shape[1] * block_size} "
                         f"tokens, max_context is {max_context}")


def abi_version() -> int:
    return lib().fp8kv_abi_version()


def set_checked(enabled: bool) -> bool:
    """Switch the library's checked mode (process-wide) and return the
    previous setting. In checked mode every call also verifies that its
    pointers are device memory of the current device and range-checks the
    device-resident ids (slot ids, context lengths, page tables, valid
    counts, chunk lengths) on the host, synchronizing the stream; it is
    refused under graph capture."""
    return bool(lib().fp8kv_set_checked(1 if enabled else 0))


def kv_quant_scatter(k: torch.Tensor, v: torch.Tensor, slot_ids: torch.Tensor,
                     k_cache: torch.Tensor, v_cache: torch.Tensor,
                     k_scale: torch.Tensor, v_scale: torch.Tensor) -> None:
    """Quantize K and V ([T, Hkv, D] bf16 views, each at its own strides) to
    E4M3 + fp32 row scales and scatter them to ``slot_ids`` (int64 [T],
    device) in one launch. Slot ids < 0 or >= num_slots are skipped."""
    if k.shape != v.shape or k.dim() != 3:
        raise ValueError("k and v must both be [T, Hkv, D]")
    if k.dtype != v.dtype or k.dtype not in _TORCH_DTYPE:
        raise ValueError("k and v must share a float dtype")
    if k.stride(2) != 1 or v.stride(2) != 1:
        raise ValueError("head_dim must be the contiguous dimension")
    if slot_ids.dtype != torch.int64 or slot_ids.shape != (k.shape[0],):
        raise ValueError("slot_ids must be int64 [T]")
    if not slot_ids.is_contiguous():
        raise ValueError("slot_ids must be contiguous")
    css, csh, S, H, D = _kv_caches(k_cache, v_cache)
    sss, ssh = _scale_pair(k_scale, v_scale, S, H)
    T, Hk, Dk = k.shape
    if (Hk, Dk) != (H, D):
        raise ValueError("K/V head count or head_dim differs from the cache")
    _dev(k, v, slot_ids, k_cache, v_cache, k_scale, v_scale)
    _check(lib().fp8kv_kv_quant_scatter(
        k.data_ptr(), k.stride(0), k.stride(1),
        v.data_ptr(), v.stride(0), v.stride(1),
        _TORCH_DTYPE[k.dtype], T, H, D, slot_ids.data_ptr(),
        k_cache.data_ptr(), v_cache.data_ptr(), css, csh,
        k_scale.data_ptr(), v_scale.data_ptr(), sss, ssh, S,
        _stream(k.device)))


CODES_E4M3 = 0   # unscaled cache code formats
CODES_E5M2 = 1


def kv_quant_scatter_unscaled(k: torch.Tensor, v: torch.Tensor, slot_ids: torch.Tensor,
                              k_cache: torch.Tensor, v_cache: torch.Tensor,
                              code_format: int = CODES_E4M3) -> None:
    """Store K and V ([T, Hkv, D] bf16 views) as unscaled E4M3 or E5M2 codes
    (round to nearest even, saturating) at ``slot_ids``; no scale planes."""
    if k.dim() != 3 or v.shape != k.shape or k.dtype not in _TORCH_DTYPE or v.dtype != k.dtype:
        raise ValueError("k and v must be [T, Hkv, D] views of one float dtype")
    if k.stride(2) != 1 or v.stride(2) != 1:
        raise ValueError("head_dim must be the contiguous dimension")
    if slot_ids.dtype != torch.int64 or slot_ids.shape != (k.shape[0],) or \
            not slot_ids.is_contiguous():
        raise ValueError("slot_ids must be contiguous int64 [T]")
    css, csh, S, H, D = _kv_caches(k_cache, v_cache)
    T, Hk, Dk = k.shape
    if (Hk, Dk) != (H, D):
        raise ValueError("K/V head count or head_dim differs from the cache")
    _dev(k, v, slot_ids, k_cache, v_cache)
    _check(lib().fp8kv_kv_quant_scatter_unscaled(
        k.data_ptr(), k.stride(0), k.stride(1),
        v.data_ptr(), v.stride(0), v.stride(1),
        _TORCH_DTYPE[k.dtype], T, H, D, slot_ids.data_ptr(),
        k_cache.data_ptr(), v_cache.data_ptr(), css, csh, S,
        int(code_format), _stream(k.device)))


def decode_workspace_bytes(batch, rows, num_q_heads, num_kv_heads, head_dim,
                           num_ranges=0) -> int:
    """Workspace bytes of a decode call (num_ranges 0 = library choice)."""
    n = lib().fp8kv_paged_decode_workspace_bytes(
        batch, rows, num_q_heads, num_kv_heads, head_dim, int(num_ranges))
    if n < 0:
        _check(int(n))
    return int(n)


def decode_num_ranges(num_kv_heads, num_ranges=0) -> int:
    """The number of ranges each KV head's tile sequence is split into
    (resolves 0 on the current device)."""
    n = lib().fp8kv_paged_decode_num_ranges(num_kv_heads, int(num_ranges))
    if n < 0:
        _check(int(n))
    return int(n)


def _decode_args(q, k_cache, v_cache, k_scale, v_scale, block_tables,
                 context_lens, num_kv_heads, block_size, softmax_scale,
                 max_context, num_ranges, workspace, with_workspace=True):
    """Argument list of the scaled decode calls; with k_scale = v_scale =
    None that of the unscaled ones (no scale planes); with_workspace=False
    leaves out the workspace arguments (and allocates none)."""
    unscaled = k_scale is None and v_scale is None
    if q.dim() != 4 or q.stride(3) != 1:
        raise ValueError("q must be [B, R, Hq, D] with contiguous head_dim")
    if q.dtype not in _TORCH_DTYPE:
        raise ValueError("unsupported q dtype")
    B, R, Hq, D = q.shape
    css, csh, S, H, Dc = _kv_caches(k_cache, v_cache)
    if H != num_kv_heads or Dc != D:
        raise ValueError("cache geometry does not match q / num_kv_heads")
    if not unscaled:
        sss, ssh = _scale_pair(k_scale, v_scale, S, H)
    _tables(block_tables, context_lens, B, block_size, int(max_context))
    _dev(q, k_cache, v_cache, block_tables, context_lens)
    if not unscaled:
        _dev(k_scale, v_scale)
    scales = [] if unscaled else [k_scale.data_ptr(), v_scale.data_ptr(), sss, ssh]
    args = [q.data_ptr(), q.stride(0), q.stride(1), q.stride(2),
            _TORCH_DTYPE[q.dtype], k_cache.data_ptr(), v_cache.data_ptr(),
            css, csh] + scales + [S,
            block_tables.data_ptr(), block_tables.stride(0),
            context_lens.data_ptr(), B, R, Hq, num_kv_heads, D, block_size,
            float(softmax_scale), int(num_ranges), int(max_context)]
    if not with_workspace:
        return args, None
    ws_bytes = decode_workspace_bytes(B, R, Hq, num_kv_heads, D, num_ranges)
    if workspace is None:
        workspace = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8,
                                device=q.device)
    _dev(workspace)
    args += [workspace.data_ptr(), workspace.numel() * workspace.element_size()]
    return args, workspace


def paged_decode_attn_fp8(q, k_cache, v_cache, k_scale, v_scale, block_tables,
                          context_lens, *, num_kv_heads, block_size,
                          softmax_scale, max_context, num_ranges=0,
                          out=None, out_dtype=torch.bfloat16, workspace=None):
    """Paged GQA decode attention over the E4M3 cache. q: [B, R, Hq, D]
    bf16 (R verify rows, causal among themselves). Returns out [B, R, Hq, D]
    (bf16 or fp32)."""
    args, workspace = _decode_args(q, k_cache, v_cache, k_scale, v_scale,
                                   block_tables, context_lens, num_kv_heads,
                                   block_size, softmax_scale, max_context,
                                   num_ranges, workspace)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    _dev(out)
    if out.shape != q.shape or out.stride(3) != 1:
        raise ValueError("out must be [B, R, Hq, D] with contiguous head_dim")
    _check(lib().fp8kv_paged_decode_attn_fp8(
        *args, out.data_ptr(), out.stride(0), out.stride(1), out.stride(2),
        _TORCH_DTYPE[out.dtype], _stream(q.device)))
    return out


def _append_args(q, k_new, v_new, k_cache, v_cache, k_scale, v_scale, block_tables,
                 context_lens, num_kv_heads, block_size, softmax_scale, max_context,
                 num_ranges, workspace):
    """Argument list of the append calls (without out) and the workspace."""
    if q.dim() != 4:
        raise ValueError("q must be [B, R, Hq, D]")
    B, R, _, D = q.shape
    for t in (k_new, v_new):
        if t.dim() != 4 or t.dtype != torch.bfloat16 or t.stride(3) != 1:
            raise ValueError("k_new and v_new must be bf16 [B, R, Hkv, D], contiguous D")
        if tuple(t.shape) != (B, R, num_kv_heads, D):
            raise ValueError("k_new / v_new must be [B, R, Hkv, D] matching q")
    args, workspace = _decode_args(q, k_cache, v_cache, k_scale, v_scale,
                                   block_tables, context_lens, num_kv_heads,
                                   block_size, softmax_scale, max_context,
                                   num_ranges, workspace)
    _dev(k_new, v_new)
    new = [k_new.data_ptr(), k_new.stride(0), k_new.stride(1), k_new.stride(2),
           v_new.data_ptr(), v_new.stride(0), v_new.stride(1), v_new.stride(2), DTYPE_BF16]
    return args[:5] + new + args[5:], workspace


def paged_decode_append_attn_fp8(q, k_new, v_new, k_cache, v_cache, k_scale, v_scale,
                                 block_tables, context_lens, *, num_kv_heads, block_size,
                                 softmax_scale, max_context, num_ranges=0, out=None,
                                 out_dtype=torch.bfloat16, workspace=None):
    """One decode step: k_new / v_new [B, R, Hkv, D] bf16 (each at its own
    strides) are the K/V rows of every request's last R positions (already
    counted in context_lens); they are quantized into the cache at the slots
    its page table gives, and the decode attention of paged_decode_attn_fp8
    runs over the cache including them. Returns out [B, R, Hq, D]."""
    args, workspace = _append_args(q, k_new, v_new, k_cache, v_cache, k_scale, v_scale,
                                   block_tables, context_lens, num_kv_heads, block_size,
                                   softmax_scale, max_context, num_ranges, workspace)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    _dev(out)
    if out.shape != q.shape or out.stride(3) != 1:
        raise ValueError("out must be [B, R, Hq, D] with contiguous head_dim")
    _check(lib().fp8kv_paged_decode_append_attn_fp8(
        *args, out.data_ptr(), out.stride(0), out.stride(1), out.stride(2),
        _TORCH_DTYPE[out.dtype], _stream(q.device)))
    return out


def paged_decode_append_partials(q, k_new, v_new, k_cache, v_cache, k_scale, v_scale,
                                 block_tables, context_lens, *, num_kv_heads, block_size,
                                 softmax_scale, max_context, num_ranges=0, workspace=None):
    """Split phase of paged_decode_append_attn_fp8 (the new rows' store and
    the partials); returns the workspace for paged_decode_merge."""
    args, workspace = _append_args(q, k_new, v_new, k_cache, v_cache, k_scale, v_scale,
                                   block_tables, context_lens, num_kv_heads, block_size,
                                   softmax_scale, max_context, num_ranges, workspace)
    _check(lib().fp8kv_paged_decode_append_partials(*args, _stream(q.device)))
    return workspace


NOALLOC_SCRATCH_BYTES = 16 << 20


def paged_decode_attn_fp8_noalloc(q, k_cache, v_cache, k_scale, v_scale, block_tables,
                                  context_lens, out, *, num_kv_heads, block_size,
                                  softmax_scale, max_context, num_ranges=0):
    """paged_decode_attn_fp8 without a workspace: the partials go to a device
    array the library holds (NOALLOC_SCRATCH_BYTES per GPU), so the call
    allocates nothing; ``out`` [B, R, Hq, D] (bf16 or fp32) is required.
    Calls on one GPU share that array: order them on one stream."""
    args, _ = _decode_args(q, k_cache, v_cache, k_scale, v_scale, block_tables,
                           context_lens, num_kv_heads, block_size, softmax_scale,
                           max_context, num_ranges, None, with_workspace=False)
    _dev(out)
    if out.shape != q.shape or out.stride(3) != 1 or out.dtype not in _TORCH_DTYPE:
        raise ValueError("out must be [B, R, Hq, D] with contiguous head_dim")
    _check(lib().fp8kv_paged_decode_attn_fp8_noalloc(
        *args, out.data_ptr(), out.stride(0), out.stride(1), out.stride(2),
        _TORCH_DTYPE[out.dtype], _stream(q.device)))
    return out


def paged_decode_partials(q, k_cache, v_cache, k_scale, v_scale, block_tables,
                          context_lens, *, num_kv_heads, block_size,
                          softmax_scale, max_context, num_ranges=0,
                          workspace=None):
    """Split phase only; returns the workspace holding the partials."""
    args, workspace = _decode_args(q, k_cache, v_cache, k_scale, v_scale,
                                   block_tables, context_lens, num_kv_heads,
                                   block_size, softmax_scale, max_context,
                                   num_ranges, workspace)
    _check(lib().fp8kv_paged_decode_partials(*args, _stream(q.device)))
    return workspace


def paged_decode_attn_unscaled(q, k_cache, v_cache, block_tables, context_lens, *,
                               num_kv_heads, block_size, softmax_scale, max_context,
                               code_format=CODES_E4M3, num_ranges=0, out=None,
                               out_dtype=torch.bfloat16, workspace=None):
    """Paged GQA decode attention over an unscaled E4M3 or E5M2 cache
    (scale 1); otherwise as paged_decode_attn_fp8."""
    args, workspace = _decode_args(q, k_cache, v_cache, None, None, block_tables,
                                   context_lens, num_kv_heads, block_size,
                                   softmax_scale, max_context, num_ranges, workspace)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    _dev(out)
    if out.shape != q.shape or out.stride(3) != 1:
        raise ValueError("out must be [B, R, Hq, D] with contiguous head_dim")
    _check(lib().fp8kv_paged_decode_attn_unscaled(
        *args, out.data_ptr(), out.stride(0), out.stride(1), out.stride(2),
        _TORCH_DTYPE[out.dtype], int(code_format), _stream(q.device)))
    return out


def paged_decode_partials_unscaled(q, k_cache, v_cache, block_tables, context_lens, *,
                                   num_kv_heads, block_size, softmax_scale, max_context,
                                   code_format=CODES_E4M3, num_ranges=0, workspace=None):
    """Split phase only over an unscaled cache; returns the workspace."""
    args, workspace = _decode_args(q, k_cache, v_cache, None, None, block_tables,
                                   context_lens, num_kv_heads, block_size,
                                   softmax_scale, max_context, num_ranges, workspace)
    _check(lib().fp8kv_paged_decode_partials_unscaled(*args, int(code_format),
                                                      _stream(q.device)))
    return workspace


def _sparse_args(args, block_valid):
    """Insert the selected blocks' valid counts after the block table."""
    _dev(block_valid)
    if block_valid.dtype != torch.int32 or block_valid.dim() != 2 or \
            block_valid.stride(1) != 1:
        raise ValueError("block_valid must be int32 [B, max_sel], rows contiguous")
    return args[:16] + [block_valid.data_ptr(), block_valid.stride(0)] + args[16:]


def sparse_decode_attn_fp8(q, k_cache, v_cache, k_scale, v_scale, block_tables,
                           block_valid, context_lens, *, num_kv_heads,
                           block_size, softmax_scale, max_context,
                           num_ranges=0, out=None, out_dtype=torch.bfloat16,
                           workspace=None):
    """Decode attention over selected blocks: block_tables [B, max_sel]
    lists each request's selected blocks in position order, block_valid
    [B, max_sel] the keys of each from its start, context_lens the virtual
    positions (verify rows are causal on them). Returns out [B, R, Hq, D]."""
    if block_valid.shape != block_tables.shape:
        raise ValueError("block_valid must have the shape of block_tables")
    args, workspace = _decode_args(q, k_cache, v_cache, k_scale, v_scale,
                                   block_tables, context_lens, num_kv_heads,
                                   block_size, softmax_scale, max_context,
                                   num_ranges, workspace)
    args = _sparse_args(args, block_valid)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    _dev(out)
    if out.shape != q.shape or out.stride(3) != 1:
        raise ValueError("out must be [B, R, Hq, D] with contiguous head_dim")
    _check(lib().fp8kv_sparse_decode_attn_fp8(
        *args, out.data_ptr(), out.stride(0), out.stride(1), out.stride(2),
        _TORCH_DTYPE[out.dtype], _stream(q.device)))
    return out


def sparse_decode_partials(q, k_cache, v_cache, k_scale, v_scale, block_tables,
                           block_valid, context_lens, *, num_kv_heads,
                           block_size, softmax_scale, max_context,
                           num_ranges=0, workspace=None):
    """Split phase of sparse_decode_attn_fp8; merge with paged_decode_merge."""
    if block_valid.shape != block_tables.shape:
        raise ValueError("block_valid must have the shape of block_tables")
    args, workspace = _decode_args(q, k_cache, v_cache, k_scale, v_scale,
                                   block_tables, context_lens, num_kv_heads,
                                   block_size, softmax_scale, max_context,
                                   num_ranges, workspace)
    _check(lib().fp8kv_sparse_decode_partials(*_sparse_args(args, block_valid),
                                              _stream(q.device)))
    return workspace


def _prefill_args(q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens,
                  q_lens, num_kv_heads, block_size, softmax_scale, max_context, out,
                  out_dtype, block_valid=None):
    """Argument list of the prefill calls (with block_valid: the selected-
    block call) and the output tensor."""
    if q.dim() != 4 or q.stride(3) != 1 or q.dtype not in _TORCH_DTYPE:
        raise ValueError("q must be [B, max_q, Hq, D] with contiguous head_dim")
    B, Q, Hq, D = q.shape
    css, csh, S, H, Dc = _kv_caches(k_cache, v_cache)
    if H != num_kv_heads or Dc != D:
        raise ValueError("cache geometry does not match q / num_kv_heads")
    sss, ssh = _scale_pair(k_scale, v_scale, S, H)
    _tables(block_tables, context_lens, B, block_size, int(max_context), extra=(q_lens,))
    if block_valid is not None:
        if block_valid.shape != block_tables.shape or block_valid.dtype != torch.int32 or \
                (block_valid.shape[1] > 1 and block_valid.stride(1) != 1):
            raise ValueError("block_valid must be int32 with the shape of block_tables, "
                             "rows contiguous")
    _dev(q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens, q_lens)
    if block_valid is not None:
        _dev(block_valid)
    if out is None:
        out = torch.zeros(q.shape, dtype=out_dtype, device=q.device)
    _dev(out)
    if out.shape != q.shape or out.stride(3) != 1:
        raise ValueError("out must be [B, max_q, Hq, D] with contiguous head_dim")
    sel = [] if block_valid is None else [block_valid.data_ptr(), block_valid.stride(0)]
    args = [q.data_ptr(), q.stride(0), q.stride(1), q.stride(2), _TORCH_DTYPE[q.dtype],
            k_cache.data_ptr(), v_cache.data_ptr(), css, csh, k_scale.data_ptr(),
            v_scale.data_ptr(), sss, ssh, S, block_tables.data_ptr(),
            block_tables.stride(0)] + sel + [context_lens.data_ptr(), q_lens.data_ptr(), B, Q,
            Hq, num_kv_heads, D, block_size, float(softmax_scale), int(max_context),
            out.data_ptr(), out.stride(0), out.stride(1), out.stride(2),
            _TORCH_DTYPE[out.dtype], _stream(q.device)]
    return args, out


def prefill_attn_fp8(q, k_cache, v_cache, k_scale, v_scale, block_tables,
                     context_lens, q_lens, *, num_kv_heads, block_size,
                     softmax_scale, max_context, out=None,
                     out_dtype=torch.bfloat16):
    """Chunked-prefill attention: q [B, max_q, Hq, D] bf16 holds each
    request's last q_lens[b] tokens (already in the cache); token i attends
    to the cached tokens 0 .. context_lens[b] - q_lens[b] + i. Returns out
    [B, max_q, Hq, D] (rows i >= q_lens[b] are left untouched)."""
    args, out = _prefill_args(q, k_cache, v_cache, k_scale, v_scale, block_tables,
                              context_lens, q_lens, num_kv_heads, block_size,
                              softmax_scale, max_context, out, out_dtype)
    _check(lib().fp8kv_prefill_attn_fp8(*args))
    return out


def sparse_prefill_attn_fp8(q, k_cache, v_cache, k_scale, v_scale, block_tables,
                            block_valid, context_lens, q_lens, *, num_kv_heads,
                            block_size, softmax_scale, max_context, out=None,
                            out_dtype=torch.bfloat16):
    """Chunked-prefill attention over selected blocks: block_tables [B,
    max_sel] lists each request's selected blocks in position order (the
    chunk's blocks among them), block_valid [B, max_sel] the keys of each
    from its start, context_lens the virtual positions; chunk token i
    attends positions 0 .. context_lens[b] - q_lens[b] + i."""
    args, out = _prefill_args(q, k_cache, v_cache, k_scale, v_scale, block_tables,
                              context_lens, q_lens, num_kv_heads, block_size,
                              softmax_scale, max_context, out, out_dtype,
                              block_valid=block_valid)
    _check(lib().fp8kv_sparse_prefill_attn_fp8(*args))
    return out


def paged_decode_merge(workspace, out, *, rows, num_q_heads, num_kv_heads,
                       num_ranges=0):
    """Log-sum-exp merge of the partials in ``workspace`` (written by
    paged_decode_partials with the same num_ranges) into out [B, R, Hq, D]."""
    _dev(workspace, out)
    B, R, Hq, D = out.shape
    _check(lib().fp8kv_paged_decode_merge(
        B, rows, num_q_heads, num_kv_heads, D, int(num_ranges),
        workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        out.data_ptr(), out.stride(0), out.stride(1), out.stride(2),
        _TORCH_DTYPE[out.dtype], _stream(out.device)))
    return out


def index_keys_quantize(keys: torch.Tensor, key_format: int, codes=None,
                        scales=None):
    """Encode bf16 index keys [..., N, 128] (rows of unit inner stride).
    KEYS_MXFP4: returns (packed uint8 [..., N, 64], E8M0 codes uint8
    [..., N, 4]); KEYS_E4M3: (codes uint8 [..., N, 128], fp32 scales
    [..., N])."""
    _dev(keys)
    if keys.dtype != torch.bfloat16 or keys.shape[-1] != 128:
        raise ValueError("keys must be bf16 [..., 128]")
    lead = keys.shape[:-1]
    flat = keys.reshape(-1, 128)
    if flat.stride(1) != 1:
        raise ValueError("keys need a contiguous last dimension")
    n = flat.shape[0]
    mx = key_format == KEYS_MXFP4
    if codes is None:
        codes = torch.empty(lead + ((64,) if mx else (128,)), dtype=torch.uint8,
                            device=keys.device)
    if scales is None:
        scales = torch.empty(lead + ((4,) if mx else ()),
                             dtype=torch.uint8 if mx else torch.float32,
                             device=keys.device)
    _dev(codes, scales)
    cf = codes.view(-1, codes.shape[-1])
    sf = scales.view(-1, 4) if mx else scales.view(-1)
    if cf.shape[0] != n or sf.shape[0] != n:
        raise ValueError("codes / scales do not match the number of keys")
    _check(lib().fp8kv_index_keys_quantize(
        flat.data_ptr(), flat.stride(0), n, 128, int(key_format),
        cf.data_ptr(), cf.stride(0), sf.data_ptr(), sf.stride(0),
        _stream(keys.device)))
    return codes, scales


def index_keys_build(raw: torch.Tensor, g0: int, g1: int, key_format: int,
                     codes: torch.Tensor, scales=None) -> None:
    """Compressed keys g0 .. g1-1 of every request from raw bf16 index keys
    raw [B, L, 128] (4*g1 <= L): mean of 4, L2-normalized, rounded to bf16,
    stored in key_format into codes [B, N, 64 | 128 | 256 bytes] (and
    scales [B, N, 4] uint8 or [B, N] fp32) at rows g0 .. g1-1."""
    _dev(raw, codes)
    if raw.dim() != 3 or raw.dtype != torch.bfloat16 or raw.shape[2] != 128 or \
            raw.stride(2) != 1:
        raise ValueError("raw must be bf16 [B, L, 128], contiguous last dim")
    B, L, _ = raw.shape
    if not (0 <= g0 <= g1 and 4 * g1 <= L):
        raise ValueError("need 0 <= g0 <= g1 and 4 * g1 <= L")
    nbytes = {KEYS_MXFP4: 64, KEYS_E4M3: 128, KEYS_BF16: 256}[key_format]
    if codes.dim() != 3 or codes.dtype != torch.uint8 or codes.shape[0] != B or \
            codes.shape[1] < g1 or codes.shape[2] != nbytes or codes.stride(2) != 1:
        raise ValueError(f"codes must be uint8 [B, >= g1, {nbytes}]")
    if key_format == KEYS_BF16:
        sp, s0, s1 = None, 0, 0
    else:
        if scales is None:
            raise ValueError("scales are required for quantized keys")
        _dev(scales)
        if key_format == KEYS_MXFP4 and (scales.dtype != torch.uint8 or scales.dim() != 3
                                         or scales.shape[2] != 4 or scales.stride(2) != 1):
            raise ValueError("MXFP4 exponents must be uint8 [B, N, 4]")
        if key_format == KEYS_E4M3 and (scales.dtype != torch.float32 or scales.dim() != 2):
            raise ValueError("E4M3 key scales must be fp32 [B, N]")
        if scales.shape[0] != B or scales.shape[1] < g1:
            raise ValueError("scales do not cover the keys")
        sp, s0, s1 = scales.data_ptr(), scales.stride(0), scales.stride(1)
    _check(lib().fp8kv_index_keys_build(
        raw.data_ptr(), raw.stride(0), raw.stride(1), B, int(g0), int(g1), 128,
        int(key_format), codes.data_ptr(), codes.stride(0), codes.stride(1),
        sp, s0, s1, _stream(raw.device)))


def index_score_mxfp4(q: torch.Tensor, w: torch.Tensor, key_format: int,
                      codes: torch.Tensor, scales: torch.Tensor, *,
                      key_chunk: int = 0, out=None):
    """score[b, r, n] = sum_h w[b, r, h] * relu(q[b, r, h, :] . k^[b, n, :]).

    q       bf16 [B, R, H, 128] (H <= 16), w fp32 [B, R, H];
    codes   uint8 [B, N, 64] (MXFP4) or [B, N, 128] (E4M3);
    scales  uint8 [B, N, 4] (MXFP4 exponents) or fp32 [B, N] (E4M3).
    Returns out fp32 [B, R, N]."""
    _dev(q, w, codes, scales)
    if q.dim() != 4 or q.dtype != torch.bfloat16 or q.stride(3) != 1:
        raise ValueError("q must be bf16 [B, R, H, D], contiguous D")
    B, R, H, D = q.shape
    if w.shape != (B, R, H) or w.dtype != torch.float32:
        raise ValueError("w must be fp32 [B, R, H]")
    mx = key_format == KEYS_MXFP4
    if codes.dim() != 3 or codes.dtype != torch.uint8 or codes.stride(2) != 1:
        raise ValueError("codes must be uint8 [B, N, bytes], contiguous bytes")
    N = codes.shape[1]
    if mx:
        if scales.shape != (B, N, 4) or scales.dtype != torch.uint8 or \
                scales.stride(2) != 1:
            raise ValueError("MXFP4 exponents must be uint8 [B, N, 4]")
    elif scales.shape != (B, N) or scales.dtype != torch.float32:
        raise ValueError("E4M3 key scales must be fp32 [B, N]")
    if out is None:
        out = torch.empty((B, R, N), dtype=torch.float32, device=q.device)
    _dev(out)
    if out.shape != (B, R, N) or out.dtype != torch.float32 or \
            (N > 1 and out.stride(2) != 1):
        raise ValueError("out must be fp32 [B, R, N], contiguous N")
    _check(lib().fp8kv_index_score_mxfp4(
        q.data_ptr(), q.stride(0), q.stride(1), q.stride(2), DTYPE_BF16,
        w.data_ptr(), w.stride(0), w.stride(1), w.stride(2), int(key_format),
        codes.data_ptr(), codes.stride(0), codes.stride(1),
        scales.data_ptr(), scales.stride(0), scales.stride(1),
        B, R, H, D, N, int(key_chunk), out.data_ptr(), out.stride(0),
        out.stride(1), _stream(q.device)))
    return out
