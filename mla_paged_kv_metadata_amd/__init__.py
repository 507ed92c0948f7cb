"""Python binding of libmla_decode.so: MLA decode over a paged KV cache on MI355X.

Argument marshalling only (ctypes over the C ABI in include/mla_decode.h);
every step of the computation runs in the library's HIP kernels.  PyTorch
provides device memory and the current stream.

The two calls follow the FlashMLA interface page (get_mla_metadata and
flash_mla_with_kvcache); they are exported under the C names
(mla_get_metadata, mla_decode_fwd) and under the pages' Python names.
"""
from __future__ import annotations

import contextlib
import ctypes
import math
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmla_decode.so")
# Race-check build: page copies never overlap LDS reads (see csrc/mla_decode.hip).
SERIAL_LIB_PATH = os.path.join(_PKG, "libmla_decode_serial.so")

TILE_MD_INTS = 8
HEAD_DIM = 576
HEAD_DIM_V = 512
NOALLOC_SCRATCH_BYTES = 128 << 20   # MLA_NOALLOC_SCRATCH_BYTES
PAGE_BLOCK_SIZE = 64        # tokens per scheduling page (and the usual cache block)
PAGE_BLOCK_ALIGN = 16       # a cache's page_block_size must be a multiple of this
KV_BF16 = 0
KV_FP8_E4M3FN = 1

_lib = None

_c_int, _c_size, _vp = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p


def load_library(path: Optional[str] = None):
    """Load the HIP library.  Raises if it is not built: there is no fallback path."""
    global _lib
    if _lib is not None:
        return _lib
    _lib = _open(path or LIB_PATH)
    return _lib


@contextlib.contextmanager
def library_variant(path: str):
    """Within the block, every call goes to the library at path (e.g. the
    race-check build SERIAL_LIB_PATH) instead of the default one."""
    global _lib
    prev = load_library()
    _lib = _open(path)
    try:
        yield _lib
    finally:
        _lib = prev


def _open(p: str):
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing; build it with __graft_entry__.build() "
                           "(the HIP library is required, there is no CPU fallback)")
    lib = ctypes.CDLL(p)
    lib.mla_status_str.restype = ctypes.c_char_p
    lib.mla_status_str.argtypes = [_c_int]
    lib.mla_num_parts.restype = _c_int
    lib.mla_num_parts.argtypes = [_c_int, _c_int, _c_int, ctypes.POINTER(_c_int)]
    lib.mla_get_metadata.restype = _c_int
    lib.mla_get_metadata.argtypes = [_vp, _c_int, _c_int, _c_int, _vp, _c_int, _vp, _vp]
    lib.mla_get_metadata_ex.restype = _c_int
    lib.mla_get_metadata_ex.argtypes = [_vp, _c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp]
    lib.mla_workspace_bytes.restype = _c_int
    lib.mla_workspace_bytes.argtypes = [_c_int] * 6 + [ctypes.POINTER(_c_size)]
    for fn in (lib.mla_decode_fwd, lib.mla_decode_splits, lib.mla_combine_splits):
        fn.restype = _c_int
        fn.argtypes = _DECODE_ARGTYPES
    lib.mla_decode_fwd_ext.restype = _c_int
    lib.mla_decode_fwd_ext.argtypes = _DECODE_ARGTYPES + [ctypes.POINTER(DecodeExt)]
    lib.mla_decode_fwd_noalloc.restype = _c_int
    lib.mla_decode_fwd_noalloc.argtypes = _DECODE_ARGTYPES[:20] + _DECODE_ARGTYPES[22:]
    lib.mla_lds_dma_read.restype = _c_int
    lib.mla_lds_dma_read.argtypes = [_vp, _c_size, _vp]
    return lib


_DECODE_ARGTYPES = [
    _vp, _c_int, _c_int, _c_int, _c_int,            # q, batch, s_q, num_heads_q, head_dim
    _vp, _c_int, _c_int, _c_int, _c_int,            # kv_cache, kv_dtype, num_blocks, page_block_size, num_heads_k
    _vp, _c_int, _vp,                               # block_table, max_blocks_per_seq, cache_seqlens
    _c_int, ctypes.c_float, ctypes.c_float, _c_int,  # head_dim_v, softmax_scale, v_scale, causal
    _vp, _c_int, _vp,                               # tile_md, num_parts, num_splits
    _vp, _c_size,                                   # workspace, workspace_bytes
    _vp, _vp, _vp,                                  # out, lse, stream
]


class DecodeExt(ctypes.Structure):
    """mla_decode_ext of include/mla_decode.h."""
    _fields_ = [("sinks", _vp), ("bmm1_scale", _vp), ("bmm2_scale", _vp), ("kv_rope", _vp), ("q_rope", _vp),
                ("stages", _c_int), ("bmm1_scale_log2", _vp), ("qk_descale", _vp), ("pv_descale", _vp),
                ("q_dtype", _c_int)]


Q_BF16 = 0
Q_FP8_E4M3FN = 1


# Status codes of include/mla_decode.h.
MLA_OK = 0
MLA_ERR_INVALID_ARG = 1
MLA_ERR_UNSUPPORTED = 2
MLA_ERR_WORKSPACE_TOO_SMALL = 3
MLA_ERR_NO_DEVICE = 4
MLA_ERR_HIP = 5


class MlaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (mla status {status})")
        self.status = status


def _check(rc: int):
    if rc != 0:
        raise MlaError(rc, load_library().mla_status_str(rc).decode())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need(t: torch.Tensor, name: str, dtype=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def mla_num_parts(batch: int, heads_per_head_k: int, num_heads_k: int) -> int:
    """Recommended number of parts (rows of the tile-scheduler table) on the current device."""
    n = _c_int(0)
    _check(load_library().mla_num_parts(batch, heads_per_head_k, num_heads_k, ctypes.byref(n)))
    return n.value


def mla_get_metadata(cache_seqlens: torch.Tensor, num_heads_per_head_k: int, num_heads_k: int,
                     num_parts: Optional[int] = None, fixed_cost: Optional[int] = None,
                     tile_md: Optional[torch.Tensor] = None, num_splits: Optional[torch.Tensor] = None
                     ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Split-KV tile-scheduler metadata (FlashMLA interface page, get_mla_metadata).

    cache_seqlens: (batch,) int32 on the GPU.  num_heads_per_head_k =
    seq_len_q * num_heads_q // num_heads_k.  num_parts is the balancing
    target (default: about one workgroup per compute unit).  Returns
    (tile_scheduler_metadata (num_parts, 8) int32, one row per part,
    num_splits (batch + 1) int32), computed by the scheduler kernel on the
    current stream.
    """
    lib = load_library()
    _need(cache_seqlens, "cache_seqlens", torch.int32)
    if not cache_seqlens.is_cuda or cache_seqlens.dim() != 1:
        raise ValueError("cache_seqlens must be a 1-D int32 GPU tensor")
    B = cache_seqlens.shape[0]
    dev = cache_seqlens.device
    with torch.cuda.device(dev):
        if num_parts is None:
            num_parts = mla_num_parts(B, num_heads_per_head_k, num_heads_k)
        md, ns = tile_md, num_splits
        if md is None:
            md = torch.empty((num_parts, TILE_MD_INTS), dtype=torch.int32, device=dev)
        if ns is None:
            ns = torch.empty((B + 1,), dtype=torch.int32, device=dev)
        _need(md, "tile_md", torch.int32, dev)
        _need(ns, "num_splits", torch.int32, dev)
        if tuple(md.shape) != (num_parts, TILE_MD_INTS) or tuple(ns.shape) != (B + 1,):
            raise ValueError("tile_md must be (num_parts, 8) and num_splits (batch + 1,)")
        if fixed_cost is None:
            rc = lib.mla_get_metadata(_ptr(cache_seqlens), B, num_heads_per_head_k, num_heads_k, _ptr(md),
                                      num_parts, _ptr(ns), _stream(dev))
        else:
            rc = lib.mla_get_metadata_ex(_ptr(cache_seqlens), B, num_heads_per_head_k, num_heads_k, num_parts,
                                         fixed_cost, _ptr(md), _ptr(ns), _stream(dev))
    _check(rc)
    return md, ns


def mla_workspace_bytes(batch: int, s_q: int, num_heads_q: int, num_heads_k: int, head_dim_v: int,
                        num_parts: int) -> int:
    n = _c_size(0)
    _check(load_library().mla_workspace_bytes(batch, s_q, num_heads_q, num_heads_k, head_dim_v, num_parts,
                                              ctypes.byref(n)))
    return n.value


def _kv_layout(kv_cache: torch.Tensor):
    """(num_blocks, page_block_size, num_heads_k, dtype code) of a 3-D or 4-D cache."""
    if kv_cache.dtype == torch.bfloat16:
        code = KV_BF16
    elif kv_cache.dtype in (torch.float8_e4m3fn, torch.uint8):
        code = KV_FP8_E4M3FN
    else:
        raise TypeError(f"kv_cache must be bfloat16 or float8_e4m3fn (uint8 codes), got {kv_cache.dtype}")
    if kv_cache.dim() == 4:
        nb, page, hk, d = kv_cache.shape
    elif kv_cache.dim() == 3:
        (nb, page, d), hk = kv_cache.shape, 1
    else:
        raise ValueError("kv_cache must be (num_blocks, page_block_size, num_heads_k, head_dim) "
                         "or (num_blocks, page_block_size, head_dim)")
    return nb, page, hk, d, code


def mla_decode_fwd(q: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor, cache_seqlens: torch.Tensor,
                   head_dim_v: int, tile_scheduler_metadata: torch.Tensor, num_splits: torch.Tensor,
                   softmax_scale: Optional[float] = None, causal: bool = False, v_scale: float = 1.0,
                   out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None, stage: str = "all",
                   sinks: Optional[torch.Tensor] = None, bmm1_scale_tensor: Optional[torch.Tensor] = None,
                   bmm2_scale_tensor: Optional[torch.Tensor] = None, kv_rope: Optional[torch.Tensor] = None,
                   q_rope: Optional[torch.Tensor] = None, bmm1_scale_log2_tensor: Optional[torch.Tensor] = None,
                   qk_descale: Optional[torch.Tensor] = None,
                   pv_descale: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """MLA decode attention (FlashMLA interface page, flash_mla_with_kvcache).

    q (B, s_q, H_q, 576) bf16; kv_cache (num_blocks, page_block_size, H_k, 576)
    bf16 or e4m3fn, page_block_size a multiple of 16 (64 in the pages'
    caches); block_table (B, max_blocks) int32; cache_seqlens (B,) int32.
    stage: "all" (mla_decode_fwd), or "splits" / "combine" to run one of its
    two kernels (mla_decode_splits / mla_combine_splits; pass the same out,
    lse and workspace to both).
    softmax_scale defaults to 1/sqrt(576) (for an fp8 cache pass the fused
    bmm1 scale); v_scale is the fused bmm2 scale.  Returns
    out (B, s_q, H_q, 512) bf16 and softmax_lse (B, H_q, s_q) fp32.

    Optional inputs (mla_decode_fwd_ext; FlashInfer MLA page and Ascend ATB
    MLA page): sinks (H_q,) fp32 per-head sink logits; bmm1_scale_tensor /
    bmm2_scale_tensor (1,) fp32 device scales replacing softmax_scale /
    v_scale; kv_rope (num_blocks, page_block_size, H_k, 64) with kv_cache
    then (num_blocks, page_block_size, H_k, 512) (split cache); q_rope
    (B, s_q, H_q, 64) bf16
    with q then (B, s_q, H_q, 512) (split query); bmm1_scale_log2_tensor (1,)
    fp32, bmm1 * log2(e), replacing softmax_scale and bmm1_scale_tensor;
    qk_descale / pv_descale (H_q,) fp32 per-head factors on the scores / the
    output.  q may be torch.float8_e4m3fn (joined layout only) with its
    q_scale folded into the bmm1 scale.
    """
    lib = load_library()
    if softmax_scale is None:
        softmax_scale = HEAD_DIM ** (-0.5)
    dev = q.device
    q_fp8 = q.dtype == torch.float8_e4m3fn
    _need(q, "q", torch.float8_e4m3fn if q_fp8 else torch.bfloat16, dev)
    if q_fp8 and q_rope is not None:
        raise ValueError("an fp8 q must be joined (no q_rope)")
    _need(kv_cache, "kv_cache", None, dev)
    _need(block_table, "block_table", torch.int32, dev)
    _need(cache_seqlens, "cache_seqlens", torch.int32, dev)
    _need(tile_scheduler_metadata, "tile_scheduler_metadata", torch.int32, dev)
    _need(num_splits, "num_splits", torch.int32, dev)
    if q.dim() != 4:
        raise ValueError("q must be (batch, seq_len_q, num_heads_q, head_dim)")
    B, s_q, Hq, D = q.shape
    nb, page, hk, dk, code = _kv_layout(kv_cache)
    if q_rope is not None:
        _need(q_rope, "q_rope", torch.bfloat16, dev)
        if D != HEAD_DIM_V or tuple(q_rope.shape) != (B, s_q, Hq, HEAD_DIM - HEAD_DIM_V):
            raise ValueError("with q_rope, q must be (B, s_q, H_q, 512) and q_rope (B, s_q, H_q, 64)")
        D = HEAD_DIM
    if kv_rope is not None:
        _need(kv_rope, "kv_rope", kv_cache.dtype, dev)
        if dk != HEAD_DIM_V or tuple(kv_rope.shape[:-1]) != tuple(kv_cache.shape[:-1]) \
                or kv_rope.shape[-1] != HEAD_DIM - HEAD_DIM_V:
            raise ValueError("with kv_rope, kv_cache must end in 512 and kv_rope in 64 columns, "
                             "with the same leading shape")
        dk = HEAD_DIM
    if dk != D:
        raise ValueError("q and kv_cache head_dim differ")
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be (batch, max_num_blocks_per_seq)")
    if cache_seqlens.shape != (B,):
        raise ValueError("cache_seqlens must be (batch,)")
    if (tile_scheduler_metadata.dim() != 2 or tile_scheduler_metadata.shape[1] != TILE_MD_INTS
            or tile_scheduler_metadata.shape[0] < 1):
        raise ValueError("tile_scheduler_metadata must be (num_parts, 8)")
    if num_splits.shape != (B + 1,):
        raise ValueError("num_splits must be (batch + 1,)")
    num_parts = tile_scheduler_metadata.shape[0]
    if out is None:
        out = torch.empty((B, s_q, Hq, head_dim_v), dtype=torch.bfloat16, device=dev)
    else:
        _need(out, "out", torch.bfloat16, dev)
        if tuple(out.shape) != (B, s_q, Hq, head_dim_v):
            raise ValueError("out has the wrong shape")
    if lse is None:
        lse = torch.empty((B, Hq, s_q), dtype=torch.float32, device=dev)
    else:
        _need(lse, "lse", torch.float32, dev)
        if tuple(lse.shape) != (B, Hq, s_q):
            raise ValueError("lse has the wrong shape")
    if Hq % hk:
        raise ValueError("num_heads_q must be a multiple of num_heads_k")
    need = mla_workspace_bytes(B, s_q, Hq, hk, head_dim_v, num_parts)
    if workspace is None:
        workspace = torch.empty((need,), dtype=torch.uint8, device=dev)
    else:
        _need(workspace, "workspace", torch.uint8, dev)
    if sinks is not None:
        _need(sinks, "sinks", torch.float32, dev)
        if tuple(sinks.shape) != (Hq,):
            raise ValueError("sinks must be (num_heads_q,)")
    for t, name in ((bmm1_scale_tensor, "bmm1_scale_tensor"), (bmm2_scale_tensor, "bmm2_scale_tensor"),
                    (bmm1_scale_log2_tensor, "bmm1_scale_log2_tensor")):
        if t is not None:
            _need(t, name, torch.float32, dev)
            if t.numel() != 1:
                raise ValueError(f"{name} must hold one value")
    for t, name in ((qk_descale, "qk_descale"), (pv_descale, "pv_descale")):
        if t is not None:
            _need(t, name, torch.float32, dev)
            if tuple(t.shape) != (Hq,):
                raise ValueError(f"{name} must be (num_heads_q,)")
    stages = {"all": 3, "splits": 1, "combine": 2}[stage]
    args = (_ptr(q), B, s_q, Hq, D, _ptr(kv_cache), code, nb, page, hk,
            _ptr(block_table), block_table.shape[1], _ptr(cache_seqlens),
            head_dim_v, float(softmax_scale), float(v_scale), int(bool(causal)),
            _ptr(tile_scheduler_metadata), num_parts, _ptr(num_splits),
            _ptr(workspace), workspace.numel(), _ptr(out), _ptr(lse), _stream(dev))
    with torch.cuda.device(dev):
        if q_fp8 or any(t is not None for t in (sinks, bmm1_scale_tensor, bmm2_scale_tensor, kv_rope, q_rope,
                                                 bmm1_scale_log2_tensor, qk_descale, pv_descale)):
            ext = DecodeExt(_ptr(sinks), _ptr(bmm1_scale_tensor), _ptr(bmm2_scale_tensor), _ptr(kv_rope),
                            _ptr(q_rope), stages, _ptr(bmm1_scale_log2_tensor), _ptr(qk_descale),
                            _ptr(pv_descale), Q_FP8_E4M3FN if q_fp8 else Q_BF16)
            rc = lib.mla_decode_fwd_ext(*args, ctypes.byref(ext))
        else:
            fn = {3: lib.mla_decode_fwd, 1: lib.mla_decode_splits, 2: lib.mla_combine_splits}[stages]
            rc = fn(*args)
    _check(rc)
    return out, lse


def mla_decode_fwd_noalloc(q: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
                           cache_seqlens: torch.Tensor, head_dim_v: int, tile_scheduler_metadata: torch.Tensor,
                           num_splits: torch.Tensor, out: torch.Tensor, lse: torch.Tensor,
                           softmax_scale: Optional[float] = None, causal: bool = False,
                           v_scale: float = 1.0) -> Tuple[torch.Tensor, torch.Tensor]:
    """mla_decode_fwd without a workspace (the library's static device scratch
    holds the split partials); the caller provides out and lse.  Calls that
    overlap in time on one GPU share that scratch and must not overlap."""
    lib = load_library()
    if softmax_scale is None:
        softmax_scale = HEAD_DIM ** (-0.5)
    dev = q.device
    for t, name, dt in ((q, "q", torch.bfloat16), (kv_cache, "kv_cache", None), (block_table, "block_table", torch.int32),
                        (cache_seqlens, "cache_seqlens", torch.int32),
                        (tile_scheduler_metadata, "tile_scheduler_metadata", torch.int32),
                        (num_splits, "num_splits", torch.int32), (out, "out", torch.bfloat16),
                        (lse, "lse", torch.float32)):
        _need(t, name, dt, dev)
    B, s_q, Hq, D = q.shape
    nb, page, hk, _, code = _kv_layout(kv_cache)
    if tuple(out.shape) != (B, s_q, Hq, head_dim_v) or tuple(lse.shape) != (B, Hq, s_q):
        raise ValueError("out must be (B, s_q, H_q, head_dim_v) and lse (B, H_q, s_q)")
    if block_table.dim() != 2 or block_table.shape[0] != B or cache_seqlens.shape != (B,) \
            or num_splits.shape != (B + 1,) or tile_scheduler_metadata.dim() != 2 \
            or tile_scheduler_metadata.shape[1] != TILE_MD_INTS:
        raise ValueError("block_table, cache_seqlens, tile_scheduler_metadata or num_splits has the wrong shape")
    with torch.cuda.device(dev):
        rc = lib.mla_decode_fwd_noalloc(
            _ptr(q), B, s_q, Hq, D, _ptr(kv_cache), code, nb, page, hk, _ptr(block_table), block_table.shape[1],
            _ptr(cache_seqlens), head_dim_v, float(softmax_scale), float(v_scale), int(bool(causal)),
            _ptr(tile_scheduler_metadata), tile_scheduler_metadata.shape[0], _ptr(num_splits), _ptr(out), _ptr(lse),
            _stream(dev))
    _check(rc)
    return out, lse


def fp8_fused_scales(q_scale=1.0, k_scale=1.0, v_scale=1.0, o_scale=1.0, sm_scale=1.0, head_dim_qk=HEAD_DIM):
    """(bmm1_scale, bmm2_scale) as the FlashInfer MLA page fuses them."""
    return q_scale * k_scale * sm_scale / math.sqrt(head_dim_qk), v_scale * o_scale


# The pages' Python names.
get_mla_metadata = mla_get_metadata


def flash_mla_with_kvcache(q, k_cache, block_table, cache_seqlens, head_dim_v, tile_scheduler_metadata,
                           num_splits, softmax_scale=None, causal=False):
    return mla_decode_fwd(q, k_cache, block_table, cache_seqlens, head_dim_v, tile_scheduler_metadata,
                          num_splits, softmax_scale=softmax_scale, causal=causal)


__all__ = ["load_library", "mla_num_parts", "mla_get_metadata", "mla_workspace_bytes", "mla_decode_fwd",
           "mla_decode_fwd_noalloc",
           "get_mla_metadata", "flash_mla_with_kvcache", "fp8_fused_scales", "MlaError", "LIB_PATH"]


def lds_dma_read(src: torch.Tensor) -> None:
    """Measurement aid (mla_lds_dma_read): reads the bytes of a contiguous
    device tensor (a multiple of 1 KiB) into LDS with the page copies' LDS-DMA
    instruction, for calibrating HBM traffic counters."""
    if not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous device tensor")
    n = src.numel() * src.element_size()
    with torch.cuda.device(src.device):
        _check(load_library().mla_lds_dma_read(_ptr(src), n, _stream(src.device)))
