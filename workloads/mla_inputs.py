"""Seeded synthetic MLA-decode inputs (no attention arithmetic here).

Shapes follow the FlashMLA interface page (docstring of
``flash_mla_with_kvcache``): q is (batch, seq_len_q, num_heads_q, head_dim),
the cache is (num_blocks, page_block_size, num_heads_k, head_dim), the block
table is (batch, max_num_blocks_per_seq) int32 and cache_seqlens is (batch,)
int32.  head_dim = 576 is the 512-wide latent part followed by the 64-wide
rope part (FlashInfer ``trtllm_batch_decode_with_kv_cache_mla`` page,
parameters ``query`` and ``kv_cache``).

Random numbers come from ``numpy.random.Generator(PCG64(seed))`` in a fixed
draw order: sequence lengths, then the page permutation, then q, then the
cache.  Normals are drawn as float32 and rounded to bf16 with
round-to-nearest-even; fp8 caches are quantised with one per-tensor scale.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

HEAD_DIM = 576      # kv_lora_rank 512 + qk_rope_head_dim 64
HEAD_DIM_V = 512    # V is the latent (first 512) columns of the cached rows
PAGE = 64           # page_block_size used by every workload here
E4M3FN_MAX = 448.0

_CHUNK = 1 << 24    # values per chunk when drawing large caches


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); returns uint16 bits.

    Inputs here are finite normals, so the NaN/inf special cases never arise.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def _normal_bf16(rng: np.random.Generator, n: int, mul: float = 1.0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        x = rng.standard_normal(e - s, dtype=np.float32)
        if mul != 1.0:
            x *= np.float32(mul)
        out[s:e] = bf16_bits_from_f32(x)
    return out


def _normal_e4m3fn(rng: np.random.Generator, n: int):
    """Draw N(0,1) float32, quantise with one per-tensor scale amax/448 (RNE, saturating).

    Returns (codes uint8, scale).  The encoding uses torch's float8_e4m3fn cast
    (the OCP e4m3 format with finite max 448) after clamping to +-448.
    """
    import torch  # used only as a format converter for the synthetic cache

    x = np.empty(n, dtype=np.float32)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        x[s:e] = rng.standard_normal(e - s, dtype=np.float32)
    amax = float(np.max(np.abs(x)))
    scale = amax / E4M3FN_MAX
    codes = np.empty(n, dtype=np.uint8)
    inv = np.float32(1.0 / scale)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        y = np.clip(x[s:e] * inv, -E4M3FN_MAX, E4M3FN_MAX)
        codes[s:e] = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, float(scale)


@dataclasses.dataclass
class Workload:
    """One decode batch, as raw bytes.  Arrays are host numpy arrays."""

    name: str
    batch: int
    s_q: int
    num_heads_q: int
    num_heads_k: int
    cache_seqlens: np.ndarray            # (B,) int32
    block_table: np.ndarray              # (B, max_blocks) int32
    q_bits: np.ndarray                   # (B, s_q, H, 576) uint16 (bf16 bits)
    kv: np.ndarray                       # (num_blocks, page_block_size, H_k, 576) bf16 bits or e4m3fn codes
    kv_dtype: str                        # "bf16" or "fp8_e4m3fn"
    causal: bool
    k_scale: float = 1.0                 # per-tensor dequant scale of the cache (fp8 only)
    v_scale: float = 1.0
    head_dim: int = HEAD_DIM
    head_dim_v: int = HEAD_DIM_V
    page_block_size: int = PAGE

    @property
    def num_blocks(self) -> int:
        return int(self.kv.shape[0])

    @property
    def heads_per_head_k(self) -> int:
        return self.s_q * self.num_heads_q // self.num_heads_k

    def nblk(self) -> np.ndarray:
        L = self.cache_seqlens.astype(np.int64)
        return (L + self.page_block_size - 1) // self.page_block_size


def fp8_query(w: "Workload", seed: int):
    """An e4m3fn query of the workload's q shape: N(0, 1) draws quantised with
    one per-tensor scale (as the fp8 cache).  Returns (codes uint8, q_scale)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    codes, q_scale = _normal_e4m3fn(rng, int(np.prod(w.q_bits.shape)))
    return codes.reshape(w.q_bits.shape), q_scale


def _page_pool(rng, seqlens, num_heads_k, extra_pages=0, padding="zero", page=PAGE):
    """Shuffled page pool: pages assigned b-major from one random permutation."""
    nblk = [(int(L) + page - 1) // page for L in seqlens]
    used = sum(nblk)
    num_blocks = max(1, used + extra_pages)
    perm = rng.permutation(num_blocks).astype(np.int32)
    maxblk = max(1, max(nblk) if nblk else 1)
    if padding == "zero":
        bt = np.zeros((len(seqlens), maxblk), dtype=np.int32)
    elif padding == "oob":   # entries past a sequence's pages are never read
        bt = np.full((len(seqlens), maxblk), 0x7FFFFFF0, dtype=np.int32)
    else:
        raise ValueError(padding)
    o = 0
    for b, n in enumerate(nblk):
        bt[b, :n] = perm[o:o + n]
        o += n
    return bt, num_blocks


def make_workload(*, name="custom", seqlens: Sequence[int], s_q=1, num_heads_q=16, num_heads_k=1,
                  causal=False, kv_dtype="bf16", seed=0, q_mul=1.0, extra_pages=0,
                  padding="zero", rng: Optional[np.random.Generator] = None,
                  block_table: Optional[np.ndarray] = None, num_blocks: Optional[int] = None,
                  page_block_size: int = PAGE) -> Workload:
    """General seeded workload.  Draw order: (lengths drawn by caller), permutation, q, cache.
    page_block_size: tokens per cache block (64 unless a test asks for another)."""
    rng = rng if rng is not None else np.random.Generator(np.random.PCG64(seed))
    seqlens = np.asarray(seqlens, dtype=np.int32)
    B = int(seqlens.shape[0])
    if block_table is None:
        bt, nb = _page_pool(rng, seqlens, num_heads_k, extra_pages, padding, page_block_size)
    else:
        bt, nb = np.ascontiguousarray(block_table, dtype=np.int32), int(num_blocks)
    q = _normal_bf16(rng, B * s_q * num_heads_q * HEAD_DIM, q_mul).reshape(B, s_q, num_heads_q, HEAD_DIM)
    nkv = nb * page_block_size * num_heads_k * HEAD_DIM
    k_scale = v_scale = 1.0
    if kv_dtype == "bf16":
        kv = _normal_bf16(rng, nkv)
    elif kv_dtype == "fp8_e4m3fn":
        kv, s = _normal_e4m3fn(rng, nkv)
        k_scale = v_scale = s            # K and V are the same cached rows
    else:
        raise ValueError(kv_dtype)
    kv = kv.reshape(nb, page_block_size, num_heads_k, HEAD_DIM)
    return Workload(name=name, batch=B, s_q=s_q, num_heads_q=num_heads_q, num_heads_k=num_heads_k,
                    cache_seqlens=seqlens, block_table=bt, q_bits=q, kv=kv, kv_dtype=kv_dtype,
                    causal=causal, k_scale=k_scale, v_scale=v_scale, page_block_size=page_block_size)


CONFIGS = {
    1: "tiny: B=2 s_q=1 H=16 L={127,300}, 8-page pool, non-causal",
    2: "standard: B=64 s_q=1 H=128 L~U[1024,4096]",
    3: "mtp-causal: B=128 s_q=2 H=128 L~U[2048,8192] causal, q*0.5",
    4: "skewed: B=32 s_q=1 H=16, one 65536 + 31 lognormal(512, 1.0) in [1,8192]",
    5: "fp8: B=128 s_q=1 H=128 L=8192 e4m3fn cache",
}


def make_config(cfg: int, seed: Optional[int] = None, *, padding="zero", long_at_end=False) -> Workload:
    """The five decode workloads, seeded (default seed = config number)."""
    seed = cfg if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    if cfg == 1:
        seqlens = np.array([127, 300], dtype=np.int32)
        perm = rng.permutation(8).astype(np.int32)
        bt = np.empty((2, 5), dtype=np.int32)
        bt[0, :2] = perm[0:2]
        bt[0, 2:] = perm[7] if padding == "zero" else 0x7FFFFFF0
        bt[1, :] = perm[2:7]
        return make_workload(name="c1_tiny", seqlens=seqlens, num_heads_q=16, rng=rng,
                             block_table=bt, num_blocks=8)
    if cfg == 2:
        seqlens = rng.integers(1024, 4096 + 1, size=64).astype(np.int32)
        return make_workload(name="c2_standard", seqlens=seqlens, num_heads_q=128, rng=rng, padding=padding)
    if cfg == 3:
        seqlens = rng.integers(2048, 8192 + 1, size=128).astype(np.int32)
        return make_workload(name="c3_mtp_causal", seqlens=seqlens, s_q=2, num_heads_q=128, causal=True,
                             q_mul=0.5, rng=rng, padding=padding)
    if cfg == 4:
        z = rng.standard_normal(31)
        rest = np.clip(np.rint(np.exp(math.log(512.0) + 1.0 * z)), 1, 8192).astype(np.int32)
        seqlens = np.concatenate([rest, [65536]]) if long_at_end else np.concatenate([[65536], rest])
        return make_workload(name="c4_skewed", seqlens=seqlens.astype(np.int32), num_heads_q=16, rng=rng,
                             padding=padding)
    if cfg == 5:
        seqlens = np.full(128, 8192, dtype=np.int32)
        return make_workload(name="c5_fp8", seqlens=seqlens, num_heads_q=128, kv_dtype="fp8_e4m3fn",
                             rng=rng, padding=padding)
    raise ValueError(f"unknown config {cfg}")


def repage(w: Workload, page_block_size: int, seed: int = 0, pad: str = "nan") -> Workload:
    """The same workload with its cache re-laid in blocks of page_block_size tokens.

    Token t of sequence b keeps its row; the sequence's blocks come from a
    fresh seeded permutation of the new pool.  Rows of a last block past the
    sequence's end are filled per ``pad``: "nan" (bf16 0x7FC0 / e4m3fn 0x7F,
    so that any use of them shows), or "oob" = table entries past a
    sequence's blocks set to 0x7FFFFFF0 as well.
    """
    P = int(page_block_size)
    rng = np.random.Generator(np.random.PCG64(seed))
    nblk = [(int(L) + P - 1) // P for L in w.cache_seqlens]
    nb = max(1, sum(nblk))
    perm = rng.permutation(nb).astype(np.int32)
    fill = 0x7FC0 if w.kv.dtype == np.uint16 else 0x7F
    kv = np.full((nb, P) + w.kv.shape[2:], fill, dtype=w.kv.dtype)
    bt = np.zeros((w.batch, max(1, max(nblk) if nblk else 1)), dtype=np.int32)
    if pad == "oob":
        bt[:] = 0x7FFFFFF0
    old = w.page_block_size
    o = 0
    for b, n in enumerate(nblk):
        L = int(w.cache_seqlens[b])
        if L == 0:
            continue
        rows = np.concatenate([w.kv[w.block_table[b, j]] for j in range((L + old - 1) // old)])[:L]
        for j in range(n):
            blk = perm[o + j]
            bt[b, j] = blk
            seg = rows[j * P:(j + 1) * P]
            kv[blk, :seg.shape[0]] = seg
        o += n
    return dataclasses.replace(w, name=f"{w.name}_ps{P}", block_table=bt, kv=kv, page_block_size=P)


def batch_share(w: Workload, n: int, index: int = 0) -> Workload:
    """One GPU's share when the batch is split evenly over n GPUs (data-
    parallel attention): sequences index*B/n .. (index+1)*B/n - 1, their q
    rows, and only their cache blocks, renumbered in pool order (the shuffled
    placement is kept).  Table entries past a sequence's blocks become 0."""
    if n < 1 or w.batch % n or not 0 <= index < n:
        raise ValueError(f"batch {w.batch} does not split into {n} equal shares")
    Bs = w.batch // n
    rows = slice(index * Bs, (index + 1) * Bs)
    P = w.page_block_size
    L = w.cache_seqlens[rows]
    nblk = [(int(x) + P - 1) // P for x in L]
    bt_old = w.block_table[rows]
    used = np.unique(np.concatenate([bt_old[b, :nblk[b]] for b in range(Bs)] + [np.zeros(0, np.int32)]))
    used = used if used.size else np.zeros(1, np.int32)
    remap = np.zeros(w.num_blocks, dtype=np.int64)
    remap[used] = np.arange(used.size)
    bt = np.zeros((Bs, max(1, max(nblk) if nblk else 1)), dtype=np.int32)
    for b in range(Bs):
        bt[b, :nblk[b]] = remap[bt_old[b, :nblk[b]]]
    return dataclasses.replace(w, name=f"{w.name}_share{index}of{n}", batch=Bs, cache_seqlens=L.copy(),
                               block_table=bt, q_bits=w.q_bits[rows].copy(), kv=w.kv[used])
