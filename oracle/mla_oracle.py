"""Plain fp64 oracle for MLA decode over a paged KV cache.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg; never by the library.  It shares no code with
the HIP path.  Everything is float64 NumPy with no blocking, fusion or
reordering beyond the definition: gather the pages, scale q.k, softmax,
weighted sum of V.

What it follows (page titles as cited everywhere in this repository):
  * FlashMLA interface page (flash_mla_interface.py), docstring of
    ``flash_mla_with_kvcache``: q (B, s_q, H_q, D), k_cache
    (num_blocks, page_block_size, H_k, D), block_table (B, max_blocks) int32,
    cache_seqlens (B,) int32, head_dim_v, softmax_scale "scaling of QK^T
    before softmax, default 1/sqrt(head_dim)", causal flag; returns out
    (B, s_q, H_q, head_dim_v) and softmax_lse (B, H_q, s_q) float32 -- the log
    of the softmax sum.  The wrapper passes no separate V cache, so V is read
    from the same cached rows.
  * vLLM ``vllm.attention.ops.flashmla`` page: the same signature and shapes.
  * FlashInfer ``trtllm_batch_decode_with_kv_cache_mla`` page: query is
    q_nope ++ q_rope (512 + 64), kv_cache is ckv ++ kpe, so V = the first 512
    (kv_lora_rank) columns; note on fused scales
    bmm1 = q_scale*k_scale*sm_scale/sqrt(head_dim_qk), bmm2 = v_scale*o_scale;
    ``sinks``, a per-head extra term of the softmax denominator.

Readings where the pages are silent (each is listed with its reason in the
design notes): natural-log lse with the scale inside the exponent; bottom-right
causal alignment (query i of s_q sees keys t < L - s_q + 1 + i); a row with no
visible key gives out = 0 and lse = -inf; q head h uses KV head h // (H_q/H_k);
a sink is a logit on the scale of softmax_scale * q.k, so head h's softmax
denominator gains exp(sink_h) (no value row goes with it) and lse includes it.
"""
from __future__ import annotations

import math

import numpy as np

# ---------------------------------------------------------------- formats


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 is the upper 16 bits of an IEEE-754 binary32; widen exactly to float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):         # NaN codes stay NaN
        return b.view(np.float32).astype(np.float64)


def e4m3fn_code_to_f64(code: int) -> float:
    """Value of one OCP FP8 E4M3 ("fn": finite, no infinities) code.

    Bit 7 sign, bits 6..3 exponent with bias 7, bits 2..0 mantissa.  Exponent 0
    encodes subnormals m/8 * 2^-6; the all-ones exponent with mantissa 7 is NaN
    (there is no infinity), every other code is normal (1 + m/8) * 2^(e-7).
    """
    s = -1.0 if (code >> 7) & 1 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3FN_TABLE = np.array([e4m3fn_code_to_f64(c) for c in range(256)], dtype=np.float64)


def decode_kv(raw: np.ndarray, kv_format: str) -> np.ndarray:
    """Cache codes -> float64.  bf16 bits (uint16) or e4m3fn codes (uint8, unscaled)."""
    if kv_format == "bf16":
        return bf16_bits_to_f64(raw)
    if kv_format == "fp8_e4m3fn":
        return E4M3FN_TABLE[np.asarray(raw, dtype=np.uint8)]
    raise ValueError(kv_format)


def fused_fp8_scales(q_scale=1.0, k_scale=1.0, v_scale=1.0, o_scale=1.0, sm_scale=1.0, head_dim_qk=576):
    """FlashInfer MLA page, note on fused scales: (bmm1_scale, bmm2_scale)."""
    return (q_scale * k_scale * sm_scale / math.sqrt(head_dim_qk), v_scale * o_scale)


# ---------------------------------------------------------------- attention


def visible_keys(L: int, s_q: int, i: int, causal: bool) -> int:
    """Number of cached keys query i (of s_q) may attend to.

    Non-causal: all L.  Causal: bottom-right aligned, the last query sees all L
    keys and query i sees L - (s_q - 1 - i); clamped at 0.
    """
    n = L - s_q + 1 + i if causal else L
    return max(0, min(L, n))


def gather_rows(kv: np.ndarray, block_table_row: np.ndarray, L: int, page_block_size: int) -> np.ndarray:
    """Paged gather: token t lives at kv[block_table_row[t // P], t % P]; returns rows 0..L-1 in order."""
    nblk = -(-L // page_block_size)
    if nblk == 0:
        return kv[:0].reshape((0,) + kv.shape[2:])
    pages = [kv[int(block_table_row[j])] for j in range(nblk)]
    return np.concatenate(pages, axis=0)[:L]


def attend(qh: np.ndarray, K: np.ndarray, V: np.ndarray, scale, v_scale=1.0, sink=None):
    """Softmax attention of query rows qh (G, D) over keys K (n, D), values V (n, Dv).

    Returns (out (G, Dv), lse (G,)) with lse = ln sum_j exp(scale * q.k_j).
    ``scale`` and ``v_scale`` are scalars or per-row (G,) factors (the per-head
    qkDescale / pvDescale of the Ascend ATB MLA page fold into them).
    n == 0 gives out = 0, lse = -inf.  With ``sink`` (G,) (FlashInfer MLA
    page, ``sinks``: a per-head extra term of the softmax denominator, read as
    a logit): the denominator is sum_j exp(s_j) + exp(sink), lse includes the
    sink term, and the sink carries no value.  A sink of -inf is no sink.
    """
    G = qh.shape[0]
    n = K.shape[0]
    scale = np.broadcast_to(np.asarray(scale, dtype=np.float64), (G,))[:, None]
    v_scale = np.broadcast_to(np.asarray(v_scale, dtype=np.float64), (G,))[:, None]
    if sink is None:
        if n == 0:
            return np.zeros((G, V.shape[1])), np.full(G, -np.inf)
        s = scale * (qh @ K.T)                  # (G, n)
        mx = s.max(axis=1, keepdims=True)
        e = np.exp(s - mx)
        Z = e.sum(axis=1, keepdims=True)
        out = v_scale * (e @ V) / Z
        lse = (mx + np.log(Z))[:, 0]
        return out, lse
    sink = np.asarray(sink, dtype=np.float64).reshape(G, 1)
    s = scale * (qh @ K.T) if n else np.zeros((G, 0))
    mx = np.maximum(s.max(axis=1, keepdims=True) if n else np.full((G, 1), -np.inf), sink)
    empty = ~np.isfinite(mx)                    # no key and no sink: out = 0, lse = -inf
    mx = np.where(empty, 0.0, mx)
    e = np.exp(s - mx)
    Z = e.sum(axis=1, keepdims=True) + np.exp(sink - mx)
    Zs = np.where(empty, 1.0, Z)
    out = np.where(empty, 0.0, v_scale * (e @ V[:n]) / Zs)
    lse = np.where(empty, -np.inf, mx + np.log(Zs))[:, 0]
    return out, lse


def lse_merge(outs, lses):
    """Merge attention results over disjoint key sets by their log-sum-exps.

    outs: list of (G, Dv) normalised outputs, lses: list of (G,).  A part with
    lse = -inf carries no weight.  Returns (out, lse) of the union.
    """
    L = np.stack(lses)                          # (k, G)
    O = np.stack(outs)                          # (k, G, Dv)
    mu = L.max(axis=0)                          # (G,)
    empty = ~np.isfinite(mu)
    mu_safe = np.where(empty, 0.0, mu)
    w = np.where(np.isfinite(L), np.exp(L - mu_safe), 0.0)
    Z = w.sum(axis=0)
    Zs = np.where(Z > 0, Z, 1.0)
    out = (w[:, :, None] * O).sum(axis=0) / Zs[:, None]
    lse = np.where(empty, -np.inf, mu_safe + np.log(Zs))
    out = np.where(empty[:, None], 0.0, out)
    return out, lse


def mla_decode_f64(q: np.ndarray, rows_of, cache_seqlens, num_heads_k: int, head_dim_v: int,
                   softmax_scale: float, causal: bool, v_scale: float = 1.0, batches=None, sinks=None,
                   qk_descale=None, pv_descale=None):
    """Core oracle on float64 operands.

    q: (B, s_q, H_q, D) float64.  rows_of(b) -> (L_b, H_k, D) float64, the
    sequence's cached rows in logical order.  Returns out (B, s_q, H_q, Dv) and
    lse (B, H_q, s_q) float64.  ``batches`` restricts the work to some b (the
    other entries stay 0 / -inf).  ``sinks``: None or (H_q,) per-head sink
    logits (see attend).  ``qk_descale`` / ``pv_descale``: None or (H_q,)
    per-head factors (Ascend ATB MLA page, qkDescale / pvDescale [num_heads]):
    head h's scores are softmax_scale * qk_descale[h] * q.k and its output is
    multiplied by v_scale * pv_descale[h]; lse follows the scores, the sink
    logits are not rescaled.
    """
    B, s_q, H, D = q.shape
    if H % num_heads_k:
        raise ValueError("num_heads_q must be a multiple of num_heads_k")
    G = H // num_heads_k
    qk = np.ones(H) if qk_descale is None else np.asarray(qk_descale, dtype=np.float64)
    pv = np.ones(H) if pv_descale is None else np.asarray(pv_descale, dtype=np.float64)
    out = np.zeros((B, s_q, H, head_dim_v))
    lse = np.full((B, H, s_q), -np.inf)
    for b in (range(B) if batches is None else batches):
        L = int(cache_seqlens[b])
        rows = rows_of(b)
        assert rows.shape[0] == L
        for i in range(s_q):
            n = visible_keys(L, s_q, i, causal)
            for hk in range(num_heads_k):
                K = rows[:n, hk, :]
                V = K[:, :head_dim_v]
                hs = slice(hk * G, (hk + 1) * G)
                o, l = attend(q[b, i, hs, :], K, V, softmax_scale * qk[hs], v_scale * pv[hs],
                              None if sinks is None else np.asarray(sinks, dtype=np.float64)[hs])
                out[b, i, hs, :] = o
                lse[b, hs, i] = l
    return out, lse


def mla_decode(q_bits, kv_raw, kv_format, block_table, cache_seqlens, head_dim_v, softmax_scale,
               causal=False, v_scale=1.0, batches=None, sinks=None, q_format="bf16", qk_descale=None,
               pv_descale=None):
    """Oracle on the raw input bytes the GPU also receives.

    q_bits: (B, s_q, H_q, D) uint16 bf16 bits, or uint8 e4m3fn codes when
    q_format is "fp8_e4m3fn" (FlashInfer MLA page, note on fused scales: an
    fp8 query's q_scale is folded into bmm1_scale, so the codes enter the
    product unscaled).  kv_raw: (num_blocks, P, H_k, D) uint16 bf16 bits or
    uint8 e4m3fn codes.  softmax_scale is the full factor on q.k (bmm1 for an
    fp8 cache); v_scale multiplies the weighted sum (bmm2).  qk_descale /
    pv_descale: see mla_decode_f64.  Only the pages a sequence uses are
    decoded.
    """
    q = decode_kv(q_bits, q_format)
    P = kv_raw.shape[1]
    Hk = kv_raw.shape[2]

    def rows_of(b):
        L = int(cache_seqlens[b])
        return decode_kv(gather_rows(kv_raw, block_table[b], L, P), kv_format)

    return mla_decode_f64(q, rows_of, cache_seqlens, Hk, head_dim_v, softmax_scale, causal, v_scale, batches,
                          sinks, qk_descale, pv_descale)
