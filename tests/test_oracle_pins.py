"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

Each test would fail on a plausible slip in the oracle: a wrong V slice, a
missing scale, a transposed head mapping, a mis-aligned causal mask, a paged
gather that indexes the wrong axis, a wrong fp8 exponent bias.
"""
import math

import numpy as np
import pytest
import torch

from oracle import (E4M3FN_TABLE, attend, bf16_bits_to_f64, decode_kv, fused_fp8_scales,
                    gather_rows, lse_merge, mla_decode, mla_decode_f64, visible_keys)
from workloads import bf16_bits_from_f32, make_config, make_workload, repage

D, DV = 576, 512


def _same_nan(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.array_equal(np.isnan(a), np.isnan(b)) and np.array_equal(a[~np.isnan(a)], b[~np.isnan(b)])


# ------------------------------------------------------------------ P1/P2 formats

def test_bf16_decode_all_codes_match_torch():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = bf16_bits_to_f64(codes)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert _same_nan(ours, ref)


def test_e4m3fn_table_matches_torch_and_format_landmarks():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert _same_nan(E4M3FN_TABLE, ref)
    assert E4M3FN_TABLE[0x7E] == 448.0            # largest finite
    assert E4M3FN_TABLE[0x01] == 2.0 ** -9        # smallest subnormal
    assert E4M3FN_TABLE[0x08] == 2.0 ** -6        # smallest normal
    assert E4M3FN_TABLE[0x38] == 1.0              # exponent bias 7
    assert math.isnan(E4M3FN_TABLE[0x7F]) and math.isnan(E4M3FN_TABLE[0xFF])
    assert np.isfinite(E4M3FN_TABLE[[c for c in range(256) if c & 0x7F != 0x7F]]).all()
    assert E4M3FN_TABLE[0xC0] == -2.0


def test_generator_bf16_rounding_is_rne():
    x = np.random.default_rng(0).standard_normal(1 << 16).astype(np.float32)
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 2 ** -130]   # ties and a subnormal
    ours = bf16_bits_from_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


# ------------------------------------------------------------------ P3 brute force

def _brute(q, kv, bt, seqlens, Hk, scale, causal, v_scale=1.0):
    """Scalar loops with math.fsum; token t of b lives at kv[bt[b][t // P]][t % P]."""
    B, s_q, H, Dq = q.shape
    P = kv.shape[1]
    G = H // Hk
    out = np.zeros((B, s_q, H, DV))
    lse = np.full((B, H, s_q), -np.inf)
    for b in range(B):
        L = int(seqlens[b])
        for i in range(s_q):
            n = L - (s_q - 1 - i) if causal else L
            n = max(0, min(L, n))
            for h in range(H):
                hk = h // G
                if n == 0:
                    continue
                rows = [kv[bt[b][t // P]][t % P][hk] for t in range(n)]
                s = [scale * math.fsum(float(q[b, i, h, d]) * float(r[d]) for d in range(Dq)) for r in rows]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                Z = math.fsum(e)
                for d in range(DV):
                    out[b, i, h, d] = v_scale * math.fsum(e[t] * float(rows[t][d]) for t in range(n)) / Z
                lse[b, h, i] = m + math.log(Z)
    return out, lse


@pytest.mark.parametrize("causal,s_q,Hk,P", [(False, 1, 1, 4), (True, 2, 1, 4), (True, 2, 2, 3), (False, 2, 2, 64)])
def test_oracle_equals_bruteforce_on_tiny_inputs(causal, s_q, Hk, P):
    rng = np.random.default_rng(7 + s_q + Hk + P)
    seqlens = np.array([9, 1, 0, 5], dtype=np.int32)
    B, H = len(seqlens), 4
    nblk = [-(-int(L) // P) for L in seqlens]
    nb = sum(nblk) + 2
    perm = rng.permutation(nb)
    bt = np.full((B, max(nblk)), nb - 1, dtype=np.int32)
    o = 0
    for b, n in enumerate(nblk):
        bt[b, :n] = perm[o:o + n]
        o += n
    q_bits = bf16_bits_from_f32(rng.standard_normal((B, s_q, H, D)).astype(np.float32)).reshape(B, s_q, H, D)
    kv_bits = bf16_bits_from_f32(rng.standard_normal((nb, P, Hk, D)).astype(np.float32)).reshape(nb, P, Hk, D)
    scale = D ** -0.5
    out, lse = mla_decode(q_bits, kv_bits, "bf16", bt, seqlens, DV, scale, causal)
    bo, bl = _brute(bf16_bits_to_f64(q_bits), bf16_bits_to_f64(kv_bits), bt, seqlens, Hk, scale, causal)
    assert np.allclose(out, bo, rtol=1e-12, atol=1e-13)
    fin = np.isfinite(bl)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.allclose(lse[fin], bl[fin], rtol=1e-12, atol=1e-13)
    assert (lse[~fin] == -np.inf).all() and (out[2] == 0).all()


# ------------------------------------------------------------------ closed forms

def _contig(rows, P=64):
    """Put (L, Hk, D) rows into a contiguous page pool with identity block table."""
    L = rows.shape[0]
    nblk = max(1, -(-L // P))
    kv = np.zeros((nblk, P) + rows.shape[1:])
    kv.reshape(nblk * P, *rows.shape[1:])[:L] = rows
    return kv, np.arange(nblk, dtype=np.int32)[None, :]


def _run_f64(q, rows_list, Hk, scale, causal=False, v_scale=1.0):
    seqlens = np.array([r.shape[0] for r in rows_list], dtype=np.int32)
    return mla_decode_f64(q, lambda b: rows_list[b], seqlens, Hk, DV, scale, causal, v_scale)


@pytest.mark.parametrize("n", [1, 2, 63, 64, 65, 1000])
def test_identical_rows_give_value_row_and_log_n(n):
    rng = np.random.default_rng(n)
    k = rng.standard_normal(D)
    q = rng.standard_normal((1, 1, 8, D))
    rows = np.tile(k, (n, 1, 1))
    scale, vs = 1 / 24, 0.37
    out, lse = _run_f64(q, [rows], 1, scale, v_scale=vs)
    assert np.allclose(out[0, 0], vs * k[:DV][None, :], rtol=1e-13, atol=1e-14)
    assert np.allclose(lse[0, :, 0], math.log(n) + scale * (q[0, 0] @ k), rtol=1e-13, atol=1e-13)


def test_zero_latent_query_gives_mean_of_distinct_values():
    rng = np.random.default_rng(5)
    n = 300
    q = rng.standard_normal((1, 1, 4, D))
    q[..., :DV] = 0.0
    kr = rng.standard_normal(64)
    rows = rng.standard_normal((n, 1, D))
    rows[:, 0, DV:] = kr
    out, lse = _run_f64(q, [rows], 1, 1 / 24)
    assert np.allclose(out[0, 0], rows[:, 0, :DV].mean(axis=0)[None, :], rtol=1e-12, atol=1e-14)
    assert np.allclose(lse[0, :, 0], math.log(n) + (q[0, 0, :, DV:] @ kr) / 24, rtol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_scale_gives_mean_over_visible_keys(causal):
    rng = np.random.default_rng(11)
    L, s_q = 130, 3
    rows = rng.standard_normal((L, 1, D))
    q = rng.standard_normal((1, s_q, 2, D))
    out, lse = _run_f64(q, [rows], 1, 0.0, causal=causal)
    for i in range(s_q):
        n = L - (s_q - 1 - i) if causal else L
        assert np.allclose(out[0, i], rows[:n, 0, :DV].mean(axis=0)[None, :], rtol=1e-12, atol=1e-14)
        assert np.allclose(lse[0, :, i], math.log(n), rtol=1e-14)


def test_one_and_two_keys():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 1, 3, D))
    k0, k1 = rng.standard_normal(D), rng.standard_normal(D)
    out, lse = _run_f64(q, [k0[None, None, :]], 1, 0.5)
    assert np.allclose(out[0, 0], k0[None, :DV], rtol=1e-14)
    assert np.allclose(lse[0, :, 0], 0.5 * q[0, 0] @ k0, rtol=1e-14)
    out, lse = _run_f64(q, [np.stack([k0, k1])[:, None, :]], 1, 0.5)
    s0, s1 = 0.5 * q[0, 0] @ k0, 0.5 * q[0, 0] @ k1
    p0 = 1 / (1 + np.exp(s1 - s0))
    assert np.allclose(out[0, 0], p0[:, None] * k0[None, :DV] + (1 - p0)[:, None] * k1[None, :DV], rtol=1e-12)
    assert np.allclose(lse[0, :, 0], np.logaddexp(s0, s1), rtol=1e-14)


def test_golden_hand_example():
    """tests/golden/hand_two_keys.txt: q.k0 scaled = ln 3, q.k1 = 0 -> weights 3/4, 1/4."""
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "hand_two_keys.txt")
    vals = {}
    for line in open(path):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split("=")
            vals[k.strip()] = float(v)
    q = np.zeros((1, 1, 1, D))
    q[0, 0, 0, 0] = vals["q0"]
    k0 = np.zeros(D)
    k0[0] = 1.0
    k1 = np.zeros(D)
    k1[DV] = 5.0                                  # rope-only key: contributes 0 to V and q.k
    out, lse = _run_f64(q, [np.stack([k0, k1])[:, None, :]], 1, vals["scale"])
    assert abs(out[0, 0, 0, 0] - vals["out0"]) < 1e-15
    assert np.abs(out[0, 0, 0, 1:]).max() == 0.0
    assert abs(lse[0, 0, 0] - vals["lse"]) < 1e-15


# ------------------------------------------------------------------ invariances

def test_paging_layout_is_bitwise_invisible():
    w = make_workload(seqlens=[200, 64, 1, 129], num_heads_q=8, seed=9, extra_pages=3)
    out1, lse1 = mla_decode(w.q_bits, w.kv, "bf16", w.block_table, w.cache_seqlens, DV, 1 / 24)
    # rebuild the same logical sequences in a contiguous pool with an identity table
    pools, tables, o = [], [], 0
    maxblk = w.block_table.shape[1]
    for b in range(w.batch):
        n = int(w.nblk()[b])
        pools.append(w.kv[w.block_table[b, :n]])
        tables.append(list(range(o, o + n)) + [0] * (maxblk - n))
        o += n
    kv2 = np.concatenate(pools)
    out2, lse2 = mla_decode(w.q_bits, kv2, "bf16", np.array(tables, dtype=np.int32), w.cache_seqlens, DV, 1 / 24)
    assert np.array_equal(out1, out2) and np.array_equal(lse1, lse2)


@pytest.mark.parametrize("causal", [False, True])
def test_split_merge_equals_unsplit(causal):
    rng = np.random.default_rng(21)
    L, s_q, G = 517, 2, 6
    rows = rng.standard_normal((L, 1, D))
    q = rng.standard_normal((1, s_q, G, D))
    out, lse = _run_f64(q, [rows], 1, 1 / 24, causal=causal)
    for trial in range(3):
        cuts = np.sort(rng.choice(np.arange(1, L), size=5 + trial, replace=False))
        bounds = [0, *cuts.tolist(), L]
        for i in range(s_q):
            n = visible_keys(L, s_q, i, causal)
            parts = [attend(q[0, i], rows[a:min(c, n), 0], rows[a:min(c, n), 0, :DV], 1 / 24)
                     for a, c in zip(bounds[:-1], bounds[1:])]
            # ranges past the visible keys are empty -> lse -inf, zero weight
            mo, ml = lse_merge([p[0] for p in parts], [p[1] for p in parts])
            assert np.allclose(mo, out[0, i], rtol=1e-12, atol=1e-15)
            assert np.allclose(ml, lse[0, :, i], rtol=1e-13)


def test_lse_merge_all_empty_is_zero_and_minus_inf():
    o, l = lse_merge([np.ones((2, DV)), np.ones((2, DV))], [np.full(2, -np.inf), np.full(2, -np.inf)])
    assert (o == 0).all() and (l == -np.inf).all()


def test_causal_mtp_alignment():
    rng = np.random.default_rng(4)
    L = 70
    rows = rng.standard_normal((L, 1, D))
    q = rng.standard_normal((1, 2, 4, D))
    out, lse = _run_f64(q, [rows], 1, 1 / 24, causal=True)
    nc0 = _run_f64(q[:, :1], [rows[:L - 1]], 1, 1 / 24)
    nc1 = _run_f64(q[:, 1:], [rows], 1, 1 / 24)
    assert np.array_equal(out[0, 0], nc0[0][0, 0]) and np.array_equal(lse[0, :, 0], nc0[1][0, :, 0])
    assert np.array_equal(out[0, 1], nc1[0][0, 0]) and np.array_equal(lse[0, :, 1], nc1[1][0, :, 0])
    # spike: a huge last key aligned with query 0 must not move query 0, must move query 1
    rows2 = rows.copy()
    rows2[L - 1, 0] = 50 * q[0, 0, 0] / np.linalg.norm(q[0, 0, 0])
    out2, _ = _run_f64(q, [rows2], 1, 1 / 24, causal=True)
    assert np.array_equal(out2[0, 0], out[0, 0])
    assert not np.allclose(out2[0, 1], out[0, 1])
    assert visible_keys(5, 2, 0, True) == 4 and visible_keys(1, 3, 0, True) == 0


def test_token_order_invariance_noncausal():
    rng = np.random.default_rng(8)
    rows = rng.standard_normal((333, 1, D))
    q = rng.standard_normal((1, 1, 5, D))
    a = _run_f64(q, [rows], 1, 1 / 24)
    b = _run_f64(q, [rows[rng.permutation(333)]], 1, 1 / 24)
    assert np.allclose(a[0], b[0], rtol=1e-12, atol=1e-15) and np.allclose(a[1], b[1], rtol=1e-13)


def test_head_permutation_and_grouped_heads():
    rng = np.random.default_rng(12)
    L, Hk, G = 100, 2, 3
    rows = rng.standard_normal((L, Hk, D))
    q = rng.standard_normal((1, 1, Hk * G, D))
    out, lse = _run_f64(q, [rows], Hk, 1 / 24)
    for hk in range(Hk):                          # H_k > 1 == H_k independent single-head problems
        o1, l1 = _run_f64(q[:, :, hk * G:(hk + 1) * G], [rows[:, hk:hk + 1]], 1, 1 / 24)
        assert np.array_equal(out[0, 0, hk * G:(hk + 1) * G], o1[0, 0])
        assert np.array_equal(lse[0, hk * G:(hk + 1) * G], l1[0])
    perm = rng.permutation(G)                     # permuting q heads within a group permutes outputs
    o2, l2 = _run_f64(q[:, :, perm], [rows[:, :1]], 1, 1 / 24)
    o1, l1 = _run_f64(q[:, :, :G], [rows[:, :1]], 1, 1 / 24)
    assert np.array_equal(o2[0, 0], o1[0, 0][perm]) and np.array_equal(l2[0, :, 0], l1[0, :, 0][perm])


# ------------------------------------------------------------------ fp8

def test_fused_scale_formula_and_fp8_dequant_equivalence():
    b1, b2 = fused_fp8_scales(q_scale=2.0, k_scale=0.5, v_scale=3.0, o_scale=0.25, sm_scale=1.5, head_dim_qk=576)
    assert b1 == 2.0 * 0.5 * 1.5 / 24.0 and b2 == 0.75
    w = make_workload(seqlens=[70, 3], num_heads_q=4, kv_dtype="fp8_e4m3fn", seed=13)
    s = w.k_scale
    bmm1, bmm2 = fused_fp8_scales(k_scale=s, v_scale=s)
    out, lse = mla_decode(w.q_bits, w.kv, "fp8_e4m3fn", w.block_table, w.cache_seqlens, DV, bmm1, False, bmm2)
    deq = s * E4M3FN_TABLE[w.kv]
    q = bf16_bits_to_f64(w.q_bits)
    ref = mla_decode_f64(q, lambda b: gather_rows(deq, w.block_table[b], int(w.cache_seqlens[b]), 64),
                         w.cache_seqlens, 1, DV, 1 / 24, False, 1.0)
    assert np.allclose(out, ref[0], rtol=1e-12, atol=1e-15) and np.allclose(lse, ref[1], rtol=1e-12)
    assert np.abs(s * E4M3FN_TABLE[w.kv]).max() <= 448 * s * (1 + 1e-12)


def test_tolerance_is_reachable_by_bf16_rounded_output():
    w = make_config(1)
    out, lse = mla_decode(w.q_bits, w.kv, "bf16", w.block_table, w.cache_seqlens, DV, 576 ** -0.5)
    rounded = bf16_bits_to_f64(bf16_bits_from_f32(out.astype(np.float32)))
    assert np.abs(rounded - out).max() <= 1e-2 * np.abs(out).max() + 1e-3
    assert np.abs(lse.astype(np.float32) - lse).max() <= 2e-3


def test_config1_shapes_and_pool():
    w = make_config(1)
    assert w.block_table.shape == (2, 5) and w.num_blocks == 8
    used = set(w.block_table[0, :2].tolist()) | set(w.block_table[1].tolist())
    assert len(used) == 7 and used <= set(range(8))
    assert w.q_bits.shape == (2, 1, 16, 576) and w.kv.shape == (8, 64, 1, 576)


# ------------------------------------------------------------------ attention sinks
# FlashInfer MLA page, ``sinks``: a per-head extra term of the softmax
# denominator, read as a logit on the scale of softmax_scale * q.k.

def _sink_workload():
    return make_workload(seqlens=[300, 1, 0, 129], num_heads_q=8, s_q=2, seed=31)


@pytest.mark.parametrize("causal", [False, True])
def test_sink_of_minus_inf_is_no_sink(causal):
    w = _sink_workload()
    o1, l1 = mla_decode(w.q_bits, w.kv, "bf16", w.block_table, w.cache_seqlens, DV, 1 / 24, causal)
    o2, l2 = mla_decode(w.q_bits, w.kv, "bf16", w.block_table, w.cache_seqlens, DV, 1 / 24, causal,
                        sinks=np.full(8, -np.inf))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("causal", [False, True])
def test_sink_adds_one_denominator_term_per_head(causal):
    """With sink logit z_h: lse' = logaddexp(lse, z_h) and out' = out * exp(lse - lse') -- the
    no-sink result rescaled by the share of the keys in the enlarged denominator.  Distinct
    sinks per head catch a wrong head mapping; the empty sequence (L = 0) and the causal row
    with no key give lse' = z_h, out' = 0."""
    w = _sink_workload()
    sinks = np.linspace(-3.0, 4.0, 8)
    o1, l1 = mla_decode(w.q_bits, w.kv, "bf16", w.block_table, w.cache_seqlens, DV, 1 / 24, causal, v_scale=0.7)
    o2, l2 = mla_decode(w.q_bits, w.kv, "bf16", w.block_table, w.cache_seqlens, DV, 1 / 24, causal, v_scale=0.7,
                        sinks=sinks)
    z = sinks[None, :, None]                                  # lse is (B, H, s_q)
    assert np.allclose(l2, np.logaddexp(l1, z), rtol=1e-13, atol=1e-13)
    ratio = np.exp(l1 - l2)                                   # (B, H, s_q); 0 where l1 = -inf
    assert np.allclose(o2, o1 * np.transpose(ratio, (0, 2, 1))[..., None], rtol=1e-12, atol=1e-14)
    assert np.array_equal(l2[2], np.broadcast_to(z[0], (8, 2)))     # L = 0
    assert (o2[2] == 0).all()


def test_sink_single_key_closed_form():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 1, 2, D))
    k = rng.standard_normal(D)
    z = np.array([0.25, -1.5])
    out, lse = mla_decode_f64(q, lambda b: k[None, None, :], [1], 1, DV, 0.5, False, v_scale=2.0, sinks=z)
    s = 0.5 * q[0, 0] @ k
    for h in range(2):
        p = 1.0 / (1.0 + math.exp(z[h] - s[h]))                  # e^s / (e^s + e^z)
        assert np.allclose(out[0, 0, h], 2.0 * p * k[:DV], rtol=1e-13)
        assert abs(lse[0, h, 0] - math.log(math.exp(s[h]) + math.exp(z[h]))) < 1e-13


def test_dominant_sink_silences_the_keys():
    w = _sink_workload()
    o, l = mla_decode(w.q_bits, w.kv, "bf16", w.block_table, w.cache_seqlens, DV, 1 / 24, sinks=np.full(8, 200.0))
    assert np.abs(o).max() < 1e-40
    assert np.allclose(l, 200.0, rtol=0, atol=1e-12)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3fn"])
@pytest.mark.parametrize("P", [16, 48, 128])
def test_block_size_is_bitwise_invisible(kv_dtype, P):
    """The same token rows in blocks of P tokens, with NaN in the rows past each
    sequence's end, give bitwise the oracle's 64-token-block result."""
    w = make_workload(seqlens=[0, 1, 17, 64, 65, 300, 129], num_heads_q=8, s_q=2, causal=True,
                      kv_dtype=kv_dtype, seed=23)
    r = repage(w, P, seed=4, pad="oob")
    assert r.kv.shape[1] == P
    s = 1 / 24
    o1, l1 = mla_decode(w.q_bits, w.kv, kv_dtype, w.block_table, w.cache_seqlens, DV, s, True)
    o2, l2 = mla_decode(r.q_bits, r.kv, kv_dtype, r.block_table, r.cache_seqlens, DV, s, True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_product_fp8_scale_helper_equals_the_oracle():
    """The package's fp8_fused_scales (argument marshalling for callers) and the
    oracle's fused_fp8_scales follow the same note of the FlashInfer MLA page;
    they must agree exactly for any inputs."""
    import mla_paged_kv_metadata_amd as mla
    rng = np.random.default_rng(17)
    for _ in range(50):
        qs, ks, vs, os_, sm = rng.uniform(0.01, 4.0, 5)
        hd = int(rng.choice([64, 192, 576]))
        a = mla.fp8_fused_scales(q_scale=qs, k_scale=ks, v_scale=vs, o_scale=os_, sm_scale=sm, head_dim_qk=hd)
        b = fused_fp8_scales(q_scale=qs, k_scale=ks, v_scale=vs, o_scale=os_, sm_scale=sm, head_dim_qk=hd)
        assert a == b


# ------------------------------------------------------------------ fp8 query, per-head descales

def _e4m3_codes(rng, shape):
    """Random finite e4m3fn codes of moderate magnitude (exponent field 3..10,
    so |value| lies in [2^-4, 2^4)), both signs."""
    e = rng.integers(3, 11, size=shape)
    m = rng.integers(0, 8, size=shape)
    sgn = rng.integers(0, 2, size=shape)
    return ((sgn << 7) | (e << 3) | m).astype(np.uint8)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3fn"])
def test_fp8_query_dequantise_then_attend(kv_dtype):
    """An e4m3 query with q_scale folded into bmm1 (FlashInfer MLA page, note on
    fused scales) equals the bf16 query q_scale * code with the plain scale: a
    power-of-two q_scale keeps every q_scale * code exact in bf16."""
    w = make_workload(seqlens=[70, 3, 130], num_heads_q=8, kv_dtype=kv_dtype, seed=23)
    rng = np.random.default_rng(24)
    codes = _e4m3_codes(rng, w.q_bits.shape)
    q_scale = 2.0 ** -3
    base = 1 / 24 if kv_dtype == "bf16" else w.k_scale / 24
    vs = 1.0 if kv_dtype == "bf16" else w.v_scale
    o1, l1 = mla_decode(codes, w.kv, kv_dtype, w.block_table, w.cache_seqlens, DV, q_scale * base, False, vs,
                        q_format="fp8_e4m3fn")
    qv = (q_scale * E4M3FN_TABLE[codes]).astype(np.float32)
    qb = bf16_bits_from_f32(qv)
    assert np.array_equal(bf16_bits_to_f64(qb), q_scale * E4M3FN_TABLE[codes])     # exact in bf16
    o2, l2 = mla_decode(qb, w.kv, kv_dtype, w.block_table, w.cache_seqlens, DV, base, False, vs)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-14) and np.allclose(l1, l2, rtol=1e-12, atol=1e-14)
    # and the codes really matter: a wrong decode of the query changes the result
    o3, _ = mla_decode(codes.astype(np.uint16), w.kv, kv_dtype, w.block_table, w.cache_seqlens, DV, base, False,
                       vs)
    assert not np.allclose(o1, o3)


def test_fp8_query_and_cache_equal_dequantised_operands():
    """Both operands as codes with the fused scales equal dequantise-then-attend
    with scale 1/sqrt(576) and unit v_scale (P13 with a quantised query)."""
    w = make_workload(seqlens=[40, 90], num_heads_q=4, kv_dtype="fp8_e4m3fn", seed=25)
    codes = _e4m3_codes(np.random.default_rng(26), w.q_bits.shape)
    q_s = 0.37
    b1, b2 = fused_fp8_scales(q_scale=q_s, k_scale=w.k_scale, v_scale=w.v_scale)
    o1, l1 = mla_decode(codes, w.kv, "fp8_e4m3fn", w.block_table, w.cache_seqlens, DV, b1, False, b2,
                        q_format="fp8_e4m3fn")
    q = q_s * E4M3FN_TABLE[codes]
    deq = w.k_scale * E4M3FN_TABLE[w.kv]
    o2, l2 = mla_decode_f64(q, lambda b: gather_rows(deq, w.block_table[b], int(w.cache_seqlens[b]), 64),
                            w.cache_seqlens, 1, DV, 1 / 24, False, 1.0)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-14) and np.allclose(l1, l2, rtol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_qk_descale_equals_a_per_head_scaled_query(causal):
    """qkDescale[h] (Ascend ATB MLA page) multiplies head h's scores: with
    power-of-two factors this equals scaling head h's query rows exactly.
    Distinct factors per head and two KV heads catch a wrong head mapping."""
    w = make_workload(seqlens=[50, 1, 129], s_q=2, num_heads_q=8, num_heads_k=2, causal=causal, seed=27)
    d = 2.0 ** np.array([-2, -1, 0, 1, 2, 0, -1, 1], dtype=np.float64)
    o1, l1 = mla_decode(w.q_bits, w.kv, "bf16", w.block_table, w.cache_seqlens, DV, 1 / 24, causal,
                        qk_descale=d)
    qd = bf16_bits_to_f64(w.q_bits) * d[None, None, :, None]
    qb = bf16_bits_from_f32(qd.astype(np.float32))
    assert np.array_equal(bf16_bits_to_f64(qb), qd)
    o2, l2 = mla_decode(qb, w.kv, "bf16", w.block_table, w.cache_seqlens, DV, 1 / 24, causal)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-14)
    fin = np.isfinite(l2)
    assert np.array_equal(fin, np.isfinite(l1)) and np.allclose(l1[fin], l2[fin], rtol=1e-12)
    o0, _ = mla_decode(w.q_bits, w.kv, "bf16", w.block_table, w.cache_seqlens, DV, 1 / 24, causal)
    assert not np.allclose(o0, o1)


def test_pv_descale_scales_the_output_only():
    """pvDescale[h] multiplies head h's output; lse does not depend on it."""
    w = make_workload(seqlens=[33, 200], num_heads_q=6, num_heads_k=2, seed=28)
    p = np.array([0.5, 2.0, 1.0, 3.0, -1.0, 0.25])
    o0, l0 = mla_decode(w.q_bits, w.kv, "bf16", w.block_table, w.cache_seqlens, DV, 1 / 24)
    o1, l1 = mla_decode(w.q_bits, w.kv, "bf16", w.block_table, w.cache_seqlens, DV, 1 / 24, pv_descale=p)
    assert np.allclose(o1, o0 * p[None, None, :, None], rtol=1e-14, atol=0)
    assert np.array_equal(l1, l0)


def test_descales_leave_sinks_unscaled():
    """A sink is a logit on the softmax's own scale: qkDescale scales the scores
    and not the sink, so with one key the weight of the key is
    e^(d s) / (e^(d s) + e^z)."""
    w = make_workload(seqlens=[1], num_heads_q=2, seed=29)
    d = np.array([2.0, 0.5])
    z = np.array([0.3, -1.0])
    o, l = mla_decode(w.q_bits, w.kv, "bf16", w.block_table, w.cache_seqlens, DV, 1 / 24, sinks=z, qk_descale=d)
    k = bf16_bits_to_f64(w.kv[w.block_table[0, 0], 0, 0])
    q = bf16_bits_to_f64(w.q_bits[0, 0])
    s = d * (q @ k) / 24
    wk = np.exp(s) / (np.exp(s) + np.exp(z))
    assert np.allclose(o[0, 0], wk[:, None] * k[None, :DV], rtol=1e-12)
    assert np.allclose(l[0, :, 0], np.logaddexp(s, z), rtol=1e-12)
