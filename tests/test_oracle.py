"""Pins of the CPU oracle against things other than itself (CPU only).

Each test checks the oracle against a library routine, a closed form, an
invariant or brute force, chosen so that a dropped term, a wrong sign, index
or operand in the oracle fails at least one of them.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from workloads import as_bits, from_bits, rope_cos_sin_table

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_bits(rng, shape, scale=1.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return as_bits(torch.from_numpy(x).to(torch.bfloat16))


# ----------------------------------------------------------------- bf16 -----

def test_bf16_rne_matches_torch_cast():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(1_000_000).astype(np.float32)
    x *= np.exp2(rng.integers(-140, 120, size=x.size)).astype(np.float32)
    u = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    ties = ((u & np.uint32(0xFFFF0000)) | np.uint32(0x8000)).view(np.float32)
    specials = np.array([0.0, -0.0, np.inf, -np.inf, 3.4028235e38, -3.4028235e38,
                         1e-45, -1e-45, 1.1754944e-38, 3.3961776e38, 3.3961775e38,
                         1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20],
                        dtype=np.float32)
    raw = np.concatenate([x, ties, specials])
    finite = raw[np.isfinite(raw) | np.isinf(raw)]
    ref = as_bits(torch.from_numpy(finite).to(torch.bfloat16))
    got = oracle.f32_to_bf16_rne(finite)
    assert np.array_equal(got, ref)


def test_bf16_nan_is_canonical_quiet_nan():
    x = np.array([np.nan, -np.nan], dtype=np.float32)
    assert (oracle.f32_to_bf16_rne(x) == 0x7FC0).all()


def test_bf16_widening_is_exact_for_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = from_bits(bits).to(torch.float32).numpy()
    got = oracle.bf16_to_f32(bits)
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.array_equal(got[~both_nan].view(np.uint32), ref[~both_nan].view(np.uint32))
    assert np.array_equal(oracle.bf16_to_f64(bits)[~both_nan], ref[~both_nan].astype(np.float64))


def test_bf16_ulp_is_the_spacing_of_neighbours():
    bits = np.arange(0x0080, 0x7F7F, dtype=np.uint16)  # positive normals
    x = oracle.bf16_to_f64(bits)
    nxt = oracle.bf16_to_f64(bits + 1)
    assert np.array_equal(oracle.bf16_ulp(x), nxt - x)
    sub = oracle.bf16_to_f64(np.arange(1, 0x80, dtype=np.uint16))
    assert (oracle.bf16_ulp(sub) == 2.0 ** -133).all()


def test_f64_to_bf16_is_round_to_nearest_even():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(200_000) * np.exp2(rng.integers(-30, 30, size=200_000))
    y_bits = oracle.f64_to_bf16_rne(x)
    y = oracle.bf16_to_f64(y_bits)
    err = np.abs(y - x)
    half = oracle.bf16_ulp(x) / 2
    # exact halfway points of x's binade can also round up into the next one
    assert (err <= half * (1 + 1e-15)).all()
    tie = err == half
    assert (y_bits[tie] & 1 == 0).all()
    # for fp32-representable inputs a single rounding from fp64 equals the fp32 path
    x32 = x.astype(np.float32)
    assert np.array_equal(oracle.f64_to_bf16_rne(x32.astype(np.float64)), oracle.f32_to_bf16_rne(x32))


# ------------------------------------------------------ RoPE angle table ---

def test_rope_table_against_libm():
    D, theta = 128, 1e6
    tab = rope_cos_sin_table(theta, D, 8192).numpy()
    rng = np.random.default_rng(3)
    for _ in range(2000):
        p = int(rng.integers(0, 8192))
        j = int(rng.integers(0, D // 2))
        ang = p * math.pow(theta, -2.0 * j / D)
        for val, ref in ((tab[p, j], math.cos(ang)), (tab[p, D // 2 + j], math.sin(ang))):
            # within half an fp32 ulp of libm plus angle-rounding slack
            assert abs(float(val) - ref) <= 2 ** -24 * max(abs(ref), 2 ** -30) + 8 * p * 2 ** -52
    assert (tab[0, : D // 2] == 1.0).all() and (tab[0, D // 2:] == 0.0).all()
    # frequency of pair 0 is 1 rad per position
    p = np.arange(8192)
    assert np.allclose(tab[:, 0], np.cos(p), atol=1e-6)
    assert np.allclose(tab[:, D // 2], np.sin(p), atol=1e-6)


# -------------------------------------------------------------- RoPE -------

def _rotate_half_torch(x64, cos64, sin64):
    """rotate_half formulation: x*cos + rotate_half(x)*sin, rotate_half = (-x2, x1)."""
    x1, x2 = x64.chunk(2, dim=-1)
    rh = torch.cat([-x2, x1], dim=-1)
    return x64 * torch.cat([cos64, cos64], -1) + rh * torch.cat([sin64, sin64], -1)


def test_rope_position_zero_is_identity_bit_exact():
    rng = np.random.default_rng(4)
    x = _rand_bits(rng, (50, 128))
    tab = rope_cos_sin_table(1e4, 128, 1).numpy()
    assert np.array_equal(oracle.rope_rotate_half(x, tab[0, :64], tab[0, 64:]), x)


def test_rope_matches_rotate_half_and_complex_forms():
    rng = np.random.default_rng(5)
    D = 128
    tab = rope_cos_sin_table(1e6, D, 4096).numpy()
    pos = rng.integers(0, 4096, size=400)
    x = _rand_bits(rng, (400, D))
    c, s = tab[pos, : D // 2], tab[pos, D // 2:]
    got = oracle.bf16_to_f64(oracle.rope_rotate_half(x, c, s))
    xf = oracle.bf16_to_f64(x)
    ref_rh = _rotate_half_torch(torch.from_numpy(xf), torch.from_numpy(c.astype(np.float64)),
                                torch.from_numpy(s.astype(np.float64))).numpy()
    z = (xf[:, : D // 2] + 1j * xf[:, D // 2:]) * (c.astype(np.float64) + 1j * s.astype(np.float64))
    ref_cx = np.concatenate([z.real, z.imag], axis=1)
    assert np.allclose(ref_rh, ref_cx, rtol=0, atol=1e-12)
    # only fp32 products/sum and the final bf16 rounding separate the forms
    tol = oracle.bf16_ulp(ref_cx) * 0.5 + 4e-7 * (np.abs(xf[:, : D // 2]).repeat(2, 1).reshape(ref_cx.shape) + 1)
    assert (np.abs(got - ref_cx) <= tol + 1e-30).all()
    # most elements are the correctly rounded bf16 of the exact rotation
    frac = np.mean(oracle.f64_to_bf16_rne(ref_cx) == oracle.rope_rotate_half(x, c, s))
    assert frac > 0.99


def test_rope_relative_position_property():
    # (R_m q).(R_n k) = q.(R_{n-m} k): the rotation depends on positions only
    # through their difference.  Checked on the exact (fp64) rotation using the
    # same table entries; catches a wrong pairing of angles to elements.
    rng = np.random.default_rng(6)
    D = 64
    tab = rope_cos_sin_table(1e4, D, 512).numpy().astype(np.float64)
    q = oracle.bf16_to_f64(_rand_bits(rng, (D,)))
    k = oracle.bf16_to_f64(_rand_bits(rng, (D,)))

    def rot(x, p):
        c, s = tab[p, : D // 2], tab[p, D // 2:]
        a, b = x[: D // 2], x[D // 2:]
        return np.concatenate([a * c - b * s, b * c + a * s])

    def rot_oracle(x, p):
        xb = oracle.f64_to_bf16_rne(x)
        return oracle.bf16_to_f64(oracle.rope_rotate_half(xb, tab[p, : D // 2].astype(np.float32),
                                                         tab[p, D // 2:].astype(np.float32)))

    for m, n in [(3, 10), (100, 101), (7, 300), (0, 511)]:
        lhs = rot(q, m) @ rot(k, n)
        rhs = q @ rot(k, n - m)
        assert abs(lhs - rhs) < 1e-5 * (1 + abs(rhs))
        # the oracle's bf16 rotation agrees up to bf16 rounding of each element
        assert abs(rot_oracle(q, m) @ rot_oracle(k, n) - lhs) < 0.05 * np.sqrt(D)
        assert np.allclose(np.linalg.norm(rot_oracle(q, m)), np.linalg.norm(q), rtol=1e-2)


# ---------------------------------------------------------- cache store ----

def test_cache_store_scatter_brute_force():
    rng = np.random.default_rng(7)
    T, Hq, Hkv, D, NB = 9, 4, 2, 64, 12
    q = _rand_bits(rng, (T, Hq, D))
    k = _rand_bits(rng, (T, Hkv, D))
    v = _rand_bits(rng, (T, Hkv, D))
    kc = _rand_bits(rng, (NB, Hkv, 16, D))
    vc = _rand_bits(rng, (NB, Hkv, 16, D))
    slots = rng.choice(NB * 16, size=T, replace=False).astype(np.int32)
    slots[[2, 5]] = -1  # padding tokens
    pos = rng.integers(0, 300, size=T).astype(np.int32)
    tab = rope_cos_sin_table(1e4, D, 300).numpy()
    q2, kc2, vc2 = oracle.cache_store(q, k, v, kc, vc, slots, pos, tab)
    touched = np.zeros((NB, 16), bool)
    for i in range(T):
        if slots[i] < 0:
            assert np.array_equal(q2[i], q[i])
            continue
        blk, row = slots[i] // 16, slots[i] % 16
        touched[blk, row] = True
        c, s = tab[pos[i], : D // 2], tab[pos[i], D // 2:]
        for g in range(Hkv):
            assert np.array_equal(vc2[blk, g, row], v[i, g])
            # row 0 of the pool is never the target: compare to an explicit rotation
            a = oracle.bf16_to_f64(k[i, g, : D // 2])
            b = oracle.bf16_to_f64(k[i, g, D // 2:])
            exact = np.concatenate([a * c - b * s, b * c + a * s])
            assert np.all(np.abs(oracle.bf16_to_f64(kc2[blk, g, row]) - exact)
                          <= oracle.bf16_ulp(exact) * 0.5 + 1e-6 * (np.abs(exact) + 1))
    mask = ~touched[:, None, :, None].repeat(Hkv, 1).repeat(D, 3)
    assert np.array_equal(kc2[mask], kc[mask]) and np.array_equal(vc2[mask], vc[mask])
    # inputs are not modified
    assert kc2 is not kc
    # no query passed: only the pool changes
    qn, kc3, _ = oracle.cache_store(None, k, v, kc, vc, slots, pos, tab)
    assert qn is None and np.array_equal(kc3, kc2)


# ------------------------------------------------------------ attention ----

def _scatter_contiguous(Ks, Vs, tables, NB, Hkv, D, fill_bits=0):
    """Write contiguous per-sequence K/V into a pool through the tables (test side)."""
    kc = np.full((NB, Hkv, 16, D), fill_bits, np.uint16)
    vc = np.full((NB, Hkv, 16, D), fill_bits, np.uint16)
    for b, (K, V) in enumerate(zip(Ks, Vs)):
        for t in range(K.shape[0]):
            kc[tables[b][t // 16], :, t % 16, :] = K[t]
            vc[tables[b][t // 16], :, t % 16, :] = V[t]
    return kc, vc


def _sdpa64(q64, K64, V64, G, mask=None):
    """torch SDPA in fp64 over contiguous K/V, GQA by repeat_interleave.

    q64 [C, Hq, D], K64/V64 [L, Hkv, D]; returns [C, Hq, D]."""
    qt = torch.from_numpy(q64).permute(1, 0, 2)[None]
    kt = torch.from_numpy(K64).repeat_interleave(G, dim=1).permute(1, 0, 2)[None]
    vt = torch.from_numpy(V64).repeat_interleave(G, dim=1).permute(1, 0, 2)[None]
    m = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m)
    return o[0].permute(1, 0, 2).numpy()


def _random_paged(rng, lens, Hq, Hkv, D, NB):
    Ks = [_rand_bits(rng, (L, Hkv, D)) for L in lens]
    Vs = [_rand_bits(rng, (L, Hkv, D)) for L in lens]
    perm = rng.permutation(NB)
    tables = np.full((len(lens), max(1, max(-(-L // 16) for L in lens))), -1, np.int32)
    cur = 0
    for b, L in enumerate(lens):
        n = -(-L // 16)
        tables[b, :n] = perm[cur:cur + n]
        cur += n
    kc, vc = _scatter_contiguous(Ks, Vs, tables, NB, Hkv, D)
    return Ks, Vs, tables, kc, vc


@pytest.mark.parametrize("Hq,Hkv,D", [(4, 4, 64), (6, 1, 64), (12, 2, 128)])
def test_decode_equals_contiguous_sdpa(Hq, Hkv, D):
    rng = np.random.default_rng(8 + Hq)
    lens = [1, 15, 16, 17, 40, 129]
    Ks, Vs, tables, kc, vc = _random_paged(rng, lens, Hq, Hkv, D, 40)
    q = _rand_bits(rng, (len(lens), Hq, D))
    scale = 1 / math.sqrt(D)
    got = oracle.decode(q, kc, vc, tables, np.array(lens), scale)
    for b, L in enumerate(lens):
        ref = _sdpa64(oracle.bf16_to_f64(q[b])[None] * 1.0, oracle.bf16_to_f64(Ks[b]),
                      oracle.bf16_to_f64(Vs[b]), Hq // Hkv)
        # SDPA's default scale is 1/sqrt(D), the scale used here
        assert np.abs(got[b] - ref[0]).max() < 1e-12


def test_gqa_head_mapping_is_consecutive():
    # query head h reads KV head h // G: heads 0..G-1 share KV head 0
    rng = np.random.default_rng(9)
    Hq, Hkv, D, L = 6, 2, 64, 20
    Ks, Vs, tables, kc, vc = _random_paged(rng, [L], Hq, Hkv, D, 4)
    qrow = _rand_bits(rng, (1, 1, D))
    q = np.repeat(qrow, Hq, axis=1)  # identical query in every head
    out = oracle.decode(q, kc, vc, tables, np.array([L]), 0.125)[0]
    assert np.array_equal(out[0], out[2]) and np.array_equal(out[3], out[5])
    assert not np.allclose(out[0], out[3])
    # MHA on the KV heads repeated G times gives the same result
    Kr = np.repeat(Ks[0], 3, axis=1)
    Vr = np.repeat(Vs[0], 3, axis=1)
    kc2, vc2 = _scatter_contiguous([Kr], [Vr], tables, 4, Hq, D)
    out2 = oracle.decode(q, kc2, vc2, tables, np.array([L]), 0.125)[0]
    assert np.array_equal(out, out2)


def test_decode_invariant_under_block_permutation():
    rng = np.random.default_rng(10)
    Hq, Hkv, D, NB = 4, 2, 64, 30
    lens = [33, 70, 5]
    Ks, Vs, tables, kc, vc = _random_paged(rng, lens, Hq, Hkv, D, NB)
    q = _rand_bits(rng, (3, Hq, D))
    out1 = oracle.decode(q, kc, vc, tables, np.array(lens), 0.125)
    sigma = rng.permutation(NB)          # physical block b moves to sigma[b]
    kc2 = np.empty_like(kc)
    vc2 = np.empty_like(vc)
    kc2[sigma] = kc
    vc2[sigma] = vc
    tables2 = np.where(tables >= 0, sigma[np.maximum(tables, 0)], -1).astype(np.int32)
    out2 = oracle.decode(q, kc2, vc2, tables2, np.array(lens), 0.125)
    assert np.array_equal(out1, out2)


def test_decode_aliased_prefix_equals_private_copies():
    rng = np.random.default_rng(11)
    Hq, Hkv, D = 4, 1, 64
    pre = 48  # three whole blocks
    Kp, Vp = _rand_bits(rng, (pre, Hkv, D)), _rand_bits(rng, (pre, Hkv, D))
    suf = [5, 20]
    Ks = [np.concatenate([Kp, _rand_bits(rng, (s, Hkv, D))]) for s in suf]
    Vs = [np.concatenate([Vp, _rand_bits(rng, (s, Hkv, D))]) for s in suf]
    lens = [pre + s for s in suf]
    q = _rand_bits(rng, (2, Hq, D))
    # private: every block its own
    priv = np.array([[0, 1, 2, 3, -1], [4, 5, 6, 7, 8]], np.int32)
    kc, vc = _scatter_contiguous(Ks, Vs, priv, 16, Hkv, D)
    out_priv = oracle.decode(q, kc, vc, priv, np.array(lens), 0.125)
    # aliased: sequence 1 reuses sequence 0's three prefix blocks (ref_count 2)
    alias = np.array([[0, 1, 2, 3, -1], [0, 1, 2, 7, 8]], np.int32)
    kc2, vc2 = _scatter_contiguous(Ks, Vs, alias, 16, Hkv, D)
    out_alias = oracle.decode(q, kc2, vc2, alias, np.array(lens), 0.125)
    assert np.array_equal(out_priv, out_alias)


def test_decode_hand_computed_tiny_contexts():
    fx = json.load(open(os.path.join(GOLDEN, "tiny_contexts.json")))
    D, scale = fx["head_dim"], fx["scale"]
    vrows = np.array(fx["v_rows"], dtype=np.float32)
    for case in fx["cases"]:
        krows = np.array(case["k_rows"], dtype=np.float32)
        L = len(krows)
        q = np.array(case["q"], dtype=np.float32)
        bits = lambda a: as_bits(torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16))
        assert np.array_equal(oracle.bf16_to_f32(bits(vrows)), vrows)  # exact in bf16
        kc = np.zeros((4, 1, 16, D), np.uint16)
        vc = np.zeros((4, 1, 16, D), np.uint16)
        table = np.array([[2, -1]], np.int32)
        kc[2, 0, :L] = bits(krows)
        vc[2, 0, :L] = bits(vrows[:L])
        out = oracle.decode(bits(q[None, None]), kc, vc, table, np.array([L]), scale)[0, 0]
        if case["expect"] == "v0":
            assert np.array_equal(out, vrows[0].astype(np.float64))
            continue
        s = case["scores"]
        assert np.allclose(scale * (krows.astype(np.float64) @ q.astype(np.float64)), s, atol=0)
        w = [math.exp(x) for x in s]
        exp = sum(wi * vrows[t].astype(np.float64) for t, wi in enumerate(w)) / sum(w)
        assert np.abs(out - exp).max() < 1e-14
        if case["name"].startswith("zero query"):
            assert np.allclose(out, vrows[:L].astype(np.float64).mean(0), atol=1e-15)


def test_decode_empty_sequence_is_zero():
    rng = np.random.default_rng(12)
    kc = _rand_bits(rng, (2, 1, 16, 64))
    vc = _rand_bits(rng, (2, 1, 16, 64))
    q = _rand_bits(rng, (2, 2, 64))
    out = oracle.decode(q, kc, vc, np.array([[0], [1]], np.int32), np.array([0, 3]), 0.125)
    assert (out[0] == 0).all() and np.isfinite(out).all() and (out[1] != 0).any()


@pytest.mark.parametrize("P", [16, 32, 48, 512, 4096])
def test_split_combine_equals_single_pass(P):
    rng = np.random.default_rng(13)
    lens = [1, 16, 100, 513, 1000]
    Hq, Hkv, D = 6, 2, 64
    Ks, Vs, tables, kc, vc = _random_paged(rng, lens, Hq, Hkv, D, 120)
    q = _rand_bits(rng, (len(lens), Hq, D), scale=3.0)  # peaked softmax
    one = oracle.decode(q, kc, vc, tables, np.array(lens), 0.125)
    split = oracle.decode_split(q, kc, vc, tables, np.array(lens), 0.125, P)
    assert np.abs(one - split).max() < 1e-12


def test_combine_of_one_partition_is_normalisation():
    rng = np.random.default_rng(14)
    m = rng.standard_normal((1, 3))
    l = rng.random((1, 3)) + 0.5
    o = rng.standard_normal((1, 3, 8))
    assert np.allclose(oracle.combine_partials(m, l, o), o[0] / l[0][:, None], atol=1e-15)


def test_prefill_equals_masked_sdpa():
    rng = np.random.default_rng(15)
    Hq, Hkv, D = 6, 2, 64
    prefix, chunk = [0, 16, 37, 50], [5, 16, 20, 1]
    lens = [p + c for p, c in zip(prefix, chunk)]
    Ks, Vs, tables, kc, vc = _random_paged(rng, lens, Hq, Hkv, D, 40)
    T = sum(chunk)
    q = _rand_bits(rng, (T, Hq, D))
    qsl = np.concatenate([[0], np.cumsum(chunk)])
    got = oracle.prefill(q, kc, vc, tables, np.array(lens), qsl, 0.125)
    for b in range(4):
        C, L = chunk[b], lens[b]
        r = np.arange(C)[:, None]
        t = np.arange(L)[None, :]
        allowed = t <= (prefix[b] + r)  # row r sits at absolute position prefix + r
        mask = np.where(allowed, 0.0, -np.inf)
        ref = _sdpa64(oracle.bf16_to_f64(q[qsl[b]:qsl[b + 1]]), oracle.bf16_to_f64(Ks[b]),
                      oracle.bf16_to_f64(Vs[b]), Hq // Hkv, mask[None])
        assert np.abs(got[qsl[b]:qsl[b + 1]] - ref).max() < 1e-12


def test_prefill_last_row_equals_decode():
    rng = np.random.default_rng(16)
    Hq, Hkv, D = 4, 2, 64
    lens = [40, 17]
    chunk = [8, 17]
    Ks, Vs, tables, kc, vc = _random_paged(rng, lens, Hq, Hkv, D, 8)
    q = _rand_bits(rng, (sum(chunk), Hq, D))
    qsl = np.array([0, 8, 25])
    pf = oracle.prefill(q, kc, vc, tables, np.array(lens), qsl, 0.125)
    for b in range(2):
        for i in range(chunk[b]):
            L_i = lens[b] - chunk[b] + i + 1
            dec = oracle.decode(q[qsl[b] + i][None], kc, vc, tables[b][None], np.array([L_i]), 0.125)
            assert np.array_equal(pf[qsl[b] + i], dec[0])


def test_chunked_prefill_ranges_match_one_pass():
    fx = json.load(open(os.path.join(GOLDEN, "paging_examples.json")))["chunked_prefill"]
    n, c = fx["prompt_len"], fx["chunk_size"]
    starts = list(range(0, n, c))
    assert len(starts) == fx["chunks"]
    rng = np.random.default_rng(17)
    Hq, Hkv, D = 2, 1, 64
    Ks, Vs, tables, kc, vc = _random_paged(rng, [n], Hq, Hkv, D, n // 16)
    q = _rand_bits(rng, (n, Hq, D))
    full = oracle.prefill(q, kc, vc, tables, np.array([n]), np.array([0, n]), 0.125)
    for s in starts:
        e = min(s + c, n)
        part = oracle.prefill(q[s:e], kc, vc, tables, np.array([e]), np.array([0, e - s]), 0.125)
        assert np.array_equal(part, full[s:e])


def test_shared_system_prompt_example():
    fx = json.load(open(os.path.join(GOLDEN, "paging_examples.json")))
    ex = fx["shared_system_prompt"]
    bs = fx["block_size"]["value"]
    assert ex["prefix_tokens"] // bs == ex["shared_blocks"] and ex["prefix_tokens"] % bs == 0
    rng = np.random.default_rng(18)
    Hq, Hkv, D = 2, 1, 64
    pre = ex["prefix_tokens"]
    Kp, Vp = _rand_bits(rng, (pre, Hkv, D)), _rand_bits(rng, (pre, Hkv, D))
    Ks = [np.concatenate([Kp, _rand_bits(rng, (7, Hkv, D))]) for _ in range(2)]
    Vs = [np.concatenate([Vp, _rand_bits(rng, (7, Hkv, D))]) for _ in range(2)]
    nb = ex["shared_blocks"]
    shared = list(range(nb))
    alias = np.array([shared + [nb], shared + [nb + 1]], np.int32)
    priv = np.array([shared + [nb], list(range(nb + 1, 2 * nb + 1)) + [2 * nb + 1]], np.int32)
    counts = np.bincount(alias[:, :nb].ravel())
    assert (counts == ex["ref_count"]).all()
    q = _rand_bits(rng, (2, Hq, D))
    lens = np.array([pre + 7, pre + 7])
    kc, vc = _scatter_contiguous(Ks, Vs, alias, 2 * nb + 2, Hkv, D)
    kc2, vc2 = _scatter_contiguous(Ks, Vs, priv, 2 * nb + 2, Hkv, D)
    assert np.array_equal(oracle.decode(q, kc, vc, alias, lens, 0.125),
                          oracle.decode(q, kc2, vc2, priv, lens, 0.125))


def test_store_then_decode_equals_contiguous_attention():
    # the new token is rotated and scattered by the store, then attended by decode;
    # the result equals attention over [history ; rotated k] with the rotated q.
    from workloads import decode_batch
    wb = decode_batch([1, 15, 16, 33], 2, 1, 64, 32, 2401, theta=1e4)
    kc, vc = as_bits(wb.k_cache), as_bits(wb.v_cache)
    q2, kc2, vc2 = oracle.cache_store(as_bits(wb.q), as_bits(wb.k), as_bits(wb.v), kc, vc,
                                      wb.slot_mapping.numpy(), wb.positions.numpy(),
                                      wb.cos_sin.numpy())
    tables = wb.block_tables.numpy()
    lens = wb.context_lens.numpy()
    out = oracle.decode(q2, kc2, vc2, tables, lens, wb.scale)
    tab = wb.cos_sin.numpy()
    for b, L in enumerate(lens):
        hist_k = np.stack([kc[tables[b][t // 16], :, t % 16] for t in range(L - 1)]) if L > 1 \
            else np.zeros((0, 1, 64), np.uint16)
        hist_v = np.stack([vc[tables[b][t // 16], :, t % 16] for t in range(L - 1)]) if L > 1 \
            else np.zeros((0, 1, 64), np.uint16)
        c, s = tab[L - 1, :32], tab[L - 1, 32:]
        knew = oracle.rope_rotate_half(as_bits(wb.k)[b], c, s)
        qnew = oracle.rope_rotate_half(as_bits(wb.q)[b], c, s)
        K = oracle.bf16_to_f64(np.concatenate([hist_k, knew[None]]))
        V = oracle.bf16_to_f64(np.concatenate([hist_v, as_bits(wb.v)[b][None]]))
        ref = _sdpa64(oracle.bf16_to_f64(qnew)[None], K, V, 2)
        assert np.abs(out[b] - ref[0]).max() < 1e-12


def test_rope_rounds_each_fp32_operation():
    # Reading: two fp32 products and one fp32 add/sub, each rounded to nearest
    # even, no fused multiply-add.  Independent emulation: a product of two fp32
    # values is exact in binary64 and one cast to float32 rounds it correctly;
    # the sum of two fp32 values is exact in binary64 whenever their exponents
    # are close (checked), so one cast rounds it correctly too.  Inputs are
    # searched for cases where rounding once (fused) and rounding each step give
    # different bf16 results, and the oracle must follow the stepwise order there.
    rng = np.random.default_rng(19)
    D, N = 128, 4_000_000
    tab = rope_cos_sin_table(1e6, D, 8192).numpy()
    pos = rng.integers(0, 8192, size=N)
    j = rng.integers(0, D // 2, size=N)
    ab = oracle.bf16_to_f32(_rand_bits(rng, (N, 2)))
    a, b = ab[:, 0].astype(np.float64), ab[:, 1].astype(np.float64)
    c, s = tab[pos, j].astype(np.float64), tab[pos, D // 2 + j].astype(np.float64)
    to32 = lambda x: x.astype(np.float32).astype(np.float64)
    step_lo = to32(to32(a * c) - to32(b * s))
    step_hi = to32(to32(b * c) + to32(a * s))
    fused_lo = to32(a * c - b * s)
    fused_hi = to32(b * c + a * s)
    bf = lambda x: oracle.f64_to_bf16_rne(x)
    cand = np.nonzero((bf(step_lo) != bf(fused_lo)) | (bf(step_hi) != bf(fused_hi)))[0]
    assert len(cand) >= 10, "search found too few distinguishing inputs"
    # exactness of the binary64 sums for the selected cases
    for u, w in ((to32(a * c), to32(b * s)), (to32(b * c), to32(a * s))):
        eu = np.frexp(u[cand])[1]
        ew = np.frexp(w[cand])[1]
        assert (np.abs(eu - ew) < 29).all()
    x = np.zeros((len(cand), D), np.uint16)
    x[:, 0] = oracle.f64_to_bf16_rne(a[cand])
    x[:, D // 2] = oracle.f64_to_bf16_rne(b[cand])
    cc = np.zeros((len(cand), D // 2), np.float32)
    ss = np.zeros((len(cand), D // 2), np.float32)
    cc[:, 0] = c[cand]
    ss[:, 0] = s[cand]
    got = oracle.rope_rotate_half(x, cc, ss)
    assert np.array_equal(got[:, 0], bf(step_lo[cand]))
    assert np.array_equal(got[:, D // 2], bf(step_hi[cand]))


# --------------------------------------------------------------------------
# Block copies (copy-on-write, swap)
# --------------------------------------------------------------------------

def _pool(nb, seed, hkv=2, d=8):
    rng = np.random.default_rng(seed)
    return rng.integers(0, 2 ** 16, size=(nb, hkv, 16, d), dtype=np.uint16)


def test_copy_blocks_equals_index_copy():
    src, dst = _pool(10, 1), _pool(12, 2)
    s_ids = np.array([3, 0, 9, 3], dtype=np.int32)
    d_ids = np.array([11, 2, 5, 7], dtype=np.int32)
    got = oracle.copy_blocks(dst, src, s_ids, d_ids)
    want = torch.from_numpy(dst.astype(np.int32)).index_copy(
        0, torch.from_numpy(d_ids.astype(np.int64)),
        torch.from_numpy(src[s_ids].astype(np.int32))).numpy().astype(np.uint16)
    assert np.array_equal(got, want)
    untouched = np.setdiff1d(np.arange(12), d_ids)
    assert np.array_equal(got[untouched], dst[untouched])


def test_copy_within_one_pool_reads_the_old_tiles():
    pool = _pool(6, 3)
    got = oracle.copy_blocks(pool, pool, [1, 2], [4, 5])
    assert np.array_equal(got[4], pool[1]) and np.array_equal(got[5], pool[2])
    assert np.array_equal(got[:4], pool[:4])


def test_swap_out_then_in_restores_the_sequence():
    dev = _pool(16, 4)
    seq_blocks = np.array([7, 2, 11], dtype=np.int32)
    host = np.zeros((4, 2, 16, 8), dtype=np.uint16)
    host = oracle.copy_blocks(host, dev, seq_blocks, [0, 1, 2])        # swap out
    new_blocks = np.array([5, 13, 0], dtype=np.int32)
    back = oracle.copy_blocks(np.zeros_like(dev), host, [0, 1, 2], new_blocks)  # swap in elsewhere
    assert np.array_equal(back[new_blocks], dev[seq_blocks])


def test_copy_on_write_then_decode_is_unchanged():
    # a shared prefix block copied to a fresh block: the sequence that now points at the
    # copy attends to exactly the same keys and values (aliasing vs private copy)
    b = W.decode_batch([40, 40], 4, 2, 64, 16, 77, shared_prefix=([0, 1], 2))
    qb, kc, vc = as_bits(b.q), as_bits(b.k_cache), as_bits(b.v_cache)
    bt = b.block_tables.numpy().copy()
    lens = b.context_lens.numpy()
    ref = oracle.decode(qb, kc, vc, bt, lens, b.scale)
    assert bt[0, 0] == bt[1, 0] and bt[0, 1] == bt[1, 1]  # shared blocks
    free = np.setdiff1d(np.arange(16), bt[bt >= 0])[:2]
    kc2 = oracle.copy_blocks(kc, kc, bt[1, :2], free)
    vc2 = oracle.copy_blocks(vc, vc, bt[1, :2], free)
    bt[1, :2] = free
    got = oracle.decode(qb, kc2, vc2, bt, lens, b.scale)
    assert np.array_equal(got, ref)


# --------------------------------------------------------------------------
# Residual add + RMSNorm, SwiGLU
# --------------------------------------------------------------------------

def _bf16_bits(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_rmsnorm_matches_torch_rms_norm():
    rng = np.random.default_rng(5)
    x = _bf16_bits(rng.standard_normal((6, 96)))
    w = _bf16_bits(rng.standard_normal(96))
    got, r = oracle.rmsnorm_residual(x, w, None, eps=1e-6)
    xt = torch.from_numpy(oracle.bf16_to_f64(x))
    want = torch.nn.functional.rms_norm(xt, (96,), torch.from_numpy(oracle.bf16_to_f64(w)), eps=1e-6)
    assert r is None and np.allclose(got, want.numpy(), rtol=1e-12, atol=1e-12)


def test_rmsnorm_closed_forms():
    # constant row c: rms = |c|, out = w * sign(c); unit weight: the output's rms is 1 (eps 0)
    c = _bf16_bits(np.full((1, 64), -2.5))
    w = _bf16_bits(np.linspace(-1, 1, 64))
    out, _ = oracle.rmsnorm_residual(c, w, None, eps=0.0)
    assert np.allclose(out, -oracle.bf16_to_f64(w))
    x = _bf16_bits(np.random.default_rng(6).standard_normal((3, 128)))
    ones = _bf16_bits(np.ones(128))
    out, _ = oracle.rmsnorm_residual(x, ones, None, eps=0.0)
    assert np.allclose(np.sqrt((out ** 2).mean(-1)), 1.0, atol=1e-12)
    # scale invariance: 4x has the same normalised output (4 is exact in bf16)
    x4 = _bf16_bits(oracle.bf16_to_f64(x) * 4)
    assert np.allclose(oracle.rmsnorm_residual(x4, ones, None, 0.0)[0], out, atol=1e-12)


def test_residual_add_is_torch_bf16_addition():
    rng = np.random.default_rng(7)
    x = _bf16_bits(rng.standard_normal((5, 64)) * 3)
    r = _bf16_bits(rng.standard_normal((5, 64)) * 1e-3)
    _, nr = oracle.rmsnorm_residual(x, _bf16_bits(np.ones(64)), r)
    tx = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16)
    tr = torch.from_numpy(r.view(np.int16)).view(torch.bfloat16)
    assert np.array_equal(nr, (tx + tr).view(torch.int16).numpy().view(np.uint16))


def test_swiglu_matches_torch_silu():
    rng = np.random.default_rng(8)
    gu = _bf16_bits(rng.standard_normal((4, 2 * 40)) * 4)
    got = oracle.swiglu(gu)
    t = torch.from_numpy(oracle.bf16_to_f64(gu))
    want = torch.nn.functional.silu(t[:, :40]) * t[:, 40:]
    assert np.allclose(got, want.numpy(), rtol=1e-12, atol=1e-12)
    z = oracle.swiglu(_bf16_bits(np.array([[0.0, 60.0, -60.0, 1.0, 2.0, 2.0]])))
    assert z[0, 0] == 0.0 and abs(z[0, 1] - 2 * 60.0) < 1e-9 and abs(z[0, 2]) < 1e-20
