"""Pins for the CPU oracle: each test ties it to something other than itself.

* the explainer's 2-D absorption example with its printed numbers (golden fixture);
* the explainer's and the wiki's cache arithmetic (golden fixture);
* brute force with explicit Python loops on tiny shapes, non-square so a transposed operand fails;
* closed forms and special cases (one token, zero query, identical rows, the needle);
* invariants (absorbed == decompressed, split-and-merge == single pass, softmax sums to one).
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import mla_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------------------------------
# The explainer's worked example (Step 6)
# --------------------------------------------------------------------------------------------------

def test_toy_absorption_example():
    g = _load("toy_absorption.json")
    w_q = np.array(g["W_Q"], float)
    w_uk = np.array(g["W_UK"], float)
    h = np.array(g["h"], float)
    c = np.array(g["c"], float)
    q = w_q @ h
    assert q.tolist() == g["q"]
    # slow path: rebuild the key from the note, then score
    row = c[None, :]                        # one cached token, no RoPE part
    k_nope, _ = O.decompress_head(row, w_uk, np.eye(2), d_c=2)
    assert k_nope[0].tolist() == g["k"]
    assert float(q @ k_nope[0]) == g["score"]
    # absorbed path: move the query into latent space, score the note directly
    q_lat = O.absorb_query(q, w_uk)
    assert float(q_lat @ c) == g["score"]
    # the merged matrix M = W_Q^T W_UK, built column by column with the oracle's absorption
    m = np.stack([O.absorb_query(w_q @ e, w_uk) for e in np.eye(2)])
    assert m.tolist() == g["M"]
    assert (m @ c).tolist() == g["Mc"]
    assert float(h @ (m @ c)) == g["score"]


def test_toy_example_through_decode_head():
    """With one token, softmax weight is 1 and lse equals the (scaled) score 13."""
    g = _load("toy_absorption.json")
    q = np.array(g["q"], float)
    w_uk = np.array(g["W_UK"], float)
    rows = np.array([g["c"]], float)          # d_c = 2, d_R = 0
    out, lse, p = O.decode_head(q, rows, w_uk, np.eye(2), scale=1.0)
    assert p.tolist() == [1.0]
    assert lse == g["score"]
    o_lat, lse2, _ = O.latent_attention(O.absorb_query(q, w_uk), rows, 2, 1.0)
    assert lse2 == g["score"]
    assert o_lat.tolist() == g["c"]


# --------------------------------------------------------------------------------------------------
# Cache arithmetic (explainer Steps 2, 4, 5, 8; wiki)
# --------------------------------------------------------------------------------------------------

def test_cache_arithmetic_closed_forms():
    g = _load("cache_arithmetic.json")
    s = g["shapes"]
    mha = O.mha_numbers_per_token(s["heads"], s["head_dim"], s["layers"])
    assert mha == 1_966_080
    assert O.mha_numbers_per_token(s["heads"], s["head_dim"], 1) == g["step5"]["numbers_of_keys_and_values_per_layer"]
    assert round(O.cache_bytes(mha, 16) / 1e6, 2) == g["step2"]["mb_per_token_bf16"]
    report = O.cache_bytes(mha, 16) * s["report_tokens"] / 1e9
    assert abs(report - g["step2"]["gb_per_report_approx"]) < 1.0
    assert report < g["step2"]["node_gb"]
    # Step 4: grouped and multi-query caching
    assert mha // O.gqa_numbers_per_token(g["step4"]["gqa_groups"], s["head_dim"], s["layers"]) == g["step4"]["gqa_cut"]
    assert mha // O.gqa_numbers_per_token(1, s["head_dim"], s["layers"]) == g["step4"]["mqa_cut"]
    # Step 8: the MLA row
    assert O.mla_numbers_per_token(s["d_c"], s["d_r"], 1) == g["step8"]["numbers_per_token_per_layer"]
    mla = O.mla_numbers_per_token(s["d_c"], s["d_r"], s["layers"])
    assert mla == 34_560
    assert round(mha / mla, 1) == g["step8"]["factor"]
    assert round(O.cache_bytes(mla, 16) * s["report_tokens"] / 1e9, 1) == g["step8"]["gb_per_report_approx"]
    assert O.gqa_equivalent_groups(s["d_c"], s["d_r"], s["head_dim"]) == g["step8"]["gqa_equivalent_groups"]
    assert round(100 * (1 - mla / mha), 1) == g["step8"]["same_precision_reduction_pct"]
    # the 93.3% audit: the dense 67B model (95 layers, GQA with Step 4's 8 groups) at 2 bytes per
    # number against V2 at about 6 bits per number
    d67 = O.gqa_numbers_per_token(g["step4"]["gqa_groups"], s["head_dim"], g["step8"]["dense67b_layers"])
    assert abs(d67 - g["step8"]["dense67b_numbers_approx"]) < 1000
    d67_kb = O.cache_bytes(d67, 16) / 1e3
    assert round(d67_kb) == g["step8"]["dense67b_kb_approx"]
    v2_kb = O.cache_bytes(mla, g["step8"]["v2_bits_per_number"]) / 1e3
    assert round(v2_kb) == g["step8"]["v2_kb_approx"]
    assert round(100 * v2_kb / d67_kb, 1) == g["step8"]["ratio_pct_approx"]
    assert round(100 * (1 - v2_kb / d67_kb), 1) == g["step8"]["headline_reduction_pct"]
    # wiki: (d_K + d_V) / d_KV x heads, with the MLA row as d_KV
    f = O.wiki_reduction_factor(s["head_dim"], s["head_dim"], s["d_c"] + s["d_r"], s["heads"])
    assert round(f, 1) == g["wiki"]["factor_approx"] == round(mha / mla, 1)


# --------------------------------------------------------------------------------------------------
# Brute force on tiny shapes
# --------------------------------------------------------------------------------------------------

def _tiny(seed, lens, H=2, d_c=8, d_r=4, d_nope=4, d_v=3, page=2):
    rng = np.random.default_rng(seed)
    blocks = [(n + page - 1) // page for n in lens]
    total = sum(blocks)
    perm = rng.permutation(total)
    mb = max(max(blocks), 1)
    bt = np.full((len(lens), mb), -1, np.int32)
    k = 0
    for b, nb in enumerate(blocks):
        bt[b, :nb] = perm[k:k + nb]
        k += nb
    cache = rng.normal(size=(total, page, d_c + d_r))
    q = rng.normal(size=(len(lens), H, d_nope + d_r))
    w_uk = rng.normal(size=(H, d_nope, d_c)) / math.sqrt(d_c)
    w_uv = rng.normal(size=(H, d_c, d_v)) / math.sqrt(d_c)
    return cache, bt, q, w_uk, w_uv


def _brute(cache, bt, q, w_uk, w_uv, lens, scale):
    """Explicit loops straight from the definitions: rebuild each head's key and value from the
    note, add the RoPE score, softmax, mix."""
    page = cache.shape[1]
    B, H, _ = q.shape
    d_nope, d_c = w_uk.shape[1], w_uk.shape[2]
    d_v = w_uv.shape[2]
    out = np.zeros((B, H, d_v))
    lse = np.zeros((B, H))
    for b in range(B):
        for h in range(H):
            scores = []
            values = []
            for t in range(lens[b]):
                row = cache[bt[b][t // page]][t % page]
                c = row[:d_c]
                k_r = row[d_c:]
                s = 0.0
                for i in range(d_nope):
                    k_i = 0.0
                    for j in range(d_c):
                        k_i += w_uk[h][i][j] * c[j]
                    s += q[b][h][i] * k_i
                for i in range(len(k_r)):
                    s += q[b][h][d_nope + i] * k_r[i]
                scores.append(scale * s)
                v = [sum(c[j] * w_uv[h][j][d] for j in range(d_c)) for d in range(d_v)]
                values.append(v)
            m = max(scores)
            z = sum(math.exp(x - m) for x in scores)
            for t in range(lens[b]):
                w = math.exp(scores[t] - m) / z
                for d in range(d_v):
                    out[b][h][d] += w * values[t][d]
            lse[b][h] = m + math.log(z)
    return out, lse


@pytest.mark.parametrize("lens", [[1], [2], [3, 5], [5, 1, 2]])
def test_decode_reference_vs_brute_force(lens):
    cache, bt, q, w_uk, w_uv = _tiny(7 + len(lens), lens)
    scale = 0.37
    out, lse = O.decode_reference(q, cache.astype(np.float64), bt, lens, w_uk, w_uv, scale)
    bo, bl = _brute(cache, bt, q, w_uk, w_uv, lens, scale)
    np.testing.assert_allclose(out, bo, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, bl, rtol=1e-12, atol=1e-13)


def test_latent_decode_vs_brute_force():
    lens = [3, 5]
    cache, bt, q, w_uk, w_uv = _tiny(3, lens)
    d_c = w_uk.shape[2]
    q_abs = O.absorb_batch(q, w_uk)
    o_lat, lse = O.latent_decode_batch(q_abs, cache, bt, lens, 0.5, d_c=d_c)
    page = cache.shape[1]
    # q_abs itself was pinned by its own brute-force test below; here it is only an input
    for b in range(len(lens)):
        for h in range(q.shape[1]):
            s = []
            for t in range(lens[b]):
                row = cache[bt[b][t // page]][t % page]
                s.append(0.5 * sum(q_abs[b][h][i] * row[i] for i in range(len(row))))
            m = max(s)
            w = [math.exp(x - m) for x in s]
            z = sum(w)
            ref = [sum(w[t] / z * cache[bt[b][t // page]][t % page][j] for t in range(lens[b]))
                   for j in range(d_c)]
            np.testing.assert_allclose(o_lat[b, h], ref, rtol=1e-12, atol=1e-14)
            assert abs(lse[b, h] - (m + math.log(z))) < 1e-12


# --------------------------------------------------------------------------------------------------
# Invariants and special cases at the real widths (d_c = 512, d_R = 64, d_nope = d_v = 128)
# --------------------------------------------------------------------------------------------------

def _real(seed, T, H=3):
    rng = np.random.default_rng(seed)
    rows = rng.normal(size=(T, 576))
    q = rng.normal(size=(H, 192))
    w_uk = rng.normal(size=(H, 128, 512)) / math.sqrt(512)
    w_uv = rng.normal(size=(H, 512, 128)) / math.sqrt(512)
    return rows, q, w_uk, w_uv


def test_absorbed_equals_decompressed():
    rows, q, w_uk, w_uv = _real(1, 300)
    scale = 1 / math.sqrt(192)
    for h in range(q.shape[0]):
        out, lse, p = O.decode_head(q[h], rows, w_uk[h], w_uv[h], scale)
        q_abs = O.absorb_query(q[h], w_uk[h])
        o_lat, lse2, p2 = O.latent_attention(q_abs, rows, 512, scale)
        out2 = O.up_project(o_lat, w_uv[h])
        np.testing.assert_allclose(out2, out, rtol=1e-11, atol=1e-13)
        assert abs(lse - lse2) < 1e-11
        np.testing.assert_allclose(p2, p, rtol=1e-11, atol=1e-15)
        assert abs(p.sum() - 1) < 1e-12


def test_channels_add_inside_softmax():
    """Zeroing q^R leaves the content-only score; zeroing q_nope leaves the RoPE-only score."""
    rows, q, w_uk, w_uv = _real(2, 50, H=1)
    s_full = O.decode_head(q[0], rows, w_uk[0], w_uv[0], 1.0)[1]
    q_c = q[0].copy(); q_c[128:] = 0
    q_r = q[0].copy(); q_r[:128] = 0
    k_nope = rows[:, :512] @ w_uk[0].T
    s_c = k_nope @ q[0][:128]
    s_r = rows[:, 512:] @ q[0][128:]
    assert abs(O.decode_head(q_c, rows, w_uk[0], w_uv[0], 1.0)[1] - np.log(np.exp(s_c).sum())) < 1e-10
    assert abs(O.decode_head(q_r, rows, w_uk[0], w_uv[0], 1.0)[1] - np.log(np.exp(s_r).sum())) < 1e-10
    assert abs(s_full - np.log(np.exp(s_c + s_r).sum())) < 1e-10


def test_single_token_gives_its_value():
    rows, q, w_uk, w_uv = _real(3, 1)
    out, lse, p = O.decode_head(q[0], rows, w_uk[0], w_uv[0], 0.1)
    assert p.tolist() == [1.0]
    np.testing.assert_array_equal(out, rows[0, :512] @ w_uv[0])


def test_zero_query_is_uniform_mean():
    rows, _, _, _ = _real(4, 37)
    o_lat, lse, p = O.latent_attention(np.zeros(576), rows, 512, 1.0)
    np.testing.assert_allclose(p, np.full(37, 1 / 37), rtol=1e-14)
    np.testing.assert_allclose(o_lat, rows[:, :512].mean(axis=0), rtol=1e-12, atol=1e-14)
    assert abs(lse - math.log(37)) < 1e-14


def test_identical_rows_give_that_row():
    rows, q, w_uk, _ = _real(5, 1)
    rep = np.repeat(rows, 9, axis=0)
    q_abs = O.absorb_query(q[0], w_uk[0])
    o_lat, _, _ = O.latent_attention(q_abs, rep, 512, 0.3)
    np.testing.assert_allclose(o_lat, rows[0, :512], rtol=1e-14, atol=1e-15)


def test_empty_sequence():
    o_lat, lse, p = O.latent_attention(np.ones(576), np.zeros((0, 576)), 512, 1.0)
    assert lse == -math.inf and not o_lat.any() and p.size == 0


@pytest.mark.parametrize("cuts", [[0, 200], [0, 1, 200], [0, 64, 65, 128, 200], [0, 7, 100, 199, 200]])
def test_split_and_merge_equals_single_pass(cuts):
    rows, q, w_uk, _ = _real(6, 200, H=1)
    q_abs = O.absorb_query(q[0], w_uk[0])
    o_ref, l_ref, _ = O.latent_attention(q_abs, rows, 512, 1 / math.sqrt(192))
    parts = [O.latent_attention(q_abs, rows[a:b], 512, 1 / math.sqrt(192)) for a, b in zip(cuts, cuts[1:])]
    o, l = O.merge_partials([p[0] for p in parts], [p[1] for p in parts])
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-14)
    assert abs(l - l_ref) < 1e-12
    # an empty part (lse = -inf) changes nothing
    o2, l2 = O.merge_partials([p[0] for p in parts] + [np.zeros(512)], [p[1] for p in parts] + [-math.inf])
    np.testing.assert_allclose(o2, o, rtol=0, atol=0)
    assert l2 == l


def test_needle_selects_one_row_exactly():
    """A RoPE-only query that matches one token's k^R and opposes every other makes the softmax a
    one-hot: o_lat equals that token's note exactly."""
    rng = np.random.default_rng(9)
    rows = rng.normal(size=(130, 576))
    rows[:, 512] = -1.0
    star = 77
    rows[star, 512] = 1.0
    q_abs = np.zeros(576)
    q_abs[512] = 1000.0
    o_lat, lse, p = O.latent_attention(q_abs, rows, 512, 1 / math.sqrt(192))
    np.testing.assert_array_equal(o_lat, rows[star, :512])
    assert p[star] == 1.0


# --------------------------------------------------------------------------------------------------
# Paged bookkeeping
# --------------------------------------------------------------------------------------------------

def test_gather_and_append_through_a_shuffled_table():
    page = 4
    lens = [5, 8, 1]
    rng = np.random.default_rng(11)
    blocks = [(n + 1 + page - 1) // page for n in lens]     # room for one append each
    perm = rng.permutation(sum(blocks))
    bt = np.full((3, max(blocks)), -1, np.int32)
    k = 0
    for b, nb in enumerate(blocks):
        bt[b, :nb] = perm[k:k + nb]
        k += nb
    # fill each logical token with a code that names it: (b, t) -> 1000 b + t
    cache = np.zeros((sum(blocks), page, 3), np.uint16)
    for b, n in enumerate(lens):
        for t in range(n):
            cache[bt[b][t // page], t % page] = [b, t, 1000 * b + t]
    for b, n in enumerate(lens):
        rows = O.gather_rows(cache, bt, b, n)
        assert [tuple(r) for r in rows] == [(b, t, 1000 * b + t) for t in range(n)]
    new = np.array([[9, 9, b] for b in range(3)], np.uint16)
    after = O.append_rows(cache, bt, lens, new)
    for b, n in enumerate(lens):
        rows = O.gather_rows(after, bt, b, n + 1)
        assert tuple(rows[-1]) == (9, 9, b)
        assert [tuple(r) for r in rows[:-1]] == [(b, t, 1000 * b + t) for t in range(n)]
    changed = np.argwhere((after != cache).any(axis=2))
    assert len(changed) == 3
    with pytest.raises(ValueError):
        O.gather_rows(cache, np.full((1, 1), -1, np.int32), 0, 1)


def test_bf16_widening_is_exact():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x8000, 0x7F7F, 0x0001], np.uint16)
    vals = O.bf16_to_f64(bits)
    assert vals[0] == 1.0 and vals[1] == -1.0 and vals[3] == 0.0
    assert vals[2] == 3.140625
    assert vals[5] == float(np.float32(3.3895313892515355e38))
    assert vals[6] == 2.0 ** -133


# --------------------------------------------------------------------------------------------------
# The producer side of the cache: eq. 9 (explainer Step 5) and the rotated key (Step 7)
# --------------------------------------------------------------------------------------------------

def test_rope_closed_forms():
    """Hand-computable rotations (d = 4, base 100, so the two pairs turn at 1 and 0.1 rad per
    position): a wrong sign, pairing or frequency exponent fails one of these."""
    c1, s1 = math.cos(1.0), math.sin(1.0)
    # pair 0 of e_0 at position 1 turns by 1 rad
    assert np.allclose(O.rope_rotate([1.0, 0.0, 0.0, 0.0], 1, 100.0), [c1, s1, 0, 0], atol=1e-15)
    # pair 0 of e_1: (0, 1) -> (-sin, cos)
    assert np.allclose(O.rope_rotate([0.0, 1.0, 0.0, 0.0], 1, 100.0), [-s1, c1, 0, 0], atol=1e-15)
    # pair 1 (dims 2, 3) turns at 100^(-2/4) = 0.1 rad per position: 1 rad at position 10
    assert np.allclose(O.rope_rotate([0.0, 0.0, 1.0, 0.0], 10, 100.0), [0, 0, c1, s1], atol=1e-15)
    assert np.allclose(O.rope_rotate([0.0, 0.0, 0.0, 1.0], 10, 100.0), [0, 0, -s1, c1], atol=1e-15)
    # position 0 is the identity, exactly
    x = np.random.default_rng(3).normal(size=64)
    assert np.array_equal(O.rope_rotate(x, 0, 10000.0), x)


def test_rope_scores_depend_only_on_distance():
    """The property the explainer states for RoPE (Step 7): a rotated query-key score depends on the
    positions only through their difference; rotations also keep lengths and compose."""
    rng = np.random.default_rng(5)
    q, k = rng.normal(size=64), rng.normal(size=64)
    base = 10000.0
    for m, n, shift in ((3, 17, 1000), (0, 131072, 7), (91204, 5, 40000)):
        a = O.rope_rotate(q, m, base) @ O.rope_rotate(k, n, base)
        b = O.rope_rotate(q, m + shift, base) @ O.rope_rotate(k, n + shift, base)
        c = q @ O.rope_rotate(k, n - m, base)
        assert abs(a - b) <= 1e-9 * (abs(a) + 1) and abs(a - c) <= 1e-9 * (abs(a) + 1)
    for pos in (1, 77, 131071):
        r = O.rope_rotate(q, pos, base)
        assert np.allclose(np.hypot(r[0::2], r[1::2]), np.hypot(q[0::2], q[1::2]), rtol=1e-12)
    assert np.allclose(O.rope_rotate(O.rope_rotate(q, 1234, base), 4321, base),
                       O.rope_rotate(q, 5555, base), atol=1e-9)


def test_latent_row_vs_brute_force():
    """eq. 9 and the rotated key with explicit loops on a tiny non-square shape (a transposed weight
    fails): d_model 6, d_c 4, d_R 2."""
    rng = np.random.default_rng(9)
    h = rng.normal(size=6)
    w_dkv = rng.normal(size=(6, 4))
    w_kr = rng.normal(size=(6, 2))
    pos, base = 3, 10000.0
    row = O.latent_row(h, w_dkv, w_kr, pos, base)
    c = [sum(h[i] * w_dkv[i, j] for i in range(6)) for j in range(4)]
    k = [sum(h[i] * w_kr[i, j] for i in range(6)) for j in range(2)]
    ang = pos * base ** 0.0                      # one pair: frequency base^0 = 1
    kr = [k[0] * math.cos(ang) - k[1] * math.sin(ang), k[0] * math.sin(ang) + k[1] * math.cos(ang)]
    assert np.allclose(row, c + kr, rtol=1e-13, atol=1e-13)
    rows = O.latent_rows_batch(np.stack([h, -h]), w_dkv, w_kr, [pos, 0], base)
    assert np.allclose(rows[0], row) and np.allclose(rows[1, :4], -np.array(c))
    assert np.allclose(rows[1, 4:], -np.array(k))      # position 0: no rotation


# --------------------------------------------------------------------------------------------------
# The ~6-bit cache: FP6 E2M3 codes with one power-of-two scale per row
# --------------------------------------------------------------------------------------------------

# The 32 non-negative E2M3 magnitudes as the format lists them (subnormals k/8, then three binades
# with steps 1/8, 1/4, 1/2), written out by hand rather than from the field formula.
_E2M3_MAGNITUDES = [0, 0.125, 0.25, 0.375, 0.5, 0.625, 0.75, 0.875,
                    1.0, 1.125, 1.25, 1.375, 1.5, 1.625, 1.75, 1.875,
                    2.0, 2.25, 2.5, 2.75, 3.0, 3.25, 3.5, 3.75,
                    4.0, 4.5, 5.0, 5.5, 6.0, 6.5, 7.0, 7.5]


def test_fp6_code_table():
    """Every code against the format's value list; the sign bit negates (code 32 is -0)."""
    assert O.FP6_VALUES[:32].tolist() == _E2M3_MAGNITUDES
    assert (O.FP6_VALUES[32:] == -O.FP6_VALUES[:32]).all()
    assert math.copysign(1.0, O.fp6_e2m3_value(32)) == -1.0
    assert O.fp6_e2m3_value(0b011111) == 7.5 and O.fp6_e2m3_value(0b001000) == 1.0
    assert O.fp6_e2m3_value(0b000001) == 0.125


def _grid_round(y):
    """Rounding by grid spacing, a formulation independent of the oracle's search: steps 1/8 below
    2, 1/4 below 4, 1/2 above, half to even on the grid index, magnitudes capped at 7.5."""
    a = min(abs(y), 7.5)
    step = 0.125 if a < 2 else 0.25 if a < 4 else 0.5
    k = a / step
    r = math.floor(k)
    if k - r > 0.5 or (k - r == 0.5 and r % 2 == 1):
        r += 1
    return math.copysign(min(r * step, 7.5), y)


def test_fp6_rounding_ties_and_saturation():
    cases = {0.0625: 0.0, 0.1875: 0.25, 0.9375: 1.0, 1.9375: 2.0, 2.125: 2.0, 3.875: 4.0,
             6.75: 7.0, 7.25: 7.0, 7.75: 7.5, 100.0: 7.5, 0.3: 0.25, 5.2: 5.0}
    for y, want in cases.items():
        for sgn in (1.0, -1.0):
            got = O.FP6_VALUES[O.fp6_e2m3_round(np.array([sgn * y]))[0]]
            assert got == sgn * want, (sgn * y, got)
    assert O.fp6_e2m3_round(np.array([-0.0]))[0] == 32


def test_fp6_rounding_against_the_grid():
    """Random values and every midpoint between neighbouring magnitudes, against _grid_round."""
    rng = np.random.default_rng(11)
    mids = [(a + b) / 2 for a, b in zip(_E2M3_MAGNITUDES, _E2M3_MAGNITUDES[1:])]
    ys = np.concatenate([rng.uniform(-8, 8, 4000), rng.normal(0, 2, 2000), mids, np.negative(mids)])
    got = O.FP6_VALUES[O.fp6_e2m3_round(ys)]
    want = np.array([_grid_round(float(y)) for y in ys])
    assert np.array_equal(got, want)


def test_fp6_packing_layout():
    """Code i at bits 6i .. 6i+5, least significant bit first, bytes little-endian."""
    assert O.pack_fp6([1, 0, 0, 0]).tolist() == [0x01, 0x00, 0x00]
    assert O.pack_fp6([0, 1, 0, 0]).tolist() == [0x40, 0x00, 0x00]
    assert O.pack_fp6([0, 0, 1, 0]).tolist() == [0x00, 0x10, 0x00]
    assert O.pack_fp6([0, 0, 0, 63]).tolist() == [0x00, 0x00, 0xFC]
    assert O.pack_fp6([63, 0, 0, 0]).tolist() == [0x3F, 0x00, 0x00]
    codes = np.random.default_rng(3).integers(0, 64, (5, 576)).astype(np.uint8)
    packed = O.pack_fp6(codes)
    assert packed.shape == (5, 432)
    assert np.array_equal(O.unpack_fp6(packed), codes)


def test_fp6_row_exponent():
    assert O.fp6_row_exponent(7.5) == 0
    assert O.fp6_row_exponent(7.5 * 2.0 ** -3) == -3
    assert O.fp6_row_exponent(np.nextafter(7.5, 8.0)) == 1
    assert O.fp6_row_exponent(3.0) == -1            # 3 <= 3.75 but > 1.875
    assert O.fp6_row_exponent(0.0) == -126
    assert O.fp6_row_exponent(1e-40) == -126


def test_fp6_quantization_error_bound():
    """A stored number is within half a grid step (at its binade, times the row scale) of the bf16
    input, and the row's largest magnitude lands in (3.75, 7.5] times the scale."""
    rng = np.random.default_rng(5)
    for _ in range(20):
        x = (rng.normal(0, 1, 576) * 2.0 ** rng.integers(-20, 20)).astype(np.float32)
        codes, e = O.quantize_row_fp6(x.astype(np.float64))
        deq = O.FP6_VALUES[codes] * 2.0 ** e
        y = np.abs(x) / 2.0 ** e
        step = np.where(y < 2, 0.125, np.where(y < 4, 0.25, 0.5)) * 2.0 ** e
        assert (np.abs(deq - x) <= step / 2).all()
        assert 3.75 < np.abs(x).max() / 2.0 ** e <= 7.5


def test_fp6_bytes_per_token_matches_the_pages():
    """432 bytes of codes plus a 4-byte scale per row; over DeepSeek-V2's 60 layers that is 26,160
    bytes, the "near 26 KB per token" of the audit (within 1 %)."""
    assert O.FP6_ROW_BYTES == 432
    per_token = O.mla_numbers_per_token(512, 64, 60) * 6 / 8 + 60 * 4
    assert per_token == 26160
    assert abs(per_token - 26000) / 26000 < 0.01
    assert O.FP6_PAGE_BYTES == 64 * 436


def test_fp6_decode_is_attention_on_the_stored_numbers():
    """The fp6 decode equals the plain latent decode run on the dequantized rows, and a cache whose
    numbers are already code values times a power of two is stored without loss."""
    rng = np.random.default_rng(8)
    pages = 3
    k = rng.integers(-3, 3, (pages, 64, 1)).astype(np.float64)
    exact = O.FP6_VALUES[rng.integers(0, 64, (pages, 64, 576))] * 2.0 ** k
    exact[:, :, 0] = 7.5 * 2.0 ** k[:, :, 0]      # every row's largest magnitude is 7.5 * 2^k
    bits = (exact.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(O.bf16_to_f64(bits), exact)
    pages6 = O.quantize_pages_fp6(bits)
    bt = np.array([[2, 0], [1, -1]], np.int32)
    lens = np.array([100, 37])
    q = rng.normal(0, 0.5, (2, 4, 576))
    o6, l6 = O.latent_decode_batch_fp6(q, pages6, bt, lens, 0.07)
    o, l = O.latent_decode_batch(q, bits, bt, lens, 0.07)
    assert np.array_equal(o6, o) and np.array_equal(l6, l)


def test_fp6_many_rows_match_one_row():
    """The batched page quantizer and exponent agree with the one-row definitions."""
    rng = np.random.default_rng(12)
    amax = np.concatenate([[0.0, 1e-45, 7.5, np.nextafter(7.5, 8), 3.75, np.nextafter(3.75, 0)],
                           np.exp2(rng.uniform(-140, 120, 3000)), 7.5 * np.exp2(rng.integers(-126, 120, 500))])
    assert np.array_equal(O.fp6_row_exponents(amax), [O.fp6_row_exponent(float(a)) for a in amax])
    x = (rng.normal(0, 1, (2, 64, 576)) * np.exp2(rng.integers(-30, 30, (2, 64, 1)))).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    pages6 = O.quantize_pages_fp6(bits)
    for p in range(2):
        for t in (0, 17, 63):
            codes, e = O.quantize_row_fp6(bits[p, t])
            assert np.array_equal(O.unpack_fp6(pages6[p, t * 432:(t + 1) * 432]), codes)
            assert pages6[p, 27648 + 4 * t:27648 + 4 * t + 4].view(np.float32)[0] == 2.0 ** e


# --------------------------------------------------------------------------------------------------
# Output projection to the hidden width (explainer Step 6)
# --------------------------------------------------------------------------------------------------

def test_hidden_out_vs_brute_force():
    """Explicit loops on a tiny non-square shape: B 2, H 3, d_v 2, d_model 5 (a transposed W^O or a
    wrong head order fails)."""
    rng = np.random.default_rng(21)
    out = rng.normal(size=(2, 3, 2))
    w_o = rng.normal(size=(6, 5))
    want = np.zeros((2, 5))
    for b in range(2):
        for n in range(5):
            for h in range(3):
                for v in range(2):
                    want[b, n] += out[b, h, v] * w_o[h * 2 + v, n]
    np.testing.assert_allclose(O.hidden_out(out, w_o), want, rtol=1e-13, atol=1e-13)


def test_hidden_out_folded_equals_two_step():
    """The fold the explainer states (Step 6): W^UV applied after the weighted sum and then W^O
    equals the folded per-head matrix W^UV[h] W^O[h] applied to the latent-form output."""
    rng = np.random.default_rng(22)
    B, H, d_c, d_v, d = 3, 4, 16, 8, 12
    o_lat = rng.normal(size=(B, H, d_c))
    w_uv = rng.normal(size=(H, d_c, d_v))
    w_o = rng.normal(size=(H * d_v, d))
    two_step = O.hidden_out(O.out_proj_batch(o_lat, w_uv), w_o)
    np.testing.assert_allclose(O.hidden_out_folded(o_lat, w_uv, w_o), two_step, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------------------------------
# Top-k selection over a cheap index (wiki "KV cache data movement minimization")
# --------------------------------------------------------------------------------------------------

def test_top_k_by_hand():
    """Hand-worked selections: largest scores win, ties go to the earlier position, the result is in
    position order, and short sequences keep every token."""
    assert O.top_k_positions([5, 1, 9, 3, 9, 0], 3).tolist() == [0, 2, 4]
    assert O.top_k_positions([2, 2, 2, 2], 2).tolist() == [0, 1]
    assert O.top_k_positions([-3, -1, -2], 1).tolist() == [1]
    assert O.top_k_positions([7, 7], 5).tolist() == [0, 1]
    assert O.top_k_positions([], 4).tolist() == []


def test_top_k_against_brute_force():
    """Brute force: a position is kept exactly when fewer than k positions beat it, where t beats u
    if its score is higher or equal with t < u."""
    rng = np.random.default_rng(31)
    for _ in range(50):
        n = int(rng.integers(1, 60))
        k = int(rng.integers(1, 20))
        sc = rng.integers(-4, 5, n)                      # many ties
        keep = [t for t in range(n)
                if sum(1 for u in range(n) if sc[u] > sc[t] or (sc[u] == sc[t] and u < t)) < k]
        assert O.top_k_positions(sc, k).tolist() == keep


def test_index_scores_through_the_table():
    """Scores gathered through a shuffled table equal the dot products written out by loops."""
    rng = np.random.default_rng(32)
    idx = rng.integers(-128, 128, (4, 64, 128)).astype(np.int8)
    bt = np.array([[3, 1, -1], [0, 2, -1]], np.int32)
    q = rng.integers(-128, 128, 128).astype(np.int8)
    got = O.index_scores(idx, bt, 0, 100, q)
    for t in (0, 63, 64, 99):
        page = bt[0, t // 64]
        assert got[t] == sum(int(q[j]) * int(idx[page, t % 64, j]) for j in range(128))


def test_sparse_decode_with_k_at_least_the_length_is_dense():
    """With k >= every length the top-k attention is the full attention, bit for bit."""
    rng = np.random.default_rng(33)
    cache = rng.integers(0, 1 << 16, (3, 64, 576)).astype(np.uint16) & 0x3FFF   # finite bf16 patterns
    idx = rng.integers(-128, 128, (3, 64, 128)).astype(np.int8)
    bt = np.array([[2, 0], [1, -1]], np.int32)
    lens = np.array([100, 40])
    q = rng.normal(0, 0.3, (2, 4, 576))
    qi = rng.integers(-128, 128, (2, 128)).astype(np.int8)
    o, l, chosen = O.sparse_latent_decode(q, cache, bt, lens, idx, qi, 128, 0.05)
    o2, l2 = O.latent_decode_batch(q, cache, bt, lens, 0.05)
    assert np.array_equal(o, o2) and np.array_equal(l, l2)
    assert chosen[0].tolist() == list(range(100))


# --------------------------------------------------------------------------------------------------
# The batched absorption and up-projection (explainer Step 6) against explicit loops
# --------------------------------------------------------------------------------------------------

def _tiny_proj(seed):
    """Batch 3, heads 2, d_nope 3, d_R 2, d_c 5, d_v 4: every axis a different length, so a swapped
    batch/head index, a transposed weight or a misplaced q^R strip changes the shape or the values."""
    rng = np.random.default_rng(seed)
    B, H, d_nope, d_r, d_c, d_v = 3, 2, 3, 2, 5, 4
    q = rng.normal(size=(B, H, d_nope + d_r))
    w_uk = rng.normal(size=(H, d_nope, d_c))
    o_lat = rng.normal(size=(B, H, d_c))
    w_uv = rng.normal(size=(H, d_c, d_v))
    return q, w_uk, o_lat, w_uv


def test_absorb_batch_vs_explicit_loops():
    """q_abs[b][h][j] = sum_i q[b][h][i] W_UK[h][i][j] for j < d_c, then q^R copied: the content
    query moved into latent space (explainer Step 6), the RoPE strip untouched (Step 7)."""
    q, w_uk, _, _ = _tiny_proj(11)
    B, H, _ = q.shape
    d_nope, d_c = w_uk.shape[1:]
    got = O.absorb_batch(q, w_uk)
    assert got.shape == (B, H, d_c + q.shape[2] - d_nope)
    for b in range(B):
        for h in range(H):
            for j in range(d_c):
                want = sum(q[b][h][i] * w_uk[h][i][j] for i in range(d_nope))
                assert abs(got[b, h, j] - want) < 1e-12, (b, h, j)
            for r in range(q.shape[2] - d_nope):
                assert got[b, h, d_c + r] == q[b][h][d_nope + r]
    # a selection computes the same entries and leaves the rest NaN
    part = O.absorb_batch(q, w_uk, batch=[2], heads=[1])
    assert np.array_equal(part[2, 1], got[2, 1])
    assert np.isnan(part[0]).all() and np.isnan(part[2, 0]).all()


def test_out_proj_batch_vs_explicit_loops():
    """out[b][h][k] = sum_j o_lat[b][h][j] W_UV[h][j][k] (explainer Step 6: W^UV after the sum)."""
    _, _, o_lat, w_uv = _tiny_proj(12)
    B, H, d_c = o_lat.shape
    d_v = w_uv.shape[2]
    got = O.out_proj_batch(o_lat, w_uv)
    assert got.shape == (B, H, d_v)
    for b in range(B):
        for h in range(H):
            for k in range(d_v):
                want = sum(o_lat[b][h][j] * w_uv[h][j][k] for j in range(d_c))
                assert abs(got[b, h, k] - want) < 1e-12, (b, h, k)
