"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every test here checks an oracle function against something other than the
oracle itself: numbers the pages print (tests/golden), hand-packed words, closed
forms, invariants, special cases that reduce to a library routine, and brute force
on tiny inputs. A plausible slip in the oracle (nibble order, group index, zero
point, sign of the rotation, pairing, window bound, head mapping, norm placement)
fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle as O
import synth
from synth import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def rng(seed=0):
    return np.random.default_rng(seed)


def f16_bits(vals):
    return np.asarray(vals, np.float16).view(np.uint16)


# ---- number formats ---------------------------------------------------------------

def test_f16_decode_matches_numpy_all_finite():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    fin = np.isfinite(ref)
    got = np.array([O.f16_to_f64(b) for b in bits[fin][::7]])
    np.testing.assert_array_equal(got, ref[fin][::7])


def test_bf16_decode_known_values():
    assert O.bf16_to_f64(0x3F80) == 1.0
    assert O.bf16_to_f64(0xC000) == -2.0
    assert O.bf16_to_f64(0x4049) == 3.140625
    assert O.bf16_to_f64(0x0000) == 0.0


# ---- packing (P1) -------------------------------------------------------------------

def test_hand_packed_words():
    g = golden("packing.json")
    for e in g["words"]:
        w = np.array([int(e["word"], 16)], np.uint32)
        assert list(O.unpack_codes(w, 8)[0]) == e["codes"]


def test_symmetric_form_stored_nibble_is_q_plus_8():
    # Pages' symmetric form: zero table absent => w = (nibble - 8) * scale.
    g = golden("packing.json")
    for e in g["words"]:
        w = np.array([int(e["word"], 16)], np.uint32)
        sc = f16_bits([1.0])
        deq = O.dequant(w, sc, None, 8, group=8)
        assert list(deq[0].astype(int)) == e["symmetric_q"]


def pack_rows(codes):
    """Pack an [N][K] array of 4-bit codes by the model card's rule (column j -> word
    j/8, nibble j%8 little-endian)."""
    N, K = codes.shape
    c = codes.reshape(N, K // 8, 8).astype(np.uint32)
    return np.bitwise_or.reduce(c << (4 * np.arange(8, dtype=np.uint32)), axis=2)


def test_pack_unpack_roundtrip_random_words():
    words = synth.codes(synth.key(5, 77), 4096).reshape(64, 64)
    codes = O.unpack_codes(words, 512)
    np.testing.assert_array_equal(pack_rows(codes), words)


# ---- dequant and GEMV (P2) -------------------------------------------------------

def _w4_problem(N, K, group=128, seed=1):
    G = -(-K // group)
    r = rng(seed)
    C = r.integers(0, 16, (N, K))
    Z = r.integers(0, 16, (N, G))
    S = r.uniform(0.002, 0.02, (N, G)).astype(np.float16)
    qw = pack_rows(C)
    zw = np.zeros((N, -(-G // 8)), np.uint32)
    for g in range(G):
        zw[:, g // 8] |= (Z[:, g].astype(np.uint32) << (4 * (g % 8)))
    return C, Z, S, qw, S.view(np.uint16), zw


@pytest.mark.parametrize("N,K", [(5, 256), (7, 1728), (3, 640)])
def test_dequant_exact_against_integer_matrices(N, K):
    C, Z, S, qw, sb, zw = _w4_problem(N, K)
    gidx = np.arange(K) // 128
    ref = (C - Z[:, gidx]).astype(np.float64) * S.astype(np.float64)[:, gidx]
    got = O.dequant(qw, sb, zw, K)
    np.testing.assert_array_equal(got.astype(np.float64), ref)  # exact (P2, C6)


def test_all_codes_equal_zero_point_gives_zero():
    N, K = 6, 512
    qw = np.full((N, K // 8), 0x55555555, np.uint32)        # every code 5
    zw = np.full((N, 1), 0x55555555, np.uint32)             # every zero 5
    sb = f16_bits(np.full((N, 4), 0.01))
    x = rng(2).standard_normal(K).astype(np.float32)
    y = O.w4_gemv(qw, sb, zw, K, x)
    assert np.all(y == 0.0)


@pytest.mark.parametrize("K,probes", [(1728, [(0, 0), (3, 7), (2, 8), (1, 127), (4, 128), (0, 1663),
                                               (5, 1664), (6, 1727)]),
                                      (5120, [(0, 5119), (1, 4096), (2, 9)])])
def test_one_hot_probe_isolates_nibble_group_and_row(K, probes):
    """Codes equal the zero point everywhere except one (row, column); with x = e_j the
    output is (c - z) * s at that row and exactly 0 elsewhere. Catches nibble order,
    group index (incl. the partial last group of K = 1728) and zero-table slips."""
    N, group = 7, 128
    G = -(-K // group)
    for (r, j) in probes:
        z = np.full((N, G), 3)
        z[r, j // group] = 11                     # a distinct zero in the probed group
        C = z[:, np.arange(K) // group].copy()
        C[r, j] = 14
        qw = pack_rows(C)
        zw = np.zeros((N, -(-G // 8)), np.uint32)
        for g in range(G):
            zw[:, g // 8] |= (z[:, g].astype(np.uint32) << (4 * (g % 8)))
        S = np.full((N, G), 0.25, np.float16)
        S[r, j // group] = 0.0078125              # 2^-7, distinct per probed group
        x = np.zeros(K, np.float32)
        x[j] = 3.0
        y = O.w4_gemv(qw, S.view(np.uint16), zw, K, x)
        expect = np.zeros(N)
        expect[r] = (14 - 11) * 0.0078125 * 3.0
        np.testing.assert_array_equal(y.astype(np.float64), expect)


@pytest.mark.parametrize("N,K", [(9, 256), (13, 1728)])
def test_gemv_brute_force_dense_matmul(N, K):
    C, Z, S, qw, sb, zw = _w4_problem(N, K, seed=3)
    gidx = np.arange(K) // 128
    Wd = (C - Z[:, gidx]).astype(np.float64) * S.astype(np.float64)[:, gidx]
    x = rng(4).standard_normal(K).astype(np.float32)
    y = O.w4_gemv(qw, sb, zw, K, x)
    ref = Wd @ x.astype(np.float64)
    np.testing.assert_allclose(y, ref, rtol=1e-6, atol=1e-6 * np.abs(ref).max())


def test_gemv_linear_in_x():
    N, K = 11, 640
    C, Z, S, qw, sb, zw = _w4_problem(N, K, seed=5)
    r = rng(6)
    x1 = r.standard_normal(K).astype(np.float32)
    x2 = r.standard_normal(K).astype(np.float32)
    y12 = O.w4_gemv(qw, sb, zw, K, (x1 + x2).astype(np.float32))
    y1, y2 = O.w4_gemv(qw, sb, zw, K, x1), O.w4_gemv(qw, sb, zw, K, x2)
    np.testing.assert_allclose(y12, y1 + y2, rtol=1e-5, atol=1e-5)


def test_bf16_gemv_one_hot_column_and_brute_force():
    r = rng(7)
    Wf = r.standard_normal((17, 96)).astype(np.float32)
    Wb = (Wf.view(np.uint32) >> 16).astype(np.uint16)          # truncation gives valid bf16 bits
    Wup = (Wb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    x = np.zeros(96, np.float32)
    x[40] = 1.0
    np.testing.assert_array_equal(O.bf16_gemv(Wb, x).astype(np.float64), Wup[:, 40])
    x = r.standard_normal(96).astype(np.float32)
    np.testing.assert_allclose(O.bf16_gemv(Wb, x), Wup @ x.astype(np.float64), rtol=1e-6, atol=1e-6)


# ---- RMSNorm (P9) --------------------------------------------------------------------

def test_rmsnorm_unit_rms_and_scale_invariance():
    x = rng(8).standard_normal(5120).astype(np.float32) * 3.7
    g = np.ones(5120, np.float32)
    y = O.rmsnorm(x, g).astype(np.float64)
    ms = np.mean(x.astype(np.float64) ** 2)
    assert abs(np.mean(y ** 2) - ms / (ms + 1e-6)) < 1e-6
    y2 = O.rmsnorm((x * 64.0).astype(np.float32), g)
    np.testing.assert_allclose(y2, y, rtol=2e-6, atol=1e-7)


def test_rmsnorm_constant_vector_closed_form_and_gain():
    x = np.full(10, 0.5, np.float32)
    g = np.arange(10, dtype=np.float32)
    y = O.rmsnorm(x, g, eps=1e-6)
    np.testing.assert_allclose(y, g * (0.5 / math.sqrt(0.25 + 1e-6)), rtol=1e-7)


def test_rmsnorm_residual_zero_branch_is_identity():
    r = rng(9).standard_normal(640).astype(np.float32)
    out = O.rmsnorm_residual(np.zeros(640, np.float32), np.ones(640, np.float32), r)
    np.testing.assert_array_equal(out, r)


# ---- RoPE / YaRN (P6, P7, P8) ------------------------------------------------------

def test_inv_freq_geometric_from_one():
    inv = O.rope_inv_freq(128, 500000.0)
    assert inv[0] == 1.0
    ratios = inv[1:] / inv[:-1]
    np.testing.assert_allclose(ratios, 500000.0 ** (-2.0 / 128), rtol=1e-13)
    np.testing.assert_allclose(inv[-1], 500000.0 ** (-126 / 128), rtol=1e-13)


def test_yarn_by_parts_criteria():
    """YaRN NTK-by-parts (Peng et al. 2023): pairs turning more than beta_fast times
    over the native context keep their frequency; pairs turning fewer than beta_slow
    times are divided by the factor exactly; in between the factor ramps linearly and
    monotonically."""
    D, theta, s, L = 128, 500000.0, 8.0, 8192
    base = O.rope_inv_freq(D, theta)
    yarn = O.rope_inv_freq(D, theta, s, L, 32.0, 1.0)
    r = L * base / (2 * math.pi)
    ratio = yarn / base
    assert np.all(ratio[r >= 32.0] == 1.0)
    assert np.all(np.abs(ratio[r <= 1.0] - 1.0 / s) < 1e-15)
    assert np.all(np.diff(ratio) <= 1e-15)
    mid = np.where((ratio < 1.0) & (ratio > 1.0 / s))[0]
    assert len(mid) > 5
    # linear in the pair index inside the ramp: constant first differences of the blend
    blend = (1.0 - ratio) / (1.0 - 1.0 / s)
    d1 = np.diff(blend[mid[0] - 1:mid[-1] + 2])
    np.testing.assert_allclose(d1, d1[0], rtol=1e-9)
    # rounded-outward correction range: the first ramped pair follows the last pair
    # whose frequency stays unchanged, the last ramped pair precedes the first fully
    # divided one
    assert ratio[mid[0] - 1] == 1.0 and abs(ratio[mid[-1] + 1] - 1.0 / s) < 1e-15


def test_attention_factor_matches_page():
    g = golden("page_numbers.json")["attention_factor"]
    af = O.yarn_attention_factor(8.0)
    assert abs(af - g["value"]) < g["tol"]
    assert O.yarn_attention_factor(1.0) == 1.0


def test_rope_position_zero_is_identity_times_m():
    x = rng(10).standard_normal(3 * 128).astype(np.float32)
    inv = O.rope_inv_freq(128, 500000.0)
    np.testing.assert_array_equal(O.rope(x, 3, 128, 0, inv), x)
    y = O.rope(x, 3, 128, 0, inv, 1.25)
    np.testing.assert_allclose(y, x.astype(np.float64) * 1.25, rtol=1e-7)


def test_rope_single_pair_rotation_closed_form():
    # D = 2: one pair with inverse frequency theta^0 = 1, so the angle is pos radians.
    inv = O.rope_inv_freq(2, 500000.0)
    for pos in (1, 2, 7, 1000):
        y = O.rope(np.array([1.0, 0.0], np.float32), 1, 2, pos, inv).astype(np.float64)
        np.testing.assert_allclose(y, [math.cos(pos), math.sin(pos)], atol=1e-7)
        y = O.rope(np.array([0.0, 1.0], np.float32), 1, 2, pos, inv).astype(np.float64)
        np.testing.assert_allclose(y, [-math.sin(pos), math.cos(pos)], atol=1e-7)


def test_rope_rotate_half_pairing_and_norms():
    """Pair i is (i, i + 64): a vector with only dims 3 and 67 set stays in them."""
    inv = O.rope_inv_freq(128, 500000.0)
    x = np.zeros(128, np.float32)
    x[3], x[67] = 0.6, -0.8
    y = O.rope(x, 1, 128, 12345, inv)
    nz = np.nonzero(y)[0]
    assert set(nz) <= {3, 67}
    assert abs(float(y[3]) ** 2 + float(y[67]) ** 2 - 1.0) < 1e-6
    xx = rng(11).standard_normal(8 * 128).astype(np.float32)
    m = O.yarn_attention_factor(8.0)
    invy = O.rope_inv_freq(128, 500000.0, 8.0, 8192)
    yy = O.rope(xx, 8, 128, 16384, invy, m).astype(np.float64).reshape(8, 2, 64)
    xr = xx.astype(np.float64).reshape(8, 2, 64)
    np.testing.assert_allclose(np.hypot(yy[:, 0], yy[:, 1]), m * np.hypot(xr[:, 0], xr[:, 1]), rtol=1e-6)


def test_rope_relative_position_property():
    inv = O.rope_inv_freq(128, 500000.0)
    r = rng(12)
    q = r.standard_normal(128).astype(np.float32)
    k = r.standard_normal(128).astype(np.float32)
    for p, pp in ((100, 37), (4096, 1), (16384, 16000)):
        lhs = float(np.dot(O.rope(q, 1, 128, p, inv).astype(np.float64),
                           O.rope(k, 1, 128, pp, inv).astype(np.float64)))
        rhs = float(np.dot(O.rope(q, 1, 128, p - pp, inv).astype(np.float64), k.astype(np.float64)))
        assert abs(lhs - rhs) < 2e-5 * 128


# ---- attention (P10, P11) ----------------------------------------------------------

def _attn_brute(q, Kc, Vc, Hq, Hkv, D, pos, window):
    lo = max(0, pos - window + 1) if window > 0 else 0
    out = np.zeros((Hq, D))
    for h in range(Hq):
        kv = h // (Hq // Hkv)
        s = np.array([np.dot(q[h].astype(np.float64), Kc[kv, j].astype(np.float64))
                      for j in range(lo, pos + 1)]) / math.sqrt(D)
        p = scipy.special.softmax(s)
        out[h] = p @ Vc[kv, lo:pos + 1].astype(np.float64)
    return out.reshape(-1)


def _attn_problem(Hq, Hkv, D, T, seed):
    r = rng(seed)
    q = r.standard_normal((Hq, D)).astype(np.float32)
    Kc = r.standard_normal((Hkv, T, D)).astype(np.float32)
    Vc = r.standard_normal((Hkv, T, D)).astype(np.float32)
    return q, Kc, Vc


@pytest.mark.parametrize("Hq,Hkv,D,T,pos,window", [(4, 2, 8, 20, 17, 5), (5, 1, 16, 40, 39, 0),
                                                   (6, 3, 4, 9, 0, 3), (2, 2, 8, 12, 11, 12)])
def test_attention_brute_force(Hq, Hkv, D, T, pos, window):
    q, Kc, Vc = _attn_problem(Hq, Hkv, D, T, 13)
    got = O.attention(q, Kc, Vc, Hq, Hkv, D, pos, window)
    np.testing.assert_allclose(got, _attn_brute(q, Kc, Vc, Hq, Hkv, D, pos, window), rtol=1e-6, atol=1e-6)


def test_attention_zero_query_is_window_mean():
    Hq, Hkv, D, T, pos, W_ = 4, 1, 8, 30, 29, 7
    q, Kc, Vc = _attn_problem(Hq, Hkv, D, T, 14)
    got = O.attention(np.zeros_like(q), Kc, Vc, Hq, Hkv, D, pos, W_).reshape(Hq, D)
    ref = Vc[0, pos - W_ + 1:pos + 1].astype(np.float64).mean(axis=0)
    for h in range(Hq):
        np.testing.assert_allclose(got[h], ref, rtol=1e-6, atol=1e-7)


def test_attention_single_key_returns_value():
    q, Kc, Vc = _attn_problem(3, 3, 8, 5, 15)
    got = O.attention(q, Kc, Vc, 3, 3, 8, 0, 0).reshape(3, 8)
    np.testing.assert_array_equal(got, Vc[:, 0, :])


def test_swa_equals_full_when_window_covers_context():
    q, Kc, Vc = _attn_problem(5, 1, 16, 64, 16)
    a = O.attention(q, Kc, Vc, 5, 1, 16, 40, 41)
    b = O.attention(q, Kc, Vc, 5, 1, 16, 40, 0)
    c = O.attention(q, Kc, Vc, 5, 1, 16, 40, 4096)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(c, b)


def test_gqa_equals_mha_with_repeated_kv_heads():
    Hq, Hkv, D, T = 10, 2, 8, 24
    q, Kc, Vc = _attn_problem(Hq, Hkv, D, T, 17)
    g = O.attention(q, Kc, Vc, Hq, Hkv, D, 20, 9)
    Kr = np.repeat(Kc, Hq // Hkv, axis=0)
    Vr = np.repeat(Vc, Hq // Hkv, axis=0)
    m = O.attention(q, Kr, Vr, Hq, Hq, D, 20, 9)
    np.testing.assert_array_equal(g, m)


@pytest.mark.parametrize("pos,window", [(256, 64), (4096, 4096), (100, 7)])
def test_window_boundary_probes(pos, window):
    """A dominating key at j = pos - window must be ignored; the same key at
    j = pos - window + 1 must take over the output (bit-level decision)."""
    Hq, Hkv, D = 5, 1, 16
    T = pos + 1
    r = rng(18)
    q = np.ones((Hq, D), np.float32)
    Kc = (r.standard_normal((Hkv, T, D)) * 0.01).astype(np.float32)
    Vc = (r.standard_normal((Hkv, T, D)) * 0.01).astype(np.float32)
    marker_v = np.full(D, 1000.0, np.float32)
    for j, inside in ((pos - window, False), (pos - window + 1, True)):
        if j < 0:
            continue
        K2, V2 = Kc.copy(), Vc.copy()
        K2[0, j] = 100.0
        V2[0, j] = marker_v
        o = O.attention(q, K2, V2, Hq, Hkv, D, pos, window).reshape(Hq, D)
        if inside:
            assert np.all(np.abs(o - 1000.0) < 1e-3)
        else:
            assert np.all(np.abs(o) < 1.0)


# ---- elementwise --------------------------------------------------------------------

def test_swiglu_against_expit():
    u = np.linspace(-30, 30, 1001).astype(np.float32)
    v = rng(19).standard_normal(1001).astype(np.float32)
    z = O.swiglu(u, v)
    ref = u.astype(np.float64) * scipy.special.expit(u.astype(np.float64)) * v.astype(np.float64)
    np.testing.assert_allclose(z, ref, rtol=1e-6, atol=1e-30)
    assert O.swiglu(np.zeros(3, np.float32), np.ones(3, np.float32)).tolist() == [0.0, 0.0, 0.0]


def test_argmax_lowest_index_on_ties():
    x = np.array([1.0, 5.0, 2.0, 5.0, 5.0], np.float32)
    assert O.argmax(x) == 1
    assert O.argmax(np.array([-1.0, -1.0], np.float32)) == 0


def test_embed_exact_upcast():
    bits = np.array([0x3F80, 0xBF00, 0x0001], np.uint16)
    x = O.embed(bits)
    assert x[0] == 1.0 and x[1] == -0.5 and x[2] > 0.0


# ---- one decoder layer (P12 and the block structure) ---------------------------------

def _zeroed_layer(model, seed):
    """Layer tensors whose codes all equal their zero points (every projection is 0)."""
    T = W.layer_tensors(model, seed, 0)
    for name in ("qkv", "o", "gate", "up", "down"):
        qw, sc, zw = T[name]
        T[name] = (np.full_like(qw, 0x77777777), sc, np.full_like(zw, 0x77777777))
    return T


def test_layer_with_zero_projections_is_identity():
    wl = W.config(0)
    m = wl.model
    T = _zeroed_layer(m, 0)
    Kc, Vc = W.kv_cache(m, 0, 0, wl.n_cached, wl.t_max)
    x = W.x_in(m, 0)
    y = O.layer_step(m, 0, T, x, Kc, Vc, wl.n_cached)
    np.testing.assert_array_equal(y, x)


def test_post_norm_places_unit_rms_branches_on_the_residual():
    """Reordered post-norm: h - x = RMSNorm(attn) and y - h = RMSNorm(mlp), so with unit
    gains each branch adds a vector of RMS ~1 whatever the scale of x (a pre-norm block
    would add an unnormalised branch)."""
    wl = W.config(0)
    m = wl.model
    T = W.layer_tensors(m, 0, 0)
    for gname in ("g_pa", "g_pf"):
        T[gname] = np.ones_like(T[gname])
    for scale in (1.0, 50.0):
        Kc, Vc = W.kv_cache(m, 0, 0, wl.n_cached, wl.t_max)
        x = (W.x_in(m, 0) * scale).astype(np.float32)
        tr = {}
        y = O.layer_step(m, 0, T, x, Kc, Vc, wl.n_cached, tr)
        h = tr["h"].astype(np.float64)
        rms_attn = math.sqrt(np.mean((h - x) ** 2))
        rms_mlp = math.sqrt(np.mean((y.astype(np.float64) - h) ** 2))
        assert abs(rms_attn - 1.0) < 1e-4 * scale and abs(rms_mlp - 1.0) < 1e-4 * scale


def test_qk_norm_is_over_the_full_projection():
    """At pos 0 RoPE is the identity, so with unit gains the q fed to attention has RMS 1
    over all 5 heads together, while single heads do not."""
    wl = W.config(0)
    m = wl.model
    T = W.layer_tensors(m, 0, 0)
    T["g_q"] = np.ones_like(T["g_q"])
    T["g_k"] = np.ones_like(T["g_k"])
    Kc, Vc = W.kv_cache(m, 0, 0, 0, 8)
    tr = {}
    O.layer_step(m, 0, T, W.x_in(m, 0), Kc, Vc, 0, tr)
    q = tr["q"].astype(np.float64)
    assert abs(np.mean(q ** 2) - 1.0) < 1e-5
    per_head = np.mean(q.reshape(m.hq, m.hd) ** 2, axis=1)
    assert np.max(np.abs(per_head - 1.0)) > 1e-3
    np.testing.assert_array_equal(Kc[:, 0, :].reshape(-1), tr["k"])   # k appended at slot pos
    np.testing.assert_array_equal(Vc[:, 0, :].reshape(-1), tr["v"])


def test_qk_norm_comes_before_the_rotation():
    """Norm first, then RoPE: with gains that differ between the two members of each
    rotation pair (i, i + 64), the q and k the layer feeds to attention at position p
    are a pure per-pair rotation of those at position 0, so every pair keeps its
    length. Rotating first and normalising afterwards would scale the rotated pair by
    unequal gains and change the lengths; the test computes that order too and checks
    that the invariant catches it."""
    wl = W.config(0)
    m = wl.model
    T = W.layer_tensors(m, 0, 0)
    half = np.concatenate([np.ones(64), 3.0 * np.ones(64)]).astype(np.float32)
    T["g_q"] = np.tile(half, m.hq)
    T["g_k"] = np.tile(half, m.hkv)
    x = W.x_in(m, 0)
    outs = {}
    for p in (0, 37):
        Kc, Vc = W.kv_cache(m, 0, 0, 40, 64)
        tr = {}
        O.layer_step(m, 0, T, x, Kc, Vc, p, tr)
        outs[p] = tr

    def pair_len(v, H):
        v = v.astype(np.float64).reshape(H, 2, 64)
        return np.sqrt(v[:, 0] ** 2 + v[:, 1] ** 2)

    for key, H in (("q", m.hq), ("k", m.hkv)):
        l0, lp = pair_len(outs[0][key], H), pair_len(outs[37][key], H)
        assert np.max(np.abs(lp - l0) / l0) < 1e-5
        assert np.max(np.abs(outs[37][key] - outs[0][key])) > 1e-2   # position 37 does rotate
    # the other order on the same projection: rotate, then normalise
    q_raw = outs[37]["qkv"][:m.hq * m.hd]
    inv, msc = O.rope_params(m, 0)
    swapped = O.rmsnorm(O.rope(q_raw, m.hq, m.hd, 37, inv, msc), T["g_q"], m.eps)
    ls = pair_len(swapped, m.hq)
    assert np.max(np.abs(ls - pair_len(outs[0]["q"], m.hq)) / ls) > 1e-2


def test_layer_types_use_yarn_only_on_full_layers():
    m = W.olmo3_32b(n_layers=8)
    assert m.layer_types == [0, 0, 0, 1, 0, 0, 0, 1]
    inv_s, m_s = O.rope_params(m, 0)
    inv_f, m_f = O.rope_params(m, 1)
    assert m_s == 1.0 and abs(m_f - 1.2079441541679836) < 1e-15
    np.testing.assert_array_equal(inv_s, O.rope_inv_freq(128, 500000.0))
    assert np.all(inv_f <= inv_s) and inv_f[-1] == inv_s[-1] / 8.0
