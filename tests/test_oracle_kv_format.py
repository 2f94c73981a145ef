"""Pins of the oracle's KV-cache formats: bfloat16 elements and the sliding-window
ring (the card's planned cache: bf16, and only the window kept on the SWA layers).

Each pin ties the oracle to something other than itself: torch's own float ->
bfloat16 conversion and hand-worked bit patterns for the rounding; exact
equivalences between storage layouts that hold the same values (a ring read through
j mod W against the flat cache, bf16 bits against f32 copies of the same values).
"""
import numpy as np
import pytest
import torch

import oracle as O
from oracle import runner as R
from synth import workloads as W


def _bits(x):
    return np.asarray(x, np.float32).view(np.uint32)


def _f32(bits):
    return np.asarray(bits, np.uint32).view(np.float32)


def _up(b16):
    """Exact f32 values of bfloat16 bit patterns."""
    return (np.asarray(b16, np.uint32) << 16).view(np.float32)


# ---- rounding at the store -----------------------------------------------------------------

def test_round_bf16_hand_worked_patterns():
    cases = [
        (0x3F800000, 0x3F80),   # 1.0 exact
        (0x3F808000, 0x3F80),   # tie, kept pattern even: stays
        (0x3F818000, 0x3F82),   # tie, kept pattern odd: rounds up to even
        (0x3F808001, 0x3F81),   # just above half: up
        (0x3F807FFF, 0x3F80),   # just below half: down
        (0xBF818000, 0xBF82),   # sign does not change the rule
        (0x7F7FFFFF, 0x7F80),   # largest f32 rounds to infinity
        (0x7F7F7FFF, 0x7F7F),   # largest bf16 stays finite
        (0x00000001, 0x0000),   # smallest subnormal rounds to +0
        (0x00008000, 0x0000),   # tie at zero: even
        (0x00018000, 0x0002),   # subnormal tie, odd: up
        (0x80000000, 0x8000),   # -0
        (0x7F800000, 0x7F80),   # +inf
        (0xFF800000, 0xFF80),   # -inf
    ]
    got = O.round_bf16(_f32([c[0] for c in cases]))
    assert [int(g) for g in got] == [c[1] for c in cases]
    nan = O.round_bf16(_f32([0x7FC00000, 0xFFA00001, 0x7F800001]))
    assert all(np.isnan(_up(nan)))


def test_round_bf16_matches_torch_conversion():
    r = np.random.default_rng(7)
    # random bit patterns over every finite exponent, plus scaled normals
    bits = r.integers(0, 2**32, 200000, dtype=np.uint64).astype(np.uint32)
    bits = bits[(bits & 0x7F800000) != 0x7F800000]
    x = np.concatenate([_f32(bits), r.standard_normal(100000).astype(np.float32) * 3])
    ours = O.round_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


# ---- bf16 storage reads back exactly ---------------------------------------------------------

def _cache(Hkv, T, D, seed):
    r = np.random.default_rng(seed)
    return (r.standard_normal((Hkv, T, D)).astype(np.float32), r.standard_normal((Hkv, T, D)).astype(np.float32))


def test_bf16_cache_equals_f32_cache_of_the_same_values():
    Hq, Hkv, D, T, pos = 6, 2, 16, 50, 43
    K, V = _cache(Hkv, T, D, 1)
    q = np.random.default_rng(2).standard_normal(Hq * D).astype(np.float32)
    Kb, Vb = O.round_bf16(K), O.round_bf16(V)
    for window in (0, 9):
        a = O.attention_kv(q, Kb, Vb, Hq, Hkv, D, pos, window, False)
        b = O.attention(q, _up(Kb), _up(Vb), Hq, Hkv, D, pos, window)
        assert np.array_equal(a, b)
        # and the rounding matters: the unrounded cache gives another result
        assert not np.array_equal(a, O.attention(q, K, V, Hq, Hkv, D, pos, window))


# ---- the sliding-window ring -----------------------------------------------------------------

@pytest.mark.parametrize("Wn,pos", [(8, 43), (8, 7), (8, 8), (16, 16), (5, 49)])
def test_ring_attention_equals_flat(Wn, pos):
    """Key j stored at slot j mod W of a W-slot ring gives exactly the flat result."""
    Hq, Hkv, D, T = 4, 2, 16, 50
    K, V = _cache(Hkv, T, D, 3)
    q = np.random.default_rng(4).standard_normal(Hq * D).astype(np.float32)
    Kr = np.zeros((Hkv, Wn, D), np.float32)
    Vr = np.zeros((Hkv, Wn, D), np.float32)
    for j in range(max(0, pos - Wn + 1), pos + 1):
        Kr[:, j % Wn] = K[:, j]
        Vr[:, j % Wn] = V[:, j]
    flat = O.attention(q, K, V, Hq, Hkv, D, pos, Wn)
    assert np.array_equal(O.attention_kv(q, Kr, Vr, Hq, Hkv, D, pos, Wn, True), flat)
    Kb, Vb = O.round_bf16(Kr), O.round_bf16(Vr)
    assert np.array_equal(O.attention_kv(q, Kb, Vb, Hq, Hkv, D, pos, Wn, True),
                          O.attention(q, _up(O.round_bf16(K)), _up(O.round_bf16(V)), Hq, Hkv, D, pos, Wn))


def test_ring_with_a_shifted_slot_map_is_detected():
    """A ring filled one slot off (key j at (j + 1) mod W) must not reproduce the flat
    result: the slot map is what the ring test pins."""
    Hq, Hkv, D, T, Wn, pos = 4, 2, 16, 50, 8, 43
    K, V = _cache(Hkv, T, D, 5)
    q = np.random.default_rng(6).standard_normal(Hq * D).astype(np.float32)
    Kr = np.zeros((Hkv, Wn, D), np.float32)
    Vr = np.zeros((Hkv, Wn, D), np.float32)
    for j in range(pos - Wn + 1, pos + 1):
        Kr[:, (j + 1) % Wn] = K[:, j]
        Vr[:, j % Wn] = V[:, j]
    assert not np.array_equal(O.attention_kv(q, Kr, Vr, Hq, Hkv, D, pos, Wn, True),
                              O.attention(q, K, V, Hq, Hkv, D, pos, Wn))


def _tiny_wl(kv_dtype, ring, n_cached, layer_type=W.SWA, model_id=40):
    m = W.tiny(model_id)
    m.layer_types = [layer_type]
    m.kv_dtype, m.swa_ring = kv_dtype, ring
    return W.Workload("tiny-kv-format", m, seed=0, n_cached=n_cached, t_max=n_cached + 1)


@pytest.mark.parametrize("kv_dtype", [0, 1])
@pytest.mark.parametrize("layer_type", [W.SWA, W.FULL])
def test_ring_layer_step_equals_flat(kv_dtype, layer_type):
    """One layer at a position past the window (the ring has wrapped three times):
    the ring model's output and the new key's stored bits equal the flat model's."""
    n = 200
    tr_f, tr_r = {}, {}
    yf, Kf, Vf = R.run_layer(_tiny_wl(kv_dtype, False, n, layer_type), trace=tr_f)
    yr, Kr, Vr = R.run_layer(_tiny_wl(kv_dtype, True, n, layer_type), trace=tr_r)
    assert np.array_equal(yf, yr)
    slot = n % Kr.shape[1]
    assert Kr.shape[1] == (64 if layer_type == W.SWA else n + 1)
    assert np.array_equal(Kr[:, slot], Kf[:, n]) and np.array_equal(Vr[:, slot], Vf[:, n])


def test_bf16_layer_stores_the_rounded_key_and_attends_to_it():
    n = 100
    tr = {}
    wl = _tiny_wl(1, True, n)
    y, Kc, Vc = R.run_layer(wl, trace=tr)
    m = wl.model
    slot = n % Kc.shape[1]
    assert np.array_equal(Kc[:, slot].ravel(), O.round_bf16(tr["k"]))
    assert np.array_equal(Vc[:, slot].ravel(), O.round_bf16(tr["v"]))
    # the attention output is the f32 attention over the exact values the ring holds
    o = O.attention_kv(tr["q"], _up(Kc), _up(Vc), m.hq, m.hkv, m.hd, n, m.window, True)
    assert np.array_equal(o, tr["o"])
    # while the f32-cache model, whose new key is not rounded, differs
    tr32 = {}
    R.run_layer(_tiny_wl(0, True, n), trace=tr32)
    assert not np.array_equal(tr32["o"], tr["o"])


def test_prefill_through_a_wrapping_ring_equals_flat():
    """Teacher-forced prefill of 150 tokens over [SWA, FULL] with a 64-slot ring: every
    SWA slot is overwritten twice, and the last hidden state equals the flat cache's."""
    def wl(ring):
        m = W.tiny(41)
        m.n_layers, m.layer_types, m.vocab = 2, [W.SWA, W.FULL], 512
        m.kv_dtype, m.swa_ring = 1, ring
        return W.Workload("tiny-prefill-ring", m, seed=0, n_cached=10, t_max=170, use_tokens=True)
    toks = W.prompt_tokens(wl(False).model, 0, 150)
    a = R.run_prefill(wl(False), toks, final=False)
    b = R.run_prefill(wl(True), toks, final=False)
    assert np.array_equal(a["y"], b["y"])
    assert b["K"][0].shape[1] == 64 and b["K"][1].shape[1] == 170
    for j in range(160 - 64, 160):   # the ring holds the last 64 positions
        assert np.array_equal(b["K"][0][:, j % 64], a["K"][0][:, j])
        assert np.array_equal(b["V"][0][:, j % 64], a["V"][0][:, j])
    assert np.array_equal(b["K"][1], a["K"][1])
