"""The seeded generator (bits and distributions) and the byte/FLOP accounting,
pinned to the numbers the pages print (tests/golden/page_numbers.json)."""
import json
import os

import numpy as np

import synth
from synth import workloads as W
from swa_attention_amd import accounting as A

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def page(name):
    with open(os.path.join(GOLD, "page_numbers.json")) as f:
        return json.load(f)[name]


def near(name, got):
    g = page(name)
    assert abs(got - g["value"]) <= g["tol"], (name, got, g)


# ---- generator ------------------------------------------------------------------

def test_splitmix64_reference_stream():
    # SplitMix64 seeded with 0: state advances by GAMMA, output = finaliser(state).
    # First outputs of the published generator for seed 0.
    expect = [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    got = [synth.lib().synth_hash(0, i) for i in range(3)]
    assert got == expect


def test_generator_is_deterministic_and_keyed():
    a = synth.codes(synth.key(0, 5), 1000)
    b = synth.codes(synth.key(0, 5), 1000)
    c = synth.codes(synth.key(0, 6), 1000)
    d = synth.codes(synth.key(1, 5), 1000)
    assert np.array_equal(a, b) and not np.array_equal(a, c) and not np.array_equal(a, d)


def test_code_and_zero_distributions():
    w = synth.codes(synth.key(0, 9), 200000)
    nib = ((w[:, None] >> (4 * np.arange(8, dtype=np.uint32))) & 15).reshape(-1)
    counts = np.bincount(nib, minlength=16)
    assert counts.min() > 0.95 * len(nib) / 16 and counts.max() < 1.05 * len(nib) / 16
    z = synth.zeros(synth.key(0, 10), 1000, 14)            # 14 groups: 2 words, 6 valid nibbles
    assert z.shape == (1000, 2) and np.all(z[:, 1] >> 24 == 0)


def test_f16_rounding_matches_numpy():
    vals = np.concatenate([np.linspace(0.002, 0.02, 5001), [1.0, 0.1, 65504.0, 1e-7, 3.0000001]])
    got = np.array([synth.f64_to_f16_bits(v) for v in vals], np.uint16)
    np.testing.assert_array_equal(got, vals.astype(np.float16).view(np.uint16))


def test_uniform_scales_range():
    s = synth.uniform_f16(synth.key(0, 11), 100000, 0.002, 0.02).view(np.float16).astype(np.float64)
    assert s.min() >= 0.002 - 1e-6 and s.max() <= 0.02 + 1e-5
    assert abs(s.mean() - 0.011) < 1e-4


def test_normal_moments_and_exact_grid():
    x = synth.normal_f32(synth.key(0, 12), 400000)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1.0) < 0.01
    assert np.all((x.astype(np.float64) * 65536) == np.round(x.astype(np.float64) * 65536))
    g = synth.normal_f32(synth.key(0, 13), 100000, 1.0, 0.02)
    assert abs(g.mean() - 1.0) < 1e-3 and abs(g.std() - 0.02) < 1e-3


def test_strided_fill_matches_dense_indexing():
    k = synth.key(0, 14)
    dense = synth.normal_f32(k, 2 * 3 * 8).reshape(2, 3, 8)
    buf = np.full((2, 5, 8), -7.0, np.float32)
    synth.normal_f32_3d_into(k, 2, 3, 8, 5 * 8, 8, 0.0, 1.0, buf)
    np.testing.assert_array_equal(buf[:, :3], dense)
    assert np.all(buf[:, 3:] == -7.0)


def test_tokens_in_vocab():
    t = synth.tokens(synth.key(0, 15), 100000, 100278)
    assert t.min() >= 0 and t.max() < 100278 and t.max() > 99000


def test_bf16_rows_are_row_slices():
    k = synth.key(0, 16)
    full = synth.normal_bf16_rows(k, 0, 10, 32, 0.0, 0.02)
    part = synth.normal_bf16_rows(k, 4, 3, 32, 0.0, 0.02)
    np.testing.assert_array_equal(part, full[4:7])


# ---- accounting pinned to the pages ---------------------------------------------

def test_parameter_counts():
    m = W.olmo3_32b()
    p = A.param_counts(m)
    assert p["per_layer"] == 487_604_224
    near("params_largest_layer", p["per_layer"])
    near("params_backbone", p["backbone"])
    near("params_embedding_head", p["emb_head"])
    near("params_total", p["total"])


def test_flop_model():
    m = W.olmo3_32b()
    near("decode_gflop_4k", A.decode_flops(m, 4096) / 1e9)
    near("prefill_tflop_4k", A.prefill_flops(m, 4096) / 1e12)


def test_kv_bytes():
    m = W.olmo3_32b()
    per_tok = sum(2 * m.hkv * m.hd * 4 for _ in range(m.n_layers))
    near("kv_f32_bytes_per_token", per_tok)
    full = m.layer_types.count(1)
    swa = m.layer_types.count(0)
    near("kv_swa_aware_f32_16k_gb", (full * 16384 + swa * 4096) * 2 * m.hkv * m.hd * 4 / 1e9)
    near("kv_bf16_global_bytes_per_token", full * 2 * m.hkv * m.hd * 2)
    near("kv_bf16_bytes_131k", full * 2 * m.hkv * m.hd * 2 * 131072 + swa * 2 * m.hkv * m.hd * 2 * 4096)


def test_checkpoint_bytes_in_the_pages_layout():
    """The card's layout (symmetric int4, group 32, bf16 scales) plus bf16 embedding and
    head reproduces the 19.6 GB checkpoint."""
    m = W.olmo3_32b()
    w4 = m.n_layers * sum(A.w4_bytes(N, K, group=32, zeros=False) for _, _, N, K in m.linears())
    total = w4 + 2 * m.vocab * m.d * 2
    near("checkpoint_gb", total / 1e9)


def test_our_layout_bytes():
    m = W.olmo3_32b()
    assert A.layer_w4_bytes(m) == 253_317_120
    sb = A.decode_step_bytes(m, 16384)
    assert sb.w4 == 64 * 253_317_120
    assert sb.kv == 48 * 33_554_432 + 16 * 134_225_920
    assert sb.lm_head == 1_026_846_720
    assert abs(sb.total / 1e9 - 21.0) < 0.01


def test_card_format_layer_bytes_and_generator():
    """The card's own W4 recipe (symmetric codes, group 32, bf16 scales): 0.5625 bytes per
    weight, 274,268,160 per full-size layer (the 274.3 MB of the scope table); the
    generator gives bf16 scale bits inside the scale range and no zero table."""
    m = W.card_format(W.olmo3_32b())
    assert A.layer_weight_count(m) == 487_587_840
    assert A.layer_w4_bytes(m) == 487_587_840 * 9 // 16 == 274_268_160
    c, sc, z = W.w4_linear(m, 0, 0, W.K_O, 64, 5120)
    assert z is None and c.shape == (64, 640) and sc.shape == (64, 160)
    v = (sc.astype(np.uint32) << 16).view(np.float32)
    assert v.min() >= 0.002 * (1 - 2 ** -8) and v.max() <= 0.02 * (1 + 2 ** -8)
    wl = W.config(5)
    assert wl.model.symmetric and wl.model.group == 32 and wl.model.scale_dtype == 1
    assert A.decode_step_bytes(wl.model, 16384).w4 == 64 * 274_268_160


def test_batch_sequence_zero_is_the_single_workload_and_others_differ():
    """Sequence 0 of a batch has exactly the single-sequence workload's token and
    caches; later sequences draw from their own streams, at their ragged positions."""
    m = W.tiny(60)
    single = W.Workload("s", m, seed=0, n_cached=100, t_max=120, use_tokens=True)
    batch = W.Workload("b", m, seed=0, n_cached=100, t_max=120, use_tokens=True, batch=3, batch_gap=30)
    assert [batch.seq_cached(b) for b in range(3)] == [100, 70, 40]
    toks = W.batch_tokens(batch)
    assert toks[0] == int(W.prompt_tokens(m, 0, 1)[0])
    assert len(set(toks.tolist())) == 3
    k0, v0 = W.kv_cache(m, 0, 0, 100, 120)
    kb0, vb0 = W.kv_cache(m, 0, 0, 100, 120, seq=0)
    kb1, _ = W.kv_cache(m, 0, 0, 70, 120, seq=1)
    assert np.array_equal(k0, kb0) and np.array_equal(v0, vb0)
    assert not np.array_equal(kb1[:, :70], k0[:, :70])
    assert not np.any(kb1[:, 70:])
