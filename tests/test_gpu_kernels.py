"""Per-entry-point parity of the HIP path against the CPU oracle (GPU required).

Bars: bit-exact for unpacking/dequantisation and for the attention window's index
set; normwise ||gpu - oracle||_inf / ||oracle||_inf for floats (1e-5 for a single
GEMV, whose only deviation is the 24-bit block encoding of x and f32 summation;
1e-5 for norms and rotary; 1e-5 for attention)."""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth
from synth import workloads as W
from synth.device import w4_to_device
from swa_attention_amd import ops
from gpu_util import announce, device, normwise

pytestmark = pytest.mark.gpu


def _w4(N, K, seed, group=128, zeros=True, scale_dtype=0):
    m = W.tiny()
    m.group = group
    c, s, z = W.w4_linear(m, seed, 0, W.K_QKV, N, K)
    if scale_dtype == 1:
        s = synth.uniform_bf16(synth.key(seed, 999), s.size, 0.002, 0.02).reshape(s.shape)
    return c, s, (z if zeros else None)


@pytest.mark.parametrize("N,K,group,zeros,sd", [(896, 640, 128, True, 0), (640, 1728, 128, True, 0),
                                                (37, 256, 32, False, 1), (5, 5120, 128, True, 0)])
def test_dequant_bit_exact(N, K, group, zeros, sd):
    dev = device()
    announce(f"dequant N={N} K={K} group={group}")
    c, s, z = _w4(N, K, 1, group, zeros, sd)
    w = w4_to_device(c, s, z, K, dev, group, sd)
    got = ops.atlas_w4_dequant(w).cpu().numpy()
    ref = O.dequant(c, s, z, K, group, sd)
    np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("N,K", [(64, 640), (40, 1728), (16, 5120)])
def test_gemv_one_hot_columns_bit_exact(N, K):
    """x = e_j makes the integer-dot GEMV return column j of the dequantised matrix;
    it must match the oracle bit for bit (unpacking, zero and scale selection)."""
    dev = device()
    announce(f"gemv one-hot N={N} K={K}")
    c, s, z = _w4(N, K, 2)
    w = w4_to_device(c, s, z, K, dev)
    ref = O.dequant(c, s, z, K)
    cols = sorted(set([0, 1, 7, 8, 31, 32, 127, 128, K // 2, K - 65, K - 33, K - 1]))
    for j in cols:
        x = torch.zeros(K, dtype=torch.float32, device=dev)
        x[j] = 1.0
        y = ops.atlas_w4_gemv(w, x).cpu().numpy()
        np.testing.assert_array_equal(y.view(np.uint32), ref[:, j].copy().view(np.uint32), err_msg=f"col {j}")


@pytest.mark.parametrize("N,K", [(896, 640), (640, 640), (1728, 640), (640, 1728), (1001, 5120),
                                 (7168, 5120), (5120, 5120), (27648, 5120), (5120, 27648), (3, 256), (130, 4096)])
def test_gemv_matches_oracle(N, K):
    dev = device()
    announce(f"gemv N={N} K={K}")
    c, s, z = _w4(N, K, 3)
    x = synth.normal_f32(synth.key(3, 7), K)
    w = w4_to_device(c, s, z, K, dev)
    y = ops.atlas_w4_gemv(w, torch.from_numpy(x).to(dev)).cpu().numpy()
    ref = O.w4_gemv(c, s, z, K, x)
    assert normwise(y, ref) < 1e-5


@pytest.mark.parametrize("N,K,B,group,zeros,sd", [
    (896, 640, 3, 128, True, 0), (1728, 640, 8, 128, True, 0), (640, 1728, 5, 128, True, 0),
    (33, 640, 7, 128, False, 1), (1001, 1024, 2, 256, False, 1), (300, 2048, 1, 512, True, 0),
    (130, 4096, 8, 1024, True, 0), (7168, 5120, 8, 128, True, 0), (5120, 6144, 4, 128, True, 0),
    (5120, 27648, 8, 128, True, 0), (27648, 5120, 6, 128, True, 0)])
def test_gemv_batch_matches_oracle(N, K, B, group, zeros, sd):
    """The batched W4 GEMV (int8 matrix cores, 24-bit block fixed-point activations)
    against the f64 oracle, vector by vector: ragged row tiles, a 64-column last block
    (K = 1,728), groups of 128 to 1,024, symmetric codes and bf16 scales, chunks split
    over blocks (K = 27,648), 1 to 8 vectors. The only deviation is the 24-bit encoding
    of x and f32 summation, so the single GEMV's 1e-5 bar applies."""
    dev = device()
    announce(f"gemv batch N={N} K={K} B={B} group={group}")
    c, s, z = _w4(N, K, 11, group, zeros, sd)
    w = w4_to_device(c, s, z, K, dev, group, sd)
    xs = np.stack([synth.normal_f32(synth.key(11, 100 + v), K) for v in range(B)])
    y = ops.atlas_w4_gemv_batch(w, torch.from_numpy(xs).to(dev)).cpu().numpy()
    for v in range(B):
        ref = O.w4_gemv(c, s, z, K, xs[v], group, sd)
        assert normwise(y[v], ref) < 1e-5, v


def test_gemv_batch_one_hot_columns_bit_exact():
    """Eight one-hot vectors at once: each output row is its column of the dequantised
    matrix bit for bit (code and zero selection, scale, the digit recombination; the
    power-of-two block scale makes the encoding exact)."""
    dev = device()
    N, K = 1001, 1728
    announce(f"gemv batch one-hot N={N} K={K}")
    c, s, z = _w4(N, K, 12)
    w = w4_to_device(c, s, z, K, dev)
    ref = O.dequant(c, s, z, K)
    for cols in ([0, 1, 7, 8, 31, 32, 127, 128], [129, 511, 512, 640, 1023, K - 65, K - 64, K - 1]):
        x = np.zeros((8, K), dtype=np.float32)
        for v, j in enumerate(cols):
            x[v, j] = 1.0
        y = ops.atlas_w4_gemv_batch(w, torch.from_numpy(x).to(dev)).cpu().numpy()
        for v, j in enumerate(cols):
            np.testing.assert_array_equal(y[v].view(np.uint32), ref[:, j].copy().view(np.uint32), err_msg=f"col {j}")


def test_gemv_batch_heavy_tailed_and_zero_rows():
    """Inputs spanning 12 orders of magnitude, an all-zero vector and a vector of equal
    values: the block encoding keeps f32-level error, and a zero vector gives exact
    zeros."""
    dev = device()
    N, K = 512, 5120
    c, s, z = _w4(N, K, 13)
    r = np.random.default_rng(6)
    xs = np.stack([(r.standard_normal(K) * 10.0 ** r.uniform(-6, 6, K)).astype(np.float32),
                   np.zeros(K, dtype=np.float32), np.full(K, 0.37, dtype=np.float32)])
    w = w4_to_device(c, s, z, K, dev)
    y = ops.atlas_w4_gemv_batch(w, torch.from_numpy(xs).to(dev)).cpu().numpy()
    assert normwise(y[0], O.w4_gemv(c, s, z, K, xs[0])) < 1e-5
    assert not y[1].any()
    assert normwise(y[2], O.w4_gemv(c, s, z, K, xs[2])) < 1e-5


@pytest.mark.parametrize("M,N,K,group,zeros,sd", [
    (1, 96, 640, 128, True, 0), (17, 130, 640, 128, True, 0), (64, 256, 1728, 128, True, 0),
    (130, 200, 640, 64, False, 1), (70, 64, 256, 32, True, 0), (200, 896, 640, 128, True, 0),
    (65, 129, 5120, 128, True, 0),
    # a few rows (the 16-row tile of batched decode)
    (8, 300, 640, 32, False, 1), (5, 1001, 5120, 64, True, 0), (16, 7168, 1728, 128, True, 0)])
def test_gemm_matches_oracle(M, N, K, group, zeros, sd):
    """The matrix-core W4 GEMM (prefill projections) against the f64 oracle row by row:
    ragged row and column tiles, a partial last group (K = 1,728), groups 32/64/128,
    symmetric codes and bf16 scales. The activations pass through bf16 hi/lo planes (16
    significant bits), so the bar is 2e-5 normwise. More than 16 rows with whole groups
    of 128 take the int8 kernel, which rounds those planes to integer multiples of a
    power-of-two s with max|row group| / (127 * 2^16) <= s: at most s/2 more (1.2e-7 of
    the group's largest value), under the same bar."""
    dev = device()
    announce(f"gemm M={M} N={N} K={K} group={group}")
    c, s, z = _w4(N, K, 11, group, zeros, sd)
    A = np.stack([synth.normal_f32(synth.key(11, 100 + i), K) for i in range(M)])
    w = w4_to_device(c, s, z, K, dev, group, sd)
    C = ops.atlas_w4_gemm(w, torch.from_numpy(A).to(dev)).cpu().numpy()
    ref = np.stack([O.w4_gemv(c, s, z, K, A[i], group, sd) for i in range(M)])
    assert normwise(C, ref) < _gemm_bar(M, K, group)


def _gemm_bar(M, K, group):
    return 2e-5


@pytest.mark.parametrize("K,group", [(1728, 128), (1280, 128), (1280, 32)])
def test_gemm_one_hot_rows_bit_exact(K, group):
    """Rows of A that are unit vectors e_j (exact in bf16, lo plane zero) give column j
    of the dequantised matrix bit for bit: unpacking, zero point and scale selection.
    A few rows take the small-row paths: K = 1,728 the 16-row LDS tile, K a multiple
    of 128 the kernel that feeds the codes to the matrix cores through a transpose."""
    dev = device()
    N = 200
    c, s, z = _w4(N, K, 12, group)
    cols = [0, 1, 7, 8, 31, 32, 63, 64, 127, 128, 129, 1000, K - 65, K - 64, K - 1]
    A = np.zeros((len(cols), K), dtype=np.float32)
    for i, j in enumerate(cols):
        A[i, j] = 1.0
    w = w4_to_device(c, s, z, K, dev, group)
    C = ops.atlas_w4_gemm(w, torch.from_numpy(A).to(dev)).cpu().numpy()
    ref = O.dequant(c, s, z, K, group)
    for i, j in enumerate(cols):
        np.testing.assert_array_equal(C[i].view(np.uint32), ref[:, j].copy().view(np.uint32), err_msg=f"col {j}")


@pytest.mark.parametrize("K,group", [(1280, 128), (2048, 256), (1536, 512)])
def test_gemm_int8_one_hot_rows_bit_exact(K, group):
    """The int8 kernel (more than 16 rows, groups of 128-512): a unit row e_j is scaled
    by a power of two, so its digits and the group's digit sums are exact and the row
    equals column j of the dequantised matrix bit for bit; zero rows give zeros. Also
    a row of one value repeated (every group at its full range) against the oracle."""
    dev = device()
    N = 200
    c, s, z = _w4(N, K, 14, group)
    cols = [0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 63, 64, 127, 128, 129, K - 8, K - 1]
    M = len(cols) + 4
    A = np.zeros((M, K), dtype=np.float32)
    for i, j in enumerate(cols):
        A[i, j] = 1.0
    A[len(cols) + 1, :] = -0.75
    w = w4_to_device(c, s, z, K, dev, group)
    C = ops.atlas_w4_gemm(w, torch.from_numpy(A).to(dev)).cpu().numpy()
    ref = O.dequant(c, s, z, K, group)
    for i, j in enumerate(cols):
        np.testing.assert_array_equal(C[i].view(np.uint32), ref[:, j].copy().view(np.uint32), err_msg=f"col {j}")
    for i in (len(cols), len(cols) + 2, len(cols) + 3):
        assert not C[i].any(), i
    row = len(cols) + 1
    assert normwise(C[row], O.w4_gemv(c, s, z, K, A[row], group)) < 1e-6


@pytest.mark.parametrize("group", [64, 128])
def test_gemm_large_grid_sampled_rows(group):
    """A grid of 8,192 tiles (several per CU, tail round included): sampled rows of C
    against the oracle, and one-hot rows bit for bit."""
    dev = device()
    M, N, K = 1024, 32768, 256
    announce(f"gemm large grid M={M} N={N} K={K} group={group}")
    c, s, z = _w4(N, K, 13, group)
    A = np.stack([synth.normal_f32(synth.key(13, 100 + i), K) for i in range(M)])
    onehot = [(5, 0), (100, 63), (517, 64), (1023, K - 1)]
    for i, j in onehot:
        A[i] = 0.0
        A[i, j] = 1.0
    w = w4_to_device(c, s, z, K, dev, group)
    C = ops.atlas_w4_gemm(w, torch.from_numpy(A).to(dev)).cpu().numpy()
    for i in [0, 1, 63, 64, 511, 700, 1000, 1022]:
        ref = O.w4_gemv(c, s, z, K, A[i], group)
        assert normwise(C[i], ref) < _gemm_bar(M, K, group), i
    deq = O.dequant(c, s, z, K, group)
    for i, j in onehot:
        np.testing.assert_array_equal(C[i].view(np.uint32), deq[:, j].copy().view(np.uint32), err_msg=f"row {i}")


@pytest.mark.parametrize("group", [128, 512])
def test_gemm_int8_heavy_tailed_and_zero_groups(group):
    """The int8 kernel's group-scaled fixed point on rows whose values span twelve
    orders of magnitude, with whole groups of zeros and one group of a single huge
    value: each group takes its own power-of-two scale, so normwise error stays at the
    bf16 planes' level (2e-5), zero groups contribute exactly nothing, and rows that
    are zero except for one group equal that group's product alone."""
    dev = device()
    M, N, K = 40, 256, 2048
    c, s, z = _w4(N, K, 15, group)
    r = np.random.default_rng(16)
    A = (r.standard_normal((M, K)) * 10.0 ** r.uniform(-6, 6, (M, K))).astype(np.float32)
    A[3, :] = 0.0
    A[5, group:] = 0.0                    # only the first group is non-zero
    A[7, :group] = 0.0
    A[7, group + 3] = 3.0e7               # one huge value, the rest of its group at 1e-6..1e6
    w = w4_to_device(c, s, z, K, dev, group)
    C = ops.atlas_w4_gemm(w, torch.from_numpy(A).to(dev)).cpu().numpy()
    ref = np.stack([O.w4_gemv(c, s, z, K, A[i], group) for i in range(M)])
    for i in range(M):
        if i == 3:
            assert not C[i].any()
        else:
            assert normwise(C[i], ref[i]) < 2e-5, i


def test_gemv_heavy_tailed_input():
    """Inputs spanning 12 orders of magnitude within a chunk stay at f32-level error."""
    dev = device()
    N, K = 512, 5120
    c, s, z = _w4(N, K, 4)
    r = np.random.default_rng(5)
    x = (r.standard_normal(K) * 10.0 ** r.uniform(-6, 6, K)).astype(np.float32)
    w = w4_to_device(c, s, z, K, dev)
    y = ops.atlas_w4_gemv(w, torch.from_numpy(x).to(dev)).cpu().numpy()
    ref = O.w4_gemv(c, s, z, K, x)
    assert normwise(y, ref) < 1e-5


@pytest.mark.parametrize("n,resid", [(640, True), (5120, True), (5120, False), (1000, True)])
def test_rmsnorm_residual(n, resid):
    dev = device()
    x = synth.normal_f32(synth.key(6, n), n, 0.0, 30.0)
    g = synth.normal_f32(synth.key(7, n), n, 1.0, 0.02)
    r = synth.normal_f32(synth.key(8, n), n)
    t = lambda a: torch.from_numpy(a).to(dev)
    out = ops.atlas_rmsnorm_residual(t(x), t(g), t(r) if resid else None).cpu().numpy()
    ref = O.rmsnorm_residual(x, g, r) if resid else O.rmsnorm(x, g)
    assert normwise(out, ref) < 1e-6


@pytest.mark.parametrize("Hq,Hkv,pos,yarn", [(5, 1, 256, 1.0), (40, 8, 4096, 1.0), (40, 8, 16384, 8.0),
                                             (40, 8, 0, 8.0), (40, 8, 65535, 8.0)])
def test_qk_norm_rope(Hq, Hkv, pos, yarn):
    dev = device()
    announce(f"qk_norm_rope Hq={Hq} pos={pos} yarn={yarn}")
    D = 128
    q = synth.normal_f32(synth.key(9, 1), Hq * D, 0.0, 5.0)
    k = synth.normal_f32(synth.key(9, 2), Hkv * D, 0.0, 5.0)
    gq = synth.normal_f32(synth.key(9, 3), Hq * D, 1.0, 0.02)
    gk = synth.normal_f32(synth.key(9, 4), Hkv * D, 1.0, 0.02)
    t = lambda a: torch.from_numpy(a).to(dev)
    dq, dk = t(q), t(k)
    dpos = torch.tensor([pos], dtype=torch.int32, device=dev)
    rope = ops.rope_params(500000.0, yarn, 8192)
    ops.atlas_qk_norm_rope(dq, dk, t(gq), t(gk), Hq, Hkv, D, dpos, rope)
    inv = O.rope_inv_freq(D, 500000.0, yarn, 8192)
    m = O.yarn_attention_factor(yarn)
    rq = O.rope(O.rmsnorm(q, gq), Hq, D, pos, inv, m)
    rk = O.rope(O.rmsnorm(k, gk), Hkv, D, pos, inv, m)
    assert normwise(dq.cpu().numpy(), rq) < 1e-5
    assert normwise(dk.cpu().numpy(), rk) < 1e-5


def _attn_inputs(Hq, Hkv, T_max, n_fill, seed, dev):
    D = 128
    q = synth.normal_f32(synth.key(seed, 1), Hq * D)
    Kc = np.zeros((Hkv, T_max, D), np.float32)
    Vc = np.zeros((Hkv, T_max, D), np.float32)
    synth.normal_f32_3d_into(synth.key(seed, 2), Hkv, n_fill, D, T_max * D, D, 0.0, 1.0, Kc)
    synth.normal_f32_3d_into(synth.key(seed, 3), Hkv, n_fill, D, T_max * D, D, 0.0, 1.0, Vc)
    return q, Kc, Vc


@pytest.mark.parametrize("Hq,Hkv,T_max,pos,window", [(5, 1, 257, 256, 64), (40, 8, 4097, 4096, 4096),
                                                    (40, 8, 16385, 16384, 0), (40, 8, 16385, 16384, 4096),
                                                    (8, 8, 100, 0, 0), (10, 2, 1000, 999, 3),
                                                    (40, 8, 20000, 777, 4096)])
def test_gqa_decode_matches_oracle(Hq, Hkv, T_max, pos, window):
    dev = device()
    announce(f"gqa Hq={Hq} Hkv={Hkv} T_max={T_max} pos={pos} window={window}")
    q, Kc, Vc = _attn_inputs(Hq, Hkv, T_max, pos + 1, 11, dev)
    t = lambda a: torch.from_numpy(a).to(dev)
    dpos = torch.tensor([pos], dtype=torch.int32, device=dev)
    out = ops.atlas_gqa_decode(t(q), t(Kc), t(Vc), Hq, Hkv, 128, T_max, dpos, window).cpu().numpy()
    ref = O.attention(q, Kc, Vc, Hq, Hkv, 128, pos, window)
    assert normwise(out, ref) < 1e-5


@pytest.mark.parametrize("pos,window", [(256, 64), (4096, 4096), (5000, 4096), (70, 7)])
def test_gqa_window_probes_bit_level(pos, window):
    """A dominating key/value planted at pos - window is excluded, at pos - window + 1
    it takes over: the window's index set is exact."""
    dev = device()
    Hq, Hkv, D, T_max = 5, 1, 128, pos + 1
    r = np.random.default_rng(12)
    q = np.full(Hq * D, 0.05, np.float32)
    Kc = (r.standard_normal((Hkv, T_max, D)) * 0.01).astype(np.float32)
    Vc = (r.standard_normal((Hkv, T_max, D)) * 0.01).astype(np.float32)
    t = lambda a: torch.from_numpy(a).to(dev)
    dpos = torch.tensor([pos], dtype=torch.int32, device=dev)
    for j, inside in ((pos - window, False), (pos - window + 1, True)):
        if j < 0:
            continue
        K2, V2 = Kc.copy(), Vc.copy()
        K2[0, j] = 40.0
        V2[0, j] = 1000.0
        o = ops.atlas_gqa_decode(t(q), t(K2), t(V2), Hq, Hkv, D, T_max, dpos, window).cpu().numpy()
        if inside:
            assert np.all(o > 999.0), (j, o.min())
        else:
            assert np.all(np.abs(o) < 1.0), (j, np.abs(o).max())


def test_gqa_swa_equals_full_when_window_covers_context_and_split_invariance():
    dev = device()
    Hq, Hkv, pos = 40, 8, 3000
    q, Kc, Vc = _attn_inputs(Hq, Hkv, 4097, pos + 1, 13, dev)
    t = lambda a: torch.from_numpy(a).to(dev)
    dpos = torch.tensor([pos], dtype=torch.int32, device=dev)
    a = ops.atlas_gqa_decode(t(q), t(Kc), t(Vc), Hq, Hkv, 128, 4097, dpos, 0).cpu().numpy()
    b = ops.atlas_gqa_decode(t(q), t(Kc), t(Vc), Hq, Hkv, 128, 4097, dpos, 4096).cpu().numpy()
    assert normwise(a, b) < 1e-6
    # a larger cache allocation changes the split count, not the result
    Kb = np.zeros((Hkv, 16385, 128), np.float32)
    Vb = np.zeros((Hkv, 16385, 128), np.float32)
    Kb[:, :4097] = Kc
    Vb[:, :4097] = Vc
    c = ops.atlas_gqa_decode(t(q), t(Kb), t(Vb), Hq, Hkv, 128, 16385, dpos, 0).cpu().numpy()
    assert normwise(c, a) < 1e-6


def test_gqa_single_key_returns_value():
    dev = device()
    q, Kc, Vc = _attn_inputs(40, 8, 16, 1, 14, dev)
    t = lambda a: torch.from_numpy(a).to(dev)
    dpos = torch.tensor([0], dtype=torch.int32, device=dev)
    o = ops.atlas_gqa_decode(t(q), t(Kc), t(Vc), 40, 8, 128, 16, dpos, 4096).cpu().numpy().reshape(40, 128)
    for h in range(40):
        np.testing.assert_allclose(o[h], Vc[h // 5, 0], rtol=1e-6, atol=1e-6)
