"""On-device sampling (temperature, nucleus, inverse-CDF draw) against the oracle (GPU).

Where floating point decides the integer, the two sides decide from probabilities that
agree to about 1e-7 (f32 exp against f64), so a draw whose u lies within that distance
of a boundary between two tokens may go either way. The bar: the token is identical for
at least 95% of random draws at the card's settings over the full vocabulary, and every
token is valid by the oracle's own arithmetic (its probability reaches the nucleus
threshold, and u falls inside its cumulative interval, both up to 1e-5). Greedy, edge
and small cases must match exactly."""
import numpy as np
import pytest
import torch

import oracle as O
from swa_attention_amd import ops
from gpu_util import announce, device

pytestmark = pytest.mark.gpu

V_FULL = 100278


def _draw(logits_t, T, top_p, u, ws, dev):
    du = torch.tensor([u], dtype=torch.float32, device=dev)
    tok = ops.atlas_sample(logits_t, T, top_p, du, ws=ws)
    return int(tok.item())


def _oracle_structures(l, T, top_p):
    """The oracle's probabilities, nucleus threshold and cumulative masses (float64)."""
    l = np.asarray(l, np.float64)
    e = np.exp((l - l.max()) / T)
    order = np.argsort(-e, kind="stable")
    cum = np.cumsum(e[order])
    k = min(int(np.searchsorted(cum, top_p * e.sum(), side="left")), e.size - 1)
    tau = e[order[k]]
    inN = e >= tau
    cN = np.cumsum(np.where(inN, e, 0.0))
    return e, tau, inN, cN


def test_greedy_is_the_first_maximum():
    dev = device()
    r = np.random.default_rng(11)
    l = r.standard_normal(V_FULL).astype(np.float32)
    l[5000] = l[77000] = 9.0   # a tie: the lower index wins
    lt = torch.from_numpy(l).to(dev)
    ws = torch.empty(ops.atlas_sample_workspace_bytes(V_FULL), dtype=torch.uint8, device=dev)
    tok = ops.atlas_sample(lt, 0.0, ws=ws)
    assert int(tok.item()) == 5000 == O.sample_top_p(l, 0.0, 0.95, 0.5)


def test_card_settings_full_vocab_against_oracle():
    dev = device()
    announce("sampling, temperature 0.6, top-p 0.95, 100,278 tokens, 200 draws")
    r = np.random.default_rng(12)
    l = (r.standard_normal(V_FULL) * 1.43).astype(np.float32)
    lt = torch.from_numpy(l).to(dev)
    ws = torch.empty(ops.atlas_sample_workspace_bytes(V_FULL), dtype=torch.uint8, device=dev)
    e, tau, inN, cN = _oracle_structures(l, 0.6, 0.95)
    S = cN[-1]
    same = 0
    us = r.random(200)
    for u in us:
        t = _draw(lt, 0.6, 0.95, float(np.float32(u)), ws, dev)
        o = O.sample_top_p(l, 0.6, 0.95, float(np.float32(u)))
        same += t == o
        assert e[t] >= tau * (1 - 1e-5), (u, t, o)
        lo, hi = cN[t] - (e[t] if inN[t] else 0.0), cN[t]
        assert lo - 1e-5 * S <= np.float32(u) * S <= hi + 1e-5 * S, (u, t, o)
    print(f"identical tokens: {same}/200, nucleus size {int(inN.sum())}")
    assert same >= 190


def test_peaked_logits_every_draw_matches():
    dev = device()
    r = np.random.default_rng(13)
    l = r.standard_normal(V_FULL).astype(np.float32)
    l[r.choice(V_FULL, 10, replace=False)] += 9.0
    lt = torch.from_numpy(l).to(dev)
    ws = torch.empty(ops.atlas_sample_workspace_bytes(V_FULL), dtype=torch.uint8, device=dev)
    for m in range(64):
        u = (m + 0.37) / 64
        assert _draw(lt, 0.6, 0.95, u, ws, dev) == O.sample_top_p(l, 0.6, 0.95, float(np.float32(u)))


def test_vanishing_top_p_is_the_maximum():
    dev = device()
    r = np.random.default_rng(14)
    l = r.standard_normal(V_FULL).astype(np.float32)
    lt = torch.from_numpy(l).to(dev)
    ws = torch.empty(ops.atlas_sample_workspace_bytes(V_FULL), dtype=torch.uint8, device=dev)
    for u in (0.0, 0.3, 0.999):
        assert _draw(lt, 1.0, 1e-7, u, ws, dev) == int(np.argmax(l))


def test_stratified_draws_small_vocab():
    """2,000 draws on a grid of u over 37 tokens: the token counts equal the oracle's
    (a boundary flip moves one draw between neighbours)."""
    dev = device()
    r = np.random.default_rng(15)
    l = (r.standard_normal(37) * 1.4).astype(np.float32)
    lt = torch.from_numpy(l).to(dev)
    ws = torch.empty(ops.atlas_sample_workspace_bytes(37), dtype=torch.uint8, device=dev)
    g = np.zeros(37, np.int64)
    o = np.zeros(37, np.int64)
    M = 2000
    for m in range(M):
        u = float(np.float32((m + 0.5) / M))
        g[_draw(lt, 1.0, 0.9, u, ws, dev)] += 1
        o[O.sample_top_p(l, 1.0, 0.9, u)] += 1
    assert np.abs(g - o).sum() <= 4, (g, o)


def test_u_at_and_beyond_the_edges():
    dev = device()
    l = np.array([0.5, -3.0, 2.0, 1.0, -9.0, 2.0], np.float32)
    lt = torch.from_numpy(l).to(dev)
    ws = torch.empty(ops.atlas_sample_workspace_bytes(l.size), dtype=torch.uint8, device=dev)
    first, last = O.sample_top_p(l, 1.0, 0.9, 0.0), O.sample_top_p(l, 1.0, 0.9, 0.99999994)
    assert _draw(lt, 1.0, 0.9, 0.0, ws, dev) == first
    assert _draw(lt, 1.0, 0.9, -1.0, ws, dev) == first           # clamped to 0
    assert _draw(lt, 1.0, 0.9, 0.99999994, ws, dev) == last
    assert _draw(lt, 1.0, 0.9, 1.5, ws, dev) == last              # clamped below 1


def test_graph_replays_draw_like_eager_calls():
    dev = device()
    r = np.random.default_rng(16)
    l = (r.standard_normal(V_FULL) * 1.43).astype(np.float32)
    lt = torch.from_numpy(l).to(dev)
    ws = torch.empty(ops.atlas_sample_workspace_bytes(V_FULL), dtype=torch.uint8, device=dev)
    du = torch.zeros(1, dtype=torch.float32, device=dev)
    tok = torch.zeros(1, dtype=torch.int32, device=dev)
    s = torch.cuda.Stream()
    ops.atlas_sample(lt, 0.6, 0.95, du, tok, ws)   # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        ops.atlas_sample(lt, 0.6, 0.95, du, tok, ws, stream=s)
    for u in r.random(6):
        du.fill_(float(u))
        g.replay()
        torch.cuda.synchronize()
        replayed = int(tok.item())
        eager = _draw(lt, 0.6, 0.95, float(np.float32(u)), ws, dev)
        assert replayed == eager


@pytest.mark.parametrize("case", ["all_equal", "threshold_ties", "two_levels"])
def test_many_tied_values_at_the_threshold(case):
    """Inputs whose nucleus threshold sits among many equal probabilities, so the
    candidate list that pins the threshold's low bits is long: every logit equal (the
    nucleus is the whole vocabulary and the draw is uniform over it), half of the
    vocabulary tied just below a few large logits, and values spread over two
    adjacent binary orders of magnitude. Every draw must be valid by the oracle's own
    arithmetic (as in the full-vocabulary test: f32 against f64 probabilities can move
    a draw that lies within ~1e-7 of a boundary); where every probability is exactly 1
    the draw must equal the oracle's."""
    dev = device()
    r = np.random.default_rng(17)
    if case == "all_equal":
        l = np.zeros(V_FULL, np.float32)
    elif case == "threshold_ties":
        l = np.full(V_FULL, -1.0, np.float32)
        l[r.choice(V_FULL, V_FULL // 2, replace=False)] = 0.25
        l[r.choice(V_FULL, 5, replace=False)] = 6.0
    else:
        l = (np.log(1.0 + r.random(V_FULL)) * 0.6).astype(np.float32)
    lt = torch.from_numpy(l).to(dev)
    ws = torch.empty(ops.atlas_sample_workspace_bytes(V_FULL), dtype=torch.uint8, device=dev)
    announce(f"sampling with many ties ({case})")
    for T, p in ((0.6, 0.95), (1.0, 0.5), (1.0, 1.0)):
        e, tau, inN, cN = _oracle_structures(l, T, p)
        S = cN[-1]
        for u in (0.0, 0.1234, 0.5, 0.87654, 0.99999994):
            u32 = float(np.float32(u))
            t = _draw(lt, T, p, u32, ws, dev)
            o = O.sample_top_p(l, T, p, u32)
            if case == "all_equal":
                assert t == o, (u, T, p)
            assert e[t] >= tau * (1 - 1e-5), (case, u, T, p, t, o)
            lo, hi = cN[t] - (e[t] if inN[t] else 0.0), cN[t]
            assert lo - 1e-5 * S <= np.float32(u) * S <= hi + 1e-5 * S, (case, u, T, p, t, o)
