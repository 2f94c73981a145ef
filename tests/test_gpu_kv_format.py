"""Parity of the KV-cache formats on the GPU: bf16 elements and the sliding-window
ring (key j in slot j mod window), in the standalone attention, the decode step and
the prefill, against the CPU oracle (GPU).

Bar: attention outputs normwise 1e-5 on identical cache contents; hidden states and
logits normwise 1e-3 with identical argmax; stored f32 keys/values normwise 1e-3.
Stored bf16 keys/values: each side rounds its own f32 value, and those agree only to
the normwise tolerance, so each element may differ by that much plus one rounding
step (one unit in the last place of the larger of the two); the elements that differ
must not lean to one side (a truncating or away-from-zero rule would). The rounding
rule itself is checked bit for bit on values both sides compute exactly. Only the
expected slots are written."""
import numpy as np
import pytest
import torch

import oracle as O
import synth as S
from oracle import runner as R
from synth import workloads as W
from synth.device import build_model
from swa_attention_amd import ops
from gpu_util import TOL, announce, device, normwise

pytestmark = pytest.mark.gpu


def _up(b):
    """f32 values of bf16 bit patterns."""
    return (np.asarray(b).view(np.uint16).astype(np.uint32) << 16).view(np.float32)


def _np(t):
    a = t.detach().cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


def assert_kv_close(g, o, what=""):
    """GPU cache contents g against the oracle's o (same layout)."""
    if o.dtype == np.uint16:
        g = np.asarray(g).view(np.uint16)
        gv, ov = _up(g).astype(np.float64), _up(o).astype(np.float64)
        big = np.maximum(np.abs(gv), np.abs(ov))
        ulp = np.exp2(np.floor(np.log2(np.maximum(big, 2.0 ** -126))) - 7)
        bound = TOL * np.abs(ov).max() + ulp
        assert np.all(np.abs(gv - ov) <= bound), what
        diff = g != o
        assert np.mean(diff) < 0.25, what
        if diff.sum() >= 50:
            smaller = np.mean(np.abs(gv[diff]) < np.abs(ov[diff]))
            assert 0.3 < smaller < 0.7, (what, smaller)
    else:
        assert normwise(g, o) < TOL, what


# ---- standalone attention over every layout -------------------------------------------------

@pytest.mark.parametrize("Hq,Hkv,kv_dtype,ring,slots,pos,window", [
    (40, 8, 1, True, 4096, 16384, 4096),     # full-size SWA ring, wrapped four times
    (40, 8, 1, False, 16385, 16384, 0),      # full-size full layer, bf16
    (5, 1, 0, True, 64, 200, 64),            # f32 ring
    (5, 1, 1, True, 100, 250, 64),           # ring larger than the window
    (8, 1, 1, True, 64, 10, 64),             # ring not yet wrapped
    (10, 2, 1, False, 1000, 999, 3),         # bf16 flat, tiny window
])
def test_gqa_decode_kv_matches_oracle(Hq, Hkv, kv_dtype, ring, slots, pos, window):
    dev = device()
    announce(f"gqa_kv Hq={Hq} Hkv={Hkv} dtype={kv_dtype} ring={ring} slots={slots} pos={pos} window={window}")
    D = 128
    q = S.normal_f32(S.key(21, 1), Hq * D)
    npdt = np.uint16 if kv_dtype == 1 else np.float32
    Kc = np.zeros((Hkv, slots, D), npdt)
    Vc = np.zeros((Hkv, slots, D), npdt)
    j0 = max(0, pos + 1 - slots)
    S.normal_kv_into(S.key(21, 2), Hkv, pos + 1, D, j0, slots, kv_dtype, 0.0, 1.0, Kc)
    S.normal_kv_into(S.key(21, 3), Hkv, pos + 1, D, j0, slots, kv_dtype, 0.0, 1.0, Vc)
    t = lambda a: torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)
    dpos = torch.tensor([pos], dtype=torch.int32, device=dev)
    out = ops.atlas_gqa_decode_kv(t(q), t(Kc), t(Vc), Hq, Hkv, D, dpos, window, ring).cpu().numpy()
    ref = O.attention_kv(q, Kc, Vc, Hq, Hkv, D, pos, window, ring)
    err = normwise(out, ref)
    print("normwise", err)
    assert err < 1e-5


def test_gqa_decode_kv_rejects_positions_outside_the_layout():
    dev = device()
    Hq, Hkv, D, slots = 5, 1, 128, 64
    q = torch.ones(Hq * D, dtype=torch.float32, device=dev)
    Kc = torch.full((Hkv, slots, D), 0x3F80, dtype=torch.int16, device=dev)   # bf16 1.0
    Vc = torch.full_like(Kc, 0x3F80)
    for ring, pos in ((False, slots), (True, -1)):
        dpos = torch.tensor([pos], dtype=torch.int32, device=dev)
        out = ops.atlas_gqa_decode_kv(q, Kc, Vc, Hq, Hkv, D, dpos, 64, ring)
        assert torch.count_nonzero(out).item() == 0
    # a ring accepts any later position
    out = ops.atlas_gqa_decode_kv(q, Kc, Vc, Hq, Hkv, D, torch.tensor([10 ** 6], dtype=torch.int32, device=dev), 64,
                                  True)
    assert torch.count_nonzero(out).item() == Hq * D


# ---- decode step -------------------------------------------------------------------------------

def test_decode_swa_layer_full_size_bf16_ring():
    """One full-size SWA layer at 16,384 cached positions with a bf16 ring of 4,096
    slots (wrapped four times): output and the one slot written."""
    dev = device()
    wl = W.config(9)
    m = wl.model
    announce("decode OLMo-3-32B SWA layer, bf16 ring of 4,096 slots, 16,384 cached")
    dm = build_model(wl, dev, head=False)
    assert dm.layers[0].k_cache.shape == (m.hkv, m.window, m.hd)
    x = torch.from_numpy(W.x_in(m, wl.seed)).to(dev)
    out = torch.empty(m.d, dtype=torch.float32, device=dev)
    p = wl.n_cached
    ws = torch.empty(ops.atlas_decode_workspace_bytes(dm), dtype=torch.uint8, device=dev)
    k_before = _np(dm.layers[0].k_cache).copy()
    ops.atlas_decode_step(dm, torch.tensor([p], dtype=torch.int32, device=dev), hidden_in=x, hidden_out=out, ws=ws)
    torch.cuda.synchronize()
    assert ops.atlas_device_status(ws) == 0
    y, Kc, Vc = R.run_layer(wl, 0)
    gk, gv = _np(dm.layers[0].k_cache), _np(dm.layers[0].v_cache)
    slot = p % m.window
    changed = np.nonzero(np.any(gk != k_before, axis=(0, 2)))[0]
    assert list(changed) == [slot]
    assert_kv_close(gk[:, slot], Kc[:, slot], "k")
    assert_kv_close(gv[:, slot], Vc[:, slot], "v")
    err = normwise(out.cpu().numpy(), y)
    print("normwise", err)
    assert err < TOL


def test_bf16_store_rounds_to_nearest_even_bit_exact():
    """Integer inputs in [-3, 3], zero points 8 and unit scales make the raw value
    projection an exact integer on both sides (integer dot products; every partial sum
    is a small integer times a power of two), so the stored bf16 value of v must match
    the oracle's bit for bit. Odd integers in [257, 511] are halfway cases."""
    from synth.device import layer_to_device
    dev = device()
    m = W.tiny(45)
    m.layer_types = [W.SWA]
    m.kv_dtype = 1
    wl = W.Workload("tiny-exact-v", m, seed=0, n_cached=20, t_max=32)
    announce("bf16 store of exactly computed values (decode, tiny layer)")
    T = W.layer_tensors(m, 0, 0)
    codes, scales, zeros = T["qkv"]
    T["qkv"] = (codes, np.full_like(scales, 0x3C00), np.full_like(zeros, 0x88888888))   # f16 1.0, zero 8
    x = np.random.default_rng(3).integers(-3, 4, m.d).astype(np.float32)
    dm = build_model(wl, dev, head=False)
    dm.layers[0] = layer_to_device(m, 0, 0, wl.n_cached, wl.t_max, dev, tensors=T)
    ws = torch.empty(ops.atlas_decode_workspace_bytes(dm), dtype=torch.uint8, device=dev)
    ops.atlas_decode_step(dm, torch.tensor([20], dtype=torch.int32, device=dev), hidden_in=torch.from_numpy(x).to(dev),
                          ws=ws)
    torch.cuda.synchronize()
    Kc, Vc = W.kv_cache(m, 0, 0, wl.n_cached, wl.t_max)
    tr = {}
    O.layer_step(m, W.SWA, T, x, Kc, Vc, 20, tr)
    v = tr["v"]
    assert np.array_equal(v, np.round(v))                     # the projection is exact
    ties = np.sum((np.abs(v) > 256) & (np.abs(v) < 512) & (np.abs(v) % 2 == 1))
    assert ties >= 5, ties
    np.testing.assert_array_equal(_np(dm.layers[0].v_cache)[:, 20].ravel(), O.round_bf16(v))


def _tiny_stack(kv_dtype, ring, n_cached, t_max, model_id):
    m = W.tiny(model_id)
    m.n_layers = 4
    m.layer_types = [W.FULL if l % 4 == 3 else W.SWA for l in range(4)]
    m.vocab = 1000
    m.window = 64
    m.kv_dtype, m.swa_ring = kv_dtype, ring
    return W.Workload("tiny-stack-kv", m, seed=0, n_cached=n_cached, t_max=t_max, use_tokens=True, final_head=True)


@pytest.mark.parametrize("kv_dtype,ring", [(1, True), (1, False), (0, True)])
def test_decode_steps_tiny_stack_across_the_ring_wrap(kv_dtype, ring):
    """Three teacher-forced decode steps at positions 190..192 of a 4-layer stack with a
    64-slot ring (slot 190 mod 64 = 62, then 63, then 0): logits, argmax and caches."""
    dev = device()
    wl = _tiny_stack(kv_dtype, ring, 190, 200, 43)
    announce(f"decode tiny stack kv_dtype={kv_dtype} ring={ring}, 3 steps across the wrap")
    toks = W.prompt_tokens(wl.model, wl.seed, 3, stream=2)
    dm = build_model(wl, dev)
    ws = torch.empty(ops.atlas_decode_workspace_bytes(dm), dtype=torch.uint8, device=dev)
    d_toks = torch.from_numpy(toks).to(dev)
    logits = torch.empty(wl.model.vocab, dtype=torch.float32, device=dev)
    am = torch.empty(1, dtype=torch.int32, device=dev)
    for t in range(3):
        ops.atlas_decode_step(dm, torch.tensor([190 + t], dtype=torch.int32, device=dev), d_token=d_toks[t:t + 1],
                              logits=logits if t == 2 else None, argmax=am if t == 2 else None, ws=ws)
    torch.cuda.synchronize()
    assert ops.atlas_device_status(ws) == 0
    ref = R.run_prefill(wl, toks)   # teacher-forced decode of the three tokens
    assert normwise(logits.cpu().numpy(), ref["logits"]) < TOL
    assert int(am.item()) == ref["argmax"]
    for l in range(4):
        assert_kv_close(_np(dm.layers[l].k_cache), ref["K"][l], f"K layer {l}")
        assert_kv_close(_np(dm.layers[l].v_cache), ref["V"][l], f"V layer {l}")


# ---- prefill -----------------------------------------------------------------------------------

@pytest.mark.parametrize("kv_dtype,ring", [(1, True), (0, True), (1, False)])
def test_prefill_through_the_ring_then_decode(kv_dtype, ring):
    """150 prompt tokens after 10 cached ones: on a 64-slot ring every SWA slot is
    written twice within the prompt, and queries early in the prompt still read the
    keys the later ones displace. Then one decode step continues from the prefill."""
    dev = device()
    wl = _tiny_stack(kv_dtype, ring, 10, 170, 44)
    announce(f"prefill tiny stack kv_dtype={kv_dtype} ring={ring}: 150 tokens from position 10, then decode")
    toks = W.prompt_tokens(wl.model, wl.seed, 151, stream=3)
    dm = build_model(wl, dev)
    d_toks = torch.from_numpy(toks).to(dev)
    logits = torch.empty(wl.model.vocab, dtype=torch.float32, device=dev)
    am = torch.empty(1, dtype=torch.int32, device=dev)
    ws = torch.empty(ops.atlas_prefill_workspace_bytes(dm, 150), dtype=torch.uint8, device=dev)
    ops.atlas_prefill(dm, d_toks[:150], wl.n_cached, logits, am, ws)
    torch.cuda.synchronize()
    assert ops.atlas_device_status(ws) == 0
    ref = R.run_prefill(wl, toks[:150])
    assert normwise(logits.cpu().numpy(), ref["logits"]) < TOL
    assert int(am.item()) == ref["argmax"]
    for l in range(4):
        assert_kv_close(_np(dm.layers[l].k_cache), ref["K"][l], f"K layer {l}")
        assert_kv_close(_np(dm.layers[l].v_cache), ref["V"][l], f"V layer {l}")
    # one decode step at position 160 on top of the prefilled caches
    wsd = torch.empty(ops.atlas_decode_workspace_bytes(dm), dtype=torch.uint8, device=dev)
    ops.atlas_decode_step(dm, torch.tensor([160], dtype=torch.int32, device=dev), d_token=d_toks[150:151],
                          logits=logits, argmax=am, ws=wsd)
    torch.cuda.synchronize()
    ref2 = R.run_prefill(wl, toks)
    assert normwise(logits.cpu().numpy(), ref2["logits"]) < TOL
    assert int(am.item()) == ref2["argmax"]
