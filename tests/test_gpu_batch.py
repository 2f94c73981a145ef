"""Batched decode (B sequences, one token each, shared weights) against the oracle (GPU).

A batch is by definition B independent decode steps; the oracle runs them one by one.
Bar: per sequence, logits and hidden states normwise 1e-3 with identical argmax; the
new key and value of every layer in that sequence's own cache slot (f32 normwise 1e-3;
bf16 within the tolerance plus one rounding step), and no other slot written."""
import numpy as np
import pytest
import torch

from oracle import runner as R
from synth import workloads as W
from synth.device import build_model
from swa_attention_amd import ops
from gpu_util import TOL, announce, device, normwise

pytestmark = pytest.mark.gpu


def _up(b):
    return (np.asarray(b).view(np.uint16).astype(np.uint32) << 16).view(np.float32)


def _close_kv(g, o):
    if o.dtype == np.uint16 or g.dtype == np.int16:
        gv, ov = _up(g), _up(o)
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.maximum(np.abs(gv), np.abs(ov)), 2.0 ** -126))) - 7)
        return bool(np.all(np.abs(gv.astype(np.float64) - ov) <= TOL * np.abs(ov).max() + ulp))
    return normwise(g, o) < TOL


def _tiny_batch(kv_dtype, ring, batch=3, gap=37, model_id=50):
    m = W.tiny(model_id)
    m.n_layers = 4
    m.layer_types = [W.FULL if l % 4 == 3 else W.SWA for l in range(4)]
    m.vocab = 1000
    m.window = 64
    m.kv_dtype, m.swa_ring = kv_dtype, ring
    return W.Workload("tiny-batch", m, seed=0, n_cached=150, t_max=160, use_tokens=True, final_head=True,
                      batch=batch, batch_gap=gap)


def _run_batch(wl, dev, hidden=False):
    dm = build_model(wl, dev)
    B, m = wl.batch, wl.model
    toks = torch.from_numpy(W.batch_tokens(wl)).to(dev)
    pos = torch.tensor([wl.seq_cached(b) for b in range(B)], dtype=torch.int32, device=dev)
    logits = torch.empty((B, m.vocab), dtype=torch.float32, device=dev) if wl.final_head else None
    am = torch.empty(B, dtype=torch.int32, device=dev) if wl.final_head else None
    hid = torch.empty((B, m.d), dtype=torch.float32, device=dev) if hidden else None
    before = [(L.k_cache.clone(), L.v_cache.clone()) for L in dm.layers]
    ws = ops.atlas_decode_batch(dm, toks, pos, hidden_out=hid, logits=logits, argmax=am)
    torch.cuda.synchronize()
    return dm, ws, before, logits, am, hid


@pytest.mark.parametrize("kv_dtype,ring", [(0, False), (1, True), (0, True)])
def test_batch_tiny_stack_matches_oracle(kv_dtype, ring):
    dev = device()
    wl = _tiny_batch(kv_dtype, ring)
    announce(f"batched decode, tiny 4-layer stack, 3 sequences at 150/113/76, kv_dtype={kv_dtype} ring={ring}")
    dm, ws, before, logits, am, _ = _run_batch(wl, dev)
    assert ops.atlas_device_status(ws) == 0
    refs = R.run_decode_batch(wl, keep_kv=True)
    for b, ref in enumerate(refs):
        assert normwise(logits[b].cpu().numpy(), ref["logits"]) < TOL, b
        assert int(am[b].item()) == ref["argmax"], b
        pos = wl.seq_cached(b)
        for l, L in enumerate(dm.layers):
            slots = L.k_cache.shape[2]
            slot = pos % slots if (ring and wl.model.layer_types[l] == W.SWA) else pos
            gk, gv = L.k_cache[b].cpu().numpy(), L.v_cache[b].cpu().numpy()
            k0 = before[l][0][b].cpu().numpy()
            changed = np.nonzero(np.any(gk != k0, axis=(0, 2)))[0]
            assert list(changed) == [slot], (b, l, changed)
            k, v = ref["kv"][l]
            hk = k.reshape(wl.model.hkv, -1)
            hv = v.reshape(wl.model.hkv, -1)
            if kv_dtype == 1:
                import oracle as O
                hk, hv = O.round_bf16(hk), O.round_bf16(hv)
            assert _close_kv(gk[:, slot], hk) and _close_kv(gv[:, slot], hv), (b, l)


def test_batch_of_sixteen_the_maximum():
    """The largest batch (16 sequences, the 16-row MFMA tile full) at ragged positions
    150 down to 0 through the tiny 4-layer stack with bf16 KV on rings: logits and argmax
    of every sequence against the oracle."""
    dev = device()
    wl = _tiny_batch(1, True, batch=16, gap=10, model_id=53)
    announce("batched decode, tiny 4-layer stack, 16 sequences at 150..0, bf16 ring")
    dm, ws, before, logits, am, _ = _run_batch(wl, dev)
    assert ops.atlas_device_status(ws) == 0
    for b, ref in enumerate(R.run_decode_batch(wl)):
        assert normwise(logits[b].cpu().numpy(), ref["logits"]) < TOL, b
        assert int(am[b].item()) == ref["argmax"], b


def test_batch_of_one_matches_the_single_step():
    dev = device()
    wl = _tiny_batch(0, False, batch=1, gap=0, model_id=51)
    dm, ws, _, logits, am, _ = _run_batch(wl, dev)
    ref = R.run_decode(wl)
    assert normwise(logits[0].cpu().numpy(), ref["logits"]) < TOL
    assert int(am[0].item()) == ref["argmax"]
    dm2 = build_model(wl, dev)
    lg2 = torch.empty(wl.model.vocab, dtype=torch.float32, device=dev)
    ws2 = torch.empty(ops.atlas_decode_workspace_bytes(dm2), dtype=torch.uint8, device=dev)
    ops.atlas_decode_step(dm2, torch.tensor([wl.n_cached], dtype=torch.int32, device=dev),
                          d_token=torch.tensor([ref["token"]], dtype=torch.int32, device=dev), logits=lg2, ws=ws2)
    torch.cuda.synchronize()
    assert normwise(logits[0].cpu().numpy(), lg2.cpu().numpy()) < TOL


def test_batch_full_size_swa_layer():
    """One full-size SWA layer, four sequences at 4,096 / 3,000 / 1,904 / 808 cached
    positions: each sequence's output against the oracle."""
    dev = device()
    m = W.olmo3_32b(model_id=1, n_layers=1)
    m.layer_types = [W.SWA]
    wl = W.Workload("olmo3-32b-swa-layer-batch4", m, seed=0, n_cached=4096, t_max=4097, use_tokens=True,
                    batch=4, batch_gap=1096)
    announce("batched decode, full-size SWA layer, 4 sequences")
    dm, ws, _, _, _, hid = _run_batch(wl, dev, hidden=True)
    assert ops.atlas_device_status(ws) == 0
    for b, ref in enumerate(R.run_decode_batch(wl)):
        err = normwise(hid[b].cpu().numpy(), ref["y"])
        print(f"sequence {b}: normwise {err:.2e}")
        assert err < TOL


def test_batch_full_size_4_layers_8_sequences_bf16_ring():
    """The config-10 format at full size: four layers [SWA, SWA, SWA, full] of the 32B
    shape, bf16 KV with window rings, eight sequences at 16,384 down to 5,884 cached
    positions (the int8 matrix-core projections at their largest batch, the full layer
    over 16K keys, rings wrapped). Each sequence's last hidden state against the
    oracle, and each layer's new key and value in that sequence's ring slot."""
    dev = device()
    m = W.bf16_ring_kv(W.olmo3_32b(model_id=10, n_layers=4))
    wl = W.Workload("olmo3-32b-4-layers-bf16kv-ring-batch8", m, seed=0, n_cached=16384, t_max=16385,
                    use_tokens=True, batch=8, batch_gap=1500)
    announce("batched decode, 4 full-size layers, 8 sequences, bf16 KV rings, 16K")
    dm, ws, _, _, _, hid = _run_batch(wl, dev, hidden=True)
    assert ops.atlas_device_status(ws) == 0
    refs = R.run_decode_batch(wl, keep_kv=True)
    for b, ref in enumerate(refs):
        err = normwise(hid[b].cpu().numpy(), ref["y"])
        print(f"sequence {b} at {wl.seq_cached(b)}: normwise {err:.2e}")
        assert err < TOL
        pos = wl.seq_cached(b)
        import oracle as O
        for l, L in enumerate(dm.layers):
            slot = pos % L.k_cache.shape[2] if m.layer_types[l] == W.SWA else pos
            k, v = ref["kv"][l]
            hk, hv = O.round_bf16(k.reshape(m.hkv, -1)), O.round_bf16(v.reshape(m.hkv, -1))
            assert _close_kv(L.k_cache[b][:, slot].cpu().numpy(), hk), (b, l)
            assert _close_kv(L.v_cache[b][:, slot].cpu().numpy(), hv), (b, l)


def test_batch_bad_position_sets_status_and_spares_the_cache():
    dev = device()
    wl = _tiny_batch(0, False, batch=2, gap=10, model_id=52)
    dm = build_model(wl, dev)
    toks = torch.from_numpy(W.batch_tokens(wl)).to(dev)
    pos = torch.tensor([wl.t_max, 5], dtype=torch.int32, device=dev)   # sequence 0 out of range
    before = dm.layers[0].k_cache[0].clone()
    ws = ops.atlas_decode_batch(dm, toks, pos, logits=torch.empty((2, wl.model.vocab), device=dev))
    assert ops.atlas_device_status(ws) == 1
    assert torch.equal(before, dm.layers[0].k_cache[0])
