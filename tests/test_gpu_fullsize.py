"""Parity at the full sizes the benchmark times (GPU).

- The 64-layer decode step at 16,384 cached positions (the bench workload, same
  launch configuration) against the oracle: logits normwise within 1e-3, identical
  greedy argmax (the oracle's top-1/top-2 margin is printed), last hidden state.
- The 1,200-token prefill on the matrix cores against 1,200 teacher-forced decode
  steps of the GPU decode path (prefill's definition), at full size: the decode path
  is itself checked against the oracle above, and the oracle is too slow for 1,200
  positions of 64 layers. Logits, argmax and sampled KV slots are compared.
"""
import numpy as np
import pytest
import torch

from oracle import runner as R
from synth import workloads as W
from synth.device import build_model
from swa_attention_amd import ops
from gpu_util import TOL, announce, device, normwise

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def olmo3_model():
    dev = device()
    wl = W.config(3)
    announce("building the 64-layer OLMo-3-32B-shaped W4 model (16,385 KV slots per layer)")
    dm = build_model(wl, dev)
    torch.cuda.synchronize()
    yield wl, dm
    del dm
    torch.cuda.empty_cache()


def test_decode_64_layers_16k_matches_oracle(olmo3_model):
    wl, dm = olmo3_model
    dev = device()
    m = wl.model
    announce("decode step, 64 layers at 16,384 cached + lm_head vs oracle")
    tok = R.decode_token(wl)
    d_tok = torch.tensor([tok], dtype=torch.int32, device=dev)
    pos = torch.tensor([wl.n_cached], dtype=torch.int32, device=dev)
    logits = torch.empty(m.vocab, dtype=torch.float32, device=dev)
    hidden = torch.empty(m.d, dtype=torch.float32, device=dev)
    am = torch.empty(1, dtype=torch.int32, device=dev)
    ws = torch.empty(ops.atlas_decode_workspace_bytes(dm), dtype=torch.uint8, device=dev)
    ops.atlas_decode_step(dm, pos, d_token=d_tok, hidden_out=hidden, logits=logits, argmax=am, ws=ws)
    torch.cuda.synchronize()
    assert ops.atlas_device_status(ws) == 0
    ref = R.run_decode(wl)
    lg = logits.cpu().numpy()
    top2 = np.sort(ref["logits"])[-2:]
    err_l = normwise(lg, ref["logits"])
    err_y = normwise(hidden.cpu().numpy(), ref["y"])
    print(f"logits normwise {err_l:.2e}, hidden normwise {err_y:.2e}, oracle top1-top2 margin {top2[1] - top2[0]:.3e}, "
          f"max |logit err| {np.max(np.abs(lg - ref['logits'])):.3e}")
    assert err_y < TOL
    assert err_l < TOL
    assert int(am.item()) == ref["argmax"]
    # the new key/value went to slot 16,384 of every layer; slot 16,383 still holds the cache
    k_new = dm.layers[63].k_cache[:, wl.n_cached]
    assert torch.count_nonzero(k_new).item() > 0


@pytest.mark.parametrize("cfg", [7, 8])
def test_decode_64_layers_bf16_ring_layer_by_layer(cfg):
    """The card's planned KV format (bf16, 4,096-slot rings on the sliding-window
    layers) at 16,384 and at 65,535 cached positions (the YaRN context limit).

    With a bf16 cache the step stores rounded keys and values, and a rounding that
    goes the other way on one side (both sides round their own f32 value, which
    agree to about 1e-6) moves that element by a whole bf16 unit; later layers
    amplify it. The oracle shows the same against itself: nudging its layer-0 input
    by 1e-7 (relative, random signs) makes it differ from itself by 1.5e-4 after 32 of
    these layers and by 1.03e-3 after all 64 (logits 9.1e-4, configuration 7), while
    the f32 cache stays at 5e-7. So the 1e-3 bar tests the kernels layer by layer, at
    full size and in the step's launch configuration: GPU layer l gets the oracle's
    input to layer l, and its output is compared with the oracle's; the head gets the
    oracle's last hidden state. End to end on fresh caches, the last hidden state is
    held to 1e-2, ten times the oracle's own spread under that nudge, and the argmax
    must match whenever the oracle's top-1/top-2 margin exceeds twice the largest
    logit error (otherwise several tokens are within rounding of the maximum)."""
    import dataclasses
    dev = device()
    wl = W.config(cfg)
    m = wl.model
    announce(f"decode step, {wl.name}: 64 layers layer by layer + lm_head vs oracle")
    ref = R.run_decode(wl, keep_hidden=True)
    dm = build_model(wl, dev)
    d_tok = torch.tensor([ref["token"]], dtype=torch.int32, device=dev)
    pos = torch.tensor([wl.n_cached], dtype=torch.int32, device=dev)
    logits = torch.empty(m.vocab, dtype=torch.float32, device=dev)
    am = torch.empty(1, dtype=torch.int32, device=dev)
    out = torch.empty(m.d, dtype=torch.float32, device=dev)
    ws = torch.empty(ops.atlas_decode_workspace_bytes(dm), dtype=torch.uint8, device=dev)
    errs = []
    for l in range(m.n_layers):
        one = dataclasses.replace(dm, layers=[dm.layers[l]], _c=None, _arr=None)
        last = l == m.n_layers - 1
        x = None if l == 0 else torch.from_numpy(ref["hidden"][l - 1]).to(dev)
        ops.atlas_decode_step(one, pos, d_token=d_tok if l == 0 else None, hidden_in=x, hidden_out=out,
                              logits=logits if last else None, argmax=am if last else None, ws=ws)
        torch.cuda.synchronize()
        assert ops.atlas_device_status(ws) == 0
        errs.append(normwise(out.cpu().numpy(), ref["hidden"][l]))
    err_l = normwise(logits.cpu().numpy(), ref["logits"])
    print(f"per-layer normwise: max {max(errs):.2e} (layer {int(np.argmax(errs))}), median {np.median(errs):.2e}; "
          f"logits from the oracle's last hidden state {err_l:.2e}")
    assert max(errs) < TOL
    assert err_l < TOL
    assert int(am.item()) == ref["argmax"]
    # end to end on fresh caches: printed (the definition itself amplifies rounding order)
    del dm
    torch.cuda.empty_cache()
    dm = build_model(wl, dev)
    ops.atlas_decode_step(dm, pos, d_token=d_tok, hidden_out=out, logits=logits, argmax=am, ws=ws)
    torch.cuda.synchronize()
    assert ops.atlas_device_status(ws) == 0
    top2 = np.sort(ref["logits"])[-2:]
    margin = float(top2[1] - top2[0])
    lg = logits.cpu().numpy()
    max_err = float(np.max(np.abs(lg.astype(np.float64) - ref["logits"])))
    err_y = normwise(out.cpu().numpy(), ref["y"])
    print(f"end to end: hidden normwise {err_y:.2e}, logits {normwise(lg, ref['logits']):.2e}, "
          f"argmax {int(am.item())} vs {ref['argmax']} (oracle top1-top2 margin {margin:.3e}, "
          f"max |logit err| {max_err:.3e})")
    assert err_y < 1e-2
    if margin > 2.0 * max_err:
        assert int(am.item()) == ref["argmax"]
    else:
        print("argmax not compared: the margin is within twice the logit error")


def test_prefill_1200_matches_teacher_forced_decode(olmo3_model):
    wl, dm = olmo3_model
    dev = device()
    m = wl.model
    pw = W.config(4)
    n = pw.prompt_len
    announce(f"prefill of {n} tokens (64 layers, matrix cores) vs {n} teacher-forced GPU decode steps")
    toks = torch.from_numpy(W.prompt_tokens(m, pw.seed, n)).to(dev)
    logits_p = torch.empty(m.vocab, dtype=torch.float32, device=dev)
    am_p = torch.empty(1, dtype=torch.int32, device=dev)
    ws_p = torch.empty(ops.atlas_prefill_workspace_bytes(dm, n), dtype=torch.uint8, device=dev)
    ops.atlas_prefill(dm, toks, 0, logits_p, am_p, ws_p)
    torch.cuda.synchronize()
    assert ops.atlas_device_status(ws_p) == 0
    sample_layers = [0, 3, 62, 63]
    kv_p = {l: (dm.layers[l].k_cache[:, :n].cpu(), dm.layers[l].v_cache[:, :n].cpu()) for l in sample_layers}
    del ws_p
    # the decode path over the same positions (overwrites slots 0..n-1 with its own values)
    logits_d = torch.empty_like(logits_p)
    am_d = torch.empty(1, dtype=torch.int32, device=dev)
    ws = torch.empty(ops.atlas_decode_workspace_bytes(dm), dtype=torch.uint8, device=dev)
    cm = dm.c()
    pos = torch.arange(n, dtype=torch.int32, device=dev)
    for t in range(n):
        last = t == n - 1
        ops.atlas_decode_step(dm, pos[t:t + 1], d_token=toks[t:t + 1], logits=logits_d if last else None,
                              argmax=am_d if last else None, ws=ws, cm=cm)
    torch.cuda.synchronize()
    assert ops.atlas_device_status(ws) == 0
    err = normwise(logits_p.cpu().numpy(), logits_d.cpu().numpy())
    print(f"prefill vs decode logits normwise {err:.2e}")
    assert err < TOL
    assert int(am_p.item()) == int(am_d.item())
    for l in sample_layers:
        kp, vp = kv_p[l]
        assert normwise(kp.numpy(), dm.layers[l].k_cache[:, :n].cpu().numpy()) < TOL, l
        assert normwise(vp.numpy(), dm.layers[l].v_cache[:, :n].cpu().numpy()) < TOL, l


def test_prefill_full_width_4_layers_matches_oracle():
    """Prefill at full width against the oracle itself: 4 full-size layers
    [SWA, SWA, SWA, full] of the 32B shape, a 20-token prompt after 3 cached positions.
    At this width the GEMMs take their production paths: the int8 kernel for every
    projection, the two-way K split of qkv, o and down (down's K = 27,648), and
    gate+up's N = 55,296 with the SwiGLU epilogue; the prompt spans two 16-row
    attention tiles. Every KV slot written and the last row's logits are compared at
    the 1e-3 bar, with identical argmax."""
    dev = device()
    m = W.olmo3_32b(model_id=3, n_layers=4)
    wl = W.Workload("olmo3-32b-4-layer-prefill", m, seed=0, n_cached=3, t_max=32, use_tokens=True,
                    final_head=True)
    n = 20
    announce(f"prefill of {n} tokens after 3 cached through 4 full-size layers + lm_head vs oracle")
    toks = W.prompt_tokens(m, wl.seed, n, stream=1)
    dm = build_model(wl, dev)
    d_toks = torch.from_numpy(toks).to(dev)
    logits = torch.empty(m.vocab, dtype=torch.float32, device=dev)
    am = torch.empty(1, dtype=torch.int32, device=dev)
    ws = torch.empty(ops.atlas_prefill_workspace_bytes(dm, n), dtype=torch.uint8, device=dev)
    ops.atlas_prefill(dm, d_toks, wl.n_cached, logits, am, ws)
    torch.cuda.synchronize()
    assert ops.atlas_device_status(ws) == 0
    kv = [(L.k_cache.cpu().numpy(), L.v_cache.cpu().numpy()) for L in dm.layers]
    lg = logits.cpu().numpy()
    del dm, ws
    torch.cuda.empty_cache()
    ref = R.run_prefill(wl, toks)
    p0, p1 = wl.n_cached, wl.n_cached + n
    errs = []
    for l in range(m.n_layers):
        gk, gv = kv[l]
        errs.append(max(normwise(gk[:, p0:p1], ref["K"][l][:, p0:p1]), normwise(gv[:, p0:p1], ref["V"][l][:, p0:p1])))
        np.testing.assert_array_equal(gk[:, :p0], ref["K"][l][:, :p0])
        assert not np.any(gk[:, p1:])
    err_l = normwise(lg, ref["logits"])
    top2 = np.sort(ref["logits"])[-2:]
    print(f"KV normwise per layer {['%.2e' % e for e in errs]}, logits {err_l:.2e}, "
          f"oracle top1-top2 margin {top2[1] - top2[0]:.3e}")
    assert max(errs) < TOL
    assert err_l < TOL
    assert int(am.item()) == ref["argmax"]
