"""Decode-step and prefill parity of the HIP path against the CPU oracle (GPU).

Bar: normwise ||gpu - oracle||_inf / ||oracle||_inf <= 1e-3 on f32 hidden states and
logits, identical greedy argmax, bit-identical KV slot placement (the new key and
value land in slot pos and nowhere else)."""
import numpy as np
import pytest
import torch

import oracle as O
from oracle import runner as R
from synth import workloads as W
from synth.device import build_model
from swa_attention_amd import ops
from gpu_util import TOL, announce, device, normwise

pytestmark = pytest.mark.gpu


def _ws(dm, dev):
    return torch.empty(ops.atlas_decode_workspace_bytes(dm), dtype=torch.uint8, device=dev)


def _run_layer_case(wl, dev):
    m = wl.model
    dm = build_model(wl, dev, head=False)
    x = torch.from_numpy(W.x_in(m, wl.seed)).to(dev)
    out = torch.empty(m.d, dtype=torch.float32, device=dev)
    pos = torch.tensor([wl.n_cached], dtype=torch.int32, device=dev)
    ws = _ws(dm, dev)
    k_before = dm.layers[0].k_cache.clone()
    ops.atlas_decode_step(dm, pos, hidden_in=x, hidden_out=out, ws=ws)
    torch.cuda.synchronize()
    assert ops.atlas_device_status(ws) == 0
    tr = {}
    y, Kc, Vc = R.run_layer(wl, 0, trace=tr)
    p = wl.n_cached
    gk = dm.layers[0].k_cache.cpu().numpy()
    gv = dm.layers[0].v_cache.cpu().numpy()
    # only slot p changed, and it holds the rotated k / raw v
    kb = k_before.cpu().numpy()
    changed = np.nonzero(np.any(gk != kb, axis=(0, 2)))[0]
    assert list(changed) == [p]
    assert normwise(gk[:, p], Kc[:, p]) < 1e-5
    assert normwise(gv[:, p], Vc[:, p]) < 1e-5
    return normwise(out.cpu().numpy(), y)


def test_decode_step_tiny_layer():
    dev = device()
    announce("decode tiny layer (d 640, 5/1 heads, window 64, 256 cached)")
    err = _run_layer_case(W.config(0), dev)
    assert err < TOL, err


def test_decode_step_swa_layer_full_size():
    dev = device()
    announce("decode OLMo-3-32B SWA layer, 4,096 cached")
    err = _run_layer_case(W.config(1), dev)
    print("normwise", err)
    assert err < TOL, err


def test_decode_step_full_layer_yarn_full_size():
    dev = device()
    announce("decode OLMo-3-32B full layer with YaRN, 16,384 cached")
    err = _run_layer_case(W.config(2), dev)
    print("normwise", err)
    assert err < TOL, err


def _tiny_stack(n_layers=4, vocab=1000, n_cached=80, t_max=128, window=64, model_id=7, card=False):
    m = W.card_format(W.tiny(model_id)) if card else W.tiny(model_id)
    m.n_layers = n_layers
    m.layer_types = [W.FULL if l % 4 == 3 else W.SWA for l in range(n_layers)]
    m.vocab = vocab
    m.window = window
    return W.Workload("tiny-stack", m, seed=0, n_cached=n_cached, t_max=t_max, use_tokens=True, final_head=True)


def test_decode_step_tiny_stack_with_head():
    dev = device()
    wl = _tiny_stack()
    announce("decode tiny 4-layer stack + lm_head + argmax")
    dm = build_model(wl, dev)
    tok = R.decode_token(wl)
    d_tok = torch.tensor([tok], dtype=torch.int32, device=dev)
    pos = torch.tensor([wl.n_cached], dtype=torch.int32, device=dev)
    logits = torch.empty(wl.model.vocab, dtype=torch.float32, device=dev)
    am = torch.empty(1, dtype=torch.int32, device=dev)
    hid = torch.empty(wl.model.d, dtype=torch.float32, device=dev)
    ws = _ws(dm, dev)
    ops.atlas_decode_step(dm, pos, d_token=d_tok, hidden_out=hid, logits=logits, argmax=am, ws=ws)
    ref = R.run_decode(wl)
    assert normwise(hid.cpu().numpy(), ref["y"]) < TOL
    assert normwise(logits.cpu().numpy(), ref["logits"]) < TOL
    assert int(am.item()) == ref["argmax"]


def test_decode_steps_replay_from_a_hip_graph():
    """One decode step (positions and token in device memory) captured into a HIP graph
    replays a token-by-token decode: three replays, with eager work and synchronisation
    between them, give bit-for-bit the logits, argmax and KV slots of three eager steps
    (the step is deterministic: no atomics, fixed reduction orders)."""
    dev = device()
    wl = _tiny_stack()
    announce("decode tiny 4-layer stack: eager steps vs HIP graph replays")
    dm = build_model(wl, dev)
    m = wl.model
    tok = torch.tensor([R.decode_token(wl)], dtype=torch.int32, device=dev)
    pos = torch.tensor([wl.n_cached], dtype=torch.int32, device=dev)
    logits = torch.empty(m.vocab, dtype=torch.float32, device=dev)
    ws = _ws(dm, dev)
    cm = dm.c()
    caches = [(L.k_cache.clone(), L.v_cache.clone()) for L in dm.layers]
    tok0, pos0 = tok.clone(), pos.clone()

    def step():
        ops.atlas_decode_step(dm, pos, d_token=tok, logits=logits, argmax=tok, ws=ws, cm=cm)
        pos.add_(1)

    def restore():
        for L, (k, v) in zip(dm.layers, caches):
            L.k_cache.copy_(k)
            L.v_cache.copy_(v)
        tok.copy_(tok0)
        pos.copy_(pos0)

    eager = []
    for _ in range(3):
        step()
        eager.append((logits.clone(), tok.clone()))
    kv_eager = [L.k_cache[:, wl.n_cached:wl.n_cached + 3].clone() for L in dm.layers]
    torch.cuda.synchronize()

    restore()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                  # warm-up on the capture stream's pool
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    restore()
    torch.cuda.synchronize()
    for i in range(3):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(logits, eager[i][0]), f"replay {i}: logits"
        assert torch.equal(tok, eager[i][1]), f"replay {i}: argmax"
        assert int(pos.item()) == wl.n_cached + i + 1
    for L, k in zip(dm.layers, kv_eager):
        assert torch.equal(L.k_cache[:, wl.n_cached:wl.n_cached + 3], k)
    assert ops.atlas_device_status(ws) == 0


def test_card_format_swa_layer_full_size():
    """The card's own W4 recipe (symmetric codes, group 32, bf16 scales, no zero table) on
    a full-size SWA layer at 4,096 cached keys, against the oracle."""
    dev = device()
    announce("decode OLMo-3-32B SWA layer in the card's W4 recipe (symmetric, group 32, bf16 scales)")
    err = _run_layer_case(W.config(6), dev)
    print("normwise", err)
    assert err < TOL, err


def test_card_format_tiny_stack_decode_and_prefill():
    """The card's W4 recipe through a tiny 4-layer stack with the head: one decode step
    and a 40-token prefill (group-32 GEMM path), both against the oracle."""
    dev = device()
    announce("card W4 recipe: tiny 4-layer stack, decode + 40-token prefill")
    wl = _tiny_stack(model_id=9, card=True)
    dm = build_model(wl, dev)
    d_tok = torch.tensor([R.decode_token(wl)], dtype=torch.int32, device=dev)
    pos = torch.tensor([wl.n_cached], dtype=torch.int32, device=dev)
    logits = torch.empty(wl.model.vocab, dtype=torch.float32, device=dev)
    am = torch.empty(1, dtype=torch.int32, device=dev)
    ops.atlas_decode_step(dm, pos, d_token=d_tok, logits=logits, argmax=am, ws=_ws(dm, dev))
    ref = R.run_decode(wl)
    assert normwise(logits.cpu().numpy(), ref["logits"]) < TOL
    assert int(am.item()) == ref["argmax"]
    _prefill_vs_oracle(_tiny_stack(model_id=9, card=True, n_cached=0, t_max=64), 40, dev)


def test_bad_position_sets_status_and_leaves_cache():
    dev = device()
    wl = _tiny_stack(n_layers=1)
    dm = build_model(wl, dev)
    pos = torch.tensor([wl.t_max], dtype=torch.int32, device=dev)     # one past the end
    x = torch.zeros(wl.model.d, dtype=torch.float32, device=dev)
    ws = _ws(dm, dev)
    before = dm.layers[0].k_cache.clone()
    ops.atlas_decode_step(dm, pos, hidden_in=x, ws=ws)
    assert ops.atlas_device_status(ws) == 1
    assert torch.equal(before, dm.layers[0].k_cache)
    pos.fill_(5)
    ops.atlas_decode_step(dm, pos, hidden_in=x, ws=ws)
    assert ops.atlas_device_status(ws) == 0


def test_prefill_equals_teacher_forced_decode_and_oracle():
    dev = device()
    wl = _tiny_stack(n_cached=0, t_max=64)
    announce("prefill tiny 4-layer stack, 12 tokens")
    toks = W.prompt_tokens(wl.model, wl.seed, 12, stream=1)
    dm = build_model(wl, dev)
    d_toks = torch.from_numpy(toks).to(dev)
    logits = torch.empty(wl.model.vocab, dtype=torch.float32, device=dev)
    am = torch.empty(1, dtype=torch.int32, device=dev)
    ws = torch.empty(ops.atlas_prefill_workspace_bytes(dm, len(toks)), dtype=torch.uint8, device=dev)
    ops.atlas_prefill(dm, d_toks, 0, logits, am, ws)
    ref = R.run_prefill(wl, toks)
    n = len(toks)
    for l in range(wl.model.n_layers):
        assert normwise(dm.layers[l].k_cache[:, :n].cpu().numpy(), ref["K"][l][:, :n]) < TOL
        assert normwise(dm.layers[l].v_cache[:, :n].cpu().numpy(), ref["V"][l][:, :n]) < TOL
        assert torch.count_nonzero(dm.layers[l].k_cache[:, n:]).item() == 0
    assert normwise(logits.cpu().numpy(), ref["logits"]) < TOL
    assert int(am.item()) == ref["argmax"]
    # teacher-forced GPU decode on a fresh copy of the model
    dm2 = build_model(wl, dev)
    ws2 = _ws(dm2, dev)
    lg2 = torch.empty_like(logits)
    for t in range(n):
        ops.atlas_decode_step(dm2, torch.tensor([t], dtype=torch.int32, device=dev),
                              d_token=d_toks[t:t + 1], logits=lg2 if t == n - 1 else None, ws=ws2)
    assert normwise(logits.cpu().numpy(), lg2.cpu().numpy()) < TOL
    for l in range(wl.model.n_layers):
        assert normwise(dm.layers[l].k_cache.cpu().numpy(), dm2.layers[l].k_cache.cpu().numpy()) < TOL


def _prefill_vs_oracle(wl, n_tokens, dev):
    toks = W.prompt_tokens(wl.model, wl.seed, n_tokens, stream=1)
    dm = build_model(wl, dev)
    d_toks = torch.from_numpy(toks).to(dev)
    logits = torch.empty(wl.model.vocab, dtype=torch.float32, device=dev)
    am = torch.empty(1, dtype=torch.int32, device=dev)
    ws = torch.empty(ops.atlas_prefill_workspace_bytes(dm, len(toks)), dtype=torch.uint8, device=dev)
    ops.atlas_prefill(dm, d_toks, wl.n_cached, logits, am, ws)
    torch.cuda.synchronize()
    assert ops.atlas_device_status(ws) == 0
    ref = R.run_prefill(wl, toks)
    p0, p1 = wl.n_cached, wl.n_cached + n_tokens
    for l in range(wl.model.n_layers):
        gk, gv = dm.layers[l].k_cache.cpu().numpy(), dm.layers[l].v_cache.cpu().numpy()
        assert normwise(gk[:, p0:p1], ref["K"][l][:, p0:p1]) < TOL, l
        assert normwise(gv[:, p0:p1], ref["V"][l][:, p0:p1]) < TOL, l
        np.testing.assert_array_equal(gk[:, :p0], ref["K"][l][:, :p0])   # earlier slots untouched
        assert not np.any(gk[:, p1:])                                     # later slots untouched
    assert normwise(logits.cpu().numpy(), ref["logits"]) < TOL
    assert int(am.item()) == ref["argmax"]


def test_prefill_long_prompt_crosses_the_window():
    """100 tokens through the tiny 4-layer stack (window 64): the sliding window cuts
    into the prompt itself, and the positions span seven 16-token attention tiles with
    a ragged last one."""
    dev = device()
    announce("prefill tiny stack, 100 tokens, window 64")
    _prefill_vs_oracle(_tiny_stack(n_cached=0, t_max=160), 100, dev)


def test_prefill_continues_a_filled_cache():
    """A prompt of 37 tokens after 50 cached positions (start_pos = 50): attention
    reads the earlier cache, the window reaches back into it, and only slots 50..86
    are written."""
    dev = device()
    announce("prefill tiny stack, 37 tokens after 50 cached")
    _prefill_vs_oracle(_tiny_stack(n_cached=50, t_max=128), 37, dev)


@pytest.mark.parametrize("n_tokens,n_cached,fmt", [(40, 20, "g128"), (1, 0, "g128"), (1, 30, "g128"),
                                                   (17, 5, "g128"), (40, 20, "card"), (17, 5, "card"),
                                                   (23, 9, "g64"), (23, 9, "g256"), (40, 20, "g512"),
                                                   (17, 5, "g256-sym-bf16")])
def test_prefill_split_k_shapes_match_oracle(n_tokens, n_cached, fmt):
    """A 2-layer stack with d = 1,024 (8 q / 2 KV heads) and dff = 2,048: half of the qkv,
    o and down GEMMs' K is whole 128-column groups, so the prefill splits their K in two
    (the rotary kernel, the residual kernel and the head add the halves). With groups of
    128 this runs the int8 kernel; in the card's recipe (symmetric, group 32, bf16
    scales) and with groups of 64 it runs the bf16 kernel's split path. Against the
    oracle: 40 positions after 20 cached; a one-token prompt on an empty and on a filled
    cache (one GEMM row); 17 positions, one past a 16-row tile; 23 after 9. Groups of 256
    and 512 (asymmetric f16 scales, and symmetric codes with bf16 scales) run the int8
    kernel with groups spanning several 128-column k tiles."""
    dev = device()
    m = W.Model(d=1024, hq=8, hkv=2, hd=128, dff=2048, n_layers=2, layer_types=[W.SWA, W.FULL], window=64,
                model_id=61)
    if fmt == "card":
        W.card_format(m)
    elif fmt == "g64":
        m.group = 64
    elif fmt == "g256":
        m.group = 256
    elif fmt == "g512":
        m.group = 512
    elif fmt == "g256-sym-bf16":
        m.group, m.scale_dtype, m.symmetric = 256, 1, True
    m.vocab = 1000
    wl = W.Workload("tiny-split-k", m, seed=0, n_cached=n_cached, t_max=96, use_tokens=True, final_head=True)
    announce(f"prefill 2-layer d=1024 stack ({fmt}), {n_tokens} tokens after {n_cached} cached (split-K GEMMs)")
    _prefill_vs_oracle(wl, n_tokens, dev)


def test_prefill_bad_token_sets_status():
    dev = device()
    wl = _tiny_stack(n_cached=0, t_max=64)
    announce("prefill with an out-of-range token id")
    dm = build_model(wl, dev)
    toks = W.prompt_tokens(wl.model, wl.seed, 8, stream=1)
    toks[3] = wl.model.vocab + 5
    d_toks = torch.from_numpy(toks).to(dev)
    am = torch.empty(1, dtype=torch.int32, device=dev)
    ws = torch.empty(ops.atlas_prefill_workspace_bytes(dm, len(toks)), dtype=torch.uint8, device=dev)
    ops.atlas_prefill(dm, d_toks, 0, None, am, ws)
    torch.cuda.synchronize()
    assert ops.atlas_device_status(ws) == 1


@pytest.mark.parametrize("rows", [(4800, 37), (26, 25), (4999, 1000, 999)])
def test_argmax_ties_take_the_lowest_index(rows):
    """Equal rows of the lm_head give bit-identical logits (same bits, same arithmetic).
    Copies of twice the winning row are planted at rows far apart (handled by
    different head blocks), at neighbouring rows (different waves of one block) and at
    three rows; every copy then ties for the maximum, and the argmax must be the
    lowest planted index (lowest index wins on ties)."""
    dev = device()
    wl = _tiny_stack(n_layers=1, vocab=5000)
    announce(f"argmax ties at rows {rows}")
    dm = build_model(wl, dev)
    d_tok = torch.tensor([R.decode_token(wl)], dtype=torch.int32, device=dev)
    pos = torch.tensor([wl.n_cached], dtype=torch.int32, device=dev)
    logits = torch.empty(wl.model.vocab, dtype=torch.float32, device=dev)
    am = torch.empty(1, dtype=torch.int32, device=dev)
    ws = _ws(dm, dev)
    base_pos = pos.clone()
    ops.atlas_decode_step(dm, pos, d_token=d_tok, logits=logits, argmax=am, ws=ws)
    torch.cuda.synchronize()
    win = int(am.item())
    assert float(logits[win].item()) > 0.0
    row2 = (dm.lm_head[win].view(torch.bfloat16).float() * 2.0).to(torch.bfloat16).view(torch.int16)
    assert torch.equal(row2.view(torch.bfloat16).float(), dm.lm_head[win].view(torch.bfloat16).float() * 2.0)
    for r in rows:
        dm.lm_head[r].copy_(row2)
    pos.copy_(base_pos)
    ops.atlas_decode_step(dm, pos, d_token=d_tok, logits=logits, argmax=am, ws=ws)
    torch.cuda.synchronize()
    assert ops.atlas_device_status(ws) == 0
    lg = logits.cpu()
    vals = [lg[r].item() for r in rows]
    assert all(v == vals[0] for v in vals), vals
    assert vals[0] == lg.max().item()
    assert int(am.item()) == min(rows)
