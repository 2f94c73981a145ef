"""The no-allocation decode step (atlas_decode_step_noalloc, GPU) against the step
with a caller workspace (atlas_decode_step) on the same inputs: two calls in a row
through the C ABI, the second with a smaller model and context (a smaller
workspace), each compared with its own workspace-taking call. The two share their
kernels, so logits, argmax, hidden state and the KV slot written must agree bit for
bit, and the status word reported by the no-allocation call must be ATLAS_OK."""
import pytest
import torch

from oracle import runner as R
from synth import workloads as W
from synth.device import build_model
from swa_attention_amd import ops
from gpu_util import TOL, announce, device, normwise

pytestmark = pytest.mark.gpu


def _stack(n_layers, vocab, n_cached, t_max, model_id):
    m = W.tiny(model_id)
    m.n_layers = n_layers
    m.layer_types = [W.FULL if l % 4 == 3 else W.SWA for l in range(n_layers)]
    m.vocab = vocab
    return W.Workload("tiny-stack", m, seed=0, n_cached=n_cached, t_max=t_max, use_tokens=True, final_head=True)


def _compare(wl, dev):
    m = wl.model
    tok = torch.tensor([R.decode_token(wl)], dtype=torch.int32, device=dev)
    pos = torch.tensor([wl.n_cached], dtype=torch.int32, device=dev)
    outs = []
    need = 0
    for noalloc in (False, True):
        dm = build_model(wl, dev)            # fresh caches for each call
        need = ops.atlas_decode_workspace_bytes(dm)
        logits = torch.full((m.vocab,), float("nan"), dtype=torch.float32, device=dev)
        hidden = torch.full((m.d,), float("nan"), dtype=torch.float32, device=dev)
        am = torch.full((1,), -1, dtype=torch.int32, device=dev)
        if noalloc:
            status = torch.full((1,), -1, dtype=torch.int32, device=dev)
            ops.atlas_decode_step_noalloc(dm, pos, d_token=tok, hidden_out=hidden, logits=logits, argmax=am,
                                          status_out=status)
            torch.cuda.synchronize()
            assert int(status.item()) == 0
        else:
            ws = torch.empty(ops.atlas_decode_workspace_bytes(dm), dtype=torch.uint8, device=dev)
            ops.atlas_decode_step(dm, pos, d_token=tok, hidden_out=hidden, logits=logits, argmax=am, ws=ws)
            torch.cuda.synchronize()
            assert ops.atlas_device_status(ws) == 0
        kv = [L.k_cache[:, wl.n_cached].cpu() for L in dm.layers]
        outs.append((logits.cpu(), hidden.cpu(), int(am.item()), kv))
        del dm
    (l0, h0, a0, k0), (l1, h1, a1, k1) = outs
    assert normwise(l1.numpy(), l0.numpy()) < TOL and a1 == a0
    assert torch.equal(l0, l1) and torch.equal(h0, h1)
    for x, y in zip(k0, k1):
        assert torch.equal(x, y)
    return a0, need


def test_noalloc_step_matches_workspace_step_twice():
    dev = device()
    big = _stack(n_layers=4, vocab=5000, n_cached=200, t_max=256, model_id=7)
    small = _stack(n_layers=1, vocab=700, n_cached=30, t_max=40, model_id=8)
    announce("no-allocation decode step: 4-layer stack (vocab 5,000, 200 cached), then 1 layer (vocab 700)")
    a_big, need_big = _compare(big, dev)
    a_small, need_small = _compare(small, dev)
    assert need_small < need_big <= 4 << 20     # the second call uses less of the scratch area
    print(f"argmax {a_big}, {a_small}; workspace {need_big} then {need_small} bytes")
