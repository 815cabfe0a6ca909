"""The entry points under HIP graph capture: a captured decode step (append the
new token's composed row, then the cross layers' split-K decodes with the fused
merge) replays to the same bits as the eager calls, replay after replay, with
other eager work and synchronisations in between. The fused merge resets its
ticket counters on the device, so no memset node is needed between replays."""
import numpy as np
import pytest
import torch

import cross_layer_shared_amd as Y
from synthetic import inputs as S
from tests.gpu_util import dev

pytestmark = pytest.mark.gpu


def test_captured_decode_step_replays_bitwise():
    w = S.Workload("graph", 140, B=4, T=2048, Hq=16, Hkv=4, D=128, dtype="bf16", layers=4)
    k, v = S.cache_kv(w)
    kc, vc = dev(k), dev(v)
    qs = [dev(S.queries(w, layer=l)) for l in range(w.layers)]
    src = {n: dev(x) for n, x in S.compose_sources(w, layer=3, n=1).items()}      # [B, 1, Hkv, D]
    new = {n: x[:, 0] for n, x in src.items()}                                    # [B, Hkv, D] views
    alpha = S.alphas(w.seed, 3)
    splits = Y.yoco_decode_num_splits(w.B, w.T, w.Hq, w.Hkv, w.D)
    assert splits > 1
    ws = Y.decode_workspace(w.B, w.T, w.Hq, w.Hkv, w.D, splits)
    out = torch.empty((w.layers + 1, w.B, w.Hq, w.D), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.layers + 1, w.B, w.Hq), dtype=torch.float32, device="cuda")
    # the self-decoder's own cache for the fused append (separate from the shared cache)
    ks, vs = dev(k), dev(v)
    ks0, vs0 = ks.clone(), vs.clone()
    stream = torch.cuda.Stream()

    def step():
        Y.yoco_compose_kv(src["k1"], src["ki"], src["v1"], src["vi"], kc, vc, w.T - 1, alpha, stream=stream)
        for l in range(w.layers):
            Y.yoco_cross_attn_decode(qs[l], kc, vc, out[l], lse[l], workspace=ws, num_splits=splits, stream=stream)
        Y.yoco_self_attn_decode(qs[0], new["k1"], new["ki"], new["v1"], new["vi"], ks, vs, alpha, out[w.layers],
                                lse[w.layers], workspace=ws, num_splits=splits, stream=stream)

    with torch.cuda.stream(stream):
        step()
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()
    ref_ks, ref_vs = ks.clone(), vs.clone()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step()
    torch.cuda.synchronize()
    for i in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        ks.copy_(ks0)
        vs.copy_(vs0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"replay {i}"
        assert torch.equal(ks, ref_ks) and torch.equal(vs, ref_vs), f"replay {i}"
        # eager work between replays on the same workspace
        Y.yoco_cross_attn_decode(qs[1], kc, vc, out[0], workspace=ws, num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(out[0], ref_o[1])
    assert np.isfinite(ref_o.cpu().numpy()).all()
