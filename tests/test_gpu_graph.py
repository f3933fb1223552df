"""The decode calls inside a captured HIP graph: the library only launches
kernels on the caller's stream (no allocation, no memset, no synchronization),
so a whole decode pass can be captured once and replayed.  Every replay, with
eager work and synchronizations between replays, must reproduce the eager
results bit for bit."""
import numpy as np
import pytest
import torch

import varq_inputs as vi
import visual_autoregressive_kv_amd as K
from gpu_common import DEV, fill_both, to_dev

pytestmark = pytest.mark.gpu


def _clear(tensors):
    for t in tensors:
        t.zero_()


def test_fused_decode_pass_replays(oracle):
    wl = vi.WORKLOADS["var_d20_b128_int4"].with_(batch=4)
    Lg = K.make_layout(wl.batch, wl.heads, wl.head_dim, wl.bits, wl.blocks)
    ins = [(to_dev(vi.kv_block(wl, 0, "k", j)), to_dev(vi.kv_block(wl, 0, "v", j)),
            to_dev(vi.q_block(wl, 0, j))) for j in range(len(wl.blocks))]

    def decode(kc, vc, outs):
        for j, (kb, vb, qb) in enumerate(ins):
            K.kvq_quantize_attend(Lg, j, kb, vb, qb, kc, vc, outs[j])

    def fresh():
        kc, vc = K.alloc_cache(Lg), K.alloc_cache(Lg)
        outs = [torch.zeros(tuple(q.shape), dtype=torch.float32, device=DEV) for _, _, q in ins]
        return kc, vc, outs

    kc_e, vc_e, outs_e = fresh()
    decode(kc_e, vc_e, outs_e)
    torch.cuda.synchronize()

    kc, vc, outs = fresh()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # one eager pass on the capture stream first
        decode(kc, vc, outs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        decode(kc, vc, outs)
    state = list(kc.values()) + list(vc.values()) + outs
    for rep in range(3):
        _clear(state)  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for j in range(len(ins)):
            assert torch.equal(outs[j].view(torch.int32), outs_e[j].view(torch.int32)), (rep, j)
        for a, b in ((kc, kc_e), (vc, vc_e)):
            for key in ("codes", "zero", "scale"):
                assert torch.equal(a[key], b[key]), (rep, key)


def test_key_range_attention_replays(oracle):
    wl = vi.WORKLOADS["video_16x1560_h40d128_int3"].with_(blocks=(1560, 1560))
    Lg, Lo, kg, vg, ko, vo = fill_both(oracle, wl)
    q = to_dev(vi.q_block(wl, 0, 1))
    ws = torch.empty(K.kvq_attend_split_workspace(Lg, 1, 8), dtype=torch.uint8, device=DEV)
    ref = torch.empty(tuple(q.shape), dtype=torch.float32, device=DEV)
    K.kvq_attend_packed_split(Lg, 1, q, kg, vg, ref, ws, max_splits=8)
    torch.cuda.synchronize()

    out = torch.zeros_like(ref)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        K.kvq_attend_packed_split(Lg, 1, q, kg, vg, out, ws, max_splits=8)
    for rep in range(3):
        out.zero_()
        ws.fill_(rep + 1)  # the workspace is rewritten by every replay
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), ref.view(torch.int32)), rep
    assert np.isfinite(out.cpu().numpy()).all()
