"""The entry points under HIP graph capture: every step of the path is a
kernel launch on the caller's stream (no device allocation, no memset, no
host synchronisation), so a captured prefill + split-KV decode (+ merge), and
a captured backward, replay correctly.  Each replay runs after unrelated eager work that
overwrites the inputs and is compared bit for bit with an eager call on the
same inputs."""

import pytest
import torch

import online_softmax_exact_amd as attn
from online_softmax_exact_amd import inputs
from gpu_util import dev, ensure_built

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def test_graph_replays_match_eager():
    d = dev()
    pre = inputs.make_random(1, 4, 2, 500, 500, 128, 128, seed=11, causal=True)
    dec = inputs.make_random(3, 8, 2, 1, 3000, 128, 128, seed=12, causal=True, q_offset=2999)
    pq, pk, pv = (t.to(d) for t in (pre.q, pre.k, pre.v))
    dq, dk, dv = (t.to(d) for t in (dec.q, dec.k, dec.v))
    lens = torch.tensor([3000, 17, 1500], dtype=torch.int32, device=d)
    po = torch.empty(1, 4, 500, 128, dtype=torch.bfloat16, device=d)
    pl = torch.empty(1, 4, 500, device=d)
    do = torch.empty(3, 8, 1, 128, dtype=torch.bfloat16, device=d)
    dl = torch.empty(3, 8, 1, device=d)
    ws = torch.empty(attn.attn_decode_workspace_bytes(dq, dk, dv, split_size=256), dtype=torch.uint8, device=d)

    def step(stream=None):
        attn.attn_fwd(pq, pk, pv, scale=pre.scale, causal=True, out=po, lse=pl, stream=stream)
        attn.attn_decode_splitkv(dq, dk, dv, split_size=256, scale=dec.scale, seqlens_k=lens, workspace=ws,
                                 out=do, lse=dl, stream=stream)

    s = torch.cuda.Stream(device=d)
    s.wait_stream(torch.cuda.current_stream(d))
    with torch.cuda.stream(s):
        step(s)                       # warm-up on the capture stream
    torch.cuda.current_stream(d).wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step(s)
    torch.cuda.synchronize()

    gen = torch.Generator(device="cpu")
    for rep in range(4):
        # New inputs through eager work, then the replay, then an eager
        # reference on the same inputs into separate outputs.
        gen.manual_seed(rep)
        for t in (pq, pk, pv, dq, dk, dv):
            t.copy_(torch.randn(t.shape, generator=gen).to(t.dtype))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [x.clone() for x in (po, pl, do, dl)]
        ro, rl = attn.attn_fwd(pq, pk, pv, scale=pre.scale, causal=True)
        rdo, rdl, _ = attn.attn_decode_splitkv(dq, dk, dv, split_size=256, scale=dec.scale, seqlens_k=lens)
        torch.cuda.synchronize()
        for name, a, b in zip(("o", "lse", "decode o", "decode lse"), got, (ro, rl, rdo, rdl)):
            ai = a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32)
            bi = b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)
            assert torch.equal(ai, bi), f"replay {rep}: {name} differs from the eager call"


def test_graph_backward_replays_match_eager():
    """attn_bwd (dense GQA and packed sequences) captured with its outputs and
    workspace given: the D, dQ, dV and dK launches replay bit for bit."""
    d = dev()
    wl = inputs.make_random(2, 8, 2, 300, 300, 128, 128, seed=21, causal=True)
    q, k, v = wl.q.to(d), wl.k.to(d), wl.v.to(d)
    pq, pk, pv, _, cu_q, cu_k = inputs.make_packed([100, 257, 3], [140, 257, 3], 4, 4, 64, 128, seed=22)
    pq, pk, pv, cu_q, cu_k = (t.to(d) for t in (pq, pk, pv, cu_q, cu_k))
    pkw = dict(scale=inputs.default_scale(64), causal=True, cu_seqlens_q=cu_q, cu_seqlens_k=cu_k, max_seqlen_q=257)
    o, lse = attn.attn_fwd(q, k, v, scale=wl.scale, causal=True)
    po, plse = attn.attn_fwd(pq, pk, pv, **pkw)
    g, pg = torch.empty_like(o), torch.empty_like(po)
    outs = [torch.zeros_like(t) for t in (q, k, v, pq, pk, pv)]
    ws = torch.empty(2 * 8 * 300 * 4 + 256, dtype=torch.uint8, device=d)
    pws = torch.empty(4 * 360 * 4 + 256, dtype=torch.uint8, device=d)

    def step(stream=None):
        attn.attn_bwd(q, k, v, o, lse, g, scale=wl.scale, causal=True, d_q=outs[0], d_k=outs[1], d_v=outs[2],
                      workspace=ws, stream=stream)
        attn.attn_bwd(pq, pk, pv, po, plse, pg, d_q=outs[3], d_k=outs[4], d_v=outs[5], workspace=pws,
                      stream=stream, **pkw)

    s = torch.cuda.Stream(device=d)
    s.wait_stream(torch.cuda.current_stream(d))
    with torch.cuda.stream(s):
        step(s)
    torch.cuda.current_stream(d).wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        step(s)
    torch.cuda.synchronize()
    gen = torch.Generator(device="cpu")
    for rep in range(4):
        gen.manual_seed(100 + rep)
        for t in (g, pg):
            t.copy_(torch.randn(t.shape, generator=gen).to(t.dtype))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [x.clone() for x in outs]
        ref = list(attn.attn_bwd(q, k, v, o, lse, g, scale=wl.scale, causal=True))
        ref += list(attn.attn_bwd(pq, pk, pv, po, plse, pg, **pkw))
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"replay {rep}: gradient {i} differs"
