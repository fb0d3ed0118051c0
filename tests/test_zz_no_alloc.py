"""The decode entry point that allocates nothing (attn_decode_splitkv_noalloc,
for callers that cannot allocate device memory), called through the C ABI:
on two calls in a row, the second smaller and with per-batch KV lengths (so
the fixed workspace still holds the first call's partials where the second
writes none), its outputs equal attn_decode_splitkv's bit for bit on the same
problem (the same kernels), and the oracle's within the bf16 bar."""

import ctypes

import pytest
import torch

import online_softmax_exact_amd as attn
from online_softmax_exact_amd import _lib, inputs
from gpu_util import assert_close_full, ensure_built, oracle_by_group, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def noalloc(q, k, v, split, scale, q_offset, seqlens_k=None):
    """One call of the C entry point on the current stream."""
    lib = _lib.load_library()
    o = torch.empty(q.shape[:3] + (v.shape[3],), dtype=q.dtype, device=q.device)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    p = _lib.make_params(q, k, v, o, scale=scale, causal=True, q_offset=q_offset, bias=None,
                         seqlens_k=seqlens_k)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    st = lib.attn_decode_splitkv_noalloc(ctypes.byref(p), split, ptr(q), ptr(k), ptr(v), ptr(o),
                                         ptr(lse), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, _lib.strerror(st)
    return o, lse


def test_noalloc_equals_workspace_call_twice():
    # 1: the GQA decode workload (16.9 MB of partials in the 32 MiB array).
    wl = inputs.make_config(3)
    print("call 1:", wl.name, flush=True)
    q, k, v, _ = to_dev(wl)
    need = attn.attn_decode_workspace_bytes(q, k, v, split_size=wl.split_size, q_offset=wl.q_offset)
    assert 0 < need <= _lib.DECODE_SCRATCH_BYTES
    o1, l1 = noalloc(q, k, v, wl.split_size, wl.scale, wl.q_offset)
    r1, rl1, _ = attn.attn_decode_splitkv(q, k, v, split_size=wl.split_size, scale=wl.scale,
                                          causal=True, q_offset=wl.q_offset)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), r1.view(torch.int16)), "call 1: O differs"
    assert torch.equal(l1, rl1), "call 1: LSE differs"
    del q, k, v, o1, l1, r1, rl1
    # 2: a smaller problem right after, with per-batch KV lengths: batch 1's
    # cache holds 5 keys, so only its first partial is written and read.
    wl2 = inputs.make_random(2, 8, 2, 3, 3000, 128, 128, seed=77, causal=True, q_offset=0)
    print("call 2: B2 Hq8/Hkv2 Tq3 Tk3000 lengths [1700, 5] split 256", flush=True)
    q, k, v, _ = to_dev(wl2)
    lens = torch.tensor([1700, 5], dtype=torch.int32, device=q.device)
    o2, l2 = noalloc(q, k, v, 256, wl2.scale, 0, seqlens_k=lens)
    r2, rl2, _ = attn.attn_decode_splitkv(q, k, v, split_size=256, scale=wl2.scale, causal=True,
                                          q_offset=0, seqlens_k=lens)
    torch.cuda.synchronize()
    assert torch.equal(o2.view(torch.int16), r2.view(torch.int16)), "call 2: O differs"
    assert torch.equal(l2, rl2), "call 2: LSE differs"
    # And the oracle: batch b sees its first L_b keys, rows at the end of them.
    for b, n in enumerate((1700, 5)):
        sub = inputs.Workload(name="kvlens", q=wl2.q[b:b + 1], k=wl2.k[b:b + 1, :, :n],
                              v=wl2.v[b:b + 1, :, :n], scale=wl2.scale, causal=True, q_offset=n - 3)
        ro, rl, _ = oracle_by_group(sub)
        assert_close_full(o2[b:b + 1], l2[b:b + 1], ro, rl, torch.bfloat16, what=f"call 2 batch {b}")
