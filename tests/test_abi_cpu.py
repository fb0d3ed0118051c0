"""The C-ABI library on the CPU: it loads without a GPU, exports every entry
point the header declares, and rejects invalid arguments before launching
anything (only calls that fail validation, or have nothing to do, are made)."""

import ctypes
import os
import re

import pytest

from online_softmax_exact_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_mi355x.h")
FAKE = ctypes.c_void_p(0x100000)  # never dereferenced: validation fails first


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return _lib.load_library()


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_poisoning_build_exports_the_same_symbols(lib):
    """The LDS-poisoning debug build (linked by build() beside the library)
    loads on the host and exports the same entry points."""
    import ctypes
    from online_softmax_exact_amd import build as B
    if not os.path.exists(B.POISON_LIB):
        import __graft_entry__
        __graft_entry__.build()
    plib = ctypes.CDLL(B.POISON_LIB)
    for n in declared_functions():
        assert hasattr(plib, n), n


def test_abi_version_and_params_layout(lib):
    assert lib.attn_abi_version() == 4
    assert lib.attn_params_sizeof() == ctypes.sizeof(_lib.Params) == 256


def test_strerror(lib):
    for code in range(-8, 1):
        assert lib.attn_strerror(code)
    assert b"unknown" in lib.attn_strerror(-99)


def good_params(**kw):
    p = _lib.Params()
    p.batch, p.heads_q, p.heads_kv, p.t_q, p.t_k, p.d_h, p.d_v = 2, 4, 2, 8, 16, 64, 64
    p.q_stride[:] = (4 * 8 * 64, 8 * 64, 64)
    p.k_stride[:] = (2 * 16 * 64, 16 * 64, 64)
    p.v_stride[:] = (2 * 16 * 64, 16 * 64, 64)
    p.o_stride[:] = (4 * 8 * 64, 8 * 64, 64)
    p.scale, p.dtype, p.causal = 0.125, _lib.ATTN_BF16, 1
    for key, val in kw.items():
        setattr(p, key, val)
    return p


def fwd(lib, p, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE):
    return lib.attn_fwd(ctypes.byref(p) if p is not None else None, q, k, v, o, lse, None, None)


@pytest.mark.parametrize("field,value,code", [
    ("dtype", 7, -3), ("heads_q", 3, -2), ("heads_kv", 0, -2), ("batch", -1, -2),
    ("t_q", -5, -2), ("t_k", -1, -2), ("d_h", 0, -4), ("d_h", 257, -4), ("d_v", 300, -4),
    ("causal", 2, -2), ("window", -1, -2), ("scale", float("nan"), -4),
    ("scale", float("inf"), -4), ("q_offset", 1 << 62, -2), ("batch", 1 << 41, -2),
])
def test_fwd_rejects(lib, field, value, code):
    assert fwd(lib, good_params(**{field: value})) == code


def test_fwd_rejects_strides_and_nulls(lib):
    p = good_params()
    p.k_stride[1] = -1
    assert fwd(lib, p) == -5
    p = good_params()
    p.bias_stride[3] = -2
    assert fwd(lib, p) == -5
    assert fwd(lib, None) == -1
    assert fwd(lib, good_params(), q=None) == -1
    assert fwd(lib, good_params(), v=None) == -1
    assert fwd(lib, good_params(), lse=None) == -1


def test_fwd_nothing_to_do(lib):
    # T_q = 0 and B = 0 are successful no-ops (nothing launched, NULLs allowed).
    assert fwd(lib, good_params(t_q=0), q=None, o=None, lse=None) == 0
    assert fwd(lib, good_params(batch=0), q=None, k=None, v=None, o=None, lse=None) == 0


def test_decode_workspace_bytes(lib):
    p = good_params(t_q=1, t_k=1000)
    rows, s, dv = 2 * 4 * 1, -(-1000 // 96), 64
    o_bytes = rows * s * dv * 4
    want = (o_bytes + 255) // 256 * 256 + (rows * s * 4 + 255) // 256 * 256
    assert lib.attn_decode_workspace_bytes(ctypes.byref(p), 96) == want
    assert lib.attn_decode_workspace_bytes(ctypes.byref(p), 0) == 0
    assert lib.attn_decode_workspace_bytes(ctypes.byref(good_params(dtype=9)), 96) == 0
    huge = lib.attn_decode_workspace_bytes(ctypes.byref(p), 1 << 62)  # one split
    assert huge == (rows * dv * 4 + 255) // 256 * 256 + 256


def test_decode_rejects(lib):
    p = good_params(t_q=1, t_k=1000)
    need = lib.attn_decode_workspace_bytes(ctypes.byref(p), 128)
    call = lambda split, ws, nbytes, **kw: lib.attn_decode_splitkv(
        ctypes.byref(p), split, FAKE, FAKE, FAKE, FAKE, FAKE, ws, nbytes, None)
    assert call(0, FAKE, need) == -2
    assert call(-3, FAKE, need) == -2
    assert call(128, None, need) == -6
    assert call(128, FAKE, need - 1) == -6
    assert call(128, ctypes.c_void_p(0x100010), need) == -6  # not 256-byte aligned
    bad = good_params(t_q=1, t_k=1000, heads_q=5)
    assert lib.attn_decode_splitkv(ctypes.byref(bad), 128, FAKE, FAKE, FAKE, FAKE, FAKE,
                                   FAKE, need, None) == -2


def test_merge_rejects(lib):
    m = lambda **kw: lib.attn_merge_states(
        kw.get("rows", 4), kw.get("states", 3), kw.get("dv", 64), kw.get("o", FAKE), 192, 64,
        kw.get("l", FAKE), 3, 1, kw.get("dtype", 0), kw.get("out", FAKE), 64,
        kw.get("lo", FAKE), None)
    assert m(dtype=5) == -3
    assert m(rows=-1) == -2
    assert m(states=0) == -2
    assert m(dv=0) == -4
    assert m(dv=257) == -4
    assert m(o=None) == -1
    assert m(lo=None) == -1
    assert m(rows=0, o=None, l=None, out=None, lo=None) == 0


def test_bwd_workspace_bytes(lib):
    p = good_params()
    assert lib.attn_bwd_workspace_bytes(ctypes.byref(p)) == (2 * 4 * 8 * 4 + 255) // 256 * 256
    assert lib.attn_bwd_workspace_bytes(ctypes.byref(good_params(t_q=0))) == 256
    assert lib.attn_bwd_workspace_bytes(ctypes.byref(good_params(dtype=9))) == 0


def test_bwd_rejects(lib):
    p = good_params()
    need = lib.attn_bwd_workspace_bytes(ctypes.byref(p))
    def call(params=p, ws=FAKE, nbytes=need, **kw):
        ptr = lambda name: kw.get(name, FAKE)
        return lib.attn_bwd(ctypes.byref(params) if params is not None else None, ptr("q"), ptr("k"),
                            ptr("v"), ptr("o"), ptr("lse"), ptr("d_o"), ptr("d_q"), ptr("d_k"),
                            ptr("d_v"), ws, nbytes, None)
    assert call(params=None) == -1
    assert call(params=good_params(heads_q=3)) == -2
    assert call(params=good_params(window=-2)) == -2
    assert call(params=good_params(dtype=4)) == -3
    assert call(params=good_params(d_v=0)) == -4
    for name in ("q", "k", "v", "o", "lse", "d_o", "d_q", "d_k", "d_v"):
        assert call(**{name: None}) == -1, name
    assert call(ws=None) == -6
    assert call(nbytes=need - 1) == -6
    assert call(ws=ctypes.c_void_p(0x100010)) == -6
    # Nothing to do: no rows and no keys.
    assert call(params=good_params(batch=0), q=None, k=None, v=None, o=None, lse=None, d_o=None,
                d_q=None, d_k=None, d_v=None, ws=None, nbytes=0) == 0


def packed_params(**kw):
    """One packed batch: 3 sequences in T_q = 8 rows and T_k = 16 keys."""
    base = dict(batch=1, cu_seqlens_q=0x200000, cu_seqlens_k=0x300000, n_seqs=3, max_seqlen_q=4)
    base.update(kw)
    return good_params(**base)


def test_varlen_rejects(lib):
    # Packed sequences: key offsets required, batch 1, no per-batch lengths,
    # sizes that fit the int32 offsets, n_seqs and max_seqlen_q >= 0.
    assert fwd(lib, packed_params(cu_seqlens_k=None)) == -1
    assert fwd(lib, packed_params(batch=2)) == -2
    assert fwd(lib, packed_params(seqlens_k=0x400000)) == -2
    assert fwd(lib, packed_params(n_seqs=-1)) == -2
    assert fwd(lib, packed_params(max_seqlen_q=-1)) == -2
    assert fwd(lib, packed_params(t_k=1 << 31)) == -2
    # Key offsets without row offsets are ambiguous.
    assert fwd(lib, good_params(cu_seqlens_k=0x300000)) == -2
    # Per-batch lengths are int32.
    assert fwd(lib, good_params(seqlens_k=0x400000, t_k=1 << 31)) == -2
    # No sequences: nothing to do (device arrays are never read on the host).
    assert fwd(lib, packed_params(n_seqs=0)) == 0


def test_varlen_unsupported_entry_points(lib):
    # Split-KV decode takes per-batch lengths but not packed sequences (the
    # backward takes both; with no rows and no keys it has nothing to do).
    p = packed_params()
    need = lib.attn_decode_workspace_bytes(ctypes.byref(p), 4)
    assert lib.attn_decode_splitkv(ctypes.byref(p), 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need,
                                   None) == -4
    params = good_params(seqlens_k=0x400000, batch=0)
    assert lib.attn_bwd(ctypes.byref(params), None, None, None, None, None, None, None, None,
                        None, None, 0, None) == 0
    assert lib.attn_bwd(ctypes.byref(packed_params(seqlens_k=0x400000)), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                        FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == -2   # not with packed sequences


def test_packed_backward_host_checks(lib):
    # Packed sequences reach the backward's kernels only through the same
    # checks as attn_fwd; no sequence is a successful call that launches
    # nothing (no GPU is touched here).
    params = packed_params(n_seqs=0)
    need = lib.attn_bwd_workspace_bytes(ctypes.byref(params))
    assert lib.attn_bwd(ctypes.byref(params), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                        FAKE, FAKE, need, None) == 0
    for bad, code in ((packed_params(cu_seqlens_k=None), -1), (packed_params(batch=2), -2),
                      (packed_params(seqlens_k=0x400000), -2), (packed_params(n_seqs=-1), -2)):
        assert lib.attn_bwd(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                            FAKE, FAKE, need, None) == code


def test_binding_varlen_arguments():
    # The binding checks the offset vectors before anything reaches the library.
    import torch
    q = torch.zeros(1, 2, 10, 64)
    kv = torch.zeros(1, 2, 12, 64)
    cu = torch.tensor([0, 4, 10], dtype=torch.int32)
    cuk = torch.tensor([0, 5, 12], dtype=torch.int32)
    p = _lib.make_params(q, kv, kv, q, scale=None, causal=True, q_offset=0, bias=None,
                         cu_seqlens_q=cu, cu_seqlens_k=cuk, max_seqlen_q=6)
    assert (p.n_seqs, p.max_seqlen_q) == (2, 6)
    assert p.cu_seqlens_q == cu.data_ptr() and p.cu_seqlens_k == cuk.data_ptr()
    assert _lib.make_params(q, kv, kv, q, scale=None, causal=True, q_offset=0, bias=None,
                            cu_seqlens_q=cu, cu_seqlens_k=cuk).max_seqlen_q == 10
    with pytest.raises(ValueError):
        _lib.make_params(q, kv, kv, q, scale=None, causal=True, q_offset=0, bias=None,
                         cu_seqlens_q=cu, cu_seqlens_k=cuk[:2])
    with pytest.raises(ValueError):
        _lib.make_params(q, kv, kv, q, scale=None, causal=True, q_offset=0, bias=None,
                         cu_seqlens_q=cu.long(), cu_seqlens_k=cuk)
    with pytest.raises(ValueError):
        _lib.make_params(q, kv, kv, q, scale=None, causal=True, q_offset=0, bias=None,
                         cu_seqlens_q=cu)
    q2 = torch.zeros(2, 2, 10, 64)
    kv2 = torch.zeros(2, 2, 12, 64)
    with pytest.raises(ValueError):
        _lib.make_params(q2, kv2, kv2, q2, scale=None, causal=True, q_offset=0, bias=None,
                         cu_seqlens_q=cu, cu_seqlens_k=cuk)
    lens = torch.tensor([3, 12], dtype=torch.int32)
    assert _lib.make_params(q2, kv2, kv2, q2, scale=None, causal=True, q_offset=0, bias=None,
                            seqlens_k=lens).seqlens_k == lens.data_ptr()
    with pytest.raises(ValueError):
        _lib.make_params(q2, kv2, kv2, q2, scale=None, causal=True, q_offset=0, bias=None,
                         seqlens_k=lens[:1])


def test_binding_rejects_bad_outputs_and_devices():
    # Caller-supplied outputs must hold every write the kernels make, and no
    # host tensor may reach a kernel: each bad argument raises before a launch.
    import torch
    q = torch.zeros(1, 2, 10, 64, dtype=torch.bfloat16)
    kv = torch.zeros(1, 2, 12, 64, dtype=torch.bfloat16)
    good_o = torch.zeros(1, 2, 10, 64, dtype=torch.bfloat16)
    good_l = torch.zeros(1, 2, 10)
    assert _lib._outputs(q, 64, good_o, good_l) == (good_o, good_l)
    for bad_o, bad_l in ((good_o.float(), None),                                    # out dtype
                         (torch.zeros(1, 2, 9, 64, dtype=torch.bfloat16), None),     # out rows
                         (torch.zeros(1, 2, 10, 32, dtype=torch.bfloat16), None),    # out d_v
                         (None, good_l.double()),                                    # lse dtype
                         (None, torch.zeros(1, 2, 9)),                               # lse shape
                         (None, torch.zeros(1, 10, 2).transpose(1, 2)),              # lse strides
                         (good_o.to("meta"), None), (None, good_l.to("meta"))):     # device
        with pytest.raises(ValueError):
            _lib._outputs(q, 64, bad_o, bad_l)
    # Operands on different devices.
    with pytest.raises(ValueError):
        _lib.make_params(q, kv.to("meta"), kv, q, scale=None, causal=True, q_offset=0, bias=None)
    # Host tensors never reach the library.
    with pytest.raises(ValueError, match="GPU tensors"):
        _lib.attn_fwd(q, kv, kv)
    with pytest.raises(ValueError, match="GPU tensors"):
        _lib.attn_decode_splitkv(q, kv, kv, split_size=4)
    with pytest.raises(ValueError, match="GPU tensors"):
        _lib.attn_bwd(q, kv, kv, good_o, good_l, good_o)
    # The merge checks its outputs' shapes and dtypes, then the device.
    st = torch.zeros(5, 3, 16)
    ls = torch.zeros(5, 3)
    for kw in (dict(out=torch.zeros(4, 16)), dict(out=torch.zeros(5, 8)),
               dict(out=torch.zeros(5, 16, dtype=torch.float64)),
               dict(lse_out=torch.zeros(4)), dict(lse_out=torch.zeros(5, dtype=torch.float64)),
               dict(out_dtype=torch.float16)):
        with pytest.raises(ValueError):
            _lib.attn_merge_states(st, ls, **kw)
    with pytest.raises(ValueError, match="GPU tensors"):
        _lib.attn_merge_states(st, ls)


def test_decode_noalloc_validation(lib):
    # The entry point without a workspace validates like attn_decode_splitkv
    # and rejects a problem whose workspace exceeds its fixed array before it
    # touches the device.
    p = good_params(t_q=1, t_k=1 << 20)
    need = lib.attn_decode_workspace_bytes(ctypes.byref(p), 64)
    assert need > _lib.DECODE_SCRATCH_BYTES
    assert lib.attn_decode_splitkv_noalloc(ctypes.byref(p), 64, FAKE, FAKE, FAKE, FAKE, FAKE,
                                           None) == -8
    assert b"no-allocation" in lib.attn_strerror(-8)
    p = good_params()
    assert lib.attn_decode_splitkv_noalloc(ctypes.byref(p), 0, FAKE, FAKE, FAKE, FAKE, FAKE,
                                           None) == -2
    assert lib.attn_decode_splitkv_noalloc(None, 4, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -1
    assert lib.attn_decode_splitkv_noalloc(ctypes.byref(p), 4, None, FAKE, FAKE, FAKE, FAKE,
                                           None) == -1
    bad = good_params(heads_q=3)
    assert lib.attn_decode_splitkv_noalloc(ctypes.byref(bad), 4, FAKE, FAKE, FAKE, FAKE, FAKE,
                                           None) == -2
    # Nothing to do: no rows.
    empty = good_params(t_q=0)
    assert lib.attn_decode_splitkv_noalloc(ctypes.byref(empty), 4, None, None, None, None, None,
                                           None) == 0


def test_probe_library_exports_its_header():
    from online_softmax_exact_amd import _probes
    header = os.path.join(ROOT, "include", "attn_probes.h")
    text = re.sub(r"/\*.*?\*/", "", open(header, encoding="utf-8").read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(attn_probe_[a-z_0-9]+)\s*\(", text)))
    assert set(names) == set(_probes.EXPORTED)
    if not os.path.exists(_probes.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    plib = _probes.load_library()
    for n in names:
        assert hasattr(plib, n), n
    # Invalid arguments are rejected before any launch (no GPU needed).
    assert plib.attn_probe_exp(None, 1, 1, None) == -2
    assert plib.attn_probe_mfma(ctypes.c_void_p(0x100000), 0, 1, None) == -2
    assert plib.attn_probe_lds_read(None, 1, 1, 0, None) == -2
    assert plib.attn_probe_stream_read(ctypes.c_void_p(0x100001), 64, ctypes.c_void_p(0x100000), 1, None) == -2
