"""Host-side checks of libgdn (no GPU): exported symbols, the chunk metadata
(bit-exact against the oracle's definition) and every validation error,
which the library raises before any HIP call."""
import ctypes
import os
import random
import re

import pytest

from chunked_gated_delta_05_amd import binding as gb
from oracle import varlen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "gdn.h")).read()
    return sorted(set(re.findall(r"^gdn_status\s+(gdn_\w+)\s*\(", src, re.M)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert names == ["gdn_chunk_bwd", "gdn_chunk_fwd", "gdn_chunk_fwd_noalloc", "gdn_split_meta",
                     "gdn_state_grad_summary", "gdn_state_merge", "gdn_state_merge_adjoint",
                     "gdn_state_merge_pieces", "gdn_state_summary", "gdn_varlen_meta"]
    L = gb.lib()
    for n in names:
        assert hasattr(L, n), n


# ------------------------------------------------------------------ varlen metadata
@pytest.mark.parametrize("lens", [[1], [63], [64], [65], [1, 1, 1], [128, 1, 64, 65, 200], [4000] * 3 + [100]])
def test_varlen_meta_matches_definition(lens):
    offs = [0]
    for x in lens:
        offs.append(offs[-1] + x)
    ci, co = gb.gdn_varlen_meta(offs, offs[-1])
    assert [tuple(r) for r in ci.tolist()] == varlen.chunk_indices(offs)
    assert co.tolist() == varlen.chunk_offsets(offs)


def test_varlen_meta_random():
    rnd = random.Random(11)
    for _ in range(200):
        lens = [rnd.randint(1, 500) for _ in range(rnd.randint(1, 30))]
        offs = [0]
        for x in lens:
            offs.append(offs[-1] + x)
        ci, co = gb.gdn_varlen_meta(offs, offs[-1])
        assert [tuple(r) for r in ci.tolist()] == varlen.chunk_indices(offs)
        assert co.tolist() == varlen.chunk_offsets(offs)


@pytest.mark.parametrize("offs,total", [([0], 0), ([1, 5], 5), ([0, 5], 6), ([0, 5, 5, 9], 9),
                                        ([0, 6, 5, 9], 9), ([0, 4.0, 9], 9), ([0, True, 9], 9)])
def test_varlen_meta_rejects(offs, total):
    assert not varlen.valid_offsets(offs, total)
    with pytest.raises(ValueError):
        gb.gdn_varlen_meta(offs, total)


def test_varlen_meta_capacity():
    offs = (ctypes.c_int32 * 3)(0, 100, 300)
    ci = (ctypes.c_int32 * 4)()
    n = ctypes.c_int32(0)
    st = gb.lib().gdn_varlen_meta(offs, 3, 300, 64, ci, 2, None, ctypes.byref(n))
    assert st == gb.GDN_ERR_CAPACITY and n.value == 6   # ceil(100/64) + ceil(200/64)


# ------------------------------------------------------------------ validation
def desc(**kw):
    d = gb.GdnDesc()
    d.B, d.T, d.H, d.K, d.V = 2, 200, 3, 128, 128
    d.layout, d.dtype, d.o_dtype, d.gate_kind, d.use_exp2 = 0, 1, 0, 0, 0
    d.chunk_size, d.scale, d.n_units = 64, 0.0883883, 0
    for k, v in kw.items():
        setattr(d, k, v)
    return d


FAKE = 1 << 20   # an aligned non-null "device" address; never dereferenced


def fwd(d, *, ws=FAKE, nbytes=None, q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, o=FAKE, flags=0):
    nb = ctypes.c_size_t(nbytes if nbytes is not None else (1 << 40))
    return gb.lib().gdn_chunk_fwd(ctypes.byref(d), q, k, v, g, beta, None, o, None, None, flags, ws,
                                  ctypes.byref(nb), None), nb.value


def test_workspace_query_sizes():
    st, nb = fwd(desc(), ws=None)
    # bf16 inputs, scalar gate: T and P as 64x64 fp16 operand tiles and a
    # 1 KiB per-row coefficient block per chunk-head; every region starts
    # 256-aligned
    nch = 2 * 4 * 3
    a256 = lambda x: ((x + 255) // 256) * 256
    expect = 2 * a256(nch * 64 * 64 * 2) + a256(nch * 1024)
    assert st == gb.GDN_OK and nb == expect
    st, nb2 = fwd(desc(gate_kind=1), ws=None)
    assert st == gb.GDN_OK and nb2 > nb


@pytest.mark.parametrize("kw,code", [
    ({"chunk_size": 32}, gb.GDN_ERR_INVALID),
    ({"K": 64, "V": 64}, gb.GDN_ERR_UNSUPPORTED),
    ({"V": 64}, gb.GDN_ERR_UNSUPPORTED),
    ({"B": 0}, gb.GDN_ERR_INVALID),
    ({"H": 0}, gb.GDN_ERR_INVALID),
    ({"T": -1}, gb.GDN_ERR_INVALID),
    ({"layout": 5}, gb.GDN_ERR_INVALID),
    ({"dtype": 7}, gb.GDN_ERR_INVALID),
    ({"o_dtype": 3}, gb.GDN_ERR_INVALID),
    ({"gate_kind": 2}, gb.GDN_ERR_INVALID),
    ({"use_exp2": 2}, gb.GDN_ERR_INVALID),
    ({"scale": float("nan")}, gb.GDN_ERR_INVALID),
    ({"layout": 1}, gb.GDN_ERR_INVALID),            # TND needs offsets and B = 1
    ({"n_units": -1}, gb.GDN_ERR_INVALID),
])
def test_descriptor_errors(kw, code):
    st, _ = fwd(desc(**kw))
    assert st == code


def _with_offsets(offs, **kw):
    arr = (ctypes.c_int32 * len(offs))(*offs)
    d = desc(n_units=len(offs) - 1, offsets_host=ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32)),
             offsets_dev=FAKE, chunk_offsets_dev=FAKE, chunk_indices_dev=FAKE, **kw)
    return d, arr


@pytest.mark.parametrize("offs,kw,code", [
    ([0, 100, 200, 400], {}, gb.GDN_OK),                          # segments of rows 0 and 1
    ([0, 100, 400], {}, gb.GDN_ERR_INVALID),                      # a unit crossing the row start 200
    ([0, 150, 400], {}, gb.GDN_ERR_INVALID),
    ([0, 100, 100, 400], {}, gb.GDN_ERR_INVALID),                 # empty unit
    ([0, 300, 200, 400], {}, gb.GDN_ERR_INVALID),                 # decreasing
    ([0, 100, 399], {}, gb.GDN_ERR_INVALID),                      # does not end at B*T
    ([5, 100, 400], {}, gb.GDN_ERR_INVALID),                      # does not start at 0
    ([0, 100, 200, 400], {"layout": 1}, gb.GDN_ERR_INVALID),      # TND with B = 2
    ([0, 7, 200], {"layout": 1, "B": 1}, gb.GDN_OK),              # TND documents
])
def test_offset_errors(offs, kw, code):
    d, arr = _with_offsets(offs, **kw)
    st, _ = fwd(d, ws=None)
    assert st == code


def test_missing_device_metadata():
    d, arr = _with_offsets([0, 7, 200], layout=1, B=1)
    d.chunk_indices_dev = None
    assert fwd(d, ws=None)[0] == gb.GDN_ERR_INVALID


def test_workspace_errors():
    st, need = fwd(desc(), ws=None)
    assert st == gb.GDN_OK
    st, nb = fwd(desc(), nbytes=need - 1)
    assert st == gb.GDN_ERR_CAPACITY and nb == need
    assert fwd(desc(), ws=FAKE + 128)[0] == gb.GDN_ERR_INVALID          # not 256-byte aligned
    nb = ctypes.c_size_t(0)
    assert gb.lib().gdn_chunk_fwd(ctypes.byref(desc()), None, None, None, None, None, None, None, None,
                                  None, 0, None, None, None) == gb.GDN_ERR_INVALID   # no size pointer
    assert gb.lib().gdn_chunk_fwd(None, None, None, None, None, None, None, None, None, None, 0, None,
                                  ctypes.byref(nb), None) == gb.GDN_ERR_INVALID   # no descriptor


@pytest.mark.parametrize("missing", ["q", "k", "v", "g", "beta", "o"])
def test_missing_tensors(missing):
    st, _ = fwd(desc(), **{missing: None})
    assert st == gb.GDN_ERR_INVALID


def test_flag_errors():
    assert fwd(desc(), flags=3)[0] == gb.GDN_ERR_INVALID
    assert fwd(desc(), flags=16)[0] == gb.GDN_ERR_INVALID
    assert fwd(desc(), flags=3 | 4)[0] == gb.GDN_ERR_INVALID


def test_summary_and_merge_errors():
    L = gb.lib()
    nb = ctypes.c_size_t(1 << 40)
    d, arr = _with_offsets([0, 100, 200, 300, 400])   # two segments per row
    def summ(mode=0, flags=0, units=None, n_sel=-1, ext=FAKE, m=FAKE):
        return L.gdn_state_summary(ctypes.byref(d), None, FAKE, FAKE, FAKE, FAKE, mode, flags, units, n_sel,
                                   ext, m, FAKE, ctypes.byref(nb), None)
    for mode in (-1, 3):
        assert summ(mode=mode) == gb.GDN_ERR_INVALID
    # mode 1 needs S_ext, mode 2 needs M
    assert summ(mode=1, ext=None) == gb.GDN_ERR_INVALID
    assert summ(mode=2, m=None) == gb.GDN_ERR_INVALID
    # flags other than REUSE_PREPARED; more units selected than exist; a
    # selection without its list
    for fl in (2, 3, 16, 2 | 4):
        assert summ(flags=fl) == gb.GDN_ERR_INVALID
    assert summ(units=FAKE, n_sel=5) == gb.GDN_ERR_INVALID     # 4 units
    assert summ(units=None, n_sel=2) == gb.GDN_ERR_INVALID
    assert L.gdn_state_merge(2, 3, 4, 64, 64, FAKE, FAKE, None, FAKE, None, None) == gb.GDN_ERR_UNSUPPORTED
    assert L.gdn_state_merge(2, 3, -1, 128, 128, FAKE, FAKE, None, FAKE, None, None) == gb.GDN_ERR_INVALID
    assert L.gdn_state_merge(0, 3, 4, 128, 128, FAKE, FAKE, None, FAKE, None, None) == gb.GDN_ERR_INVALID
    assert L.gdn_state_merge(2, 3, 4, 128, 128, None, FAKE, None, FAKE, None, None) == gb.GDN_ERR_INVALID


def test_merge_pieces_errors():
    L = gb.lib()
    doc = ctypes.c_void_p(1 << 40)
    assert L.gdn_state_merge_pieces(3, 2, 4, 64, 128, doc, FAKE, FAKE, None, FAKE, None) == gb.GDN_ERR_UNSUPPORTED
    assert L.gdn_state_merge_pieces(-1, 2, 4, 128, 128, doc, FAKE, FAKE, None, FAKE, None) == gb.GDN_ERR_INVALID
    assert L.gdn_state_merge_pieces(3, 0, 4, 128, 128, doc, FAKE, FAKE, None, FAKE, None) == gb.GDN_ERR_INVALID
    assert L.gdn_state_merge_pieces(3, 2, 0, 128, 128, doc, FAKE, FAKE, None, FAKE, None) == gb.GDN_ERR_INVALID
    for i in range(4):
        ptrs = [doc, FAKE, FAKE, FAKE]
        ptrs[i] = None
        assert L.gdn_state_merge_pieces(3, 2, 4, 128, 128, ptrs[0], ptrs[1], ptrs[2], None, ptrs[3],
                                        None) == gb.GDN_ERR_INVALID
    # no pieces: nothing to launch
    assert L.gdn_state_merge_pieces(0, 1, 4, 128, 128, None, None, None, None, None, None) == gb.GDN_OK


# ------------------------------------------------------------------ split pieces
def _random_offsets(rnd, total, n):
    cuts = sorted(rnd.sample(range(1, total), min(n - 1, total - 1))) if total > 1 else []
    return [0] + cuts + [total]


def test_split_meta_matches_definition():
    rnd = random.Random(23)
    for _ in range(300):
        total = rnd.randint(1, 2000)
        docs = _random_offsets(rnd, total, rnd.randint(1, 25))
        segs = _random_offsets(rnd, total, rnd.randint(1, 9))
        po, pd, ps = gb.gdn_split_meta(docs, segs)
        assert (po, pd, ps) == tuple(list(x) for x in varlen.split_pieces(docs, segs))


def test_split_meta_rejects_and_capacity():
    L = gb.lib()
    with pytest.raises(ValueError):
        gb.gdn_split_meta([0, 5, 9], [0, 4, 8])          # segments end before the tokens
    with pytest.raises(ValueError):
        gb.gdn_split_meta([0, 5, 5, 9], [0, 9])          # empty document
    docs = (ctypes.c_int32 * 3)(0, 100, 300)
    segs = (ctypes.c_int32 * 3)(0, 150, 300)
    po = (ctypes.c_int32 * 3)()
    n = ctypes.c_int32(0)
    st = L.gdn_split_meta(docs, 3, segs, 3, 300, po, None, None, 2, ctypes.byref(n))
    assert st == gb.GDN_ERR_CAPACITY and n.value == 3   # [0,100), [100,150), [150,300)
    st = L.gdn_split_meta(docs, 3, segs, 3, 300, None, None, None, 0, ctypes.byref(n))
    assert st == gb.GDN_OK and n.value == 3


def test_status_maps_to_page_exceptions():
    with pytest.raises(ValueError):
        gb.check(gb.GDN_ERR_INVALID, "x")
    with pytest.raises(NotImplementedError):
        gb.check(gb.GDN_ERR_UNSUPPORTED, "x")
    with pytest.raises(RuntimeError):
        gb.check(gb.GDN_ERR_DEVICE, "x")


# ------------------------------------------------------------------ allocation-free forward
def noalloc(d, *, q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, o=FAKE, flags=0):
    return gb.lib().gdn_chunk_fwd_noalloc(ctypes.byref(d), q, k, v, g, beta, None, o, None, None, flags, None)


def test_noalloc_rejects_before_any_hip_call():
    # sizing and every validation run on the host first, so these statuses
    # come back without a GPU
    big = desc(B=1, T=8192, H=64)        # 128 chunks x 64 heads x 17 KiB = 136 MiB > 128 MiB
    st, need = fwd(big, ws=None)
    assert st == gb.GDN_OK and need > 128 << 20
    assert noalloc(big) == gb.GDN_ERR_CAPACITY
    assert noalloc(desc(chunk_size=32)) == gb.GDN_ERR_INVALID
    assert noalloc(desc(K=64, V=64)) == gb.GDN_ERR_UNSUPPORTED
    assert noalloc(desc(), q=None) == gb.GDN_ERR_INVALID
    assert noalloc(desc(), flags=3) == gb.GDN_ERR_INVALID


# ------------------------------------------------------------------ backward
def bwd(d, *, ws=FAKE, nbytes=None, ptrs=None, flags=0):
    # q, k, v, g, beta, h, dout, dht, dq, dk, dv, dg, dbeta, dh0
    p = [FAKE] * 14 if ptrs is None else ptrs
    nb = ctypes.c_size_t(nbytes if nbytes is not None else (1 << 40))
    return gb.lib().gdn_chunk_bwd(ctypes.byref(d), *p, flags, ws, ctypes.byref(nb), None), nb.value


def test_backward_host_checks():
    st, need = bwd(desc(), ws=None)
    # fp32 preparation (T, P, five gate rows), dL/dh at each chunk exit and dvn,
    # every region 256-byte aligned
    nch = 2 * 4 * 3
    a256 = lambda x: ((x + 255) // 256) * 256
    prep = 2 * a256(nch * 64 * 64 * 4) + a256(nch * 5 * 64 * 4)
    assert st == gb.GDN_OK and need == a256(prep + nch * 128 * 128 * 4) + a256(nch * 64 * 128 * 4)
    # per key: T, P, the gated q and k tiles (q b^G, k b^G, k b^{G_L - G}) and
    # G_last in fp32, then the same dL/dh region and, in place of dvn, the
    # fp32 chunk maps A (K x K) of the state gradient
    stk, needk = bwd(desc(gate_kind=1), ws=None)
    prepk = 2 * a256(nch * 64 * 64 * 4) + 3 * a256(nch * 64 * 128 * 4) + a256(nch * 128 * 4)
    assert stk == gb.GDN_OK and needk == a256(prepk + nch * 128 * 128 * 4) + a256(nch * 128 * 128 * 4)
    assert bwd(desc(chunk_size=32), ws=None)[0] == gb.GDN_ERR_INVALID
    for f in (2, 3, 4, 8, -1):                       # only REUSE_PREPARED is a backward flag
        assert bwd(desc(), flags=f)[0] == gb.GDN_ERR_INVALID, f
    assert bwd(desc(), nbytes=need - 1)[0] == gb.GDN_ERR_CAPACITY
    assert bwd(desc(), ws=FAKE + 128)[0] == gb.GDN_ERR_INVALID
    for i in range(14):
        p = [FAKE] * 14
        p[i] = None
        want = gb.GDN_OK if i in (7, 13) else gb.GDN_ERR_INVALID    # dht and dh0 may be NULL
        if want == gb.GDN_OK:
            continue                                                  # would launch: GPU only
        assert bwd(desc(), ptrs=p)[0] == want, i


def test_gradient_summary_and_adjoint_errors():
    L = gb.lib()
    nb = ctypes.c_size_t(0)
    d = desc()
    # the backward's workspace size, and its checks
    st = L.gdn_state_grad_summary(ctypes.byref(d), None, None, None, None, None, None, None, None, 0, None,
                                  ctypes.byref(nb), None)
    assert st == gb.GDN_OK and nb.value == bwd(desc(), ws=None)[1]
    assert L.gdn_state_grad_summary(ctypes.byref(desc(gate_kind=1)), None, None, None, None, None, None, None,
                                    None, 0, None, ctypes.byref(nb), None) == gb.GDN_OK
    assert nb.value == bwd(desc(gate_kind=1), ws=None)[1]
    big = ctypes.c_size_t(1 << 40)
    # no output
    assert L.gdn_state_grad_summary(ctypes.byref(d), *[FAKE] * 7, None, 0, FAKE, ctypes.byref(big),
                                    None) == gb.GDN_ERR_INVALID
    assert L.gdn_state_grad_summary(ctypes.byref(d), *[FAKE] * 8, 2, FAKE, ctypes.byref(big),
                                    None) == gb.GDN_ERR_INVALID
    assert L.gdn_state_merge_adjoint(2, 3, 4, 64, 128, FAKE, FAKE, None, FAKE, None, None) == gb.GDN_ERR_UNSUPPORTED
    assert L.gdn_state_merge_adjoint(0, 3, 4, 128, 128, FAKE, FAKE, None, FAKE, None, None) == gb.GDN_ERR_INVALID
    assert L.gdn_state_merge_adjoint(2, 3, -1, 128, 128, FAKE, FAKE, None, FAKE, None, None) == gb.GDN_ERR_INVALID
    for i in range(3):
        ptrs = [FAKE, FAKE, FAKE]
        ptrs[i] = None
        assert L.gdn_state_merge_adjoint(2, 3, 4, 128, 128, ptrs[0], ptrs[1], None, ptrs[2], None,
                                         None) == gb.GDN_ERR_INVALID


def test_pieced_forward_workspace():
    # long dense rows with few (row, head) pairs run in pieces: the size query
    # covers every piece's preparation and the state between pieces, more than
    # one pass needs; the allocation-free entry keeps the one-pass size
    L = gb.lib()
    d = desc(B=1, T=16384 + 37, H=4)              # 257 chunks, 16 state workgroups
    st, need = fwd(d, ws=None)
    one_pass = fwd(desc(B=1, T=16384 + 37, H=64), ws=None)[1] // 16   # 64 pairs: not pieced
    assert st == gb.GDN_OK and need > one_pass
    assert need - one_pass >= 4 * 128 * 128 * 4   # the state carried between pieces
    st, got = fwd(d, nbytes=need - 1)
    assert st == gb.GDN_ERR_CAPACITY and got == need
