"""ctypes binding of libgdn (include/gdn.h): argument marshalling only.

Every step of the forward runs in the HIP library; this module turns torch
tensors into device pointers, allocates outputs and the workspace through
torch (memory plumbing), passes torch's current HIP stream, and maps status
codes to the exception types the pages' adapters use (ValueError for
contract violations, NotImplementedError for unsupported features,
RuntimeError for device failures). It fails loudly when the library has not
been built: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_OK, GDN_ERR_INVALID, GDN_ERR_UNSUPPORTED, GDN_ERR_DEVICE, GDN_ERR_CAPACITY = range(5)
LAYOUT_BSND, LAYOUT_TND = 0, 1
DTYPE_F32, DTYPE_BF16 = 0, 1
GATE_SCALAR, GATE_PER_KEY = 0, 1
FLAG_REUSE_PREPARED, FLAG_PREPARE_ONLY, FLAG_QK_L2NORM, FLAG_BETA_SIGMOID = 1, 2, 4, 8
_TRANSFORMS = FLAG_QK_L2NORM | FLAG_BETA_SIGMOID

_i32p = ctypes.POINTER(ctypes.c_int32)


class GdnDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
                ("K", ctypes.c_int32), ("V", ctypes.c_int32), ("layout", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("o_dtype", ctypes.c_int32),
                ("gate_kind", ctypes.c_int32), ("use_exp2", ctypes.c_int32),
                ("chunk_size", ctypes.c_int32), ("scale", ctypes.c_float),
                ("n_units", ctypes.c_int32), ("offsets_host", _i32p), ("offsets_dev", ctypes.c_void_p),
                ("chunk_offsets_dev", ctypes.c_void_p), ("chunk_indices_dev", ctypes.c_void_p)]


class GdnSlots(ctypes.Structure):
    _fields_ = [("g_cumsum", ctypes.c_void_p), ("A", ctypes.c_void_p), ("h", ctypes.c_void_p),
                ("v_new", ctypes.c_void_p), ("q_hat", ctypes.c_void_p), ("k_hat", ctypes.c_void_p),
                ("q_rstd", ctypes.c_void_p), ("k_rstd", ctypes.c_void_p), ("beta_eff", ctypes.c_void_p)]


SLOT_NAMES = ("g_cumsum", "A", "h", "v_new", "q_hat", "k_hat", "q_rstd", "k_rstd", "beta_eff")


_LIB = None


def lib():
    """The loaded libgdn.so; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libgdn.so is not built ({LIB_PATH}); run "
                               "`python -m chunked_gated_delta_05_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz = ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t)
        L.gdn_varlen_meta.restype = ctypes.c_int
        L.gdn_varlen_meta.argtypes = [_i32p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _i32p,
                                      ctypes.c_int32, _i32p, _i32p]
        L.gdn_chunk_fwd.restype = ctypes.c_int
        L.gdn_chunk_fwd.argtypes = [ctypes.POINTER(GdnDesc), vp, vp, vp, vp, vp, vp, vp, vp,
                                    ctypes.POINTER(GdnSlots), ctypes.c_int32, vp, sz, vp]
        L.gdn_state_summary.restype = ctypes.c_int
        L.gdn_state_summary.argtypes = [ctypes.POINTER(GdnDesc), vp, vp, vp, vp, vp, ctypes.c_int32,
                                        ctypes.c_int32, vp, ctypes.c_int32, vp, vp, vp, sz, vp]
        L.gdn_split_meta.restype = ctypes.c_int
        L.gdn_split_meta.argtypes = [_i32p, ctypes.c_int32, _i32p, ctypes.c_int32, ctypes.c_int32, _i32p,
                                     _i32p, _i32p, ctypes.c_int32, _i32p]
        L.gdn_state_grad_summary.restype = ctypes.c_int
        L.gdn_state_grad_summary.argtypes = [ctypes.POINTER(GdnDesc)] + [vp] * 8 + [ctypes.c_int32, vp, sz, vp]
        L.gdn_state_merge_adjoint.restype = ctypes.c_int
        L.gdn_state_merge_adjoint.argtypes = [ctypes.c_int32] * 5 + [vp] * 6
        L.gdn_state_merge_pieces.restype = ctypes.c_int
        L.gdn_state_merge_pieces.argtypes = [ctypes.c_int32] * 5 + [vp, vp, vp, vp, vp, vp]
        L.gdn_state_merge.restype = ctypes.c_int
        L.gdn_state_merge.argtypes = [ctypes.c_int32] * 5 + [vp, vp, vp, vp, vp, vp]
        L.gdn_chunk_bwd.restype = ctypes.c_int
        L.gdn_chunk_bwd.argtypes = [ctypes.POINTER(GdnDesc)] + [vp] * 14 + [ctypes.c_int32, vp, sz, vp]
        L.gdn_chunk_fwd_noalloc.restype = ctypes.c_int
        L.gdn_chunk_fwd_noalloc.argtypes = [ctypes.POINTER(GdnDesc), vp, vp, vp, vp, vp, vp, vp, vp,
                                            ctypes.POINTER(GdnSlots), ctypes.c_int32, vp]
        _LIB = L
    return _LIB


def check(status: int, what: str) -> None:
    if status == GDN_OK:
        return
    msg = f"{what}: libgdn status {status}"
    if status in (GDN_ERR_INVALID, GDN_ERR_CAPACITY):
        raise ValueError(msg)
    if status == GDN_ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    raise RuntimeError(msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(dt):
    if dt == torch.bfloat16:
        return DTYPE_BF16
    if dt == torch.float32:
        return DTYPE_F32
    raise ValueError(f"unsupported dtype {dt}")


# ------------------------------------------------------------------ metadata
def gdn_varlen_meta(offsets, total_tokens: int, chunk_size: int = 64):
    """Host chunk metadata: (chunk_indices int32 [n, 2], chunk_offsets int32
    [len(offsets)]) as CPU tensors. Offsets must be ints (no bools), start at
    0, end at total_tokens and strictly increase."""
    offs = list(offsets.tolist() if isinstance(offsets, torch.Tensor) else offsets)
    if any(isinstance(x, bool) or not isinstance(x, int) for x in offs):
        raise ValueError("offsets must be integers")
    if any(x < -2 ** 31 or x >= 2 ** 31 for x in offs):
        raise ValueError("offsets must fit in int32")
    n = len(offs)
    arr = (ctypes.c_int32 * max(n, 1))(*offs)
    cnt = ctypes.c_int32(0)
    check(lib().gdn_varlen_meta(arr, n, int(total_tokens), int(chunk_size), None, 0, None,
                                ctypes.byref(cnt)), "gdn_varlen_meta")
    ci = torch.empty((max(cnt.value, 1), 2), dtype=torch.int32)
    co = torch.empty((n,), dtype=torch.int32)
    check(lib().gdn_varlen_meta(arr, n, int(total_tokens), int(chunk_size),
                                ctypes.cast(ci.data_ptr(), _i32p), cnt.value,
                                ctypes.cast(co.data_ptr(), _i32p), ctypes.byref(cnt)), "gdn_varlen_meta")
    return ci[:cnt.value], co


@dataclass
class UnitMeta:
    """Units of a call: host offsets (validated by the library) and their
    device copies with the chunk metadata. Build once per offsets list."""
    offsets: list
    host: ctypes.Array
    offsets_dev: torch.Tensor
    chunk_offsets_dev: torch.Tensor
    chunk_indices_dev: torch.Tensor
    n_chunks: int


def make_meta(offsets, total_tokens: int, device) -> UnitMeta:
    offs = [int(x) for x in offsets]
    ci, co = gdn_varlen_meta(offs, total_tokens)
    dev = torch.device(device)
    ci_dev = ci.to(dev) if ci.numel() else torch.zeros((1, 2), dtype=torch.int32, device=dev)
    return UnitMeta(offs, (ctypes.c_int32 * len(offs))(*offs),
                    torch.tensor(offs, dtype=torch.int32, device=dev), co.to(dev), ci_dev,
                    int(co[-1]))


def segment_offsets(B: int, T: int, seg) -> list:
    """Flat unit offsets of a split: every row b cut at the in-row offsets seg."""
    seg = [int(x) for x in seg]
    return [b * T + s for b in range(B) for s in seg[:-1]] + [B * T]


# ------------------------------------------------------------------ descriptor
def _desc(q_like, H, dtype, o_dtype, per_key, use_exp2, scale, meta: UnitMeta | None):
    d = GdnDesc()
    if q_like.dim() == 4:
        d.B, d.T = q_like.shape[0], q_like.shape[1]
        d.layout = LAYOUT_BSND
    elif q_like.dim() == 3:
        d.B, d.T = 1, q_like.shape[0]
        d.layout = LAYOUT_TND
    else:
        raise ValueError("GDN inputs must have shape [B,T,H,K] or [T,H,K]")
    d.H, d.K = H, q_like.shape[-1]
    d.V = d.K
    d.dtype, d.o_dtype = _dtype_code(dtype), _dtype_code(o_dtype)
    d.gate_kind = GATE_PER_KEY if per_key else GATE_SCALAR
    d.use_exp2 = int(bool(use_exp2))
    d.chunk_size = 64
    d.scale = float(scale)
    if meta is not None:
        d.n_units = len(meta.offsets) - 1
        d.offsets_host = ctypes.cast(meta.host, _i32p)
        d.offsets_dev = meta.offsets_dev.data_ptr()
        d.chunk_offsets_dev = meta.chunk_offsets_dev.data_ptr()
        d.chunk_indices_dev = meta.chunk_indices_dev.data_ptr()
    return d


def _check_tensor(name, t, dtype, shape, device):
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def _check_inputs(q, k, v, g, beta, meta=None, device_check=True):
    """Every input against k's dtype, layout and device, before any C call:
    the C ABI takes bare pointers and cannot check buffer sizes, so this is
    the guard against reading past a buffer. q and v may be None where the
    call does not read them. Returns (H, per_key)."""
    if k is None or k.dim() not in (3, 4):
        raise ValueError("GDN inputs must have shape [B,T,H,K] or [T,H,K]")
    if k.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError(f"unsupported dtype {k.dtype}")
    lead, H, K = tuple(k.shape[:-2]), k.shape[-2], k.shape[-1]
    _check_tensor("k", k, k.dtype, k.shape, None)
    if q is not None:
        _check_tensor("q", q, k.dtype, k.shape, None)
    if v is not None:
        _check_tensor("v", v, k.dtype, (*lead, H, v.shape[-1] if v.dim() == k.dim() else -1), None)
    if g is None or g.dim() not in (k.dim() - 1, k.dim()):
        raise ValueError("g must be [..., H] (scalar gate) or [..., H, K] (per-key gate)")
    per_key = g.dim() == k.dim()
    _check_tensor("g", g, torch.float32, (*lead, H, K) if per_key else (*lead, H), None)
    _check_tensor("beta", beta, k.dtype, (*lead, H), None)
    if device_check:
        _require_gpu(q, k, v, g, beta, meta)
    return H, per_key


def _require_gpu(q, k, v, g, beta, meta):
    dev = k.device
    if dev.type != "cuda":
        raise ValueError(f"inputs must be GPU tensors, got {dev}")
    for name, t in (("q", q), ("v", v), ("g", g), ("beta", beta)):
        if t is not None and t.device != dev:
            raise ValueError(f"{name} must be on {dev}, got {t.device}")
    if meta is not None:
        for t in (meta.offsets_dev, meta.chunk_offsets_dev, meta.chunk_indices_dev):
            if t.device != dev:
                raise ValueError(f"unit metadata must be on {dev}, got {t.device}")


def n_units_of(q_like, meta):
    return q_like.shape[0] if meta is None else len(meta.offsets) - 1


def workspace_bytes(desc: GdnDesc, fn="fwd") -> int:
    nb = ctypes.c_size_t(0)
    if fn == "fwd":
        st = lib().gdn_chunk_fwd(ctypes.byref(desc), None, None, None, None, None, None, None, None,
                                 None, 0, None, ctypes.byref(nb), None)
    else:
        st = lib().gdn_state_summary(ctypes.byref(desc), None, None, None, None, None, 0, 0, None, -1,
                                     None, None, None, ctypes.byref(nb), None)
    check(st, "workspace query")
    return nb.value


# ------------------------------------------------------------------ argument checks
def _state_shape(k, v, meta):
    return (n_units_of(k, meta), k.shape[-2], k.shape[-1], v.shape[-1])


def _fwd_args(q, k, v, g, beta, scale, meta, initial_state, o_dtype, out, final_out, want_final,
              use_exp2, flags, extras_wanted=()):
    """Checked arguments of one forward call: (desc, o, final, slots, extras)."""
    prep_only = bool(flags & FLAG_PREPARE_ONLY)
    H, per_key = _check_inputs(q, k, None if prep_only else v, g, beta, meta, device_check=False)
    if not prep_only and (q is None or v is None):
        raise ValueError("q and v are required unless only preparing")
    if per_key and q is None and not flags & FLAG_REUSE_PREPARED:
        raise ValueError("the per-key preparation needs q")
    if o_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"unsupported output dtype {o_dtype}")
    if scale is None:
        scale = k.shape[-1] ** -0.5
    desc = _desc(k, H, k.dtype, o_dtype, per_key, use_exp2, scale, meta)
    dev = k.device
    vv = v if v is not None else k
    sshape = _state_shape(k, vv, meta)
    o = fin = None
    if not prep_only:
        o = out if out is not None else torch.empty(v.shape, dtype=o_dtype, device=dev)
        _check_tensor("out", o, o_dtype, v.shape, dev)
        if want_final or final_out is not None:
            fin = final_out if final_out is not None else torch.empty(sshape, dtype=torch.float32, device=dev)
            _check_tensor("final_out", fin, torch.float32, sshape, dev)
    if initial_state is not None:
        _check_tensor("initial_state", initial_state, torch.float32, sshape, dev)
    extras = {}
    tokens = k.shape[0] * k.shape[1] if k.dim() == 4 else k.shape[0]
    lead = tuple(k.shape[:-2])
    if any(n not in SLOT_NAMES for n in extras_wanted):
        raise ValueError(f"unknown slots {extras_wanted}; known: {SLOT_NAMES}")
    if any(n in extras_wanted for n in ("q_hat", "q_rstd")) and q is None:
        raise ValueError("q_hat and q_rstd need q")
    if "g_cumsum" in extras_wanted:
        extras["g_cumsum"] = torch.empty(g.shape, dtype=torch.float32, device=dev)
    if "A" in extras_wanted:
        extras["A"] = torch.empty((tokens, H, 64), dtype=torch.float32, device=dev)
    if "h" in extras_wanted:
        n_chunks = meta.n_chunks if meta is not None else k.shape[0] * ((k.shape[1] + 63) // 64)
        extras["h"] = torch.empty((n_chunks, H, k.shape[-1], vv.shape[-1]), dtype=torch.float32, device=dev)
    if "v_new" in extras_wanted:
        extras["v_new"] = torch.empty(vv.shape, dtype=torch.float32, device=dev)
    for n in ("q_hat", "k_hat"):
        if n in extras_wanted:
            extras[n] = torch.empty(k.shape, dtype=k.dtype, device=dev)
    for n in ("q_rstd", "k_rstd"):
        if n in extras_wanted:
            extras[n] = torch.empty((*lead, H), dtype=torch.float32, device=dev)
    if "beta_eff" in extras_wanted:
        extras["beta_eff"] = torch.empty(beta.shape, dtype=beta.dtype, device=dev)
    _require_gpu(q, k, None if prep_only else v, g, beta, meta)
    slots = GdnSlots(*[_ptr(extras.get(n)) for n in SLOT_NAMES])
    return desc, o, fin, slots, extras


# ------------------------------------------------------------------ entry points
def gdn_chunk_fwd(q, k, v, g, beta, scale=None, *, meta: UnitMeta | None = None, initial_state=None,
                  output_final_state=False, use_exp2=False, o_dtype=torch.float32,
                  want_g_cumsum=False, want_A=False, want_h=False, flags=0, workspace=None, out=None,
                  final_out=None, qk_l2norm=False, beta_sigmoid=False, slots=()):
    """Chunked gated delta rule forward through libgdn.

    q, k [B,T,H,K] (BSND) or [T,H,K] (TND, needs meta); v like q; g fp32
    [..,H] (scalar gate) or [..,H,K] (per-key gate); beta [..,H]. Given
    out / final_out buffers are written in place (out: o_dtype, v's shape;
    final_out: fp32 [units,H,K,V]). qk_l2norm / beta_sigmoid: the in-kernel
    input transforms (FLAG_QK_L2NORM, FLAG_BETA_SIGMOID). slots: names from
    SLOT_NAMES to return (want_* are the older spellings of three of them).
    Returns (o, final_state or None, extras dict)."""
    wanted = [n for n, f in (("g_cumsum", want_g_cumsum), ("A", want_A), ("h", want_h)) if f] + list(slots)
    flags = int(flags) | (FLAG_QK_L2NORM if qk_l2norm else 0) | (FLAG_BETA_SIGMOID if beta_sigmoid else 0)
    desc, o, fin, slots, extras = _fwd_args(q, k, v, g, beta, scale, meta, initial_state, o_dtype, out,
                                            final_out, output_final_state, use_exp2, flags, wanted)
    dev = k.device
    nb = workspace_bytes(desc)
    ws = workspace if workspace is not None else torch.empty(nb, dtype=torch.uint8, device=dev)
    if ws.dtype != torch.uint8 or ws.device != dev or ws.numel() < nb:
        raise ValueError(f"workspace must be a uint8 tensor of at least {nb} bytes on {dev}")
    nbytes = ctypes.c_size_t(ws.numel())
    check(lib().gdn_chunk_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                              _ptr(initial_state), _ptr(o), _ptr(fin), ctypes.byref(slots), int(flags),
                              _ptr(ws), ctypes.byref(nbytes), _stream(dev)), "gdn_chunk_fwd")
    return o, fin, extras


def gdn_chunk_fwd_noalloc(q, k, v, g, beta, scale=None, *, out, final_out=None, meta: UnitMeta | None = None,
                          initial_state=None, use_exp2=False, flags=0):
    """gdn_chunk_fwd_noalloc: the forward with the library's own per-GPU
    scratch instead of a workspace; the caller passes every output buffer
    (out, and final_out when the final state is wanted)."""
    desc, o, fin, slots, _ = _fwd_args(q, k, v, g, beta, scale, meta, initial_state, out.dtype, out,
                                       final_out, False, use_exp2, flags)
    check(lib().gdn_chunk_fwd_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                      _ptr(initial_state), _ptr(o), _ptr(fin), ctypes.byref(slots), int(flags),
                                      _stream(k.device)), "gdn_chunk_fwd_noalloc")
    return o, fin


class FwdCall:
    """gdn_chunk_fwd with its arguments marshalled once, for repeated calls
    on the same tensors (timing loops, serving steps): call(flags) issues the
    C call with the stored descriptor, pointers, workspace and stream. The
    tensors must stay alive and in place while the object is used."""

    def __init__(self, q, k, v, g, beta, scale=None, *, out, workspace, meta: UnitMeta | None = None,
                 initial_state=None, final_out=None, use_exp2=False, transforms=0):
        self._desc, o, fin, self._slots, _ = _fwd_args(q, k, v, g, beta, scale, meta, initial_state, out.dtype,
                                                       out, final_out, False, use_exp2, 0)
        if transforms & ~_TRANSFORMS:
            raise ValueError("transforms takes FLAG_QK_L2NORM and FLAG_BETA_SIGMOID only")
        self._xf = int(transforms)
        nb = workspace_bytes(self._desc)
        if workspace.dtype != torch.uint8 or workspace.device != k.device or workspace.numel() < nb:
            raise ValueError(f"workspace must be a uint8 tensor of at least {nb} bytes on {k.device}")
        self._keep = (q, k, v, g, beta, out, workspace, meta, initial_state, final_out)
        self._nbytes = ctypes.c_size_t(workspace.numel())
        self._args = [ctypes.byref(self._desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                      _ptr(initial_state), _ptr(o), _ptr(fin), ctypes.byref(self._slots)]
        self._tail = [_ptr(workspace), ctypes.byref(self._nbytes), _stream(k.device)]
        self._fn = lib().gdn_chunk_fwd

    def __call__(self, flags: int = 0) -> None:
        check(self._fn(*self._args, int(flags) | self._xf, *self._tail), "gdn_chunk_fwd")


def gdn_state_summary(k, v, g, beta, *, meta: UnitMeta, mode=0, use_exp2=False, q=None,
                      workspace=None, S_ext=None, M=None, flags=0, units=None, qk_l2norm=False,
                      beta_sigmoid=False):
    """Per-unit summaries (S_ext [units,H,K,V], M [units,H,K,K]; given
    buffers are written in place); pass q to leave a per-key preparation
    that a reusing forward can use. units: None (all) or a device int32
    tensor of the unit indices to summarise (the other slots are left
    as they are); flags: 0 or FLAG_REUSE_PREPARED."""
    if mode not in (0, 1, 2):
        raise ValueError("mode must be 0 (both), 1 (S_ext) or 2 (M)")
    if flags & ~(FLAG_REUSE_PREPARED | _TRANSFORMS):
        raise ValueError("flags take FLAG_REUSE_PREPARED and the transform flags only")
    flags = int(flags) | (FLAG_QK_L2NORM if qk_l2norm else 0) | (FLAG_BETA_SIGMOID if beta_sigmoid else 0)
    if v is None:
        raise ValueError("v is required")
    H, per_key = _check_inputs(q, k, v, g, beta, meta)
    desc = _desc(k, H, k.dtype, torch.float32, per_key, use_exp2, 1.0, meta)
    dev = k.device
    nb = workspace_bytes(desc)
    ws = workspace if workspace is not None else torch.empty(nb, dtype=torch.uint8, device=dev)
    if ws.dtype != torch.uint8 or ws.device != dev or ws.numel() < nb:
        raise ValueError(f"workspace must be a uint8 tensor of at least {nb} bytes on {dev}")
    if flags & FLAG_REUSE_PREPARED and workspace is None:
        raise ValueError("FLAG_REUSE_PREPARED needs the workspace of the preparing call")
    n_units = n_units_of(k, meta)
    n_sel = -1
    if units is not None:
        if units.dtype != torch.int32 or units.dim() != 1 or units.device != dev or not units.is_contiguous():
            raise ValueError(f"units must be a contiguous 1-D int32 tensor on {dev}")
        n_sel = units.numel()
        if n_sel > n_units:
            raise ValueError(f"{n_sel} units selected out of {n_units}")
    K, V = k.shape[-1], v.shape[-1]
    if mode != 2 and S_ext is None:
        S_ext = torch.empty((n_units, H, K, V), dtype=torch.float32, device=dev)
    if mode != 1 and M is None:
        M = torch.empty((n_units, H, K, K), dtype=torch.float32, device=dev)
    if mode != 2:
        _check_tensor("S_ext", S_ext, torch.float32, (n_units, H, K, V), dev)
    if mode != 1:
        _check_tensor("M", M, torch.float32, (n_units, H, K, K), dev)
    nbytes = ctypes.c_size_t(ws.numel())
    check(lib().gdn_state_summary(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                  int(mode), int(flags), _ptr(units) if n_sel > 0 else None, n_sel,
                                  _ptr(S_ext if mode != 2 else None), _ptr(M if mode != 1 else None),
                                  _ptr(ws), ctypes.byref(nbytes), _stream(dev)), "gdn_state_summary")
    return (S_ext if mode != 2 else None), (M if mode != 1 else None), ws


def gdn_state_merge(S_ext, M, S0=None, *, B: int, n_seg: int, want_final=True, S_init=None,
                    S_final=None):
    """S_ext [B*n_seg,H,K,V], M [B*n_seg,H,K,K] (units row-major) -> S_init
    [B*n_seg,H,K,V] (the state entering every segment) and S_final [B,H,K,V]
    (given buffers are written in place)."""
    if S_ext.dim() != 4:
        raise ValueError("S_ext must be [B*n_seg, H, K, V]")
    H, K, V = S_ext.shape[1], S_ext.shape[2], S_ext.shape[3]
    dev = S_ext.device
    if dev.type != "cuda":
        raise ValueError(f"summaries must be GPU tensors, got {dev}")
    _check_tensor("S_ext", S_ext, torch.float32, (B * n_seg, H, K, V), dev)
    _check_tensor("M", M, torch.float32, (B * n_seg, H, K, K), dev)
    if S0 is not None:
        _check_tensor("S0", S0, torch.float32, (B, H, K, V), dev)
    if S_init is None:
        S_init = torch.empty_like(S_ext)
    if want_final and S_final is None:
        S_final = torch.empty((B, H, K, V), dtype=torch.float32, device=dev)
    if not want_final:
        S_final = None
    _check_tensor("S_init", S_init, torch.float32, tuple(S_ext.shape), dev)
    if S_final is not None:
        _check_tensor("S_final", S_final, torch.float32, (B, H, K, V), dev)
    check(lib().gdn_state_merge(B, H, n_seg, K, V, _ptr(S_ext), _ptr(M), _ptr(S0), _ptr(S_init),
                                _ptr(S_final), _stream(dev)), "gdn_state_merge")
    return S_init, S_final


def workspace_bytes_bwd(k, g, meta: UnitMeta | None = None, *, use_exp2=False) -> int:
    """Workspace bytes of gdn_chunk_bwd / gdn_state_grad_summary for inputs
    shaped like k and g (the query form of the call)."""
    H = k.shape[-2]
    desc = _desc(k, H, k.dtype, k.dtype, g.dim() == k.dim(), use_exp2, 1.0, meta)
    nb = ctypes.c_size_t(0)
    check(lib().gdn_chunk_bwd(ctypes.byref(desc), *([None] * 14), 0, None, ctypes.byref(nb), None), "workspace query")
    return nb.value


def gdn_chunk_bwd(q, k, v, g, beta, h, dout, scale=None, *, meta: UnitMeta | None = None, dht=None,
                  use_exp2=False, want_dh0=True, workspace=None, reuse_prepared=False):
    """Gradients of the chunked forward (scalar or per-key gate) through libgdn.

    h: the forward's entry states (gdn_chunk_fwd(..., want_h=True) extras
    "h", fp32 [n_chunks, H, K, V]); dout: dL/do in the input dtype, v's
    shape; dht: dL/d(final state) fp32 [units, H, K, V] or None. Returns a
    dict of fp32 tensors dq, dk, dv, dg (g's shape), dbeta and dh0 (dL/d
    initial state, when wanted). reuse_prepared: the given workspace holds the
    backward preparation of these inputs (from gdn_state_grad_summary or an
    earlier call)."""
    H, per_key = _check_inputs(q, k, v, g, beta, meta, device_check=False)
    if scale is None:
        scale = k.shape[-1] ** -0.5
    desc = _desc(k, H, k.dtype, k.dtype, per_key, use_exp2, scale, meta)
    dev = k.device
    units = n_units_of(k, meta)
    K, V = k.shape[-1], v.shape[-1]
    n_chunks = meta.n_chunks if meta is not None else k.shape[0] * ((k.shape[1] + 63) // 64)
    _check_tensor("h", h, torch.float32, (n_chunks, H, K, V), dev)
    _check_tensor("dout", dout, k.dtype, v.shape, dev)
    if dht is not None:
        _check_tensor("dht", dht, torch.float32, (units, H, K, V), dev)
    _require_gpu(q, k, v, g, beta, meta)
    out = {"dq": torch.empty(q.shape, dtype=torch.float32, device=dev),
           "dk": torch.empty(k.shape, dtype=torch.float32, device=dev),
           "dv": torch.empty(v.shape, dtype=torch.float32, device=dev),
           "dg": torch.empty(g.shape, dtype=torch.float32, device=dev),
           "dbeta": torch.empty(beta.shape, dtype=torch.float32, device=dev)}
    if want_dh0:
        out["dh0"] = torch.empty((units, H, K, V), dtype=torch.float32, device=dev)
    nb = ctypes.c_size_t(0)
    if reuse_prepared and workspace is None:
        raise ValueError("reuse_prepared needs the workspace that holds the preparation")
    flags = FLAG_REUSE_PREPARED if reuse_prepared else 0
    check(lib().gdn_chunk_bwd(ctypes.byref(desc), *([None] * 14), 0, None, ctypes.byref(nb), None), "workspace query")
    ws = workspace if workspace is not None else torch.empty(nb.value, dtype=torch.uint8, device=dev)
    if ws.dtype != torch.uint8 or ws.device != dev or ws.numel() < nb.value:
        raise ValueError(f"workspace must be a uint8 tensor of at least {nb.value} bytes on {dev}")
    nbytes = ctypes.c_size_t(ws.numel())
    check(lib().gdn_chunk_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h),
                              _ptr(dout), _ptr(dht), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                              _ptr(out["dg"]), _ptr(out["dbeta"]), _ptr(out.get("dh0")), flags, _ptr(ws),
                              ctypes.byref(nbytes), _stream(dev)), "gdn_chunk_bwd")
    return out


def gdn_state_grad_summary(q, k, v, g, beta, h, dout, scale=None, *, meta: UnitMeta, use_exp2=False,
                           workspace=None):
    """dS_ext [units,H,K,V]: dL/d(entry state) of every unit through its own
    outputs only (zero gradient at its exit); arguments as gdn_chunk_bwd."""
    H, per_key = _check_inputs(q, k, v, g, beta, meta, device_check=False)
    if scale is None:
        scale = k.shape[-1] ** -0.5
    desc = _desc(k, H, k.dtype, k.dtype, per_key, use_exp2, scale, meta)
    dev = k.device
    K, V = k.shape[-1], v.shape[-1]
    _check_tensor("h", h, torch.float32, (meta.n_chunks, H, K, V), dev)
    _check_tensor("dout", dout, k.dtype, v.shape, dev)
    _require_gpu(q, k, v, g, beta, meta)
    dS = torch.empty((n_units_of(k, meta), H, K, V), dtype=torch.float32, device=dev)
    nb = ctypes.c_size_t(0)
    check(lib().gdn_state_grad_summary(ctypes.byref(desc), *([None] * 8), 0, None, ctypes.byref(nb), None),
          "workspace query")
    ws = workspace if workspace is not None else torch.empty(nb.value, dtype=torch.uint8, device=dev)
    if ws.dtype != torch.uint8 or ws.device != dev or ws.numel() < nb.value:
        raise ValueError(f"workspace must be a uint8 tensor of at least {nb.value} bytes on {dev}")
    nbytes = ctypes.c_size_t(ws.numel())
    check(lib().gdn_state_grad_summary(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h),
                                       _ptr(dout), _ptr(dS), 0, _ptr(ws), ctypes.byref(nbytes), _stream(dev)),
          "gdn_state_grad_summary")
    return dS


def gdn_state_merge_adjoint(dS_ext, M, dS_final=None, *, B: int, n_seg: int, want_dS0=True):
    """dS_ext [B*n_seg,H,K,V], M [B*n_seg,H,K,K] (units row-major) ->
    dS_exit [B*n_seg,H,K,V] (the gradient arriving at each segment's exit)
    and dS0 [B,H,K,V] (at the first segment's entry) or None."""
    if dS_ext.dim() != 4:
        raise ValueError("dS_ext must be [B*n_seg, H, K, V]")
    H, K, V = dS_ext.shape[1], dS_ext.shape[2], dS_ext.shape[3]
    dev = dS_ext.device
    if dev.type != "cuda":
        raise ValueError(f"summaries must be GPU tensors, got {dev}")
    _check_tensor("dS_ext", dS_ext, torch.float32, (B * n_seg, H, K, V), dev)
    _check_tensor("M", M, torch.float32, (B * n_seg, H, K, K), dev)
    if dS_final is not None:
        _check_tensor("dS_final", dS_final, torch.float32, (B, H, K, V), dev)
    dS_exit = torch.empty_like(dS_ext)
    dS0 = torch.empty((B, H, K, V), dtype=torch.float32, device=dev) if want_dS0 else None
    check(lib().gdn_state_merge_adjoint(B, H, n_seg, K, V, _ptr(dS_ext), _ptr(M), _ptr(dS_final), _ptr(dS_exit),
                                        _ptr(dS0), _stream(dev)), "gdn_state_merge_adjoint")
    return dS_exit, dS0


def split_backward(q, k, v, g, beta, h, dout, scale=None, *, seg, M, use_exp2=False, dht=None):
    """Backward of a sequence split of BSND rows (seg: in-row offsets) on one
    GPU, in the order of the reverse wavefront: every segment's gradient
    summary, the adjoint merge with the transfer maps M [B*n_seg,H,K,K] of
    the forward's summaries, then every segment's backward from its true
    exit gradient. h: the correction forward's chunk entry states over the
    segments. Returns gdn_chunk_bwd's dict, dh0 being dL/d(initial state)
    per row [B,H,K,V]."""
    B, T = k.shape[0], k.shape[1]
    n_seg = len(seg) - 1
    meta = make_meta(segment_offsets(B, T, seg), B * T, k.device)
    ws = torch.empty(workspace_bytes_bwd(k, g, meta, use_exp2=use_exp2), dtype=torch.uint8, device=k.device)
    # the gradient summaries prepare the chunks once; the segment backward reuses it
    dS_ext = gdn_state_grad_summary(q, k, v, g, beta, h, dout, scale, meta=meta, use_exp2=use_exp2, workspace=ws)
    dS_exit, dS0 = gdn_state_merge_adjoint(dS_ext, M, dht, B=B, n_seg=n_seg)
    out = gdn_chunk_bwd(q, k, v, g, beta, h, dout, scale, meta=meta, dht=dS_exit, use_exp2=use_exp2,
                        want_dh0=False, workspace=ws, reuse_prepared=True)
    out["dh0"] = dS0
    return out


class GatedDeltaRule(torch.autograd.Function):
    """The chunked forward and its backward as one autograd op (the shape of
    the pages' _AscendCGDN adapter): forward keeps the chunk entry states,
    backward returns dq, dk, dv, dg, dbeta (and dL/d initial_state). Inputs
    in the library's layouts; gradients come back in the inputs' dtypes."""

    @staticmethod
    def forward(ctx, q, k, v, g, beta, initial_state=None, scale=None, meta=None, use_exp2=False):
        o, fin, ex = gdn_chunk_fwd(q, k, v, g, beta, scale, meta=meta, initial_state=initial_state,
                                   output_final_state=True, use_exp2=use_exp2, o_dtype=torch.float32, want_h=True)
        ctx.save_for_backward(q, k, v, g, beta, ex["h"])
        ctx.scale, ctx.meta, ctx.use_exp2 = scale, meta, use_exp2
        ctx.has_s0 = initial_state is not None
        ctx.mark_non_differentiable(fin)
        return o, fin

    @staticmethod
    def backward(ctx, do, dfin):
        q, k, v, g, beta, h = ctx.saved_tensors
        r = gdn_chunk_bwd(q, k, v, g, beta, h, do.to(k.dtype).contiguous(), ctx.scale, meta=ctx.meta,
                          dht=None if dfin is None else dfin.float().contiguous(), use_exp2=ctx.use_exp2,
                          want_dh0=ctx.has_s0)
        cast = lambda x, t: x.to(t.dtype)
        return (cast(r["dq"], q), cast(r["dk"], k), cast(r["dv"], v), r["dg"], cast(r["dbeta"], beta),
                r.get("dh0"), None, None, None)


def gdn_split_meta(doc_offsets, seg_offsets):
    """Pieces of packed documents cut at segment offsets (host): returns
    (piece_offsets, piece_doc, piece_seg) as lists. Both offset lists follow
    the _packed_offsets rules and end at the same token count."""
    docs, segs = [int(x) for x in doc_offsets], [int(x) for x in seg_offsets]
    if not docs or not segs:
        raise ValueError("offsets must not be empty")
    da = (ctypes.c_int32 * len(docs))(*docs)
    sa = (ctypes.c_int32 * len(segs))(*segs)
    n = ctypes.c_int32(0)
    check(lib().gdn_split_meta(da, len(docs), sa, len(segs), docs[-1], None, None, None, 0, ctypes.byref(n)),
          "gdn_split_meta")
    po = (ctypes.c_int32 * (n.value + 1))()
    pd = (ctypes.c_int32 * max(n.value, 1))()
    ps = (ctypes.c_int32 * max(n.value, 1))()
    check(lib().gdn_split_meta(da, len(docs), sa, len(segs), docs[-1], po, pd, ps, n.value, ctypes.byref(n)),
          "gdn_split_meta")
    return list(po), list(pd)[:n.value], list(ps)[:n.value]


def gdn_state_merge_pieces(S_ext, M, piece_doc, *, n_docs: int, S0_docs=None, S_in=None):
    """Entry states S_in [n_pieces,H,K,V] of the pieces of a split packed
    sequence. piece_doc: device int32 [n_pieces] (non-decreasing); S_ext /
    M: summaries over the pieces (M may be None when no continuing piece
    enters from a nonzero state); S0_docs: [n_docs,H,K,V] or None."""
    if S_ext is None or S_ext.dim() != 4:
        raise ValueError("S_ext must be [n_pieces, H, K, V]")
    n_pieces, H, K, V = S_ext.shape
    dev = S_ext.device
    if dev.type != "cuda":
        raise ValueError(f"summaries must be GPU tensors, got {dev}")
    _check_tensor("S_ext", S_ext, torch.float32, (n_pieces, H, K, V), dev)
    if M is not None:
        _check_tensor("M", M, torch.float32, (n_pieces, H, K, K), dev)
    _check_tensor("piece_doc", piece_doc, torch.int32, (n_pieces,), dev)
    if S0_docs is not None:
        _check_tensor("S0_docs", S0_docs, torch.float32, (n_docs, H, K, V), dev)
    if S_in is None:
        S_in = torch.empty_like(S_ext)
    _check_tensor("S_in", S_in, torch.float32, (n_pieces, H, K, V), dev)
    if M is None:
        # legal only if no continuing piece enters from a nonzero state
        doc = piece_doc.tolist()
        for p in range(1, n_pieces):
            if doc[p] == doc[p - 1] and (p >= 2 and doc[p - 2] == doc[p - 1] or S0_docs is not None):
                raise ValueError("M is needed: a continuing piece enters from a nonzero state")
        M = S_ext   # never read; any valid device pointer
    check(lib().gdn_state_merge_pieces(n_pieces, int(n_docs), H, K, V, _ptr(piece_doc), _ptr(S_ext), _ptr(M),
                                       _ptr(S0_docs), _ptr(S_in), _stream(dev)), "gdn_state_merge_pieces")
    return S_in


class SplitPlan:
    """A sequence split on one GPU, planned once and run per call: the units
    are pieces (segments of rows, or pieces of packed documents cut at
    segment offsets), piece_doc names the row or document of each, and a
    piece continues the previous one when both share it.

    A call runs (1) the summaries that something consumes, those of the
    pieces followed by a piece of the same document: the last piece of a
    document needs none, its exit state comes from the correction
    (needs_summary on the Diff Coverage page); (2) the piece merge; (3) the
    correction forward of every piece from its true entry state, reusing the
    preparation of (1), with the final states of all pieces. Buffers are
    allocated once; the results of the last call are in o, S_in and the
    final states (final_of_docs picks each document's).

    ext_only_launch: a piece that starts its document from zero needs only
    S_ext, not M (half the summary columns); with it set (the default) those
    pieces are summarised in a launch of their own in mode 1, else every
    consumed summary is computed in full in one launch (one launch fewer,
    more work)."""

    def __init__(self, q, k, v, g, beta, scale, *, pieces, piece_doc, use_exp2=False, with_s0=False,
                 o_dtype=torch.float32, ext_only_launch=True):
        H, per_key = _check_inputs(q, k, v, g, beta)
        dev = k.device
        self.shape = (tuple(k.shape), tuple(v.shape), tuple(g.shape), k.dtype)
        self.scale, self.use_exp2, self.o_dtype, self.with_s0 = scale, use_exp2, o_dtype, with_s0
        self.meta = make_meta(pieces, pieces[-1], dev)
        pdoc = [int(x) for x in piece_doc]
        n = len(pdoc)
        if n != len(pieces) - 1 or any(b < a for a, b in zip(pdoc, pdoc[1:])):
            raise ValueError("piece_doc must give a non-decreasing document per piece")
        self.n_docs = pdoc[-1] + 1
        cont = [p for p in range(n - 1) if pdoc[p + 1] == pdoc[p]]
        starts = {p for p in cont if p == 0 or pdoc[p - 1] != pdoc[p]}
        ext_only = sorted(starts) if ext_only_launch and not with_s0 else []
        both = [p for p in cont if p not in ext_only]
        self.sel = [(1, torch.tensor(ext_only, dtype=torch.int32).to(dev)),
                    (0, torch.tensor(both, dtype=torch.int32).to(dev))]
        K, V = k.shape[-1], v.shape[-1]
        self.S_ext = torch.empty((n, H, K, V), dtype=torch.float32, device=dev)
        self.M = torch.empty((n, H, K, K), dtype=torch.float32, device=dev) if both else None
        self.S_in = torch.empty_like(self.S_ext)
        self.final = torch.empty_like(self.S_ext)
        self.o = torch.empty(v.shape, dtype=o_dtype, device=dev)
        self.piece_doc = torch.tensor(pdoc, dtype=torch.int32).to(dev)
        self.last = torch.tensor([p for p in range(n) if p == n - 1 or pdoc[p + 1] != pdoc[p]],
                                 dtype=torch.long).to(dev)
        desc = _desc(k, H, k.dtype, o_dtype, per_key, use_exp2, scale, self.meta)
        self.ws = torch.empty(workspace_bytes(desc), dtype=torch.uint8, device=dev)

    def __call__(self, q, k, v, g, beta, initial_state=None, rec=None):
        """rec(i), when given, is called after stage i (0 summaries, 1 merge,
        2 correction) to let the caller record events between them."""
        if (tuple(k.shape), tuple(v.shape), tuple(g.shape), k.dtype) != self.shape:
            raise ValueError("inputs differ from the planned shapes")
        if (initial_state is not None) != self.with_s0:
            raise ValueError("the plan was made " + ("with" if self.with_s0 else "without") + " entry states")
        flags = 0
        for mode, units in self.sel:
            if units.numel() == 0 and flags:
                continue
            gdn_state_summary(k, v, g, beta, meta=self.meta, mode=mode, use_exp2=self.use_exp2, q=q,
                              workspace=self.ws, S_ext=self.S_ext, M=self.M if mode == 0 else None,
                              flags=flags, units=units)
            flags = FLAG_REUSE_PREPARED
        if rec:
            rec(0)
        # without a map buffer no continuing piece enters from a nonzero
        # state (the plan asked for none), so the merge reads no map: S_ext
        # (the same shape, as K = V) stands in for the pointer
        gdn_state_merge_pieces(self.S_ext, self.M if self.M is not None else self.S_ext, self.piece_doc,
                               n_docs=self.n_docs, S0_docs=initial_state, S_in=self.S_in)
        if rec:
            rec(1)
        gdn_chunk_fwd(q, k, v, g, beta, self.scale, meta=self.meta, initial_state=self.S_in,
                      use_exp2=self.use_exp2, o_dtype=self.o_dtype, flags=FLAG_REUSE_PREPARED,
                      workspace=self.ws, out=self.o, final_out=self.final)
        if rec:
            rec(2)
        return self.o

    def final_of_docs(self):
        return self.final.index_select(0, self.last)


def split_forward_packed(q, k, v, g, beta, scale=None, *, doc_offsets, seg_offsets, use_exp2=False,
                         initial_state=None, o_dtype=torch.float32, ext_only_launch=True):
    """Packed documents (TND, q/k/v [T,H,K]) split into segments on one GPU
    (SplitPlan over the pieces of gdn_split_meta). initial_state:
    [n_docs,H,K,V] or None. Returns (o, final state of every document
    [n_docs,H,K,V], S_in [n_pieces,H,K,V])."""
    if k.dim() != 3:
        raise ValueError("packed input must be [T, H, K]")
    pieces, pdoc, _ = gdn_split_meta(doc_offsets, seg_offsets)
    plan = SplitPlan(q, k, v, g, beta, scale, pieces=pieces, piece_doc=pdoc, use_exp2=use_exp2,
                     with_s0=initial_state is not None, o_dtype=o_dtype, ext_only_launch=ext_only_launch)
    o = plan(q, k, v, g, beta, initial_state)
    return o, plan.final_of_docs(), plan.S_in


def split_plan_rows(q, k, v, g, beta, scale=None, *, seg, use_exp2=False, with_s0=False,
                    o_dtype=torch.float32, ext_only_launch=True):
    """SplitPlan of BSND rows, each cut at the in-row offsets seg."""
    B, T = k.shape[0], k.shape[1]
    n_seg = len(seg) - 1
    return SplitPlan(q, k, v, g, beta, scale, pieces=segment_offsets(B, T, seg),
                     piece_doc=[b for b in range(B) for _ in range(n_seg)], use_exp2=use_exp2,
                     with_s0=with_s0, o_dtype=o_dtype, ext_only_launch=ext_only_launch)


def split_forward(q, k, v, g, beta, scale=None, *, seg, use_exp2=False, initial_state=None,
                  o_dtype=torch.float32, ext_only_launch=True):
    """Sequence split of BSND rows on one GPU: the summaries that something
    consumes, their merge, then the correction pass (the forward of every
    segment from its true entry state, reusing the preparation). seg: in-row
    segment offsets [0, ..., T]. Returns (o, S_final [B,H,K,V], S_init
    [B*n_seg,H,K,V])."""
    plan = split_plan_rows(q, k, v, g, beta, scale, seg=seg, use_exp2=use_exp2,
                           with_s0=initial_state is not None, o_dtype=o_dtype, ext_only_launch=ext_only_launch)
    o = plan(q, k, v, g, beta, initial_state)
    return o, plan.final_of_docs(), plan.S_in


