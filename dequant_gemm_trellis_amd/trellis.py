"""ctypes binding over libtrellis.so (include/trellis.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI. PyTorch supplies device memory and the stream.
Importing this module raises ImportError when the library is not built; there
is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

from .synth import Shape

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtrellis.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
        "(hipcc --offload-arch=gfx950)")
_lib = C.CDLL(LIB_PATH)

OK = 0
ERR_NULL = -1
ERR_GEOMETRY = -2
ERR_ALIGN = -3
ERR_LUT = -4
ERR_WORKSPACE = -5
ERR_HIP = -6
ERR_OVERLAP = -7
OP_GEMV = 0
OP_GEMV_SCATTER = 1
OP_PREFILL = 2
MAX_M = 32

# Every function the headers under include/ declare, for the export check.
EXPORTED = ("trellis_lut_upload", "trellis_gemv", "trellis_gemv_dual", "trellis_gemv_scatter",
            "trellis_prefill", "trellis_prefill_dual", "trellis_gate_up_swiglu",
            "trellis_gemv_scatter_static", "trellis_static_scratch_bytes", "trellis_workspace_bytes",
            "trellis_expand", "trellis_repack", "trellis_strerror", "trellis_gather_probe",
            "trellis_gather_probe_values", "trellis_gather_probe_out_floats")
PROBE_PAIR_B64, PROBE_COPIES8_B32, PROBE_SINGLE_B32 = 0, 1, 2


class Geometry(C.Structure):
    _fields_ = [("axis", C.c_int32), ("T", C.c_int32), ("L", C.c_int32), ("k", C.c_int32),
                ("in_features", C.c_int32), ("out_features", C.c_int32),
                ("block_interleave", C.c_int32)]

    @classmethod
    def of(cls, shape: Shape) -> "Geometry":
        return cls(shape.axis, shape.T, shape.L, shape.k, shape.in_features, shape.out_features,
                   shape.block_interleave)


_vp = C.c_void_p
_GP = C.POINTER(Geometry)
_lib.trellis_lut_upload.argtypes = [_vp, C.c_int32, _vp, _vp]
_lib.trellis_gemv.argtypes = [_vp, _vp, _vp, _vp, _GP, _vp, _vp]
_lib.trellis_gemv_dual.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _GP, _vp]
_lib.trellis_gemv_scatter.argtypes = [_vp, _vp, _vp, _vp, _GP, _vp, C.c_size_t, _vp, _vp]
_lib.trellis_prefill.argtypes = [_vp, C.c_int32, _vp, _vp, _vp, _GP, _vp, C.c_size_t, _vp, _vp]
_lib.trellis_prefill_dual.argtypes = [_vp, C.c_int32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _GP,
                                      _vp]
_lib.trellis_gate_up_swiglu.argtypes = [_vp, C.c_int32, _vp, _vp, _vp, _vp, _vp, _vp, _GP, _vp,
                                        _vp]
_lib.trellis_gemv_scatter_static.argtypes = [_vp, _vp, _vp, _vp, _GP, _vp, _vp]
_lib.trellis_static_scratch_bytes.argtypes = []
_lib.trellis_static_scratch_bytes.restype = C.c_size_t
_lib.trellis_workspace_bytes.argtypes = [_GP, C.c_int32, C.c_int32]
_lib.trellis_workspace_bytes.restype = C.c_size_t
_lib.trellis_expand.argtypes = [_vp, _vp, _vp, _GP, _vp, _vp]
_lib.trellis_repack.argtypes = [_vp, _vp, _GP, C.c_int32, _vp]
_lib.trellis_strerror.argtypes = [C.c_int]
_lib.trellis_strerror.restype = C.c_char_p
_lib.trellis_gather_probe.argtypes = [C.c_int32, C.c_int32, _vp, C.c_size_t, _vp]
_lib.trellis_gather_probe.restype = C.c_int
_lib.trellis_gather_probe_values.argtypes = [C.c_int32, C.c_int32]
_lib.trellis_gather_probe_values.restype = C.c_uint64
_lib.trellis_gather_probe_out_floats.argtypes = []
_lib.trellis_gather_probe_out_floats.restype = C.c_size_t
for _f in ("trellis_lut_upload", "trellis_gemv", "trellis_gemv_dual", "trellis_gemv_scatter",
           "trellis_prefill", "trellis_prefill_dual", "trellis_gate_up_swiglu", "trellis_expand",
           "trellis_repack", "trellis_gemv_scatter_static"):
    getattr(_lib, _f).restype = C.c_int


class TrellisError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {strerror(status)} (status {status})")
        self.status = status


def strerror(status: int) -> str:
    return _lib.trellis_strerror(status).decode()


def raw() -> C.CDLL:
    """The loaded library, for callers that marshal their own arguments."""
    return _lib


def _check(fn: str, status: int) -> None:
    if status != OK:
        raise TrellisError(fn, status)


def _dev(t: torch.Tensor | None) -> _vp:
    if t is None:
        return _vp(0)
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("device tensors must be contiguous and on the GPU")
    return _vp(t.data_ptr())


def _stream(stream: torch.cuda.Stream | None) -> _vp:
    s = stream if stream is not None else torch.cuda.current_stream()
    return _vp(s.cuda_stream)


def _geom(g: Shape | Geometry) -> Geometry:
    return g if isinstance(g, Geometry) else Geometry.of(g)


def workspace_bytes(g: Shape | Geometry, M: int, op: int) -> int:
    n = _lib.trellis_workspace_bytes(C.byref(_geom(g)), M, op)
    if n == C.c_size_t(-1).value:
        raise TrellisError("trellis_workspace_bytes", ERR_GEOMETRY)
    return n


def lut_upload(host_lut, dev_lut: torch.Tensor | None = None, device=None,
               stream: torch.cuda.Stream | None = None) -> torch.Tensor:
    import numpy as np

    h = np.ascontiguousarray(host_lut, dtype=np.float32)
    if dev_lut is None:
        dev_lut = torch.empty(h.size, dtype=torch.float32, device=device or "cuda")
    s = stream if stream is not None else torch.cuda.current_stream()
    _check("trellis_lut_upload", _lib.trellis_lut_upload(
        _vp(h.ctypes.data), h.size, _dev(dev_lut), _vp(s.cuda_stream)))
    s.synchronize()  # the copy is stream-ordered and h is this call's own array
    return dev_lut


def gemv(x, codes, scales, lut, g, y=None, stream=None) -> torch.Tensor:
    geom = _geom(g)
    if y is None:
        y = torch.empty(geom.out_features, dtype=torch.bfloat16, device=x.device)
    _check("trellis_gemv", _lib.trellis_gemv(_dev(x), _dev(codes), _dev(scales), _dev(lut),
                                             C.byref(geom), _dev(y), _stream(stream)))
    return y


def gemv_dual(x, a, b, g, y_a=None, y_b=None, stream=None) -> tuple[torch.Tensor, torch.Tensor]:
    """Two axis-1 GEMVs over the same x in one launch; a and b are
    (codes, scales, lut) triples of the same geometry g."""
    geom = _geom(g)
    if y_a is None:
        y_a = torch.empty(geom.out_features, dtype=torch.bfloat16, device=x.device)
    if y_b is None:
        y_b = torch.empty(geom.out_features, dtype=torch.bfloat16, device=x.device)
    (ca, sa, la), (cb, sb, lb) = a, b
    _check("trellis_gemv_dual", _lib.trellis_gemv_dual(
        _dev(x), _dev(ca), _dev(sa), _dev(la), _dev(y_a), _dev(cb), _dev(sb), _dev(lb),
        _dev(y_b), C.byref(geom), _stream(stream)))
    return y_a, y_b


def gemv_scatter(x, codes, scales, lut, g, workspace=None, y=None, stream=None) -> torch.Tensor:
    geom = _geom(g)
    if y is None:
        y = torch.empty(geom.out_features, dtype=torch.bfloat16, device=x.device)
    if workspace is None:
        workspace = torch.empty(workspace_bytes(geom, 1, OP_GEMV_SCATTER) // 4,
                                dtype=torch.float32, device=x.device)
    _check("trellis_gemv_scatter", _lib.trellis_gemv_scatter(
        _dev(x), _dev(codes), _dev(scales), _dev(lut), C.byref(geom), _dev(workspace),
        workspace.numel() * workspace.element_size(), _dev(y), _stream(stream)))
    return y


def gemv_scatter_static(x, codes, scales, lut, g, y=None, stream=None) -> torch.Tensor:
    """trellis_gemv_scatter with its partials in the library's static device
    array (no workspace); calls overlapping on one device race."""
    geom = _geom(g)
    if y is None:
        y = torch.empty(geom.out_features, dtype=torch.bfloat16, device=x.device)
    _check("trellis_gemv_scatter_static", _lib.trellis_gemv_scatter_static(
        _dev(x), _dev(codes), _dev(scales), _dev(lut), C.byref(geom), _dev(y), _stream(stream)))
    return y


def static_scratch_bytes() -> int:
    return int(_lib.trellis_static_scratch_bytes())


def prefill(x, codes, scales, lut, g, workspace=None, y=None, stream=None,
            balanced=True) -> torch.Tensor:
    """Without a workspace one of workspace_bytes is allocated. At axis 1 the
    workspace is optional: balanced=False passes none (the plan whose last
    16-row group of each workgroup may be partly empty)."""
    geom = _geom(g)
    M = x.shape[0] if x.dim() == 2 else 1
    if y is None:
        y = torch.empty((M, geom.out_features), dtype=torch.bfloat16, device=x.device)
    if geom.axis == 1 and not balanced:
        workspace, nbytes = None, 0
    else:
        nbytes = workspace_bytes(geom, M, OP_PREFILL)
    if workspace is None and nbytes:
        workspace = torch.empty(nbytes // 4, dtype=torch.float32, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("trellis_prefill", _lib.trellis_prefill(
        _dev(x), M, _dev(codes), _dev(scales), _dev(lut), C.byref(geom), _dev(workspace),
        ws_bytes, _dev(y), _stream(stream)))
    return y


def prefill_dual(x, a, b, g, y_a=None, y_b=None, stream=None) -> tuple[torch.Tensor, torch.Tensor]:
    """Two axis-1 prefills over the same x [M][in]; a and b are (codes,
    scales, lut) triples of the same geometry g."""
    geom = _geom(g)
    M = x.shape[0] if x.dim() == 2 else 1
    if y_a is None:
        y_a = torch.empty((M, geom.out_features), dtype=torch.bfloat16, device=x.device)
    if y_b is None:
        y_b = torch.empty((M, geom.out_features), dtype=torch.bfloat16, device=x.device)
    (ca, sa, la), (cb, sb, lb) = a, b
    _check("trellis_prefill_dual", _lib.trellis_prefill_dual(
        _dev(x), M, _dev(ca), _dev(sa), _dev(la), _dev(y_a), _dev(cb), _dev(sb), _dev(lb),
        _dev(y_b), C.byref(geom), _stream(stream)))
    return y_a, y_b


def gate_up_swiglu(x, gate, up, g, h=None, stream=None) -> torch.Tensor:
    """h = bf16(silu(x Wg^T) * (x Wu^T)) for x [M][in] (or [in] for M = 1);
    gate and up are (codes, scales, lut) triples of the same axis-1 geometry
    g. Returns h, [M][out] (or [out] for a 1-D x)."""
    geom = _geom(g)
    M = x.shape[0] if x.dim() == 2 else 1
    if h is None:
        shape = (M, geom.out_features) if x.dim() == 2 else (geom.out_features,)
        h = torch.empty(shape, dtype=torch.bfloat16, device=x.device)
    (cg, sg, lg), (cu, su, lu) = gate, up
    _check("trellis_gate_up_swiglu", _lib.trellis_gate_up_swiglu(
        _dev(x), M, _dev(cg), _dev(sg), _dev(lg), _dev(cu), _dev(su), _dev(lu), C.byref(geom),
        _dev(h), _stream(stream)))
    return h


def expand(codes, scales, lut, g, w=None, stream=None) -> torch.Tensor:
    geom = _geom(g)
    rows = geom.out_features if geom.axis == 1 else geom.in_features
    cols = geom.in_features if geom.axis == 1 else geom.out_features
    if w is None:
        w = torch.empty((rows, cols), dtype=torch.bfloat16, device=codes.device)
    _check("trellis_expand", _lib.trellis_expand(_dev(codes), _dev(scales), _dev(lut),
                                                 C.byref(geom), _dev(w), _stream(stream)))
    return w


def repack(codes, g, to_block_interleave: int, out=None, stream=None) -> torch.Tensor:
    """Rewrite `codes` (in the layout g's block_interleave names) into layout
    `to_block_interleave` (0 row-major, 2 block pairs); returns `out`."""
    geom = _geom(g)
    if out is None:
        out = torch.empty_like(codes)
    _check("trellis_repack", _lib.trellis_repack(_dev(codes), _dev(out), C.byref(geom),
                                                 to_block_interleave, _stream(stream)))
    return out


def gather_probe(kind: int, rounds: int, out: torch.Tensor, stream=None) -> int:
    """Enqueue one launch of the LDS codebook-gather probe (trellis_probe.h);
    returns the number of decoded-weight values its timed loop reads."""
    status = _lib.trellis_gather_probe(kind, rounds, _dev(out), out.numel(), _stream(stream))
    if status != OK:
        raise RuntimeError(f"trellis_gather_probe: status {status}")
    return int(_lib.trellis_gather_probe_values(kind, rounds))


def gather_probe_out_floats() -> int:
    return int(_lib.trellis_gather_probe_out_floats())
