"""Python binding of libmoesq (ctypes).

Argument marshalling only: every function here checks tensor placement,
dtype and contiguity, passes raw device pointers and the current HIP stream
to the C ABI in include/moesq.h, and raises MoesqError on a non-zero status.
All compute runs in the library's HIP kernels.  Torch supplies device memory
and streams; the convenience helpers at the bottom allocate outputs with
torch and call the same entry points.

The library must be built first (python -m sparse_fp4_expert_amd.build);
importing this module without it raises ImportError.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoesq.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is missing: build it with `python -m sparse_fp4_expert_amd.build`")
_lib = ctypes.CDLL(_LIB_PATH)

OK, ERR_NULL, ERR_SHAPE, ERR_WORKSPACE, ERR_LAYOUT, ERR_HIP, ERR_ARG = 0, -1, -2, -3, -4, -5, -6
EPI_NONE, EPI_SWIGLU = 0, 1
# OR-ed into the epilogue of the gather and fused-routing GEMMs: rows come out
# in flat order (row r stored at y[perm[r]]), the scatter fused into the GEMM.
OUT_FLAT = 0x100
LAYOUT_CANONICAL, LAYOUT_TILED, LAYOUT_PAIRED, LAYOUT_PAIRED_TILED = 0, 1, 2, 3
PAIRED_LAYOUTS = (LAYOUT_PAIRED, LAYOUT_PAIRED_TILED)
MAX_EXPERTS = 1024

_vp, _i32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t


class WeightsDesc(ctypes.Structure):
    """moesq_weights_t."""
    _fields_ = [("values", _vp), ("masks", _vp), ("scales", _vp), ("global_scale", _vp),
                ("E", _i32), ("N", _i32), ("K", _i32), ("layout", _i32)]


class Act4Desc(ctypes.Structure):
    """moesq_act4_t."""
    _fields_ = [("codes", _vp), ("scales", _vp), ("row_scale", _vp), ("rows", _i32), ("K", _i32)]


def _sig(name, restype, *argtypes):
    f = getattr(_lib, name)
    f.restype = restype
    f.argtypes = list(argtypes)
    return f


_route = _sig("moesq_route", _i32, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp)
_route_ws = _sig("moesq_route_workspace_bytes", _sz, _i32, _i32, _i32)
_route_noalloc = _sig("moesq_route_noalloc", _i32, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp)
_permute = _sig("moesq_permute", _i32, _vp, _vp, _i32, _i32, _i32, _vp, _vp)
_spgemm = _sig("moesq_grouped_spgemm", _i32, _vp, _vp, _i32, ctypes.POINTER(WeightsDesc), _i32,
               _vp, _vp, _sz, _vp)
_spgemm_ws = _sig("moesq_spgemm_workspace_bytes", _sz, _i32, ctypes.POINTER(WeightsDesc))
_spgemm_gather = _sig("moesq_grouped_spgemm_gather", _i32, _vp, _vp, _i32, _i32, _vp,
                      ctypes.POINTER(WeightsDesc), _i32, _vp, _vp, _sz, _vp)
_route_spgemm = _sig("moesq_route_grouped_spgemm", _i32, _vp, _vp, _i32, _i32,
                     ctypes.POINTER(WeightsDesc), _i32, _vp, _vp, _vp, _vp, _vp)
_quant_act = _sig("moesq_quantize_activations", _i32, _vp, _i32, _i32, _vp, _vp, _vp, _vp)
_spgemm_act4 = _sig("moesq_grouped_spgemm_act4", _i32, ctypes.POINTER(Act4Desc), _vp, _i32, _i32,
                    _vp, _i32, ctypes.POINTER(WeightsDesc), _i32, _vp, _vp)
_unpermute = _sig("moesq_unpermute", _i32, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp)
_pack = _sig("moesq_pack_weights", _i32, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp)
_pack_paired = _sig("moesq_pack_weights_paired", _i32, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp,
                    _vp)
_decode = _sig("moesq_decode_weights", _i32, ctypes.POINTER(WeightsDesc), _i32, _vp, _vp)
_tile = _sig("moesq_tile_weights", _i32, ctypes.POINTER(WeightsDesc), _vp, _vp, _vp, _vp)
_validate = _sig("moesq_validate", _i32, _vp, _i32, _i32, _i32, _vp, ctypes.POINTER(WeightsDesc),
                 ctypes.POINTER(ctypes.c_uint64), _vp)
_stream_read = _sig("moesq_stream_read", _i32, _vp, _sz, _vp, _vp)
_status_string = _sig("moesq_status_string", ctypes.c_char_p, _i32)
_last_error = _sig("moesq_last_error", ctypes.c_char_p)
_version = _sig("moesq_version", _i32)

EXPORTED = ["moesq_route", "moesq_route_workspace_bytes", "moesq_route_noalloc",
            "moesq_permute",
            "moesq_grouped_spgemm", "moesq_spgemm_workspace_bytes",
            "moesq_grouped_spgemm_gather", "moesq_route_grouped_spgemm", "moesq_unpermute",
            "moesq_quantize_activations", "moesq_grouped_spgemm_act4",
            "moesq_pack_weights", "moesq_pack_weights_paired", "moesq_tile_weights",
            "moesq_decode_weights",
            "moesq_validate", "moesq_stream_read", "moesq_status_string",
            "moesq_last_error", "moesq_version"]


class MoesqError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{_status_string(status).decode()} ({detail})")


def _check(st: int):
    if st != OK:
        raise MoesqError(st, _last_error().decode())


def version() -> int:
    return _version()


def _ptr(t, dtype, name, allow_none=False):
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.numel() and not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr() if t.numel() else None


def _sizes(*checks):
    """Raises ValueError unless every (tensor, elements, name) matches: the
    library sizes its loads and stores from the shape arguments, so a tensor
    of another size would be read or written out of bounds on the device.
    A None tensor is skipped (the C call decides whether it may be NULL)."""
    for t, n, name in checks:
        if t is None or not isinstance(t, torch.Tensor):
            continue
        if t.numel() != n:
            raise ValueError(f"{name} has {t.numel()} elements ({tuple(t.shape)}), "
                             f"the shape arguments need {n}")


def _out_cols(w, epilogue: int) -> int:
    return w.N // 2 if (epilogue & ~OUT_FLAT) == EPI_SWIGLU else w.N


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


class Weights:
    """Device tensors of compressed experts.

    values uint8 [E, N, K/4], masks uint8 [E, N, K/8] (paired layouts: the
    pattern bytes, [E, N, K/16]), scales uint8 [E, N, K/32], global_scale
    float32 [E].  `layout` is one of the LAYOUT_* constants; a tiled layout has
    the shapes of its canonical one, bytes arranged as include/moesq.h
    describes."""

    def __init__(self, values, masks, scales, global_scale, layout=LAYOUT_CANONICAL):
        E, N, K4 = values.shape
        self.E, self.N, self.K = int(E), int(N), int(K4) * 4
        meta = self.K // 16 if layout in PAIRED_LAYOUTS else self.K // 8
        for t, shape, name in [(masks, (E, N, meta), "masks"),
                               (scales, (E, N, self.K // 32), "scales"),
                               (global_scale, (E,), "global_scale")]:
            if tuple(t.shape) != shape:
                raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")
        self.values, self.masks, self.scales, self.global_scale = values, masks, scales, global_scale
        self.layout = layout
        self.desc = WeightsDesc(_ptr(values, torch.uint8, "values"), _ptr(masks, torch.uint8, "masks"),
                                _ptr(scales, torch.uint8, "scales"),
                                _ptr(global_scale, torch.float32, "global_scale"),
                                self.E, self.N, self.K, layout)

    @property
    def nbytes(self) -> int:
        return self.values.numel() + self.masks.numel() + self.scales.numel() + 4 * self.E

    @property
    def paired(self) -> bool:
        return self.layout in PAIRED_LAYOUTS

    def expert_nbytes(self) -> int:
        """Bytes of one expert: 13/32 per weight (4:8 masks) or 11/32 (paired
        pattern indices: 2.75 bits per weight), plus the fp32 global scale."""
        return self.N * self.K * (11 if self.paired else 13) // 32 + 4

    @staticmethod
    def empty(E: int, N: int, K: int, device="cuda", layout=LAYOUT_CANONICAL):
        u8 = dict(dtype=torch.uint8, device=device)
        meta = K // 16 if layout in PAIRED_LAYOUTS else K // 8
        return Weights(torch.empty(E, N, K // 4, **u8), torch.empty(E, N, meta, **u8),
                       torch.empty(E, N, K // 32, **u8),
                       torch.empty(E, dtype=torch.float32, device=device), layout)


class Act4:
    """Device tensors of NVFP4 activation rows (W4A4): codes uint8 [rows, K/2],
    scales uint8 [rows, K/32], row_scale float32 [rows]."""

    def __init__(self, codes, scales, row_scale):
        rows, K2 = codes.shape
        self.rows, self.K = int(rows), int(K2) * 2
        for t, shape, name in [(scales, (rows, self.K // 32), "scales"), (row_scale, (rows,), "row_scale")]:
            if tuple(t.shape) != shape:
                raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")
        self.codes, self.scales, self.row_scale = codes, scales, row_scale
        self.desc = Act4Desc(_ptr(codes, torch.uint8, "codes", True),
                             _ptr(scales, torch.uint8, "scales", True),
                             _ptr(row_scale, torch.float32, "row_scale", True), self.rows, self.K)

    @staticmethod
    def empty(rows: int, K: int, device="cuda"):
        u8 = dict(dtype=torch.uint8, device=device)
        return Act4(torch.empty(rows, K // 2, **u8), torch.empty(rows, K // 32, **u8),
                    torch.empty(rows, dtype=torch.float32, device=device))


# ------------------------------------------------------------ C-ABI mirrors

def moesq_route(topk_ids, T: int, k: int, E: int, expert_offsets, perm, inv_perm,
                ws=None, stream=None):
    _sizes((topk_ids, T * k, "topk_ids"), (expert_offsets, E + 1, "expert_offsets"),
           (perm, T * k, "perm"), (inv_perm, T * k, "inv_perm"))
    _check(_route(_ptr(topk_ids, torch.int32, "topk_ids"), T, k, E,
                  _ptr(expert_offsets, torch.int32, "expert_offsets"),
                  _ptr(perm, torch.int32, "perm"), _ptr(inv_perm, torch.int32, "inv_perm"),
                  _ptr(ws, torch.uint8, "ws", True), 0 if ws is None else ws.numel(),
                  _stream(stream)))


def moesq_route_workspace_bytes(T: int, k: int, E: int) -> int:
    return int(_route_ws(T, k, E))


ROUTE_SCRATCH_BYTES = 4 << 20


def moesq_route_noalloc(topk_ids, T: int, k: int, E: int, expert_offsets, perm, inv_perm,
                        stream=None):
    """moesq_route without a workspace: the block counts go to the library's
    own device scratch (ROUTE_SCRATCH_BYTES per device; calls that overlap on
    one device race)."""
    _sizes((topk_ids, T * k, "topk_ids"), (expert_offsets, E + 1, "expert_offsets"),
           (perm, T * k, "perm"), (inv_perm, T * k, "inv_perm"))
    _check(_route_noalloc(_ptr(topk_ids, torch.int32, "topk_ids"), T, k, E,
                          _ptr(expert_offsets, torch.int32, "expert_offsets"),
                          _ptr(perm, torch.int32, "perm"), _ptr(inv_perm, torch.int32, "inv_perm"),
                          _stream(stream)))


def moesq_permute(x, perm, T: int, k: int, K: int, x_routed, stream=None):
    _sizes((x, T * K, "x"), (perm, T * k, "perm"), (x_routed, T * k * K, "x_routed"))
    _check(_permute(_ptr(x, torch.bfloat16, "x"), _ptr(perm, torch.int32, "perm"), T, k, K,
                    _ptr(x_routed, torch.bfloat16, "x_routed"), _stream(stream)))


def moesq_grouped_spgemm(x_routed, expert_offsets, M: int, w: Weights, epilogue: int, y,
                         ws=None, stream=None):
    _sizes((x_routed, M * w.K, "x_routed"), (expert_offsets, w.E + 1, "expert_offsets"),
           (y, M * _out_cols(w, epilogue), "y"))
    _check(_spgemm(_ptr(x_routed, torch.bfloat16, "x_routed"),
                   _ptr(expert_offsets, torch.int32, "expert_offsets"), M,
                   ctypes.byref(w.desc), epilogue, _ptr(y, torch.bfloat16, "y"),
                   _ptr(ws, torch.uint8, "ws", True), 0 if ws is None else ws.numel(),
                   _stream(stream)))


def moesq_grouped_spgemm_gather(x, perm, T: int, k: int, expert_offsets, w: Weights,
                                epilogue: int, y, ws=None, stream=None):
    _sizes((x, T * w.K, "x"), (perm, T * k, "perm"), (expert_offsets, w.E + 1, "expert_offsets"),
           (y, T * k * _out_cols(w, epilogue), "y"))
    _check(_spgemm_gather(_ptr(x, torch.bfloat16, "x"), _ptr(perm, torch.int32, "perm"), T, k,
                          _ptr(expert_offsets, torch.int32, "expert_offsets"), ctypes.byref(w.desc),
                          epilogue, _ptr(y, torch.bfloat16, "y"), _ptr(ws, torch.uint8, "ws", True),
                          0 if ws is None else ws.numel(), _stream(stream)))


def moesq_route_grouped_spgemm(topk_ids, x, T: int, k: int, w: Weights, epilogue: int, y,
                               expert_offsets, perm, inv_perm, stream=None):
    _sizes((topk_ids, T * k, "topk_ids"), (x, T * w.K, "x"),
           (y, T * k * _out_cols(w, epilogue), "y"), (expert_offsets, w.E + 1, "expert_offsets"),
           (perm, T * k, "perm"), (inv_perm, T * k, "inv_perm"))
    _check(_route_spgemm(_ptr(topk_ids, torch.int32, "topk_ids", True), _ptr(x, torch.bfloat16, "x", True),
                         T, k, ctypes.byref(w.desc), epilogue, _ptr(y, torch.bfloat16, "y", True),
                         _ptr(expert_offsets, torch.int32, "expert_offsets"),
                         _ptr(perm, torch.int32, "perm", True), _ptr(inv_perm, torch.int32, "inv_perm", True),
                         _stream(stream)))


def moesq_spgemm_workspace_bytes(M: int, w: Weights) -> int:
    return int(_spgemm_ws(M, ctypes.byref(w.desc)))


def moesq_unpermute(y, inv_perm, topk_weights, T: int, k: int, N: int, out, stream=None):
    rows = T if topk_weights is not None else T * k
    _sizes((y, T * k * N, "y"), (inv_perm, T * k, "inv_perm"),
           (topk_weights, T * k, "topk_weights"), (out, rows * N, "out"))
    _check(_unpermute(_ptr(y, torch.bfloat16, "y"), _ptr(inv_perm, torch.int32, "inv_perm"),
                      _ptr(topk_weights, torch.float32, "topk_weights", True), T, k, N,
                      _ptr(out, torch.bfloat16, "out"), _stream(stream)))


def moesq_quantize_activations(x, T: int, K: int, codes, scales, row_scale, stream=None):
    _sizes((x, T * K, "x"), (codes, T * K // 2, "codes"), (scales, T * K // 32, "scales"),
           (row_scale, T, "row_scale"))
    _check(_quant_act(_ptr(x, torch.bfloat16, "x", True), T, K,
                      _ptr(codes, torch.uint8, "codes", True), _ptr(scales, torch.uint8, "scales", True),
                      _ptr(row_scale, torch.float32, "row_scale", True), _stream(stream)))


def moesq_grouped_spgemm_act4(x: Act4, perm, T: int, k: int, expert_offsets, M: int, w: Weights,
                              epilogue: int, y, stream=None):
    _sizes((perm, M, "perm"), (expert_offsets, w.E + 1, "expert_offsets"),
           (y, M * _out_cols(w, epilogue), "y"))
    if x.K != w.K:
        raise ValueError(f"activations have K = {x.K}, the weights {w.K}")
    if x.rows != (T if perm is not None else M):
        raise ValueError(f"activations have {x.rows} rows, need {T if perm is not None else M}")
    _check(_spgemm_act4(ctypes.byref(x.desc), _ptr(perm, torch.int32, "perm", True), T, k,
                        _ptr(expert_offsets, torch.int32, "expert_offsets"), M,
                        ctypes.byref(w.desc), epilogue, _ptr(y, torch.bfloat16, "y", True),
                        _stream(stream)))


def moesq_pack_weights(dense, E: int, N: int, K: int, values, masks, scales, global_scale,
                       stream=None):
    _sizes((dense, E * N * K, "dense"), (values, E * N * K // 4, "values"),
           (masks, E * N * K // 8, "masks"), (scales, E * N * K // 32, "scales"),
           (global_scale, E, "global_scale"))
    _check(_pack(_ptr(dense, torch.float32, "dense"), E, N, K, _ptr(values, torch.uint8, "values"),
                 _ptr(masks, torch.uint8, "masks"), _ptr(scales, torch.uint8, "scales"),
                 _ptr(global_scale, torch.float32, "global_scale"), _stream(stream)))


def moesq_pack_weights_paired(dense, E: int, N: int, K: int, values, patterns, scales,
                              global_scale, stream=None):
    _sizes((dense, E * N * K, "dense"), (values, E * N * K // 4, "values"),
           (patterns, E * N * K // 16, "patterns"), (scales, E * N * K // 32, "scales"),
           (global_scale, E, "global_scale"))
    _check(_pack_paired(_ptr(dense, torch.float32, "dense"), E, N, K,
                        _ptr(values, torch.uint8, "values"), _ptr(patterns, torch.uint8, "patterns"),
                        _ptr(scales, torch.uint8, "scales"),
                        _ptr(global_scale, torch.float32, "global_scale"), _stream(stream)))


def moesq_tile_weights(src: Weights, values, masks, scales, stream=None):
    _sizes((values, src.values.numel(), "values"), (masks, src.masks.numel(), "masks"),
           (scales, src.scales.numel(), "scales"))
    _check(_tile(ctypes.byref(src.desc), _ptr(values, torch.uint8, "values"),
                 _ptr(masks, torch.uint8, "masks"), _ptr(scales, torch.uint8, "scales"),
                 _stream(stream)))


def moesq_decode_weights(w: Weights, expert: int, dense, stream=None):
    _sizes((dense, w.N * w.K, "dense"))
    _check(_decode(ctypes.byref(w.desc), expert, _ptr(dense, torch.bfloat16, "dense"),
                   _stream(stream)))


VALIDATE_CHECKS = ("ids", "offsets", "masks", "scales", "global_scales")


def moesq_validate(topk_ids=None, T: int = 0, k: int = 1, E: int = 1, expert_offsets=None,
                   w: Weights | None = None, stream=None) -> dict:
    """Debug check of the caller contracts (synchronises).  Returns the
    violation count of each check; a failed check is not an exception (the
    counts say which), bad sizes and HIP failures are."""
    _sizes((topk_ids, T * k, "topk_ids"), (expert_offsets, E + 1, "expert_offsets"))
    counts = (ctypes.c_uint64 * len(VALIDATE_CHECKS))()
    st = _validate(_ptr(topk_ids, torch.int32, "topk_ids", True), T, k, E,
                   _ptr(expert_offsets, torch.int32, "expert_offsets", True),
                   None if w is None else ctypes.byref(w.desc), counts, _stream(stream))
    if st != ERR_ARG:
        _check(st)
    return dict(zip(VALIDATE_CHECKS, (int(c) for c in counts)))


def moesq_stream_read(buf, sink, stream=None):
    """Measurement utility: one streaming read of the uint8 device tensor
    `buf` (the practical HBM read ceiling); `sink` is a 1-element int32 tensor."""
    _check(_stream_read(_ptr(buf, torch.uint8, "buf"), buf.numel(),
                        _ptr(sink, torch.int32, "sink"), _stream(stream)))


# ------------------------------------------------------------ helpers (allocate with torch)

def route(topk_ids, E: int, k: int, stream=None):
    """Returns (expert_offsets [E+1], perm [M], inv_perm [M]) as int32 device tensors."""
    M = topk_ids.numel()
    if M % k:
        raise ValueError(f"topk_ids has {M} entries, not a multiple of k = {k}")
    dev = topk_ids.device
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(M, dtype=torch.int32, device=dev)
    inv = torch.empty(M, dtype=torch.int32, device=dev)
    nws = moesq_route_workspace_bytes(M // k, k, E)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None
    moesq_route(topk_ids, M // k, k, E, off, perm, inv, ws, stream)
    return off, perm, inv


def permute(x, perm, k: int, stream=None):
    if x.dim() != 2:
        raise ValueError(f"x must be [T, K], got {tuple(x.shape)}")
    T, K = x.shape
    out = torch.empty(T * k, K, dtype=torch.bfloat16, device=x.device)
    moesq_permute(x, perm, T, k, K, out, stream)
    return out


def grouped_spgemm(x_routed, expert_offsets, w: Weights, epilogue: int = EPI_NONE, out=None,
                   stream=None):
    if x_routed.dim() != 2 or x_routed.shape[1] != w.K:
        raise ValueError(f"x_routed must be [M, {w.K}], got {tuple(x_routed.shape)}")
    M = x_routed.shape[0]
    n_out = _out_cols(w, epilogue)
    if out is None:
        out = torch.empty(M, n_out, dtype=torch.bfloat16, device=x_routed.device)
    elif tuple(out.shape) != (M, n_out):
        raise ValueError(f"out must be [{M}, {n_out}], got {tuple(out.shape)}")
    moesq_grouped_spgemm(x_routed, expert_offsets, M, w, epilogue, out, None, stream)
    return out


def grouped_spgemm_gather(x, perm, k: int, expert_offsets, w: Weights, epilogue: int = EPI_NONE,
                          out=None, stream=None):
    """Dispatch fused into the GEMM: routed row r reads token perm[r] // k of x
    (with OUT_FLAT in `epilogue`, row r is stored at out[perm[r]])."""
    if x.dim() != 2 or x.shape[1] != w.K:
        raise ValueError(f"x must be [T, {w.K}], got {tuple(x.shape)}")
    T = x.shape[0]
    n_out = _out_cols(w, epilogue)
    if out is None:
        out = torch.empty(T * k, n_out, dtype=torch.bfloat16, device=x.device)
    elif tuple(out.shape) != (T * k, n_out):
        raise ValueError(f"out must be [{T * k}, {n_out}], got {tuple(out.shape)}")
    moesq_grouped_spgemm_gather(x, perm, T, k, expert_offsets, w, epilogue, out, None, stream)
    return out


def route_grouped_spgemm(topk_ids, x, k: int, w: Weights, epilogue: int = EPI_NONE, out=None,
                         stream=None):
    """Routing, dispatch and GEMM of a decode batch in one launch.  Returns
    (out [T*k, N or N/2], expert_offsets [E+1], perm [T*k], inv_perm [T*k])."""
    if x.dim() != 2 or x.shape[1] != w.K:
        raise ValueError(f"x must be [T, {w.K}], got {tuple(x.shape)}")
    T = x.shape[0]
    dev = x.device
    n_out = _out_cols(w, epilogue)
    if out is None:
        out = torch.empty(T * k, n_out, dtype=torch.bfloat16, device=dev)
    elif tuple(out.shape) != (T * k, n_out):
        raise ValueError(f"out must be [{T * k}, {n_out}], got {tuple(out.shape)}")
    off = torch.empty(w.E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(T * k, dtype=torch.int32, device=dev)
    inv = torch.empty(T * k, dtype=torch.int32, device=dev)
    moesq_route_grouped_spgemm(topk_ids, x, T, k, w, epilogue, out, off, perm, inv, stream)
    return out, off, perm, inv


def quantize_activations(x, stream=None) -> Act4:
    """bf16 [T, K] on the GPU -> its NVFP4 rows (Act4)."""
    if x.dim() != 2:
        raise ValueError(f"x must be [T, K], got {tuple(x.shape)}")
    T, K = x.shape
    q = Act4.empty(T, K, device=x.device)
    moesq_quantize_activations(x, T, K, q.codes, q.scales, q.row_scale, stream)
    return q


def grouped_spgemm_act4(xq: Act4, expert_offsets, w: Weights, epilogue: int = EPI_NONE, perm=None,
                        k: int = 1, out=None, stream=None):
    """W4A4 grouped GEMM.  With `perm`, routed row r reads quantized token
    perm[r] // k of xq (dispatch fused; rows = T*k); else xq's rows are the
    routed rows."""
    M = xq.rows * k if perm is not None else xq.rows
    n_out = _out_cols(w, epilogue)
    if out is None:
        out = torch.empty(M, n_out, dtype=torch.bfloat16, device=xq.codes.device)
    elif tuple(out.shape) != (M, n_out):
        raise ValueError(f"out must be [{M}, {n_out}], got {tuple(out.shape)}")
    moesq_grouped_spgemm_act4(xq, perm, xq.rows if perm is not None else 0, k, expert_offsets, M, w,
                              epilogue, out, stream)
    return out


def unpermute(y, inv_perm, topk_weights, T: int, k: int, stream=None):
    if y.dim() != 2 or y.shape[0] != T * k:
        raise ValueError(f"y must be [T*k = {T * k}, N], got {tuple(y.shape)}")
    N = y.shape[1]
    rows = T if topk_weights is not None else T * k
    out = torch.empty(rows, N, dtype=torch.bfloat16, device=y.device)
    moesq_unpermute(y, inv_perm, topk_weights, T, k, N, out, stream)
    return out


def pack_weights(dense, stream=None, paired: bool = False) -> Weights:
    """dense float32 [E, N, K] on the GPU -> canonical (or paired) Weights."""
    if dense.dim() != 3:
        raise ValueError(f"dense must be [E, N, K], got {tuple(dense.shape)}")
    E, N, K = dense.shape
    w = Weights.empty(E, N, K, device=dense.device,
                      layout=LAYOUT_PAIRED if paired else LAYOUT_CANONICAL)
    pack = moesq_pack_weights_paired if paired else moesq_pack_weights
    pack(dense, E, N, K, w.values, w.masks, w.scales, w.global_scale, stream)
    return w


def tile_weights(w: Weights, stream=None) -> Weights:
    """Canonical (paired) Weights -> a new tiled (paired tiled) Weights
    (shares global_scale)."""
    t = Weights(torch.empty_like(w.values), torch.empty_like(w.masks), torch.empty_like(w.scales),
                w.global_scale, LAYOUT_PAIRED_TILED if w.paired else LAYOUT_TILED)
    moesq_tile_weights(w, t.values, t.masks, t.scales, stream)
    return t


def decode_weights(w: Weights, expert: int, stream=None):
    out = torch.empty(w.N, w.K, dtype=torch.bfloat16, device=w.values.device)
    moesq_decode_weights(w, expert, out, stream)
    return out
