"""ctypes binding of librotattn.so (argument marshalling only).

Every step of the forward pass runs in the HIP kernels behind the C ABI of
include/rotattn.h; this module only turns torch tensors into device pointers
and the current HIP stream.  torch is used for device memory and streams.
Loading fails loudly when the shared library has not been built:

    python -m video_diffusion_transformers_amd.build_lib
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librotattn.so")

BLOCK = 128
MAX_HEADS = 4096
LAYOUT_PACKED = 0      # two INT4 codes per byte, i8 MFMA
LAYOUT_FP8 = 1         # one INT4 code per byte as FP8 E4M3, f8f6f4 MFMA
LAYOUT_FP6 = 2         # INT4 codes as FP6 E2M3 fields, 32 per 32 bytes, f8f6f4 MFMA at the FP6 rate
LAYOUTS = {"packed": LAYOUT_PACKED, "fp8": LAYOUT_FP8, "fp6": LAYOUT_FP6}

STATUS = {0: "ok", -1: "null pointer argument", -2: "inconsistent shape",
          -3: "unsupported head dimension, RoPE split or head count", -4: "workspace too small",
          -5: "device pointer not 16-byte aligned", -6: "HIP launch or runtime error",
          -7: "argument out of range", -8: "one head exceeds the library's static scratch"}
NOALLOC_SCRATCH_BYTES = 256 << 20   # ROTATTN_NOALLOC_SCRATCH_BYTES

EXPORTS = sorted(["rotattn_validate", "rotattn_strerror", "rotattn_rope_tables_host",
                  "rotattn_rope_tables_phase_host",
                  "rotattn_pcode_thresholds_host", "rotattn_kappa_host", "rotattn_prepared_bytes",
                  "rotattn_prepared_bytes_layout", "rotattn_prepared_carve",
                  "rotattn_prepare_qkv", "rotattn_int4_fwd", "rotattn_fp16_fwd",
                  "rotattn_fp16_fwd_strided", "rotattn_fp16_workspace_bytes",
                  "rotattn_fp16_fwd_prepared", "rotattn_fp16_fwd_prepared_strided",
                  "rotattn_fp16_fwd_noalloc",
                  "rotattn_workspace_bytes", "rotattn_mixed_fwd", "rotattn_pcode_sweep",
                  "rotattn_pcode_eval", "rotattn_prepare_qkv_strided", "rotattn_int4_fwd_strided",
                  "rotattn_mixed_fwd_strided", "rotattn_qkv_proj_prepare"])


class Shape(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("B", "H", "N", "D", "grid_t", "grid_h", "grid_w",
                                          "d_t", "d_h", "d_w")]


class RopeRot(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("cos_t", "sin_t", "cos_h", "sin_h", "cos_w", "sin_w",
                                          "rot_t", "rot_h", "rot_w")]


class Strides(C.Structure):
    _fields_ = [("batch", C.c_int64), ("head", C.c_int64), ("token", C.c_int64)]


class Int4Opts(C.Structure):
    _fields_ = [("normalizer", C.c_int32)]


NORMALIZERS = {"exp": 0, "codes": 1}


class Prepared(C.Structure):
    _fields_ = [("layout", C.c_int32)] + [
        (n, C.c_void_p) for n in ("q4", "k4", "v4", "q_scale_l2", "k_scale", "v_scale", "q_rope",
                                  "k_rope", "v_t", "rot64")]


class Debug(C.Structure):
    _fields_ = [("b", C.c_int32), ("h", C.c_int32), ("q_block", C.c_int32),
                ("s_int", C.c_void_p), ("p_code", C.c_void_p), ("pv_int", C.c_void_p),
                ("m_final", C.c_void_p), ("l_final", C.c_void_p)]


class RotAttnError(RuntimeError):
    pass


_lib = None


def lib() -> C.CDLL:
    """The loaded shared library (raises if it is missing)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RotAttnError(f"{LIB_PATH} is missing: build it with "
                               "`python -m video_diffusion_transformers_amd.build_lib`")
        L = C.CDLL(LIB_PATH)
        P = C.c_void_p
        S = C.POINTER(Shape)
        sigs = {
            "rotattn_validate": (C.c_int, [S]),
            "rotattn_strerror": (C.c_char_p, [C.c_int]),
            "rotattn_rope_tables_host": (C.c_int, [S, C.c_double] + [P] * 6),
            "rotattn_rope_tables_phase_host": (C.c_int, [S, C.c_double] + [P] * 9),
            "rotattn_pcode_thresholds_host": (C.c_int, [P]),
            "rotattn_kappa_host": (C.c_float, [C.c_int32]),
            "rotattn_prepared_bytes": (C.c_size_t, [S]),
            "rotattn_prepared_bytes_layout": (C.c_size_t, [S, C.c_int, C.c_int]),
            "rotattn_prepared_carve": (C.c_int, [S, P, C.c_size_t, C.c_int, C.c_int,
                                                 C.POINTER(Prepared)]),
            "rotattn_prepare_qkv": (C.c_int, [S, P, P, P, C.POINTER(RopeRot), P,
                                              C.POINTER(Prepared), P]),
            "rotattn_int4_fwd": (C.c_int, [S, C.POINTER(Prepared), P, P, C.POINTER(Debug), P]),
            "rotattn_fp16_fwd": (C.c_int, [S, P, P, P, P, P, C.c_size_t, P, P]),
            "rotattn_fp16_fwd_strided": (C.c_int, [S, P, P, P, C.POINTER(Strides), P, P,
                                                   C.c_size_t, P, C.POINTER(Strides), P]),
            "rotattn_fp16_workspace_bytes": (C.c_size_t, [S]),
            "rotattn_fp16_fwd_prepared": (C.c_int, [S, P, P, P, P]),
            "rotattn_fp16_fwd_noalloc": (C.c_int, [S, P, P, P, P, P, P]),
            "rotattn_workspace_bytes": (C.c_size_t, [S]),
            "rotattn_mixed_fwd": (C.c_int, [S, P, P, P, C.POINTER(RopeRot), P, P, C.c_size_t, P, P]),
            "rotattn_pcode_sweep": (C.c_int, [C.c_int, C.c_uint32, C.c_uint32, P, C.c_uint32, P, P]),
            "rotattn_pcode_eval": (C.c_int, [C.c_int, P, C.c_uint32, C.c_float, C.c_float, P, P]),
            "rotattn_prepare_qkv_strided": (C.c_int, [S, P, P, P, C.POINTER(Strides),
                                                      C.POINTER(RopeRot), P, C.POINTER(Prepared), P]),
            "rotattn_int4_fwd_strided": (C.c_int, [S, C.POINTER(Prepared), P, P,
                                                   C.POINTER(Strides), C.POINTER(Int4Opts),
                                                   C.POINTER(Debug), P]),
            "rotattn_fp16_fwd_prepared_strided": (C.c_int, [S, P, P, P, C.POINTER(Strides), P]),
            "rotattn_mixed_fwd_strided": (C.c_int, [S, P, P, P, C.POINTER(Strides),
                                                    C.POINTER(RopeRot), P, P, C.c_size_t, P,
                                                    C.POINTER(Strides), P]),
            "rotattn_qkv_proj_prepare": (C.c_int, [S, P, C.c_int64, C.c_int64, C.c_int32, P, P,
                                                   C.POINTER(RopeRot), P, C.POINTER(Prepared), P,
                                                   P]),
        }
        for name, (res, args) in sigs.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def check(status: int, what: str = "") -> None:
    if status != 0:
        raise RotAttnError(f"{what}: {STATUS.get(status, status)} ({status})")


def make_shape(B, H, grid, D, split) -> Shape:
    T, Hg, Wg = grid
    return Shape(B, H, T * Hg * Wg, D, T, Hg, Wg, *split)


def shape_of(cfg) -> Shape:
    """Shape of a synth.Config."""
    return make_shape(cfg.B, cfg.H, cfg.grid, cfg.D, cfg.split)


def validate(shape: Shape) -> int:
    return lib().rotattn_validate(C.byref(shape))


def n_blocks(shape: Shape) -> int:
    return -(-shape.N // BLOCK)


# ------------------------------------------------------------------ host constants

def rope_tables(shape: Shape, base: float = 10000.0, phases=None):
    """Host float32 RoPE tables [(cos_t, sin_t), (cos_h, sin_h), (cos_w, sin_w)];
    phases: three float64 arrays of d_a/2 pair phase offsets (a merged
    rotation), or None."""
    ext = (shape.grid_t, shape.grid_h, shape.grid_w)
    wid = (shape.d_t, shape.d_h, shape.d_w)
    arrs = [np.zeros((e, w // 2), np.float32) for e, w in zip(ext, wid) for _ in range(2)]
    ptrs = [a.ctypes.data_as(C.c_void_p) for a in arrs]
    if phases is None:
        check(lib().rotattn_rope_tables_host(C.byref(shape), C.c_double(base), *ptrs), "rope_tables")
    else:
        ph = [np.ascontiguousarray(x, np.float64) for x in phases]
        for x, w in zip(ph, wid):
            if x.shape != (w // 2,):
                raise ValueError(f"phase array of shape {x.shape}, expected ({w // 2},)")
        pp = [x.ctypes.data_as(C.c_void_p) for x in ph]
        check(lib().rotattn_rope_tables_phase_host(C.byref(shape), C.c_double(base), *pp, *ptrs),
              "rope_tables_phase")
    return [(arrs[0], arrs[1]), (arrs[2], arrs[3]), (arrs[4], arrs[5])]


def pcode_thresholds() -> np.ndarray:
    tau = np.zeros(15, np.float32)
    check(lib().rotattn_pcode_thresholds_host(tau.ctypes.data_as(C.c_void_p)), "thresholds")
    return tau


def kappa(D: int) -> np.float32:
    return np.float32(lib().rotattn_kappa_host(D))


# ------------------------------------------------------------------ device plumbing

def _torch():
    import torch
    return torch


def _ptr(t) -> C.c_void_p:
    return C.c_void_p(0 if t is None else t.data_ptr())


def _stream(stream=None) -> C.c_void_p:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def strides_of(t):
    """Strides of a 4-D [B][H][N][D] torch view with unit channel stride, or
    None for a contiguous tensor (the library's default layout)."""
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("expected a [B][H][N][D] view with unit channel stride")
    if t.is_contiguous():
        return None
    return Strides(t.stride(0), t.stride(1), t.stride(2))


def _strides_arg(st):
    return None if st is None else C.byref(st)


def _shared_strides(q, k, v):
    sq, sk, sv = (strides_of(x) for x in (q, k, v))
    key = [None if x is None else (x.batch, x.head, x.token) for x in (sq, sk, sv)]
    if not key[0] == key[1] == key[2]:
        raise ValueError("q, k and v must share one layout")
    return sq


def _mask_arg(mask):
    if mask is None:
        return None, C.c_void_p(0)
    m = np.ascontiguousarray(np.asarray(mask, np.uint8))
    return m, m.ctypes.data_as(C.c_void_p)


class RopeRotDevice:
    """Device copies of the RoPE tables and rotation matrices (fp32).
    rot32=None: no dense rotation (with phases: the rotation merged into RoPE)."""

    def __init__(self, shape: Shape, rot32, base: float = 10000.0, device="cuda", phases=None):
        torch = _torch()
        tabs = rope_tables(shape, base, phases)
        self.tensors = [torch.from_numpy(np.ascontiguousarray(x)).to(device)
                        for pair in tabs for x in pair]
        ptrs = [t.data_ptr() for t in self.tensors]
        if rot32 is not None:
            rots = [torch.from_numpy(np.ascontiguousarray(r, np.float32)).to(device) for r in rot32]
            self.tensors += rots
            ptrs += [t.data_ptr() for t in rots]
        else:
            ptrs += [0, 0, 0]
        self.struct = RopeRot(*ptrs)


class PreparedDevice:
    """Device buffers of a rotattn_prepared, carved from one allocation."""

    def __init__(self, shape: Shape, with_rope: bool = True, layout: int = LAYOUT_FP6,
                 device="cuda"):
        torch = _torch()
        self.shape = shape
        self.layout = layout
        nbytes = lib().rotattn_prepared_bytes_layout(C.byref(shape), int(with_rope), layout)
        if nbytes == 0:
            check(validate(shape) or -7, "prepared_bytes")
        self.buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
        base = (self.buf.data_ptr() + 255) // 256 * 256
        self.struct = Prepared()
        check(lib().rotattn_prepared_carve(C.byref(shape), C.c_void_p(base), nbytes, int(with_rope),
                                           layout, C.byref(self.struct)), "prepared_carve")
        self.base = base

    def view(self, field: str, dtype, count: int):
        """A torch view of one carved buffer (for inspection in tests)."""
        torch = _torch()
        addr = getattr(self.struct, field)
        off = addr - self.buf.data_ptr()
        nbytes = count * torch.empty((), dtype=dtype).element_size()
        return self.buf[off:off + nbytes].view(dtype)


def prepare_qkv(shape: Shape, q, k, v, rr: RopeRotDevice, prep: PreparedDevice, mask=None,
                stream=None) -> None:
    """q, k, v: [B][H][N][D] fp16 tensors or views sharing one layout (e.g.
    slices of a fused QKV projection's token-major output); no copies."""
    keep, m = _mask_arg(mask)
    st = _shared_strides(q, k, v)
    check(lib().rotattn_prepare_qkv_strided(C.byref(shape), _ptr(q), _ptr(k), _ptr(v),
                                            _strides_arg(st), C.byref(rr.struct), m,
                                            C.byref(prep.struct), _stream(stream)), "prepare_qkv")


def qkv_proj_prepare(shape: Shape, x, w, bias, rr: RopeRotDevice, prep: PreparedDevice,
                     mask=None, qkv_out=None, stream=None) -> None:
    """The QKV projection with the prologue as its epilogue: x [B][N][C] fp16
    (channel stride 1), w [3*H*D][C] fp16 contiguous (Q heads, then K, then V),
    bias [3*H*D] fp16 or None; qkv_out: None or fp16 [3][B*H][N_pad][D]."""
    keep, m = _mask_arg(mask)
    if x.dim() != 3 or x.stride(2) != 1:
        raise ValueError("x must be [B][N][C] with channel stride 1")
    if not w.is_contiguous() or w.dim() != 2 or w.shape[1] != x.shape[2]:
        raise ValueError("w must be a contiguous [3*H*D][C] tensor")
    check(lib().rotattn_qkv_proj_prepare(C.byref(shape), _ptr(x), x.stride(0), x.stride(1),
                                         int(x.shape[2]), _ptr(w),
                                         _ptr(bias) if bias is not None else None,
                                         C.byref(rr.struct), m, C.byref(prep.struct),
                                         _ptr(qkv_out) if qkv_out is not None else None,
                                         _stream(stream)), "qkv_proj_prepare")


def int4_fwd(shape: Shape, prep: PreparedDevice, o, mask=None, debug: Debug | None = None,
             stream=None, normalizer: str = "exp") -> None:
    """normalizer "exp": l = sum of the unquantized 2^x; "codes": the sum of
    the P codes (FP8 and FP6 layouts)."""
    keep, m = _mask_arg(mask)
    dbg = C.byref(debug) if debug is not None else None
    opts = Int4Opts(NORMALIZERS[normalizer])
    check(lib().rotattn_int4_fwd_strided(C.byref(shape), C.byref(prep.struct), m, _ptr(o),
                                         _strides_arg(strides_of(o)), C.byref(opts), dbg,
                                         _stream(stream)), "int4_fwd")


def fp16_fwd_prepared(shape: Shape, prep: PreparedDevice, o, head_select=None,
                      stream=None) -> None:
    """FP16 attention of the selected heads from the prologue's fallback
    buffers (q_rope, k_rope, v_t of `prep`)."""
    keep, m = _mask_arg(head_select)
    check(lib().rotattn_fp16_fwd_prepared_strided(C.byref(shape), C.byref(prep.struct), m, _ptr(o),
                                                  _strides_arg(strides_of(o)), _stream(stream)),
          "fp16_fwd_prepared")


def fp16_fwd_noalloc(shape: Shape, q_rope, k_rope, v, o, head_select=None,
                     stream=None) -> None:
    """FP16 attention on contiguous caller tensors with the staging in the
    library's static device scratch (no allocation; calls that overlap on one
    GPU race)."""
    keep, m = _mask_arg(head_select)
    for t in (q_rope, k_rope, v, o):
        if not t.is_contiguous():
            raise ValueError("fp16_fwd_noalloc takes contiguous [B][H][N][D] tensors")
    check(lib().rotattn_fp16_fwd_noalloc(C.byref(shape), _ptr(q_rope), _ptr(k_rope), _ptr(v), m,
                                         _ptr(o), _stream(stream)), "fp16_fwd_noalloc")


def fp16_workspace_bytes(shape: Shape) -> int:
    return lib().rotattn_fp16_workspace_bytes(C.byref(shape))


def fp16_fwd(shape: Shape, q_rope, k_rope, v, o, workspace, head_select=None,
             stream=None) -> None:
    """FP16 attention of the selected heads on caller tensors: RoPE'd fp16
    Q'/K' and V ([B][H][N][D] views sharing one layout), staging through the
    uint8 device tensor `workspace` (at least fp16_workspace_bytes)."""
    keep, m = _mask_arg(head_select)
    st = _shared_strides(q_rope, k_rope, v)
    check(lib().rotattn_fp16_fwd_strided(C.byref(shape), _ptr(q_rope), _ptr(k_rope), _ptr(v),
                                         _strides_arg(st), m, _ptr(workspace),
                                         workspace.numel() * workspace.element_size(), _ptr(o),
                                         _strides_arg(strides_of(o)), _stream(stream)), "fp16_fwd")


def workspace_bytes(shape: Shape) -> int:
    return lib().rotattn_workspace_bytes(C.byref(shape))


def prepared_bytes(shape: Shape) -> int:
    return lib().rotattn_prepared_bytes(C.byref(shape))


def mixed_fwd(shape: Shape, q, k, v, rr: RopeRotDevice, mask, workspace, o, stream=None) -> None:
    keep, m = _mask_arg(mask)
    st = _shared_strides(q, k, v)
    check(lib().rotattn_mixed_fwd_strided(C.byref(shape), _ptr(q), _ptr(k), _ptr(v),
                                          _strides_arg(st), C.byref(rr.struct), m,
                                          _ptr(workspace),
                                          workspace.numel() * workspace.element_size(), _ptr(o),
                                          _strides_arg(strides_of(o)), _stream(stream)),
          "mixed_fwd")


def pcode_sweep(mag_lo: int, count: int, max_transitions: int = 4096, layout: int = LAYOUT_FP6,
                stream=None):
    """Transitions (magnitude bits, code before, code after) of the device P code."""
    torch = _torch()
    trans = torch.zeros(3 * max_transitions, dtype=torch.int32, device="cuda")
    n = torch.zeros(1, dtype=torch.int32, device="cuda")
    check(lib().rotattn_pcode_sweep(layout, mag_lo, count, _ptr(trans), max_transitions, _ptr(n),
                                    _stream(stream)), "pcode_sweep")
    return trans, n


def pcode_eval(I, c: float, m: float, layout: int = LAYOUT_FP6, stream=None):
    torch = _torch()
    codes = torch.empty(I.numel(), dtype=torch.uint8, device=I.device)
    check(lib().rotattn_pcode_eval(layout, _ptr(I), I.numel(), C.c_float(c), C.c_float(m),
                                   _ptr(codes), _stream(stream)), "pcode_eval")
    return codes
