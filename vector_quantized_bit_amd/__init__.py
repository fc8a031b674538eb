"""Thin Python binding of libvqkv.so (VQ-KV decode attention for MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/vqkv.h``.  PyTorch supplies
device memory and the current stream; nothing here computes on tensors.
The functions keep the C entry points' names without the ``vq_`` prefix.

The library must have been built (``python -m vector_quantized_bit_amd.build``);
importing works without it, but the first call raises if it is missing.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "LIB_PATH", "VqError", "Layout", "library", "make_layout", "transform_query",
    "encode_append", "decode_attention", "decode_attention_workspace_bytes",
    "decode_attention_default_splits", "fp16_decode_attention",
    "fp16_attention_workspace_bytes", "status_string", "PreparedCall",
    "prepare_encode_append", "prepare_decode_attention", "decode_attention_plan_splits",
    "decode_attention_partials", "merge_partials", "prepare_decode_attention_partials",
    "prepare_merge_partials", "decode_step", "prepare_decode_step", "decode_step_partials",
    "prepare_decode_step_partials", "decode_step_num_partials", "decode_step_workspace_bytes",
    "decode_step_window", "prepare_decode_step_window", "decode_step_window_num_partials",
    "decode_step_window_workspace_bytes", "flush_window", "calibrate_lambda", "transform_keys",
    "kmeans_workspace_bytes", "kmeans",
]

# VQKV_LIBRARY names another build of the library to load instead (the
# tests' host-sanitized build, for one)
LIB_PATH = os.environ.get("VQKV_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libvqkv.so")

VQ_F16, VQ_F32 = 0, 1
_c_int = ctypes.c_int
_i32 = ctypes.c_int32
_vp = ctypes.c_void_p
_size = ctypes.c_size_t


class Layout(ctypes.Structure):
    """The C ``vq_layout`` struct."""

    _fields_ = [("head_dim", _i32), ("sub_dim", _i32), ("k_code_bits", _i32),
                ("v_code_bits", _i32), ("num_kv_heads", _i32), ("capacity", _i32)]


class VqError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} ({status}): {_last_error()}")
        self.status = status


_lib = None


def library() -> ctypes.CDLL:
    """Load libvqkv.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m vector_quantized_bit_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    lp = ctypes.POINTER(Layout)
    sig = {
        "vq_transform_query": (_c_int, [lp, _vp, _c_int, _vp, _i32, _i32, _vp, _vp]),
        "vq_encode_append": (_c_int, [lp, _vp, _vp, _c_int, _vp, _vp, _vp, _vp, _vp, _i32,
                                      _i32, _i32, _vp]),
        "vq_decode_attention_default_splits": (_i32, [lp, _i32, _i32, _i32]),
        "vq_decode_attention_workspace_bytes": (_size, [lp, _i32, _i32, _i32, _i32]),
        "vq_decode_attention": (_c_int, [lp, _vp, _c_int, _vp, _vp, _vp, _vp, _vp, _i32, _i32,
                                         _i32, _i32, _vp, _vp, _size, _vp]),
        "vq_decode_attention_plan_splits": (_i32, [lp, _i32, _i32, _i32, _i32]),
        "vq_decode_attention_partials": (_c_int, [lp, _vp, _c_int, _vp, _vp, _vp, _vp, _vp, _i32,
                                                  _i32, _i32, _i32, _vp, _vp, _vp, _vp]),
        "vq_merge_partials": (_c_int, [_i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp]),
        "vq_decode_step_num_partials": (_i32, [lp, _i32, _i32, _i32, _i32]),
        "vq_decode_step_workspace_bytes": (_size, [lp, _i32, _i32, _i32, _i32]),
        "vq_decode_step": (_c_int, [lp, _vp, _c_int, _vp, _vp, _c_int, _vp, _vp, _vp, _vp, _vp,
                                    _i32, _i32, _i32, _i32, _vp, _vp, _size, _vp]),
        "vq_decode_step_noalloc": (_c_int, [lp, _vp, _c_int, _vp, _vp, _c_int, _vp, _vp, _vp,
                                            _vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp]),
        "vq_decode_step_partials": (_c_int, [lp, _vp, _c_int, _vp, _vp, _c_int, _vp, _vp, _vp,
                                             _vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp,
                                             _vp]),
        "vq_decode_step_window_num_partials": (_i32, [lp, _i32, _i32, _i32, _i32]),
        "vq_decode_step_window_workspace_bytes": (_size, [lp, _i32, _i32, _i32, _i32]),
        "vq_decode_step_window": (_c_int, [lp, _vp, _c_int, _vp, _vp, _c_int, _vp, _vp, _vp, _vp,
                                           _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                           _vp, _vp, _size, _vp]),
        "vq_flush_window": (_c_int, [lp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                                     _vp]),
        "vq_calibrate_lambda": (_c_int, [_vp, _c_int, _i32, _i32, _vp, _vp]),
        "vq_transform_keys": (_c_int, [_vp, _c_int, _vp, _i32, _i32, _vp, _vp]),
        "vq_kmeans_workspace_bytes": (_size, [_i32, _i32, _i32, _i32]),
        "vq_kmeans": (_c_int, [_vp, _i32, _i32, _i32, _i32, _vp, _i32, _vp, _vp, _vp, _vp,
                               _size, _vp]),
        "vq_fp16_attention_workspace_bytes": (_size, [_i32, _i32, _i32, _i32, _i32]),
        "vq_fp16_decode_attention": (_c_int, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                              _vp, _vp, _size, _vp]),
        "vq_set_deterministic": (_c_int, [_c_int]),
        "vq_set_score_method": (_c_int, [_c_int]),
        "vq_status_string": (ctypes.c_char_p, [_c_int]),
        "vq_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def set_deterministic(on: bool) -> bool:
    """Library-wide deterministic mode (vq_set_deterministic): a fixed tile
    order in the split kernel, so repeated calls give bit-identical results.
    Returns the previous setting."""
    return bool(library().vq_set_deterministic(1 if on else 0))


SCORES_MFMA = 0
SCORES_LUT = 1


def set_score_method(method: int) -> int:
    """Library-wide score method (vq_set_score_method): SCORES_MFMA (default)
    or SCORES_LUT (the lookup-table scores; 8-bit keys, d = 4, G <= 4).
    Returns the previous method."""
    prev = int(library().vq_set_score_method(int(method)))
    if prev < 0:
        raise ValueError(_last_error())
    return prev


def status_string(status: int) -> str:
    return library().vq_status_string(status).decode()


def _last_error() -> str:
    return library().vq_last_error().decode()


def _check(status: int, what: str) -> None:
    if status != 0:
        raise VqError(status, what)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float16:
        return VQ_F16
    if t.dtype == torch.float32:
        return VQ_F32
    raise TypeError(f"expected float16 or float32, got {t.dtype}")


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def make_layout(codes_k: torch.Tensor, codes_v: torch.Tensor, cb_k: torch.Tensor,
                cb_v: torch.Tensor) -> Layout:
    """Cache geometry from the tensors: codes_* [B][Hkv][cap][row] uint8,
    cb_* [Hkv][2^bits][4] float16."""
    _need(codes_k.dim() == 4 and codes_v.dim() == 4, "codes must be [B][Hkv][cap][row]")
    _need(cb_k.dim() == 3 and cb_v.dim() == 3, "codebooks must be [Hkv][entries][4]")
    k_bits = cb_k.shape[1].bit_length() - 1
    v_bits = cb_v.shape[1].bit_length() - 1
    return Layout(head_dim=128, sub_dim=int(cb_k.shape[2]), k_code_bits=k_bits,
                  v_code_bits=v_bits, num_kv_heads=int(codes_k.shape[1]),
                  capacity=int(codes_k.shape[2]))


def _check_cache(codes_k, codes_v, cb_k, cb_v, lam):
    """Every shape the kernels index by: the C ABI receives raw pointers, so a
    tensor smaller than the layout says would be read (or written) past its
    end on the device."""
    for name, t, dt in (("codes_k", codes_k, torch.uint8), ("codes_v", codes_v, torch.uint8),
                        ("cb_k", cb_k, torch.float16), ("cb_v", cb_v, torch.float16),
                        ("lambda", lam, torch.float32)):
        _need(t.is_cuda and t.is_contiguous(), f"{name} must be a contiguous device tensor")
        _need(t.dtype == dt, f"{name} must be {dt}, got {t.dtype}")
        _need(t.device == codes_k.device, f"{name} is on {t.device}, the cache on {codes_k.device}")
    _need(codes_k.dim() == 4 and codes_v.dim() == 4, "codes must be [B][Hkv][cap][row]")
    _need(codes_k.shape[:3] == codes_v.shape[:3], "codes_k and codes_v disagree in [B][Hkv][cap]")
    hkv = codes_k.shape[1]
    _need(lam.dim() == 2 and tuple(lam.shape) == (hkv, 128),
          f"lambda must be [Hkv={hkv}][128], got {tuple(lam.shape)}")
    _need(cb_k.dim() == 3 and cb_v.dim() == 3, "codebooks must be [Hkv][entries][d]")
    sub = int(cb_k.shape[2])
    for name, cb in (("cb_k", cb_k), ("cb_v", cb_v)):
        ent = int(cb.shape[1])
        _need(cb.shape[0] == hkv and ent >= 1 and ent & (ent - 1) == 0 and cb.shape[2] == sub,
              f"{name} must be [Hkv={hkv}][2^bits][d={sub}], got {tuple(cb.shape)}")
    _need(sub in (4, 8), f"sub-vector size {sub} unsupported (4 or 8)")
    for name, codes, cb in (("codes_k", codes_k, cb_k), ("codes_v", codes_v, cb_v)):
        row = (128 // sub) * (int(cb.shape[1]).bit_length() - 1) // 8
        _need(codes.shape[3] == row,
              f"{name} rows must be {row} bytes for {cb.shape[1]}-entry codebooks of "
              f"{sub}-dim sub-vectors, got {codes.shape[3]}")


def _check_query(q, codes_k):
    _need(q.is_cuda and q.is_contiguous() and q.dim() == 3 and q.shape[2] == 128,
          "q must be contiguous [B][Hq][128]")
    _need(q.device == codes_k.device, f"q is on {q.device}, the cache on {codes_k.device}")
    _need(q.shape[0] == codes_k.shape[0],
          f"q has {q.shape[0]} sequences, the cache {codes_k.shape[0]}")
    _need(q.shape[1] % codes_k.shape[1] == 0,
          f"query heads {q.shape[1]} are not a multiple of KV heads {codes_k.shape[1]}")
    _dtype_code(q)


def _check_out(out, batch, hq, device):
    _need(out.is_cuda and out.is_contiguous() and out.dtype == torch.float32
          and tuple(out.shape) == (batch, hq, 128) and out.device == device,
          f"out must be contiguous float32 [{batch}][{hq}][128] on {device}")
    return out


def _check_workspace(ws, device):
    _need(ws.is_cuda and ws.is_contiguous() and ws.dtype == torch.uint8 and ws.device == device,
          f"workspace must be a contiguous uint8 tensor on {device}")
    return ws


def transform_query(q: torch.Tensor, lam: torch.Tensor, out: torch.Tensor | None = None):
    """q~ = q diag(lambda) H_128 -> float32 [B][Hq][128]."""
    _need(q.is_cuda and q.is_contiguous() and q.dim() == 3 and q.shape[2] == 128,
          "q must be contiguous [B][Hq][128]")
    _need(lam.is_cuda and lam.is_contiguous() and lam.dtype == torch.float32 and lam.dim() == 2
          and lam.shape[1] == 128 and lam.device == q.device,
          "lambda must be contiguous float32 [Hkv][128] on q's device")
    _need(q.shape[1] % lam.shape[0] == 0, "query heads must be a multiple of KV heads")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    _check_out(out, q.shape[0], q.shape[1], q.device)
    lay = Layout(128, 4, 8, 8, int(lam.shape[0]), 1)
    _check(library().vq_transform_query(ctypes.byref(lay), _ptr(q), _dtype_code(q), _ptr(lam),
                                        q.shape[0], q.shape[1], _ptr(out), _stream(q)),
           "vq_transform_query")
    return out


class PreparedCall:
    """A C entry point with its arguments marshalled once.

    Calling it passes the same pointers and sizes again, with the stream that
    is current at call time (or ``stream``, a raw HIP stream handle), and
    raises on a non-zero status.  The tensors named at preparation are kept
    alive by the object; the caller must not resize or reallocate them."""

    def __init__(self, name: str, fn, args: tuple, keep: tuple, device: torch.device):
        self._name, self._fn, self._args, self._keep, self._device = name, fn, args, keep, device

    def __call__(self, stream: int | None = None) -> None:
        if stream is None:
            stream = torch.cuda.current_stream(self._device).cuda_stream
        _check(self._fn(*self._args, stream), self._name)


def _encode_append_args(k_new, v_new, lam, cb_k, cb_v, codes_k, codes_v, cur_len: int):
    _check_cache(codes_k, codes_v, cb_k, cb_v, lam)
    _need(k_new.shape == v_new.shape and k_new.dim() == 4, "k_new/v_new must be [B][Hkv][T][128]")
    _need(k_new.dtype == v_new.dtype, "k_new and v_new must share a dtype")
    _need(k_new.is_contiguous() and v_new.is_contiguous(), "k_new/v_new must be contiguous")
    _need(k_new.shape[0] == codes_k.shape[0] and k_new.shape[1] == codes_k.shape[1]
          and k_new.shape[3] == 128, "k_new [B][Hkv][T][128] disagrees with the cache")
    _need(k_new.device == codes_k.device and v_new.device == codes_k.device,
          "k_new/v_new must be on the cache's device")
    _dtype_code(k_new)
    lay = make_layout(codes_k, codes_v, cb_k, cb_v)
    return (ctypes.byref(lay), _ptr(k_new), _ptr(v_new), _dtype_code(k_new), _ptr(lam),
            _ptr(cb_k), _ptr(cb_v), _ptr(codes_k), _ptr(codes_v), k_new.shape[0], cur_len,
            k_new.shape[2]), lay


def encode_append(k_new, v_new, lam, cb_k, cb_v, codes_k, codes_v, cur_len: int) -> None:
    """Encode k_new / v_new [B][Hkv][T][128] into slots [cur_len, cur_len+T)."""
    args, _ = _encode_append_args(k_new, v_new, lam, cb_k, cb_v, codes_k, codes_v, cur_len)
    _check(library().vq_encode_append(*args, _stream(k_new)), "vq_encode_append")


def prepare_encode_append(k_new, v_new, lam, cb_k, cb_v, codes_k, codes_v,
                          cur_len: int) -> PreparedCall:
    """``encode_append`` with its arguments validated and marshalled once."""
    args, lay = _encode_append_args(k_new, v_new, lam, cb_k, cb_v, codes_k, codes_v, cur_len)
    return PreparedCall("vq_encode_append", library().vq_encode_append, args,
                        (lay, k_new, v_new, lam, cb_k, cb_v, codes_k, codes_v), k_new.device)


def decode_attention_default_splits(codes_k, codes_v, cb_k, cb_v, batch, num_q_heads,
                                    context_len) -> int:
    lay = make_layout(codes_k, codes_v, cb_k, cb_v)
    return int(library().vq_decode_attention_default_splits(ctypes.byref(lay), batch,
                                                            num_q_heads, context_len))


def decode_attention_workspace_bytes(codes_k, codes_v, cb_k, cb_v, batch, num_q_heads,
                                     context_len, num_splits: int = 0) -> int:
    lay = make_layout(codes_k, codes_v, cb_k, cb_v)
    return int(library().vq_decode_attention_workspace_bytes(ctypes.byref(lay), batch,
                                                             num_q_heads, context_len,
                                                             num_splits))


def _decode_attention_args(q, lam, cb_k, cb_v, codes_k, codes_v, context_len, num_splits, out,
                           workspace):
    _check_cache(codes_k, codes_v, cb_k, cb_v, lam)
    _check_query(q, codes_k)
    batch, hq = q.shape[0], q.shape[1]
    if out is None:
        out = torch.empty((batch, hq, 128), dtype=torch.float32, device=q.device)
    _check_out(out, batch, hq, q.device)
    if workspace is None:
        nbytes = decode_attention_workspace_bytes(codes_k, codes_v, cb_k, cb_v, batch, hq,
                                                  context_len, num_splits)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _check_workspace(workspace, q.device)
    lay = make_layout(codes_k, codes_v, cb_k, cb_v)
    args = (ctypes.byref(lay), _ptr(q), _dtype_code(q), _ptr(lam), _ptr(cb_k), _ptr(cb_v),
            _ptr(codes_k), _ptr(codes_v), batch, hq, context_len, num_splits, _ptr(out),
            _ptr(workspace), workspace.numel())
    return args, lay, out, workspace


def decode_attention(q, lam, cb_k, cb_v, codes_k, codes_v, context_len: int,
                     num_splits: int = 0, out=None, workspace=None):
    """Decode attention over the VQ cache -> float32 [B][Hq][128].

    ``workspace`` (optional, reusable): a uint8 device tensor of at least
    ``decode_attention_workspace_bytes(...)`` bytes; its contents do not
    matter."""
    args, _, out, _ = _decode_attention_args(q, lam, cb_k, cb_v, codes_k, codes_v, context_len,
                                             num_splits, out, workspace)
    _check(library().vq_decode_attention(*args, _stream(q)), "vq_decode_attention")
    return out


def prepare_decode_attention(q, lam, cb_k, cb_v, codes_k, codes_v, context_len: int,
                             num_splits: int = 0, out=None, workspace=None) -> PreparedCall:
    """``decode_attention`` with its arguments validated and marshalled once;
    the output tensor is the prepared call's ``out`` attribute."""
    args, lay, out, workspace = _decode_attention_args(q, lam, cb_k, cb_v, codes_k, codes_v,
                                                       context_len, num_splits, out, workspace)
    call = PreparedCall("vq_decode_attention", library().vq_decode_attention, args,
                        (lay, q, lam, cb_k, cb_v, codes_k, codes_v, out, workspace), q.device)
    call.out = out
    return call


def decode_attention_plan_splits(codes_k, codes_v, cb_k, cb_v, batch, num_q_heads,
                                 context_len, requested: int = 0) -> int:
    """Split count the library uses for ``requested`` splits (0 = default)."""
    lay = make_layout(codes_k, codes_v, cb_k, cb_v)
    return int(library().vq_decode_attention_plan_splits(ctypes.byref(lay), batch, num_q_heads,
                                                         context_len, requested))


def _partials_args(q, lam, cb_k, cb_v, codes_k, codes_v, context_len, num_splits, partials):
    _check_cache(codes_k, codes_v, cb_k, cb_v, lam)
    _check_query(q, codes_k)
    batch, hq = q.shape[0], q.shape[1]
    splits = decode_attention_plan_splits(codes_k, codes_v, cb_k, cb_v, batch, hq, context_len,
                                          num_splits)
    if partials is None:
        m = torch.empty((batch, hq, splits), dtype=torch.float32, device=q.device)
        partials = (m, torch.empty_like(m),
                    torch.empty((batch, hq, splits, 128), dtype=torch.float32, device=q.device))
    m, l, o = partials
    for name, t, shape in (("m", m, (batch, hq, splits)), ("l", l, (batch, hq, splits)),
                           ("o", o, (batch, hq, splits, 128))):
        _need(t.is_cuda and t.is_contiguous() and t.dtype == torch.float32
              and tuple(t.shape) == shape and t.device == q.device,
              f"partials {name} must be contiguous float32 {shape} on q's device")
    lay = make_layout(codes_k, codes_v, cb_k, cb_v)
    args = (ctypes.byref(lay), _ptr(q), _dtype_code(q), _ptr(lam), _ptr(cb_k), _ptr(cb_v),
            _ptr(codes_k), _ptr(codes_v), batch, hq, context_len, splits, _ptr(m), _ptr(l),
            _ptr(o))
    return args, lay, partials


def decode_attention_partials(q, lam, cb_k, cb_v, codes_k, codes_v, context_len: int,
                              num_splits: int = 0, partials=None):
    """The split pass alone -> (m [B][Hq][S], l [B][Hq][S], o [B][Hq][S][128]),
    S = decode_attention_plan_splits(..., num_splits)."""
    args, _, partials = _partials_args(q, lam, cb_k, cb_v, codes_k, codes_v, context_len,
                                       num_splits, partials)
    _check(library().vq_decode_attention_partials(*args, _stream(q)),
           "vq_decode_attention_partials")
    return partials


def prepare_decode_attention_partials(q, lam, cb_k, cb_v, codes_k, codes_v, context_len: int,
                                      num_splits: int = 0, partials=None) -> PreparedCall:
    """``decode_attention_partials`` marshalled once; the partials are the
    prepared call's ``partials`` attribute."""
    args, lay, partials = _partials_args(q, lam, cb_k, cb_v, codes_k, codes_v, context_len,
                                         num_splits, partials)
    call = PreparedCall("vq_decode_attention_partials", library().vq_decode_attention_partials,
                        args, (lay, q, lam, cb_k, cb_v, codes_k, codes_v) + tuple(partials),
                        q.device)
    call.partials = partials
    return call


def _merge_args(partials, out):
    m, l, o = partials
    _need(m.dim() == 3 and l.shape == m.shape and o.dim() == 4 and o.shape[:3] == m.shape
          and o.shape[3] == 128, "partials must be m, l [B][Hq][S] and o [B][Hq][S][128]")
    for name, t in (("m", m), ("l", l), ("o", o)):
        _need(t.is_cuda and t.is_contiguous() and t.dtype == torch.float32,
              f"partials {name} must be a contiguous float32 device tensor")
    batch, hq, splits = m.shape
    if out is None:
        out = torch.empty((batch, hq, 128), dtype=torch.float32, device=m.device)
    _need(out.is_cuda and out.is_contiguous() and out.dtype == torch.float32
          and tuple(out.shape) == (batch, hq, 128), "out must be contiguous float32 [B][Hq][128]")
    return (batch, hq, splits, _ptr(m), _ptr(l), _ptr(o), _ptr(out)), out


def merge_partials(partials, out=None):
    """Log-sum-exp merge of (m, l, o) partials over their split axis."""
    args, out = _merge_args(partials, out)
    _check(library().vq_merge_partials(*args, _stream(out)), "vq_merge_partials")
    return out


def prepare_merge_partials(partials, out=None) -> PreparedCall:
    """``merge_partials`` marshalled once; the output is the prepared call's
    ``out`` attribute."""
    args, out = _merge_args(partials, out)
    call = PreparedCall("vq_merge_partials", library().vq_merge_partials, args,
                        tuple(partials) + (out,), out.device)
    call.out = out
    return call


def _step_common(q, k_new, v_new, lam, cb_k, cb_v, codes_k, codes_v):
    _check_cache(codes_k, codes_v, cb_k, cb_v, lam)
    _check_query(q, codes_k)
    batch, hkv = codes_k.shape[0], codes_k.shape[1]
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        _need(t.is_cuda and t.is_contiguous() and t.numel() == batch * hkv * 128
              and t.shape[0] == batch and t.shape[1] == hkv and t.shape[-1] == 128
              and t.device == q.device,
              f"{name} must be contiguous [B][Hkv][128] (or [B][Hkv][1][128]) on q's device")
    _need(k_new.dtype == v_new.dtype, "k_new and v_new must share a dtype")
    _dtype_code(k_new)
    return batch, q.shape[1]


def _step_args(q, k_new, v_new, lam, cb_k, cb_v, codes_k, codes_v, cur_len, num_splits, out,
               workspace):
    batch, hq = _step_common(q, k_new, v_new, lam, cb_k, cb_v, codes_k, codes_v)
    if out is None:
        out = torch.empty((batch, hq, 128), dtype=torch.float32, device=q.device)
    _check_out(out, batch, hq, q.device)
    lay = make_layout(codes_k, codes_v, cb_k, cb_v)
    if workspace is None:
        nbytes = library().vq_decode_step_workspace_bytes(ctypes.byref(lay), batch, hq, cur_len,
                                                         num_splits)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _check_workspace(workspace, q.device)
    args = (ctypes.byref(lay), _ptr(q), _dtype_code(q), _ptr(k_new), _ptr(v_new),
            _dtype_code(k_new), _ptr(lam), _ptr(cb_k), _ptr(cb_v), _ptr(codes_k), _ptr(codes_v),
            batch, hq, cur_len, num_splits, _ptr(out), _ptr(workspace), workspace.numel())
    return args, lay, out, workspace


def decode_step(q, k_new, v_new, lam, cb_k, cb_v, codes_k, codes_v, cur_len: int,
                num_splits: int = 0, out=None, workspace=None):
    """Encode k_new / v_new [B][Hkv][128] into slot ``cur_len``, then decode
    attention over ``cur_len + 1`` tokens -> float32 [B][Hq][128]."""
    args, _, out, _ = _step_args(q, k_new, v_new, lam, cb_k, cb_v, codes_k, codes_v, cur_len,
                                 num_splits, out, workspace)
    _check(library().vq_decode_step(*args, _stream(q)), "vq_decode_step")
    return out


def prepare_decode_step(q, k_new, v_new, lam, cb_k, cb_v, codes_k, codes_v, cur_len: int,
                        num_splits: int = 0, out=None, workspace=None) -> PreparedCall:
    """``decode_step`` marshalled once; the output is the call's ``out``."""
    args, lay, out, workspace = _step_args(q, k_new, v_new, lam, cb_k, cb_v, codes_k, codes_v,
                                           cur_len, num_splits, out, workspace)
    call = PreparedCall("vq_decode_step", library().vq_decode_step, args,
                        (lay, q, k_new, v_new, lam, cb_k, cb_v, codes_k, codes_v, out,
                         workspace), q.device)
    call.out = out
    return call


def decode_step_noalloc(q, k_new, v_new, lam, cb_k, cb_v, codes_k, codes_v, cur_len: int,
                        num_splits: int = 0, out=None):
    """``decode_step`` through vq_decode_step_noalloc: the library keeps the
    split partials in its static device buffer (VQ_NOALLOC_SCRATCH_BYTES, 4
    MiB per GPU), so the call needs no workspace.  Calls on one GPU must not
    overlap.  ``out`` (float32 [B][Hq][128]) is allocated here if not given."""
    batch, hq = _step_common(q, k_new, v_new, lam, cb_k, cb_v, codes_k, codes_v)
    if out is None:
        out = torch.empty((batch, hq, 128), dtype=torch.float32, device=q.device)
    _check_out(out, batch, hq, q.device)
    lay = make_layout(codes_k, codes_v, cb_k, cb_v)
    _check(library().vq_decode_step_noalloc(
        ctypes.byref(lay), _ptr(q), _dtype_code(q), _ptr(k_new), _ptr(v_new), _dtype_code(k_new),
        _ptr(lam), _ptr(cb_k), _ptr(cb_v), _ptr(codes_k), _ptr(codes_v), batch, hq, cur_len,
        num_splits, _ptr(out), _stream(q)), "vq_decode_step_noalloc")
    return out


NOALLOC_SCRATCH_BYTES = 4 << 20


def _check_window(win_k, win_v, codes_k):
    batch, hkv = codes_k.shape[0], codes_k.shape[1]
    for name, t in (("win_k", win_k), ("win_v", win_v)):
        _need(t.is_cuda and t.is_contiguous() and t.dtype == torch.float16 and t.dim() == 4
              and t.shape[0] == batch and t.shape[1] == hkv and t.shape[3] == 128
              and t.device == codes_k.device,
              f"{name} must be contiguous float16 [B][Hkv][win_cap][128] on the cache's device")
    _need(win_k.shape == win_v.shape, "win_k and win_v must have the same shape")
    return int(win_k.shape[2])


def decode_step_window_workspace_bytes(codes_k, codes_v, cb_k, cb_v, batch, num_q_heads,
                                       num_codes, requested: int = 0) -> int:
    lay = make_layout(codes_k, codes_v, cb_k, cb_v)
    return int(library().vq_decode_step_window_workspace_bytes(ctypes.byref(lay), batch,
                                                               num_q_heads, num_codes, requested))


def decode_step_window_num_partials(codes_k, codes_v, cb_k, cb_v, batch, num_q_heads, num_codes,
                                    requested: int = 0) -> int:
    lay = make_layout(codes_k, codes_v, cb_k, cb_v)
    return int(library().vq_decode_step_window_num_partials(ctypes.byref(lay), batch,
                                                            num_q_heads, num_codes, requested))


def _window_step_args(q, k_new, v_new, lam, cb_k, cb_v, codes_k, codes_v, win_k, win_v,
                      num_codes, win_len, num_splits, out, workspace):
    batch, hq = _step_common(q, k_new, v_new, lam, cb_k, cb_v, codes_k, codes_v)
    win_cap = _check_window(win_k, win_v, codes_k)
    if out is None:
        out = torch.empty((batch, hq, 128), dtype=torch.float32, device=q.device)
    _check_out(out, batch, hq, q.device)
    lay = make_layout(codes_k, codes_v, cb_k, cb_v)
    if workspace is None:
        nbytes = library().vq_decode_step_window_workspace_bytes(ctypes.byref(lay), batch, hq,
                                                                 num_codes, num_splits)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _check_workspace(workspace, q.device)
    args = (ctypes.byref(lay), _ptr(q), _dtype_code(q), _ptr(k_new), _ptr(v_new),
            _dtype_code(k_new), _ptr(lam), _ptr(cb_k), _ptr(cb_v), _ptr(codes_k), _ptr(codes_v),
            _ptr(win_k), _ptr(win_v), win_cap, batch, hq, num_codes, win_len, num_splits,
            _ptr(out), _ptr(workspace), workspace.numel())
    return args, lay, out, workspace


def decode_step_window(q, k_new, v_new, lam, cb_k, cb_v, codes_k, codes_v, win_k, win_v,
                       num_codes: int, win_len: int, num_splits: int = 0, out=None,
                       workspace=None):
    """Store k_new / v_new [B][Hkv][128] (as fp16) in window slot ``win_len``
    of win_k / win_v [B][Hkv][win_cap][128], then decode attention over the
    ``num_codes`` coded tokens and window slots 0 .. win_len in one softmax
    -> float32 [B][Hq][128]."""
    args, _, out, _ = _window_step_args(q, k_new, v_new, lam, cb_k, cb_v, codes_k, codes_v,
                                        win_k, win_v, num_codes, win_len, num_splits, out,
                                        workspace)
    _check(library().vq_decode_step_window(*args, _stream(q)), "vq_decode_step_window")
    return out


def prepare_decode_step_window(q, k_new, v_new, lam, cb_k, cb_v, codes_k, codes_v, win_k,
                               win_v, num_codes: int, win_len: int, num_splits: int = 0,
                               out=None, workspace=None) -> PreparedCall:
    """``decode_step_window`` marshalled once; the output is the call's ``out``."""
    args, lay, out, workspace = _window_step_args(q, k_new, v_new, lam, cb_k, cb_v, codes_k,
                                                  codes_v, win_k, win_v, num_codes, win_len,
                                                  num_splits, out, workspace)
    call = PreparedCall("vq_decode_step_window", library().vq_decode_step_window, args,
                        (lay, q, k_new, v_new, lam, cb_k, cb_v, codes_k, codes_v, win_k, win_v,
                         out, workspace), q.device)
    call.out = out
    return call


def flush_window(win_k, win_v, lam, cb_k, cb_v, codes_k, codes_v, num_codes: int) -> None:
    """Encode the full window into code slots [num_codes, num_codes + win_cap)."""
    _check_cache(codes_k, codes_v, cb_k, cb_v, lam)
    win_cap = _check_window(win_k, win_v, codes_k)
    lay = make_layout(codes_k, codes_v, cb_k, cb_v)
    _check(library().vq_flush_window(ctypes.byref(lay), _ptr(win_k), _ptr(win_v), _ptr(lam),
                                     _ptr(cb_k), _ptr(cb_v), _ptr(codes_k), _ptr(codes_v),
                                     win_cap, codes_k.shape[0], num_codes, _stream(win_k)),
           "vq_flush_window")


def decode_step_num_partials(codes_k, codes_v, cb_k, cb_v, batch, num_q_heads, cur_len,
                             requested: int = 0) -> int:
    """Partials of a decode step: attention splits (``requested``, 0 =
    default) + 1 for the new token."""
    lay = make_layout(codes_k, codes_v, cb_k, cb_v)
    return int(library().vq_decode_step_num_partials(ctypes.byref(lay), batch, num_q_heads,
                                                     cur_len, requested))


def decode_step_workspace_bytes(codes_k, codes_v, cb_k, cb_v, batch, num_q_heads, cur_len,
                                requested: int = 0) -> int:
    lay = make_layout(codes_k, codes_v, cb_k, cb_v)
    return int(library().vq_decode_step_workspace_bytes(ctypes.byref(lay), batch, num_q_heads,
                                                        cur_len, requested))


def _step_partials_args(q, k_new, v_new, lam, cb_k, cb_v, codes_k, codes_v, cur_len,
                        num_splits, partials):
    batch, hq = _step_common(q, k_new, v_new, lam, cb_k, cb_v, codes_k, codes_v)
    splits = decode_step_num_partials(codes_k, codes_v, cb_k, cb_v, batch, hq, cur_len,
                                      num_splits)
    if partials is None:
        m = torch.empty((batch, hq, splits), dtype=torch.float32, device=q.device)
        partials = (m, torch.empty_like(m),
                    torch.empty((batch, hq, splits, 128), dtype=torch.float32, device=q.device))
    m, l, o = partials
    for name, t, shape in (("m", m, (batch, hq, splits)), ("l", l, (batch, hq, splits)),
                           ("o", o, (batch, hq, splits, 128))):
        _need(t.is_cuda and t.is_contiguous() and t.dtype == torch.float32
              and tuple(t.shape) == shape and t.device == q.device,
              f"partials {name} must be contiguous float32 {shape} on q's device")
    lay = make_layout(codes_k, codes_v, cb_k, cb_v)
    args = (ctypes.byref(lay), _ptr(q), _dtype_code(q), _ptr(k_new), _ptr(v_new),
            _dtype_code(k_new), _ptr(lam), _ptr(cb_k), _ptr(cb_v), _ptr(codes_k), _ptr(codes_v),
            batch, hq, cur_len, splits, _ptr(m), _ptr(l), _ptr(o))
    return args, lay, partials


def decode_step_partials(q, k_new, v_new, lam, cb_k, cb_v, codes_k, codes_v, cur_len: int,
                         num_splits: int = 0, partials=None):
    """``decode_step``'s split pass alone -> (m, l, o) partials over
    ``decode_step_num_partials(..., num_splits)`` partials (the last is the new
    token's)."""
    args, _, partials = _step_partials_args(q, k_new, v_new, lam, cb_k, cb_v, codes_k, codes_v,
                                            cur_len, num_splits, partials)
    _check(library().vq_decode_step_partials(*args, _stream(q)), "vq_decode_step_partials")
    return partials


def prepare_decode_step_partials(q, k_new, v_new, lam, cb_k, cb_v, codes_k, codes_v,
                                 cur_len: int, num_splits: int = 0,
                                 partials=None) -> PreparedCall:
    """``decode_step_partials`` marshalled once; the partials are the call's
    ``partials`` attribute."""
    args, lay, partials = _step_partials_args(q, k_new, v_new, lam, cb_k, cb_v, codes_k,
                                              codes_v, cur_len, num_splits, partials)
    call = PreparedCall("vq_decode_step_partials", library().vq_decode_step_partials, args,
                        (lay, q, k_new, v_new, lam, cb_k, cb_v, codes_k, codes_v)
                        + tuple(partials), q.device)
    call.partials = partials
    return call


def fp16_attention_workspace_bytes(batch, num_q_heads, num_kv_heads, context_len,
                                   num_splits: int = 0) -> int:
    return int(library().vq_fp16_attention_workspace_bytes(batch, num_q_heads, num_kv_heads,
                                                           context_len, num_splits))


def fp16_decode_attention(q, k, v, context_len: int, num_splits: int = 0, out=None,
                          workspace=None):
    """Uncompressed comparator: q [B][Hq][128], k/v [B][Hkv][cap][128], all fp16."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t.is_cuda and t.is_contiguous() and t.dtype == torch.float16,
              f"{name} must be a contiguous float16 device tensor")
    _need(k.shape == v.shape and k.dim() == 4 and k.shape[3] == 128,
          "k/v must be [B][Hkv][cap][128]")
    _need(q.dim() == 3 and q.shape[2] == 128 and q.shape[0] == k.shape[0],
          "q must be [B][Hq][128] with the cache's B")
    _need(k.device == q.device and v.device == q.device, "q, k and v must share a device")
    batch, hq = q.shape[0], q.shape[1]
    hkv, cap = k.shape[1], k.shape[2]
    if out is None:
        out = torch.empty((batch, hq, 128), dtype=torch.float32, device=q.device)
    _check_out(out, batch, hq, q.device)
    if workspace is None:
        nbytes = fp16_attention_workspace_bytes(batch, hq, hkv, context_len, num_splits)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _check_workspace(workspace, q.device)
    _check(library().vq_fp16_decode_attention(_ptr(q), _ptr(k), _ptr(v), batch, hq, hkv, cap,
                                              context_len, num_splits, _ptr(out),
                                              _ptr(workspace), workspace.numel(), _stream(q)),
           "vq_fp16_decode_attention")
    return out


# --- offline calibration --------------------------------------------------------

def _check_calib_keys(keys):
    _need(keys.is_cuda and keys.is_contiguous() and keys.dim() == 3 and keys.shape[2] == 128,
          "keys must be contiguous [Hkv][T][128]")


def calibrate_lambda(keys: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """lambda = sqrt(max_t |K|) per (KV head, channel) from calibration keys
    [Hkv][T][128] (float16/float32) -> float32 [Hkv][128]."""
    _check_calib_keys(keys)
    if out is None:
        out = torch.empty((keys.shape[0], 128), dtype=torch.float32, device=keys.device)
    _need(out.is_contiguous() and out.dtype == torch.float32 and
          tuple(out.shape) == (keys.shape[0], 128), "out must be contiguous float32 [Hkv][128]")
    _check(library().vq_calibrate_lambda(_ptr(keys), _dtype_code(keys), keys.shape[0],
                                         keys.shape[1], _ptr(out), _stream(keys)),
           "vq_calibrate_lambda")
    return out


def transform_keys(keys: torch.Tensor, lam: torch.Tensor,
                   out: torch.Tensor | None = None) -> torch.Tensor:
    """K~ = K diag(lambda)^-1 H_128 of calibration keys [Hkv][T][128] -> float32
    [Hkv][T][128] (view it as [Hkv][T*32][4] for K-Means)."""
    _check_calib_keys(keys)
    _need(lam.is_cuda and lam.is_contiguous() and lam.dtype == torch.float32 and
          tuple(lam.shape) == (keys.shape[0], 128), "lambda must be contiguous float32 [Hkv][128]")
    if out is None:
        out = torch.empty(keys.shape, dtype=torch.float32, device=keys.device)
    _need(out.is_contiguous() and out.dtype == torch.float32 and out.shape == keys.shape,
          "out must be contiguous float32 like keys")
    _check(library().vq_transform_keys(_ptr(keys), _dtype_code(keys), _ptr(lam), keys.shape[0],
                                       keys.shape[1], _ptr(out), _stream(keys)),
           "vq_transform_keys")
    return out


def kmeans_workspace_bytes(num_sets: int, num_samples: int, code_bits: int,
                           sub_dim: int = 4) -> int:
    return int(library().vq_kmeans_workspace_bytes(num_sets, num_samples, sub_dim, code_bits))


def kmeans(samples: torch.Tensor, init: torch.Tensor, iters: int, *, codebook: bool = True,
           assign: bool = False, centroids: torch.Tensor | None = None,
           workspace: torch.Tensor | None = None):
    """Lloyd K-Means of fp32 samples [S][n][d] from fp64 init [S][2^bits][d]
    (d = 4 or 8).

    Returns (centroids float64 [S][2^bits][d], codebook float16 or None,
    assign int32 [S][n] or None).  ``centroids`` may be ``init`` (updated in
    place); ``workspace`` is an optional reusable uint8 device tensor of at
    least ``kmeans_workspace_bytes(...)`` bytes."""
    _need(samples.is_cuda and samples.is_contiguous() and samples.dtype == torch.float32 and
          samples.dim() == 3, "samples must be contiguous float32 [S][n][d]")
    sub = int(samples.shape[2])
    _need(init.is_cuda and init.is_contiguous() and init.dtype == torch.float64 and
          init.dim() == 3 and init.shape[0] == samples.shape[0] and init.shape[2] == sub,
          "init must be contiguous float64 [S][entries][d] with the samples' d")
    entries = int(init.shape[1])
    bits = entries.bit_length() - 1
    _need(entries == 1 << bits, "the number of centroids must be a power of two")
    sets, n = int(samples.shape[0]), int(samples.shape[1])
    dev = samples.device
    if centroids is None:
        centroids = torch.empty_like(init)
    _need(centroids.is_contiguous() and centroids.dtype == torch.float64 and
          centroids.shape == init.shape, "centroids must be contiguous float64 like init")
    cb = torch.empty(init.shape, dtype=torch.float16, device=dev) if codebook else None
    asg = torch.empty((sets, n), dtype=torch.int32, device=dev) if assign else None
    need = kmeans_workspace_bytes(sets, n, bits, sub)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check(library().vq_kmeans(_ptr(samples), sets, n, sub, bits, _ptr(init), int(iters),
                               _ptr(centroids), _ptr(cb), _ptr(asg), _ptr(workspace),
                               workspace.numel(), _stream(samples)),
           "vq_kmeans")
    return centroids, cb, asg
