"""Python binding of libsq (ctypes): argument marshalling only.

Every function here forwards to the C ABI declared in include/sq.h with the
same name; all computation happens in the HIP library (device calls) or in its
host-side calibration.  Device tensors are torch tensors on the current HIP
device; work is enqueued on torch's current stream.

The library is built in-tree (``python -m compression_sq_compress_amd.build``);
if it is missing it is built once on first import, and any failure raises --
there is no fallback implementation.  A library built from other sources than
the ones beside it (its compiled-in source digest differs) is refused.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsq.so")

SQ_F32, SQ_BF16 = 0, 1
_STATUS = {0: "SQ_OK", 1: "SQ_ERR_ARG", 2: "SQ_ERR_UNSUPPORTED", 3: "SQ_ERR_NUMERIC",
           4: "SQ_ERR_HIP", 5: "SQ_ERR_ALLOC", 6: "SQ_ERR_IO", 7: "SQ_ERR_STATE"}

# symbols declared in include/sq.h
EXPORTS = ("sq_calib_default_opts", "sq_calibrate", "sq_calib_upload", "sq_calib_n_heads",
           "sq_calib_info", "sq_calib_export", "sq_calib_save", "sq_calib_load",
           "sq_calib_destroy", "sq_packed_head_words", "sq_compress", "sq_compress_append", "sq_scores",
           "sq_attend_workspace_bytes", "sq_attend", "sq_dequantize", "sq_unpack",
           "sq_last_error", "sq_build_digest", "sq_plan_decode",
           "sq_attend_noalloc", "sq_decode", "sq_calibrate_tq", "sq_calibrate_device",
           "sq_paged_block_words", "sq_compress_append_paged", "sq_decode_paged")


class StaleLibraryError(RuntimeError):
    """libsq.so does not match the sources beside it."""


class SQError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


class CalibOpts(C.Structure):
    _fields_ = [("head_dim", C.c_int), ("avg_bits", C.c_double),
                ("qjl_bits_per_signal_dim", C.c_int), ("max_bits", C.c_int),
                ("lloyd_max_iters", C.c_int), ("n_threads", C.c_int), ("normalize", C.c_int),
                ("deff_cumvar", C.c_double)]


class HeadInfo(C.Structure):
    _fields_ = [("head_dim", C.c_int), ("d_eff", C.c_int), ("m", C.c_int),
                ("code_bits", C.c_int), ("record_words", C.c_int),
                ("n_thresholds", C.c_int), ("n_centroids", C.c_int),
                ("n_regions", C.c_int), ("lloyd_unconverged", C.c_int),
                ("participation_ratio", C.c_double), ("kappa", C.c_double),
                ("normalized", C.c_int)]


class Paged(C.Structure):
    """sq_paged: block table (device int32 [batch][table_stride]), tiles per block, pool blocks."""
    _fields_ = [("block_table", C.c_void_p), ("table_stride", C.c_int64), ("block_tiles", C.c_int32),
                ("n_blocks", C.c_int32)]


class DecodePlan(C.Structure):
    _fields_ = [("score_passes", C.c_int), ("score_quads", C.c_int), ("score_wave_groups", C.c_int),
                ("attend_placement", C.c_int), ("attend_waves", C.c_int), ("attend_blocks", C.c_int),
                ("attend_chunks", C.c_int), ("decode_launches", C.c_int),
                ("decode_waves", C.c_int), ("decode_lds_bytes", C.c_int)]


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from .build import build
        build()
    lib = C.CDLL(LIB_PATH)
    from .digest import source_digest
    lib.sq_build_digest.restype = C.c_char_p
    lib.sq_build_digest.argtypes = []
    built, want = lib.sq_build_digest().decode(), source_digest()
    if built != want:
        raise StaleLibraryError(
            f"{LIB_PATH} was built from other sources (digest {built}, sources {want}); "
            "rebuild it with: python -m compression_sq_compress_amd.build")
    P, I, I64, U64 = C.c_void_p, C.c_int, C.c_int64, C.c_size_t
    sig = {
        "sq_calib_default_opts": (I, [C.POINTER(CalibOpts), I]),
        "sq_calibrate": (I, [P, I, I64, C.POINTER(CalibOpts), P, C.POINTER(C.c_void_p)]),
        "sq_calib_upload": (I, [P, P]),
        "sq_calib_n_heads": (I, [P]),
        "sq_calib_info": (I, [P, I, C.POINTER(HeadInfo)]),
        "sq_calib_export": (I, [P, I, P, P, P, P, P, P]),
        "sq_calib_save": (I, [P, C.c_char_p]),
        "sq_calib_load": (I, [C.c_char_p, C.POINTER(C.c_void_p)]),
        "sq_calib_destroy": (None, [P]),
        "sq_packed_head_words": (I64, [P, I64]),
        "sq_compress": (I, [P, I, I, I, I, P, I, I64, I64, I64, I64, P, I64, I64, P]),
        "sq_compress_append": (I, [P, I, I, I, I, P, I, I64, I64, I64, I64, P, I64, I64, I64, P]),
        "sq_scores": (I, [P, I, I, I, I, I, P, I, P, I64, I64, I64, P, P]),
        "sq_attend_workspace_bytes": (U64, [I, I, I64, I]),
        "sq_attend": (I, [P, I, I, I, I, I, P, C.c_float, P, I64, I64, I64, P, U64, P, P]),
        "sq_dequantize": (I, [P, I, I, I, I, P, I64, I64, I64, P, P]),
        "sq_unpack": (I, [P, I, P, I64, P, P, P, P]),
        "sq_calibrate_tq": (I, [P, P, I, C.POINTER(CalibOpts), C.POINTER(C.c_void_p)]),
        "sq_calibrate_device": (I, [P, I, I64, C.POINTER(CalibOpts), P, P, C.POINTER(C.c_void_p)]),
        "sq_paged_block_words": (I64, [P, I]),
        "sq_compress_append_paged": (I, [P, I, I, I, I, P, I, I64, I64, I64, I64, P, C.POINTER(Paged), I64, P]),
        "sq_decode_paged": (I, [P, P, I, I, I, I, I, P, I, P, P, C.POINTER(Paged), I64, C.c_float, P, U64, P, P]),
        "sq_last_error": (C.c_char_p, []),
        "sq_build_digest": (C.c_char_p, []),
        "sq_plan_decode": (I, [P, P, I, I, I, I, I, I64, C.POINTER(DecodePlan)]),
        "sq_attend_noalloc": (I, [P, I, I, I, I, I, P, C.c_float, P, I64, I64, I64, P, P]),
        "sq_decode": (I, [P, P, I, I, I, I, I, P, I, P, I64, I64, P, I64, I64, I64, C.c_float, P, U64,
                          P, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def lib():
    return _load()


def _check(st: int):
    if st != 0:
        raise SQError(st, _load().sq_last_error().decode())


def _ptr(a) -> Optional[int]:
    if a is None:
        return None
    if isinstance(a, np.ndarray):
        return a.ctypes.data
    return a.data_ptr()


def _stream(stream=None) -> Optional[int]:
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


# ------------------------------------------------------------------ calibration

class Calibration:
    """Owns an ``sq_calib`` handle."""

    def __init__(self, handle: int):
        self.handle = C.c_void_p(handle)

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value and _lib is not None:
            _lib.sq_calib_destroy(h)
            self.handle = C.c_void_p(0)

    @property
    def n_heads(self) -> int:
        return _load().sq_calib_n_heads(self.handle)

    def upload(self, stream=None):
        _check(_load().sq_calib_upload(self.handle, _stream(stream)))
        return self

    def info(self, head: int) -> HeadInfo:
        out = HeadInfo()
        _check(_load().sq_calib_info(self.handle, head, C.byref(out)))
        return out

    def export(self, head: int) -> dict:
        inf = self.info(head)
        d = inf.head_dim
        lam = np.zeros(d, np.float64)
        R = np.zeros((d, d), np.float64)
        w = np.zeros(d, np.int32)
        thr = np.zeros(max(1, inf.n_thresholds), np.float32)
        cent = np.zeros(max(1, inf.n_centroids), np.float32)
        S = np.zeros(max(1, inf.m * inf.d_eff), np.float32)
        _check(_load().sq_calib_export(self.handle, head, _ptr(lam), _ptr(R), _ptr(w),
                                       _ptr(thr), _ptr(cent), _ptr(S)))
        return dict(eigenvalues=lam, rotation=R, widths=w, thresholds=thr[:inf.n_thresholds],
                    centroids=cent[:inf.n_centroids],
                    qjl=S[:inf.m * inf.d_eff].reshape(inf.m, inf.d_eff), info=inf)

    def save(self, path: str):
        _check(_load().sq_calib_save(self.handle, path.encode()))

    @staticmethod
    def load(path: str) -> "Calibration":
        h = C.c_void_p()
        _check(_load().sq_calib_load(path.encode(), C.byref(h)))
        return Calibration(h.value)

    def packed_head_words(self, n_tokens: int) -> int:
        return int(_load().sq_packed_head_words(self.handle, n_tokens))


def sq_calib_default_opts(head_dim: int) -> CalibOpts:
    o = CalibOpts()
    _check(_load().sq_calib_default_opts(C.byref(o), head_dim))
    return o


def _calib_opts(d, avg_bits, qjl_bits, max_bits, lloyd_max_iters, n_threads, normalize,
                deff_cumvar) -> CalibOpts:
    o = sq_calib_default_opts(d)
    o.avg_bits = float(avg_bits)
    o.qjl_bits_per_signal_dim = int(qjl_bits)
    o.max_bits = int(max_bits)
    o.lloyd_max_iters = int(lloyd_max_iters)
    o.n_threads = int(n_threads)
    o.normalize = 1 if normalize else 0
    o.deff_cumvar = float(deff_cumvar)
    return o


def _gauss(qjl_gauss, H, qjl_bits, d):
    if qjl_gauss is None:
        return None
    g = np.ascontiguousarray(qjl_gauss, dtype=np.float32)
    assert g.shape == (H, max(1, qjl_bits) * d, d), g.shape
    return g


def sq_calibrate(samples: np.ndarray, avg_bits: float, qjl_bits: int,
                 qjl_gauss: Optional[np.ndarray] = None, max_bits: int = 8,
                 lloyd_max_iters: int = 200, n_threads: int = 0,
                 normalize: bool = False, deff_cumvar: float = 0.0) -> Calibration:
    """samples: host float32 [n_heads][n_samples][d]; qjl_gauss: host float32
    [n_heads][qjl_bits*d][d] (required when qjl_bits > 0); normalize: the
    normalised variant (per-vector norm stored); deff_cumvar: 0 for d_eff by
    the rounded participation ratio, else the cumulative-variance fraction."""
    x = np.ascontiguousarray(samples, dtype=np.float32)
    assert x.ndim == 3
    H, n, d = x.shape
    o = _calib_opts(d, avg_bits, qjl_bits, max_bits, lloyd_max_iters, n_threads, normalize, deff_cumvar)
    g = _gauss(qjl_gauss, H, qjl_bits, d)
    h = C.c_void_p()
    _check(_load().sq_calibrate(_ptr(x), H, n, C.byref(o), _ptr(g), C.byref(h)))
    return Calibration(h.value)


def sq_calibrate_device(samples, avg_bits: float, qjl_bits: int,
                        qjl_gauss: Optional[np.ndarray] = None, max_bits: int = 8,
                        lloyd_max_iters: int = 200, n_threads: int = 0,
                        normalize: bool = False, deff_cumvar: float = 0.0,
                        stream=None) -> Calibration:
    """As sq_calibrate with samples a contiguous device float32 tensor
    [n_heads][n_samples][d] (covariance, eigendecomposition and rotation on
    the GPU); qjl_gauss stays a host array."""
    assert samples.is_cuda and samples.dim() == 3 and samples.is_contiguous()
    import torch
    assert samples.dtype == torch.float32
    H, n, d = samples.shape
    o = _calib_opts(d, avg_bits, qjl_bits, max_bits, lloyd_max_iters, n_threads, normalize, deff_cumvar)
    g = _gauss(qjl_gauss, H, qjl_bits, d)
    h = C.c_void_p()
    _check(_load().sq_calibrate_device(_ptr(samples), H, n, C.byref(o), _ptr(g), _stream(stream),
                                       C.byref(h)))
    return Calibration(h.value)


def sq_calibrate_tq(rotation: np.ndarray, bits: int, keys: bool,
                    qjl_gauss: Optional[np.ndarray] = None) -> Calibration:
    """TurboQuant-style calibration: rotation host float32 [n_heads][d][d];
    keys: (bits - 1)-bit codes + QJL over all dims from qjl_gauss [n_heads][d][d];
    values: bits-bit codes."""
    r = np.ascontiguousarray(rotation, dtype=np.float32)
    assert r.ndim == 3 and r.shape[1] == r.shape[2]
    H, d, _ = r.shape
    o = sq_calib_default_opts(d)
    o.avg_bits = float(bits)
    o.qjl_bits_per_signal_dim = 1 if keys else 0
    g = None
    if keys:
        g = np.ascontiguousarray(qjl_gauss, dtype=np.float32)
        assert g.shape == (H, d, d), g.shape
    h = C.c_void_p()
    _check(_load().sq_calibrate_tq(_ptr(r), _ptr(g), H, C.byref(o), C.byref(h)))
    return Calibration(h.value)


# ------------------------------------------------------------------ device calls

def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return SQ_F32
    if t.dtype == torch.bfloat16:
        return SQ_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def sq_compress(cal: Calibration, x, packed, first_head: int = 0, calib_batch_stride: int = 0,
                stream=None):
    """x: device [batch][n_heads][T][d] (last dim contiguous, any other strides);
    packed: device int32/uint32 [batch][n_heads][>= packed_head_words(T)]."""
    assert x.dim() == 4 and x.stride(3) == 1 and x.is_cuda
    B, H, T, d = x.shape
    assert packed.dim() == 3 and packed.stride(2) == 1 and packed.element_size() == 4
    _check(_load().sq_compress(cal.handle, first_head, H, B, calib_batch_stride, _ptr(x),
                               _dtype_code(x), T, x.stride(0), x.stride(1), x.stride(2),
                               _ptr(packed), packed.stride(0), packed.stride(1), _stream(stream)))


def sq_compress_append(cal: Calibration, x, packed, token0: int, first_head: int = 0,
                       calib_batch_stride: int = 0, stream=None):
    """As sq_compress, with token t of x going to token slot token0 + t of each
    head's packed slot (packed: [batch][n_heads][>= packed_head_words(token0 + T)])."""
    assert x.dim() == 4 and x.stride(3) == 1 and x.is_cuda
    B, H, T, d = x.shape
    assert packed.dim() == 3 and packed.stride(2) == 1 and packed.element_size() == 4
    _check(_load().sq_compress_append(cal.handle, first_head, H, B, calib_batch_stride, _ptr(x),
                                      _dtype_code(x), T, x.stride(0), x.stride(1), x.stride(2),
                                      _ptr(packed), packed.stride(0), packed.stride(1), int(token0),
                                      _stream(stream)))


def sq_scores(cal: Calibration, q, kpacked, n_tokens: int, scores, n_kv_heads: int,
              first_head: int = 0, calib_batch_stride: int = 0, stream=None):
    """q: device [batch][n_q_heads][d] contiguous; kpacked [batch][n_kv][slot];
    scores: device float32 [batch][n_q_heads][n_tokens]."""
    import torch
    assert q.is_contiguous() and q.dim() == 3
    B, Hq, d = q.shape
    assert scores.dtype == torch.float32 and scores.is_contiguous()
    assert tuple(scores.shape) == (B, Hq, n_tokens)
    _check(_load().sq_scores(cal.handle, first_head, calib_batch_stride, B, Hq, n_kv_heads,
                             _ptr(q), _dtype_code(q), _ptr(kpacked), kpacked.stride(0),
                             kpacked.stride(1), n_tokens, _ptr(scores), _stream(stream)))


def sq_attend_workspace_bytes(batch: int, n_q_heads: int, n_tokens: int, head_dim: int) -> int:
    return int(_load().sq_attend_workspace_bytes(batch, n_q_heads, n_tokens, head_dim))


def sq_attend(cal: Calibration, scores, scale: float, vpacked, n_tokens: int, workspace, out,
              n_kv_heads: int, first_head: int = 0, calib_batch_stride: int = 0, stream=None):
    """scores float32 [batch][n_q][n_tokens]; out float32 [batch][n_q][d]."""
    import torch
    B, Hq, d = out.shape
    assert out.dtype == torch.float32 and out.is_contiguous()
    assert scores.is_contiguous() and scores.dtype == torch.float32
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_load().sq_attend(cal.handle, first_head, calib_batch_stride, B, Hq, n_kv_heads,
                             _ptr(scores), float(scale), _ptr(vpacked), vpacked.stride(0),
                             vpacked.stride(1), n_tokens, _ptr(workspace), ws_bytes, _ptr(out),
                             _stream(stream)))


def sq_decode(kcal: Calibration, vcal: Calibration, q, kpacked, vpacked, n_tokens: int, scale: float,
              workspace, out, n_kv_heads: int, first_head: int = 0, calib_batch_stride: int = 0,
              stream=None):
    """Fused decode step: q device [batch][n_q_heads][d] contiguous; kpacked /
    vpacked [batch][n_kv][slot]; workspace of sq_attend_workspace_bytes;
    out float32 [batch][n_q_heads][d]."""
    import torch
    assert q.is_contiguous() and q.dim() == 3
    B, Hq, d = q.shape
    assert out.dtype == torch.float32 and out.is_contiguous() and tuple(out.shape) == (B, Hq, d)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_load().sq_decode(kcal.handle, vcal.handle, first_head, calib_batch_stride, B, Hq, n_kv_heads,
                             _ptr(q), _dtype_code(q), _ptr(kpacked), kpacked.stride(0), kpacked.stride(1),
                             _ptr(vpacked), vpacked.stride(0), vpacked.stride(1), n_tokens, float(scale),
                             _ptr(workspace), ws_bytes, _ptr(out), _stream(stream)))


def paged(block_table, block_tiles: int, n_blocks: int) -> Paged:
    """Describe a paged cache: block_table device int32 [batch][table_stride]."""
    import torch
    assert block_table.is_cuda and block_table.dtype == torch.int32 and block_table.dim() == 2
    assert block_table.stride(1) == 1
    pg = Paged(block_table.data_ptr(), block_table.stride(0), int(block_tiles), int(n_blocks))
    # the description holds the table's address only: keep the tensor alive
    # with it, or the caching allocator may hand that memory to another tensor
    pg._table = block_table
    return pg


def sq_paged_block_words(cal: Calibration, block_tiles: int) -> int:
    return int(_load().sq_paged_block_words(cal.handle, int(block_tiles)))


def sq_compress_append_paged(cal: Calibration, x, pool, pg: Paged, token0: int, first_head: int = 0,
                             calib_batch_stride: int = 0, stream=None):
    """sq_compress_append into a paged pool (device int32/uint32, flat):
    x device [batch][n_heads][T][d]; pg from paged()."""
    assert x.dim() == 4 and x.stride(3) == 1 and x.is_cuda
    B, H, T, d = x.shape
    assert pool.is_cuda and pool.element_size() == 4
    _check(_load().sq_compress_append_paged(cal.handle, first_head, H, B, calib_batch_stride, _ptr(x),
                                            _dtype_code(x), T, x.stride(0), x.stride(1), x.stride(2),
                                            _ptr(pool), C.byref(pg), int(token0), _stream(stream)))


def sq_decode_paged(kcal: Calibration, vcal: Calibration, q, kpool, vpool, pg: Paged, n_tokens: int,
                    scale: float, workspace, out, n_kv_heads: int, first_head: int = 0,
                    calib_batch_stride: int = 0, stream=None):
    """sq_decode over paged key / value pools sharing the block table of pg."""
    import torch
    assert q.is_contiguous() and q.dim() == 3
    B, Hq, d = q.shape
    assert out.dtype == torch.float32 and out.is_contiguous() and tuple(out.shape) == (B, Hq, d)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_load().sq_decode_paged(kcal.handle, vcal.handle, first_head, calib_batch_stride, B, Hq, n_kv_heads,
                                   _ptr(q), _dtype_code(q), _ptr(kpool), _ptr(vpool), C.byref(pg), n_tokens,
                                   float(scale), _ptr(workspace), ws_bytes, _ptr(out), _stream(stream)))


def sq_attend_noalloc(cal: Calibration, scores, scale: float, vpacked, n_tokens: int, out,
                      n_kv_heads: int, first_head: int = 0, calib_batch_stride: int = 0, stream=None):
    """sq_attend with the partials in the library's fixed device scratch
    (no workspace argument, nothing allocated)."""
    import torch
    B, Hq, d = out.shape
    assert out.dtype == torch.float32 and out.is_contiguous()
    assert scores.is_contiguous() and scores.dtype == torch.float32
    _check(_load().sq_attend_noalloc(cal.handle, first_head, calib_batch_stride, B, Hq, n_kv_heads,
                                     _ptr(scores), float(scale), _ptr(vpacked), vpacked.stride(0),
                                     vpacked.stride(1), n_tokens, _ptr(out), _stream(stream)))


def sq_dequantize(cal: Calibration, packed, n_tokens: int, out, first_head: int = 0,
                  calib_batch_stride: int = 0, stream=None):
    """out float32 [batch][n_heads][n_tokens][d]."""
    B, H = out.shape[0], out.shape[1]
    assert out.is_contiguous()
    _check(_load().sq_dequantize(cal.handle, first_head, H, B, calib_batch_stride,
                                 _ptr(packed), packed.stride(0), packed.stride(1), n_tokens,
                                 _ptr(out), _stream(stream)))


def sq_plan_decode(kcal: Optional[Calibration], vcal: Optional[Calibration], batch: int,
                   n_q_heads: int, n_kv_heads: int, n_tokens: int, first_head: int = 0,
                   calib_batch_stride: int = 0) -> DecodePlan:
    """Diagnostic: how sq_scores / sq_attend would launch for these sizes."""
    out = DecodePlan()
    _check(_load().sq_plan_decode(kcal.handle if kcal else None, vcal.handle if vcal else None,
                                  first_head, calib_batch_stride, batch, n_q_heads, n_kv_heads,
                                  n_tokens, C.byref(out)))
    return out


def sq_unpack(cal: Calibration, head: int, packed_host: np.ndarray, n_tokens: int,
              with_norm: bool = False):
    """Host decode of one head's slot -> (codes uint8 [T][d], qjl uint8 [T][m],
    gamma float32 [T]) and, with with_norm, nu float32 [T]."""
    inf = cal.info(head)
    p = np.ascontiguousarray(packed_host).view(np.uint32)
    need = -(-n_tokens // 64) * 64 * inf.record_words
    assert p.size >= need
    codes = np.zeros((n_tokens, inf.head_dim), np.uint8)
    qjl = np.zeros((n_tokens, max(1, inf.m)), np.uint8)
    gamma = np.zeros(n_tokens, np.float32)
    nu = np.zeros(n_tokens, np.float32)
    _check(_load().sq_unpack(cal.handle, head, _ptr(p), n_tokens, _ptr(codes), _ptr(qjl),
                             _ptr(gamma), _ptr(nu)))
    if with_norm:
        return codes, qjl[:, :inf.m], gamma, nu
    return codes, qjl[:, :inf.m], gamma
