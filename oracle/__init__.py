"""fp64 CPU oracle of the ReplaySSM decode path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check in ``__graft_entry__`` and the CPU-baseline leg
of ``bench.py`` may import this package.  The product path (the HIP library
and its Python binding) never imports, links or calls it, and this package
never imports the product.  The two share nothing but the seeded input
generators in ``synth``.

What it computes (article "NVIDIA ReplaySSM: hybrid model SSM decoding with a
state buffer", devotd.net; English edition sections 1-4):

* ``recurrent``   -- the conventional per-token SSM update (section 1),
                     y uses the post-update state.
* ``spec_round``  -- speculative verification (section 3): outputs for T
                     draft positions, then only ``n_keep`` positions applied.
* ``decode_run``  -- a whole decode run of a layer: since replay from a
                     checkpoint plus buffered inputs reproduces the recurrence
                     exactly (section 1), the oracle for every replay output
                     and every interval checkpoint is the recurrence itself,
                     evaluated token by token.
* codecs, Philox4x32-10 and stochastic rounding for the precision split
  (section 4).  The split path's outputs and commits are the recurrence
  replayed from the exactly decoded output copy / update checkpoint (the
  tests anchor it on the stored bytes at each commit).

The arithmetic lives in ``oracle.c`` (plain C, fp64); this module only
marshals numpy arrays.  Inputs arrive as their stored values (fp32 or bf16)
and are promoted exactly to fp64 here.
"""
from __future__ import annotations

import ctypes
import functools
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

_i64 = ctypes.c_int64
_u64 = ctypes.c_uint64
_u32 = ctypes.c_uint32
_dp = ctypes.POINTER(ctypes.c_double)
_fp = ctypes.POINTER(ctypes.c_float)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_u32p = ctypes.POINTER(ctypes.c_uint32)
_i32p = ctypes.POINTER(ctypes.c_int32)


def lib():
    """Load (building on first use if absent) the oracle shared library."""
    global _LIB
    if _LIB is None:
        path = os.path.join(_HERE, "liboracle.so")
        src = os.path.join(_HERE, "oracle.c")
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(src):
            _build.build()
        L = ctypes.CDLL(path)
        L.oracle_recurrent.argtypes = [_i64] * 6 + [_dp] * 8
        L.oracle_recurrent.restype = None
        L.oracle_spec_round.argtypes = [_i64] * 6 + [_dp] * 7 + [_i32p, _dp]
        L.oracle_spec_round.restype = None
        L.oracle_philox4x32_10.argtypes = [_u32p, _u32p, _u32p]
        L.oracle_philox4x32_10.restype = None
        L.oracle_sr_draw.argtypes = [_u64, _u32, _u32, _u64]
        L.oracle_sr_draw.restype = _u32
        L.oracle_bf16_decode.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_decode.restype = ctypes.c_double
        L.oracle_bf16_sr.argtypes = [ctypes.c_float, _u32]
        L.oracle_bf16_sr.restype = ctypes.c_uint16
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_decode.restype = ctypes.c_double
        L.oracle_e4m3_rne.argtypes = [ctypes.c_double]
        L.oracle_e4m3_rne.restype = ctypes.c_uint8
        L.oracle_e4m3_sr.argtypes = [ctypes.c_float, _u32]
        L.oracle_e4m3_sr.restype = ctypes.c_uint8
        L.oracle_e2m1_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e2m1_decode.restype = ctypes.c_double
        L.oracle_fp4_quantize.argtypes = [_fp, _i64, _u8p, _u8p]
        L.oracle_fp4_quantize.restype = None
        L.oracle_fp4_dequantize.argtypes = [_u8p, _u8p, _i64, _dp]
        L.oracle_fp4_dequantize.restype = None
        L.oracle_sr_quantize.argtypes = [_fp, _i64, ctypes.c_int, _u64, _u32, _u32, _u64, _u8p]
        L.oracle_sr_quantize.restype = None
        L.oracle_num_threads.argtypes = []
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_set_num_threads.argtypes = [ctypes.c_int]
        L.oracle_set_num_threads.restype = None
        _LIB = L
    return _LIB


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """OpenMP threads for later oracle calls (the parallel loops run over
    independent (slot, head) pairs, so results do not depend on it)."""
    lib().oracle_set_num_threads(int(n))


def _f64(a) -> np.ndarray:
    """Exact promotion of stored values (fp32 / fp64 numpy, or a torch CPU
    tensor of any float dtype incl. bf16) to a C-contiguous fp64 array."""
    if hasattr(a, "detach"):  # torch tensor
        a = a.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray, ct):
    return a.ctypes.data_as(ct)


# --------------------------------------------------------------------------
# The recurrence and the speculative round.
# --------------------------------------------------------------------------

def recurrent(S, x, Bm, Cm, dt, A, D, groups: int):
    """Run the per-token recurrence over ``steps`` tokens.

    S [batch, H, P, N]; x [steps, batch, H, P]; Bm, Cm [steps, batch, G, N];
    dt [steps, batch, H]; A, D [H].  Returns (S_final fp64, y fp64
    [steps, batch, H, P])."""
    S = _f64(S).copy()
    x, Bm, Cm, dt, A, D = (_f64(t) for t in (x, Bm, Cm, dt, A, D))
    steps, batch, H, P = x.shape
    N = S.shape[-1]
    assert S.shape == (batch, H, P, N)
    assert Bm.shape == (steps, batch, groups, N) and Cm.shape == Bm.shape
    assert dt.shape == (steps, batch, H) and A.shape == (H,) and D.shape == (H,)
    y = np.empty((steps, batch, H, P), dtype=np.float64)
    lib().oracle_recurrent(batch, H, P, N, groups, steps, _ptr(S, _dp),
                           _ptr(x, _dp), _ptr(Bm, _dp), _ptr(Cm, _dp), _ptr(dt, _dp),
                           _ptr(A, _dp), _ptr(D, _dp), _ptr(y, _dp))
    return S, y


def spec_round(S, x, Bm, Cm, dt, A, D, n_keep, groups: int):
    """One speculative round of T draft positions (shapes as ``recurrent``
    with steps = T).  Returns (S after n_keep[b] positions, y for all T)."""
    S = _f64(S).copy()
    x, Bm, Cm, dt, A, D = (_f64(t) for t in (x, Bm, Cm, dt, A, D))
    T, batch, H, P = x.shape
    N = S.shape[-1]
    nk = np.ascontiguousarray(np.asarray(n_keep, dtype=np.int32))
    assert nk.shape == (batch,) and np.all((nk >= 0) & (nk <= T))
    y = np.empty((T, batch, H, P), dtype=np.float64)
    lib().oracle_spec_round(batch, H, P, N, groups, T, _ptr(S, _dp),
                            _ptr(x, _dp), _ptr(Bm, _dp), _ptr(Cm, _dp), _ptr(dt, _dp),
                            _ptr(A, _dp), _ptr(D, _dp), _ptr(nk, _i32p), _ptr(y, _dp))
    return S, y


# --------------------------------------------------------------------------
# Codecs, Philox and stochastic rounding.
# --------------------------------------------------------------------------

def philox4x32_10(counter, key):
    c = (ctypes.c_uint32 * 4)(*[int(v) & 0xFFFFFFFF for v in counter])
    k = (ctypes.c_uint32 * 2)(*[int(v) & 0xFFFFFFFF for v in key])
    o = (ctypes.c_uint32 * 4)()
    lib().oracle_philox4x32_10(c, k, o)
    return [int(v) for v in o]


def sr_draw(seed: int, layer: int, interval: int, elem: int) -> int:
    return int(lib().oracle_sr_draw(seed, layer, interval, elem))


def bf16_decode(code: int) -> float:
    return float(lib().oracle_bf16_decode(code))


def bf16_sr(v: float, r16: int) -> int:
    return int(lib().oracle_bf16_sr(v, r16))


def e4m3_decode(code: int) -> float:
    return float(lib().oracle_e4m3_decode(code))


def e4m3_rne(v: float) -> int:
    return int(lib().oracle_e4m3_rne(v))


def e4m3_sr(v: float, r16: int) -> int:
    return int(lib().oracle_e4m3_sr(v, r16))


def e2m1_decode(code: int) -> float:
    return float(lib().oracle_e2m1_decode(code))


def fp4_quantize(v):
    """fp32 values (last dim a multiple of 32) -> (codes u8 [..., n/2],
    scales u8 [..., n/32])."""
    v = np.ascontiguousarray(np.asarray(v, dtype=np.float32))
    n = v.size
    assert v.shape[-1] % 32 == 0
    codes = np.zeros(v.shape[:-1] + (v.shape[-1] // 2,), dtype=np.uint8)
    scales = np.zeros(v.shape[:-1] + (v.shape[-1] // 32,), dtype=np.uint8)
    lib().oracle_fp4_quantize(_ptr(v, _fp), n, _ptr(codes, _u8p), _ptr(scales, _u8p))
    return codes, scales


def fp4_dequantize(codes, scales):
    codes = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
    scales = np.ascontiguousarray(np.asarray(scales, dtype=np.uint8))
    n = codes.size * 2
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), dtype=np.float64)
    lib().oracle_fp4_dequantize(_ptr(codes, _u8p), _ptr(scales, _u8p), n, _ptr(out, _dp))
    return out


def sr_quantize(v, fmt: str, seed: int, layer: int, interval: int, elem0: int = 0):
    """Stochastically round fp32 values to 'bf16' (returns u16 codes) or 'e4m3'
    (u8 codes); element i uses the draw of global element elem0 + i."""
    v = np.ascontiguousarray(np.asarray(v, dtype=np.float32))
    f = {"bf16": 0, "e4m3": 1}[fmt]
    nbytes = v.size * (2 if f == 0 else 1)
    out = np.empty(nbytes, dtype=np.uint8)
    lib().oracle_sr_quantize(_ptr(v, _fp), v.size, f, seed, layer, interval, elem0,
                             _ptr(out, _u8p))
    if f == 0:
        return out.view("<u2").reshape(v.shape)
    return out.reshape(v.shape)


@functools.lru_cache(maxsize=None)
def _table(kind: str) -> np.ndarray:
    L = lib()
    if kind == "bf16":
        return np.array([L.oracle_bf16_decode(i) for i in range(65536)], dtype=np.float64)
    if kind == "e4m3":
        return np.array([L.oracle_e4m3_decode(i) for i in range(256)], dtype=np.float64)
    if kind == "e2m1":
        return np.array([L.oracle_e2m1_decode(i) for i in range(16)], dtype=np.float64)
    raise ValueError(kind)


def bf16_decode_array(codes) -> np.ndarray:
    """Exact decode of u16 bf16 codes through the C decoder (tabulated)."""
    return _table("bf16")[np.asarray(codes, dtype=np.uint16)]


def e4m3_decode_array(codes) -> np.ndarray:
    """Exact decode of u8 E4M3 codes through the C decoder (tabulated)."""
    return _table("e4m3")[np.asarray(codes, dtype=np.uint8)]


from .drivers import decode_run, spec_run  # noqa: E402,F401
