"""Oracle for the vision PatchEmbed -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may import this
package. The product path (the HIP library and its Python binding) never loads it and shares
no code with it.

The PatchEmbed arithmetic lives in ``pe_oracle.c`` (plain C, fp64, a direct five-loop Conv3d per
output row; its header states the definition and the passages of the pages it follows). This
module compiles it with gcc on first use, converts inputs to fp64 exactly and calls it via
ctypes. The PatchMerger front end (``layer_norm``, ``merger_front``) is plain numpy in fp64.

Parity pins for every function here are in ``tests/test_oracle.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pe_oracle.c")
_LIB = os.path.join(_HERE, "libpe_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, IEEE semantics: no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                               "-shared", "-fPIC", "-pthread", _SRC, "-o", tmp])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.POINTER
        lib.pe_oracle_forward.restype = ctypes.c_int
        lib.pe_oracle_forward.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, P(ctypes.c_int32), P(ctypes.c_int32),
            P(ctypes.c_double), P(ctypes.c_double), P(ctypes.c_double), P(ctypes.c_int64),
            ctypes.c_int64, P(ctypes.c_double), ctypes.c_int]
        lib.pe_oracle_num_rows.restype = ctypes.c_int64
        lib.pe_oracle_num_rows.argtypes = [P(ctypes.c_int32), ctypes.c_int]
        lib.pe_oracle_row_positions.restype = ctypes.c_int
        lib.pe_oracle_row_positions.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, P(ctypes.c_int32), P(ctypes.c_int32), P(ctypes.c_int32)]
        _lib = lib
    return _lib


def _f64(a):
    """Exact fp64 copy of a torch tensor (any float dtype) or array-like."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            return np.ascontiguousarray(a.detach().to("cpu").to(torch.float64).numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _i32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32).reshape(-1))


def _ptr(a, ct):
    return a.ctypes.data_as(ctypes.POINTER(ct)) if a is not None else None


# Significant bits (implicit one included) and the exponent of the smallest normal number of
# the two storage formats. Both have an 8-bit exponent field: bf16 is fp32 with 16 fewer
# fraction bits.
_FORMATS = {"bf16": (8, -126), "f32": (24, -126)}


def round_to(a, dtype: str):
    """Round each value ONCE to ``dtype`` ("bf16" or "f32"), round-to-nearest, ties to even,
    and return the results as fp64 (exact: both formats are subsets of fp64).

    This is the cast of the input to the weight dtype that the Qwen3-VL module applies before its
    convolution ("Optimize VLM PatchEmbed", the forward of the Qwen3VLVisionPatchEmbed class),
    written from the definition of the format rather than through another cast, so that an
    fp64 value that is not an fp32 value is also rounded once:
      - a finite nonzero v = f * 2^e with 0.5 <= |f| < 1 has, in a format with `bits` significant
        bits and smallest normal exponent emin, the spacing q = 2^(max(e, emin + 1) - bits)
        (below the normal range the spacing stays that of the subnormals);
      - v / q is exact in fp64 (a power-of-two scaling), np.rint rounds it to the nearest integer
        with ties to even, and multiplying back by q is exact;
      - a result at or beyond 2^128 overflows to infinity with the sign of v;
      - zeros (with their sign), infinities and NaN pass through.
    """
    if dtype not in _FORMATS:
        raise ValueError("dtype must be 'bf16' or 'f32'")
    bits, emin = _FORMATS[dtype]
    v = _f64(a)
    out = v.copy()
    fin = np.isfinite(v) & (v != 0)
    x = v[fin]
    _, e = np.frexp(x)
    q = np.ldexp(1.0, np.maximum(e, emin + 1) - bits)
    r = np.rint(x / q) * q
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, x), r)
    out[fin] = r
    return out


def round_via_f32(a, dtype: str = "bf16"):
    """fp64 -> fp32 -> dtype, each step rounded to nearest even: how a value the GPU holds in an
    fp32 accumulator reaches its output dtype. Differs from ``round_to`` only where the first
    rounding lands exactly on a midpoint of the second format (double rounding)."""
    return round_to(round_to(a, "f32"), dtype)


def num_rows(grid) -> int:
    g = _i32(grid)
    n = _load().pe_oracle_num_rows(_ptr(g, ctypes.c_int32), g.size // 3)
    if n < 0:
        raise ValueError("bad grid %r (code %d)" % (grid, n))
    return int(n)


def row_positions(grid, frames=None, order="raster", m=2, C=3, Tp=2, P=14):
    """For every output row of a frames input, the source patch (item, t, h, w) as int32 [N, 4]."""
    g = _i32(grid)
    n_items = g.size // 3
    fr = _i32(frames) if frames is not None else _i32([1] * n_items)
    out = np.zeros((num_rows(g), 4), dtype=np.int32)
    rc = _load().pe_oracle_row_positions(1, 1 if order == "merge" else 0, m, C, Tp, P, n_items,
                                          _ptr(g, ctypes.c_int32), _ptr(fr, ctypes.c_int32),
                                          _ptr(out, ctypes.c_int32))
    if rc != 0:
        raise ValueError("oracle row_positions failed (code %d)" % rc)
    return out


def forward(x, w, b=None, *, grid, frames=None, kind="frames", order="raster", m=2,
            rows=None, threads=None, cast_input_to=None, addend=None):
    """PatchEmbed in fp64. Returns a numpy array [n_rows, E] (all N rows if ``rows`` is None).

    x       frames kind: all items' frames back to back (any shape, flattened in C order);
            patches kind: [N, C*Tp*P*P]
    w       [E, C, Tp, P, P]
    b       [E] or None
    grid    per item (t, h, w); frames: per item frame count (frames kind)
    cast_input_to  "bf16"/"f32": round the input to this dtype first (input cast to the
            weight dtype); None leaves the values as they are.
    addend  [N, E] or None: added to the result row by row, in output row order (the Qwen3-VL
            vision forward adds the interpolated position embeddings right after the PatchEmbed:
            "Optimize VLM PatchEmbed", the Model forward, hidden_states + pos_embeds).
    """
    wd = _f64(w)
    if wd.ndim != 5:
        raise ValueError("weight must be [E, C, Tp, P, P]")
    E, C, Tp, P, P2 = wd.shape
    if P != P2:
        raise ValueError("square patches only")
    xd = _f64(x) if cast_input_to is None else round_to(x, cast_input_to)
    xd = np.ascontiguousarray(xd.reshape(-1))
    bd = _f64(b).reshape(-1) if b is not None else None
    g = _i32(grid)
    n_items = g.size // 3
    fr = _i32(frames) if frames is not None else None
    if kind == "frames" and fr is None:
        raise ValueError("frames kind needs per-item frame counts")
    rr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64)) if rows is not None else None
    n_out = rr.size if rr is not None else num_rows(g)
    out = np.empty((n_out, E), dtype=np.float64)
    if threads is None:
        threads = max(1, min(os.cpu_count() or 1, 64))
    wflat = np.ascontiguousarray(wd.reshape(-1))
    rc = _load().pe_oracle_forward(
        C, Tp, P, E, 1 if kind == "frames" else 0, 1 if order == "merge" else 0, m, n_items,
        _ptr(g, ctypes.c_int32), _ptr(fr, ctypes.c_int32), _ptr(xd, ctypes.c_double),
        _ptr(wflat, ctypes.c_double), _ptr(bd, ctypes.c_double),
        _ptr(rr, ctypes.c_int64), n_out, _ptr(out, ctypes.c_double), int(threads))
    if rc != 0:
        raise ValueError("oracle forward failed (code %d)" % rc)
    if addend is not None:
        ad = _f64(addend).reshape(-1, E)
        out += ad[rr] if rr is not None else ad
    return out


def layer_norm(x, gamma=None, beta=None, eps=1e-6):
    """LayerNorm over the last dimension, in fp64, from its definition: per row the mean, the
    biased variance (mean of the squared deviations), then (x - mean) / sqrt(var + eps) * gamma
    + beta. It opens the PatchMerger ("freechatgpt/mytransformer", section 3.2's vision encoder
    diagram and section 4.1's PatchMerger bullet: LayerNorm, then the 2x2 concatenation).
    gamma / beta None mean ones / zeros. Returns a numpy array shaped like x."""
    xd = _f64(x)
    mean = xd.sum(axis=-1, keepdims=True) / xd.shape[-1]
    dev = xd - mean
    var = (dev * dev).sum(axis=-1, keepdims=True) / xd.shape[-1]
    with np.errstate(divide="ignore", invalid="ignore"):
        y = dev / np.sqrt(var + eps)
    if gamma is not None:
        y = y * _f64(gamma)
    if beta is not None:
        y = y + _f64(beta)
    return y


def merger_front(rows, gamma=None, beta=None, eps=1e-6, m=2):
    """The PatchMerger's LayerNorm and m x m concatenation: rows [N, E] in merge-window order
    (the m*m patches of each window consecutive) -> [N / m^2, m^2 * E], row j holding the
    normalized patches of window j side by side in their window order (the section 3.2 diagram
    of "freechatgpt/mytransformer": 2x2 neighbours joined into 1280 x 4 = 5120)."""
    y = layer_norm(rows, gamma, beta, eps)
    n, e = y.shape
    if n % (m * m):
        raise ValueError("row count %d is not a multiple of %d" % (n, m * m))
    return y.reshape(n // (m * m), m * m * e)
