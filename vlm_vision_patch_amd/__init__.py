"""MI355X (gfx950) vision PatchEmbed: Python binding of libpe.so (include/pe.h).

The binding only marshals arguments; every step of the operation runs in the library's HIP
kernels. PyTorch supplies device memory and the current stream. There is no fallback: if the
library is not built, importing this package raises.

    pe = PatchEmbed(weight, bias, order="merge", out_dtype=torch.bfloat16)
    out = pe(frames, grid_thw=[[1, 16, 64]])              # raw frames
    out = pe(pixel_values, grid_thw=[[1, 16, 64]], kind="patches")
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# PE_LIB_PATH names another build of the same library, e.g. the LDS sentinel debug build
# libpe_sentinel.so (build.py); by default the package's libpe.so
LIB_PATH = os.environ.get("PE_LIB_PATH") or os.path.join(_PKG, "libpe.so")

PE_OK, PE_ERR_INVALID_ARG, PE_ERR_SHAPE, PE_ERR_UNSUPPORTED, PE_ERR_HIP, PE_ERR_OOM = 0, -1, -2, -3, -4, -5
PE_F32, PE_BF16 = 0, 1
PE_ORDER_RASTER, PE_ORDER_MERGE_WINDOW = 0, 1
PE_INPUT_PATCHES, PE_INPUT_FRAMES = 0, 1

# every symbol include/pe.h declares
EXPORTS = ("pe_create", "pe_forward", "pe_forward_add", "pe_forward_plan", "pe_layernorm", "pe_num_rows",
           "pe_destroy", "pe_last_error")
PE_A_MODES = ("frames", "images", "patch_rows", "folded_images", "images_lds")


class PEError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("%s (code %d)" % (msg, code))
        self.code = code


class pe_config(ctypes.Structure):
    _fields_ = [("in_channels", ctypes.c_int32), ("temporal_patch_size", ctypes.c_int32),
                ("patch_size", ctypes.c_int32), ("embed_dim", ctypes.c_int32),
                ("spatial_merge_size", ctypes.c_int32), ("weight_dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("out_order", ctypes.c_int32), ("image_fold", ctypes.c_int32),
                ("stage_images", ctypes.c_int32)]


class pe_launch_info(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_char * 32), ("tile_rows", ctypes.c_int32), ("tile_cols", ctypes.c_int32),
                ("workgroups", ctypes.c_int64), ("row0", ctypes.c_int64), ("n_rows", ctypes.c_int64),
                ("in_offset", ctypes.c_int64), ("in_bytes", ctypes.c_int64), ("n_items", ctypes.c_int32),
                ("a_mode", ctypes.c_int32)]


def _load():
    # Load torch's HIP runtime first: libpe.so then binds to it (same soname) instead of pulling
    # a second HIP/HSA runtime from /opt/rocm into the process.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError("libpe.so is not built (%s); run `python __graft_entry__.py build` or "
                          "`python vlm_vision_patch_amd/build.py`" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    pi32 = ctypes.POINTER(ctypes.c_int32)
    lib.pe_create.restype = ctypes.c_int
    lib.pe_create.argtypes = [ctypes.POINTER(pe_config), vp, vp, vp, ctypes.POINTER(vp)]
    lib.pe_forward.restype = ctypes.c_int
    lib.pe_forward.argtypes = [vp, i32, vp, i32, pi32, pi32, i32, vp, vp]
    lib.pe_forward_add.restype = ctypes.c_int
    lib.pe_forward_add.argtypes = [vp, i32, vp, i32, pi32, pi32, i32, vp, vp, vp]
    lib.pe_forward_plan.restype = ctypes.c_int
    lib.pe_forward_plan.argtypes = [vp, i32, i32, pi32, pi32, i32, ctypes.POINTER(pe_launch_info), i32]
    lib.pe_layernorm.restype = ctypes.c_int
    lib.pe_layernorm.argtypes = [vp, i32, vp, vp, i32, ctypes.c_float, i64, i32, vp, vp]
    lib.pe_num_rows.restype = i64
    lib.pe_num_rows.argtypes = [pi32, i32]
    lib.pe_destroy.restype = ctypes.c_int
    lib.pe_destroy.argtypes = [vp]
    lib.pe_last_error.restype = ctypes.c_char_p
    lib.pe_last_error.argtypes = []
    return lib


lib = _load()


def last_error() -> str:
    return lib.pe_last_error().decode("utf-8", "replace")


def _check(rc):
    if rc != PE_OK:
        raise PEError(rc, last_error())
    return rc


def _i32_array(values):
    flat = [int(v) for row in values for v in (row if hasattr(row, "__len__") else [row])]
    return (ctypes.c_int32 * max(1, len(flat)))(*flat), len(flat)


# ---- raw C-ABI calls with the header's names (plain integers / addresses) -------------------

def pe_create(cfg: pe_config, weight_ptr: int, bias_ptr: int | None, stream: int | None) -> int:
    h = ctypes.c_void_p()
    _check(lib.pe_create(ctypes.byref(cfg), weight_ptr, bias_ptr, stream, ctypes.byref(h)))
    return h.value


def pe_forward(handle: int, input_kind: int, input_ptr: int, in_dtype: int, grid_thw, frames,
               out_ptr: int, stream: int | None) -> None:
    g, n = _i32_array(grid_thw)
    f = _i32_array(frames)[0] if frames is not None else None
    _check(lib.pe_forward(handle, input_kind, input_ptr, in_dtype, g, f, n // 3, out_ptr, stream))


def pe_forward_add(handle: int, input_kind: int, input_ptr: int, in_dtype: int, grid_thw, frames,
                   addend_ptr: int, out_ptr: int, stream: int | None) -> None:
    g, n = _i32_array(grid_thw)
    f = _i32_array(frames)[0] if frames is not None else None
    _check(lib.pe_forward_add(handle, input_kind, input_ptr, in_dtype, g, f, n // 3, addend_ptr, out_ptr, stream))


def pe_forward_plan(handle: int, input_kind: int, in_dtype: int, grid_thw, frames) -> list:
    """The launches pe_forward would make for this request, as dicts (kernel name, tile, grid,
    rows, input range, items, A mode)."""
    g, n = _i32_array(grid_thw)
    f = _i32_array(frames)[0] if frames is not None else None
    count = lib.pe_forward_plan(handle, input_kind, in_dtype, g, f, n // 3, None, 0)
    if count < 0:
        raise PEError(count, last_error())
    info = (pe_launch_info * max(1, count))()
    _check(min(0, lib.pe_forward_plan(handle, input_kind, in_dtype, g, f, n // 3, info, count)))
    return [{"kernel": i.kernel.decode(), "tile": [i.tile_rows, i.tile_cols], "workgroups": i.workgroups,
             "row0": i.row0, "n_rows": i.n_rows, "in_offset": i.in_offset, "in_bytes": i.in_bytes,
             "n_items": i.n_items, "a_mode": PE_A_MODES[i.a_mode]} for i in info[:count]]


def pe_layernorm(x_ptr: int, dtype: int, gamma_ptr: int | None, beta_ptr: int | None, param_dtype: int,
                 eps: float, n_rows: int, dim: int, y_ptr: int, stream: int | None) -> None:
    _check(lib.pe_layernorm(x_ptr, dtype, gamma_ptr, beta_ptr, param_dtype, eps, n_rows, dim, y_ptr, stream))


def pe_num_rows(grid_thw) -> int:
    g, n = _i32_array(grid_thw)
    rc = lib.pe_num_rows(g, n // 3)
    if rc < 0:
        raise PEError(int(rc), last_error())
    return int(rc)


def pe_destroy(handle: int) -> None:
    _check(lib.pe_destroy(handle))


# ---- torch-facing wrapper ------------------------------------------------------------------

def _dtype_code(dt):
    import torch
    if dt == torch.bfloat16:
        return PE_BF16
    if dt == torch.float32:
        return PE_F32
    raise PEError(PE_ERR_UNSUPPORTED, "dtype %s: only bfloat16 and float32" % dt)


def _keep_for_stream(tensors, stream, device):
    """Tensors this binding allocated (an output, a contiguous copy of the input) are freed by
    torch's caching allocator on the stream current at allocation. When the kernel runs on another
    stream, mark them as used there, so their memory is not handed out again before that stream's
    work is done."""
    import torch
    if stream is None or stream == torch.cuda.current_stream(device).cuda_stream:
        return
    ext = torch.cuda.ExternalStream(stream, device=device)
    for t in tensors:
        if t is not None:
            t.record_stream(ext)


class PatchEmbed:
    """Conv3d(3, E, (2, P, P), stride (2, P, P)) PatchEmbed on the current CUDA/HIP device.

    weight  [E, 3, 2, P, P] bf16 or fp32 CUDA tensor (packed once at construction)
    bias    [E] same dtype, or None
    order   "merge" (2x2 merge-window rows) or "raster" (Conv3d view order) for frames input
    image_fold  approximate mode for single-frame items: W[:, :, 0] + W[:, :, 1] folded into one
            bf16 weight, half the matrix work (see pe.h); off by default
    stage_images  gather single images through LDS (exact; slower on MI355X, see pe.h); off by
            default
    """

    def __init__(self, weight, bias=None, *, order: str = "raster", out_dtype=None,
                 spatial_merge_size: int = 2, image_fold: bool = False, stage_images: bool = False):
        import torch
        if weight.dim() != 5 or weight.shape[3] != weight.shape[4]:
            raise PEError(PE_ERR_INVALID_ARG, "weight must be [E, C, Tp, P, P]")
        if not weight.is_cuda:
            raise PEError(PE_ERR_INVALID_ARG, "weight must be a device tensor")
        E, C, Tp, P, _ = weight.shape
        self.device = weight.device
        self.weight_dtype = weight.dtype
        self.out_dtype = out_dtype if out_dtype is not None else weight.dtype
        self.embed_dim, self.patch_size = int(E), int(P)
        self.k = int(C * Tp * P * P)
        self.order = order
        cfg = pe_config(int(C), int(Tp), int(P), int(E), int(spatial_merge_size),
                        _dtype_code(weight.dtype), _dtype_code(self.out_dtype),
                        PE_ORDER_MERGE_WINDOW if order == "merge" else PE_ORDER_RASTER, 1 if image_fold else 0,
                        1 if stage_images else 0)
        w = weight.contiguous()
        b = bias.contiguous() if bias is not None else None
        if b is not None and (b.dtype != weight.dtype or b.numel() != E):
            raise PEError(PE_ERR_INVALID_ARG, "bias must be [E] in the weight dtype")
        with torch.cuda.device(self.device):
            stream = torch.cuda.current_stream(self.device).cuda_stream
            self._h = pe_create(cfg, w.data_ptr(), b.data_ptr() if b is not None else None, stream)
        self._plans = {}

    _PLANS_MAX = 64

    def _plan(self, grid_thw, frames, kind):
        """(N, input elements, grid array, item count, frames array) of a request. The marshalled
        arguments are kept per (kind, grid, frames) value, so a repeated request reuses them (the
        library only reads the host arrays during the call)."""
        g = grid_thw.tolist() if hasattr(grid_thw, "tolist") else grid_thw
        f = frames.tolist() if (frames is not None and hasattr(frames, "tolist")) else frames
        key = (kind, tuple(tuple(row) for row in g), None if f is None else tuple(f))
        p = self._plans.get(key)
        if p is None:
            grid = [[int(v) for v in row] for row in g]
            fr = None if f is None else [int(v) for v in f]
            n = pe_num_rows(grid) if grid else 0
            need = self.input_elements(grid, fr, kind) if n else 0
            ga, ng = _i32_array(grid)
            fa = _i32_array(fr)[0] if fr is not None else None
            p = (n, need, ga, ng // 3, fa)
            if len(self._plans) >= self._PLANS_MAX:
                self._plans.clear()
            self._plans[key] = p
        return p

    def __call__(self, x, grid_thw, frames=None, *, kind: str = "frames", out=None, stream=None, add=None):
        """out = PatchEmbed(x) (+ add: an [N, E] tensor in the output dtype and row order, fused
        into the epilogue, e.g. the position embeddings that follow the PatchEmbed)."""
        import torch
        n, need, ga, n_items, fa = self._plan(grid_thw, frames, kind)
        made = []   # tensors allocated here (see _keep_for_stream)
        if out is None:
            out = torch.empty((n, self.embed_dim), dtype=self.out_dtype, device=self.device)
            made.append(out)
        elif tuple(out.shape) != (n, self.embed_dim) or out.dtype != self.out_dtype or not out.is_contiguous():
            raise PEError(PE_ERR_INVALID_ARG, "out must be a contiguous [%d, %d] %s tensor"
                          % (n, self.embed_dim, self.out_dtype))
        if n == 0:
            return out
        if not x.is_cuda or x.device != self.device:
            raise PEError(PE_ERR_INVALID_ARG, "input must be on %s" % self.device)
        if x.numel() != need:
            raise PEError(PE_ERR_SHAPE, "input has %d elements; the grid needs %d" % (x.numel(), need))
        xc = x.contiguous()
        if xc.data_ptr() != x.data_ptr():
            made.append(xc)
        x = xc
        if stream is None:
            stream = torch.cuda.current_stream(self.device).cuda_stream
        else:
            _keep_for_stream(made, stream, self.device)
        ik = PE_INPUT_PATCHES if kind == "patches" else PE_INPUT_FRAMES
        if add is None:
            _check(lib.pe_forward(self._h, ik, x.data_ptr(), _dtype_code(x.dtype), ga, fa, n_items,
                                  out.data_ptr(), stream))
        else:
            if (tuple(add.shape) != (n, self.embed_dim) or add.dtype != self.out_dtype or not add.is_contiguous()
                    or add.device != self.device):
                raise PEError(PE_ERR_INVALID_ARG, "add must be a contiguous [%d, %d] %s tensor on %s"
                              % (n, self.embed_dim, self.out_dtype, self.device))
            _check(lib.pe_forward_add(self._h, ik, x.data_ptr(), _dtype_code(x.dtype), ga, fa, n_items,
                                      add.data_ptr(), out.data_ptr(), stream))
        return out

    def plan(self, grid_thw, frames=None, *, kind: str = "frames", in_dtype=None) -> list:
        """The kernel launches a call with this grid makes (pe_forward_plan): kernel name, tile,
        workgroups, rows and input range per launch. Nothing is launched."""
        ik = PE_INPUT_PATCHES if kind == "patches" else PE_INPUT_FRAMES
        g = grid_thw.tolist() if hasattr(grid_thw, "tolist") else grid_thw
        if len(g) == 0:
            return []   # an empty batch launches nothing (the C ABI calls 0 items an error)
        return pe_forward_plan(self._h, ik, _dtype_code(in_dtype if in_dtype is not None else self.weight_dtype),
                               g, frames)

    def input_elements(self, grid, frames=None, kind="frames") -> int:
        """Elements the library will read for this grid (the C ABI trusts the caller on this)."""
        if kind == "patches":
            return pe_num_rows(grid) * self.k
        P, total = self.patch_size, 0
        for i, (t, h, w) in enumerate(grid):
            f = frames[i] if frames is not None else (1 if t == 1 else 2 * t)
            total += f * 3 * (h * P) * (w * P)
        return total

    def close(self):
        if getattr(self, "_h", None):
            pe_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def layer_norm(x, gamma=None, beta=None, eps: float = 1e-6, *, out=None, stream=None):
    """LayerNorm over the last dimension of a contiguous [..., dim] bf16 / fp32 device tensor
    (pe_layernorm): the front of the PatchMerger. ``out`` may be ``x`` (in place). On PatchEmbed
    rows in merge-window order (m = 2), ``layer_norm(rows).view(-1, 4 * dim)`` is the merger's
    2x2 concatenation of normalized rows."""
    import torch
    if not x.is_cuda or not x.is_contiguous() or x.dim() < 1:
        raise PEError(PE_ERR_INVALID_ARG, "x must be a contiguous device tensor")
    dim = int(x.shape[-1])
    n_rows = x.numel() // dim if dim else 0
    pdt = None
    for p in (gamma, beta):
        if p is not None:
            if (tuple(p.shape) != (dim,) or not p.is_contiguous() or p.device != x.device
                    or (pdt is not None and p.dtype != pdt)):
                raise PEError(PE_ERR_INVALID_ARG, "gamma / beta must be contiguous [%d] tensors of one dtype "
                              "on %s" % (dim, x.device))
            pdt = p.dtype
    made = []
    if out is None:
        out = torch.empty_like(x)
        made.append(out)
    elif out.shape != x.shape or out.dtype != x.dtype or not out.is_contiguous() or out.device != x.device:
        raise PEError(PE_ERR_INVALID_ARG, "out must be a contiguous tensor like x")
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    else:
        _keep_for_stream(made, stream, x.device)
    with torch.cuda.device(x.device):
        pe_layernorm(x.data_ptr(), _dtype_code(x.dtype), gamma.data_ptr() if gamma is not None else None,
                     beta.data_ptr() if beta is not None else None,
                     _dtype_code(pdt) if pdt is not None else _dtype_code(x.dtype), float(eps), n_rows, dim,
                     out.data_ptr(), stream)
    return out
