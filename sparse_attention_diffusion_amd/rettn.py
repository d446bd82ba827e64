"""ctypes binding of librettn.so (C ABI declared in include/rettn.h).

Argument marshalling only: torch tensors are passed as device pointers and the
current torch stream as the HIP stream.  Every computation runs in the HIP
library; if the library is missing this module raises at import.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# RETTN_LIB names another build of the same C ABI: the CPU tests use it to run
# the host checks against a sanitizer build whose kernel launches all fail.
LIB_PATH = os.environ.get("RETTN_LIB") or os.path.join(_HERE, "_lib", "librettn.so")

RT_OK, RT_E_ARG, RT_E_SHAPE, RT_E_DTYPE, RT_E_STATE, RT_E_WORKSPACE, RT_E_LAUNCH, RT_E_DEVICE = range(8)
RT_BF16, RT_F32 = 0, 1
_DTYPES = {"bf16": RT_BF16, "f32": RT_F32}
BLOCK = 64
SELECT_SCRATCH_BYTES = 16 << 20  # RT_SELECT_SCRATCH_BYTES


class RtShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("B", "H", "N", "d", "d_pad", "block", "keep", "dtype")]


class RtStatsView(ctypes.Structure):
    _fields_ = [("m", ctypes.c_void_p), ("z_full", ctypes.c_void_p), ("z_sparse", ctypes.c_void_p),
                ("R", ctypes.c_void_p), ("idx", ctypes.c_void_p), ("rows", ctypes.c_int64),
                ("valid", ctypes.c_int32), ("r_dtype", ctypes.c_int32)]


class RettnError(RuntimeError):
    def __init__(self, status, detail):
        super().__init__(f"{_lib.rt_status_string(status).decode()}: {detail}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m sparse_attention_diffusion_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, S, I32, SZ = ctypes.c_void_p, ctypes.POINTER(RtShape), ctypes.c_int32, ctypes.c_size_t
    sig = {
        "rt_status_string": (ctypes.c_char_p, [I32]),
        "rt_last_error": (ctypes.c_char_p, []),
        "rt_version": (I32, []),
        "rt_num_blocks": (I32, [S]),
        "rt_select_workspace_bytes": (SZ, [S]),
        "rt_select_blocks": (I32, [S, P, P, ctypes.POINTER(I32), I32, P, P, P, SZ, P]),
        "rt_select_blocks_noalloc": (I32, [S, P, P, ctypes.POINTER(I32), I32, P, P, P]),
        "rt_stats_cache_bytes": (SZ, [S, I32]),
        "rt_stats_cache_init": (I32, [ctypes.POINTER(P), S, I32, P, SZ]),
        "rt_stats_cache_bytes_ex": (SZ, [S, I32, I32]),
        "rt_stats_cache_init_ex": (I32, [ctypes.POINTER(P), S, I32, I32, P, SZ]),
        "rt_stats_cache_view": (I32, [P, I32, ctypes.POINTER(RtStatsView)]),
        "rt_residual_index": (ctypes.c_int64, [S, ctypes.c_int64, I32, I32]),
        "rt_stats_cache_set_valid": (I32, [P, I32, I32]),
        "rt_stats_cache_invalidate": (I32, [P, I32]),
        "rt_stats_cache_destroy": (I32, [P]),
        "rt_calibrate": (I32, [S, P, P, P, P, P, I32, P, P]),
        "rt_sparse_attn_reshape": (I32, [S, P, P, P, P, P, I32, P, P]),
        "rt_sparse_attn_reshape_ex": (I32, [S, P, P, P, P, P, I32, I32, P, P]),
        "rt_schedule_is_calibration": (I32, [I32, I32]),
        "rt_step_workspace_bytes": (SZ, [S]),
        "rt_attention_step": (I32, [S, P, P, P, ctypes.POINTER(I32), I32, P, I32, I32, I32, P, P, SZ, P,
                                    ctypes.POINTER(I32)]),
        "rt_hilbert_order": (I32, [ctypes.POINTER(I32), I32, I32, ctypes.POINTER(I32), I32]),
        "rt_permute_rows": (I32, [S, P, P, P, I32, P]),
        "rt_attention_step_ex": (I32, [S, P, P, P, ctypes.POINTER(I32), I32, P, I32, I32, I32, I32, I32, P, P, SZ,
                                       P, ctypes.POINTER(I32)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()
SYMBOLS = [
    "rt_status_string", "rt_last_error", "rt_version", "rt_num_blocks", "rt_select_workspace_bytes",
    "rt_select_blocks", "rt_stats_cache_bytes", "rt_stats_cache_init", "rt_stats_cache_bytes_ex",
    "rt_stats_cache_init_ex", "rt_stats_cache_view",
    "rt_stats_cache_set_valid", "rt_stats_cache_invalidate", "rt_stats_cache_destroy", "rt_calibrate",
    "rt_sparse_attn_reshape", "rt_sparse_attn_reshape_ex", "rt_schedule_is_calibration", "rt_step_workspace_bytes", "rt_attention_step",
    "rt_attention_step_ex", "rt_hilbert_order", "rt_permute_rows", "rt_select_blocks_noalloc",
    "rt_residual_index",
]


def lib():
    return _lib


def _check(status):
    if status != RT_OK:
        raise RettnError(status, _lib.rt_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is not None:
        return ctypes.c_void_p(stream)
    if torch.cuda.is_available():
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return ctypes.c_void_p(0)


def shape(B, H, N, d, d_pad, keep, dtype="bf16", block=BLOCK):
    return RtShape(B, H, N, d, d_pad, block, keep, RT_BF16 if dtype == "bf16" else RT_F32)


def shape_of(cfg, keep=None):
    return shape(cfg["B"], cfg["H"], cfg["N"], cfg["d"], cfg["d_pad"], cfg["keep"] if keep is None else keep,
                 cfg["dtype"])


def torch_dtype(sh):
    return torch.bfloat16 if sh.dtype == RT_BF16 else torch.float32


def num_blocks(sh):
    return _lib.rt_num_blocks(ctypes.byref(sh))


def select_workspace_bytes(sh):
    return _lib.rt_select_workspace_bytes(ctypes.byref(sh))


def step_workspace_bytes(sh):
    return _lib.rt_step_workspace_bytes(ctypes.byref(sh))


def stats_cache_bytes(sh, n_layers=1):
    return _lib.rt_stats_cache_bytes(ctypes.byref(sh), n_layers)


def stats_cache_bytes_ex(sh, n_layers=1, residual="f32"):
    return _lib.rt_stats_cache_bytes_ex(ctypes.byref(sh), n_layers, _DTYPES[residual])


def schedule_is_calibration(step, period):
    return bool(_lib.rt_schedule_is_calibration(step, period))


def _forced_arr(forced):
    forced = [] if forced is None else [int(j) for j in forced]
    arr = (ctypes.c_int32 * max(1, len(forced)))(*forced)
    return arr, len(forced)


def rt_select_blocks(sh, q, k, forced, block_idx, pooled_scores, workspace, stream=None):
    arr, n = _forced_arr(forced)
    _check(_lib.rt_select_blocks(ctypes.byref(sh), _ptr(q), _ptr(k), arr if n else None, n, _ptr(block_idx),
                                 _ptr(pooled_scores), _ptr(workspace),
                                 0 if workspace is None else workspace.numel() * workspace.element_size(),
                                 _stream(stream)))


def rt_select_blocks_noalloc(sh, q, k, forced, block_idx, pooled_scores, stream=None):
    """rt_select_blocks with the pooled means in the library's own scratch (no workspace)."""
    arr, n = _forced_arr(forced)
    _check(_lib.rt_select_blocks_noalloc(ctypes.byref(sh), _ptr(q), _ptr(k), arr if n else None, n,
                                         _ptr(block_idx), _ptr(pooled_scores), _stream(stream)))


def rt_residual_index(sh, bh, row, col):
    """Element position of the residual of head bh, row, col from the view's R."""
    at = _lib.rt_residual_index(ctypes.byref(sh), int(bh), int(row), int(col))
    if at < 0:
        raise RettnError(RT_E_ARG, _lib.rt_last_error().decode())
    return at


class StatsCache:
    """Host handle plus the device memory (a torch byte tensor) it wraps."""

    def __init__(self, sh, n_layers=1, device="cuda", memory=None, residual="f32"):
        """residual: storage type of R, "f32" (default) or "bf16"."""
        self.shape = sh
        self.n_layers = n_layers
        self.residual = residual
        nbytes = stats_cache_bytes_ex(sh, n_layers, residual)
        if memory is None:
            memory = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
        self.memory = memory
        self.handle = ctypes.c_void_p()
        _check(_lib.rt_stats_cache_init_ex(ctypes.byref(self.handle), ctypes.byref(sh), n_layers,
                                           _DTYPES[residual], _ptr(memory), memory.numel()))

    def view(self, layer=0):
        v = RtStatsView()
        _check(_lib.rt_stats_cache_view(self.handle, layer, ctypes.byref(v)))
        return v

    def tensors(self, layer=0):
        """Zero-copy torch views of one layer: m, z_full, z_sparse [B,H,N]; R flat, B*H*Nb*64*d_pad
        elements in the order of rt_residual_index; idx [B,H,Nb,keep]."""
        v = self.view(layer)
        sh = self.shape
        nb = num_blocks(sh)
        base = self.memory.data_ptr()

        def sub(ptr, count, dtype, shp):
            off = ptr - base
            esz = torch.tensor([], dtype=dtype).element_size()
            return self.memory[off: off + count * esz].view(dtype).view(shp)

        rows = sh.B * sh.H * sh.N
        return dict(
            m=sub(v.m, rows, torch.float32, (sh.B, sh.H, sh.N)),
            z_full=sub(v.z_full, rows, torch.float32, (sh.B, sh.H, sh.N)),
            z_sparse=sub(v.z_sparse, rows, torch.float32, (sh.B, sh.H, sh.N)),
            R=sub(v.R, sh.B * sh.H * nb * 64 * sh.d_pad, torch.bfloat16 if v.r_dtype == 0 else torch.float32,
                  (sh.B * sh.H * nb * 64 * sh.d_pad,)),
            idx=sub(v.idx, sh.B * sh.H * nb * sh.keep, torch.int32, (sh.B, sh.H, nb, sh.keep)),
            valid=v.valid,
        )

    def set_valid(self, layer, valid=True):
        _check(_lib.rt_stats_cache_set_valid(self.handle, layer, int(bool(valid))))

    def invalidate(self, layer=-1):
        _check(_lib.rt_stats_cache_invalidate(self.handle, layer))

    def close(self):
        if self.handle:
            _lib.rt_stats_cache_destroy(self.handle)
            self.handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def rt_calibrate(sh, q, k, v, block_idx, cache, layer, o, stream=None):
    _check(_lib.rt_calibrate(ctypes.byref(sh), _ptr(q), _ptr(k), _ptr(v), _ptr(block_idx), cache.handle, layer,
                             _ptr(o), _stream(stream)))


def rt_sparse_attn_reshape(sh, q, k, v, block_idx, cache, layer, o, stream=None):
    _check(_lib.rt_sparse_attn_reshape(ctypes.byref(sh), _ptr(q), _ptr(k), _ptr(v), _ptr(block_idx),
                                       cache.handle, layer, _ptr(o), _stream(stream)))


RT_RESHAPE_R1, RT_RESHAPE_R2 = 0, 1
RT_STEP_RESELECT = 1
_VARIANTS = {"r1": RT_RESHAPE_R1, "r2": RT_RESHAPE_R2}


def rt_sparse_attn_reshape_ex(sh, q, k, v, block_idx, cache, layer, variant, o, stream=None):
    """`variant`: "r1" / "r2" or the RT_RESHAPE_* value."""
    var = _VARIANTS.get(variant, variant) if isinstance(variant, str) else int(variant)
    if isinstance(var, str):
        raise ValueError(f"unknown reshape variant {variant!r}")
    _check(_lib.rt_sparse_attn_reshape_ex(ctypes.byref(sh), _ptr(q), _ptr(k), _ptr(v), _ptr(block_idx),
                                          cache.handle, layer, var, _ptr(o), _stream(stream)))


def rt_attention_step(sh, q, k, v, forced, cache, layer, step, period, o, workspace, stream=None):
    arr, n = _forced_arr(forced)
    did = ctypes.c_int32(0)
    _check(_lib.rt_attention_step(ctypes.byref(sh), _ptr(q), _ptr(k), _ptr(v), arr if n else None, n,
                                  cache.handle, layer, step, period, _ptr(o), _ptr(workspace),
                                  0 if workspace is None else workspace.numel() * workspace.element_size(),
                                  _stream(stream), ctypes.byref(did)))
    return bool(did.value)


def rt_attention_step_ex(sh, q, k, v, forced, cache, layer, step, period, variant, reselect, o, workspace,
                         stream=None):
    """rt_attention_step with a reshape variant ("r1" / "r2") and per-step reselection."""
    var = _VARIANTS.get(variant, variant) if isinstance(variant, str) else int(variant)
    if isinstance(var, str):
        raise ValueError(f"unknown reshape variant {variant!r}")
    arr, n = _forced_arr(forced)
    did = ctypes.c_int32(0)
    _check(_lib.rt_attention_step_ex(ctypes.byref(sh), _ptr(q), _ptr(k), _ptr(v), arr if n else None, n,
                                     cache.handle, layer, step, period, var, RT_STEP_RESELECT if reselect else 0,
                                     _ptr(o), _ptr(workspace),
                                     0 if workspace is None else workspace.numel() * workspace.element_size(),
                                     _stream(stream), ctypes.byref(did)))
    return bool(did.value)


def rt_hilbert_order(dims, n_text=0):
    """Hilbert-curve token order (host): numpy int32 permutation, text first."""
    import numpy as np
    d = (ctypes.c_int32 * len(dims))(*[int(x) for x in dims])
    n = int(n_text) + int(np.prod([int(x) for x in dims]))
    out = np.empty(n, dtype=np.int32)
    _check(_lib.rt_hilbert_order(d, len(dims), int(n_text), out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), n))
    return out


def rt_permute_rows(sh, src, dst, perm, inverse=False, stream=None):
    """Row reorder on the device: dst[..., i, :] = src[..., perm[i], :] (or the inverse)."""
    _check(_lib.rt_permute_rows(ctypes.byref(sh), _ptr(src), _ptr(dst), _ptr(perm), 1 if inverse else 0,
                                _stream(stream)))
