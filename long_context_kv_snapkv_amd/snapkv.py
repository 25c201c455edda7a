"""ctypes binding of libsnapkv: the C-ABI entry points under the same names.

Argument marshalling only: shapes are read from the tensors, raw device
pointers and the current HIP stream are handed to the library, and outputs /
workspace are allocated with torch when the caller does not pass them. Every
step of the computation runs in the library's gfx950 kernels. If the library
has not been built the first call raises SnapKVLibraryMissing; there is no
fallback.
"""

from __future__ import annotations

import ctypes
import os
import re
from typing import Iterable, Optional, Sequence, Tuple

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "_lib", "libsnapkv.so")
HEADER_PATH = os.path.join(os.path.dirname(HERE), "include", "snapkv.h")

SNAPKV_OK = 0
SNAPKV_ERR_INVALID_ARGUMENT = 1
SNAPKV_ERR_UNSUPPORTED = 2
SNAPKV_ERR_WORKSPACE = 3
SNAPKV_ERR_HIP = 4
SNAPKV_POOL_AVG = 0
SNAPKV_POOL_MAX = 1
SNAPKV_NUM_STAGES = 4
SNAPKV_CACHE_COMPRESSED = 0
SNAPKV_CACHE_PACKED = 1

_POOL_NAMES = {"avg": SNAPKV_POOL_AVG, "avgpool": SNAPKV_POOL_AVG,
               "max": SNAPKV_POOL_MAX, "maxpool": SNAPKV_POOL_MAX}

_lib = None

_i32 = ctypes.c_int32
_vp = ctypes.c_void_p
_sz = ctypes.c_size_t
_pi32 = ctypes.POINTER(ctypes.c_int32)


class SnapKVLibraryMissing(ImportError):
    """libsnapkv.so has not been built."""


class SnapKVError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        lib = load_library()
        name = lib.snapkv_status_string(status).decode()
        super().__init__(f"snapkv: {name} ({status}): {detail}")


def load_library():
    """Load libsnapkv.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise SnapKVLibraryMissing(
            f"{LIB_PATH} is missing; build it with "
            "`python -m long_context_kv_snapkv_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    lib.snapkv_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _pi32, _i32,
                                          ctypes.POINTER(_sz)]
    lib.snapkv_workspace_size.restype = _i32
    compress_args = [_i32, _i32, _i32, _i32, _vp, _vp, _vp, _pi32, _i32, _i32, _i32,
                     _i32, _vp, _vp, _vp, _vp, _sz, _vp]
    lib.snapkv_compress.argtypes = compress_args
    lib.snapkv_compress.restype = _i32
    lib.snapkv_compress_staged.argtypes = compress_args + [ctypes.POINTER(_vp)]
    lib.snapkv_compress_staged.restype = _i32
    lib.snapkv_compress_from_lse.argtypes = [_i32, _i32, _i32, _i32, _vp, _vp, _vp, _pi32, _i32,
                                             _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp]
    lib.snapkv_compress_from_lse.restype = _i32
    lib.snapkv_compress_with_scores.argtypes = [_i32, _i32, _i32, _i32, _vp, _vp, _vp, _pi32,
                                                _i32, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp,
                                                _i32, _vp, _sz, _vp]
    lib.snapkv_compress_with_scores.restype = _i32
    lib.snapkv_compress_static.argtypes = [_i32, _i32, _i32, _i32, _vp, _vp, _vp, _pi32, _i32,
                                           _i32, _i32, _i32, _vp, _vp, _vp, _vp]
    lib.snapkv_compress_static.restype = _i32
    lib.snapkv_prefill_attention.argtypes = [_i32, _i32, _i32, _i32, _vp, _vp, _vp, _pi32, _i32,
                                             _vp, _vp, _vp, _vp]
    lib.snapkv_prefill_attention.restype = _i32
    lib.snapkv_compress_int4.argtypes = [_i32, _i32, _i32, _i32, _vp, _vp, _vp, _pi32, _i32, _vp,
                                         _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                                         _vp]
    lib.snapkv_compress_int4.restype = _i32
    lib.snapkv_compress_fp8.argtypes = lib.snapkv_compress_int4.argtypes
    lib.snapkv_compress_fp8.restype = _i32
    lib.snapkv_decode_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, _pi32,
                                                 ctypes.POINTER(_sz)]
    lib.snapkv_decode_workspace_size.restype = _i32
    lib.snapkv_decode_attention.argtypes = [_i32, _i32, _i32, _i32, _vp, _vp, _vp, _i32, _i32,
                                            _pi32, _vp, _vp, _sz, _vp]
    lib.snapkv_decode_attention.restype = _i32
    lib.snapkv_decode_attention_timed.argtypes = lib.snapkv_decode_attention.argtypes + [_vp,
                                                                                           _vp]
    lib.snapkv_decode_attention_timed.restype = _i32
    lib.snapkv_decode_kernels.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, _pi32, _pi32]
    lib.snapkv_decode_kernels.restype = _i32
    lib.snapkv_window_scores.argtypes = [_i32, _i32, _i32, _i32, _vp, _vp, _pi32, _i32,
                                         _i32, _i32, _vp, _i32, _vp, _sz, _vp]
    lib.snapkv_window_scores.restype = _i32
    lib.snapkv_status_string.argtypes = [_i32]
    lib.snapkv_status_string.restype = ctypes.c_char_p
    lib.snapkv_last_error.argtypes = []
    lib.snapkv_last_error.restype = ctypes.c_char_p
    lib.snapkv_score_kernels.argtypes = [_i32, _i32, _i32, _i32, _pi32, _i32, _i32, _pi32]
    lib.snapkv_score_kernels.restype = _i32
    lib.snapkv_gather_selects.argtypes = [_i32, _i32, _i32, _i32, _pi32, _i32, _i32, _pi32]
    lib.snapkv_gather_selects.restype = _i32
    lib.snapkv_select_kernels.argtypes = [_i32, _i32, _i32, _i32, _pi32, _i32, _i32, _pi32]
    lib.snapkv_select_kernels.restype = _i32
    lib.snapkv_stage_name.argtypes = [_i32]
    lib.snapkv_stage_name.restype = ctypes.c_char_p
    _lib = lib
    return lib


def header_functions() -> list:
    """Names of the functions include/snapkv.h declares."""
    with open(HEADER_PATH) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*|int32_t)\s*(snapkv_\w+)\s*\(",
                                 text, flags=re.M)))


def pool_mode_code(pooling) -> int:
    if isinstance(pooling, str):
        if pooling not in _POOL_NAMES:
            raise ValueError(f"unknown pooling {pooling!r}")
        return _POOL_NAMES[pooling]
    return int(pooling)


def _check(status: int) -> None:
    if status != SNAPKV_OK:
        raise SnapKVError(status, load_library().snapkv_last_error().decode())


def _lens(seq_lens) -> Tuple[ctypes.Array, list]:
    if isinstance(seq_lens, torch.Tensor):
        seq_lens = seq_lens.detach().cpu().tolist()
    vals = [int(x) for x in seq_lens]
    return (ctypes.c_int32 * max(1, len(vals)))(*vals), vals


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream, device) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check_tensor(name: str, t: torch.Tensor, ndim: int, dtype=torch.bfloat16) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype or t.dim() != ndim or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name} must be a contiguous {ndim}-d {dtype} CUDA/HIP tensor, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")


def new_workspace(num_q_heads: int, num_kv_heads: int, head_dim: int,
                  seq_lens: Iterable[int], window: int, device="cuda") -> torch.Tensor:
    """A zero-filled workspace for this shape (reusable across calls that do
    not overlap in time)."""
    return torch.zeros(snapkv_workspace_size(num_q_heads, num_kv_heads, head_dim, seq_lens,
                                             window), dtype=torch.uint8, device=device)


def snapkv_workspace_size(num_q_heads: int, num_kv_heads: int, head_dim: int,
                          seq_lens: Iterable[int], window: int) -> int:
    lib = load_library()
    arr, vals = _lens(seq_lens)
    out = _sz(0)
    _check(lib.snapkv_workspace_size(len(vals), num_q_heads, num_kv_heads, head_dim, arr,
                                     window, ctypes.byref(out)))
    return out.value


def _shapes(q_win, k, seq_vals):
    batch, hq, w, d = q_win.shape
    total, hkv, dk = k.shape
    if dk != d:
        raise ValueError("q_win and k disagree on head_dim")
    if batch != len(seq_vals) or total != sum(seq_vals):
        raise ValueError("q_win batch / k rows must match seq_lens")
    return batch, hq, hkv, d, w


def _outputs(batch, hkv, budget, d, dev, out_k, out_v, out_idx):
    """The caller's output tensors (checked), or new ones."""
    if out_k is None:
        out_k = torch.empty((batch, hkv, budget, d), dtype=torch.bfloat16, device=dev)
    if out_v is None:
        out_v = torch.empty((batch, hkv, budget, d), dtype=torch.bfloat16, device=dev)
    if out_idx is None:
        out_idx = torch.empty((batch, hkv, budget), dtype=torch.int32, device=dev)
    _check_tensor("out_k", out_k, 4)
    _check_tensor("out_v", out_v, 4)
    _check_tensor("out_idx", out_idx, 3, torch.int32)
    if tuple(out_k.shape) != (batch, hkv, budget, d) or out_v.shape != out_k.shape \
            or tuple(out_idx.shape) != (batch, hkv, budget):
        raise ValueError("output shapes must be [batch, H_kv, budget, D] and [batch, H_kv, budget]")
    return out_k, out_v, out_idx


def snapkv_compress(q_win: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                    seq_lens: Sequence[int], window: int, kernel_size: int, pool_mode,
                    budget: int, *, out_k: Optional[torch.Tensor] = None,
                    out_v: Optional[torch.Tensor] = None,
                    out_idx: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, stream=None,
                    staged: bool = False, stage_events: Optional[Sequence] = None):
    """Compress one layer. Returns (out_k, out_v, out_idx); see include/snapkv.h.

    staged=True (or stage_events given) runs snapkv_compress_staged, the same
    kernels with caller events around each stage; otherwise snapkv_compress.
    A workspace needs no initialisation."""
    lib = load_library()
    _check_tensor("q_win", q_win, 4)
    _check_tensor("k", k, 3)
    _check_tensor("v", v, 3)
    arr, vals = _lens(seq_lens)
    batch, hq, hkv, d, w = _shapes(q_win, k, vals)
    if v.shape != k.shape:
        raise ValueError("k and v shapes differ")
    if w != window:
        raise ValueError(f"q_win holds {w} window rows but window={window}")
    dev = q_win.device
    out_k, out_v, out_idx = _outputs(batch, hkv, budget, d, dev, out_k, out_v, out_idx)
    if workspace is None:
        workspace = new_workspace(hq, hkv, d, vals, window, dev)
    args = (batch, hq, hkv, d, _ptr(q_win), _ptr(k), _ptr(v), arr, window, kernel_size,
            pool_mode_code(pool_mode), budget, _ptr(out_k), _ptr(out_v), _ptr(out_idx),
            _ptr(workspace), workspace.numel(), _stream(stream, dev))
    if stage_events is not None:
        if len(stage_events) != 2 * SNAPKV_NUM_STAGES:
            raise ValueError(f"stage_events needs {2 * SNAPKV_NUM_STAGES} events")
        evs = (_vp * len(stage_events))(*[int(e.cuda_event) for e in stage_events])
        _check(lib.snapkv_compress_staged(*args, evs))
    elif staged:
        _check(lib.snapkv_compress_staged(*args, None))
    else:
        _check(lib.snapkv_compress(*args))
    return out_k, out_v, out_idx


def snapkv_compress_from_lse(q_win: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                             seq_lens: Sequence[int], window: int, window_lse: torch.Tensor,
                             kernel_size: int, pool_mode, budget: int, *,
                             out_k: Optional[torch.Tensor] = None,
                             out_v: Optional[torch.Tensor] = None,
                             out_idx: Optional[torch.Tensor] = None,
                             workspace: Optional[torch.Tensor] = None, stream=None):
    """snapkv_compress with the window rows' natural-log normalisers supplied
    (float32 [batch, H_q, W]); see include/snapkv.h."""
    lib = load_library()
    _check_tensor("q_win", q_win, 4)
    _check_tensor("k", k, 3)
    _check_tensor("v", v, 3)
    _check_tensor("window_lse", window_lse, 3, torch.float32)
    arr, vals = _lens(seq_lens)
    batch, hq, hkv, d, w = _shapes(q_win, k, vals)
    if v.shape != k.shape:
        raise ValueError("k and v shapes differ")
    if w != window:
        raise ValueError(f"q_win holds {w} window rows but window={window}")
    if tuple(window_lse.shape) != (batch, hq, window):
        raise ValueError("window_lse must be [batch, H_q, W]")
    dev = q_win.device
    out_k, out_v, out_idx = _outputs(batch, hkv, budget, d, dev, out_k, out_v, out_idx)
    if workspace is None:
        workspace = new_workspace(hq, hkv, d, vals, window, dev)
    _check(lib.snapkv_compress_from_lse(
        batch, hq, hkv, d, _ptr(q_win), _ptr(k), _ptr(v), arr, window, _ptr(window_lse),
        kernel_size, pool_mode_code(pool_mode), budget, _ptr(out_k), _ptr(out_v), _ptr(out_idx),
        _ptr(workspace), workspace.numel(), _stream(stream, dev)))
    return out_k, out_v, out_idx


SNAPKV_STATIC_SCRATCH_BYTES = 32 << 20


def snapkv_compress_static(q_win: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                           seq_lens: Sequence[int], window: int, kernel_size: int, pool_mode,
                           budget: int, *, out_k: Optional[torch.Tensor] = None,
                           out_v: Optional[torch.Tensor] = None,
                           out_idx: Optional[torch.Tensor] = None, stream=None):
    """snapkv_compress without a workspace: the library's fixed scratch area
    serves as one (the C call allocates nothing; outputs not passed in are
    allocated here by torch). Calls that overlap on one device race; see
    include/snapkv.h."""
    lib = load_library()
    _check_tensor("q_win", q_win, 4)
    _check_tensor("k", k, 3)
    _check_tensor("v", v, 3)
    arr, vals = _lens(seq_lens)
    batch, hq, hkv, d, w = _shapes(q_win, k, vals)
    if v.shape != k.shape:
        raise ValueError("k and v shapes differ")
    if w != window:
        raise ValueError(f"q_win holds {w} window rows but window={window}")
    dev = q_win.device
    out_k, out_v, out_idx = _outputs(batch, hkv, budget, d, dev, out_k, out_v, out_idx)
    _check(lib.snapkv_compress_static(batch, hq, hkv, d, _ptr(q_win), _ptr(k), _ptr(v), arr,
                                      window, kernel_size, pool_mode_code(pool_mode), budget,
                                      _ptr(out_k), _ptr(out_v), _ptr(out_idx),
                                      _stream(stream, dev)))
    return out_k, out_v, out_idx


def snapkv_prefill_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                             seq_lens: Sequence[int], window: int = 0, *,
                             out: Optional[torch.Tensor] = None,
                             window_lse: Optional[torch.Tensor] = None,
                             q_win: Optional[torch.Tensor] = None, stream=None):
    """Causal prefill attention of packed prompts q [T, H_q, D] over k, v
    [T, H_kv, D]. Returns (out, window_lse, q_win): out bf16 [T, H_q, D];
    with window > 0 also the last `window` rows' natural-log normalisers
    float32 [batch, H_q, W] and their queries bf16 [batch, H_q, W, D] (the
    inputs of snapkv_compress_from_lse), else None for both; see
    include/snapkv.h."""
    lib = load_library()
    _check_tensor("q", q, 3)
    _check_tensor("k", k, 3)
    _check_tensor("v", v, 3)
    arr, vals = _lens(seq_lens)
    total, hq, d = q.shape
    if k.shape != v.shape or k.shape[0] != total or k.shape[2] != d:
        raise ValueError("q, k and v must be [T, H_q, D] and [T, H_kv, D]")
    if total != sum(vals):
        raise ValueError("q rows must equal sum(seq_lens)")
    hkv = k.shape[1]
    batch = len(vals)
    dev = q.device
    if out is None:
        out = torch.empty((total, hq, d), dtype=torch.bfloat16, device=dev)
    _check_tensor("out", out, 3)
    if tuple(out.shape) != (total, hq, d):
        raise ValueError("out must be [T, H_q, D]")
    if window > 0:
        if window_lse is None:
            window_lse = torch.empty((batch, hq, window), dtype=torch.float32, device=dev)
        if q_win is None:
            q_win = torch.empty((batch, hq, window, d), dtype=torch.bfloat16, device=dev)
        _check_tensor("window_lse", window_lse, 3, torch.float32)
        _check_tensor("q_win", q_win, 4)
        if tuple(window_lse.shape) != (batch, hq, window) or \
                tuple(q_win.shape) != (batch, hq, window, d):
            raise ValueError("window_lse / q_win must be [batch, H_q, W] / [batch, H_q, W, D]")
    else:
        window_lse = q_win = None
    _check(lib.snapkv_prefill_attention(batch, hq, hkv, d, _ptr(q), _ptr(k), _ptr(v), arr,
                                        window, _ptr(out), _ptr(window_lse), _ptr(q_win),
                                        _stream(stream, dev)))
    return out, window_lse, q_win


def snapkv_compress_with_scores(q_win: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                seq_lens: Sequence[int], window: int, kernel_size: int,
                                pool_mode, budget: int, *,
                                window_lse: Optional[torch.Tensor] = None,
                                out_k: Optional[torch.Tensor] = None,
                                out_v: Optional[torch.Tensor] = None,
                                out_idx: Optional[torch.Tensor] = None,
                                out_scores: Optional[torch.Tensor] = None,
                                workspace: Optional[torch.Tensor] = None, stream=None):
    """snapkv_compress (or, with window_lse, snapkv_compress_from_lse) that
    also returns the pooled scores its selection read: (out_k, out_v,
    out_idx, scores), scores float32 [batch, H_kv, scores_len] with zeros for
    prompts kept whole; see include/snapkv.h."""
    lib = load_library()
    _check_tensor("q_win", q_win, 4)
    _check_tensor("k", k, 3)
    _check_tensor("v", v, 3)
    arr, vals = _lens(seq_lens)
    batch, hq, hkv, d, w = _shapes(q_win, k, vals)
    if v.shape != k.shape:
        raise ValueError("k and v shapes differ")
    if w != window:
        raise ValueError(f"q_win holds {w} window rows but window={window}")
    if window_lse is not None:
        _check_tensor("window_lse", window_lse, 3, torch.float32)
        if tuple(window_lse.shape) != (batch, hq, window):
            raise ValueError("window_lse must be [batch, H_q, W]")
    dev = q_win.device
    out_k, out_v, out_idx = _outputs(batch, hkv, budget, d, dev, out_k, out_v, out_idx)
    if out_scores is None:
        out_scores = torch.empty((batch, hkv, max(1, max(vals) - window)), dtype=torch.float32,
                                 device=dev)
    _check_tensor("out_scores", out_scores, 3, torch.float32)
    if tuple(out_scores.shape[:2]) != (batch, hkv):
        raise ValueError("out_scores must be [batch, H_kv, scores_len]")
    if workspace is None:
        workspace = new_workspace(hq, hkv, d, vals, window, dev)
    _check(lib.snapkv_compress_with_scores(
        batch, hq, hkv, d, _ptr(q_win), _ptr(k), _ptr(v), arr, window,
        _ptr(window_lse) if window_lse is not None else None, kernel_size,
        pool_mode_code(pool_mode), budget, _ptr(out_k), _ptr(out_v), _ptr(out_idx),
        _ptr(out_scores), out_scores.shape[2], _ptr(workspace), workspace.numel(),
        _stream(stream, dev)))
    return out_k, out_v, out_idx, out_scores


def snapkv_compress_int4(q_win: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                         seq_lens: Sequence[int], window: int, kernel_size: int, pool_mode,
                         budget: int, *, window_lse: Optional[torch.Tensor] = None,
                         out: Optional[Sequence[torch.Tensor]] = None,
                         workspace: Optional[torch.Tensor] = None, stream=None):
    """Compression with the kept rows stored at 4 bits per value. Returns
    (kq, ks, vq, vs, idx): uint8 codes [batch, H_kv, B, D/2], float32 scales
    [batch, H_kv, B] for K and V, and int32 indices; see include/snapkv.h.
    window_lse (float32 [batch, H_q, W]) optionally replaces the statistics
    pass as in snapkv_compress_from_lse."""
    return _compress_quant("snapkv_compress_int4", 2, q_win, k, v, seq_lens, window,
                           kernel_size, pool_mode, budget, window_lse, out, workspace, stream)


def snapkv_compress_fp8(q_win: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                        seq_lens: Sequence[int], window: int, kernel_size: int, pool_mode,
                        budget: int, *, window_lse: Optional[torch.Tensor] = None,
                        out: Optional[Sequence[torch.Tensor]] = None,
                        workspace: Optional[torch.Tensor] = None, stream=None):
    """Compression with the kept rows stored as FP8 E4M3 bytes. Returns (kq,
    ks, vq, vs, idx) with codes [batch, H_kv, B, D] (uint8); see
    include/snapkv.h."""
    return _compress_quant("snapkv_compress_fp8", 1, q_win, k, v, seq_lens, window,
                           kernel_size, pool_mode, budget, window_lse, out, workspace, stream)


def _compress_quant(fn, per_byte, q_win, k, v, seq_lens, window, kernel_size, pool_mode, budget,
                    window_lse, out, workspace, stream):
    lib = load_library()
    _check_tensor("q_win", q_win, 4)
    _check_tensor("k", k, 3)
    _check_tensor("v", v, 3)
    arr, vals = _lens(seq_lens)
    batch, hq, hkv, d, w = _shapes(q_win, k, vals)
    if v.shape != k.shape:
        raise ValueError("k and v shapes differ")
    if w != window:
        raise ValueError(f"q_win holds {w} window rows but window={window}")
    if window_lse is not None:
        _check_tensor("window_lse", window_lse, 3, torch.float32)
        if tuple(window_lse.shape) != (batch, hq, window):
            raise ValueError("window_lse must be [batch, H_q, W]")
    dev = q_win.device
    if out is None:
        kq = torch.empty((batch, hkv, budget, d // per_byte), dtype=torch.uint8, device=dev)
        vq = torch.empty_like(kq)
        ks = torch.empty((batch, hkv, budget), dtype=torch.float32, device=dev)
        vs = torch.empty_like(ks)
        idx = torch.empty((batch, hkv, budget), dtype=torch.int32, device=dev)
    else:
        kq, ks, vq, vs, idx = out
    for name, t, dt, shape in (("kq", kq, torch.uint8, (batch, hkv, budget, d // per_byte)),
                               ("vq", vq, torch.uint8, (batch, hkv, budget, d // per_byte)),
                               ("ks", ks, torch.float32, (batch, hkv, budget)),
                               ("vs", vs, torch.float32, (batch, hkv, budget)),
                               ("idx", idx, torch.int32, (batch, hkv, budget))):
        _check_tensor(name, t, len(shape), dt)
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} must have shape {shape}")
    if workspace is None:
        workspace = new_workspace(hq, hkv, d, vals, window, dev)
    _check(getattr(lib, fn)(
        batch, hq, hkv, d, _ptr(q_win), _ptr(k), _ptr(v), arr, window,
        _ptr(window_lse) if window_lse is not None else None, kernel_size,
        pool_mode_code(pool_mode), budget, _ptr(kq), _ptr(ks), _ptr(vq), _ptr(vs), _ptr(idx),
        _ptr(workspace), workspace.numel(), _stream(stream, dev)))
    return kq, ks, vq, vs, idx


def _decode_layout(k_cache: torch.Tensor):
    if k_cache.dim() == 4:
        return SNAPKV_CACHE_COMPRESSED, k_cache.shape[1], k_cache.shape[2], k_cache.shape[3]
    if k_cache.dim() == 3:
        return SNAPKV_CACHE_PACKED, k_cache.shape[1], 0, k_cache.shape[2]
    raise ValueError("k_cache must be [batch, H_kv, capacity, D] or [T, H_kv, D]")


def snapkv_decode_workspace_size(num_q_heads: int, num_kv_heads: int, head_dim: int,
                                 cache_lens: Sequence[int], layout: int,
                                 capacity: int = 0) -> int:
    lib = load_library()
    arr, vals = _lens(cache_lens)
    out = _sz(0)
    _check(lib.snapkv_decode_workspace_size(len(vals), num_q_heads, num_kv_heads, head_dim,
                                            layout, capacity, arr, ctypes.byref(out)))
    return out.value


def snapkv_decode_kernels(num_q_heads: int, num_kv_heads: int, head_dim: int,
                          cache_lens: Sequence[int], layout: int, capacity: int = 0) -> int:
    """How many kernels snapkv_decode_attention launches for this shape (1 or 2)."""
    lib = load_library()
    arr, vals = _lens(cache_lens)
    out = ctypes.c_int32(0)
    _check(lib.snapkv_decode_kernels(len(vals), num_q_heads, num_kv_heads, head_dim, layout,
                                     capacity, arr, ctypes.byref(out)))
    return out.value


def snapkv_decode_attention(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                            cache_lens: Sequence[int], *, out: Optional[torch.Tensor] = None,
                            workspace: Optional[torch.Tensor] = None, stream=None,
                            events=None):
    """One decode step's attention, float32 [batch, H_q, D]. The layout
    follows k_cache's rank: [batch, H_kv, capacity, D] is a compressed cache
    (snapkv_compress's out_k / out_v), [T, H_kv, D] the packed prefill cache;
    see include/snapkv.h. With events = (start, stop) (torch.cuda.Event with
    timing, already recorded once), the dispatches record them at the step's
    first kernel start and last kernel end."""
    return prepare_decode(q, k_cache, v_cache, cache_lens, out=out, workspace=workspace,
                          stream=stream, events=events)()


class DecodeStep:
    """A decode step whose arguments were checked once: calling it launches
    the step (one C call, nothing else), for loops that repeat a step on the
    same buffers. It holds references to its tensors; their contents may
    change between calls, their shapes and storage may not."""

    def __init__(self, fn, args, out, tensors):
        self._fn, self._args, self.out, self._tensors = fn, args, out, tensors

    def __call__(self):
        _check(self._fn(*self._args))
        return self.out


def prepare_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   cache_lens: Sequence[int], *, out: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None, stream=None,
                   events=None) -> DecodeStep:
    """Check the arguments of snapkv_decode_attention and return the step as
    a DecodeStep (see snapkv_decode_attention for the arguments)."""
    lib = load_library()
    _check_tensor("q", q, 3)
    layout, hkv, capacity, d = _decode_layout(k_cache)
    _check_tensor("k_cache", k_cache, k_cache.dim())
    _check_tensor("v_cache", v_cache, k_cache.dim())
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    arr, vals = _lens(cache_lens)
    batch, hq, dq = q.shape
    if dq != d or batch != len(vals):
        raise ValueError("q must be [batch, H_q, D] matching the cache and cache_lens")
    if layout == SNAPKV_CACHE_COMPRESSED and k_cache.shape[0] != batch:
        raise ValueError("compressed cache batch differs from q")
    if layout == SNAPKV_CACHE_PACKED and k_cache.shape[0] != sum(vals):
        raise ValueError("packed cache rows must equal sum(cache_lens)")
    dev = q.device
    if out is None:
        out = torch.empty((batch, hq, d), dtype=torch.float32, device=dev)
    _check_tensor("out", out, 3, torch.float32)
    if tuple(out.shape) != (batch, hq, d):
        raise ValueError("out must be [batch, H_q, D]")
    if workspace is None:
        nbytes = snapkv_decode_workspace_size(hq, hkv, d, vals, layout, capacity)
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    args = (batch, hq, hkv, d, _ptr(q), _ptr(k_cache), _ptr(v_cache), layout, capacity, arr,
            _ptr(out), _ptr(workspace), workspace.numel(), _stream(stream, dev))
    tensors = (q, k_cache, v_cache, out, workspace)
    if events is None:
        return DecodeStep(lib.snapkv_decode_attention, args, out, tensors)
    start, stop = events
    return DecodeStep(lib.snapkv_decode_attention_timed,
                      args + (int(start.cuda_event), int(stop.cuda_event)), out,
                      tensors + (start, stop))


def snapkv_window_scores(q_win: torch.Tensor, k: torch.Tensor, seq_lens: Sequence[int],
                         window: int, kernel_size: int, pool_mode, *,
                         out_scores: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None, stream=None):
    """Pooled vote scores [batch, H_kv, scores_len] (float32); see include/snapkv.h."""
    lib = load_library()
    _check_tensor("q_win", q_win, 4)
    _check_tensor("k", k, 3)
    arr, vals = _lens(seq_lens)
    batch, hq, hkv, d, w = _shapes(q_win, k, vals)
    if w != window:
        raise ValueError(f"q_win holds {w} window rows but window={window}")
    dev = q_win.device
    if out_scores is None:
        p_max = max(1, max(vals) - window)
        out_scores = torch.empty((batch, hkv, p_max), dtype=torch.float32, device=dev)
    _check_tensor("out_scores", out_scores, 3, torch.float32)
    if tuple(out_scores.shape[:2]) != (batch, hkv):
        raise ValueError("out_scores must be [batch, H_kv, scores_len]")
    if workspace is None:
        workspace = torch.empty(snapkv_workspace_size(hq, hkv, d, vals, window),
                                dtype=torch.uint8, device=dev)
    _check(lib.snapkv_window_scores(batch, hq, hkv, d, _ptr(q_win), _ptr(k), arr, window,
                                    kernel_size, pool_mode_code(pool_mode),
                                    _ptr(out_scores), out_scores.shape[2], _ptr(workspace),
                                    workspace.numel(), _stream(stream, dev)))
    return out_scores


def snapkv_status_string(status: int) -> str:
    return load_library().snapkv_status_string(status).decode()


def snapkv_last_error() -> str:
    return load_library().snapkv_last_error().decode()


def snapkv_score_kernels(num_q_heads: int, num_kv_heads: int, head_dim: int,
                         seq_lens: Iterable[int], window: int, kernel_size: int) -> int:
    """1 when snapkv_compress runs the vote statistics and the vote as one
    kernel (snapkv_score_fused) for this shape on the current device, else 2."""
    arr, vals = _lens(seq_lens)
    n = ctypes.c_int32(0)
    _check(load_library().snapkv_score_kernels(len(vals), num_q_heads, num_kv_heads, head_dim,
                                               arr, window, kernel_size, ctypes.byref(n)))
    return n.value


def snapkv_gather_selects(num_q_heads: int, num_kv_heads: int, head_dim: int,
                          seq_lens: Iterable[int], window: int, budget: int) -> int:
    """1 when snapkv_compress runs the selection inside the gather
    (snapkv_gather_select) for this shape on the current device, else 0."""
    arr, vals = _lens(seq_lens)
    n = ctypes.c_int32(0)
    _check(load_library().snapkv_gather_selects(len(vals), num_q_heads, num_kv_heads, head_dim,
                                                arr, window, budget, ctypes.byref(n)))
    return n.value

def snapkv_select_kernels(num_q_heads: int, num_kv_heads: int, head_dim: int,
                          seq_lens: Iterable[int], window: int, budget: int) -> int:
    """Which kernels snapkv_compress's selection stage launches for this
    shape on the current device: 0 none (inside the gather, or nothing to
    select), 1 snapkv_select, 2 snapkv_select_slices (the sliced selection
    as one launch), 3 the sliced selection as three kernels."""
    arr, vals = _lens(seq_lens)
    n = ctypes.c_int32(0)
    _check(load_library().snapkv_select_kernels(len(vals), num_q_heads, num_kv_heads, head_dim,
                                                arr, window, budget, ctypes.byref(n)))
    return n.value


def snapkv_stage_name(stage: int) -> Optional[str]:
    name = load_library().snapkv_stage_name(stage)
    return None if name is None else name.decode()


def compress(q_win, k, v, seq_lens, window_size: int = 32, max_capacity_prompt: int = 4096,
             kernel_size: int = 5, pooling: str = "avgpool", **kw):
    """snapkv_compress under the hyperparameter names of the SnapKV cache object
    (window_size, max_capacity_prompt, kernel_size, pooling)."""
    return snapkv_compress(q_win, k, v, seq_lens, window_size, kernel_size, pooling,
                           max_capacity_prompt, **kw)
