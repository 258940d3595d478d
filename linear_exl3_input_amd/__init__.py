"""MI355X (gfx950) EXL3 quantized linear:  y = had(W_q . had(x*suh)) * svh.

A thin ctypes binding over the C ABI in ``include/exl3.h`` (``libexl3.so``,
built in-tree by ``linear_exl3_input_amd.build``).  Every step of the op runs
in the library's HIP kernels; this module only checks tensor metadata,
passes device pointers and the current HIP stream, and allocates outputs and
workspace with torch.  There is no CPU or PyTorch fallback: if the library is
missing, every call raises.

Functional form, as on the cuda-exl3 page ("One op per layer"):

    w = Exl3Weight(trellis, suh, svh, bits, codebook, shard_n)
    y = forward(w, x)                      # x bf16/fp16 [M, K] -> y [M, N]

or in two calls, ``input_transform`` then ``linear``.
"""
from __future__ import annotations

import ctypes
import os
import re
import threading
from dataclasses import dataclass
from typing import Dict, Optional, Sequence, Tuple

import torch

__all__ = [
    "CODEBOOKS", "Exl3Weight", "Exl3Error", "load", "lib_path", "input_transform", "linear", "forward",
    "workspace_bytes", "plan", "debug_codebook", "debug_decode", "debug_dequant", "debug_epilogue", "debug_parts",
    "debug_stream_read", "debug_mfma_loop", "debug_decode_rate", "mfma_loop_flops", "tune", "tune_clear",
    "input_transform_swiglu", "MoeWeight", "moe_rows_max", "moe_align", "moe_input_transform", "moe_linear",
    "moe_combine", "moe_forward", "reserve_workspace", "workspace_key",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libexl3.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "exl3.h")

CODEBOOKS = {"3inst": 0, "mcg": 1, "mul1": 2}
_F16, _BF16 = 0, 1
MAX_SHARDS = 16

EXL3_MODE_AUTO, EXL3_MODE_FUSED, EXL3_MODE_SLABS = -1, 0, 1
EXL3_DECODER_AUTO, EXL3_DECODER_ALU, EXL3_DECODER_TABLE, EXL3_DECODER_DENSE = -1, 0, 1, 2


class Exl3Error(RuntimeError):
    def __init__(self, status: int, name: str, message: str):
        super().__init__(f"{name}: {message}")
        self.status = status
        self.name = name


class _Weight(ctypes.Structure):
    _fields_ = [("trellis", ctypes.c_void_p), ("suh", ctypes.c_void_p), ("svh", ctypes.c_void_p),
                ("K", ctypes.c_int32), ("N", ctypes.c_int32), ("bits", ctypes.c_int32),
                ("codebook", ctypes.c_int32), ("n_shards", ctypes.c_int32),
                ("shard_n", ctypes.POINTER(ctypes.c_int32)), ("bias", ctypes.c_void_p)]


class _Plan(ctypes.Structure):
    _fields_ = [("parts", ctypes.c_int32), ("groups", ctypes.c_int32), ("mode", ctypes.c_int32),
                ("bm", ctypes.c_int32), ("decoder", ctypes.c_int32), ("unit", ctypes.c_int32),
                ("launches", ctypes.c_int32), ("wg_cols", ctypes.c_int32), ("workspace", ctypes.c_size_t)]


ABI_VERSION = 6
COUNTER_BYTES = 65536  # EXL3_WORKSPACE_COUNTER_BYTES: zeroed arrival counters at the workspace's start


_lib = None
_lib_lock = threading.Lock()


def lib_path() -> str:
    return _LIB_PATH


def load() -> ctypes.CDLL:
    """Load libexl3.so (raises if it has not been built)."""
    global _lib
    with _lib_lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"EXL3 HIP library not built: {_LIB_PATH} is missing "
                               "(run python -m linear_exl3_input_amd.build)")
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        W = ctypes.POINTER(_Weight)
        P = ctypes.POINTER(_Plan)
        sig = {
            "exl3_input_transform": (i32, [vp, i32, i32, i32, vp, i32, vp, vp]),
            "exl3_input_transform_swiglu": (i32, [vp, i32, i32, i32, vp, i32, vp, vp]),
            "exl3_workspace_bytes": (sz, [W, i32]),
            "exl3_workspace_bytes_ex": (sz, [W, i32, P]),
            "exl3_linear": (i32, [W, vp, i32, vp, i32, vp, sz, vp]),
            "exl3_linear_ex": (i32, [W, vp, i32, vp, i32, vp, sz, vp, P]),
            "exl3_linear_noalloc": (i32, [W, vp, i32, vp, i32, vp]),
            "exl3_forward": (i32, [W, vp, i32, i32, vp, i32, vp, sz, vp]),
            "exl3_forward_workspace_bytes": (sz, [W, i32]),
            "exl3_plan_query": (i32, [W, i32, P]),
            "exl3_plan_query_ex": (i32, [W, i32, P, P]),
            "exl3_status_str": (ctypes.c_char_p, [i32]),
            "exl3_last_error": (ctypes.c_char_p, []),
            "exl3_abi_version": (i32, []),
            "exl3_debug_codebook": (i32, [i32, vp, vp]),
            "exl3_debug_decode": (i32, [W, vp, vp]),
            "exl3_debug_epilogue": (i32, [vp, i32, i32, i32, W, vp, i32, vp]),
            "exl3_debug_parts": (i32, [W, vp, i32, vp, sz, vp, P]),
            "exl3_debug_stream_read": (i32, [vp, sz, vp, vp]),
            "exl3_debug_mfma_loop": (i32, [i32, ctypes.c_uint16, vp, vp]),
            "exl3_debug_decode_rate": (i32, [W, vp, vp]),
            "exl3_debug_dequant": (i32, [W, vp, sz, vp]),
            "exl3_debug_dense_gemm": (i32, [W, vp, sz, vp, i32, vp, i32, i32, ctypes.POINTER(i32), vp]),
            "exl3_tune": (i32, [W, i32, vp, i32, vp, i32, vp, sz, i32, vp, P]),
            "exl3_tune_workspace_bytes": (sz, [W, i32]),
            "exl3_tune_set": (i32, [W, i32, P]),
            "exl3_tune_clear": (None, []),
            "exl3_moe_rows_max": (i32, [i32, i32, i32, i32]),
            "exl3_moe_align": (i32, [vp, i32, i32, i32, i32, vp, vp, vp, vp]),
            "exl3_moe_input_transform": (i32, [vp, i32, i32, i32, i32, vp, i32, i32, vp, vp, i32, i32, i32, vp,
                                               vp]),
            "exl3_moe_workspace_bytes": (sz, [W, i32, i32]),
            "exl3_moe_linear": (i32, [W, i32, vp, i32, vp, i32, vp, i32, vp, sz, vp]),
            "exl3_moe_linear_ex": (i32, [W, i32, vp, i32, vp, i32, vp, i32, vp, sz, vp, i32]),
            "exl3_moe_combine": (i32, [vp, i32, vp, vp, i32, i32, i32, vp, vp]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        if L.exl3_abi_version() != ABI_VERSION:
            raise RuntimeError("libexl3.so ABI version mismatch")
        _lib = L
        return L


def header_symbols() -> Tuple[str, ...]:
    """Every function the public header declares."""
    text = open(HEADER).read()
    return tuple(sorted(set(re.findall(r"\b(exl3_[a-z_]+)\s*\(", text))))


def _check(status: int) -> None:
    if status != 0:
        L = load()
        raise Exl3Error(status, L.exl3_status_str(status).decode(), L.exl3_last_error().decode())


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dev_ptr(t: torch.Tensor, name: str, dtypes) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _out_ptr(t: torch.Tensor, name: str, shape: tuple, dtypes) -> int:
    """Device pointer of a caller-supplied output after checking its shape:
    the kernels write exactly `shape`, so a smaller tensor would be overrun."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return _dev_ptr(t, name, dtypes)


_U16 = (torch.int16, torch.uint16) if hasattr(torch, "uint16") else (torch.int16,)
_H16 = (torch.float16,) + _U16


@dataclass
class Exl3Weight:
    """An EXL3 weight on the GPU (trellis words, suh rows, svh, shard map)."""

    trellis: torch.Tensor          # int16 [K/16, N/16, 16*bits]
    suh: torch.Tensor              # fp16 [n_shards, K] (or [K] for one shard)
    svh: torch.Tensor              # fp16 [N]
    bits: int
    codebook: int | str
    shard_n: Optional[Sequence[int]] = None
    bias: Optional[torch.Tensor] = None  # fp16 [N], added before the output rounding

    def __post_init__(self):
        if isinstance(self.codebook, str):
            self.codebook = CODEBOOKS[self.codebook]
        if self.suh.dim() == 1:
            self.suh = self.suh.unsqueeze(0)
        kt, nt, words = self.trellis.shape
        self.K, self.N = kt * 16, nt * 16
        if words != 16 * self.bits:
            raise ValueError(f"trellis last dim {words} != 16*bits = {16 * self.bits}")
        if self.shard_n is None:
            self.shard_n = (self.N,)
        self.shard_n = tuple(int(n) for n in self.shard_n)
        self._shards = (ctypes.c_int32 * len(self.shard_n))(*self.shard_n)
        if self.bias is not None and self.bias.numel() != self.N:
            raise ValueError(f"bias has {self.bias.numel()} values, the layer {self.N} columns")
        self._view = _Weight(_dev_ptr(self.trellis, "trellis", _U16), _dev_ptr(self.suh, "suh", _H16),
                             _dev_ptr(self.svh, "svh", _H16), self.K, self.N, self.bits, int(self.codebook),
                             len(self.shard_n), self._shards,
                             _dev_ptr(self.bias, "bias", _H16) if self.bias is not None else None)

    @property
    def n_shards(self) -> int:
        return len(self.shard_n)

    def view(self) -> _Weight:
        return self._view


# Process-wide workspaces (the cuda-exl3 page, "VRAM": the activation and
# split-k workspaces are process-wide, not per layer), one per (device,
# stream): calls on one stream run one after another, so they may share one
# workspace, while calls on two streams may overlap and get one each.  The
# first COUNTER_BYTES of a workspace are the arrival counters that every call
# expects zero and leaves zero.  A workspace is never freed once handed out
# (a captured graph keeps its address): a larger one replaces it for later
# calls and the old one is kept alive.  Allocated under graph capture, the
# counters' zero fill is a kernel recorded in the graph (so every replay
# starts from zero), and the first eager call on that stream zeroes them
# before use.
_ws_lock = threading.Lock()
_workspaces: Dict[Tuple[int, int], torch.Tensor] = {}
_ws_needs_zero: set = set()
_ws_retired: list = []


def workspace_key(device: Optional[torch.device] = None, stream: Optional[torch.cuda.Stream] = None):
    """The (device index, stream handle) a call's workspace is kept under."""
    device = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    idx = device.index if device.index is not None else torch.cuda.current_device()
    s = stream if stream is not None else torch.cuda.current_stream(idx)
    return idx, int(s.cuda_stream)


def _workspace(nbytes: int, device: torch.device, stream: Optional[torch.cuda.Stream] = None) -> Tuple[int, int]:
    if nbytes == 0:
        return 0, 0
    key = workspace_key(device, stream)
    capturing = torch.cuda.is_current_stream_capturing()
    with _ws_lock:
        ws = _workspaces.get(key)
        if ws is None or ws.numel() < nbytes:
            new = torch.empty(max(nbytes, 1 << 20), dtype=torch.uint8, device=torch.device("cuda", key[0]))
            new[:COUNTER_BYTES].zero_()
            if capturing:
                _ws_needs_zero.add(key)
            if ws is not None:
                _ws_retired.append(ws)
            _workspaces[key] = ws = new
        elif key in _ws_needs_zero and not capturing:
            ws[:COUNTER_BYTES].zero_()
            _ws_needs_zero.discard(key)
    return ws.data_ptr(), ws.numel()


def reserve_workspace(nbytes: int, device=None, stream: Optional[torch.cuda.Stream] = None) -> None:
    """Size the workspace of (device, stream) now, e.g. before capturing a
    graph on that stream (workspace_bytes gives a call's need)."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    _workspace(nbytes, dev, stream)


def _force(parts=None, mode=None, bm=None, decoder=None, groups=None, unit=None, wg_cols=None) -> Optional[_Plan]:
    if (parts is None and mode is None and bm is None and decoder is None and groups is None and unit is None
            and wg_cols is None):
        return None
    return _Plan(parts if parts else -1, groups if groups else -1, EXL3_MODE_AUTO if mode is None else mode,
                 bm if bm else -1, EXL3_DECODER_AUTO if decoder is None else decoder, unit if unit else -1, 0,
                 wg_cols if wg_cols else -1, 0)


def workspace_bytes(w: Exl3Weight, M: int, parts=None, mode=None, bm=None, decoder=None, groups=None,
                    unit=None, wg_cols=None) -> int:
    f = _force(parts, mode, bm, decoder, groups, unit, wg_cols)
    L = load()
    n = L.exl3_workspace_bytes_ex(ctypes.byref(w.view()), M, ctypes.byref(f) if f else None)
    err = L.exl3_last_error().decode()
    if n == 0 and err:
        raise Exl3Error(1, "EXL3_ERR_INVALID_ARG", err)
    return n


def plan(w: Exl3Weight, M: int, parts=None, mode=None, bm=None, decoder=None, groups=None, unit=None,
         wg_cols=None) -> dict:
    """The plan exl3_linear uses for M rows (or with the given fields forced)."""
    f = _force(parts, mode, bm, decoder, groups, unit, wg_cols)
    p = _Plan()
    _check(load().exl3_plan_query_ex(ctypes.byref(w.view()), M, ctypes.byref(f) if f else None, ctypes.byref(p)))
    return {"parts": p.parts, "groups": p.groups, "mode": p.mode, "bm": p.bm, "decoder": p.decoder,
            "unit": p.unit, "launches": p.launches, "wg_cols": p.wg_cols, "workspace": p.workspace}


def rot_shape(n_shards: int, M: int, K: int) -> tuple:
    """Shape of the rotated activations: n_shards x K/32 k-step tiles of M rows
    x 32 values (the row's 32 values in fragment order)."""
    return (n_shards, K // 32, M, 32)


def input_transform(x: torch.Tensor, suh: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """had(x*suh) for every shard: x [M, K] bf16/fp16 -> x_rot fp16 of shape
    [S, K/32, M, 32] (the k-step tile order the GEMM reads; see rot_shape)."""
    if suh.dim() == 1:
        suh = suh.unsqueeze(0)
    M, K = x.shape
    S = suh.shape[0]
    if suh.shape[1] != K:
        raise ValueError(f"suh has K={suh.shape[1]}, x has K={K}")
    if x.dtype not in (torch.bfloat16, torch.float16):
        raise ValueError(f"x dtype {x.dtype} is not bf16/fp16")
    if out is None:
        out = torch.empty(rot_shape(S, M, K), dtype=torch.float16, device=x.device)
    elif tuple(out.shape) != rot_shape(S, M, K):
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {rot_shape(S, M, K)}")
    L = load()
    _check(L.exl3_input_transform(_dev_ptr(x, "x", (torch.bfloat16, torch.float16)),
                                  _BF16 if x.dtype == torch.bfloat16 else _F16, M, K,
                                  _dev_ptr(suh, "suh", _H16), S, _dev_ptr(out, "x_rot", _H16), _stream()))
    return out


def input_transform_swiglu(gate_up: torch.Tensor, suh: torch.Tensor,
                           out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The down projection's input rotation with SwiGLU folded in: gate_up
    [M, 2K] bf16/fp16 (gate = first K columns, up = last K) -> x_rot of
    act = rne(silu(gate) * up), as input_transform(act) would give."""
    if suh.dim() == 1:
        suh = suh.unsqueeze(0)
    M, K2 = gate_up.shape
    K = K2 // 2
    S = suh.shape[0]
    if K2 % 2 or suh.shape[1] != K:
        raise ValueError(f"gate_up has {K2} columns, suh K={suh.shape[1]}: expected 2*K")
    if gate_up.dtype not in (torch.bfloat16, torch.float16):
        raise ValueError(f"gate_up dtype {gate_up.dtype} is not bf16/fp16")
    if out is None:
        out = torch.empty(rot_shape(S, M, K), dtype=torch.float16, device=gate_up.device)
    elif tuple(out.shape) != rot_shape(S, M, K):
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {rot_shape(S, M, K)}")
    _check(load().exl3_input_transform_swiglu(_dev_ptr(gate_up, "gate_up", (torch.bfloat16, torch.float16)),
                                              _BF16 if gate_up.dtype == torch.bfloat16 else _F16, M, K,
                                              _dev_ptr(suh, "suh", _H16), S, _dev_ptr(out, "x_rot", _H16),
                                              _stream()))
    return out


def linear(w: Exl3Weight, x_rot: torch.Tensor, out_dtype: torch.dtype = torch.bfloat16,
           out: Optional[torch.Tensor] = None, parts=None, mode=None, bm=None,
           decoder=None, groups=None, unit=None, wg_cols=None) -> torch.Tensor:
    """z = x_rot . W_q per shard, then the output transform: -> y [M, N]."""
    if x_rot.dim() != 4 or x_rot.shape[3] != 32:
        raise ValueError(f"x_rot shape {tuple(x_rot.shape)} is not [S, K/32, M, 32]")
    S, KC, M, _ = x_rot.shape
    if S != w.n_shards or 32 * KC != w.K:
        raise ValueError(f"x_rot shape {tuple(x_rot.shape)} does not match the weight "
                         f"{rot_shape(w.n_shards, M, w.K)}")
    if out_dtype not in (torch.bfloat16, torch.float16):
        raise ValueError(f"out_dtype {out_dtype} is not bf16/fp16")
    if out is None:
        out = torch.empty((M, w.N), dtype=out_dtype, device=x_rot.device)
    y_ptr = _out_ptr(out, "out", (M, w.N), (out_dtype,))
    f = _force(parts, mode, bm, decoder, groups, unit, wg_cols)
    L = load()
    need = L.exl3_workspace_bytes_ex(ctypes.byref(w.view()), M, ctypes.byref(f) if f else None)
    ws, wsn = _workspace(need, x_rot.device)
    _check(L.exl3_linear_ex(ctypes.byref(w.view()), _dev_ptr(x_rot, "x_rot", _H16), M,
                            y_ptr, _BF16 if out_dtype == torch.bfloat16 else _F16,
                            ws, wsn, _stream(), ctypes.byref(f) if f else None))
    return out


def forward_workspace_bytes(w: Exl3Weight, M: int) -> int:
    L = load()
    n = L.exl3_forward_workspace_bytes(ctypes.byref(w.view()), M)
    err = L.exl3_last_error().decode()
    if n == 0 and err:
        raise Exl3Error(1, "EXL3_ERR_INVALID_ARG", err)
    return n


def forward(w: Exl3Weight, x: torch.Tensor, out_dtype: Optional[torch.dtype] = None,
            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The whole layer in one call (exl3_forward): y = had(W_q . had(x*suh)) * svh,
    the same bits as linear(w, input_transform(x, w.suh)); x [M, K] bf16 or fp16,
    y in out_dtype (default x's dtype)."""
    if x.dim() != 2 or x.shape[1] != w.K:
        raise ValueError(f"x shape {tuple(x.shape)} is not [M, {w.K}]")
    out_dtype = out_dtype or x.dtype
    if out_dtype not in (torch.bfloat16, torch.float16):
        raise ValueError(f"out_dtype {out_dtype} is not bf16/fp16")
    M = x.shape[0]
    if out is None:
        out = torch.empty((M, w.N), dtype=out_dtype, device=x.device)
    y_ptr = _out_ptr(out, "out", (M, w.N), (out_dtype,))
    x_ptr = _dev_ptr(x, "x", (torch.bfloat16, torch.float16))
    L = load()
    need = forward_workspace_bytes(w, M)
    ws, wsn = _workspace(need, x.device)
    _check(L.exl3_forward(ctypes.byref(w.view()), x_ptr, _BF16 if x.dtype == torch.bfloat16 else _F16, M, y_ptr,
                          _BF16 if out_dtype == torch.bfloat16 else _F16, ws, wsn, _stream()))
    return out


def debug_codebook(codebook: int | str, device="cuda") -> torch.Tensor:
    cb = CODEBOOKS[codebook] if isinstance(codebook, str) else codebook
    out = torch.empty(65536, dtype=torch.int16, device=device)
    _check(load().exl3_debug_codebook(cb, out.data_ptr(), _stream()))
    return out


def debug_decode(w: Exl3Weight) -> torch.Tensor:
    out = torch.empty((w.K, w.N), dtype=torch.int16, device=w.trellis.device)
    _check(load().exl3_debug_decode(ctypes.byref(w.view()), out.data_ptr(), _stream()))
    return out


def debug_dequant(w: Exl3Weight, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The dense decoder's first stage alone: W_q as matrix-core B fragments,
    int16 [K/32, N/128, 8, 64, 8] (see exl3_debug_dequant in the header)."""
    shape = (w.K // 32, w.N // 128, 8, 64, 8)
    if out is None:
        out = torch.empty(shape, dtype=torch.int16, device=w.trellis.device)
    elif tuple(out.shape) != shape:
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {shape}")
    _check(load().exl3_debug_dequant(ctypes.byref(w.view()), _dev_ptr(out, "frags", _U16), out.numel() * 2,
                                     _stream()))
    return out


def debug_dense_gemm(w: Exl3Weight, frags: torch.Tensor, x_rot: torch.Tensor, which: int = 3,
                     out_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None):
    """The dense GEMM stage alone over debug_dequant's fragments: which = 1
    the 256 x 256 launch, 2 the 256 x 128 launch over the column blocks after
    it, 3 both.  Returns (y [M, N], column blocks of the 256 x 256 launch)."""
    if x_rot.dim() != 4 or x_rot.shape[3] != 32:
        raise ValueError(f"x_rot shape {tuple(x_rot.shape)} is not [S, K/32, M, 32]")
    M = x_rot.shape[2]
    if out is None:
        out = torch.empty((M, w.N), dtype=out_dtype, device=x_rot.device)
    y_ptr = _out_ptr(out, "out", (M, w.N), (out_dtype,))
    bulk = ctypes.c_int32(0)
    _check(load().exl3_debug_dense_gemm(ctypes.byref(w.view()), _dev_ptr(frags, "frags", (torch.int16,)),
                                        frags.numel() * 2, _dev_ptr(x_rot, "x_rot", _H16), M, y_ptr,
                                        _BF16 if out_dtype == torch.bfloat16 else _F16, which, ctypes.byref(bulk),
                                        _stream()))
    return out, bulk.value


def debug_parts(w: Exl3Weight, x_rot: torch.Tensor, parts=None, bm=None, decoder=None,
                out: Optional[torch.Tensor] = None, groups=None, unit=None, wg_cols=None) -> torch.Tensor:
    """The trellis GEMM stage alone: the fp32 sum of every K part (unit 1,
    the default) or of every unit of `unit` parts, in the slab layout
    [P/unit, ceil(M/4), N, 4] (what debug_epilogue reads)."""
    if x_rot.dim() != 4 or x_rot.shape[3] != 32:
        raise ValueError(f"x_rot shape {tuple(x_rot.shape)} is not [S, K/32, M, 32]")
    M = x_rot.shape[2]
    P = parts if parts else plan(w, M)["parts"]
    shape = (P // (unit or 1), (M + 3) // 4, w.N, 4)
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=x_rot.device)
    elif tuple(out.shape) != shape or out.dtype != torch.float32:
        raise ValueError(f"out is {tuple(out.shape)} {out.dtype}, expected {shape} float32")
    f = _force(parts, EXL3_MODE_SLABS, bm, decoder, groups, unit, wg_cols)
    _check(load().exl3_debug_parts(ctypes.byref(w.view()), _dev_ptr(x_rot, "x_rot", _H16), M,
                                   _dev_ptr(out, "z_parts", (torch.float32,)), out.numel() * 4, _stream(),
                                   ctypes.byref(f)))
    return out


def debug_epilogue(w: Exl3Weight, z_parts: torch.Tensor, M: int, out_dtype=torch.bfloat16,
                   out: Optional[torch.Tensor] = None, groups: Optional[int] = None) -> torch.Tensor:
    """Ordered part sum + output transform of fp32 partials in the slab
    layout [P, ceil(M/4), N, 4]: `groups` groups of P/groups consecutive
    slabs (default P: the plain ordered fold)."""
    if z_parts.dim() != 4 or z_parts.shape[1] != (M + 3) // 4 or z_parts.shape[3] != 4:
        raise ValueError(f"z_parts shape {tuple(z_parts.shape)} is not [P, ceil(M/4), N, 4] for M={M}")
    P, _, N, _ = z_parts.shape
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=z_parts.device)
    out_dtype = out.dtype
    y_ptr = _out_ptr(out, "out", (M, N), (torch.bfloat16, torch.float16))
    _check(load().exl3_debug_epilogue(_dev_ptr(z_parts, "z_parts", (torch.float32,)), P, groups or P, M,
                                      ctypes.byref(w.view()),
                                      y_ptr, _BF16 if out_dtype == torch.bfloat16 else _F16, _stream()))
    return out


# ---------------------------------------------------------------- rulers
RULER_WORDS = 262144


def debug_stream_read(buf: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Streaming read of a whole device buffer (measurement ruler): returns
    RULER_WORDS int32 whose XOR is the XOR of the buffer's 4-byte words."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    nbytes = buf.numel() * buf.element_size()
    if out is None:
        out = torch.empty(RULER_WORDS, dtype=torch.int32, device=buf.device)
    _check(load().exl3_debug_stream_read(buf.data_ptr(), nbytes, _out_ptr(out, "out", (RULER_WORDS,), (torch.int32,)),
                                         _stream()))
    return out


def debug_mfma_loop(iters: int, one: int = 0x3C00, device="cuda", out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Matrix-core ruler: RULER_WORDS/64 waves x iters x 16 fp16 MFMAs of
    16x16x32 with all operands `one` (fp16 bits); returns the lanes' sums."""
    if out is None:
        out = torch.empty(RULER_WORDS, dtype=torch.float32, device=device)
    _check(load().exl3_debug_mfma_loop(iters, one, _out_ptr(out, "out", (RULER_WORDS,), (torch.float32,)), _stream()))
    return out


def mfma_loop_flops(iters: int) -> float:
    return 16384.0 * 16 * iters * (RULER_WORDS // 64)


def debug_decode_rate(w: Exl3Weight, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Decode ruler: stage and decode every weight as the GEMM kernels do, no
    products; returns [K/128, N/128] int32 block XORs (low half: even k, high
    half: odd k of the fp16 W_q values)."""
    if out is None:
        out = torch.empty((w.K // 128, w.N // 128), dtype=torch.int32, device=w.trellis.device)
    o_ptr = _out_ptr(out, "out", (w.K // 128, w.N // 128), (torch.int32,))
    _check(load().exl3_debug_decode_rate(ctypes.byref(w.view()), o_ptr, _stream()))
    return out


# ----------------------------------------------------------- autotuner
def _plan_dict(p: _Plan) -> dict:
    return {"parts": p.parts, "groups": p.groups, "mode": p.mode, "bm": p.bm, "decoder": p.decoder,
            "unit": p.unit, "launches": p.launches, "wg_cols": p.wg_cols, "workspace": p.workspace}


def tune(w, x_rot: torch.Tensor, reps: int = 5) -> dict:
    """Time every schedule of the shape's part tree on these rows (eager, not
    under graph capture) and record the fastest for the shape and M bucket;
    later unforced calls use it.  `w` is one Exl3Weight or a list of copies
    of one shape, cycled by the timed calls (copies that exceed the caches
    time cold weights).  Returns the chosen plan."""
    copies = list(w) if isinstance(w, (list, tuple)) else [w]
    arr = (_Weight * len(copies))(*[c.view() for c in copies])
    S, KC, M, _ = x_rot.shape
    L = load()
    need = L.exl3_tune_workspace_bytes(ctypes.byref(copies[0].view()), M)
    if need == 0 and L.exl3_last_error():
        _check(1)
    ws, wsn = _workspace(need, x_rot.device)
    y = torch.empty((M, copies[0].N), dtype=torch.bfloat16, device=x_rot.device)
    best = _Plan()
    _check(L.exl3_tune(arr, len(copies), _dev_ptr(x_rot, "x_rot", _H16), M, y.data_ptr(), _BF16, ws, wsn,
                       reps, _stream(), ctypes.byref(best)))
    return _plan_dict(best)


def tune_set(w: Exl3Weight, M: int, plan: dict) -> None:
    f = _Plan(plan["parts"], plan["groups"], plan["mode"], plan["bm"], plan["decoder"], plan["unit"], 0,
              plan["wg_cols"], 0)
    _check(load().exl3_tune_set(ctypes.byref(w.view()), M, ctypes.byref(f)))


def tune_clear() -> None:
    load().exl3_tune_clear()


# ----------------------------------------------------- mixture of experts
class MoeWeight:
    """E experts of one shape, stacked: trellis [E, K/16, N/16, 16*bits],
    suh [E, n_shards, K], svh [E, N], bias [E, N] or None.  The library sees
    expert 0's view and steps to expert e by the fixed strides."""

    def __init__(self, trellis, suh, svh, bits, codebook, shard_n=None, bias=None):
        if suh.dim() == 2:
            suh = suh.unsqueeze(1)
        self.E = trellis.shape[0]
        if suh.shape[0] != self.E or svh.shape[0] != self.E or (bias is not None and bias.shape[0] != self.E):
            raise ValueError("trellis, suh, svh (and bias) must stack the same number of experts")
        for t in (trellis, suh, svh) + ((bias,) if bias is not None else ()):
            if not t.is_contiguous():
                raise ValueError("expert stacks must be contiguous")
        self.stack = (trellis, suh, svh, bias)
        self.first = Exl3Weight(trellis[0], suh[0], svh[0], bits, codebook, shard_n,
                                bias[0] if bias is not None else None)
        self.K, self.N, self.bits, self.n_shards = self.first.K, self.first.N, bits, self.first.n_shards

    def expert(self, e: int) -> Exl3Weight:
        trellis, suh, svh, bias = self.stack
        return Exl3Weight(trellis[e], suh[e], svh[e], self.bits, self.first.codebook, self.first.shard_n,
                          bias[e] if bias is not None else None)


def moe_rows_max(T: int, topk: int, E: int, block: int = 16) -> int:
    return int(load().exl3_moe_rows_max(T, topk, E, block))


def moe_align(topk_ids: torch.Tensor, E: int, block: int = 16):
    """topk_ids [T, topk] int32 -> (row_pair [rows], block_expert [rows/block],
    pair_row [T*topk]) int32 on the same device."""
    T, k = topk_ids.shape
    rows = moe_rows_max(T, k, E, block)
    dev = topk_ids.device
    row_pair = torch.empty(max(rows, 1), dtype=torch.int32, device=dev)
    block_expert = torch.empty(max(rows // block, 1), dtype=torch.int32, device=dev)
    pair_row = torch.empty(max(T * k, 1), dtype=torch.int32, device=dev)
    _check(load().exl3_moe_align(_dev_ptr(topk_ids.contiguous(), "topk_ids", (torch.int32,)), T, k, E, block,
                                 row_pair.data_ptr(), block_expert.data_ptr(), pair_row.data_ptr(), _stream()))
    return row_pair[:rows], block_expert[:rows // block], pair_row[:T * k]


def moe_input_transform(x: torch.Tensor, w: MoeWeight, route, topk: int, block: int = 16,
                        swiglu: bool = False) -> torch.Tensor:
    row_pair, block_expert, _ = route
    T = x.shape[0]
    K = w.K
    if x.shape[1] != (2 * K if swiglu else K):
        raise ValueError(f"x has {x.shape[1]} columns, expected {2 * K if swiglu else K}")
    rows = moe_rows_max(T, topk, w.E, block)
    if row_pair.numel() != rows or block_expert.numel() != rows // block:
        raise ValueError(f"route has {row_pair.numel()} rows and {block_expert.numel()} blocks, expected "
                         f"{rows} and {rows // block} for T={T}, topk={topk}, E={w.E}, block={block}")
    out = torch.empty(rot_shape(w.n_shards, rows, K), dtype=torch.float16, device=x.device)
    _check(load().exl3_moe_input_transform(_dev_ptr(x, "x", (torch.bfloat16, torch.float16)),
                                           _BF16 if x.dtype == torch.bfloat16 else _F16, int(swiglu), T, K,
                                           _dev_ptr(w.stack[1], "suh", _H16), w.n_shards, w.E,
                                           _dev_ptr(row_pair, "row_pair", (torch.int32,)),
                                           _dev_ptr(block_expert, "block_expert", (torch.int32,)), topk, block, rows,
                                           out.data_ptr(), _stream()))
    return out


def moe_linear(w: MoeWeight, x_rot: torch.Tensor, block_expert: torch.Tensor, block: int = 16,
               out_dtype: torch.dtype = torch.bfloat16, decoder: int = EXL3_DECODER_AUTO) -> torch.Tensor:
    """The grouped GEMM (exl3_moe_linear_ex); decoder AUTO, ALU or TABLE."""
    if x_rot.dim() != 4 or tuple(x_rot.shape) != rot_shape(w.n_shards, x_rot.shape[2], w.K):
        raise ValueError(f"x_rot shape {tuple(x_rot.shape)} is not [{w.n_shards}, {w.K // 32}, rows, 32]")
    rows = x_rot.shape[2]
    if block_expert.numel() != rows // block:
        raise ValueError(f"block_expert has {block_expert.numel()} entries, expected rows/block = {rows // block}")
    L = load()
    need = L.exl3_moe_workspace_bytes(ctypes.byref(w.first.view()), rows, block)
    if need == 0 and L.exl3_last_error():
        _check(1)
    ws, wsn = _workspace(need, x_rot.device)
    y = torch.empty((rows, w.N), dtype=out_dtype, device=x_rot.device)
    _check(L.exl3_moe_linear_ex(ctypes.byref(w.first.view()), w.E, _dev_ptr(x_rot, "x_rot", _H16), rows,
                                _dev_ptr(block_expert, "block_expert", (torch.int32,)), block, y.data_ptr(),
                                _BF16 if out_dtype == torch.bfloat16 else _F16, ws, wsn, _stream(), int(decoder)))
    return y


def moe_combine(y_routed: torch.Tensor, pair_row: torch.Tensor, topk_weights: torch.Tensor) -> torch.Tensor:
    T, k = topk_weights.shape
    N = y_routed.shape[1]
    if pair_row.numel() != T * k:
        raise ValueError(f"pair_row has {pair_row.numel()} entries, expected T*topk = {T * k}")
    out = torch.empty((T, N), dtype=y_routed.dtype, device=y_routed.device)
    _check(load().exl3_moe_combine(_dev_ptr(y_routed, "y_routed", (torch.bfloat16, torch.float16)),
                                   _BF16 if y_routed.dtype == torch.bfloat16 else _F16,
                                   _dev_ptr(pair_row, "pair_row", (torch.int32,)),
                                   _dev_ptr(topk_weights.contiguous(), "topk_weights", (torch.float32,)), T, k, N,
                                   out.data_ptr(), _stream()))
    return out


def moe_forward(x: torch.Tensor, w: MoeWeight, topk_ids: torch.Tensor, topk_weights: torch.Tensor,
                block: int = 16, swiglu: bool = False, decoder: int = EXL3_DECODER_AUTO) -> torch.Tensor:
    """Routed experts: align, rotate each routed row with its expert's suh,
    the grouped GEMM, and the ordered combine.  -> [T, N] in x's dtype."""
    route = moe_align(topk_ids, w.E, block)
    xr = moe_input_transform(x, w, route, topk_ids.shape[1], block, swiglu)
    y = moe_linear(w, xr, route[1], block, x.dtype, decoder)
    return moe_combine(y, route[2], topk_weights)
