"""Python binding of libvit.so, the MI355X (gfx950) forward pass of a
Qwen3-VL-style ViT vision tower.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libvit.so`` (see ``include/vit.h`` for the contract of each
entry point).  torch provides device memory and the current stream; outputs
that a call does not receive are allocated here with torch.  The library
must be built (``python -m vision_transformer_encoder_amd.build``); every
call raises if it is missing - there is no fallback.
"""

from __future__ import annotations

import ctypes
import math
import os
import re
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch

__all__ = [
    "VitError", "require_library", "library_path", "declared_functions",
    "vit_abi_version", "vit_status_string", "vit_quant_fp8_block128", "vit_e4m3_encode",
    "vit_layernorm_quant_fp8", "vit_fp8_block128_gemm", "vit_bf16_gemm", "vit_rope2d",
    "vit_attention", "vit_attention_workspace_size", "vit_attention_noalloc",
    "vit_attention_noalloc_scratch_size", "vit_merge2x2_layernorm", "vit_block_workspace_size", "vit_block_forward",
    "vit_encoder_workspace_size", "vit_encoder_forward", "BlockWeights", "MergerWeights",
    "EncoderWeights", "EPI_BIAS", "EPI_BIAS_RESIDUAL", "EPI_BIAS_GELU_FP8", "BEPI_BIAS",
    "BEPI_BIAS_GELU", "BEPI_BIAS_ADD",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_PKG)
# VIT_LIBRARY names another build of the same library (a host-sanitizer
# build, for instance); by default the in-tree libvit.so
library_path = os.environ.get("VIT_LIBRARY") or os.path.join(_PKG, "libvit.so")
header_path = os.path.join(_ROOT, "include", "vit.h")

ABI_VERSION = 5  # VIT_ABI_VERSION of the include/vit.h these signatures follow
HIDDEN, HEADS, HEAD_DIM, MLP, MLP_PADDED = 1152, 16, 72, 4304, 4352
PATCH_DIM, DEPTH, OUT_HIDDEN, MERGED_DIM, NUM_TAPS = 1536, 27, 4096, 4608, 4
EPI_BIAS, EPI_BIAS_RESIDUAL, EPI_BIAS_GELU_FP8 = 0, 1, 2
BEPI_BIAS, BEPI_BIAS_GELU, BEPI_BIAS_ADD = 0, 1, 2

_STATUS = {0: "VIT_OK", 1: "VIT_ERR_NULL", 2: "VIT_ERR_ALIGN", 3: "VIT_ERR_SHAPE",
           4: "VIT_ERR_UNSUPPORTED", 5: "VIT_ERR_SEQLENS", 6: "VIT_ERR_WORKSPACE",
           7: "VIT_ERR_ALIAS", 8: "VIT_ERR_HIP"}


class VitError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {_STATUS.get(status, status)}")


_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_F = ctypes.c_float
_SZ = ctypes.c_size_t


class _BlockW(ctypes.Structure):
    _fields_ = [(n, _P) for n in (
        "ln1_gamma", "ln1_beta", "qkv_codes", "qkv_scales", "qkv_bias", "proj_codes", "proj_scales",
        "proj_bias", "ln2_gamma", "ln2_beta", "fc1_codes", "fc1_scales", "fc1_bias", "fc2_codes",
        "fc2_scales", "fc2_bias", "qkv_w", "proj_w", "fc1_w", "fc2_w")]


class _MergerW(ctypes.Structure):
    _fields_ = [(n, _P) for n in ("ln_gamma", "ln_beta", "fc1_w", "fc1_b", "fc2_w", "fc2_b", "fc1_codes",
                                  "fc1_scales", "fc2_codes", "fc2_scales")]


class _EncoderW(ctypes.Structure):
    _fields_ = [("patch_w", _P), ("patch_b", _P), ("blocks", _BlockW * DEPTH),
                ("mergers", _MergerW * NUM_TAPS), ("pos_table", _P), ("pos_grid_side", _I)]


_SIGS = {
    "vit_abi_version": (_I, []),
    "vit_status_string": (ctypes.c_char_p, [_I]),
    "vit_quant_fp8_block128": (_I, [_P, _I64, _I, _I, _I, _P, _P, _P]),
    "vit_e4m3_encode": (_I, [_P, _P, _I64, _P]),
    "vit_layernorm_quant_fp8": (_I, [_P, _I64, _P, _P, _F, _I, _I, _P, _P, _P, _P]),
    "vit_layernorm": (_I, [_P, _I64, _P, _P, _F, _I, _I, _P, _I64, _P]),
    "vit_fp8_block128_gemm": (_I, [_P, _P, _P, _P, _I, _I, _I, _P, _P, _I, _P, _P, _P, _P, _P]),
    "vit_bf16_gemm": (_I, [_P, _I, _P, _I, _I, _I, _P, _P, _I, _P, _I64, _P]),
    "vit_rope2d": (_I, [_P, _P, _I64, _P, _I, _I, _I, _F, _P]),
    "vit_attention_workspace_size": (_SZ, []),
    "vit_attention": (_I, [_P, _P, _P, _I64, _P, _I64, _P, _P, _I, _I, _I, _I, _F, _P, _SZ, _P]),
    "vit_attention_noalloc_scratch_size": (_SZ, []),
    "vit_attention_noalloc": (_I, [_P, _P, _P, _I64, _P, _I64, _P, _P, _I, _I, _I, _I, _F, _P]),
    "vit_merge2x2_layernorm": (_I, [_P, _I, _P, _P, _P, _I, _I, _P, _P, _F, _P, _P]),
    "vit_pos_embed_interp": (_I, [_P, _I, _I, _P, _P, _P, _I, _I, _P, _I64, _P]),
    "vit_smart_resize": (_I, [_I, _I, _I, _I64, _I64, ctypes.POINTER(_I), ctypes.POINTER(_I)]),
    "vit_preprocess_frames": (_I, [_P, _I, _I, _I, _I, _I, _P, _P, _P, _P]),
    "vit_block_workspace_size": (_SZ, [_I]),
    "vit_block_forward": (_I, [ctypes.POINTER(_BlockW), _P, _I, _P, _P, _P, _I, _P, _SZ, _P]),
    "vit_encoder_workspace_size": (_SZ, [_I, _I]),
    "vit_encoder_forward": (_I, [ctypes.POINTER(_EncoderW), _P, _P, _P, _P, _I, _I, _P, _P, _P, _SZ, _P]),
}

_lib = None


def require_library() -> ctypes.CDLL:
    """Load libvit.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise RuntimeError(f"{library_path} is missing: build it with "
                               "`python -m vision_transformer_encoder_amd.build`")
        lib = ctypes.CDLL(library_path)
        for name, (res, args) in _SIGS.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        if lib.vit_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{library_path} has ABI version {lib.vit_abi_version()}, this binding "
                               f"expects {ABI_VERSION}: rebuild it")
        _lib = lib
    return _lib


def declared_functions() -> List[str]:
    """Names of the functions include/vit.h declares."""
    txt = open(header_path).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(vit_\w+)\s*\(", txt, flags=re.M)))


# --------------------------------------------------------------------- helpers

def _call(name: str, *args) -> None:
    st = getattr(require_library(), name)(*args)
    if st != 0:
        raise VitError(name, st)


def _stream(device=None) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _p(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("device tensor expected")
    return t.data_ptr()


def _host_i32(a) -> Tuple[np.ndarray, int]:
    arr = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return arr, arr.ctypes.data


def _out_like(given: Optional[torch.Tensor], shape, dtype, dev) -> torch.Tensor:
    """A caller-provided output buffer (checked: contiguous, shape, dtype) or
    a new one."""
    if given is None:
        return torch.empty(shape, dtype=dtype, device=dev)
    if tuple(given.shape) != tuple(shape) or given.dtype != dtype or not given.is_contiguous():
        raise ValueError(f"output buffer must be a contiguous {dtype} tensor of shape {tuple(shape)}")
    return given


def _row_ld(t: torch.Tensor) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("2-D tensor with unit column stride expected")
    return t.stride(0)


def bf16_from_bits(bits: np.ndarray, device) -> torch.Tensor:
    """Upload bf16 bit patterns (uint16) as a bfloat16 tensor."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


# --------------------------------------------------------------------- ops

def vit_abi_version() -> int:
    return require_library().vit_abi_version()


def vit_status_string(status: int) -> str:
    return require_library().vit_status_string(status).decode()


def vit_quant_fp8_block128(x: torch.Tensor, cols: Optional[int] = None, block_rows: int = 1,
                           out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None):
    """Block-128 FP8 quantisation of a bf16 [rows, >=cols] tensor.
    Returns (codes uint8 [Rp, Cp], scales float32)."""
    rows = x.shape[0]
    cols = x.shape[1] if cols is None else cols
    cp = (cols + 127) // 128 * 128
    rp = rows if block_rows == 1 else (rows + 127) // 128 * 128
    oc, os_ = out if out is not None else (None, None)
    codes = _out_like(oc, (rp, cp), torch.uint8, x.device)
    scales = _out_like(os_, ((rows + block_rows - 1) // block_rows, cp // 128), torch.float32, x.device)
    _call("vit_quant_fp8_block128", _p(x), _row_ld(x), rows, cols, block_rows, _p(codes), _p(scales),
          _stream(x.device))
    return codes, scales


def vit_e4m3_encode(x: torch.Tensor) -> torch.Tensor:
    x = x.contiguous()
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _call("vit_e4m3_encode", _p(x), _p(codes), x.numel(), _stream(x.device))
    return codes


def vit_layernorm_quant_fp8(x: torch.Tensor, gamma: torch.Tensor, beta: torch.Tensor, eps: float = 1e-6,
                            prequant: bool = False, out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None):
    M, D = x.shape
    oc, os_ = out if out is not None else (None, None)
    codes = _out_like(oc, (M, D), torch.uint8, x.device)
    scales = _out_like(os_, (M, D // 128), torch.float32, x.device)
    pre = torch.empty((M, D), dtype=torch.float32, device=x.device) if prequant else None
    _call("vit_layernorm_quant_fp8", _p(x), _row_ld(x), _p(gamma), _p(beta), eps, M, D, _p(codes), _p(scales),
          _p(pre), _stream(x.device))
    return (codes, scales, pre) if prequant else (codes, scales)


def vit_layernorm(x: torch.Tensor, gamma: torch.Tensor, beta: torch.Tensor, eps: float = 1e-6,
                  out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """LayerNorm of x [M, D] bf16 rows with a bf16 result."""
    M, D = x.shape
    out = _out_like(out, (M, D), torch.bfloat16, x.device)
    _call("vit_layernorm", _p(x), _row_ld(x), _p(gamma), _p(beta), eps, M, D, _p(out), D, _stream(x.device))
    return out


def vit_fp8_block128_gemm(a: torch.Tensor, a_scales: torch.Tensor, w: torch.Tensor, w_scales: torch.Tensor,
                          N: int, K: int, bias: Optional[torch.Tensor] = None,
                          residual: Optional[torch.Tensor] = None, epilogue: int = EPI_BIAS,
                          out=None, prequant: bool = False):
    """Block-scaled FP8 GEMM.  EPI_BIAS / EPI_BIAS_RESIDUAL return the bf16
    [M, N] output (``out`` may be given, and may be ``residual`` for an
    in-place add); EPI_BIAS_GELU_FP8 returns (codes, scales[, prequant])
    (``out`` may be given as the (codes, scales) pair)."""
    M = a.shape[0]
    np_ = (N + 127) // 128 * 128
    dev = a.device
    codes = scales = pre = None
    if epilogue == EPI_BIAS_GELU_FP8:
        oc, os_ = out if out is not None else (None, None)
        codes = _out_like(oc, (M, np_), torch.uint8, dev)
        scales = _out_like(os_, (M, np_ // 128), torch.float32, dev)
        pre = torch.empty((M, np_), dtype=torch.float32, device=dev) if prequant else None
    elif out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    _call("vit_fp8_block128_gemm", _p(a), _p(a_scales), _p(w), _p(w_scales), M, N, K, _p(bias), _p(residual),
          epilogue, _p(out) if epilogue != EPI_BIAS_GELU_FP8 else None, _p(codes), _p(scales), _p(pre),
          _stream(dev))
    if epilogue == EPI_BIAS_GELU_FP8:
        return (codes, scales, pre) if prequant else (codes, scales)
    return out


def vit_bf16_gemm(a: torch.Tensor, w: torch.Tensor, bias: Optional[torch.Tensor] = None,
                  add: Optional[torch.Tensor] = None, epilogue: int = BEPI_BIAS,
                  out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bf16 GEMM a [M, K] (bf16, or fp32 rounded on load) times w [N, K]^T."""
    M, K = a.shape
    N = w.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    _call("vit_bf16_gemm", _p(a), 1 if a.dtype == torch.float32 else 0, _p(w), M, N, K, _p(bias), _p(add),
          epilogue, _p(out), _row_ld(out), _stream(a.device))
    return out


def vit_rope2d(q: torch.Tensor, k: torch.Tensor, pos_rc: torch.Tensor, num_heads: int = HEADS,
               head_dim: int = HEAD_DIM, theta: float = 10000.0) -> None:
    """In-place 2D RoPE on q and k ([T, >=H*hd] views with the same row stride)."""
    ld = _row_ld(q)
    if _row_ld(k) != ld:
        raise ValueError("q and k must share a row stride")
    _call("vit_rope2d", _p(q), _p(k), ld, _p(pos_rc), q.shape[0], num_heads, head_dim, theta,
          _stream(q.device))


def vit_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: Sequence[int],
                  cu_seqlens_dev: Optional[torch.Tensor] = None, num_heads: int = HEADS,
                  head_dim: int = HEAD_DIM, softmax_scale: Optional[float] = None,
                  out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    ld = _row_ld(q)
    if _row_ld(k) != ld or _row_ld(v) != ld:
        raise ValueError("q, k, v must share a row stride")
    T = q.shape[0]
    cu_h, cu_ptr = _host_i32(cu_seqlens)
    if cu_seqlens_dev is None:
        cu_seqlens_dev = torch.from_numpy(cu_h.copy()).to(q.device)
    if out is None:
        out = torch.empty((T, num_heads * head_dim), dtype=torch.bfloat16, device=q.device)
    scale = 1.0 / math.sqrt(head_dim) if softmax_scale is None else softmax_scale
    if workspace is None:
        workspace = _workspace(vit_attention_workspace_size(), q.device)
    _call("vit_attention", _p(q), _p(k), _p(v), ld, _p(out), _row_ld(out), _p(cu_seqlens_dev), cu_ptr,
          len(cu_h) - 1, T, num_heads, head_dim, scale, _p(workspace), workspace.numel() * workspace.element_size(),
          _stream(q.device))
    return out


def vit_attention_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: Sequence[int],
                          cu_seqlens_dev: torch.Tensor, out: torch.Tensor, num_heads: int = HEADS,
                          head_dim: int = HEAD_DIM, softmax_scale: Optional[float] = None) -> torch.Tensor:
    """vit_attention without a workspace: the library's own per-device
    scratch holds the partials.  The caller passes the device cu_seqlens
    and the output buffer; the call itself allocates nothing."""
    ld = _row_ld(q)
    if _row_ld(k) != ld or _row_ld(v) != ld:
        raise ValueError("q, k, v must share a row stride")
    cu_h, cu_ptr = _host_i32(cu_seqlens)
    scale = 1.0 / math.sqrt(head_dim) if softmax_scale is None else softmax_scale
    _call("vit_attention_noalloc", _p(q), _p(k), _p(v), ld, _p(out), _row_ld(out), _p(cu_seqlens_dev), cu_ptr,
          len(cu_h) - 1, q.shape[0], num_heads, head_dim, scale, _stream(q.device))
    return out


def vit_attention_noalloc_scratch_size() -> int:
    return int(require_library().vit_attention_noalloc_scratch_size())


def vit_attention_workspace_size() -> int:
    return int(require_library().vit_attention_workspace_size())


def _grid_arrays(grids, device, grid_dev=None, cu_dev=None):
    """Host grids [n, 2] int32 (and their address), and the device grids and
    token offsets cu [n + 1] (uploaded unless given)."""
    g_h, g_ptr = _host_i32(np.asarray(grids, dtype=np.int32).reshape(-1, 2))
    if grid_dev is None:
        grid_dev = torch.from_numpy(g_h.copy()).to(device)
    if cu_dev is None:
        cu = np.concatenate([[0], np.cumsum(g_h[:, 0].astype(np.int64) * g_h[:, 1])]).astype(np.int32)
        cu_dev = torch.from_numpy(cu).to(device)
    return g_h, g_ptr, grid_dev, cu_dev


def vit_merge2x2_layernorm(x: torch.Tensor, grids: Sequence[Tuple[int, int]], gamma: torch.Tensor,
                           beta: torch.Tensor, eps: float = 1e-6,
                           grid_dev: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                           cu_dev: Optional[torch.Tensor] = None) -> torch.Tensor:
    T, D = x.shape
    g_h, g_ptr, grid_dev, cu_dev = _grid_arrays(grids, x.device, grid_dev, cu_dev)
    out = _out_like(out, (T // 4, 4 * D), torch.bfloat16, x.device)
    _call("vit_merge2x2_layernorm", _p(x), D, _p(grid_dev), _p(cu_dev), g_ptr, len(g_h), T, _p(gamma), _p(beta),
          eps, _p(out), _stream(x.device))
    return out


def vit_pos_embed_interp(table: torch.Tensor, grids: Sequence[Tuple[int, int]], grid_side: Optional[int] = None,
                         grid_dev: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                         cu_dev: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The learned [G*G, D] position table resampled to the grids: [T, D] bf16."""
    GG, D = table.shape
    G = int(round(math.sqrt(GG))) if grid_side is None else int(grid_side)
    g_h, g_ptr, grid_dev, cu_dev = _grid_arrays(grids, table.device, grid_dev, cu_dev)
    T = int(sum(int(h) * int(w) for h, w in g_h))
    if out is None:
        out = torch.empty((T, D), dtype=torch.bfloat16, device=table.device)
    elif (out.dtype != torch.bfloat16 or tuple(out.shape) != (T, D) or out.device != table.device
          or out.stride(1) != 1):
        raise ValueError(f"output buffer must be a bfloat16 [{T}, {D}] tensor with unit column stride "
                         "(rows may be strided)")
    _call("vit_pos_embed_interp", _p(table), G, D, _p(grid_dev), _p(cu_dev), g_ptr, len(g_h), T, _p(out),
          _row_ld(out), _stream(table.device))
    return out


def vit_smart_resize(height: int, width: int, factor: int = 32, min_pixels: int = 0,
                     max_pixels: Optional[int] = None) -> Tuple[int, int]:
    """Resized (height, width), multiples of ``factor`` (host computation)."""
    h, w = _I(0), _I(0)
    _call("vit_smart_resize", int(height), int(width), int(factor), int(min_pixels or 0), int(max_pixels or 0),
          ctypes.byref(h), ctypes.byref(w))
    return h.value, w.value


def vit_preprocess_frames(frames: torch.Tensor, out_size: Tuple[int, int], mean: Sequence[float],
                          std: Sequence[float], out: Optional[torch.Tensor] = None):
    """[F, H, W, 3] uint8 frames on the device -> (pixels [P, 1536] f32, grids):
    one grid (out_h/16, out_w/16) per frame pair."""
    if frames.dtype != torch.uint8 or frames.dim() != 4 or frames.shape[3] != 3 or not frames.is_contiguous():
        raise ValueError("frames must be a contiguous uint8 [F, H, W, 3] tensor")
    F_, H, W, _ = frames.shape
    oh, ow = int(out_size[0]), int(out_size[1])
    G = (F_ + 1) // 2
    rows = G * (oh // 16) * (ow // 16)
    out = _out_like(out, (rows, PATCH_DIM), torch.float32, frames.device)
    m = (ctypes.c_float * 3)(*[float(v) for v in mean])
    sd = (ctypes.c_float * 3)(*[float(v) for v in std])
    _call("vit_preprocess_frames", _p(frames), F_, H, W, oh, ow, ctypes.cast(m, _P), ctypes.cast(sd, _P), _p(out),
          _stream(frames.device))
    return out, [(oh // 16, ow // 16)] * G


def vit_block_workspace_size(T: int) -> int:
    return int(require_library().vit_block_workspace_size(T))


def vit_encoder_workspace_size(T: int, num_images: int) -> int:
    return int(require_library().vit_encoder_workspace_size(T, num_images))


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


# --------------------------------------------------------------------- weights

def quantize_weight(w: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """128x128-block FP8 form of a bf16 [N, K] weight (padded to 128s)."""
    return vit_quant_fp8_block128(w, block_rows=128)


class BlockWeights:
    """Device copy of one block: bf16 norms and biases, and the GEMM weights
    either quantised on the GPU with vit_quant_fp8_block128(block_rows=128)
    (precision "fp8") or kept in bf16 (precision "bf16": the block runs its
    LayerNorms and GEMMs in bf16)."""

    def __init__(self, params: dict, device, precision: str = "fp8"):
        if precision not in ("fp8", "bf16"):
            raise ValueError("precision is 'fp8' or 'bf16'")
        t = {k: bf16_from_bits(v, device) for k, v in params.items()}
        self.t = t
        self.precision = precision
        self.q = {n: quantize_weight(t[n + "_w"]) for n in ("qkv", "proj", "fc1", "fc2")} if precision == "fp8" else {}
        s = _BlockW()
        s.ln1_gamma, s.ln1_beta = _p(t["ln1_g"]), _p(t["ln1_b"])
        s.ln2_gamma, s.ln2_beta = _p(t["ln2_g"]), _p(t["ln2_b"])
        for n in ("qkv", "proj", "fc1", "fc2"):
            if precision == "fp8":
                setattr(s, n + "_codes", _p(self.q[n][0]))
                setattr(s, n + "_scales", _p(self.q[n][1]))
            else:
                setattr(s, n + "_w", _p(t[n + "_w"]))
            setattr(s, n + "_bias", _p(t[n + "_b"]))
        self.struct = s


class MergerWeights:
    """Device copy of one merger: bf16, or (precision "fp8") with its two
    linears also quantised in 128x128 blocks, which selects the FP8 path."""

    def __init__(self, params: dict, device, precision: str = "bf16"):
        if precision not in ("fp8", "bf16"):
            raise ValueError("precision is 'fp8' or 'bf16'")
        t = {k: bf16_from_bits(v, device) for k, v in params.items()}
        self.t = t
        self.precision = precision
        s = _MergerW()
        s.ln_gamma, s.ln_beta = _p(t["m_ln_g"]), _p(t["m_ln_b"])
        s.fc1_w, s.fc1_b, s.fc2_w, s.fc2_b = _p(t["m_fc1_w"]), _p(t["m_fc1_b"]), _p(t["m_fc2_w"]), _p(t["m_fc2_b"])
        self.q = {}
        if precision == "fp8":
            self.q = {n: quantize_weight(t["m_" + n + "_w"]) for n in ("fc1", "fc2")}
            s.fc1_codes, s.fc1_scales = _p(self.q["fc1"][0]), _p(self.q["fc1"][1])
            s.fc2_codes, s.fc2_scales = _p(self.q["fc2"][0]), _p(self.q["fc2"][1])
        self.struct = s


class EncoderWeights:
    def __init__(self, patch: dict, blocks: Sequence[dict], mergers: Sequence[dict], device,
                 bf16_blocks: int = 0, fp8_mergers: bool = False, pos_table=None):
        """bf16_blocks: the first n blocks run in bf16 (FlashRT keeps 3);
        fp8_mergers: the mergers run their linears in FP8; pos_table: the
        learned [G*G, 1152] position table (bf16 bits), resampled to each
        forward's grids and added after the patch embedding."""
        if len(blocks) != DEPTH or len(mergers) != NUM_TAPS:
            raise ValueError("the tower has 27 blocks and 4 mergers")
        if not 0 <= bf16_blocks <= DEPTH:
            raise ValueError("bf16_blocks is in 0..27")
        self.patch = {k: bf16_from_bits(v, device) for k, v in patch.items()}
        self.blocks = [BlockWeights(b, device, "bf16" if i < bf16_blocks else "fp8") for i, b in enumerate(blocks)]
        self.mergers = [MergerWeights(m, device, "fp8" if fp8_mergers else "bf16") for m in mergers]
        s = _EncoderW()
        s.patch_w, s.patch_b = _p(self.patch["patch_w"]), _p(self.patch["patch_b"])
        for i, b in enumerate(self.blocks):
            s.blocks[i] = b.struct
        for i, m in enumerate(self.mergers):
            s.mergers[i] = m.struct
        self.pos_table = None
        if pos_table is not None:
            self.pos_table = bf16_from_bits(pos_table, device)
            g = int(round(math.sqrt(self.pos_table.shape[0])))
            if g * g != self.pos_table.shape[0] or self.pos_table.shape[1] != HIDDEN:
                raise ValueError("pos_table must be [G*G, 1152]")
            s.pos_table, s.pos_grid_side = _p(self.pos_table), g
        self.struct = s


# --------------------------------------------------------------------- block / encoder

def vit_block_forward(w: BlockWeights, x: torch.Tensor, pos_rc: torch.Tensor, cu_seqlens: Sequence[int],
                      cu_seqlens_dev: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One block in place on x [T, 1152] bf16; returns x."""
    T = x.shape[0]
    cu_h, cu_ptr = _host_i32(cu_seqlens)
    if cu_seqlens_dev is None:
        cu_seqlens_dev = torch.from_numpy(cu_h.copy()).to(x.device)
    need = vit_block_workspace_size(T)
    if workspace is None:
        workspace = _workspace(need, x.device)
    _call("vit_block_forward", ctypes.byref(w.struct), _p(x), T, _p(pos_rc), _p(cu_seqlens_dev), cu_ptr,
          len(cu_h) - 1, _p(workspace), workspace.numel(), _stream(x.device))
    return x


def vit_encoder_forward(w: EncoderWeights, pixels: torch.Tensor, grids: Sequence[Tuple[int, int]],
                        pos_embed: Optional[torch.Tensor] = None, want_last_hidden: bool = False,
                        workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                        grid_dev: Optional[torch.Tensor] = None, last_hidden: Optional[torch.Tensor] = None):
    """Whole tower.  Returns (out [4, T/4, 4096] bf16, last_hidden or None)."""
    T = pixels.shape[0]
    g_h, g_ptr = _host_i32(np.asarray(grids, dtype=np.int32).reshape(-1, 2))
    dev = pixels.device
    if grid_dev is None:
        grid_dev = torch.from_numpy(g_h.copy()).to(dev)
    if out is None:
        out = torch.empty((NUM_TAPS, T // 4, OUT_HIDDEN), dtype=torch.bfloat16, device=dev)
    if want_last_hidden and last_hidden is None:
        last_hidden = torch.empty((T, HIDDEN), dtype=torch.bfloat16, device=dev)
    need = vit_encoder_workspace_size(T, len(g_h))
    if workspace is None:
        workspace = _workspace(need, dev)
    _call("vit_encoder_forward", ctypes.byref(w.struct), _p(pixels), _p(pos_embed), _p(grid_dev), g_ptr,
          len(g_h), T, _p(out), _p(last_hidden), _p(workspace), workspace.numel(), _stream(dev))
    return out, last_hidden
