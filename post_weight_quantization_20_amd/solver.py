"""Python binding of the GPTQ layer-solver C ABI (include/gptq.h).

Argument marshalling only: tensors are torch device tensors, their data pointers and the current
HIP stream are handed to libgptq.so, and every step of the solver runs in its HIP kernels. Outputs
that the caller does not pass are allocated with torch.
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional, Tuple

import torch

from . import _lib

GPTQ_OK, GPTQ_EINVAL, GPTQ_ENOTPD, GPTQ_EUNSUPPORTED, GPTQ_EHIP, GPTQ_ENOMEM = 0, -1, -2, -3, -4, -5
GPTQ_F32, GPTQ_F16, GPTQ_BF16 = 0, 1, 2
GPTQ_WS_HESSIAN, GPTQ_WS_FACTOR, GPTQ_WS_QUANTIZE = 0, 1, 2
GPTQ_LAYOUT_FIELDS, GPTQ_LAYOUT_DENSE = 0, 1

_DTYPE = {torch.float32: GPTQ_F32, torch.float16: GPTQ_F16, torch.bfloat16: GPTQ_BF16}


class GPTQError(RuntimeError):
    """A non-zero status from the library; `info` carries gptq_factor's failed pivot."""

    def __init__(self, status: int, info: int = 0):
        msg = _lib.lib().gptq_status_string(status).decode()
        super().__init__(f"GPTQ status {status}: {msg}" + (f" (pivot {info})" if info else ""))
        self.status = status
        self.info = info


@dataclass
class Params:
    """Quantization settings (gptq_params_t)."""

    bits: int = 4
    group_size: int = 128
    block_size: int = 128
    act_order: bool = False
    sym: bool = False
    static_groups: bool = False
    damp: float = 0.01
    compact_meta: bool = False

    def c(self) -> _lib.gptq_params_t:
        return _lib.gptq_params_t(int(self.bits), int(self.group_size), int(self.block_size), int(bool(self.act_order)),
                                  int(bool(self.sym)), int(bool(self.static_groups)), int(bool(self.compact_meta)),
                                  float(self.damp))

    def groups(self, d: int) -> int:
        g = d if self.group_size <= 0 else self.group_size
        return (d + g - 1) // g


@dataclass
class QuantOutput:
    codes: torch.Tensor    # uint8 [rows, d], original column order
    scales: torch.Tensor   # float32 [rows, ngroups]
    zeros: torch.Tensor    # int32 [rows, ngroups]
    g_idx: torch.Tensor    # int32 [d]
    loss: torch.Tensor     # float64 [1]


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(status: int, info: int = 0) -> None:
    if status != GPTQ_OK:
        raise GPTQError(status, info)


def _need_cuda(*ts) -> None:
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must be on the GPU")


def _want(t: torch.Tensor, shape: tuple, dtype, name: str, device=None) -> None:
    """A caller-supplied tensor must have exactly this shape and dtype, be contiguous and sit on the
    given device: the library writes through its pointer without knowing its size."""
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}")


def _want_work(work: torch.Tensor, nbytes: int, device) -> None:
    if work.dtype != torch.uint8 or not work.is_contiguous() or work.numel() < nbytes or work.device != device:
        raise ValueError(f"work must be a contiguous uint8 tensor of at least {nbytes} bytes on {device}")


def gptq_workspace_bytes(kind: int, a: int, d: int, params: Optional[Params] = None) -> int:
    p = ctypes.byref(params.c()) if params is not None else None
    return int(_lib.lib().gptq_workspace_bytes(kind, a, d, p))


def _workspace(kind: int, a: int, d: int, params: Optional[Params], device) -> torch.Tensor:
    n = gptq_workspace_bytes(kind, a, d, params)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def _hessian_args(H: torch.Tensor, X: torch.Tensor, work: Optional[torch.Tensor], stream):
    _need_cuda(H, X, work)
    d = H.shape[0]
    if H.dtype != torch.float32 or H.shape != (d, d) or not H.is_contiguous():
        raise ValueError("H must be a contiguous float32 [d, d] tensor")
    if X.dim() != 2 or X.shape[1] != d or X.stride(1) != 1 or X.dtype not in _DTYPE:
        raise ValueError("X must be [tokens, d] with unit column stride, fp32/fp16/bf16")
    n = X.shape[0]
    if X.device != H.device:
        raise ValueError("X must be on H's device")
    if work is None:
        work = _workspace(GPTQ_WS_HESSIAN, n, d, None, H.device)
    elif work.dtype != torch.uint8 or not work.is_contiguous() or work.device != H.device:
        raise ValueError("work must be a contiguous uint8 tensor on H's device")
    return (_ptr(H), d, _ptr(X), _DTYPE[X.dtype], n, X.stride(0), _ptr(work), work.numel(), _stream(stream))


def gptq_hessian_accumulate(H: torch.Tensor, X: torch.Tensor, work: Optional[torch.Tensor] = None,
                            stream=None) -> None:
    """H (float32 [d, d], upper triangle) += 2 X^T X for X [tokens, d] (fp32 / fp16 / bf16)."""
    _check(_lib.lib().gptq_hessian_accumulate(*_hessian_args(H, X, work, stream)))


def gptq_hessian_compute(H: torch.Tensor, X: torch.Tensor, work: Optional[torch.Tensor] = None,
                         stream=None) -> None:
    """H (float32 [d, d], upper triangle) = 2 X^T X for X [tokens, d]: the first chunk, without
    zeroing H first."""
    _check(_lib.lib().gptq_hessian_compute(*_hessian_args(H, X, work, stream)))


def gptq_factor(H: torch.Tensor, n_total: int, params: Params, U: Optional[torch.Tensor] = None,
                perm: Optional[torch.Tensor] = None, work: Optional[torch.Tensor] = None,
                stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """(U, perm): U upper with (H/n + lambda I)[perm][:, perm]^-1 = U^T U. Raises GPTQError (with
    .info) when the damped Hessian is not positive definite. U may be H itself (the factor in place,
    which overwrites H)."""
    _need_cuda(H, U, perm, work)
    d = H.shape[0]
    if H.dtype != torch.float32 or H.shape != (d, d) or not H.is_contiguous():
        raise ValueError("H must be a contiguous float32 [d, d] tensor")
    if U is None:
        U = torch.empty((d, d), dtype=torch.float32, device=H.device)
    else:
        _want(U, (d, d), torch.float32, "U", H.device)
    if perm is None:
        perm = torch.empty(d, dtype=torch.int32, device=H.device)
    else:
        _want(perm, (d,), torch.int32, "perm", H.device)
    if work is None:
        work = _workspace(GPTQ_WS_FACTOR, 0, d, params, H.device)
    else:
        _want_work(work, gptq_workspace_bytes(GPTQ_WS_FACTOR, 0, d, params), H.device)
    info = ctypes.c_int64(0)
    st = _lib.lib().gptq_factor(_ptr(H), d, int(n_total), ctypes.byref(params.c()), _ptr(U), _ptr(perm), _ptr(work),
                                work.numel(), ctypes.byref(info), _stream(stream))
    _check(st, info.value)
    return U, perm


GPTQ_FACTOR_NOALLOC_MAX_D = 12288


def gptq_factor_noalloc(H: torch.Tensor, n_total: int, params: Params, U: torch.Tensor, perm: torch.Tensor,
                        stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """gptq_factor with the library's static scratch instead of a workspace, every launch on one
    stream, and no allocation in the call (U and perm are the caller's; U may be H). d is at most
    GPTQ_FACTOR_NOALLOC_MAX_D. Calls that overlap on one device race on the shared scratch."""
    _need_cuda(H, U, perm)
    d = H.shape[0]
    if H.dtype != torch.float32 or H.shape != (d, d) or not H.is_contiguous():
        raise ValueError("H must be a contiguous float32 [d, d] tensor")
    _want(U, (d, d), torch.float32, "U", H.device)
    _want(perm, (d,), torch.int32, "perm", H.device)
    info = ctypes.c_int64(0)
    st = _lib.lib().gptq_factor_noalloc(_ptr(H), d, int(n_total), ctypes.byref(params.c()), _ptr(U), _ptr(perm),
                                        ctypes.byref(info), _stream(stream))
    _check(st, info.value)
    return U, perm


def _quantize_args(W, U, perm, params, out, work):
    _need_cuda(W, U, perm, work)
    rows, d = W.shape
    if W.stride(1) != 1 or W.dtype not in _DTYPE:
        raise ValueError("W must be [rows, d] with unit column stride, fp32/fp16/bf16")
    dev = W.device
    _want(U, (d, d), torch.float32, "U", dev)
    _want(perm, (d,), torch.int32, "perm", dev)
    ng = params.groups(d)
    if out is None:
        out = QuantOutput(codes=torch.empty((rows, d), dtype=torch.uint8, device=dev),
                          scales=torch.empty((rows, ng), dtype=torch.float32, device=dev),
                          zeros=torch.empty((rows, ng), dtype=torch.int32, device=dev),
                          g_idx=torch.empty(d, dtype=torch.int32, device=dev),
                          loss=torch.empty(1, dtype=torch.float64, device=dev))
    else:
        _want(out.codes, (rows, d), torch.uint8, "out.codes", dev)
        _want(out.scales, (rows, ng), torch.float32, "out.scales", dev)
        _want(out.zeros, (rows, ng), torch.int32, "out.zeros", dev)
        _want(out.g_idx, (d,), torch.int32, "out.g_idx", dev)
        _want(out.loss, (1,), torch.float64, "out.loss", dev)
    if work is None:
        work = _workspace(GPTQ_WS_QUANTIZE, rows, d, params, dev)
    else:
        _want_work(work, gptq_workspace_bytes(GPTQ_WS_QUANTIZE, rows, d, params), dev)
    args = (_ptr(W), _DTYPE[W.dtype], rows, d, W.stride(0), _ptr(U), _ptr(perm), ctypes.byref(params.c()),
            _ptr(out.codes), _ptr(out.scales), _ptr(out.zeros), _ptr(out.g_idx), _ptr(out.loss), _ptr(work),
            work.numel())
    return out, args


def gptq_quantize_layer(W: torch.Tensor, U: torch.Tensor, perm: torch.Tensor, params: Params,
                        out: Optional[QuantOutput] = None, work: Optional[torch.Tensor] = None,
                        stream=None) -> QuantOutput:
    """The column loop: codes (original order), per-group scales and zeros, g_idx and the loss."""
    out, args = _quantize_args(W, U, perm, params, out, work)
    _check(_lib.lib().gptq_quantize_layer(*args, _stream(stream)))
    return out


QUANTIZE_PARTS = ("column_loop", "lazy_products", "other")


def gptq_quantize_layer_timed(W: torch.Tensor, U: torch.Tensor, perm: torch.Tensor, params: Params,
                              out: Optional[QuantOutput] = None, work: Optional[torch.Tensor] = None,
                              stream=None) -> Tuple[QuantOutput, dict]:
    """gptq_quantize_layer plus the device milliseconds of its parts (QUANTIZE_PARTS), from events
    between its launches; waits for the stream."""
    out, args = _quantize_args(W, U, perm, params, out, work)
    ms = (ctypes.c_double * 3)()
    _check(_lib.lib().gptq_quantize_layer_timed(*args, ms, _stream(stream)))
    return out, dict(zip(QUANTIZE_PARTS, (float(ms[0]), float(ms[1]), float(ms[2]))))


def packed_words(d: int, bits: int, dense: bool = False) -> int:
    """int32 words per row of packed codes: d/8 nibble fields, d/4 byte fields, or d*bits/32 dense."""
    return d * bits // 32 if dense else (d // 8 if bits <= 4 else d // 4)


def gptq_pack(codes: torch.Tensor, bits: int, packed: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """int32 [rows, words]: eight 4-bit fields per word (bits <= 4; column 8k + t in bits 4t..4t+3 of
    word k) or four 8-bit fields (bits 5..8)."""
    _need_cuda(codes, packed)
    rows, d = codes.shape
    if codes.dtype != torch.uint8 or not codes.is_contiguous():
        raise ValueError("codes must be contiguous uint8 [rows, d]")
    if packed is None:
        packed = torch.empty((rows, packed_words(d, bits)), dtype=torch.int32, device=codes.device)
    else:
        _want(packed, (rows, packed_words(d, bits)), torch.int32, "packed", codes.device)
    _check(_lib.lib().gptq_pack(_ptr(codes), rows, d, int(bits), _ptr(packed), _stream(stream)))
    return packed


def gptq_pack_dense(codes: torch.Tensor, bits: int, packed: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """int32 [rows, d * bits / 32]: each row as one bit stream, exactly `bits` bits per code."""
    _need_cuda(codes, packed)
    rows, d = codes.shape
    if codes.dtype != torch.uint8 or not codes.is_contiguous():
        raise ValueError("codes must be contiguous uint8 [rows, d]")
    if packed is None:
        packed = torch.empty((rows, packed_words(d, bits, True)), dtype=torch.int32, device=codes.device)
    else:
        _want(packed, (rows, packed_words(d, bits, True)), torch.int32, "packed", codes.device)
    _check(_lib.lib().gptq_pack_dense(_ptr(codes), rows, d, int(bits), _ptr(packed), _stream(stream)))
    return packed


def gptq_pack_ordered(codes: torch.Tensor, bits: int, order: torch.Tensor, packed: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
    """gptq_pack's layout with column j taken from codes[:, order[j]] (act-order layers stored in
    processing order, so that groups are contiguous)."""
    _need_cuda(codes, order, packed)
    rows, d = codes.shape
    if codes.dtype != torch.uint8 or not codes.is_contiguous():
        raise ValueError("codes must be contiguous uint8 [rows, d]")
    if order.dtype != torch.int32 or order.shape != (d,) or not order.is_contiguous():
        raise ValueError("order must be contiguous int32 [d]")
    if packed is None:
        packed = torch.empty((rows, packed_words(d, bits)), dtype=torch.int32, device=codes.device)
    else:
        _want(packed, (rows, packed_words(d, bits)), torch.int32, "packed", codes.device)
    _check(_lib.lib().gptq_pack_ordered(_ptr(codes), rows, d, int(bits), _ptr(order), _ptr(packed), _stream(stream)))
    return packed


def gptq_permute_columns(x: torch.Tensor, order: torch.Tensor, out: Optional[torch.Tensor] = None,
                         stream=None) -> torch.Tensor:
    """out[:, j] = x[:, order[j]] for a 2-D x with unit column stride."""
    _need_cuda(x, order, out)
    if x.dim() != 2 or x.stride(1) != 1 or x.dtype not in _DTYPE:
        raise ValueError("x must be 2-D with unit column stride, fp32/fp16/bf16")
    m, d = x.shape
    if order.dtype != torch.int32 or order.shape != (d,) or not order.is_contiguous():
        raise ValueError("order must be contiguous int32 [d]")
    if out is None:
        out = torch.empty((m, d), dtype=x.dtype, device=x.device)
    elif out.dim() != 2 or tuple(out.shape) != (m, d) or out.stride(1) != 1 or out.dtype != x.dtype \
            or out.device != x.device:
        raise ValueError("out must be [m, d] with unit column stride, x's dtype and device")
    _check(_lib.lib().gptq_permute_columns(_ptr(x), _DTYPE[x.dtype], m, d, x.stride(0), _ptr(order), _ptr(out),
                                           out.stride(0), _stream(stream)))
    return out


def gptq_dequant_gemm(x: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor,
                      d: int, group_size: int, g_idx: Optional[torch.Tensor] = None, bits: int = 4,
                      y: Optional[torch.Tensor] = None, dense: bool = False, stream=None) -> torch.Tensor:
    """y = x W^T (float32 [m, rows]) with W expanded from the packed codes, scales and zeros inside the
    kernel; g_idx (int32 [d]) maps columns to groups, None meaning column k is in group k // g."""
    _need_cuda(x, packed, scales, zeros, g_idx, y)
    if x.dim() != 2 or x.shape[1] != d or x.stride(1) != 1 or x.dtype not in _DTYPE:
        raise ValueError("x must be [m, d] with unit column stride, fp32/fp16/bf16")
    rows = packed.shape[0]
    g = d if group_size <= 0 else group_size
    ng = (d + g - 1) // g
    if packed.dtype != torch.int32 or packed.shape != (rows, packed_words(d, bits, dense)) or not packed.is_contiguous():
        raise ValueError("packed must be contiguous int32 [rows, words] in the chosen layout")
    if scales.dtype != torch.float32 or scales.shape != (rows, ng) or not scales.is_contiguous():
        raise ValueError("scales must be contiguous float32 [rows, ngroups]")
    if zeros.dtype != torch.int32 or zeros.shape != (rows, ng) or not zeros.is_contiguous():
        raise ValueError("zeros must be contiguous int32 [rows, ngroups]")
    if g_idx is not None and (g_idx.dtype != torch.int32 or g_idx.shape != (d,) or not g_idx.is_contiguous()):
        raise ValueError("g_idx must be contiguous int32 [d]")
    m = x.shape[0]
    if y is None:
        y = torch.empty((m, rows), dtype=torch.float32, device=x.device)
    if y.dtype != torch.float32 or y.dim() != 2 or y.shape != (m, rows) or y.stride(1) != 1 or y.device != x.device:
        raise ValueError("y must be float32 [m, rows] with unit column stride, on x's device")
    layout = GPTQ_LAYOUT_DENSE if dense else GPTQ_LAYOUT_FIELDS
    _check(_lib.lib().gptq_dequant_gemm(_ptr(x), _DTYPE[x.dtype], m, x.stride(0), _ptr(packed), int(bits), layout,
                                        _ptr(scales), _ptr(zeros), _ptr(g_idx), rows, d, int(group_size), _ptr(y),
                                        y.stride(0), _stream(stream)))
    return y


@dataclass
class LayerResult:
    H: torch.Tensor
    U: torch.Tensor
    perm: torch.Tensor
    quant: QuantOutput
    packed: Optional[torch.Tensor]


def quantize_layer(W: torch.Tensor, X_chunks, params: Params, stream=None) -> LayerResult:
    """The four calls in order for one layer: Hessian over the chunks, factor, column loop, pack."""
    d = W.shape[1]
    H = torch.zeros((d, d), dtype=torch.float32, device=W.device)
    n = 0
    work = None
    for xc in X_chunks:
        if work is None:
            work = _workspace(GPTQ_WS_HESSIAN, xc.shape[0], d, None, W.device)
        elif work.numel() < gptq_workspace_bytes(GPTQ_WS_HESSIAN, xc.shape[0], d):
            work = _workspace(GPTQ_WS_HESSIAN, xc.shape[0], d, None, W.device)
        gptq_hessian_accumulate(H, xc, work=work, stream=stream)
        n += xc.shape[0]
    U, perm = gptq_factor(H, n, params, stream=stream)
    q = gptq_quantize_layer(W, U, perm, params, stream=stream)
    packed = gptq_pack(q.codes, params.bits, stream=stream) if d % 8 == 0 else None
    return LayerResult(H=H, U=U, perm=perm, quant=q, packed=packed)


BLOCK_LAYERS = ("q", "k", "v", "o", "gate", "up", "down")


@dataclass
class BlockShape:
    """A pre-norm decoder block (gptq_block_shape_t): widths, heads and calibration sizes."""

    hidden: int
    heads: int
    inter: int
    seqs: int
    seq_len: int
    eps: float = 1e-6

    def c(self) -> _lib.gptq_block_shape_t:
        return _lib.gptq_block_shape_t(int(self.hidden), int(self.heads), int(self.inter), int(self.seqs),
                                       int(self.seq_len), float(self.eps))

    def layer_dims(self, i: int) -> Tuple[int, int]:
        """(rows, d) of layer i in BLOCK_LAYERS order."""
        rows = self.inter if i in (4, 5) else self.hidden
        return rows, (self.inter if i == 6 else self.hidden)


@dataclass
class BlockResult:
    layers: list                      # QuantOutput per layer, BLOCK_LAYERS order
    perms: list                       # int32 [d] processing order per layer
    Y: torch.Tensor                   # float32 [tokens, hidden]: block output through the quantized weights
    hessians: Optional[list]          # float32 [d, d] per stage (upper triangle), when asked for


def gptq_block_workspace_bytes(shape: BlockShape, params: Params) -> int:
    return int(_lib.lib().gptq_block_workspace_bytes(ctypes.byref(shape.c()), ctypes.byref(params.c())))


def gptq_quantize_block(X: torch.Tensor, weights, shape: BlockShape, params: Params, true_sequential: bool = True,
                        return_hessians: bool = False, work: Optional[torch.Tensor] = None,
                        stream=None) -> BlockResult:
    """Quantizes the seven layers of one decoder block (weights in BLOCK_LAYERS order, each
    contiguous [rows, d]) from its input X [seqs * seq_len, hidden], true-sequential by default."""
    _need_cuda(X, work, *weights)
    n = shape.seqs * shape.seq_len
    if len(weights) != 7:
        raise ValueError("seven weights: q, k, v, o, gate, up, down")
    if X.dim() != 2 or tuple(X.shape) != (n, shape.hidden) or not X.is_contiguous() or X.dtype not in _DTYPE:
        raise ValueError("X must be contiguous [seqs * seq_len, hidden], fp32/fp16/bf16")
    dev = X.device
    outs, perms = [], []
    arr = (_lib.gptq_block_layer_t * 7)()
    for i, W in enumerate(weights):
        rows, d = shape.layer_dims(i)
        if tuple(W.shape) != (rows, d) or not W.is_contiguous() or W.dtype not in _DTYPE:
            raise ValueError(f"{BLOCK_LAYERS[i]}: weights must be contiguous [{rows}, {d}], fp32/fp16/bf16")
        ng = params.groups(d)
        o = QuantOutput(codes=torch.empty((rows, d), dtype=torch.uint8, device=dev),
                        scales=torch.empty((rows, ng), dtype=torch.float32, device=dev),
                        zeros=torch.empty((rows, ng), dtype=torch.int32, device=dev),
                        g_idx=torch.empty(d, dtype=torch.int32, device=dev),
                        loss=torch.empty(1, dtype=torch.float64, device=dev))
        perm = torch.empty(d, dtype=torch.int32, device=dev)
        arr[i] = _lib.gptq_block_layer_t(W.data_ptr(), o.codes.data_ptr(), o.scales.data_ptr(), o.zeros.data_ptr(),
                                         o.g_idx.data_ptr(), perm.data_ptr(), o.loss.data_ptr(), _DTYPE[W.dtype])
        outs.append(o)
        perms.append(perm)
    Y = torch.empty((n, shape.hidden), dtype=torch.float32, device=dev)
    hess, hptr = None, None
    if return_hessians:
        widths = (shape.hidden, shape.hidden, shape.hidden, shape.inter)
        hess = [torch.empty((w, w), dtype=torch.float32, device=dev) for w in widths]
        hptr = (ctypes.c_void_p * 4)(*[h.data_ptr() for h in hess])
    nb = gptq_block_workspace_bytes(shape, params)
    if nb == 0:
        raise ValueError("invalid block shape or settings")
    if work is None:
        work = torch.empty(nb, dtype=torch.uint8, device=dev)
    else:
        _want_work(work, nb, dev)
    info = (ctypes.c_int64 * 2)()
    st = _lib.lib().gptq_quantize_block(ctypes.byref(shape.c()), _ptr(X), _DTYPE[X.dtype], ctypes.byref(params.c()),
                                        int(bool(true_sequential)), arr, _ptr(Y), hptr, _ptr(work), work.numel(),
                                        info, _stream(stream))
    _check(st, int(info[1]))
    return BlockResult(layers=outs, perms=perms, Y=Y, hessians=hess)
