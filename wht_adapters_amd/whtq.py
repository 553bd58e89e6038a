"""ctypes binding over libwhtq.so (C ABI in include/whtq.h).

Argument marshalling only: tensors are checked for device, dtype, layout and
shape, their pointers and the current HIP stream are handed to the library,
and every step of the computation runs in the library's HIP kernels.  There
is no CPU fallback: importing this module fails if the library is missing.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.environ.get("WHTQ_LIB", os.path.join(_HERE, "libwhtq.so"))

if not os.path.exists(lib_path):
    raise ImportError(
        f"libwhtq.so not found at {lib_path}; build it with `python -m wht_adapters_amd.build`")
_lib = ctypes.CDLL(lib_path)

_i64, _int, _vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p

_SIG = {
    "wht_batched": [_vp, _int, _vp, _int, _i64, _i64, _i64, _i64, _vp, _int, _int, _vp],
    "rht_quantize_rtn": [_vp, _int, _i64, _i64, _i64, _vp, _int, _int, _vp, _vp, _vp],
    "rht_dequantize_inverse": [_vp, _vp, _i64, _i64, _vp, _int, _int, _vp, _int, _i64, _vp],
    "qwha_adapter_forward": [_vp, _int, _i64, _i64, _i64, _vp, _vp, _vp, _int, _i64, _i64, _vp, _int,
                             _i64, _vp],
    "harp_rotate": [_vp, _vp, _int, _i64, _i64, _i64, _i64, _vp, _int, _vp, _int, _vp, _int, _vp],
    "qwha_csr_transpose": [_vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp],
    "harp_build_blocks": [_vp, _int, _vp, _i64, _vp, _int, _vp, _vp, _int, _vp],
    "qwha_permute_values": [_vp, _int, _vp, _i64, _vp, _vp],
    "qwha_adapter_backward_input": [_vp, _int, _i64, _i64, _i64, _vp, _vp, _vp, _int, _i64, _i64, _vp, _int,
                                    _i64, _vp],
    "qwha_adapter_grad_values": [_vp, _vp, _int, _i64, _i64, _i64, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _i64,
                                 _vp],
    "rht_lowbit_gemv": [_vp, _i64, _i64, _vp, _vp, _i64, _i64, _vp, _int, _int, _vp, _i64, _vp],
    "qwha_init_error_coeffs": [_vp, _int, _i64, _i64, _i64, _vp, _vp, _vp, _int, _int, _vp, _i64, _vp],
    "qwha_init_gram": [_vp, _int, _i64, _i64, _i64, _vp, _vp, _int, _vp],
    "qwha_init_channel_errors": [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp],
    "qwha_init_allocate": [_vp, _i64, _i64, _i64, _int, _int, _vp],
    "qwha_init_select": [_vp, _i64, _i64, _i64, _vp, _vp, _vp],
    "qwha_init_refine": [_vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp],
    "whtq_stream_probe": [_vp, _i64, _vp, _i64, _vp],
    "qwha_adapter_grad_values_noalloc": [_vp, _vp, _int, _i64, _i64, _i64, _i64, _i64, _vp, _vp, _i64, _vp,
                                         _vp],
    "qwha_forward_plan": [_i64, _i64, _vp, _i64, _i64, _vp, _i64, _vp],
    "qwha_adapter_forward_planned": [_vp, _int, _i64, _i64, _i64, _vp, _vp, _vp, _int, _i64, _i64, _vp, _i64,
                                     _vp, _int, _i64, _vp],
}
for _name, _args in _SIG.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _int
_lib.qwha_grad_values_workspace_bytes.argtypes = [_i64, _i64, _i64]
_lib.qwha_grad_values_workspace_bytes.restype = _i64
_lib.qwha_forward_plan_bytes.argtypes = [_i64, _i64, _i64, _i64]
_lib.qwha_forward_plan_bytes.restype = _i64
_lib.whtq_status_string.argtypes = [_int]
_lib.whtq_status_string.restype = ctypes.c_char_p
_lib.whtq_last_hip_error.restype = _int
_lib.whtq_abi_version.restype = _int

F32, BF16, F16, I8 = 0, 1, 2, 3
_DT = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16, torch.int8: I8}
SIGN_NONE, SIGN_BEFORE, SIGN_AFTER = 0, 1, 2
_SIGN_MODES = {"none": SIGN_NONE, "before": SIGN_BEFORE, "after": SIGN_AFTER}


class WhtqError(RuntimeError):
    def __init__(self, fn, status):
        msg = _lib.whtq_status_string(status).decode()
        if status == 4:
            msg += f" (hipError {_lib.whtq_last_hip_error()})"
        super().__init__(f"{fn}: {msg} [status {status}]")
        self.status = status


def abi_version():
    return _lib.whtq_abi_version()


def raw():
    """The ctypes library handle (for callers that marshal pointers themselves)."""
    return _lib


def _check(fn, status):
    if status != 0:
        raise WhtqError(fn, status)


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need_cuda(name, t):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")


def _rows_ld(name, t):
    """(rows, n, ld) of a 2-D tensor with unit stride along the last dim."""
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be 2-D with a contiguous last dimension")
    rows, n = t.shape
    # a single row's stride is meaningless (torch may report 0 or 1 for it)
    return rows, n, (t.stride(0) if rows > 1 else n)


def _sign_ptr(signs, n, device):
    if signs is None:
        return ctypes.c_void_p(0)
    _need_cuda("signs", signs)
    if signs.dtype not in (torch.int32, torch.uint32) or signs.numel() * 32 < n or not signs.is_contiguous():
        raise ValueError("signs must be a contiguous int32/uint32 bitmask of ceil(n/32) words")
    if signs.device != device:
        raise ValueError("signs must be on the same device")
    return _ptr(signs)


def wht_batched(x, out=None, *, signs=None, sign_mode="none", normalize=True, out_dtype=None):
    """y = Hn(S x) ('before'), Hn x ('none') or S Hn x ('after') along the last dim."""
    _need_cuda("x", x)
    rows, n, ldx = _rows_ld("x", x)
    if out is None:
        out = torch.empty((rows, n), dtype=out_dtype or x.dtype, device=x.device)
    _need_cuda("out", out)
    r2, n2, ldy = _rows_ld("out", out)
    if (r2, n2) != (rows, n):
        raise ValueError("out shape mismatch")
    mode = _SIGN_MODES[sign_mode]
    with torch.cuda.device(x.device):
        _check("wht_batched", _lib.wht_batched(
            _ptr(x), _DT[x.dtype], _ptr(out), _DT[out.dtype], rows, n, ldx, ldy,
            _sign_ptr(signs, n, x.device), mode, int(bool(normalize)), _stream(x)))
    return out


def rht_quantize_rtn(w, signs, bits, group, codes=None, scales=None):
    """Returns (codes uint8 [rows, n*bits/8], scales float16 [rows, n/group])."""
    _need_cuda("w", w)
    rows, n, ldw = _rows_ld("w", w)
    if codes is None:
        codes = torch.empty((rows, n * bits // 8), dtype=torch.uint8, device=w.device)
    if scales is None:
        scales = torch.empty((rows, max(1, n // group)), dtype=torch.float16, device=w.device)
    if not (codes.is_contiguous() and scales.is_contiguous()):
        raise ValueError("codes and scales must be contiguous")
    with torch.cuda.device(w.device):
        _check("rht_quantize_rtn", _lib.rht_quantize_rtn(
            _ptr(w), _DT[w.dtype], rows, n, ldw, _sign_ptr(signs, n, w.device), bits, group,
            _ptr(codes), _ptr(scales), _stream(w)))
    return codes, scales


def rht_dequantize_inverse(codes, scales, signs, bits, group, n, out=None, out_dtype=torch.bfloat16):
    """out = S Hn (q * s) for codes/scales written by rht_quantize_rtn."""
    _need_cuda("codes", codes)
    rows = codes.shape[0]
    if codes.dtype != torch.uint8 or scales.dtype != torch.float16:
        raise ValueError("codes must be uint8 and scales float16")
    if codes.shape != (rows, n * bits // 8) or scales.shape != (rows, n // group):
        raise ValueError("codes / scales shape mismatch")
    if out is None:
        out = torch.empty((rows, n), dtype=out_dtype, device=codes.device)
    r2, n2, ldo = _rows_ld("out", out)
    if (r2, n2) != (rows, n):
        raise ValueError("out shape mismatch")
    with torch.cuda.device(codes.device):
        _check("rht_dequantize_inverse", _lib.rht_dequantize_inverse(
            _ptr(codes), _ptr(scales), rows, n, _sign_ptr(signs, n, codes.device), bits, group,
            _ptr(out), _DT[out.dtype], ldo, _stream(codes)))
    return out


def rht_lowbit_gemv(x, codes, scales, signs, bits, group, out=None):
    """y = x W_hat^T for W_hat the rows rht_dequantize_inverse would decode from
    (codes, scales); x [tokens, n] bf16, y [tokens, rows] bf16."""
    _need_cuda("x", x)
    tokens, n, ldx = _rows_ld("x", x)
    rows = codes.shape[0]
    if x.dtype != torch.bfloat16:
        raise ValueError("x must be bfloat16")
    if codes.dtype != torch.uint8 or scales.dtype != torch.float16:
        raise ValueError("codes must be uint8 and scales float16")
    if codes.shape != (rows, n * bits // 8) or scales.shape != (rows, n // group):
        raise ValueError("codes / scales shape mismatch")
    if not (codes.is_contiguous() and scales.is_contiguous()):
        raise ValueError("codes and scales must be contiguous")
    if codes.device != x.device or scales.device != x.device:
        raise ValueError("x, codes and scales must be on one device")
    if out is None:
        out = torch.empty((tokens, rows), dtype=torch.bfloat16, device=x.device)
    _need_cuda("out", out)
    t2, r2, ldy = _rows_ld("out", out)
    if (t2, r2) != (tokens, rows) or out.dtype != torch.bfloat16:
        raise ValueError("out must be bfloat16 [tokens, rows]")
    with torch.cuda.device(x.device):
        _check("rht_lowbit_gemv", _lib.rht_lowbit_gemv(
            _ptr(x), tokens, ldx, _ptr(codes), _ptr(scales), rows, n, _sign_ptr(signs, n, x.device),
            bits, group, _ptr(out), ldy, _stream(x)))
    return out


def qwha_forward_plan(tokens, d_in, row_ptr, d_out, nnz, out=None):
    """The forward's per-chunk bookkeeping for a fixed support (row_ptr), as
    a uint8 device tensor to pass as `plan` to qwha_adapter_forward (built on
    row_ptr's stream; valid for this token count and device).  `out`: a
    contiguous uint8 buffer of at least qwha_forward_plan_bytes to reuse."""
    _need_cuda("row_ptr", row_ptr)
    if row_ptr.dtype != torch.int32 or not row_ptr.is_contiguous() or row_ptr.numel() != d_out + 1:
        raise ValueError("row_ptr must be contiguous int32 with d_out + 1 entries")
    with torch.cuda.device(row_ptr.device):
        nb = _lib.qwha_forward_plan_bytes(tokens, d_in, d_out, nnz)
        if nb < 0:
            raise ValueError("invalid sizes for a forward plan")
        if out is None:
            plan = torch.empty(max(int(nb), 256), dtype=torch.uint8, device=row_ptr.device)
        else:
            _need_cuda("out", out)
            if out.dtype != torch.uint8 or not out.is_contiguous() or out.numel() < nb:
                raise ValueError("out must be a contiguous uint8 buffer of qwha_forward_plan_bytes or more")
            plan = out
        _check("qwha_forward_plan", _lib.qwha_forward_plan(
            tokens, d_in, _ptr(row_ptr), d_out, nnz, _ptr(plan), plan.numel(), _stream(row_ptr)))
    return plan


def qwha_adapter_forward(x, row_ptr, col_idx, vals, d_out, out=None, plan=None):
    """y = (x Hn) F^T with F [d_out x d_in] in CSR (int32 row_ptr / col_idx);
    `plan` from qwha_forward_plan skips the per-chunk bookkeeping."""
    _need_cuda("x", x)
    tokens, d_in, ldx = _rows_ld("x", x)
    for nm, t in (("row_ptr", row_ptr), ("col_idx", col_idx), ("vals", vals)):
        _need_cuda(nm, t)
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    if row_ptr.dtype != torch.int32 or col_idx.dtype != torch.int32:
        raise ValueError("row_ptr and col_idx must be int32")
    if row_ptr.numel() != d_out + 1:
        raise ValueError("row_ptr must have d_out + 1 entries")
    nnz = col_idx.numel()
    if vals.numel() != nnz:
        raise ValueError("vals and col_idx must have the same length")
    if out is None:
        # rows of 16 bytes or more need a 16-byte row stride: pad the storage to a multiple of 8
        width = d_out if d_out < 8 else -(-d_out // 8) * 8
        out = torch.empty((tokens, width), dtype=x.dtype, device=x.device)[:, :d_out]
    r2, n2, ldy = _rows_ld("out", out)
    if (r2, n2) != (tokens, d_out):
        raise ValueError("out shape mismatch")
    with torch.cuda.device(x.device):
        if plan is None:
            _check("qwha_adapter_forward", _lib.qwha_adapter_forward(
                _ptr(x), _DT[x.dtype], tokens, d_in, ldx, _ptr(row_ptr), _ptr(col_idx), _ptr(vals),
                _DT[vals.dtype], d_out, nnz, _ptr(out), _DT[out.dtype], ldy, _stream(x)))
        else:
            _need_cuda("plan", plan)
            if plan.dtype != torch.uint8 or not plan.is_contiguous():
                raise ValueError("plan must be a contiguous uint8 tensor from qwha_forward_plan")
            _check("qwha_adapter_forward_planned", _lib.qwha_adapter_forward_planned(
                _ptr(x), _DT[x.dtype], tokens, d_in, ldx, _ptr(row_ptr), _ptr(col_idx), _ptr(vals),
                _DT[vals.dtype], d_out, nnz, _ptr(plan), plan.numel(), _ptr(out), _DT[out.dtype], ldy,
                _stream(x)))
    return out


def harp_rotate(x, blocks, radices=(16, 16, 16), signs=None, precondition=True, out=None):
    """y = stages(Hn S x) (precondition) or stages(x); blocks float32 or float16, stage-major."""
    _need_cuda("x", x)
    _need_cuda("blocks", blocks)
    tokens, d, ldx = _rows_ld("x", x)
    if blocks.dtype not in (torch.float32, torch.float16) or not blocks.is_contiguous():
        raise ValueError("blocks must be contiguous float32 or float16")
    rad = (ctypes.c_int32 * len(radices))(*[int(b) for b in radices])
    if out is None:
        out = torch.empty_like(x)
    r2, d2, ldy = _rows_ld("out", out)
    if (r2, d2) != (tokens, d) or out.dtype != x.dtype:
        raise ValueError("out shape or dtype mismatch")
    with torch.cuda.device(x.device):
        _check("harp_rotate", _lib.harp_rotate(
            _ptr(x), _ptr(out), _DT[x.dtype], tokens, d, ldx, ldy, _sign_ptr(signs, d, x.device),
            int(bool(precondition)), rad, len(radices), _ptr(blocks), _DT[blocks.dtype], _stream(x)))
    return out


def _csr_dev(**ts):
    for nm, t in ts.items():
        _need_cuda(nm, t)
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")


def qwha_csr_transpose(row_ptr, col_idx, d_in):
    """CSR of F^T from the CSR of F (host helper; numpy int32 arrays in and out).
    Returns (t_row_ptr [d_in + 1], t_col_idx [nnz], t_perm [nnz])."""
    import numpy as np
    rp = np.ascontiguousarray(row_ptr, dtype=np.int32)
    ci = np.ascontiguousarray(col_idx, dtype=np.int32)
    d_out, nnz = rp.size - 1, ci.size
    t_rp = np.empty(d_in + 1, np.int32)
    t_ci = np.empty(max(nnz, 1), np.int32)
    t_pm = np.empty(max(nnz, 1), np.int32)
    _check("qwha_csr_transpose", _lib.qwha_csr_transpose(
        rp.ctypes.data_as(_vp), ci.ctypes.data_as(_vp), d_out, d_in, nnz, t_rp.ctypes.data_as(_vp),
        t_ci.ctypes.data_as(_vp), t_pm.ctypes.data_as(_vp)))
    return t_rp, t_ci[:nnz], t_pm[:nnz]


def qwha_permute_values(vals, perm, out=None):
    """out[j] = vals[perm[j]] on the device (F's values in F^T's entry order)."""
    _csr_dev(vals=vals, perm=perm)
    if perm.dtype != torch.int32:
        raise ValueError("perm must be int32")
    if out is None:
        out = torch.empty(perm.numel(), dtype=vals.dtype, device=vals.device)
    _csr_dev(out=out)
    if out.numel() != perm.numel() or out.dtype != vals.dtype:
        raise ValueError("out must match perm's length and vals' dtype")
    with torch.cuda.device(vals.device):
        _check("qwha_permute_values", _lib.qwha_permute_values(
            _ptr(vals), _DT[vals.dtype], _ptr(perm), perm.numel(), _ptr(out), _stream(vals)))
    return out


def qwha_adapter_backward_input(dy, t_row_ptr, t_col_idx, t_vals, d_in=4096, out=None):
    """dx = (dy F) Hn from the CSR of F^T (t_row_ptr [d_in + 1], t_col_idx, t_vals)."""
    _need_cuda("dy", dy)
    tokens, d_out, lddy = _rows_ld("dy", dy)
    _csr_dev(t_row_ptr=t_row_ptr, t_col_idx=t_col_idx, t_vals=t_vals)
    if t_row_ptr.dtype != torch.int32 or t_col_idx.dtype != torch.int32:
        raise ValueError("t_row_ptr and t_col_idx must be int32")
    if t_row_ptr.numel() != d_in + 1:
        raise ValueError("t_row_ptr must have d_in + 1 entries")
    nnz = t_col_idx.numel()
    if t_vals.numel() != nnz:
        raise ValueError("t_vals and t_col_idx must have the same length")
    if out is None:
        out = torch.empty((tokens, d_in), dtype=dy.dtype, device=dy.device)
    r2, n2, lddx = _rows_ld("out", out)
    if (r2, n2) != (tokens, d_in):
        raise ValueError("out shape mismatch")
    with torch.cuda.device(dy.device):
        _check("qwha_adapter_backward_input", _lib.qwha_adapter_backward_input(
            _ptr(dy), _DT[dy.dtype], tokens, d_out, lddy, _ptr(t_row_ptr), _ptr(t_col_idx), _ptr(t_vals),
            _DT[t_vals.dtype], d_in, nnz, _ptr(out), _DT[out.dtype], lddx, _stream(dy)))
    return out


def qwha_grad_values_workspace_bytes(tokens, d_in, nnz):
    return int(_lib.qwha_grad_values_workspace_bytes(tokens, d_in, nnz))


def qwha_adapter_grad_values(x, dy, row_ptr, col_idx, out=None, workspace=None):
    """dc[e] = sum_t dy[t, row(e)] (x Hn)[t, col_idx[e]] in float32, CSR entry order."""
    _need_cuda("x", x)
    _need_cuda("dy", dy)
    tokens, d_in, ldx = _rows_ld("x", x)
    t2, d_out, lddy = _rows_ld("dy", dy)
    if t2 != tokens:
        raise ValueError("x and dy must have the same number of tokens")
    _csr_dev(row_ptr=row_ptr, col_idx=col_idx)
    if row_ptr.dtype != torch.int32 or col_idx.dtype != torch.int32:
        raise ValueError("row_ptr and col_idx must be int32")
    if row_ptr.numel() != d_out + 1:
        raise ValueError("row_ptr must have d_out + 1 entries")
    nnz = col_idx.numel()
    if out is None:
        out = torch.empty(nnz, dtype=torch.float32, device=x.device)
    _csr_dev(out=out)
    if out.dtype != torch.float32 or out.numel() != nnz:
        raise ValueError("out must be float32 with nnz entries")
    need = qwha_grad_values_workspace_bytes(tokens, d_in, nnz)
    if need < 0:
        raise WhtqError("qwha_grad_values_workspace_bytes", 2)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    _csr_dev(workspace=workspace)
    wbytes = workspace.numel() * workspace.element_size()
    with torch.cuda.device(x.device):
        _check("qwha_adapter_grad_values", _lib.qwha_adapter_grad_values(
            _ptr(x), _ptr(dy), _DT[x.dtype], tokens, d_in, d_out, ldx, lddy, _ptr(row_ptr), _ptr(col_idx),
            nnz, _ptr(out), _ptr(workspace), wbytes, _stream(x)))
    return out


def qwha_adapter_grad_values_noalloc(x, dy, row_ptr, col_idx, out=None):
    """qwha_adapter_grad_values with the library's fixed per-GPU scratch array
    instead of a workspace (the library call allocates nothing; `out` is the
    caller's).  Calls that overlap on one GPU race."""
    _need_cuda("x", x)
    _need_cuda("dy", dy)
    tokens, d_in, ldx = _rows_ld("x", x)
    t2, d_out, lddy = _rows_ld("dy", dy)
    if t2 != tokens:
        raise ValueError("x and dy must have the same number of tokens")
    _csr_dev(row_ptr=row_ptr, col_idx=col_idx)
    if row_ptr.dtype != torch.int32 or col_idx.dtype != torch.int32:
        raise ValueError("row_ptr and col_idx must be int32")
    if row_ptr.numel() != d_out + 1:
        raise ValueError("row_ptr must have d_out + 1 entries")
    nnz = col_idx.numel()
    if out is None:
        out = torch.empty(nnz, dtype=torch.float32, device=x.device)
    _csr_dev(out=out)
    if out.dtype != torch.float32 or out.numel() != nnz:
        raise ValueError("out must be float32 with nnz entries")
    with torch.cuda.device(x.device):
        _check("qwha_adapter_grad_values_noalloc", _lib.qwha_adapter_grad_values_noalloc(
            _ptr(x), _ptr(dy), _DT[x.dtype], tokens, d_in, d_out, ldx, lddy, _ptr(row_ptr), _ptr(col_idx),
            nnz, _ptr(out), _stream(x)))
    return out


def harp_build_blocks(params, radices, d, scales=None, mixers=None, out=None, out_dtype=torch.float32):
    """Blocks Q(theta) G for harp_rotate from float32 parameters, or int8 codes
    with per-stage float32 scales; mixers float32 (stage-major) or None for Sylvester."""
    _need_cuda("params", params)
    if params.dtype not in (torch.float32, torch.int8) or not params.is_contiguous():
        raise ValueError("params must be contiguous float32 or int8")
    if params.dtype == torch.int8:
        _need_cuda("scales", scales)
        if scales.dtype != torch.float32 or scales.numel() != len(radices):
            raise ValueError("int8 params need float32 scales, one per stage")
    if mixers is not None:
        _need_cuda("mixers", mixers)
        if mixers.dtype != torch.float32 or not mixers.is_contiguous():
            raise ValueError("mixers must be contiguous float32")
    nblk = sum(d * int(b) for b in radices)
    if out is None:
        out = torch.empty(nblk, dtype=out_dtype, device=params.device)
    if out.numel() != nblk or not out.is_contiguous():
        raise ValueError("out must be contiguous with sum(d * b_t) elements")
    rad = (ctypes.c_int32 * len(radices))(*[int(b) for b in radices])
    with torch.cuda.device(params.device):
        _check("harp_build_blocks", _lib.harp_build_blocks(
            _ptr(params), _DT[params.dtype], _ptr(scales), d, rad, len(radices), _ptr(mixers), _ptr(out),
            _DT[out.dtype], _stream(params)))
    return out


# ------------------------------------------------------------ QWHA initialisation

QWHA_INIT_MAX_SUPPORT = 128


def _f32_rows(name, t):
    _need_cuda(name, t)
    if t.dtype != torch.float32:
        raise ValueError(f"{name} must be float32")
    return _rows_ld(name, t)


def qwha_init_error_coeffs(w, codes, scales, signs, bits, group, out=None):
    """F_dense = (W - Q(W)) Hn, float32 [rows, n], Q the RHT + RTN round trip of
    the stored codes / scales."""
    _need_cuda("w", w)
    rows, n, ldw = _rows_ld("w", w)
    if codes.shape != (rows, n * bits // 8) or scales.shape != (rows, n // group):
        raise ValueError("codes / scales shape mismatch")
    if not (codes.is_contiguous() and scales.is_contiguous()):
        raise ValueError("codes and scales must be contiguous")
    if out is None:
        out = torch.empty((rows, n), dtype=torch.float32, device=w.device)
    r2, n2, ldf = _f32_rows("out", out)
    if (r2, n2) != (rows, n):
        raise ValueError("out must be [rows, n]")
    with torch.cuda.device(w.device):
        _check("qwha_init_error_coeffs", _lib.qwha_init_error_coeffs(
            _ptr(w), _DT[w.dtype], rows, n, ldw, _ptr(codes), _ptr(scales), _sign_ptr(signs, n, w.device),
            bits, group, _ptr(out), ldf, _stream(w)))
    return out


def qwha_init_gram(x, g=None, accumulate=False, z=None):
    """G (+)= (x Hn)^T (x Hn), float32 [n, n]; z is the [tokens, n] float32
    workspace that receives x Hn.  Returns g."""
    _need_cuda("x", x)
    tokens, n, ldx = _rows_ld("x", x)
    if g is None:
        if accumulate:
            raise ValueError("accumulate needs g")
        g = torch.empty((n, n), dtype=torch.float32, device=x.device)
    if g.shape != (n, n) or g.dtype != torch.float32 or not g.is_contiguous():
        raise ValueError("g must be contiguous float32 [n, n]")
    if z is None:
        z = torch.empty((max(tokens, 1), n), dtype=torch.float32, device=x.device)
    if z.dtype != torch.float32 or not z.is_contiguous() or z.numel() < tokens * n:
        raise ValueError("z must be contiguous float32 with tokens * n elements")
    with torch.cuda.device(x.device):
        _check("qwha_init_gram", _lib.qwha_init_gram(
            _ptr(x), _DT[x.dtype], tokens, n, ldx, _ptr(z), _ptr(g), int(bool(accumulate)), _stream(x)))
    return g


def qwha_init_channel_errors(f, g, p=None, err=None):
    """(P = F G float32 [rows, n], err float32 [rows]) with err_o = sqrt(F[o] G F[o]^T)."""
    rows, n, ldf = _f32_rows("f", f)
    if g.shape != (n, n) or g.dtype != torch.float32 or not g.is_contiguous():
        raise ValueError("g must be contiguous float32 [n, n]")
    if p is None:
        p = torch.empty((rows, n), dtype=torch.float32, device=f.device)
    if err is None:
        err = torch.empty(rows, dtype=torch.float32, device=f.device)
    if p.shape != (rows, n) or p.dtype != torch.float32 or not p.is_contiguous():
        raise ValueError("p must be contiguous float32 [rows, n]")
    if err.shape != (rows,) or err.dtype != torch.float32:
        raise ValueError("err must be float32 [rows]")
    with torch.cuda.device(f.device):
        _check("qwha_init_channel_errors", _lib.qwha_init_channel_errors(
            _ptr(f), rows, n, ldf, _ptr(g), _ptr(p), _ptr(err), _stream(f)))
    return p, err


def qwha_init_allocate(err, n, total, floor, cap):
    """Host call: int32 row_ptr [rows + 1] of the per-channel budgets."""
    e = err.detach().to("cpu", torch.float32).contiguous()
    rows = e.numel()
    row_ptr = torch.empty(rows + 1, dtype=torch.int32)
    _check("qwha_init_allocate", _lib.qwha_init_allocate(
        _ptr(e), rows, n, int(total), int(floor), int(cap), _ptr(row_ptr)))
    return row_ptr


def qwha_init_select(f, row_ptr, col_idx=None):
    """int32 col_idx: per row the budget's largest |F| columns (ties to the lower
    column), ascending.  row_ptr: int32 device [rows + 1]."""
    rows, n, ldf = _f32_rows("f", f)
    _need_cuda("row_ptr", row_ptr)
    if row_ptr.dtype != torch.int32 or row_ptr.shape != (rows + 1,) or not row_ptr.is_contiguous():
        raise ValueError("row_ptr must be contiguous int32 [rows + 1]")
    # the size check reads row_ptr[-1] on the host, which a stream under
    # graph capture does not allow: there the caller's col_idx is trusted
    capturing = torch.cuda.is_current_stream_capturing()
    if col_idx is None:
        col_idx = torch.empty(int(row_ptr[-1].item()), dtype=torch.int32, device=f.device)
    _need_cuda("col_idx", col_idx)
    if col_idx.dtype != torch.int32 or not col_idx.is_contiguous():
        raise ValueError("col_idx must be contiguous int32")
    if not capturing and col_idx.numel() < int(row_ptr[-1].item()):
        raise ValueError("col_idx must hold row_ptr[-1] entries")
    with torch.cuda.device(f.device):
        _check("qwha_init_select", _lib.qwha_init_select(
            _ptr(f), rows, n, ldf, _ptr(row_ptr), _ptr(col_idx), _stream(f)))
    return col_idx


def qwha_init_refine(g, p, row_ptr, col_idx, vals=None):
    """float32 vals (CSR order) solving G[E][E] c = P[o][E] per row."""
    n = g.shape[0]
    if g.shape != (n, n) or g.dtype != torch.float32 or not g.is_contiguous():
        raise ValueError("g must be contiguous float32 [n, n]")
    rows = p.shape[0]
    if p.shape != (rows, n) or p.dtype != torch.float32 or not p.is_contiguous():
        raise ValueError("p must be contiguous float32 [rows, n]")
    for name, t in (("g", g), ("p", p), ("row_ptr", row_ptr), ("col_idx", col_idx)):
        _need_cuda(name, t)
    if row_ptr.dtype != torch.int32 or row_ptr.shape != (rows + 1,) or col_idx.dtype != torch.int32:
        raise ValueError("row_ptr / col_idx must be int32, row_ptr [rows + 1]")
    if not (row_ptr.is_contiguous() and col_idx.is_contiguous()):
        raise ValueError("row_ptr and col_idx must be contiguous")
    if vals is None:
        vals = torch.empty(col_idx.numel(), dtype=torch.float32, device=g.device)
    _need_cuda("vals", vals)
    if vals.dtype != torch.float32 or vals.numel() != col_idx.numel() or not vals.is_contiguous():
        raise ValueError("vals must be contiguous float32 with one entry per column index")
    if not torch.cuda.is_current_stream_capturing() and col_idx.numel() < int(row_ptr[-1].item()):
        raise ValueError("col_idx and vals must hold row_ptr[-1] entries")  # (not checked under graph capture)
    with torch.cuda.device(g.device):
        _check("qwha_init_refine", _lib.qwha_init_refine(
            _ptr(g), n, _ptr(p), rows, _ptr(row_ptr), _ptr(col_idx), _ptr(vals), _stream(g)))
    return vals


def qwha_initialize(w, codes, scales, signs, bits, group, x, total, floor, cap):
    """The whole initialisation of one layer through the calls above:
    returns (row_ptr int32, col_idx int32, vals float32) on w's device, plus
    the channel errors.  The budget allocation waits for the errors on the
    host (one device-to-host copy of rows floats)."""
    f = qwha_init_error_coeffs(w, codes, scales, signs, bits, group)
    g = qwha_init_gram(x)
    p, err = qwha_init_channel_errors(f, g)
    row_ptr = qwha_init_allocate(err, f.shape[1], total, floor, cap).to(w.device)
    col_idx = qwha_init_select(f, row_ptr)
    vals = qwha_init_refine(g, p, row_ptr, col_idx)
    return row_ptr, col_idx, vals, err


def stream_probe(src, dst):
    """Measurement helper: read all bytes of `src` and write all bytes of `dst`
    with a plain 16-byte streaming kernel (the "% achievable" reference)."""
    _need_cuda("src", src)
    _need_cuda("dst", dst)
    if not (src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("src and dst must be contiguous")
    ib, ob = src.numel() * src.element_size(), dst.numel() * dst.element_size()
    with torch.cuda.device(src.device):
        _check("whtq_stream_probe", _lib.whtq_stream_probe(_ptr(src), ib, _ptr(dst), ob, _stream(src)))
    return dst
