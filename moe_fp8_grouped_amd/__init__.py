"""Python binding of libmoefp8.so, the fp8 MoE grouped-matmul hot path for
MI355X (gfx950).

Argument marshalling only: each function forwards torch tensors' device
pointers, sizes and the current HIP stream to the C entry point of the same
name (declared in include/moe_fp8.h) and raises MoeError on a non-zero
status.  All arithmetic runs in the library's HIP kernels; there is no
fallback path.  The library is built in-tree by ``python -m
moe_fp8_grouped_amd.build``; importing this module without it raises.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoefp8.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "moe_fp8.h")

# constants mirrored from include/moe_fp8.h
MOE_OK, MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(6)
MOE_DTYPE_DEFAULT, MOE_BF16, MOE_F32, MOE_E4M3FN = -1, 0, 1, 2
MOE_SCALE_ROW_DYNAMIC, MOE_SCALE_TENSOR_DYNAMIC, MOE_SCALE_TENSOR_STATIC = 0, 1, 2
MOE_SCALE_TENSOR_FROM_ROW_AMAX = 3
MOE_ACT_NONE, MOE_ACT_SILU_MUL = 0, 1
(MOE_OP_QUANTIZE_ROWS, MOE_OP_SORT_BY_EXPERT, MOE_OP_GMM, MOE_OP_TGMM, MOE_OP_GATHER_REDUCE,
 MOE_OP_QUANTIZE_WEIGHTS) = range(6)
MOE_DEVERR_EXPERT_ID, MOE_DEVERR_GROUP_SIZE, MOE_DEVERR_ROWS = 1, 2, 4
MOE_SORT_NOALLOC_SCRATCH_BYTES = 2 << 20

# C signatures: name -> (restype, argtypes)
_P, _I, _I64, _F, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "moe_quantize_rows": (_I, [_P, _P, _I, _I64, _I64, _I, _F, _P, _P, _P, _P, _SZ, _P]),
    "moe_quantize_rows_strided": (_I, [_P, _P, _I64, _I, _I64, _I64, _I, _F, _P, _P, _P, _P, _SZ, _P]),
    "moe_quantize_weights": (_I, [_P, _I64, _I64, _I64, ctypes.c_int32, ctypes.c_int32, _I, _F, _I, _P, _P, _P]),
    "moe_quantize_rows_i8": (_I, [_P, _I64, _I64, _I, _F, _P, _P, _P, _P]),
    "moe_quantize_weights_i8": (_I, [_P, _I64, _I64, _I64, ctypes.c_int32, ctypes.c_int32, _I, _F, _I, _P, _P,
                                     _P]),
    "moe_sort_by_expert": (_I, [_P, _I64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P,
                                _I, _I64, _I64, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_sort_by_expert_noalloc": (_I, [_P, _I64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P,
                                        _P, _I, _I64, _I64, _P, _P, _P, _P, _P, _P, _P]),
    "moe_quantize_sort_by_expert": (_I, [_P, _I64, _I64, _I, _F, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_int32, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_gmm_fp8": (_I, [_P, _P, _I, _P, _P, ctypes.c_int32, ctypes.c_int32, _I, _P, ctypes.c_int32, ctypes.c_int32,
                         ctypes.c_int32, _I64, _I64, _I64, _I, _P, _P, _SZ, _P]),
    "moe_gmm_i8": (_I, [_P, _P, _I, _P, _P, ctypes.c_int32, ctypes.c_int32, _I, _P, ctypes.c_int32, ctypes.c_int32,
                        ctypes.c_int32, _I64, _I64, _I64, _I, _P, _P, _SZ, _P]),
    "moe_tgmm_fp8": (_I, [_P, _P, ctypes.c_int32, _P, _P, ctypes.c_int32, _P, ctypes.c_int32, ctypes.c_int32,
                          ctypes.c_int32, _I64, _I64, _I64, _I, _P, _P, _SZ, _P]),
    "moe_sort_gather_rows": (_I, [_P, _P, _I, _P, _I64, ctypes.c_int32, _I64, _I64, _P, _P, _P, _SZ, _P]),
    "moe_tgmm_xt_cols": (_I, [_I64, ctypes.c_int32, _P]),
    "moe_sort_gather_transposed": (_I, [_P, _I, _F, _I64, ctypes.c_int32, _I64, _P, _P, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, _I64, _P, _P, _P, _SZ, _P]),
    "moe_tgmm_fp8_xt": (_I, [_P, _P, ctypes.c_int32, _P, _P, ctypes.c_int32, _P, ctypes.c_int32, ctypes.c_int32,
                             ctypes.c_int32, _I64, _I64, _I64, _I, _P, _P, _SZ, _P]),
    "moe_gather_reduce": (_I, [_P, _I, _P, _P, _I64, ctypes.c_int32, _I64, _I, _P, _P]),
    "moe_gather_reduce_backward": (_I, [_P, _P, _P, _P, _I64, ctypes.c_int32, _I64, _P, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_int32, _I64, _P, _P, _P, _P, _P, _P]),
    "moe_silu_mul_backward": (_I, [_P, _P, _I64, _P, _I64, _I64, _P, _P, _I64, _P]),
    "moe_workspace_bytes": (_I, [_I, _I64, _I64, _I64, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]),
    "moe_debug_check": (_I, [_P, _P, ctypes.POINTER(ctypes.c_int32)]),
    "moe_status_string": (ctypes.c_char_p, [_I]),
    "moe_version": (_I, []),
}


class MoeError(RuntimeError):
    def __init__(self, fn, status, text):
        super().__init__(f"{fn} failed with status {status}: {text}")
        self.status = status


_lib = None


def load_library(path=LIB_PATH):
    """dlopen libmoefp8.so and attach the C signatures (no GPU needed)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libmoefp8.so is not built ({path}); run python -m moe_fp8_grouped_amd.build")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor or None")
    if not t.is_cuda:
        raise ValueError("tensor arguments must live in GPU memory")
    if not t.is_contiguous():
        raise ValueError("tensor arguments must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _call(name, *args):
    st = getattr(load_library(), name)(*args)
    if st != MOE_OK:
        raise MoeError(name, st, status_string(st))
    return st


def status_string(status):
    return load_library().moe_status_string(status).decode()


def version():
    return load_library().moe_version()


def workspace_bytes(op, d0=0, d1=0, d2=0, E=1):
    out = ctypes.c_size_t(0)
    st = load_library().moe_workspace_bytes(op, d0, d1, d2, E, ctypes.byref(out))
    if st != MOE_OK:
        raise MoeError("moe_workspace_bytes", st, status_string(st))
    return out.value


def workspace(op, d0=0, d1=0, d2=0, E=1, device="cuda"):
    """A zeroed workspace tensor (uint8) of the size the library asks for."""
    return torch.zeros(workspace_bytes(op, d0, d1, d2, E), dtype=torch.uint8, device=device)


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def moe_quantize_rows(x, x_up, act, R, C, scale_mode, static_scale, q, scale, row_amax=None, ws=None, stream=None):
    return _call("moe_quantize_rows", _ptr(x), _ptr(x_up), act, R, C, scale_mode, float(static_scale), _ptr(q),
                 _ptr(scale), _ptr(row_amax), _ptr(ws), _nbytes(ws), _stream(stream))


def _ptr_rows(t, ld):
    """Device pointer of a 2-D view whose rows are ``ld`` elements apart (unit inner stride)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError("tensor arguments must be torch tensors in GPU memory")
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1) or (t.shape[0] > 1 and t.stride(0) != ld):
        raise ValueError("expected a 2-D view with rows %d elements apart" % ld)
    return t.data_ptr()


def moe_quantize_rows_strided(x, x_up, ldx, act, R, C, scale_mode, static_scale, q, scale, row_amax=None, ws=None,
                              stream=None):
    return _call("moe_quantize_rows_strided", _ptr_rows(x, ldx), _ptr_rows(x_up, ldx), ldx, act, R, C, scale_mode,
                 float(static_scale), _ptr(q), _ptr(scale), _ptr(row_amax), _ptr(ws), _nbytes(ws), _stream(stream))


def moe_quantize_weights(w, E, K, N, kb, nb, scale_mode, static_scale, transpose_out, q, scale, stream=None):
    return _call("moe_quantize_weights", _ptr(w), E, K, N, kb, nb, scale_mode, float(static_scale),
                 transpose_out, _ptr(q), _ptr(scale), _stream(stream))


def moe_quantize_rows_i8(x, R, C, scale_mode, static_scale, q, scale, row_amax=None, stream=None):
    return _call("moe_quantize_rows_i8", _ptr(x), R, C, scale_mode, float(static_scale), _ptr(q), _ptr(scale),
                 _ptr(row_amax), _stream(stream))


def moe_quantize_weights_i8(w, E, K, N, kb, nb, scale_mode, static_scale, transpose_out, q, scale, stream=None):
    return _call("moe_quantize_weights_i8", _ptr(w), E, K, N, kb, nb, scale_mode, float(static_scale),
                 transpose_out, _ptr(q), _ptr(scale), _stream(stream))


def moe_sort_by_expert(expert_ids, T, k, E, group_offset, num_local_experts, xq, xscale, xscale_mode, H, M_cap,
                       perm, inv_pos, group_sizes, xs, ss, ws, stream=None):
    return _call("moe_sort_by_expert", _ptr(expert_ids), T, k, E, group_offset, num_local_experts, _ptr(xq),
                 _ptr(xscale), xscale_mode, H, M_cap, _ptr(perm), _ptr(inv_pos), _ptr(group_sizes), _ptr(xs),
                 _ptr(ss), _ptr(ws), _nbytes(ws), _stream(stream))


def moe_sort_by_expert_noalloc(expert_ids, T, k, E, group_offset, num_local_experts, xq, xscale, xscale_mode, H,
                               M_cap, perm, inv_pos, group_sizes, xs, ss, device_error=None, stream=None):
    return _call("moe_sort_by_expert_noalloc", _ptr(expert_ids), T, k, E, group_offset, num_local_experts, _ptr(xq),
                 _ptr(xscale), xscale_mode, H, M_cap, _ptr(perm), _ptr(inv_pos), _ptr(group_sizes), _ptr(xs),
                 _ptr(ss), _ptr(device_error), _stream(stream))


def moe_quantize_sort_by_expert(x, T, H, scale_mode, static_scale, expert_ids, k, E, group_offset, num_local_experts,
                                M_cap, perm, inv_pos, group_sizes, xs, ss, scale=None, ws=None, stream=None,
                                row_amax=None):
    return _call("moe_quantize_sort_by_expert", _ptr(x), T, H, scale_mode, float(static_scale), _ptr(expert_ids), k,
                 E, group_offset, num_local_experts, M_cap, _ptr(perm), _ptr(inv_pos), _ptr(group_sizes), _ptr(xs),
                 _ptr(ss), _ptr(scale), _ptr(row_amax), _ptr(ws), _nbytes(ws), _stream(stream))


def moe_gmm_fp8(lhs, lhs_scale, lhs_scale_mode, rhs, rhs_scale, Kb, Nb, transpose_rhs, group_sizes, E,
                group_offset, num_local_experts, M, K, N, out_dtype, out, ws, stream=None):
    return _call("moe_gmm_fp8", _ptr(lhs), _ptr(lhs_scale), lhs_scale_mode, _ptr(rhs), _ptr(rhs_scale), Kb, Nb,
                 transpose_rhs, _ptr(group_sizes), E, group_offset, num_local_experts, M, K, N, out_dtype,
                 _ptr(out), _ptr(ws), _nbytes(ws), _stream(stream))


def moe_gmm_i8(lhs, lhs_scale, lhs_scale_mode, rhs, rhs_scale, Kb, Nb, transpose_rhs, group_sizes, E,
               group_offset, num_local_experts, M, K, N, out_dtype, out, ws, stream=None):
    return _call("moe_gmm_i8", _ptr(lhs), _ptr(lhs_scale), lhs_scale_mode, _ptr(rhs), _ptr(rhs_scale), Kb, Nb,
                 transpose_rhs, _ptr(group_sizes), E, group_offset, num_local_experts, M, K, N, out_dtype,
                 _ptr(out), _ptr(ws), _nbytes(ws), _stream(stream))


def moe_tgmm_fp8(lhs, lhs_scale, lhs_scale_len, rhs, rhs_scale, rhs_scale_len, group_sizes, E, group_offset,
                 num_local_experts, M, K, N, out_dtype, out, ws, stream=None):
    return _call("moe_tgmm_fp8", _ptr(lhs), _ptr(lhs_scale), lhs_scale_len, _ptr(rhs), _ptr(rhs_scale),
                 rhs_scale_len, _ptr(group_sizes), E, group_offset, num_local_experts, M, K, N, out_dtype,
                 _ptr(out), _ptr(ws), _nbytes(ws), _stream(stream))


def moe_sort_gather_rows(xq, xscale, xscale_mode, inv_pos, T, k, H, M_cap, xs, ss, ws, stream=None):
    return _call("moe_sort_gather_rows", _ptr(xq), _ptr(xscale), xscale_mode, _ptr(inv_pos), T, k, H, M_cap,
                 _ptr(xs), _ptr(ss), _ptr(ws), _nbytes(ws), _stream(stream))


def tgmm_xt_cols(M, E):
    out = ctypes.c_int64(0)
    st = load_library().moe_tgmm_xt_cols(M, E, ctypes.byref(out))
    if st != MOE_OK:
        raise MoeError("moe_tgmm_xt_cols", st, status_string(st))
    return out.value


def moe_sort_gather_transposed(x, x_dtype, static_scale, T, k, H, perm, group_sizes, E, group_offset,
                               num_local_experts, M, xt, scale_out, ws, stream=None):
    return _call("moe_sort_gather_transposed", _ptr(x), x_dtype, float(static_scale), T, k, H, _ptr(perm),
                 _ptr(group_sizes), E, group_offset, num_local_experts, M, _ptr(xt), _ptr(scale_out), _ptr(ws),
                 _nbytes(ws), _stream(stream))


def moe_tgmm_fp8_xt(xt, lhs_scale, lhs_scale_len, rhs, rhs_scale, rhs_scale_len, group_sizes, E, group_offset,
                    num_local_experts, M, K, N, out_dtype, out, ws, stream=None):
    return _call("moe_tgmm_fp8_xt", _ptr(xt), _ptr(lhs_scale), lhs_scale_len, _ptr(rhs), _ptr(rhs_scale),
                 rhs_scale_len, _ptr(group_sizes), E, group_offset, num_local_experts, M, K, N, out_dtype,
                 _ptr(out), _ptr(ws), _nbytes(ws), _stream(stream))


def moe_gather_reduce(y, y_dtype, inv_pos, topk_weights, T, k, N, out_dtype, out, stream=None):
    return _call("moe_gather_reduce", _ptr(y), y_dtype, _ptr(inv_pos), _ptr(topk_weights), T, k, N, out_dtype,
                 _ptr(out), _stream(stream))


def moe_gather_reduce_backward(dout, y, inv_pos, topk_weights, T, k, N, group_sizes, E, group_offset,
                               num_local_experts, M_cap, dy, dw, dy_q=None, dy_scale=None, dy_amax=None, stream=None):
    return _call("moe_gather_reduce_backward", _ptr(dout), _ptr(y), _ptr(inv_pos), _ptr(topk_weights), T, k, N,
                 _ptr(group_sizes), E, group_offset, num_local_experts, M_cap, _ptr(dy), _ptr(dw), _ptr(dy_q),
                 _ptr(dy_scale), _ptr(dy_amax), _stream(stream))


def moe_silu_mul_backward(a, b, lda, dh, R, C, da, db, ldo, stream=None):
    """a, b, da, db may be column slices of wider buffers (row strides lda, ldo)."""
    return _call("moe_silu_mul_backward", _ptr_rows(a, lda), _ptr_rows(b, lda), lda, _ptr(dh), R, C,
                 _ptr_rows(da, ldo), _ptr_rows(db, ldo), ldo, _stream(stream))


def moe_debug_check(ws, stream=None):
    """Synchronise and return the sticky device-error word of a workspace."""
    err = ctypes.c_int32(0)
    st = load_library().moe_debug_check(_ptr(ws), _stream(stream), ctypes.byref(err))
    if st != MOE_OK:
        raise MoeError("moe_debug_check", st, status_string(st))
    return err.value
