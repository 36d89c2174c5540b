"""The C-ABI library without a GPU: it loads, exports every function that
include/*.h declares, and its host-side validation rejects bad arguments
before any launch (only paths that return before touching the device are
exercised here)."""

import ctypes
import glob
import os
import re

import pytest

import moe_fp8_grouped_amd as m

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for mt in re.finditer(r"^\s*(?:const\s+)?\w+\s*\*?\s*(moe_\w+)\s*\(", text, flags=re.M):
            names.add(mt.group(1))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(m.LIB_PATH):
        pytest.skip("libmoefp8.so not built")
    return m.load_library()


def test_header_declares_the_path_calls():
    names = _declared_functions()
    for fn in ["moe_quantize_rows", "moe_quantize_rows_strided", "moe_sort_by_expert", "moe_sort_by_expert_noalloc", "moe_quantize_sort_by_expert", "moe_gmm_fp8", "moe_tgmm_fp8", "moe_gather_reduce",
               "moe_gather_reduce_backward", "moe_silu_mul_backward", "moe_quantize_weights", "moe_quantize_rows_i8",
               "moe_quantize_weights_i8", "moe_gmm_i8", "moe_tgmm_xt_cols", "moe_sort_gather_transposed", "moe_sort_gather_rows",
               "moe_tgmm_fp8_xt", "moe_workspace_bytes", "moe_debug_check", "moe_status_string", "moe_version"]:
        assert fn in names


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(m.LIB_PATH)
    for fn in _declared_functions():
        assert hasattr(raw, fn), fn
    assert set(_declared_functions()) == set(m.SIGNATURES)


def test_status_strings_and_version(lib):
    assert m.status_string(m.MOE_OK) == "ok"
    assert "workspace" in m.status_string(m.MOE_ERR_WORKSPACE)
    assert m.status_string(99) == "unknown status"
    assert m.version() >= 100


def test_workspace_sizes(lib):
    b = m.workspace_bytes(m.MOE_OP_QUANTIZE_ROWS, 100, 64, m.MOE_SCALE_ROW_DYNAMIC)
    assert b >= 256 and b % 256 == 0
    bt = m.workspace_bytes(m.MOE_OP_QUANTIZE_ROWS, 100, 64, m.MOE_SCALE_TENSOR_DYNAMIC)
    assert bt > b
    s1 = m.workspace_bytes(m.MOE_OP_SORT_BY_EXPERT, 32768, 0, 0, 64)
    s2 = m.workspace_bytes(m.MOE_OP_SORT_BY_EXPERT, 65536, 0, 0, 256)
    assert s2 > s1 >= 256 and s1 % 256 == 0
    assert m.workspace_bytes(m.MOE_OP_GMM, 32768, 2048, 768, 64) >= 256
    with pytest.raises(m.MoeError):
        m.workspace_bytes(77)
    with pytest.raises(m.MoeError):
        m.workspace_bytes(m.MOE_OP_SORT_BY_EXPERT, 10, 0, 0, 2000)


def _c(lib, name, *args):
    return getattr(lib, name)(*args)


def test_quantize_rows_validation(lib):
    f = lambda *a: _c(lib, "moe_quantize_rows", *a)
    one = 1  # non-null dummy pointer: never dereferenced on these paths
    assert f(one, None, 0, 4, 24, 0, 0.0, one, one, None, None, 0, None) == m.MOE_ERR_SHAPE      # C % 16
    assert f(one, None, 0, -1, 32, 0, 0.0, one, one, None, None, 0, None) == m.MOE_ERR_SHAPE
    assert f(one, None, 5, 4, 32, 0, 0.0, one, one, None, None, 0, None) == m.MOE_ERR_UNSUPPORTED
    assert f(one, None, 0, 4, 32, 9, 0.0, one, one, None, None, 0, None) == m.MOE_ERR_UNSUPPORTED
    assert f(one, None, 0, 4, 32, 2, -1.0, one, one, None, None, 0, None) == m.MOE_ERR_SHAPE     # bad static
    assert f(None, None, 0, 4, 32, 0, 0.0, one, one, None, None, 0, None) == m.MOE_ERR_NULL
    assert f(one, None, 1, 4, 32, 0, 0.0, one, one, None, None, 0, None) == m.MOE_ERR_NULL       # silu w/o up
    assert f(one, one, 0, 4, 32, 0, 0.0, one, one, None, None, 0, None) == m.MOE_ERR_UNSUPPORTED # up w/o silu
    assert f(one, None, 0, 4, 32, 1, 0.0, one, one, None, None, 0, None) == m.MOE_ERR_WORKSPACE
    assert f(one, None, 0, 4, 32, 1, 0.0, one, one, None, one, 16, None) == m.MOE_ERR_WORKSPACE


def test_quantize_rows_tensor_from_row_amax_validation(lib):
    f = lambda *a: _c(lib, "moe_quantize_rows", *a)
    one = 1
    mode = m.MOE_SCALE_TENSOR_FROM_ROW_AMAX
    assert f(one, None, 0, 4, 32, mode, 0.0, one, one, None, None, 0, None) == m.MOE_ERR_NULL     # row maxima needed
    assert f(one, None, 0, 4, 32, 4, 0.0, one, one, one, None, 0, None) == m.MOE_ERR_UNSUPPORTED  # unknown mode


def test_quantize_rows_strided_validation(lib):
    f = lambda *a: _c(lib, "moe_quantize_rows_strided", *a)
    al = 4096   # 16-byte aligned dummy pointer: never dereferenced on these paths
    assert f(al, None, 16, 0, 4, 32, 0, 0.0, al, al, None, None, 0, None) == m.MOE_ERR_SHAPE    # ldx < C
    assert f(al, None, 36, 0, 4, 32, 0, 0.0, al, al, None, None, 0, None) == m.MOE_ERR_SHAPE    # ldx % 8
    assert f(al + 8, None, 64, 0, 4, 32, 0, 0.0, al, al, None, None, 0, None) == m.MOE_ERR_SHAPE  # x misaligned
    assert f(al, al + 2, 64, 1, 4, 32, 0, 0.0, al, al, None, None, 0, None) == m.MOE_ERR_SHAPE  # x_up misaligned
    assert f(al, None, 64, 1, 4, 32, 0, 0.0, al, al, None, None, 0, None) == m.MOE_ERR_NULL     # silu w/o up
    assert f(al, None, 64, 0, 4, 24, 0, 0.0, al, al, None, None, 0, None) == m.MOE_ERR_SHAPE    # C % 16


def test_sort_validation(lib):
    f = lambda *a: _c(lib, "moe_sort_by_expert", *a)
    one = 1
    def call(T=4, k=2, E=8, g0=0, El=8, xq=None, xscale=None, mode=0, H=0, M_cap=8, perm=one, inv=one,
             gs=one, xs=None, ss=None, ws=one, wsb=1 << 20):
        return f(one, T, k, E, g0, El, xq, xscale, mode, H, M_cap, perm, inv, gs, xs, ss, ws, wsb, None)
    assert call(E=0) == m.MOE_ERR_SHAPE
    assert call(E=2000) == m.MOE_ERR_SHAPE
    assert call(k=0) == m.MOE_ERR_SHAPE
    assert call(g0=4, El=5) == m.MOE_ERR_SHAPE
    assert call(mode=7) == m.MOE_ERR_UNSUPPORTED
    assert call(xq=one, H=24, xs=one) == m.MOE_ERR_SHAPE
    assert call(gs=None) == m.MOE_ERR_NULL
    assert call(xq=one, H=32, xs=None) == m.MOE_ERR_NULL
    assert call(wsb=16) == m.MOE_ERR_WORKSPACE


def test_sort_noalloc_validation(lib):
    f = lambda *a: _c(lib, "moe_sort_by_expert_noalloc", *a)
    one = 1
    def call(T=4, k=2, E=8, g0=0, El=8, xq=None, xscale=None, mode=0, H=0, M_cap=8, gs=one):
        return f(one, T, k, E, g0, El, xq, xscale, mode, H, M_cap, one, one, gs, None, None, None, None)
    assert call(E=0) == m.MOE_ERR_SHAPE
    assert call(g0=4, El=5) == m.MOE_ERR_SHAPE
    assert call(mode=7) == m.MOE_ERR_UNSUPPORTED
    assert call(gs=None) == m.MOE_ERR_NULL
    # the largest sizes the library's scratch array holds, and one slot more (no launch either way here)
    assert call(T=261633, k=1, E=1024, El=1024) == m.MOE_ERR_WORKSPACE
    assert call(T=1043969, k=1, E=256, El=256) == m.MOE_ERR_WORKSPACE
    assert m.workspace_bytes(m.MOE_OP_SORT_BY_EXPERT, 261632, 0, 0, 1024) <= m.MOE_SORT_NOALLOC_SCRATCH_BYTES


def test_quantize_sort_validation(lib):
    f = lambda *a: _c(lib, "moe_quantize_sort_by_expert", *a)
    al = 4096   # 16-byte aligned dummy pointer: never dereferenced on these paths
    def call(x=al, T=4, H=32, mode=0, static=0.0, k=2, E=8, g0=0, El=8, M_cap=8, xs=al, ss=al, ws=al, wsb=1 << 20,
             scale=None, amax=None):
        return f(x, T, H, mode, static, al, k, E, g0, El, M_cap, al, al, al, xs, ss, scale, amax, ws, wsb, None)
    assert call(H=24) == m.MOE_ERR_SHAPE
    assert call(mode=1) == m.MOE_ERR_UNSUPPORTED          # tensor-dynamic needs the whole tensor first
    assert call(mode=2, static=-1.0) == m.MOE_ERR_SHAPE
    assert call(x=None) == m.MOE_ERR_NULL
    assert call(xs=None) == m.MOE_ERR_NULL
    assert call(ss=None) == m.MOE_ERR_NULL                # row mode needs the row scales
    assert call(mode=3, scale=al) == m.MOE_ERR_NULL       # the tokens' maxima are needed
    assert call(mode=3, amax=al) == m.MOE_ERR_NULL        # and somewhere to put the tensor scale
    assert call(x=al + 8) == m.MOE_ERR_SHAPE              # misaligned rows
    assert call(wsb=16) == m.MOE_ERR_WORKSPACE
    assert call(E=0) == m.MOE_ERR_SHAPE


def test_gmm_validation(lib):
    f = lambda *a: _c(lib, "moe_gmm_fp8", *a)
    one = 1
    def call(M=256, K=256, N=256, Kb=1, Nb=256, tr=1, E=8, g0=0, El=8, mode=0, od=0, ws=one, wsb=256,
             lhs=one, out=one):
        return f(lhs, one, mode, one, one, Kb, Nb, tr, one, E, g0, El, M, K, N, od, out, ws, wsb, None)
    assert call(K=200) == m.MOE_ERR_SHAPE                    # not a multiple of 16
    assert call(N=100) == m.MOE_ERR_SHAPE
    assert call(K=144, Kb=2) == m.MOE_ERR_UNSUPPORTED        # 72-row K blocks
    assert call(Kb=3) == m.MOE_ERR_SHAPE
    assert call(K=384, Kb=2) == m.MOE_ERR_UNSUPPORTED        # 192-row K blocks
    assert call(Nb=3) == m.MOE_ERR_SHAPE
    assert call(tr=2) == m.MOE_ERR_UNSUPPORTED
    assert call(mode=5) == m.MOE_ERR_UNSUPPORTED
    assert call(od=7) == m.MOE_ERR_UNSUPPORTED
    assert call(g0=1, El=8) == m.MOE_ERR_SHAPE
    assert call(E=0) == m.MOE_ERR_SHAPE
    assert call(lhs=None) == m.MOE_ERR_NULL
    assert call(ws=None) == m.MOE_ERR_WORKSPACE
    assert call(wsb=8) == m.MOE_ERR_WORKSPACE
    assert call(M=0, out=None) == m.MOE_OK                  # nothing to do, no launch


def test_tgmm_and_gather_reduce_validation(lib):
    t = lambda *a: _c(lib, "moe_tgmm_fp8", *a)
    one = 1
    assert t(one, one, 1, one, one, 1, one, 8, 0, 8, 100, 200, 256, 1, one, one, 256, None) == m.MOE_ERR_SHAPE
    assert t(one, one, 1, one, one, 1, one, 8, 0, 8, 100, 256, 72, 1, one, one, 256, None) == m.MOE_ERR_SHAPE
    assert t(one, one, 3, one, one, 1, one, 8, 0, 8, 100, 256, 256, 1, one, one, 256, None) == m.MOE_ERR_UNSUPPORTED
    assert t(one, one, 1, one, one, 7, one, 8, 0, 8, 100, 256, 256, 1, one, one, 256, None) == m.MOE_ERR_UNSUPPORTED
    assert t(one, one, 1, one, one, 1, one, 8, 0, 0, 100, 256, 256, 1, one, one, 256, None) == m.MOE_OK  # no experts
    g = lambda *a: _c(lib, "moe_gather_reduce", *a)
    assert g(one, 0, one, one, 4, 2, 12, 0, one, None) == m.MOE_ERR_SHAPE          # N % 8
    assert g(one, 2, one, one, 4, 2, 16, 0, one, None) == m.MOE_ERR_UNSUPPORTED    # fp8 input
    assert g(one, 0, one, one, 4, 0, 16, 0, one, None) == m.MOE_ERR_SHAPE
    assert g(None, 0, one, one, 4, 2, 16, 0, one, None) == m.MOE_ERR_NULL
    assert g(None, 0, None, None, 0, 2, 16, 0, None, None) == m.MOE_OK             # T = 0


def test_transposed_gather_and_product_validation(lib):
    """The transposed row gather and the weight-gradient product on its layout: the column count, and every
    argument check that returns before a launch."""
    assert m.tgmm_xt_cols(1000, 8) == 256 * ((1000 + 128 * 8 + 255) // 256)
    assert m.tgmm_xt_cols(0, 1) == 256
    with pytest.raises(m.MoeError):
        m.tgmm_xt_cols(10, 0)
    one = 1
    g = lambda *a: _c(lib, "moe_sort_gather_transposed", *a)
    # x, x_dtype, static_scale, T, k, H, perm, group_sizes, E, g0, El, M, xt, scale_out, ws, ws_bytes, stream
    assert g(one, m.MOE_E4M3FN, 1.0, 8, 2, 384, one, one, 4, 0, 4, 16, one, None, one, 256, None) == m.MOE_ERR_UNSUPPORTED
    assert g(one, m.MOE_E4M3FN, 1.0, 8, 0, 512, one, one, 4, 0, 4, 16, one, None, one, 256, None) == m.MOE_ERR_SHAPE
    assert g(one, m.MOE_F32, 1.0, 8, 2, 512, one, one, 4, 0, 4, 16, one, None, one, 256, None) == m.MOE_ERR_UNSUPPORTED
    assert g(one, m.MOE_BF16, 0.0, 8, 2, 512, one, one, 4, 0, 4, 16, one, None, one, 256, None) == m.MOE_ERR_SHAPE
    assert g(one, m.MOE_E4M3FN, 1.0, 8, 2, 512, one, one, 4, 2, 4, 16, one, None, one, 256, None) == m.MOE_ERR_SHAPE
    assert g(one, m.MOE_E4M3FN, 1.0, 8, 2, 512, one, None, 4, 0, 4, 16, one, None, one, 256, None) == m.MOE_ERR_NULL
    assert g(one, m.MOE_E4M3FN, 1.0, 8, 2, 512, one, one, 4, 0, 4, 16, one, None, None, 0, None) == m.MOE_ERR_WORKSPACE
    assert g(one, m.MOE_E4M3FN, 1.0, 8, 2, 512, one, one, 4, 0, 0, 16, one, None, one, 256, None) == m.MOE_OK  # no experts
    t = lambda *a: _c(lib, "moe_tgmm_fp8_xt", *a)
    # xt, ls, ls_len, rhs, rs, rs_len, group_sizes, E, g0, El, M, K, N, out_dtype, out, ws, ws_bytes, stream
    assert t(one, one, 1, one, one, 1, one, 8, 0, 8, 100, 384, 256, 1, one, one, 1 << 20, None) == m.MOE_ERR_UNSUPPORTED
    assert t(one, one, 1, one, one, 1, one, 8, 0, 8, 100, 512, 200, 1, one, one, 1 << 20, None) == m.MOE_ERR_UNSUPPORTED
    assert t(one, one, 3, one, one, 1, one, 8, 0, 8, 100, 512, 256, 1, one, one, 1 << 20, None) == m.MOE_ERR_UNSUPPORTED
    assert t(one, one, 1, one, one, 1, one, 8, 0, 8, 100, 512, 256, 1, one, one, 256, None) == m.MOE_ERR_WORKSPACE
    assert t(one, one, 1, one, one, 1, one, 8, 0, 0, 100, 512, 256, 1, one, one, 256, None) == m.MOE_OK  # no experts


def test_sort_gather_rows_validation(lib):
    g = lambda *a: _c(lib, "moe_sort_gather_rows", *a)
    one = 1
    # xq, xscale, mode, inv_pos, T, k, H, M_cap, xs, ss, ws, ws_bytes, stream
    assert g(one, one, m.MOE_SCALE_TENSOR_STATIC, one, 8, 0, 64, 16, one, None, one, 256, None) == m.MOE_ERR_SHAPE
    assert g(one, one, m.MOE_SCALE_TENSOR_STATIC, one, 8, 2, 60, 16, one, None, one, 256, None) == m.MOE_ERR_SHAPE
    assert g(one, one, 9, one, 8, 2, 64, 16, one, None, one, 256, None) == m.MOE_ERR_UNSUPPORTED
    assert g(one, one, m.MOE_SCALE_TENSOR_STATIC, one, 8, 2, 64, 16, None, None, one, 256, None) == m.MOE_ERR_NULL
    assert g(None, one, m.MOE_SCALE_TENSOR_STATIC, one, 8, 2, 64, 16, one, None, one, 256, None) == m.MOE_ERR_NULL
    assert g(one, one, m.MOE_SCALE_TENSOR_STATIC, one, 8, 2, 64, 16, one, None, one, 8, None) == m.MOE_ERR_WORKSPACE
    assert g(None, None, m.MOE_SCALE_TENSOR_STATIC, None, 0, 2, 64, 0, one, None, one, 256, None) == m.MOE_OK


def test_gather_reduce_backward_validation(lib):
    g = lambda *a: _c(lib, "moe_gather_reduce_backward", *a)
    b = lambda *a: g(*a[:14], None, None, None, a[14])
    one = 1
    # dout, y, inv_pos, w, T, k, N, group_sizes, E, g0, El, M_cap, dy, dw, [dy_q, dy_scale, dy_amax,] stream
    assert b(one, one, one, one, 4, 2, 12, one, 8, 0, 8, 8, one, one, None) == m.MOE_ERR_SHAPE     # N % 8
    assert b(one, one, one, one, 4, 0, 16, one, 8, 0, 8, 8, one, one, None) == m.MOE_ERR_SHAPE     # k = 0
    assert b(one, one, one, one, 4, 2, 16, one, 8, 4, 8, 8, one, one, None) == m.MOE_ERR_SHAPE     # window > E
    assert b(one, one, one, one, 4, 2, 16, one, 8, 0, 8, -1, one, one, None) == m.MOE_ERR_SHAPE    # M_cap < 0
    assert b(None, one, one, one, 4, 2, 16, one, 8, 0, 8, 8, one, one, None) == m.MOE_ERR_NULL
    assert b(one, one, one, one, 4, 2, 16, None, 8, 0, 8, 8, one, one, None) == m.MOE_ERR_NULL
    assert b(one, None, one, one, 4, 2, 16, one, 8, 0, 8, 8, one, one, None) == m.MOE_ERR_NULL
    assert b(None, None, None, None, 0, 2, 16, None, 8, 0, 8, 0, None, None, None) == m.MOE_OK  # nothing to do
    # the fused row quantization: all three outputs or none, rows of at most 8192 elements
    assert g(one, one, one, one, 4, 2, 16, one, 8, 0, 8, 8, one, one, one, None, one, None) == m.MOE_ERR_NULL
    assert g(one, one, one, one, 4, 2, 8200, one, 8, 0, 8, 8, one, one, one, one, one, None) == m.MOE_ERR_UNSUPPORTED


def test_silu_mul_backward_validation(lib):
    f = lambda *a: _c(lib, "moe_silu_mul_backward", *a)
    one = 1
    # a, b, lda, dh, R, C, da, db, ldo, stream
    assert f(one, one, 16, one, 4, 12, one, one, 16, None) == m.MOE_ERR_SHAPE      # C % 8
    assert f(one, one, 8, one, 4, 16, one, one, 16, None) == m.MOE_ERR_SHAPE       # lda < C
    assert f(one, one, 32, one, 4, 16, one, one, 20, None) == m.MOE_ERR_SHAPE      # ldo % 8
    assert f(one, one, 16, one, -1, 16, one, one, 16, None) == m.MOE_ERR_SHAPE
    assert f(one, None, 16, one, 4, 16, one, one, 16, None) == m.MOE_ERR_NULL
    assert f(None, None, 16, None, 0, 16, None, None, 16, None) == m.MOE_OK        # R = 0


def test_weight_quantizer_validation(lib):
    q = lambda *a: _c(lib, "moe_quantize_weights", *a)
    one = 1
    assert q(one, 2, 256, 250, 1, 250, 0, 0.0, 0, one, one, None) == m.MOE_ERR_SHAPE
    assert q(one, 2, 256, 256, 3, 256, 0, 0.0, 0, one, one, None) == m.MOE_ERR_SHAPE
    assert q(one, 2, 256, 256, 1, 256, 1, 0.0, 0, one, one, None) == m.MOE_ERR_UNSUPPORTED
    assert q(one, 2, 256, 256, 1, 256, 0, 0.0, 2, one, one, None) == m.MOE_ERR_UNSUPPORTED
    assert q(None, 2, 256, 256, 1, 256, 0, 0.0, 0, one, one, None) == m.MOE_ERR_NULL
    assert q(None, 0, 256, 256, 1, 256, 0, 0.0, 0, None, None, None) == m.MOE_OK


def test_int8_quantizer_validation(lib):
    f = lambda *a: _c(lib, "moe_quantize_rows_i8", *a)
    p = 4096                       # non-null, 16-byte aligned dummy pointer: never dereferenced on these paths
    assert f(p, 4, 24, 0, 0.0, p, p, None, None) == m.MOE_ERR_SHAPE                    # C % 16
    assert f(p, -1, 32, 0, 0.0, p, p, None, None) == m.MOE_ERR_SHAPE
    assert f(p, 4, 32, 7, 0.0, p, p, None, None) == m.MOE_ERR_UNSUPPORTED
    assert f(p, 4, 32, m.MOE_SCALE_TENSOR_STATIC, 0.0, p, p, None, None) == m.MOE_ERR_SHAPE   # bad static scale
    assert f(p, 4, 32, 0, 0.0, p, None, None, None) == m.MOE_ERR_NULL
    assert f(None, 4, 32, 0, 0.0, p, p, None, None) == m.MOE_ERR_NULL
    for mode in (m.MOE_SCALE_TENSOR_DYNAMIC, m.MOE_SCALE_TENSOR_FROM_ROW_AMAX):
        assert f(p, 4, 32, mode, 0.0, p, p, None, None) == m.MOE_ERR_NULL         # the row maxima are needed
    assert f(p + 8, 4, 32, 0, 0.0, p, p, None, None) == m.MOE_ERR_SHAPE            # x not 16-byte aligned
    w = lambda *a: _c(lib, "moe_quantize_weights_i8", *a)
    assert w(p, 2, 256, 250, 1, 250, 0, 0.0, 0, p, p, None) == m.MOE_ERR_SHAPE
    assert w(p, 2, 256, 256, 1, 256, 0, 0.0, 2, p, p, None) == m.MOE_ERR_UNSUPPORTED
    assert w(None, 0, 256, 256, 1, 256, 0, 0.0, 0, None, None, None) == m.MOE_OK


def test_int8_gmm_validation(lib):
    f = lambda *a: _c(lib, "moe_gmm_i8", *a)
    one = 1
    def call(M=256, K=256, N=256, Kb=1, Nb=256, tr=1, E=8, El=8, ws=one, wsb=256, lhs=one, out=one):
        return f(lhs, one, 0, one, one, Kb, Nb, tr, one, E, 0, El, M, K, N, 0, out, ws, wsb, None)
    assert call(K=200) == m.MOE_ERR_SHAPE
    assert call(K=(1 << 17) + 128, Kb=1) == m.MOE_ERR_SHAPE       # the int32 sums could overflow
    assert call(K=144, Kb=2) == m.MOE_ERR_UNSUPPORTED
    assert call(lhs=None) == m.MOE_ERR_NULL
    assert call(wsb=8) == m.MOE_ERR_WORKSPACE
    assert call(M=0, out=None) == m.MOE_OK
