"""The C-ABI library loads, exports every entry point include/qmoe.h
declares, and rejects bad arguments before touching a GPU (CPU only)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmoe.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(qmoe_\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("qmoe_router_topk", "qmoe_gemv_affine4", "qmoe_expert_ffn", "qmoe_prefill_grouped",
              "qmoe_moe_decode", "qmoe_rmsnorm", "qmoe_workspace_bytes", "qmoe_status_string"):
        assert n in names, n


def test_library_exports_every_declared_symbol():
    import bit_quantized_gemv_amd as q

    lib = C.CDLL(q.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n


def _qt(q, rows=8, cols=128, bits=4, ptr=0x1000):
    return q._QT(ptr, ptr + 0x100000, ptr + 0x200000, rows, cols, bits, 64, 0)


def test_validation_before_launch():
    import bit_quantized_gemv_amd as q

    lib = q.lib()
    W = _qt(q)
    assert lib.qmoe_gemv_affine4(C.byref(W), None, 0x3000, None) == 1      # NULL x
    W.cols = 100
    assert lib.qmoe_gemv_affine4(C.byref(W), 0x3000, 0x4000, None) == 2    # cols % 64
    W.cols, W.bits = 128, 8
    assert lib.qmoe_gemv_affine4(C.byref(W), 0x3000, 0x4000, None) == 3    # bits
    W.bits, W.group = 4, 32
    assert lib.qmoe_gemv_affine4(C.byref(W), 0x3000, 0x4000, None) == 3    # group
    W.group = 64
    W.q = 0x1004
    assert lib.qmoe_gemv_affine4(C.byref(W), 0x3000, 0x4000, None) == 5    # alignment
    R = _qt(q, rows=16, cols=128, bits=8)
    assert lib.qmoe_router_topk(C.byref(R), None, 0x3000, 0, 8, 0x5000, 0x6000, None, 0x7000,
                                1 << 20, None) == 2                         # T = 0
    assert lib.qmoe_router_topk(C.byref(R), None, 0x3000, 4, 9, 0x5000, 0x6000, None, 0x7000,
                                1 << 20, None) == 3                         # top_k > 8
    assert lib.qmoe_router_topk(C.byref(R), None, 0x3000, 4, 8, 0x5000, 0x6000, None, 0x7000,
                                16, None) == 4                              # workspace
    for i in range(8):
        assert lib.qmoe_status_string(i)


def _layer(q, H=512, E=32, K=8, I=256, Is=512):
    return q._Layer(H, E, K, I, Is, _qt(q, E, H, 8), _qt(q, I, H), _qt(q, I, H), _qt(q, H, I),
                    _qt(q, Is, H), _qt(q, Is, H), _qt(q, H, Is), None, 1e-6, None)


def test_layer_validation_and_workspace_size():
    import bit_quantized_gemv_amd as q

    lib = q.lib()
    L = _layer(q)
    n1 = lib.qmoe_workspace_bytes(C.byref(L), 1)
    assert n1 > 0
    assert lib.qmoe_workspace_bytes(C.byref(L), 128) >= n1
    assert lib.qmoe_workspace_bytes(C.byref(L), 129) == 0
    assert lib.qmoe_expert_ffn(C.byref(L), 0x3000, 0x4000, 0x5000, None, None, 0x6000, 0x7000,
                               n1 - 1, None) == 4
    bad = _layer(q, K=9)
    assert lib.qmoe_workspace_bytes(C.byref(bad), 1) == 0
    assert lib.qmoe_moe_decode(C.byref(bad), 0x3000, None, 0, 0x6000, None, None, 0x7000, 1 << 24,
                               None) == 3   # top_k above the kernels' limit of 8


def test_stack_sizes_and_validation_before_launch():
    """The stack entry points size their buffers and reject bad arguments on
    the host, before any HIP call (no GPU needed)."""
    import bit_quantized_gemv_amd as q

    lib = q.lib()
    assert lib.qmoe_stack_table_bytes(0) == 0
    assert lib.qmoe_stack_table_bytes(129) == 0
    one = lib.qmoe_stack_table_bytes(1)
    assert one > 0 and lib.qmoe_stack_table_bytes(30) == 30 * one
    L = _layer(q)
    wsn = lib.qmoe_stack_workspace_bytes(C.byref(L))
    # the one-layer workspace plus two bf16 [H] input buffers
    assert wsn >= lib.qmoe_workspace_bytes(C.byref(L), 1) + 2 * 512 * 2
    bad = _layer(q, K=9)
    assert lib.qmoe_stack_workspace_bytes(C.byref(bad)) == 0
    tab, x, out, ws = 0x10000, 0x20000, 0x30000, 0x40000

    def dec(layer=L, table=tab, n=3, xx=x, oo=out, nbytes=wsn):
        return lib.qmoe_stack_decode(C.byref(layer), table, n, xx, oo, None, None, None, ws,
                                     nbytes, None)

    assert dec(table=None) == 1
    assert dec(n=0) == 2 and dec(n=129) == 2
    assert dec(oo=x) == 2                    # output may not alias the input
    assert dec(xx=x + 2) == 5                # alignment
    assert dec(nbytes=wsn - 1) == 4
    assert dec(layer=bad) == 3
    # table set-up: every layer must have the first one's shape
    arr = (q._Layer * 2)(_layer(q), _layer(q, I=512))
    assert lib.qmoe_stack_table_init(arr, 2, tab, 2 * one, None) == 2
    arr = (q._Layer * 2)(_layer(q), _layer(q))
    assert lib.qmoe_stack_table_init(arr, 2, tab, 2 * one - 1, None) == 4
    assert lib.qmoe_stack_table_init(arr, 0, tab, 2 * one, None) == 2
    assert lib.qmoe_stack_table_init(arr, 2, None, 2 * one, None) == 1
