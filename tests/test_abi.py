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


def test_noalloc_decode_rejects_a_layer_beyond_its_array():
    """Hidden 16384, 512 experts (a 985,344-byte workspace): rejected on the
    host before anything is launched (the tensor pointers are never read)."""
    import bit_quantized_gemv_amd as q

    lib = q.lib()

    def qt(rows, cols, bits, p=0x100000):
        return q._QT(p, p + 0x1000000, p + 0x2000000, rows, cols, bits, 64, 0)

    H, E, K, I, Is = 16384, 512, 8, 2048, 1024
    L = q._Layer(H, E, K, I, Is, qt(E, H, 8), qt(I, H, 4), qt(I, H, 4), qt(H, I, 4),
                 qt(Is, H, 4), qt(Is, H, 4), qt(H, Is, 4), None, 1e-6, None)
    assert lib.qmoe_workspace_bytes(C.byref(L), 1) > (512 << 10)
    assert lib.qmoe_moe_decode_noalloc(C.byref(L), 0x3000, None, 0, 0x6000, None, None,
                                       None) == 4  # QMOE_ERR_WORKSPACE


def test_one_hip_runtime_whatever_the_import_order():
    """Importing the package before torch maps a single libamdhip64: the
    library binds to torch's HIP runtime instead of loading a second one
    (with two, device symbols set through one are unknown to the other)."""
    import subprocess
    import sys

    code = ("import sys; sys.path.insert(0, %r)\n"
            "import bit_quantized_gemv_amd\n"
            "import torch\n"
            "maps = open('/proc/self/maps').read().split('\\n')\n"
            "libs = {l.split()[-1] for l in maps if 'libamdhip64' in l}\n"
            "print(len(libs), sorted(libs))\n" % ROOT)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    assert r.stdout.split()[0] == "1", r.stdout


def test_sample_validation_before_launch():
    """qmoe_sample rejects bad arguments on the host (the pointers below are
    never read)."""
    import bit_quantized_gemv_amd as q

    lib = q.lib()
    ws = 1 << 20
    call = lambda V, T, K, P, U, wsb=ws: lib.qmoe_sample(0x1000, V, T, K, P, U, 0x2000, None,
                                                          0x3000, wsb, None)
    assert call(262144, 0.2, 65, 0.95, 0.5) == 3    # QMOE_ERR_UNSUPPORTED: top_k > 64
    assert call(32, 0.2, 64, 0.95, 0.5) == 2        # QMOE_ERR_BAD_SHAPE: top_k > V
    assert call(1 << 21, 0.2, 64, 0.95, 0.5) == 3   # past the vocabulary limit
    assert call(1000, -0.1, 64, 0.95, 0.5) == 2     # negative temperature
    assert call(1000, 0.2, 64, 0.0, 0.5) == 2       # top_p must be > 0
    assert call(1000, 0.2, 64, 1.5, 0.5) == 2       # top_p <= 1
    assert call(1000, 0.2, 64, 0.95, 1.0) == 2      # u < 1
    assert call(262144, 0.2, 64, 0.95, 0.5, 100) == 4  # QMOE_ERR_WORKSPACE
    assert q.qmoe_sample_workspace_bytes(262144, 64) == 256 * 64 * 8
    assert q.qmoe_sample_workspace_bytes(1 << 20, 64) == 256 * 64 * 8


def test_file_tier_validation_before_any_gpu_call(tmp_path):
    """qmoe_file_tier_open checks its file and sizes before it allocates
    pinned memory or starts threads."""
    import ctypes as C

    import bit_quantized_gemv_amd as q

    lib = q.lib()
    h = C.c_void_p()
    missing = str(tmp_path / "none.bin").encode()
    assert lib.qmoe_file_tier_open(missing, 2, 4, 8192, 8192, 2, 8, 0, C.byref(h)) == 2
    assert lib.qmoe_file_tier_open(missing, 2, 4, 4000, 8000, 2, 8, 0, C.byref(h)) == 5  # stride
    short = tmp_path / "short.bin"
    short.write_bytes(b"\0" * (2 * 4 * 8192 - 1))
    assert lib.qmoe_file_tier_open(str(short).encode(), 2, 4, 8192, 8192, 2, 8, 0,
                                   C.byref(h)) == 2
    assert lib.qmoe_file_tier_open(str(short).encode(), 2, 4, 8192, 8192, 0, 8, 0,
                                   C.byref(h)) == 2  # threads
    assert lib.qmoe_file_tier_open(str(short).encode(), 2, 4, 8192, 8192, 2, 9, 0,
                                   C.byref(h)) == 2  # max_misses > 8
    assert lib.qmoe_file_tier_open(str(short).encode(), 2, 4, 9000, 8192, 2, 8, 0,
                                   C.byref(h)) == 2  # stride < blob


def test_attn_validation_before_launch():
    """qmoe_attn_decode rejects bad shapes, positions and buffers on the host
    (the pointers below are never read)."""
    import bit_quantized_gemv_amd as q

    lib = q.lib()

    def shape(Hq=16, Hkv=8, D=256, S=4096, circ=0, base=10000.0, scale=0.0625):
        return q.AttnShape(Hq, Hkv, D, S, circ, base, scale)

    ws = 1 << 24
    P = (0x1000, 0x2000, 0x3000)

    def call(s, pos=5, wsb=ws, kc=0x10000, out=0x30000, qp=P[0]):
        return lib.qmoe_attn_decode(C.byref(s), qp, P[1], P[2], pos, kc, 0x20000, out, 0x40000,
                                    wsb, None)

    assert call(shape(), qp=None) == 1                  # QMOE_ERR_NULL_ARG
    assert call(shape(Hq=12)) == 2                      # Hkv does not divide Hq
    assert call(shape(), pos=-1) == 2                   # negative position
    assert call(shape(S=16), pos=16) == 2               # a linear cache is full
    assert call(shape(base=1.0)) == 2                   # RoPE base
    assert call(shape(D=64)) == 3                       # QMOE_ERR_UNSUPPORTED: head width
    assert call(shape(Hq=32, Hkv=8)) == 3               # four query heads per group at D = 256
    assert call(shape(), wsb=100) == 4                  # QMOE_ERR_WORKSPACE
    assert call(shape(), kc=0x10008) == 5               # QMOE_ERR_ALIGN
    # control words (64 bytes, then 8 epoch words per key/value head,
    # rounded to 256) and the largest split count's partials: S / 32 splits
    # of Hq (D + 2) tagged 8-byte words
    assert q.qmoe_attn_workspace_bytes(shape()) == 512 + 128 * 16 * 258 * 8
    code = C.c_int32(0)
    assert lib.qmoe_attn_workspace_status(None, 1024, 8, C.byref(code), None) == 1
    assert lib.qmoe_attn_workspace_status(0x1000, 1024, 0, C.byref(code), None) == 2
    assert lib.qmoe_attn_workspace_status(0x1000, 256, 8, C.byref(code), None) == 4
    assert q.qmoe_attn_workspace_bytes(shape(Hq=12)) == 0
