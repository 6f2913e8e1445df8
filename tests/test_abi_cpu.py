"""C-ABI checks that need no GPU: exports, the 2-bit packing format, and every
argument error (all detected on the host before anything is enqueued)."""
import ctypes
import os
import re

import numpy as np
import pytest

import compressed_mixture_experts_amd as bm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions(debug=False):
    """Functions declared by the product headers (or by bmoe_debug.h alone)."""
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h") and (h == "bmoe_debug.h") == debug:
            src = open(os.path.join(ROOT, "include", h)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(bmoe_\w+)\s*\(", src))
    return names


def test_library_exports_every_declared_function():
    L = bm.lib()
    declared = header_functions()
    assert declared == set(bm.EXPORTED_SYMBOLS)
    for name in declared:
        assert hasattr(L, name), name
    # the test hooks are in the debug build only
    dbg = header_functions(debug=True)
    assert dbg == set(bm.DEBUG_SYMBOLS)
    D = bm.debug_lib()
    for name in declared | dbg:
        assert hasattr(D, name), name
    if not os.environ.get("BMOE_LIBRARY"):
        for name in dbg:
            assert not hasattr(L, name), f"{name} exported by the product library"


def decode_packed(words: np.ndarray, cols: int) -> np.ndarray:
    """Independent decoder of the documented word layout (bmoe.h)."""
    rows = words.shape[0]
    out = np.zeros((rows, cols), dtype=np.int8)
    for r in range(rows):
        for c in range(cols):
            w = int(words[r, c // 16])
            cc = c % 16
            j, h = cc >> 1, cc & 1
            nz = (w >> (16 * h + j)) & 1
            sg = (w >> (16 * h + 8 + j)) & 1
            assert not (sg and not nz), "negative zero code"
            out[r, c] = (-1 if sg else 1) if nz else 0
    return out


def test_pack_roundtrip_and_format():
    r = np.random.default_rng(0)
    w = r.integers(-1, 2, size=(7, 48)).astype(np.int8)
    p = bm.pack_ternary(w)
    assert p.shape == (7, 3) and p.dtype == np.uint32
    assert np.array_equal(decode_packed(p, 48), w)
    # single entries land on the documented bits
    one = np.zeros((1, 16), np.int8)
    one[0, 5] = -1  # column 5 = 2*2 + 1 -> nonzero bit 16+2, sign bit 16+8+2
    assert int(bm.pack_ternary(one)[0, 0]) == (1 << 18) | (1 << 26)
    one[0, 5] = 0
    one[0, 14] = 1  # column 14 = 2*7 + 0 -> nonzero bit 7
    assert int(bm.pack_ternary(one)[0, 0]) == 1 << 7


def test_pack_errors():
    with pytest.raises(bm.BmoeError) as e:
        bm.pack_ternary(np.full((2, 16), 2, np.int8))
    assert e.value.name == "BMOE_ERR_TERNARY" and "w[0]" in str(e.value)
    w = np.zeros((3, 32), np.int8)
    w[2, 17] = -2
    with pytest.raises(bm.BmoeError) as e:
        bm.pack_ternary(w)
    assert "w[81]" in str(e.value)
    with pytest.raises(bm.BmoeError) as e:
        bm.pack_ternary(np.zeros((2, 24), np.int8))
    assert e.value.name == "BMOE_ERR_SHAPE"
    assert bm.packed_words(4, 24) == 0 and bm.packed_words(4, 32) == 8
    L = bm.lib()
    assert L.bmoe_pack_ternary(None, 1, 16, None, 1) == 1
    buf = np.zeros(1, np.uint32)
    w = np.zeros((2, 16), np.int8)
    assert L.bmoe_pack_ternary(w.ctypes.data, 2, 16, buf.ctypes.data, 1) == 2  # out too small


FAKE = 0x7F0000000000  # never dereferenced: validation fails before any device call


def make_struct(**kw):
    s = bm.LayerStruct()
    s.d_model, s.d_ff, s.n_experts, s.top_k = 512, 0, 64, 2
    s.act_dtype, s.ffn_act, s.renorm_gates, s.reserved = bm.BF16, bm.ACT_NONE, 0, 0
    s.w_gate = FAKE
    s.w_base[0], s.theta[0], s.phi[0] = FAKE + 0x100000, FAKE + 0x200000, FAKE + 0x300000
    s.w_base[1], s.theta[1], s.phi[1] = FAKE + 0x400000, FAKE + 0x500000, FAKE + 0x600000
    s.w_scale[0] = s.w_scale[1] = 1.0
    for k, v in kw.items():
        setattr(s, k, v)
    return s


def ws_size(s, T):
    n = ctypes.c_size_t(0)
    st = bm.lib().bmoe_workspace_size(ctypes.byref(s), T, ctypes.byref(n))
    return st, n.value


@pytest.mark.parametrize("field,value,status", [
    ("d_model", 500, 2), ("d_model", 32, 2), ("d_model", 16384, 2), ("d_ff", 100, 2),
    ("n_experts", 0, 2), ("n_experts", 257, 2), ("top_k", 0, 2), ("top_k", 9, 2),
    ("act_dtype", 2, 3), ("ffn_act", 1, 3), ("renorm_gates", 2, 2), ("reserved", 1, 2),
    ("w_gate", None, 1), ("w_gate", FAKE + 8, 4),
])
def test_layer_validation(field, value, status):
    s = make_struct(**{field: value})
    assert ws_size(s, 16)[0] == status
    assert bm.lib().bmoe_last_error() != b""


def test_topk_limited_by_experts_and_ffn_pointers():
    assert ws_size(make_struct(n_experts=3, top_k=4), 8)[0] == 2
    s = make_struct(d_ff=2048, ffn_act=bm.ACT_GELU_ERF)
    s.phi[1] = None
    assert ws_size(s, 8)[0] == 1
    s = make_struct(d_ff=2048, ffn_act=bm.ACT_GELU_ERF)
    s.theta[1] = FAKE + 2  # misaligned angles
    assert ws_size(s, 8)[0] == 4
    s = make_struct()
    s.w_base[0] = FAKE + 4
    assert ws_size(s, 8)[0] == 4
    assert bm.lib().bmoe_workspace_size(None, 8, ctypes.byref(ctypes.c_size_t())) == 1


def test_workspace_size_monotone_and_layout():
    s = make_struct()
    prev = -1
    for T in (0, 1, 7, 64, 4096, 16384):
        st, n = ws_size(s, T)
        assert st == 0 and n > prev
        prev = n
    # square bf16 layer of width 512 (single fused expert kernel): one [T*k][d]
    # bf16 row buffer plus the substrate at one byte per weight
    st, n = ws_size(s, 4096)
    assert n >= 4096 * 2 * 512 * 2 + 512 * 512
    # fp32 square layer (separate kernels): two [T*k][d] row buffers
    st, n32 = ws_size(make_struct(act_dtype=bm.F32), 4096)
    assert st == 0 and n32 >= 2 * 4096 * 2 * 512 * 4
    sf = make_struct(d_model=1024, d_ff=4096, ffn_act=bm.ACT_GELU_ERF)
    st, nf = ws_size(sf, 8192)
    assert st == 0 and nf >= 8192 * 2 * (1024 + 4096) * 2
    assert ws_size(s, -1)[0] == 2


def call_forward(s, x=FAKE + 0x800000, T=16, y=FAKE + 0x900000, idx=None, gate=None,
                 ws=FAKE + 0x1000000, nbytes=None):
    if nbytes is None:
        nbytes = ws_size(s, T)[1]
    return bm.lib().bmoe_forward(ctypes.byref(s), x, T, y, idx, gate, ws, nbytes, None)


def test_forward_argument_errors():
    s = make_struct()
    assert call_forward(s, x=None) == 1
    assert call_forward(s, y=None) == 1
    assert call_forward(s, ws=None) == 1
    assert call_forward(s, x=FAKE + 0x800008) == 4
    assert call_forward(s, y=FAKE + 0x900004) == 4
    assert call_forward(s, ws=FAKE + 0x1000010) == 4
    need = ws_size(s, 16)[1]
    assert call_forward(s, nbytes=need - 1) == 6
    # y overlapping x, y overlapping the workspace, x overlapping the workspace
    assert call_forward(s, y=FAKE + 0x800000 + 256) == 5
    assert call_forward(s, y=FAKE + 0x1000000 + 512) == 5
    assert call_forward(s, x=FAKE + 0x1000000 + 1024) == 5
    assert call_forward(s, idx=FAKE + 0x900000) == 5          # topk output on y
    assert call_forward(s, idx=FAKE + 0x2000004) == 4         # misaligned idx
    assert call_forward(s, T=-3) == 2
    assert call_forward(s, T=0, x=None, y=None, ws=None) == 0  # empty batch: no-op
    assert b"overlap" not in bm.lib().bmoe_last_error()


def test_route_argument_errors():
    s = make_struct()
    L = bm.lib()
    n = ws_size(s, 16)[1]
    ws = FAKE + 0x1000000
    assert L.bmoe_route(ctypes.byref(s), FAKE, 16, None, FAKE + 0x200000000, None, None, ws, n, None) == 1
    assert L.bmoe_route(ctypes.byref(s), FAKE, 16, ws + 256, FAKE + 0x200000000, None, None, ws, n, None) == 5
    assert L.bmoe_route(ctypes.byref(s), FAKE, 16, FAKE + 0x200000000, FAKE + 0x200000000, None, None, ws, n, None) == 5


def test_debug_hook_argument_errors():
    L = bm.debug_lib()
    assert L.bmoe_dbg_butterfly(2, 4, FAKE, 0, 0, FAKE, FAKE, None) == 2
    assert L.bmoe_dbg_butterfly(14, 4, FAKE, 0, 0, FAKE, FAKE, None) == 2
    assert L.bmoe_dbg_butterfly(8, 4, FAKE, 3, 0, FAKE, FAKE, None) == 2
    assert L.bmoe_dbg_butterfly(8, 4, FAKE, 0, 5, FAKE, FAKE, None) == 3
    assert L.bmoe_dbg_butterfly(8, 4, None, 0, 0, FAKE, FAKE, None) == 1
    assert L.bmoe_dbg_butterfly(8, 4, FAKE, 0, 0, FAKE + 4, FAKE + 0x100000, None) == 4
    assert L.bmoe_dbg_butterfly(8, 4, FAKE, 0, 0, FAKE, FAKE + 64, None) == 5
    assert L.bmoe_dbg_butterfly(8, 0, None, 0, 0, None, None, None) == 0
    assert L.bmoe_dbg_ternary_gemm(8, 96, 64, 1, FAKE, FAKE, ctypes.c_float(1.0), FAKE + 0x100000, None) == 2
    assert L.bmoe_dbg_ternary_gemm(8, 64, 64, 1, FAKE, FAKE, ctypes.c_float(1.0), FAKE + 16, None) == 5
    assert L.bmoe_dbg_ternary_gemm(8, 64, 64, 7, FAKE, FAKE, ctypes.c_float(1.0), FAKE + 0x100000, None) == 3
    # fp4 form: N a multiple of 256, K of 128; scratch must not alias an operand
    g = L.bmoe_dbg_ternary_gemm_fp4
    one = ctypes.c_float(1.0)
    assert g(8, 128, 128, FAKE, FAKE + 0x1000, FAKE + 0x2000, one, FAKE + 0x100000, None) == 2
    assert g(8, 256, 64, FAKE, FAKE + 0x1000, FAKE + 0x2000, one, FAKE + 0x100000, None) == 2
    assert g(0, 256, 128, None, None, None, one, None, None) == 0
    assert g(8, 256, 128, FAKE, FAKE + 0x10000, None, one, FAKE + 0x100000, None) == 1
    assert g(8, 256, 128, FAKE, FAKE + 0x10000, FAKE + 0x20008, one, FAKE + 0x100000, None) == 4
    assert g(8, 256, 128, FAKE, FAKE + 0x10000, FAKE + 0x10000, one, FAKE + 0x100000, None) == 5
    assert g(8, 256, 128, FAKE, FAKE + 0x10000, FAKE + 0x20000, one, FAKE + 0x100000, None) in (8, 9)


def test_status_strings():
    L = bm.lib()
    for code, name in bm.STATUS.items():
        assert L.bmoe_status_string(code).decode().startswith(name)


def test_prepared_bytes_layout():
    L = bm.lib()
    # square bf16 width 512: 2-bit substrate d*d/4 plus 98304 factor bytes per expert
    # every bf16 layer ends with the gate matrix in fragment order: 16-expert
    # blocks (64 experts here) of d_model bf16 each
    gate = lambda n_exp, d: (n_exp + 15) // 16 * 16 * d * 2
    s = make_struct()
    assert L.bmoe_prepared_bytes(ctypes.byref(s)) == 512 * 512 // 4 + 64 * 98304 + gate(64, 512)
    s = make_struct(d_model=256)
    assert L.bmoe_prepared_bytes(ctypes.byref(s)) == 256 * 256 // 4 + 64 * 32768 + gate(64, 256)
    s = make_struct(d_model=512, n_experts=40)       # padded to 48 experts
    assert L.bmoe_prepared_bytes(ctypes.byref(s)) == 512 * 512 // 4 + 40 * 98304 + 48 * 512 * 2
    # widths 64 / 128: one byte per weight, no factors (rounded up to 256 bytes)
    s = make_struct(d_model=128)
    assert L.bmoe_prepared_bytes(ctypes.byref(s)) == 128 * 128 + gate(64, 128)
    # wider bf16 layers: each substrate whose product the matrix-core GEMM covers
    # (output width a multiple of 256, contraction a multiple of 128), 2 bits per weight;
    # every rotation of width 1024 .. 8192: one 16 x 16 high-part block per column
    # (width / 16 columns), and at widths 4096 / 8192 the low-part block factors
    # (16 chunks x (16 blocks 16 x 16 + 16 blocks 16 x 16), or (16 blocks 32 x 32
    # + 32 blocks 16 x 16))
    # low part: per chunk of w / 16 indices, G0 blocks (max(16, w / 256) wide) and
    # w / 256 G1 blocks of 16 x 16, all bf16
    hi = lambda w: (w // 16) * 512
    lo = lambda w: 16 * ((w // 16) * max(16, w // 256) * 2 + (w // 256) * 512)
    rot = lambda w: hi(w) + lo(w)
    assert L.bmoe_prepared_bytes(ctypes.byref(make_struct(d_model=1024))) == (1024 * 1024 // 4 + 2 * 64 * rot(1024)
                                                                          + gate(64, 1024))
    s = make_struct(d_model=1024, d_ff=4096, ffn_act=bm.ACT_GELU_ERF)
    assert L.bmoe_prepared_bytes(ctypes.byref(s)) == (2 * (4096 * 1024 // 4) + 2 * 64 * rot(1024)
                                                      + 2 * 64 * rot(4096) + gate(64, 1024))
    assert lo(4096) == 16 * 16384 and lo(8192) == 16 * (32768 + 16384)
    # phi_up of width 8192, whose stages 0..7 the up product's epilogue applies:
    # 32 chunks of 256 (16 blocks 16 x 16 of G0 + 16 of G1 each) instead
    lo256 = 32 * (16 * 512 + 16 * 512)
    s = make_struct(d_model=2048, d_ff=8192, ffn_act=bm.ACT_GELU_ERF)
    assert L.bmoe_prepared_bytes(ctypes.byref(s)) == (2 * (8192 * 2048 // 4) + 2 * 64 * rot(2048)
                                                      + 64 * (hi(8192) + lo256) + 64 * rot(8192)
                                                      + gate(64, 2048))
    # d_ff = 128: the up product (128 outputs) keeps the LDS-decoding GEMM, the down
    # one runs on the prepared codes
    s = make_struct(d_model=1024, d_ff=128, ffn_act=bm.ACT_GELU_ERF)
    assert L.bmoe_prepared_bytes(ctypes.byref(s)) == 1024 * 128 // 4 + 2 * 64 * rot(1024) + gate(64, 1024)
    # a narrow FFN: only the gate fragments
    s = make_struct(d_model=128, d_ff=64, ffn_act=bm.ACT_GELU_ERF)
    assert L.bmoe_prepared_bytes(ctypes.byref(s)) == gate(64, 128)
    # fp32 activations and invalid layers use none
    assert L.bmoe_prepared_bytes(ctypes.byref(make_struct(act_dtype=bm.F32))) == 0
    assert L.bmoe_prepared_bytes(ctypes.byref(make_struct(act_dtype=bm.F32, d_model=1024, d_ff=4096,
                                                          ffn_act=bm.ACT_GELU_ERF))) == 0
    assert L.bmoe_prepared_bytes(ctypes.byref(make_struct(d_model=100))) == 0


def test_prepare_argument_errors():
    L = bm.lib()
    s = make_struct()
    need = L.bmoe_prepared_bytes(ctypes.byref(s))
    buf = FAKE + 0x10000000
    assert L.bmoe_prepare(ctypes.byref(s), None, need, None) == 1
    assert L.bmoe_prepare(ctypes.byref(s), buf + 128, need, None) == 4
    assert L.bmoe_prepare(ctypes.byref(s), buf, need - 1, None) == 6
    assert L.bmoe_prepare(ctypes.byref(s), FAKE + 0x100000 - 256, need, None) == 5   # over w_base[0]
    assert L.bmoe_prepare(ctypes.byref(make_struct(d_model=100)), buf, need, None) == 2
    # FFN: the buffer must not overlap the down substrate either
    f = make_struct(d_model=1024, d_ff=4096, ffn_act=bm.ACT_GELU_ERF)
    fneed = L.bmoe_prepared_bytes(ctypes.byref(f))
    assert L.bmoe_prepare(ctypes.byref(f), FAKE + 0x400000 - 256, fneed, None) == 5
    assert L.bmoe_prepare(ctypes.byref(f), buf, fneed, None) in (8, 9)
    # a layer without prepared data: nothing to do
    assert L.bmoe_prepare(ctypes.byref(make_struct(act_dtype=bm.F32)), None, 0, None) == 0
    # valid arguments reach the device check (no GPU here)
    assert L.bmoe_prepare(ctypes.byref(s), buf, need, None) in (8, 9)


def test_forward_checks_prepared_buffer():
    L = bm.lib()
    s = make_struct()
    need = L.bmoe_prepared_bytes(ctypes.byref(s))
    n_plain = ws_size(s, 4096)[1]
    s.prepared, s.prepared_bytes = FAKE + 0x10000000, need
    st, n_prep = ws_size(s, 4096)
    # prepared data no longer needs room in the workspace
    assert st == 0 and n_plain - n_prep >= need - 256
    assert call_forward(s) in (8, 9)
    s.prepared_bytes = need - 1
    assert call_forward(s) == 6 and ws_size(s, 16)[0] == 6
    s.prepared, s.prepared_bytes = FAKE + 0x10000000 + 64, need
    assert call_forward(s) == 4


def test_butterfly_backward_arguments():
    # workspace: per-chunk partial angle gradients, ceil(rows / CH) + N chunks
    # of L n/2 floats, CH = RT * clamp(rows // (RT * 512), 1, 256 // RT) with
    # RT = min(64, 16384 / n); zero without rows
    L = bm.lib()
    n = ctypes.c_size_t(0)

    def want(log2n, N, rows):
        if log2n >= 12:  # part passes: 32-row chunks, plus two fp32 row buffers
            ch = 32 * min(max(rows // 8192, 1), 4)
            up = lambda v: -(-v // 256) * 256
            return up((-(-rows // ch) + N) * log2n * (1 << (log2n - 1)) * 4) + 2 * up(rows * (4 << log2n))
        if log2n in (9, 10, 11):  # one register pass, a workgroup per chunk
            ch = min(max(rows // 512, 8), 64) if log2n == 9 else 16 * min(max(rows // 16384, 1), 8)
            return (-(-rows // ch) + N) * log2n * (1 << (log2n - 1)) * 4
        rt = min(64, 8192 >> log2n) if log2n <= 9 else 16384 >> log2n
        ch = rt * min(max(rows // (rt * 512), 1), max(256 // rt, 1))
        return (-(-rows // ch) + N) * log2n * (1 << (log2n - 1)) * 4

    for args in ((9, 8, 300), (9, 8, 500000), (8, 3, 70000), (11, 9, 300000), (10, 4, 9000), (13, 2, 5), (11, 256, 65536), (9, 64, 8192), (13, 256, 65536), (12, 7, 200000),
                 (2, 3, 100000)):
        assert L.bmoe_butterfly_backward_workspace(*args, ctypes.byref(n)) == 0
        assert n.value == want(*args), args
    assert L.bmoe_butterfly_backward_workspace(4, 3, 0, ctypes.byref(n)) == 0 and n.value == 0
    for args, st in (((0, 4, 10), 2), ((14, 4, 10), 2), ((5, 0, 10), 2), ((5, 257, 10), 2), ((5, 4, -1), 2),
                     ((13, 4, 1 << 18), 2)):
        assert L.bmoe_butterfly_backward_workspace(*args, ctypes.byref(n)) == st
    assert L.bmoe_butterfly_backward_workspace(5, 4, 10, None) == 1

    need = (1 + 4) * 5 * 16 * 4
    F = FAKE
    x, dy, dx = F + 0x10000, F + 0x20000, F + 0x30000
    ang, dang, off, ws = F + 0x40000, F + 0x50000, F + 0x60000, F + 0x70000

    def call(log2n=5, N=4, rows=10, off=off, ang=ang, tr=0, dt=bm.F32, x=x, dy=dy, dx=dx, dang=dang,
             ws=ws, wsb=need):
        return L.bmoe_butterfly_backward(log2n, N, rows, off, ang, tr, dt, x, dy, dx, dang, ws, wsb, None)

    assert call(tr=2) == 2
    assert call(dt=7) == 3
    assert call(off=None) == 1 and call(dang=None) == 1 and call(x=None) == 1 and call(ws=None) == 1
    assert call(x=F + 0x10002) == 4            # rows of width >= 8 must be 16-byte aligned
    assert call(dy=F + 0x20008, dt=bm.BF16) == 4
    assert call(log2n=2, rows=10, x=F + 0x10002, wsb=1 << 20) == 4  # width 4: element alignment
    assert call(ws=F + 0x70008) == 4           # workspace 16-byte aligned
    assert call(wsb=need - 1) == 6
    assert call(dx=x + 64) == 5                # dx partly over x
    assert call(dang=ang + 4) == 5             # dangles over the angles
    assert call(ws=x) == 5                     # workspace over an input


def test_substrate_grad_arguments():
    L = bm.lib()
    n = ctypes.c_size_t(0)

    def want(d_out, d_in, rows):
        # splits of the rows: none when the 128 x 128 output tiles number 256 or more,
        # else about 512 workgroups with at least 512 rows each (32-row steps)
        if rows == 0:
            return 0
        t = 256 if d_out % 256 == 0 and d_in % 256 == 0 and (d_out // 256) * (d_in // 256) >= 256 else 128
        tiles = (d_out // t) * (d_in // t)
        ns = 1
        if tiles < 256:
            ns = max(1, min(-(-512 // tiles), -(-rows // 512)))
        kc = max(32, -(-(-(-rows // ns)) // 32) * 32)
        ns = max(1, -(-rows // kc))
        return ns * d_out * d_in * 4 if ns > 1 else 0

    for args in ((512, 512, 16384), (512, 512, 100), (2048, 8192, 65536), (8192, 2048, 65536), (128, 256, 7),
                 (4096, 4096, 300), (4096, 2048, 70000), (3968, 4096, 9000),
                 (1024, 1024, 1 << 20), (128, 128, 0)):
        assert L.bmoe_substrate_grad_workspace(*args, ctypes.byref(n)) == 0
        assert n.value == want(*args), args
    for args in ((100, 512, 10), (512, 0, 10), (512, 32768, 10), (512, 512, -1), (8192, 512, 1 << 20)):
        assert L.bmoe_substrate_grad_workspace(*args, ctypes.byref(n)) == 2, args
    assert L.bmoe_substrate_grad_workspace(512, 512, 10, None) == 1

    F = FAKE
    dz, u, dw, ws = F + 0x100000, F + 0x200000, F + 0x300000, F + 0x400000
    need = want(512, 512, 1000)

    def call(d_out=512, d_in=512, rows=1000, dt=bm.BF16, dz=dz, u=u, dw=dw, ws=ws, wsb=need):
        return L.bmoe_substrate_grad(d_out, d_in, rows, dt, dz, u, ctypes.c_float(1.0), dw, ws, wsb, None)

    assert need > 0
    assert call(d_out=200) == 2
    assert call(dt=bm.F32) == 3 and call(dt=9) == 3   # bf16 rows only
    assert call(dz=None) == 1 and call(u=None) == 1 and call(dw=None) == 1 and call(ws=None) == 1
    assert call(dw=dw + 4) == 4                       # dw 16-byte aligned
    assert call(dz=dz + 1) == 4 and call(u=u + 8) == 4   # rows 16-byte aligned
    assert call(ws=ws + 8) == 4
    assert call(wsb=need - 1) == 6
    assert call(dw=dz + 64) == 5                      # dw over dz
    assert call(ws=u) == 5                            # workspace over u
    assert call(ws=dw + 256) == 5                     # workspace over dw


def test_combine_backward_arguments():
    L = bm.lib()
    F = FAKE
    dy, sl, g, o, dr, dg = F + 0x100000, F + 0x200000, F + 0x300000, F + 0x400000, F + 0x500000, F + 0x600000

    def call(T=100, k=2, d=512, dt=bm.BF16, dy=dy, sl=sl, g=g, o=o, dr=dr, dg=dg):
        return L.bmoe_combine_backward(T, k, d, dt, dy, sl, g, o, dr, dg, None)

    assert call(d=100) == 2 and call(k=9) == 2 and call(T=-1) == 2 and call(d=32768) == 2
    assert call(T=1 << 20, k=8, d=512) == 2       # T * k * d beyond 2^31
    assert call(dt=5) == 3
    assert call(o=None) == 1 and call(dg=None) == 1  # o and d_gate together
    assert call(dy=None) == 1 and call(sl=None) == 1 and call(dr=None) == 1
    assert call(dy=dy + 8) == 4 and call(dr=dr + 2) == 4 and call(sl=sl + 2) == 4
    assert call(dr=dy) == 5                        # d_rows over dy
    assert call(dg=sl) == 5                        # d_gate over the slots
    assert call(dg=dr + 64) == 5                   # d_gate inside d_rows


def test_router_backward_arguments():
    L = bm.lib()
    n = ctypes.c_size_t(0)

    def splits(T, d, N, mf):
        tiles = (-(-N // 64) * (d // 256)) if mf else (-(-N // 16) * -(-d // 256))
        target, tmin = (512, 64) if mf else (2048, 256)
        S = 1
        if tiles < target:
            S = max(1, min(-(-target // tiles), -(-T // tmin)))
        tc = max(1, -(-T // S))
        return max(1, -(-T // tc))

    def want(T, d, N):
        # the larger of the VALU and matrix-core dW_g passes' token splits
        if T == 0:
            return 0
        S = max(splits(T, d, N, False), splits(T, d, N, d % 256 == 0))
        return -(-T * N * 4 // 256) * 256 + (S * N * d * 4 if S > 1 else 0)

    for args in ((4096, 512, 64), (16384, 512, 256), (32768, 2048, 256), (777, 128, 16), (10, 8, 3), (0, 64, 4)):
        assert L.bmoe_router_backward_workspace(*args, ctypes.byref(n)) == 0
        assert n.value == want(*args), args
    for args in ((10, 4096, 4), (10, 100, 4), (10, 64, 0), (10, 64, 257), (-1, 64, 4)):
        assert L.bmoe_router_backward_workspace(*args, ctypes.byref(n)) == 2, args

    F = FAKE
    x, w, ix, dg, dx, dw, ws = (F + 0x100000 * i for i in range(1, 8))
    need = want(100, 64, 8)

    def call(T=100, d=64, N=8, k=2, rn=0, dt=bm.BF16, x=x, w=w, ix=ix, dg=dg, dx=dx, dw=dw, ws=ws, wsb=need):
        return L.bmoe_router_backward(T, d, N, k, rn, dt, x, w, ix, dg, dx, dw, ws, wsb, None)

    assert call(k=9) == 2 and call(k=9, N=8) == 2 and call(rn=2) == 2 and call(N=1, k=2) == 2
    assert call(dt=4) == 3
    assert call(w=None) == 1 and call(dw=None) == 1 and call(x=None) == 1 and call(ws=None) == 1
    assert call(x=x + 8) == 4 and call(w=w + 2) == 4 and call(dg=dg + 2) == 4 and call(ws=ws + 8) == 4
    assert call(wsb=need - 4) == 6
    assert call(dx=x) == 5 and call(dw=w + 16) == 5 and call(ws=dx) == 5


def test_gelu_backward_arguments():
    L = bm.lib()
    F = FAKE
    h, da, dh = F + 0x100000, F + 0x200000, F + 0x300000

    def call(rows=10, w=64, dt=bm.F32, h=h, da=da, dh=dh):
        return L.bmoe_gelu_backward(rows, w, dt, h, da, dh, None)

    assert call(w=12) == 2 and call(rows=-1) == 2 and call(rows=1 << 20, w=4096) == 2
    assert call(dt=3) == 3
    assert call(h=None) == 1 and call(dh=None) == 1
    assert call(h=h + 4) == 4 and call(dh=dh + 8) == 4
    assert call(dh=h + 16) == 5 and call(dh=da + 256) == 5   # partial overlaps


def test_substrate_input_grad_arguments():
    L = bm.lib()
    F = FAKE
    dz, wt, du = F + 0x100000, F + 0x200000, F + 0x300000

    def call(rows=100, d_out=256, d_in=128, dt=bm.BF16, dz=dz, wt=wt, du=du):
        return L.bmoe_substrate_input_grad(rows, d_out, d_in, dt, dz, wt, ctypes.c_float(1.0), du, None)

    assert call(d_out=100) == 2 and call(d_in=32) == 2 and call(rows=-1) == 2
    assert call(dt=bm.F32, d_in=40) == 2               # fp32: multiples of 16
    assert call(dt=9) == 3
    assert call(dz=None) == 1 and call(wt=None) == 1 and call(du=None) == 1
    assert call(dz=dz + 8) == 4 and call(du=du + 2) == 4
    assert call(du=dz + 64) == 5 and call(du=wt) == 5
    assert call(rows=0, dz=None) == 0                    # nothing to do, nothing launched


def test_forward_kernel_names_of_the_widest_layer():
    # per-call preparation of an FFN layer whose both widths use the split
    # rotations in two passes each (widths 4096 and 8192): the most launches
    # one forward makes
    L = bm.lib()
    s = make_struct(d_model=4096, d_ff=8192, n_experts=256, ffn_act=bm.ACT_GELU_ERF)
    n = ctypes.c_int32(0)
    buf = ctypes.create_string_buffer(1024)
    assert L.bmoe_forward_kernels(ctypes.byref(s), ctypes.byref(n), buf, 1024) == 0
    names = buf.value.decode().split(",")
    # (the up product's epilogue applies stages 0..7 of phi_up, the middle
    # pass stage 8 onwards: no separate low pass of phi_up)
    assert len(names) == n.value == 21
    assert names[:1] == ["prep"] and names.count("prep_lo") == 4 and names.count("prep_hi") == 4
    assert names[9] == "prep_gate"
    assert names[10:] == ["route", "bucket", "bfly_in_hi", "bfly_in_lo", "gemm_up", "bfly_mid_hi",
                         "bfly_mid_lo_t", "gemm_down", "bfly_out_lo", "bfly_out_hi", "combine"]
    # truncation keeps the string terminated
    small = ctypes.create_string_buffer(8)
    assert L.bmoe_forward_kernels(ctypes.byref(s), ctypes.byref(n), small, 8) == 0
    assert small.value == b"prep,pr"
    assert L.bmoe_forward_kernels(ctypes.byref(s), None, small, 8) == 1
    # widths 1024 and 2048: the input and output rotations in one pass each
    s = make_struct(d_model=2048, d_ff=8192, n_experts=256, ffn_act=bm.ACT_GELU_ERF)
    assert L.bmoe_forward_kernels(ctypes.byref(s), ctypes.byref(n), buf, 1024) == 0
    names = buf.value.decode().split(",")
    assert len(names) == n.value == 19
    assert names[10:] == ["route", "bucket", "bfly_in", "gemm_up", "bfly_mid_hi",
                         "bfly_mid_lo_t", "gemm_down", "bfly_out", "combine"]


def test_forward_noalloc_argument_errors():
    # rejected on the host before any device call: a workspace beyond the fixed
    # scratch, a bad layer; T = 0 is a no-op
    L = bm.lib()
    s = make_struct()                       # d=512, 64 experts, top-2, no prepared buffer
    st, need = ws_size(s, 40000)
    assert st == 0 and need > bm.NOALLOC_SCRATCH_BYTES
    assert L.bmoe_forward_noalloc(ctypes.byref(s), FAKE, 40000, FAKE + 0x10000000, None, None, None) == 6
    msg = L.bmoe_last_error()
    assert b"scratch" in msg and str(bm.NOALLOC_SCRATCH_BYTES).encode() in msg
    assert L.bmoe_forward_noalloc(ctypes.byref(make_struct(d_model=500)), FAKE, 16, FAKE, None, None, None) == 2
    assert L.bmoe_forward_noalloc(None, FAKE, 16, FAKE, None, None, None) == 1
    assert L.bmoe_forward_noalloc(ctypes.byref(s), None, 0, None, None, None, None) == 0
    assert L.bmoe_forward_noalloc(ctypes.byref(s), FAKE, -1, FAKE, None, None, None) == 2


def test_training_path_argument_errors():
    # include/bmoe_train.h: every error found on the host before a device call
    L = bm.lib()
    n = ctypes.c_size_t(0)
    s = make_struct(d_model=256)
    assert L.bmoe_train_state_size(ctypes.byref(s), 100, ctypes.byref(n)) == 0 and n.value > 0
    state_need = n.value
    assert L.bmoe_train_state_size(ctypes.byref(make_struct(d_model=64)), 100, ctypes.byref(n)) == 2
    assert L.bmoe_train_state_size(ctypes.byref(s), -1, ctypes.byref(n)) == 2
    assert L.bmoe_train_state_size(ctypes.byref(s), 100, None) == 1
    assert L.bmoe_forward_train_workspace(ctypes.byref(s), 100, ctypes.byref(n)) == 0
    fw_need = n.value
    assert L.bmoe_layer_backward_workspace(ctypes.byref(s), 100, ctypes.byref(n)) == 0
    bw_need = n.value
    f = L.bmoe_forward_train
    big = 1 << 34
    assert f(ctypes.byref(s), None, 100, FAKE, FAKE + big, state_need, FAKE + 2 * big, fw_need, None) == 1
    assert f(ctypes.byref(s), FAKE + 8, 100, FAKE + big // 2, FAKE + big, state_need, FAKE + 2 * big, fw_need, None) == 4
    assert f(ctypes.byref(s), FAKE, 100, FAKE + big // 2, FAKE + big, state_need - 1, FAKE + 2 * big, fw_need,
             None) == 6
    assert f(ctypes.byref(s), FAKE, 100, FAKE, FAKE + big, state_need, FAKE + 2 * big, fw_need, None) == 5
    assert f(ctypes.byref(s), FAKE, 0, None, None, 0, None, 0, None) == 0
    g = bm.LayerGrads()
    g.dx, g.d_w_gate = FAKE + 3 * big, FAKE + 3 * big + (1 << 24)
    g.d_theta[0], g.d_phi[0], g.d_w_base[0] = (FAKE + 3 * big + (2 << 24), FAKE + 3 * big + (3 << 24),
                                               FAKE + 3 * big + (4 << 24))
    b = L.bmoe_layer_backward
    assert b(ctypes.byref(s), FAKE, 100, FAKE + big // 2, FAKE + big, state_need, None, FAKE + 2 * big, bw_need,
             None) == 1
    assert b(ctypes.byref(s), FAKE, 100, FAKE + big // 2, FAKE + big, state_need, ctypes.byref(g), FAKE + 2 * big,
             bw_need - 1, None) == 6
    g.d_phi[0] = g.d_theta[0]  # two outputs on one buffer
    assert b(ctypes.byref(s), FAKE, 100, FAKE + big // 2, FAKE + big, state_need, ctypes.byref(g), FAKE + 2 * big,
             bw_need, None) == 5
    g.d_phi[0] = FAKE + 3 * big + (3 << 24) + 4
    assert b(ctypes.byref(s), FAKE, 100, FAKE + big // 2, FAKE + big, state_need, ctypes.byref(g), FAKE + 2 * big,
             bw_need, None) == 4
    ffn = make_struct(d_model=256, d_ff=512, ffn_act=bm.ACT_GELU_ERF)
    g.d_phi[0] = FAKE + 3 * big + (3 << 24)
    assert b(ctypes.byref(ffn), FAKE, 100, FAKE + big // 2, FAKE + big, 1 << 30, ctypes.byref(g), FAKE + 2 * big,
             1 << 30, None) == 1  # the down substrate's gradient pointers are missing
