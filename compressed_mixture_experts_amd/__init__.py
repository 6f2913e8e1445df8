"""ButterflyMoE expert layer on AMD MI355X (gfx950): Python binding.

The computation runs in ``libbmoe.so`` (hand-written HIP kernels behind the C
ABI of ``include/bmoe.h``, ``bmoe_trace.h`` and ``bmoe_grad.h``).  The test
hooks of ``include/bmoe_debug.h`` live only in ``libbmoe_debug.so`` (the same
kernels, built with -DBMOE_DEBUG_EXPORTS), loaded on first use of a
``dbg_*`` function.  This module only marshals arguments: torch tensors
provide device memory and the current HIP stream.  There is no fallback path;
if a library is missing, loading it raises.  The environment variable
BMOE_LIBRARY names another build of the debug library to load for both (the
CPU ABI tests use it for the sanitized host build).

    import compressed_mixture_experts_amd as bmoe
    layer = bmoe.Layer.from_inputs(inputs, device="cuda")   # uploads + packs
    y = layer.forward(x)                                     # x: [T][d] on the GPU
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "BmoeError", "lib", "library_path", "pack_ternary", "packed_words", "Layer",
    "dbg_butterfly", "dbg_ternary_gemm", "dbg_ternary_gemm_fp4", "butterfly_backward", "substrate_grad",
    "combine_backward", "router_backward", "gelu_backward", "substrate_input_grad", "STATUS",
    "EXPORTED_SYMBOLS", "DEBUG_SYMBOLS", "debug_lib",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libbmoe.so")
_DEBUG_LIB_PATH = os.path.join(_PKG, "libbmoe_debug.so")

STATUS = {
    0: "BMOE_OK", 1: "BMOE_ERR_NULL", 2: "BMOE_ERR_SHAPE", 3: "BMOE_ERR_DTYPE",
    4: "BMOE_ERR_ALIGN", 5: "BMOE_ERR_ALIAS", 6: "BMOE_ERR_WORKSPACE",
    7: "BMOE_ERR_TERNARY", 8: "BMOE_ERR_HIP", 9: "BMOE_ERR_DEVICE",
}
F32, BF16 = 0, 1
NOALLOC_SCRATCH_BYTES = 64 << 20   # BMOE_NOALLOC_SCRATCH_BYTES of include/bmoe.h
ACT_NONE, ACT_GELU_ERF = 0, 1

# exports of libbmoe.so (include/bmoe.h, bmoe_trace.h, bmoe_grad.h)
EXPORTED_SYMBOLS = [
    "bmoe_packed_words", "bmoe_pack_ternary", "bmoe_workspace_size", "bmoe_prepared_bytes",
    "bmoe_prepare", "bmoe_route", "bmoe_forward", "bmoe_forward_noalloc", "bmoe_status_string",
    "bmoe_last_error", "bmoe_forward_kernels", "bmoe_forward_marked",
    "bmoe_butterfly_backward_workspace", "bmoe_butterfly_backward",
    "bmoe_substrate_grad_workspace", "bmoe_substrate_grad", "bmoe_combine_backward",
    "bmoe_router_backward_workspace", "bmoe_router_backward", "bmoe_gelu_backward",
    "bmoe_substrate_input_grad",
    "bmoe_train_state_size", "bmoe_forward_train_workspace", "bmoe_forward_train",
    "bmoe_layer_backward_workspace", "bmoe_layer_backward",
]
# exported by libbmoe_debug.so only (include/bmoe_debug.h)
DEBUG_SYMBOLS = ["bmoe_dbg_butterfly", "bmoe_dbg_ternary_gemm", "bmoe_dbg_ternary_gemm_fp4"]


class BmoeError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.name = STATUS.get(status, str(status))
        super().__init__(f"{self.name}: {detail}")


class LayerGrads(ctypes.Structure):
    """bmoe_layer_grads of include/bmoe_train.h (device pointers)."""
    _fields_ = [
        ("dx", ctypes.c_void_p), ("d_w_gate", ctypes.c_void_p),
        ("d_theta", ctypes.c_void_p * 2), ("d_phi", ctypes.c_void_p * 2), ("d_w_base", ctypes.c_void_p * 2),
    ]


class LayerStruct(ctypes.Structure):
    _fields_ = [
        ("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32),
        ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
        ("act_dtype", ctypes.c_int32), ("ffn_act", ctypes.c_int32),
        ("renorm_gates", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("w_gate", ctypes.c_void_p),
        ("w_base", ctypes.c_void_p * 2),
        ("theta", ctypes.c_void_p * 2),
        ("phi", ctypes.c_void_p * 2),
        ("w_scale", ctypes.c_float * 2),
        ("prepared", ctypes.c_void_p),
        ("prepared_bytes", ctypes.c_size_t),
    ]


_lib = None
_debug_lib = None


def library_path() -> str:
    return os.environ.get("BMOE_LIBRARY") or _LIB_PATH


def _load(path: str, debug: bool) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m compressed_mixture_experts_amd.build`")
    L = ctypes.CDLL(path)
    c_i32, c_sz, c_vp, c_f = ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
    pL = ctypes.POINTER(LayerStruct)
    L.bmoe_packed_words.argtypes = [c_i32, c_i32]
    L.bmoe_packed_words.restype = c_sz
    L.bmoe_pack_ternary.argtypes = [c_vp, c_i32, c_i32, c_vp, c_sz]
    L.bmoe_workspace_size.argtypes = [pL, c_i32, ctypes.POINTER(c_sz)]
    L.bmoe_prepared_bytes.argtypes = [pL]
    L.bmoe_prepared_bytes.restype = c_sz
    L.bmoe_prepare.argtypes = [pL, c_vp, c_sz, c_vp]
    L.bmoe_route.argtypes = [pL, c_vp, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]
    L.bmoe_forward.argtypes = [pL, c_vp, c_i32, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]
    L.bmoe_forward_noalloc.argtypes = [pL, c_vp, c_i32, c_vp, c_vp, c_vp, c_vp]
    L.bmoe_status_string.argtypes = [c_i32]
    L.bmoe_status_string.restype = ctypes.c_char_p
    L.bmoe_last_error.argtypes = []
    L.bmoe_last_error.restype = ctypes.c_char_p
    L.bmoe_forward_kernels.argtypes = [pL, ctypes.POINTER(c_i32), ctypes.c_char_p, c_sz]
    L.bmoe_forward_marked.argtypes = [pL, c_vp, c_i32, c_vp, c_vp, c_sz, c_vp, c_vp, c_i32]
    L.bmoe_butterfly_backward_workspace.argtypes = [c_i32, c_i32, c_i32, ctypes.POINTER(c_sz)]
    L.bmoe_butterfly_backward.argtypes = [c_i32, c_i32, c_i32, c_vp, c_vp, c_i32, c_i32, c_vp, c_vp, c_vp,
                                          c_vp, c_vp, c_sz, c_vp]
    L.bmoe_substrate_grad_workspace.argtypes = [c_i32, c_i32, c_i32, ctypes.POINTER(c_sz)]
    L.bmoe_substrate_grad.argtypes = [c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_f, c_vp, c_vp, c_sz, c_vp]
    L.bmoe_combine_backward.argtypes = [c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]
    L.bmoe_router_backward_workspace.argtypes = [c_i32, c_i32, c_i32, ctypes.POINTER(c_sz)]
    L.bmoe_router_backward.argtypes = [c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                       c_vp, c_sz, c_vp]
    L.bmoe_gelu_backward.argtypes = [c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp]
    L.bmoe_substrate_input_grad.argtypes = [c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_f, c_vp, c_vp]
    L.bmoe_train_state_size.argtypes = [pL, c_i32, ctypes.POINTER(c_sz)]
    L.bmoe_forward_train_workspace.argtypes = [pL, c_i32, ctypes.POINTER(c_sz)]
    L.bmoe_forward_train.argtypes = [pL, c_vp, c_i32, c_vp, c_vp, c_sz, c_vp, c_sz, c_vp]
    L.bmoe_layer_backward_workspace.argtypes = [pL, c_i32, ctypes.POINTER(c_sz)]
    L.bmoe_layer_backward.argtypes = [pL, c_vp, c_i32, c_vp, c_vp, c_sz, ctypes.POINTER(LayerGrads), c_vp, c_sz,
                                      c_vp]
    ret = [n for n in EXPORTED_SYMBOLS if n not in ("bmoe_packed_words", "bmoe_prepared_bytes",
                                                    "bmoe_status_string", "bmoe_last_error")]
    if debug:
        L.bmoe_dbg_butterfly.argtypes = [c_i32, c_i32, c_vp, c_i32, c_i32, c_vp, c_vp, c_vp]
        L.bmoe_dbg_ternary_gemm.argtypes = [c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_f, c_vp, c_vp]
        L.bmoe_dbg_ternary_gemm_fp4.argtypes = [c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_f, c_vp, c_vp]
        ret += DEBUG_SYMBOLS
    for name in ret:
        getattr(L, name).restype = c_i32
    return L


def lib() -> ctypes.CDLL:
    """Load libbmoe.so (built in-tree by compressed_mixture_experts_amd.build)."""
    global _lib
    if _lib is None:
        alt = os.environ.get("BMOE_LIBRARY")
        _lib = debug_lib() if alt else _load(_LIB_PATH, debug=False)
    return _lib


def debug_lib() -> ctypes.CDLL:
    """Load libbmoe_debug.so: the product exports plus the test hooks of
    include/bmoe_debug.h (or the library BMOE_LIBRARY names)."""
    global _debug_lib
    if _debug_lib is None:
        _debug_lib = _load(os.environ.get("BMOE_LIBRARY") or _DEBUG_LIB_PATH, debug=True)
    return _debug_lib


def _check(status: int, L: Optional[ctypes.CDLL] = None) -> None:
    """Raise BmoeError for a nonzero status; the detail comes from the
    thread-local error string of the library that returned it."""
    if status != 0:
        detail = (L or lib()).bmoe_last_error().decode(errors="replace")
        raise BmoeError(status, detail)


def packed_words(rows: int, cols: int) -> int:
    return int(lib().bmoe_packed_words(rows, cols))


def pack_ternary(w: np.ndarray) -> np.ndarray:
    """int8 [rows][cols] in {-1,0,1} -> uint32 [rows][cols/16] (host, via the C ABI)."""
    w = np.ascontiguousarray(w, dtype=np.int8)
    if w.ndim != 2:
        raise ValueError("pack_ternary expects a 2-D array")
    rows, cols = w.shape
    nw = packed_words(rows, cols)
    out = np.zeros(max(nw, 1), dtype=np.uint32)
    _check(lib().bmoe_pack_ternary(w.ctypes.data, rows, cols, out.ctypes.data, nw))
    return out[:nw].reshape(rows, cols // 16)


# --------------------------------------------------------------------------- torch glue
def _torch():
    import torch
    return torch


def _stream_handle(stream=None) -> int:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _to_device_act(a: np.ndarray, act: str, device):
    torch = _torch()
    if act == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device).contiguous()


class Layer:
    """A ButterflyMoE layer resident on one GPU (weights packed and uploaded)."""

    def __init__(self, *, d_model: int, d_ff: int, n_experts: int, top_k: int, act: str,
                 ffn_act: str, renorm_gates: bool, w_gate, w_base_packed: Sequence,
                 theta: Sequence, phi: Sequence, w_scale: Sequence[float]):
        self.d_model, self.d_ff, self.n_experts, self.top_k = d_model, d_ff, n_experts, top_k
        self.act = act
        self.w_gate = w_gate
        self.w_base = list(w_base_packed)
        self.theta = list(theta)
        self.phi = list(phi)
        s = LayerStruct()
        s.d_model, s.d_ff, s.n_experts, s.top_k = d_model, d_ff, n_experts, top_k
        s.act_dtype = BF16 if act == "bf16" else F32
        s.ffn_act = ACT_GELU_ERF if ffn_act == "gelu" else ACT_NONE
        s.renorm_gates = 1 if renorm_gates else 0
        s.reserved = 0
        s.w_gate = _ptr(w_gate)
        for m in range(2):
            s.w_base[m] = _ptr(self.w_base[m]) if m < len(self.w_base) else None
            s.theta[m] = _ptr(self.theta[m]) if m < len(self.theta) else None
            s.phi[m] = _ptr(self.phi[m]) if m < len(self.phi) else None
            s.w_scale[m] = float(w_scale[m]) if m < len(w_scale) else 1.0
        s.prepared, s.prepared_bytes = None, 0
        self.struct = s
        self._ws = None
        self._prep = None

    @classmethod
    def from_inputs(cls, inp, device="cuda") -> "Layer":
        """Pack and upload the arrays of a workloads.LayerInputs."""
        torch = _torch()
        cfg = inp.cfg
        packed = [torch.from_numpy(pack_ternary(w).view(np.int32)).to(device).contiguous()
                  for w in inp.w_base]
        th = [torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device) for a in inp.theta]
        ph = [torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device) for a in inp.phi]
        wg = _to_device_act(inp.w_gate, cfg.act, device)
        nsub = len(inp.w_base)
        return cls(d_model=cfg.d_model, d_ff=cfg.d_ff, n_experts=cfg.n_experts, top_k=cfg.top_k,
                   act=cfg.act, ffn_act=cfg.ffn_act, renorm_gates=cfg.renorm_gates, w_gate=wg,
                   w_base_packed=packed, theta=th, phi=ph, w_scale=[cfg.w_scale] * nsub)

    # ---------------------------------------------------------------- prepared weights
    def prepared_bytes(self) -> int:
        return int(lib().bmoe_prepared_bytes(ctypes.byref(self.struct)))

    def prepare(self):
        """Build the prepared weights once (bmoe_prepare) and use them from now
        on; a no-op for layers whose forward uses none."""
        torch = _torch()
        need = self.prepared_bytes()
        self.struct.prepared, self.struct.prepared_bytes = None, 0
        if need == 0:
            self._prep = None
            return self
        buf = torch.empty(need + 256, dtype=torch.uint8, device=self.w_gate.device)
        off = (-int(buf.data_ptr())) % 256
        view = buf[off:off + need]
        _check(lib().bmoe_prepare(ctypes.byref(self.struct), _ptr(view), need, _stream_handle()))
        self._prep = buf
        self.struct.prepared, self.struct.prepared_bytes = _ptr(view), need
        return self

    def unprepare(self):
        """Go back to building the prepared data inside every forward."""
        self.struct.prepared, self.struct.prepared_bytes = None, 0
        self._prep = None
        return self

    # ---------------------------------------------------------------- workspace
    def workspace_size(self, T: int) -> int:
        n = ctypes.c_size_t(0)
        _check(lib().bmoe_workspace_size(ctypes.byref(self.struct), int(T), ctypes.byref(n)))
        return int(n.value)

    def workspace(self, T: int, device=None):
        """A cached device workspace large enough for T tokens."""
        torch = _torch()
        need = self.workspace_size(T)
        if self._ws is None or self._ws.numel() < need:
            dev = device if device is not None else self.w_gate.device
            self._ws = torch.empty(max(need, 256) + 256, dtype=torch.uint8, device=dev)
        ws = self._ws
        off = (-int(ws.data_ptr())) % 256
        return ws[off:], need

    # ---------------------------------------------------------------- calls
    def route(self, x, with_buckets: bool = False):
        """Top-k routing of x [T][d_model].  Returns (idx [T][k] int32, gate [T][k]
        fp32[, offsets [N+1], bucket_slots [T*k]])."""
        torch = _torch()
        T = int(x.shape[0])
        dev = x.device
        idx = torch.empty((T, self.top_k), dtype=torch.int32, device=dev)
        gate = torch.empty((T, self.top_k), dtype=torch.float32, device=dev)
        off = slots = None
        if with_buckets:
            off = torch.empty(self.n_experts + 1, dtype=torch.int32, device=dev)
            slots = torch.empty(max(T * self.top_k, 1), dtype=torch.int32, device=dev)
        ws, nbytes = self.workspace(T, dev)
        _check(lib().bmoe_route(ctypes.byref(self.struct), _ptr(x), T, _ptr(idx), _ptr(gate),
                                _ptr(off), _ptr(slots), _ptr(ws), nbytes, _stream_handle()))
        if with_buckets:
            return idx, gate, off, slots[:T * self.top_k]
        return idx, gate

    def forward(self, x, y=None, return_routing: bool = False):
        """y [T][d_model] = ButterflyMoE layer(x)."""
        torch = _torch()
        T = int(x.shape[0])
        if y is None:
            y = torch.empty_like(x)
        idx = gate = None
        if return_routing:
            idx = torch.empty((T, self.top_k), dtype=torch.int32, device=x.device)
            gate = torch.empty((T, self.top_k), dtype=torch.float32, device=x.device)
        ws, nbytes = self.workspace(T, x.device)
        _check(lib().bmoe_forward(ctypes.byref(self.struct), _ptr(x), T, _ptr(y), _ptr(idx),
                                  _ptr(gate), _ptr(ws), nbytes, _stream_handle()))
        if return_routing:
            return y, idx, gate
        return y

    def forward_noalloc(self, x, y, idx=None, gate=None):
        """bmoe_forward_noalloc: the forward into caller-given y (and optional
        idx / gate [T][top_k]) with the library's fixed device scratch as the
        workspace; nothing is allocated by the call."""
        T = int(x.shape[0])
        _check(lib().bmoe_forward_noalloc(ctypes.byref(self.struct), _ptr(x), T, _ptr(y), _ptr(idx),
                                          _ptr(gate), _stream_handle()))
        return y

    def _sized(self, fn, T: int, device) -> Tuple[object, int]:
        torch = _torch()
        n = ctypes.c_size_t(0)
        _check(fn(ctypes.byref(self.struct), T, ctypes.byref(n)))
        return torch.empty(max(int(n.value), 256), dtype=torch.uint8, device=device), int(n.value)

    def forward_train(self, x, y=None):
        """bmoe_forward_train: y = layer(x) and the state the layer backward
        reads (an opaque device buffer).  Returns (y, state)."""
        torch = _torch()
        T = int(x.shape[0])
        if y is None:
            y = torch.empty_like(x)
        state, ns = self._sized(lib().bmoe_train_state_size, T, x.device)
        ws, nw = self._sized(lib().bmoe_forward_train_workspace, T, x.device)
        _check(lib().bmoe_forward_train(ctypes.byref(self.struct), _ptr(x), T, _ptr(y), _ptr(state), ns, _ptr(ws), nw,
                                        _stream_handle()))
        return y, state

    def backward(self, x, dy, state) -> dict:
        """bmoe_layer_backward: fp32 gradients of sum(dy * y) in x, the gate
        matrix, every rotation's angles and the latent substrates, at the
        state of forward_train(x).  Returns dict(x, w_gate, theta [list],
        phi [list], w_base [list]) of device tensors."""
        torch = _torch()
        T = int(x.shape[0])
        dev = x.device
        nm = 2 if self.struct.d_ff else 1
        out = {"x": torch.empty((T, self.d_model), dtype=torch.float32, device=dev),
               "w_gate": torch.empty((self.n_experts, self.d_model), dtype=torch.float32, device=dev),
               "theta": [], "phi": [], "w_base": []}
        g = LayerGrads()
        g.dx = _ptr(out["x"])
        g.d_w_gate = _ptr(out["w_gate"])
        for m in range(nm):
            th, ph = self.theta[m], self.phi[m]
            out["theta"].append(torch.empty_like(th, dtype=torch.float32))
            out["phi"].append(torch.empty_like(ph, dtype=torch.float32))
            d_out = 1 << (ph.shape[1])
            d_in = 1 << (th.shape[1])
            out["w_base"].append(torch.empty((d_out, d_in), dtype=torch.float32, device=dev))
            g.d_theta[m] = _ptr(out["theta"][m])
            g.d_phi[m] = _ptr(out["phi"][m])
            g.d_w_base[m] = _ptr(out["w_base"][m])
        ws, nw = self._sized(lib().bmoe_layer_backward_workspace, T, dev)
        _check(lib().bmoe_layer_backward(ctypes.byref(self.struct), _ptr(x), T, _ptr(dy), _ptr(state),
                                         int(state.numel()), ctypes.byref(g), _ptr(ws), nw, _stream_handle()))
        return out

    def kernel_names(self) -> List[str]:
        """Names of the kernel launches of one forward, in order."""
        n = ctypes.c_int32(0)
        buf = ctypes.create_string_buffer(512)
        _check(lib().bmoe_forward_kernels(ctypes.byref(self.struct), ctypes.byref(n), buf, 512))
        return buf.value.decode().split(",")[: n.value]

    def forward_marked(self, x, y, marks):
        """Forward into y, recording the raw hipEvent_t handles in `marks`
        (list of ints or None) before the first and after each kernel launch."""
        T = int(x.shape[0])
        ws, nbytes = self.workspace(T, x.device)
        arr = (ctypes.c_void_p * max(len(marks), 1))(*[m if m else None for m in marks])
        _check(lib().bmoe_forward_marked(ctypes.byref(self.struct), _ptr(x), T, _ptr(y),
                                             _ptr(ws), nbytes, _stream_handle(), arr, len(marks)))
        return y


def dbg_butterfly(angles, x, transpose: bool = False, out=None):
    """Rows of x [rows][n] -> B(angles) row (or B^T row); angles [log2 n][n/2] fp32."""
    torch = _torch()
    rows, n = int(x.shape[0]), int(x.shape[1])
    log2n = n.bit_length() - 1
    dtype = BF16 if x.dtype == torch.bfloat16 else F32
    if out is None:
        out = torch.empty_like(x)
    D = debug_lib()
    _check(D.bmoe_dbg_butterfly(log2n, rows, _ptr(angles), 1 if transpose else 0, dtype,
                                _ptr(x), _ptr(out), _stream_handle()), D)
    return out


def butterfly_backward(angles, offsets, x, dy, transpose: bool = False, dx=None):
    """Backward of the bucketed rotation pass y_r = B(angles_e) x_r (or B^T x_r)
    for rows r of expert e (rows offsets[e] .. offsets[e+1]-1).  angles
    [N][L][n/2] fp32, offsets [N+1] int32, x and dy [rows][n] (fp32 or bf16).
    Returns (dx [rows][n] like x, dangles [N][L][n/2] fp32)."""
    torch = _torch()
    N, L = int(angles.shape[0]), int(angles.shape[1])
    rows = int(x.shape[0])
    dtype = BF16 if x.dtype == torch.bfloat16 else F32
    if dx is None:
        dx = torch.empty_like(x)
    dang = torch.empty_like(angles)
    nb = ctypes.c_size_t(0)
    _check(lib().bmoe_butterfly_backward_workspace(L, N, rows, ctypes.byref(nb)))
    ws = torch.empty(max(int(nb.value), 16), dtype=torch.uint8, device=x.device)
    _check(lib().bmoe_butterfly_backward(L, N, rows, _ptr(offsets), _ptr(angles), 1 if transpose else 0, dtype,
                                         _ptr(x), _ptr(dy), _ptr(dx), _ptr(dang), _ptr(ws), int(nb.value),
                                         _stream_handle()))
    return dx, dang


def substrate_grad(dz, u, alpha: float = 1.0, dw=None):
    """Latent substrate gradient through the straight-through estimator:
    dw [d_out][d_in] fp32 = alpha * dz^T u over all rows; dz [rows][d_out] and
    u [rows][d_in] bf16."""
    torch = _torch()
    rows, d_out, d_in = int(dz.shape[0]), int(dz.shape[1]), int(u.shape[1])
    if dw is None:
        dw = torch.empty((d_out, d_in), dtype=torch.float32, device=dz.device)
    nb = ctypes.c_size_t(0)
    _check(lib().bmoe_substrate_grad_workspace(d_out, d_in, rows, ctypes.byref(nb)))
    ws = torch.empty(max(int(nb.value), 16), dtype=torch.uint8, device=dz.device)
    _check(lib().bmoe_substrate_grad(d_out, d_in, rows, BF16 if dz.dtype == torch.bfloat16 else F32, _ptr(dz),
                                     _ptr(u), float(alpha), _ptr(dw), _ptr(ws), int(nb.value), _stream_handle()))
    return dw


def combine_backward(dy, bucket_slots, topk_gate, top_k: int, o=None):
    """Backward of the gated combine: d_rows [T*k][d] = gate * dy[token] in
    bucket order, and (with the experts' outputs o in bucket order) d_gate
    [T*k] by flat slot.  Returns (d_rows, d_gate or None)."""
    torch = _torch()
    T, d = int(dy.shape[0]), int(dy.shape[1])
    d_rows = torch.empty((T * top_k, d), dtype=dy.dtype, device=dy.device)
    d_gate = torch.empty(T * top_k, dtype=torch.float32, device=dy.device) if o is not None else None
    _check(lib().bmoe_combine_backward(T, top_k, d, BF16 if dy.dtype == torch.bfloat16 else F32, _ptr(dy),
                                       _ptr(bucket_slots), _ptr(topk_gate), _ptr(o), _ptr(d_rows), _ptr(d_gate),
                                       _stream_handle()))
    return d_rows, d_gate


def router_backward(x, w_gate, topk_idx, d_gate, renorm: bool = False):
    """Gating network's backward with the chosen experts held: returns
    (dx [T][d] fp32, dw_gate [N][d] fp32)."""
    torch = _torch()
    T, d, N, k = int(x.shape[0]), int(x.shape[1]), int(w_gate.shape[0]), int(topk_idx.shape[1])
    dx = torch.empty((T, d), dtype=torch.float32, device=x.device)
    dwg = torch.empty((N, d), dtype=torch.float32, device=x.device)
    nb = ctypes.c_size_t(0)
    _check(lib().bmoe_router_backward_workspace(T, d, N, ctypes.byref(nb)))
    ws = torch.empty(max(int(nb.value), 16), dtype=torch.uint8, device=x.device)
    _check(lib().bmoe_router_backward(T, d, N, k, 1 if renorm else 0, BF16 if x.dtype == torch.bfloat16 else F32,
                                      _ptr(x), _ptr(w_gate), _ptr(topk_idx), _ptr(d_gate), _ptr(dx), _ptr(dwg),
                                      _ptr(ws), int(nb.value), _stream_handle()))
    return dx, dwg


def gelu_backward(h, da, dh=None):
    """dh = da * GELU'(h) (exact erf GELU), elementwise; h, da [rows][width]."""
    torch = _torch()
    rows, width = int(h.shape[0]), int(h.shape[1])
    if dh is None:
        dh = torch.empty_like(h)
    _check(lib().bmoe_gelu_backward(rows, width, BF16 if h.dtype == torch.bfloat16 else F32, _ptr(h), _ptr(da),
                                    _ptr(dh), _stream_handle()))
    return dh


def substrate_input_grad(dz, wt_packed, d_in: int, alpha: float = 1.0):
    """du [rows][d_in] = alpha * dz [rows][d_out] * W_base, with W_base^T packed
    ([d_in][d_out/16] words)."""
    torch = _torch()
    rows, d_out = int(dz.shape[0]), int(dz.shape[1])
    du = torch.empty((rows, d_in), dtype=dz.dtype, device=dz.device)
    _check(lib().bmoe_substrate_input_grad(rows, d_out, d_in, BF16 if dz.dtype == torch.bfloat16 else F32, _ptr(dz),
                                           _ptr(wt_packed), float(alpha), _ptr(du), _stream_handle()))
    return du


def dbg_ternary_gemm(a, w_packed, n_out: int, alpha: float = 1.0):
    """z [M][n_out] = alpha * a [M][K] @ W^T with W packed [n_out][K/16]."""
    torch = _torch()
    M, K = int(a.shape[0]), int(a.shape[1])
    dtype = BF16 if a.dtype == torch.bfloat16 else F32
    z = torch.empty((M, n_out), dtype=a.dtype, device=a.device)
    D = debug_lib()
    _check(D.bmoe_dbg_ternary_gemm(M, n_out, K, dtype, _ptr(a), _ptr(w_packed), float(alpha),
                                   _ptr(z), _stream_handle()), D)
    return z


def dbg_ternary_gemm_fp4(a, w_packed, n_out: int, alpha: float = 1.0):
    """Matrix-core form of dbg_ternary_gemm for bf16 `a` (substrate re-encoded as
    paired 2-bit codes in a scratch buffer first)."""
    torch = _torch()
    M, K = int(a.shape[0]), int(a.shape[1])
    z = torch.empty((M, n_out), dtype=a.dtype, device=a.device)
    scratch = torch.empty((n_out * K // 4,), dtype=torch.uint8, device=a.device)
    D = debug_lib()
    _check(D.bmoe_dbg_ternary_gemm_fp4(M, n_out, K, _ptr(a), _ptr(w_packed), _ptr(scratch),
                                       float(alpha), _ptr(z), _stream_handle()), D)
    return z
