"""Thin ctypes binding of libtfl.so (include/tfl.h).

Argument marshalling only: every step of the forward pass runs in the HIP
kernels behind the C ABI.  PyTorch provides device memory and the stream.
If the library is not built this module raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libtfl.so")
AUDIT_LIB_PATH = os.path.join(PKG, "libtfl_audit.so")   # test build (include/tfl_audit.h)

LAYER_KEYS = ("w_qkv", "b_qkv", "w_o", "b_o", "ln1_g", "ln1_b",
              "w_1", "b_1", "w_2", "b_2", "ln2_g", "ln2_b")
SYMBOLS = ("tfl_create", "tfl_workspace_bytes", "tfl_forward", "tfl_forward_noalloc", "tfl_destroy",
           "tfl_plan_name", "tfl_plan_path", "tfl_timer_arm", "tfl_timer_read", "tfl_last_error")
STATIC_WORKSPACE_BYTES = 32 << 20   # TFL_STATIC_WORKSPACE_BYTES
STAGES = {"prep": 1, "qkv": 2, "attn": 3, "out": 4, "ln": 5, "ffn1": 6, "ffn2": 7, "fused": 8, "row": 9}

DTYPE_CODES = {"f32": 0, "f16": 1, "bf16": 2}
PATHS = {"auto": 0, "seq": 1, "pq": 2, "tiled": 3, "pq_single": 4}
PATH_NAMES = {v: k for k, v in PATHS.items()}
STATUS = {0: "TFL_OK", 1: "TFL_E_INVALID", 2: "TFL_E_UNSUPPORTED", 3: "TFL_E_WORKSPACE",
          4: "TFL_E_HIP", 5: "TFL_E_INTERNAL"}


class TflConfig(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("d_ffn", ctypes.c_int32), ("batch", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("ln_eps", ctypes.c_float), ("force_path", ctypes.c_int32)]


class TflLayer(ctypes.Structure):
    _fields_ = [(k, ctypes.c_void_p) for k in LAYER_KEYS]


class TflError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


_libs: dict = {}


def load_library(path: str = LIB_PATH):
    """Load libtfl.so (or another build of it); raises when it has not been built."""
    if path in _libs:
        return _libs[path]
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library {path} is not built; run "
                           "`python -m masked_attention_causal_amd.build` (or __graft_entry__.build())")
    # torch ships its own HIP runtime under the same soname as the system one.
    # Importing torch first makes libtfl.so bind to the runtime torch uses;
    # loaded the other way round, the process ends up with two runtimes and
    # every launch fails with "no ROCm-capable device is detected".
    import torch  # noqa: F401
    L = ctypes.CDLL(path)
    vp = ctypes.c_void_p
    L.tfl_create.argtypes = [ctypes.POINTER(TflConfig), ctypes.POINTER(TflLayer), ctypes.POINTER(vp)]
    L.tfl_create.restype = ctypes.c_int
    L.tfl_workspace_bytes.argtypes = [vp, ctypes.POINTER(ctypes.c_size_t)]
    L.tfl_workspace_bytes.restype = ctypes.c_int
    L.tfl_forward.argtypes = [vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.tfl_forward.restype = ctypes.c_int
    if hasattr(L, "tfl_forward_noalloc"):   # absent only from builds that predate it
        L.tfl_forward_noalloc.argtypes = [vp, vp, vp, vp, vp]
        L.tfl_forward_noalloc.restype = ctypes.c_int
    L.tfl_destroy.argtypes = [vp]
    L.tfl_destroy.restype = ctypes.c_int
    L.tfl_plan_name.argtypes = [vp]
    L.tfl_plan_name.restype = ctypes.c_char_p
    L.tfl_plan_path.argtypes = [vp]
    L.tfl_plan_path.restype = ctypes.c_int32
    L.tfl_timer_arm.argtypes = [vp, ctypes.c_int32, ctypes.c_int32]
    L.tfl_timer_arm.restype = ctypes.c_int
    L.tfl_timer_read.argtypes = [vp, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_int32)]
    L.tfl_timer_read.restype = ctypes.c_int
    L.tfl_last_error.argtypes = []
    L.tfl_last_error.restype = ctypes.c_char_p
    if hasattr(L, "tfl_audit_attach"):
        L.tfl_audit_attach.argtypes = [vp]
        L.tfl_audit_attach.restype = ctypes.c_int
    _libs[path] = L
    return L


def _check(st: int, L=None) -> None:
    if st != 0:
        raise TflError(st, (L or load_library()).tfl_last_error().decode())


def make_config(n_layers, d_model, n_heads, d_ffn, batch, seq_len, dtype, ln_eps=0.0, force_path="auto"):
    fp = PATHS[force_path] if isinstance(force_path, str) else int(force_path)
    dt = DTYPE_CODES[dtype] if isinstance(dtype, str) else int(dtype)
    return TflConfig(n_layers, d_model, n_heads, d_ffn, batch, seq_len, dt, ln_eps, fp)


class Handle:
    """A frozen plan over borrowed weight pointers (raw addresses)."""

    def __init__(self, cfg: TflConfig, layer_ptrs: list, lib_path: str = LIB_PATH):
        self._L = L = load_library(lib_path)
        arr = (TflLayer * max(1, len(layer_ptrs)))()
        for i, lp in enumerate(layer_ptrs):
            for k in LAYER_KEYS:
                setattr(arr[i], k, lp[k])
        h = ctypes.c_void_p()
        _check(L.tfl_create(ctypes.byref(cfg), arr, ctypes.byref(h)), L)
        self._h = h
        self.cfg = cfg

    @property
    def workspace_bytes(self) -> int:
        n = ctypes.c_size_t()
        _check(self._L.tfl_workspace_bytes(self._h, ctypes.byref(n)), self._L)
        return n.value

    @property
    def plan_name(self) -> str:
        return self._L.tfl_plan_name(self._h).decode()

    @property
    def plan_path(self) -> str:
        return PATH_NAMES.get(self._L.tfl_plan_path(self._h), "?")

    def forward_raw(self, x: int, lens: int, y: int, ws: int, ws_bytes: int, stream: int) -> None:
        _check(self._L.tfl_forward(self._h, x, lens, y, ws, ws_bytes, stream), self._L)

    def forward_noalloc_raw(self, x: int, lens: int, y: int, stream: int) -> None:
        """tfl_forward_noalloc: the library's static workspace, no allocation."""
        _check(self._L.tfl_forward_noalloc(self._h, x, lens, y, stream), self._L)

    def timer_arm(self, stage: str, max_launches: int) -> None:
        _check(self._L.tfl_timer_arm(self._h, STAGES[stage], int(max_launches)), self._L)

    def timer_read(self):
        """(summed kernel ms, launches) of the armed stage since arming."""
        ms = ctypes.c_float()
        n = ctypes.c_int32()
        _check(self._L.tfl_timer_read(self._h, ctypes.byref(ms), ctypes.byref(n)), self._L)
        return ms.value, n.value

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            self._L.tfl_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def plan_for(n_layers, d_model, n_heads, d_ffn, batch, seq_len, dtype, force_path="auto"):
    """Plan name, path and workspace size for a shape (host only: the layer
    pointers are placeholders that are never dereferenced)."""
    cfg = make_config(n_layers, d_model, n_heads, d_ffn, batch, seq_len, dtype, 0.0, force_path)
    fake = [{k: 0x10000 for k in LAYER_KEYS} for _ in range(n_layers)]
    h = Handle(cfg, fake)
    try:
        return h.plan_name, h.plan_path, h.workspace_bytes
    finally:
        h.close()


class Encoder:
    """Post-LN encoder stack on the GPU.  ``layers`` is a list of dicts of
    torch tensors on the device, in the I/O dtype, nn.Linear layout."""

    def __init__(self, n_layers, d_model, n_heads, d_ffn, batch, seq_len, dtype, layers,
                 ln_eps=0.0, force_path="auto", lib_path: str = LIB_PATH):
        import torch
        self.torch_dtype = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]
        self.dtype = dtype
        self.shape = (batch, seq_len, d_model)
        self._layers = [{k: t.contiguous() for k, t in lw.items()} for lw in layers]
        for lw in self._layers:
            for k in LAYER_KEYS:
                if lw[k].dtype != self.torch_dtype or not lw[k].is_cuda:
                    raise ValueError(f"layer tensor {k} must be a {dtype} device tensor")
        ptrs = [{k: lw[k].data_ptr() for k in LAYER_KEYS} for lw in self._layers]
        cfg = make_config(n_layers, d_model, n_heads, d_ffn, batch, seq_len, dtype, ln_eps, force_path)
        self.handle = Handle(cfg, ptrs, lib_path)
        self._ws = None

    @property
    def plan_name(self) -> str:
        return self.handle.plan_name

    @property
    def plan_path(self) -> str:
        return self.handle.plan_path

    def workspace(self):
        import torch
        n = self.handle.workspace_bytes
        if self._ws is None or self._ws.numel() < n:
            self._ws = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")
        return self._ws

    def forward(self, x, lens, y=None, workspace=None, stream=None):
        import torch
        if tuple(x.shape) != self.shape or x.dtype != self.torch_dtype or not x.is_contiguous():
            raise ValueError(f"x must be a contiguous {self.dtype} tensor of shape {self.shape}")
        if lens.dtype != torch.int32 or lens.numel() != self.shape[0] or not lens.is_cuda:
            raise ValueError("lens must be an int32 device tensor of length batch")
        if y is None:
            y = torch.empty_like(x)
        ws = self.workspace() if workspace is None else workspace
        st = torch.cuda.current_stream() if stream is None else stream
        self.handle.forward_raw(x.data_ptr(), lens.data_ptr(), y.data_ptr(), ws.data_ptr(),
                                ws.numel() * ws.element_size(), st.cuda_stream)
        return y

    __call__ = forward

    def close(self) -> None:
        self.handle.close()


def to_device(a, dtype: str, device="cuda"):
    """Upload a numpy array holding values stored in ``dtype`` (bf16 as raw
    uint16 bits) as a torch tensor of that dtype."""
    import numpy as np
    import torch
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def to_numpy_f64(t):
    """Exact float64 copy of a device tensor."""
    return t.detach().to("cpu", dtype=__import__("torch").float64).numpy()
