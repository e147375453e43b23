"""ctypes binding of libsvdq.so (include/svdq.h).

Argument marshalling only: every step of the layer runs in the library (host
pack, HIP kernels).  PyTorch provides device memory and streams.  The
functions keep the C names; ``SVDQLinear`` bundles a packed layer with its
device blob for convenience.  If the library is not built this module raises
on first use -- there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# SVDQ_LIBRARY selects another build of the same library (the host-sanitizer
# build the CPU tests use); by default the in-tree libsvdq.so
LIB_PATH = os.environ.get("SVDQ_LIBRARY") or os.path.join(_HERE, "libsvdq.so")

FMT_INT4_G64 = 0
FMT_MXFP4_G32 = 1
FMT_INT8_W8A8 = 2
F16 = 0
BF16 = 1
FLAG_GELU = 1
FLAG_UNFUSED_LOWRANK = 2
FLAG_TRACE = 4
MAX_RANK_CAPACITY = 128

FMT_CODES = {"int4_g64": FMT_INT4_G64, "mxfp4_g32": FMT_MXFP4_G32}
DTYPE_CODES = {"f16": F16, "bf16": BF16}
STATUS = {0: "SVDQ_OK", 1: "SVDQ_ERR_INVALID_ARG", 2: "SVDQ_ERR_SHAPE", 3: "SVDQ_ERR_UNSUPPORTED",
          4: "SVDQ_ERR_CAPACITY", 5: "SVDQ_ERR_NUMERIC", 6: "SVDQ_ERR_HIP"}


class SvdqError(RuntimeError):
    def __init__(self, fn: str, code: int):
        self.code = code
        super().__init__(f"{fn} failed: {STATUS.get(code, code)} ({_lib().svdq_status_string(code).decode()})")


class svdq_layer(C.Structure):
    _fields_ = [
        ("K", C.c_int64), ("N", C.c_int64),
        ("rank", C.c_int32), ("rank_active", C.c_int32), ("rank_capacity", C.c_int32),
        ("rank_slots", C.c_int32), ("fmt", C.c_int32), ("dtype", C.c_int32),
        ("has_bias", C.c_int32), ("blob_on_device", C.c_int32),
        ("blob", C.c_void_p), ("blob_bytes", C.c_size_t),
        ("off_invlam", C.c_size_t), ("off_lam", C.c_size_t), ("off_l1x", C.c_size_t),
        ("off_l2", C.c_size_t), ("off_wq", C.c_size_t), ("off_sw", C.c_size_t), ("off_bias", C.c_size_t),
    ]


_P = C.c_void_p
_I64 = C.c_int64
_I = C.c_int
_SZ = C.c_size_t
_LP = C.POINTER(svdq_layer)

# name -> argtypes (restype is the status int unless stated)
_SIGS = {
    "svdq_packed_size": [_I64, _I64, _I, _I, _I, C.POINTER(_SZ)],
    "svdq_pack_weights": [_P, _I64, _I64, _I64, _I, _P, _I, _I, _I, _P, _P, _SZ, _P, _LP],
    "svdq_pack_weights_host": [_P, _I64, _I64, _I64, _I, _P, _I, _I, _I, _P, _P, _SZ, _LP],
    "svdq_pack_weights_ex": [_P, _I64, _I64, _I64, _I, _P, _I, _I, _I, _P, _I, _P, _P, _SZ, _I, _P, _LP],
    "svdq_layer_copy": [_LP, _P, _SZ, _I, _P, _LP],
    "svdq_attach_lora": [_LP, _P, _P, _I, C.c_float, _P],
    "svdq_detach_lora": [_LP, _P],
    "svdq_workspace_size": [_LP, _I64, C.POINTER(_SZ)],
    "svdq_linear_forward": [_LP, _P, _I64, _I64, _P, _I64, _P, _SZ, C.c_uint, _P],
    "svdq_linear_forward_noalloc": [_LP, _P, _I64, _I64, _P, _I64, C.c_uint, _P],
    "svdq_quantize_activations": [_LP, _P, _I64, _I64, _P, _SZ, _P],
    "svdq_gemm_forward": [_LP, _I64, _P, _I64, _P, _SZ, C.c_uint, _P],
    "svdq_activation_absmax": [_P, _I64, _I64, _I64, _I, _P, _P],
    "svdq_layer_export": [_LP, _P, _P, _P, _P, _P, _P, _P, _P],
    "svdq_workspace_export": [_LP, _P, _SZ, _I64, _P, _P, _P, _P],
    "svdq_svd_factors": [_P, _I64, _I64, _I64, _I, _P, _I, _P, _P, _P, _P],
    "svdq_chain_workspace_size": [_LP, _LP, _I64, C.POINTER(_SZ)],
    "svdq_linear_forward_chain": [_LP, _LP, _P, _I64, _I64, _P, _I64, _P, _SZ, _P, _SZ, C.c_uint, _P],
    "svdq_int4_group_partials": [_LP, _P, _SZ, _I64, _I64, _I64, _I64, _I64, _I64, _I64, _P, _P],
    "svdq_probe_clock": [_P, C.POINTER(C.c_double)],
    "svdq_trace_read": [_P, _I, C.POINTER(_I), C.POINTER(C.c_double)],
    "svdq_probe_mfma_rate": [_I, _I, _P, C.POINTER(C.c_double), C.POINTER(C.c_double)],
    "svdq_timing_start": [_I],
    "svdq_timing_stop": [C.POINTER(_I), C.POINTER(C.c_float), _I, C.POINTER(_I)],
}

_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m diffusion_smooth_group_amd.build`")
        lib = C.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = C.c_int
        lib.svdq_status_string.argtypes = [C.c_int]
        lib.svdq_status_string.restype = C.c_char_p
        _LIB = lib
    return _LIB


def lib_handle():
    return _lib()


def _call(name, *args):
    rc = getattr(_lib(), name)(*args)
    if rc != 0:
        raise SvdqError(name, rc)


def _np_ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "host arrays must be C-contiguous"
    return a.ctypes.data_as(C.c_void_p)


def _t_ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is not None:
        return C.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))
    import torch
    if torch.cuda.is_available():
        return C.c_void_p(torch.cuda.current_stream().cuda_stream)
    return C.c_void_p(0)


# ----------------------------------------------------------------- host calls
def packed_size(K, N, rank_capacity, fmt, dtype) -> int:
    out = _SZ(0)
    _call("svdq_packed_size", K, N, rank_capacity, fmt, dtype, C.byref(out))
    return out.value


def pack_weights_host(W_bits: np.ndarray, dtype: int, act_absmax: Optional[np.ndarray], rank: int,
                      rank_capacity: int, fmt: int, bias_bits: Optional[np.ndarray] = None, refine_iters: int = 0,
                      errors: Optional[np.ndarray] = None):
    """Pack into a host blob.  Returns (layer, blob ndarray); the blob must
    outlive the layer.  refine_iters > 0 refines the low-rank split; errors
    (float64 [refine_iters + 1]) receives each round's squared weight error."""
    W_bits = np.ascontiguousarray(W_bits, dtype=np.uint16)
    K, N = W_bits.shape
    a = None if act_absmax is None else np.ascontiguousarray(act_absmax, dtype=np.float32)
    b = None if bias_bits is None else np.ascontiguousarray(bias_bits, dtype=np.uint16)
    nbytes = packed_size(K, N, rank_capacity, fmt, dtype)
    blob = np.zeros(nbytes, np.uint8)
    L = svdq_layer()
    if refine_iters == 0 and errors is None:
        _call("svdq_pack_weights_host", _np_ptr(W_bits), K, N, N, dtype, _np_ptr(a), rank, rank_capacity, fmt,
              _np_ptr(b), _np_ptr(blob), nbytes, C.byref(L))
    else:
        assert errors is None or (errors.dtype == np.float64 and errors.size >= refine_iters + 1)
        _call("svdq_pack_weights_ex", _np_ptr(W_bits), K, N, N, dtype, _np_ptr(a), rank, rank_capacity, fmt,
              _np_ptr(b), refine_iters, _np_ptr(errors), _np_ptr(blob), nbytes, 0, None, C.byref(L))
    return L, blob


def svd_factors(W_bits: np.ndarray, dtype: int, act_absmax: Optional[np.ndarray], rank: int):
    W_bits = np.ascontiguousarray(W_bits, dtype=np.uint16)
    K, N = W_bits.shape
    a = None if act_absmax is None else np.ascontiguousarray(act_absmax, dtype=np.float32)
    L1 = np.zeros((K, max(rank, 1)), np.float64)
    L2 = np.zeros((max(rank, 1), N), np.float64)
    sg = np.zeros(max(rank, 1), np.float64)
    lam = np.zeros(K, np.float32)
    _call("svdq_svd_factors", _np_ptr(W_bits), K, N, N, dtype, _np_ptr(a), rank, _np_ptr(L1), _np_ptr(L2),
          _np_ptr(sg), _np_ptr(lam))
    return L1[:, :rank], L2[:rank], sg[:rank], lam


def layer_export(L: svdq_layer, stream=None):
    K, N, ra = L.K, L.N, L.rank_active
    lam = np.zeros(K, np.float32)
    invlam = np.zeros(K, np.float32)
    l1x = np.zeros((K, max(ra, 1)), np.uint16)
    l2 = np.zeros((max(ra, 1), N), np.uint16)
    codes = np.zeros((K, N), np.uint8 if L.fmt == FMT_MXFP4_G32 else np.int8)
    if L.fmt == FMT_INT8_W8A8:
        scales = np.zeros((1, N), np.float32)
    else:
        G = 64 if L.fmt == FMT_INT4_G64 else 32
        scales = np.zeros((K // G, N), np.uint16 if L.fmt == FMT_INT4_G64 else np.uint8)
    bias = np.zeros(N, np.float32)
    _call("svdq_layer_export", C.byref(L), _np_ptr(lam), _np_ptr(invlam), _np_ptr(l1x), _np_ptr(l2),
          _np_ptr(codes), _np_ptr(scales), _np_ptr(bias), _stream(stream))
    return {"lam": lam, "invlam": invlam, "L1x": l1x[:, :ra], "L2q": l2[:ra], "codes": codes,
            "scales": scales, "bias": bias}


def attach_lora(L: svdq_layer, A_bits: np.ndarray, B_bits: np.ndarray, alpha: float = 1.0, stream=None):
    A_bits = np.ascontiguousarray(A_bits, dtype=np.uint16)
    B_bits = np.ascontiguousarray(B_bits, dtype=np.uint16)
    rL = A_bits.shape[1]
    assert A_bits.shape == (L.K, rL) and B_bits.shape == (rL, L.N)
    _call("svdq_attach_lora", C.byref(L), _np_ptr(A_bits), _np_ptr(B_bits), rL, float(alpha), _stream(stream))


def detach_lora(L: svdq_layer, stream=None):
    _call("svdq_detach_lora", C.byref(L), _stream(stream))


def layer_copy(src: svdq_layer, dst_ptr, dst_bytes: int, on_device: bool, stream=None) -> svdq_layer:
    out = svdq_layer()
    _call("svdq_layer_copy", C.byref(src), dst_ptr, dst_bytes, 1 if on_device else 0, _stream(stream), C.byref(out))
    return out


def workspace_size(L: svdq_layer, M: int) -> int:
    out = _SZ(0)
    _call("svdq_workspace_size", C.byref(L), M, C.byref(out))
    return out.value


# ---------------------------------------------------------------- GPU calls
_TORCH_DT = {F16: "float16", BF16: "bfloat16"}


def torch_dtype(dtype: int):
    import torch
    return getattr(torch, _TORCH_DT[dtype])


def bits_to_device(bits: np.ndarray, dtype: int, device="cuda"):
    """Upload 16-bit bit patterns as a torch tensor of the matching dtype."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.to(device).view(torch_dtype(dtype))


def device_to_bits(t) -> np.ndarray:
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


class SVDQLinear:
    """A packed SVDQuant linear layer resident on the GPU."""

    def __init__(self, layer: svdq_layer, blob):
        self.layer = layer
        self.blob = blob          # torch uint8 tensor holding the packed bytes
        self._ws = None

    @classmethod
    def pack(cls, W_bits: np.ndarray, dtype: int, act_absmax: Optional[np.ndarray], rank: int, fmt: int,
             bias_bits: Optional[np.ndarray] = None, rank_capacity: Optional[int] = None, device="cuda",
             stream=None, refine_iters: int = 0):
        """refine_iters > 0: iterative refinement of the low-rank split (the
        split with the smallest weight error is packed; the squared errors of
        every round land in .refine_errors)."""
        import torch
        W_bits = np.ascontiguousarray(W_bits, dtype=np.uint16)
        K, N = W_bits.shape
        cap = rank if rank_capacity is None else rank_capacity
        nbytes = packed_size(K, N, cap, fmt, dtype)
        blob = torch.empty(nbytes, dtype=torch.uint8, device=device)
        a = None if act_absmax is None else np.ascontiguousarray(act_absmax, dtype=np.float32)
        b = None if bias_bits is None else np.ascontiguousarray(bias_bits, dtype=np.uint16)
        L = svdq_layer()
        if refine_iters == 0:
            _call("svdq_pack_weights", _np_ptr(W_bits), K, N, N, dtype, _np_ptr(a), rank, cap, fmt, _np_ptr(b),
                  _t_ptr(blob), nbytes, _stream(stream), C.byref(L))
            errors = None
        else:
            errors = np.zeros(refine_iters + 1, np.float64)
            _call("svdq_pack_weights_ex", _np_ptr(W_bits), K, N, N, dtype, _np_ptr(a), rank, cap, fmt, _np_ptr(b),
                  refine_iters, _np_ptr(errors), _t_ptr(blob), nbytes, 1, _stream(stream), C.byref(L))
        lin = cls(L, blob)
        lin.refine_errors = errors
        return lin

    @property
    def K(self):
        return self.layer.K

    @property
    def N(self):
        return self.layer.N

    def workspace(self, M: int):
        import torch
        need = workspace_size(self.layer, M)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.blob.device)
        return self._ws

    def forward(self, X, gelu: bool = False, Y=None, ws=None, stream=None, unfused: bool = False):
        """unfused=True runs the low-rank branch as separate passes (the
        baseline the fused kernels are measured against)."""
        import torch
        assert X.dim() == 2 and X.shape[1] == self.K and X.stride(1) == 1
        M = X.shape[0]
        if Y is None:
            Y = torch.empty((M, self.N), dtype=X.dtype, device=X.device)
        ws = self.workspace(M) if ws is None else ws
        flags = (FLAG_GELU if gelu else 0) | (FLAG_UNFUSED_LOWRANK if unfused else 0)
        _call("svdq_linear_forward", C.byref(self.layer), _t_ptr(X), M, X.stride(0), _t_ptr(Y), Y.stride(0),
              _t_ptr(ws), ws.numel(), flags, _stream(stream))
        return Y

    __call__ = forward

    def quantize_activations(self, X, ws=None, stream=None):
        M = X.shape[0]
        ws = self.workspace(M) if ws is None else ws
        _call("svdq_quantize_activations", C.byref(self.layer), _t_ptr(X), M, X.stride(0), _t_ptr(ws), ws.numel(),
              _stream(stream))
        return ws

    def gemm(self, M: int, Y, ws, gelu: bool = False, stream=None):
        _call("svdq_gemm_forward", C.byref(self.layer), M, _t_ptr(Y), Y.stride(0), _t_ptr(ws), ws.numel(),
              FLAG_GELU if gelu else 0, _stream(stream))
        return Y

    def forward_chain(self, nxt: "SVDQLinear", X, gelu: bool = False, Y=None, ws=None, ws_next=None,
                      stream=None):
        """Run this layer on X with nxt's activation pass in the GEMM
        epilogue.  Returns ws_next (nxt's codes, scales and T); finish with
        nxt.gemm(M, Y2, ws_next).  Y: optional output of this layer."""
        import torch
        assert X.dim() == 2 and X.shape[1] == self.K and X.stride(1) == 1
        M = X.shape[0]
        out = _SZ(0)
        _call("svdq_chain_workspace_size", C.byref(self.layer), C.byref(nxt.layer), M, C.byref(out))
        if ws is None:
            ws = torch.empty(out.value, dtype=torch.uint8, device=X.device)
        if ws_next is None:
            ws_next = nxt.workspace(M)
        _call("svdq_linear_forward_chain", C.byref(self.layer), C.byref(nxt.layer), _t_ptr(X), M, X.stride(0),
              _t_ptr(Y), Y.stride(0) if Y is not None else 0, _t_ptr(ws), ws.numel(),
              _t_ptr(ws_next), ws_next.numel(), FLAG_GELU if gelu else 0, _stream(stream))
        return ws_next

    def workspace_export(self, M: int, ws=None, stream=None):
        ws = self._ws if ws is None else ws
        K, ra, fmt = self.layer.K, self.layer.rank_active, self.layer.fmt
        codes = np.zeros((M, K), np.uint8 if fmt == FMT_MXFP4_G32 else np.int8)
        if fmt == FMT_INT8_W8A8:
            scales = np.zeros((M, 1), np.float32)
        else:
            G = 64 if fmt == FMT_INT4_G64 else 32
            scales = np.zeros((M, K // G), np.uint16 if fmt == FMT_INT4_G64 else np.uint8)
        t = np.zeros((M, max(ra, 1)), np.uint16)
        _call("svdq_workspace_export", C.byref(self.layer), _t_ptr(ws), ws.numel(), M, _np_ptr(codes),
              _np_ptr(scales), _np_ptr(t), _stream(stream))
        return {"codes": codes, "scales": scales, "T": t[:, :ra]}

    def int4_group_partials(self, M: int, m0: int, nm: int, n0: int, nn: int, g0: int, ng: int, ws=None,
                            stream=None):
        import torch
        ws = self._ws if ws is None else ws
        out = torch.empty((ng, nm, nn), dtype=torch.int32, device=self.blob.device)
        _call("svdq_int4_group_partials", C.byref(self.layer), _t_ptr(ws), ws.numel(), M, m0, nm, n0, nn, g0, ng,
              _t_ptr(out), _stream(stream))
        return out

    def attach_lora(self, A_bits, B_bits, alpha=1.0, stream=None):
        attach_lora(self.layer, A_bits, B_bits, alpha, stream)

    def detach_lora(self, stream=None):
        detach_lora(self.layer, stream)

    def export(self, stream=None):
        return layer_export(self.layer, stream)


def trace_read(max_records: int = 65536):
    """Per-workgroup records of the last traced GEMM: (start wall ticks,
    start shader cycles, end wall ticks, end shader cycles) as uint64 [n, 4],
    and the wall-clock rate in Hz."""
    n = C.c_int()
    hz = C.c_double()
    buf = np.zeros((max_records, 4), dtype=np.uint64)
    _call("svdq_trace_read", _np_ptr(buf), int(max_records), C.byref(n), C.byref(hz))
    return buf[:min(n.value, max_records)].copy(), hz.value


def probe_clock(stream=None) -> float:
    """Shader clock right now (MHz), measured on every compute unit."""
    v = C.c_double()
    _call("svdq_probe_clock", _stream(stream), C.byref(v))
    return v.value


def probe_mfma_rate(random_operands: bool, iters: int = 2000, stream=None):
    """Sustained scaled-FP4 MFMA rate (TFLOP/s) and mean clock (MHz)."""
    t, m = C.c_double(), C.c_double()
    _call("svdq_probe_mfma_rate", 1 if random_operands else 0, int(iters), _stream(stream), C.byref(t), C.byref(m))
    return t.value, m.value


def activation_absmax(X, dtype: int, out=None, stream=None):
    """Per-channel running max |X| on the GPU (calibration statistic)."""
    import torch
    M, K = X.shape
    if out is None:
        out = torch.zeros(K, dtype=torch.float32, device=X.device)
    _call("svdq_activation_absmax", _t_ptr(X), M, K, X.stride(0), dtype, _t_ptr(out), _stream(stream))
    return out


KERNEL_ACT, KERNEL_GEMM, KERNEL_OTHER = 1, 2, 3


def timing_start(capacity: int):
    """Time the calling thread's next `capacity` kernel launches from their
    own dispatch timestamps (svdq_timing_stop returns them)."""
    _call("svdq_timing_start", int(capacity))


def timing_stop(max_launches: int = 1 << 16):
    """Kinds (KERNEL_*) and durations in microseconds of the launches timed
    since timing_start, in launch order."""
    kinds = np.zeros(max_launches, dtype=np.int32)
    ms = np.zeros(max_launches, dtype=np.float32)
    n = C.c_int()
    _call("svdq_timing_stop", kinds.ctypes.data_as(C.POINTER(C.c_int)), ms.ctypes.data_as(C.POINTER(C.c_float)),
          int(max_launches), C.byref(n))
    k = min(n.value, max_launches)
    return kinds[:k].copy(), ms[:k].astype(np.float64) * 1e3
