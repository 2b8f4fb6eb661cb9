"""ctypes binding of liblq (include/lq.h): argument marshalling only.

Every function here passes device pointers, sizes and the current HIP stream
of torch to the C ABI; all arithmetic of the layer runs in the library's HIP
kernels.  Importing this module opens ``liblq.so`` next to it and raises if
the library is missing -- there is no fallback.

Packed weights are held in torch.int32 tensors (the same 32 bits as the ABI's
uint32 words).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblq.so")

LQ_F32, LQ_F16, LQ_BF16 = 0, 1, 2
STATUS = {0: "LQ_OK", 1: "LQ_ERR_NULL", 2: "LQ_ERR_SHAPE", 3: "LQ_ERR_DTYPE", 4: "LQ_ERR_ALIGN",
          5: "LQ_ERR_UNSUPPORTED", 6: "LQ_ERR_HIP", 7: "LQ_ERR_WORKSPACE"}

EXPORTS = ("lq_status_string", "lq_last_error", "lq_version", "lq_pack_signs", "lq_unpack_signs",
           "lq_lift_activations", "lq_lift_kron_workspace_size", "lq_lift_kron",
           "lq_gemv_workspace_size", "lq_workspace_clear", "lq_gemv", "lq_gemm",
           "lq_encode_workspace_size", "lq_encode", "lq_softmin_workspace_size",
           "lq_softmin_grad", "lq_adam_update", "lq_gemm_decoded_workspace_size",
           "lq_gemm_decoded", "lq_layer_b1_workspace_size", "lq_layer_b1",
           "lq_gemv_noalloc", "lq_stream_read", "lq_lift_parts_size", "lq_lift_parts",
           "lq_gemv_parts_workspace_size", "lq_gemv_parts")

_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_vp = ctypes.c_void_p
_sz = ctypes.c_size_t


class LQError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m bit_lifted_gemv_amd.build`")
    lib = ctypes.CDLL(path)
    sig = {
        "lq_status_string": (ctypes.c_char_p, [_i32]),
        "lq_last_error": (ctypes.c_char_p, []),
        "lq_version": (ctypes.c_char_p, []),
        "lq_pack_signs": (_i32, [_vp, _i64, _i64, _i64, _vp, _i64, _vp]),
        "lq_unpack_signs": (_i32, [_vp, _i64, _i64, _i64, _vp, _i64, _vp]),
        "lq_lift_activations": (_i32, [_vp, _i32, _i64, _i64, _vp, _i32, _i32, _vp, _i32, _i32,
                                       _vp, _i32, _vp]),
        "lq_lift_kron_workspace_size": (_i32, [_i64, _i64, ctypes.POINTER(_sz)]),
        "lq_lift_kron": (_i32, [_vp, _i32, _i64, _i64, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _i32,
                                _vp, _i32, _vp, _sz, _vp]),
        "lq_gemv_workspace_size": (_i32, [_i64, _i64, _i64, ctypes.POINTER(_sz)]),
        "lq_workspace_clear": (_i32, [_vp, _sz, _vp]),
        "lq_gemv": (_i32, [_vp, _i64, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _sz, _vp]),
        "lq_gemm": (_i32, [_vp, _i64, _i64, _i64, _vp, _vp, _i32, _i64, _vp, _vp]),
        "lq_gemv_noalloc": (_i32, [_vp, _i64, _i64, _i64, _vp, _vp, _i64, _vp, _vp]),
        "lq_stream_read": (_i32, [_vp, _sz, _vp, _vp]),
        "lq_lift_parts_size": (_i32, [_i64, ctypes.POINTER(_sz)]),
        "lq_lift_parts": (_i32, [_vp, _i32, _i64, _i64, _vp, _i32, _i32, _vp, _i32, _i32, _vp,
                                 _sz, _vp]),
        "lq_gemv_parts_workspace_size": (_i32, [_i64, _i64, _i64, ctypes.POINTER(_sz)]),
        "lq_gemv_parts": (_i32, [_vp, _i64, _i64, _i64, _vp, _vp, _sz, _i64, _vp, _vp, _sz, _vp]),
        "lq_encode_workspace_size": (_i32, [_i32, _i32, ctypes.POINTER(_sz)]),
        "lq_encode": (_i32, [_vp, _i64, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _sz, _vp]),
        "lq_softmin_workspace_size": (_i32, [_i64, _i32, _i32, ctypes.POINTER(_sz)]),
        "lq_gemm_decoded_workspace_size": (_i32, [_i64, _i64, ctypes.POINTER(_sz)]),
        "lq_layer_b1_workspace_size": (_i32, [_i64, _i64, _i32, _i32, ctypes.POINTER(_sz)]),
        "lq_layer_b1": (_i32, [_vp, _i32, _i64, _vp, _i32, _i32, _vp, _i32, _i32, _vp, _i64, _i64,
                               _vp, _vp, _vp, _sz, _vp]),
        "lq_gemm_decoded": (_i32, [_vp, _i64, _i64, _i64, _vp, _i32, _i32, _vp, _vp, _i32, _i64,
                                   _vp, _vp, _sz, _vp]),
        "lq_softmin_grad": (_i32, [_vp, _i64, _vp, _i32, _i32, ctypes.c_float, _vp, _vp, _vp,
                                   _sz, _vp]),
        "lq_adam_update": (_i32, [_vp, _vp, _vp, _vp, _i64, _i32, ctypes.c_float,
                                  ctypes.c_float, ctypes.c_float, ctypes.c_float, _vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_LIB: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        _LIB = load_library()
    return _LIB


def check(status: int) -> None:
    if status != 0:
        raise LQError(status, lib().lq_last_error().decode())


# ----------------------------------------------------------------- helpers
def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return LQ_F32
    if t.dtype == torch.float16:
        return LQ_F16
    if t.dtype == torch.bfloat16:
        return LQ_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _torch_dt(code: int) -> torch.dtype:
    return {LQ_F32: torch.float32, LQ_F16: torch.float16, LQ_BF16: torch.bfloat16}[code]


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dev(*ts: torch.Tensor) -> None:
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _stream(stream=None) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


# ----------------------------------------------------------------- C ABI wrappers
def pack_signs(signs: torch.Tensor, ldw: Optional[int] = None, stream=None) -> torch.Tensor:
    """int8 signs [rows][K] -> int32 words [rows][ldw] (LSB-first, bit 1 = positive)."""
    _dev(signs)
    rows, K = signs.shape
    ldw = (K + 31) // 32 if ldw is None else ldw
    out = torch.empty((rows, ldw), dtype=torch.int32, device=signs.device)
    check(lib().lq_pack_signs(_ptr(signs), rows, K, K, _ptr(out), ldw, _stream(stream)))
    return out


def unpack_signs(packed: torch.Tensor, K: int, stream=None) -> torch.Tensor:
    _dev(packed)
    rows, ldw = packed.shape
    out = torch.empty((rows, K), dtype=torch.int8, device=packed.device)
    check(lib().lq_unpack_signs(_ptr(packed), rows, K, ldw, _ptr(out), K, _stream(stream)))
    return out


def lift(a: torch.Tensor, t_inv: torch.Tensor, M: torch.Tensor, d: int, D: int,
         out_dtype: torch.dtype = torch.float32, t_block: int = 128,
         out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """a [B][n], t_inv [n/128][128][128], M float [d][D] -> a_lift [B][n*D/d]."""
    _dev(a, t_inv, M)
    B, n = a.shape
    K = n // d * D
    if out is None:
        out = torch.empty((B, K), dtype=out_dtype, device=a.device)
    check(lib().lq_lift_activations(_ptr(a), _dt(a), B, n, _ptr(t_inv), _dt(t_inv), t_block,
                                    _ptr(M), d, D, _ptr(out), _dt(out), _stream(stream)))
    return out


def lift_parts_size(K: int) -> int:
    n = _sz(0)
    check(lib().lq_lift_parts_size(K, ctypes.byref(n)))
    return n.value


def lift_parts(a: torch.Tensor, t_inv: torch.Tensor, M: torch.Tensor, d: int, D: int,
               t_block: int = 128, out: Optional[torch.Tensor] = None,
               stream=None) -> torch.Tensor:
    """a [B][n] and t_inv of one 16-bit type, M float [d][D] -> the operand
    image of lq_gemv_parts (uint8, lq_lift_parts_size(n*D/d) bytes)."""
    _dev(a, t_inv, M)
    B, n = a.shape
    nb = lift_parts_size(n // d * D)
    if out is None:
        out = torch.empty(nb, dtype=torch.uint8, device=a.device)
    check(lib().lq_lift_parts(_ptr(a), _dt(a), B, n, _ptr(t_inv), _dt(t_inv), t_block, _ptr(M),
                              d, D, _ptr(out), out.numel() * out.element_size(),
                              _stream(stream)))
    return out


def lift_kron(a: torch.Tensor, s1: torch.Tensor, p1_inv: torch.Tensor, p2_inv: torch.Tensor,
              s2: torch.Tensor, M: torch.Tensor, d: int, D: int,
              out_dtype: torch.dtype = torch.float32, out: Optional[torch.Tensor] = None,
              stream=None) -> torch.Tensor:
    """a [B][n], Kronecker whitening factors (float32: s1 [n], P1^-1 [n1][n1],
    P2^-1 [n2][n2], s2 [n/d]), M float [d][D] -> a_lift [B][n*D/d]."""
    _dev(a, s1, p1_inv, p2_inv, s2, M)
    B, n = a.shape
    n1 = p1_inv.shape[0]
    K = n // d * D
    if out is None:
        out = torch.empty((B, K), dtype=out_dtype, device=a.device)
    nb = _sz(0)
    check(lib().lq_lift_kron_workspace_size(B, n, ctypes.byref(nb)))
    ws = workspace(nb.value, a.device, -1, stream)
    check(lib().lq_lift_kron(_ptr(a), _dt(a), B, n, n1, _ptr(s1), _ptr(p1_inv), _ptr(p2_inv),
                             _ptr(s2), _ptr(M), d, D, _ptr(out), _dt(out), _ptr(ws), nb.value,
                             _stream(stream)))
    return out


def encode(w: torch.Tensor, M: torch.Tensor, A: Optional[torch.Tensor] = None,
           codes: Optional[torch.Tensor] = None, err: Optional[torch.Tensor] = None,
           stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Lattice codes of float32 weight groups w [G][d] under M [d][D]:
    exhaustive when A is None, else the auxiliary-vector search with the
    completion A [D-d][D].  Returns (codes int8 [G][D], err float32 [G])."""
    _dev(w, M)
    G, d = w.shape
    D = M.shape[1]
    if codes is None:
        codes = torch.empty((G, D), dtype=torch.int8, device=w.device)
    if err is None:
        err = torch.empty((G,), dtype=torch.float32, device=w.device)
    ws, nbytes = None, 0
    if A is not None:
        _dev(A)
        if A.numel() == 0:    # D == d: A has no rows; any non-null pointer selects the search
            A = torch.zeros(1, dtype=torch.float32, device=w.device)
        nb = _sz(0)
        check(lib().lq_encode_workspace_size(d, D, ctypes.byref(nb)))
        nbytes = nb.value
        ws = workspace(nbytes, w.device, -2, stream)
    check(lib().lq_encode(_ptr(w), G, _ptr(M), _ptr(A), d, D, _ptr(codes), _ptr(err), _ptr(ws),
                          nbytes, _stream(stream)))
    return codes, err


def layer_b1(a: torch.Tensor, t_inv: torch.Tensor, M: torch.Tensor, d: int, D: int,
             w_packed: torch.Tensor, s: torch.Tensor, out: Optional[torch.Tensor] = None,
             stream=None) -> torch.Tensor:
    """The whole layer for one token (a [n] or [1][n]): lift inside the
    one-token product; out float32 [1][m]."""
    _dev(a, t_inv, M, w_packed, s)
    n = a.shape[-1]
    m, ldw = w_packed.shape
    if out is None:
        out = torch.empty((1, m), dtype=torch.float32, device=a.device)
    nb = _sz(0)
    check(lib().lq_layer_b1_workspace_size(m, n, d, D, ctypes.byref(nb)))
    ws = workspace(nb.value, a.device, m, stream) if nb.value else None
    check(lib().lq_layer_b1(_ptr(a), _dt(a), n, _ptr(t_inv), _dt(t_inv), 128, _ptr(M), d, D,
                            _ptr(w_packed), m, ldw, _ptr(s), _ptr(out), _ptr(ws), nb.value,
                            _stream(stream)))
    return out


def gemm_decoded(w_packed: torch.Tensor, s: torch.Tensor, M: torch.Tensor, d: int, D: int,
                 u: torch.Tensor, out: Optional[torch.Tensor] = None,
                 stream=None) -> torch.Tensor:
    """out [B][m] = s * (W_hat @ u^T) with W_hat decoded from the signs and M
    (float16 u [B][n], the whitened activations)."""
    _dev(w_packed, s, M, u)
    m, ldw = w_packed.shape
    B, n = u.shape
    if out is None:
        out = torch.empty((B, m), dtype=torch.float32, device=u.device)
    nb = _sz(0)
    check(lib().lq_gemm_decoded_workspace_size(m, n, ctypes.byref(nb)))
    ws = workspace(nb.value, u.device, -4, stream) if nb.value else None
    check(lib().lq_gemm_decoded(_ptr(w_packed), m, n, ldw, _ptr(M), d, D, _ptr(s), _ptr(u),
                                _dt(u), B, _ptr(out), _ptr(ws) if ws is not None else None,
                                nb.value, _stream(stream)))
    return out


def softmin_grad(w: torch.Tensor, M: torch.Tensor, T: float = 10.0,
                 loss: Optional[torch.Tensor] = None, grad: Optional[torch.Tensor] = None,
                 stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Soft-argmin objective of samples w [N][d] under M [d][D] and its
    gradient: (loss float32 [1], grad float32 [d][D]), both on the device."""
    _dev(w, M)
    N, d = w.shape
    D = M.shape[1]
    if loss is None:
        loss = torch.empty((1,), dtype=torch.float32, device=w.device)
    if grad is None:
        grad = torch.empty((d, D), dtype=torch.float32, device=w.device)
    nb = _sz(0)
    check(lib().lq_softmin_workspace_size(N, d, D, ctypes.byref(nb)))
    ws = workspace(nb.value, w.device, -3, stream)
    check(lib().lq_softmin_grad(_ptr(w), N, _ptr(M), d, D, float(T), _ptr(loss), _ptr(grad),
                                _ptr(ws), nb.value, _stream(stream)))
    return loss, grad


def adam_update(M: torch.Tensor, grad: torch.Tensor, m1: torch.Tensor, m2: torch.Tensor,
                step: int, lr: float, beta1: float = 0.9, beta2: float = 0.999,
                eps: float = 1e-8, stream=None) -> None:
    """One Adam step on M in place (m1, m2: moment buffers, zero at step 1)."""
    _dev(M, grad, m1, m2)
    check(lib().lq_adam_update(_ptr(M), _ptr(grad), _ptr(m1), _ptr(m2), M.numel(), step,
                               float(lr), float(beta1), float(beta2), float(eps),
                               _stream(stream)))


def learn_m(M0: torch.Tensor, batches, T: float = 10.0, lr: float = 0.01,
            stream=None) -> Tuple[torch.Tensor, list]:
    """Adam on the soft-argmin objective from M0, one step per batch of
    samples (float32 [N][d] device tensors drawn by the caller).  Returns
    (M, the per-step loss tensors)."""
    M = M0.detach().clone().contiguous()
    m1 = torch.zeros_like(M)
    m2 = torch.zeros_like(M)
    grad = torch.empty_like(M)
    losses = []
    for i, w in enumerate(batches, start=1):
        loss, _ = softmin_grad(w, M, T, grad=grad, stream=stream)
        adam_update(M, grad, m1, m2, i, lr, stream=stream)
        losses.append(loss)
    return M, losses


_WS = {}


def workspace(nbytes: int, device: torch.device, tag: int = 0, stream=None) -> torch.Tensor:
    """A workspace of at least nbytes, cached per (device, stream, tag) and
    grown on demand, zero-filled when allocated.  Calls on one stream run in
    order, so they may share it; calls on different streams get their own.
    The GEMV uses its row count as tag, the Kronecker lift -1, the encoder -2,
    the soft-argmin objective -3, the decode-weights product -4, the GEMV on
    the parts image -5."""
    key = (device.type, device.index, _stream(stream), tag)
    ws = _WS.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _WS[key] = ws
    return ws


def gemv_workspace_size(m: int, K: int, B: int) -> int:
    n = _sz(0)
    check(lib().lq_gemv_workspace_size(m, K, B, ctypes.byref(n)))
    return n.value


def gemv(w_packed: torch.Tensor, s: torch.Tensor, a_lift: torch.Tensor, K: Optional[int] = None,
         out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """out [B][m] = s * (sigma @ a_lift^T), float32 lifted activations, 1 <= B <= 16."""
    _dev(w_packed, s, a_lift)
    m, ldw = w_packed.shape
    B, Ka = a_lift.shape
    K = Ka if K is None else K
    if K != Ka:
        raise ValueError(f"K={K} differs from the lifted activations' row length {Ka}")
    if out is None:
        out = torch.empty((B, m), dtype=torch.float32, device=a_lift.device)
    nws = gemv_workspace_size(m, K, B)
    ws = workspace(nws, a_lift.device, m, stream) if nws else None
    check(lib().lq_gemv(_ptr(w_packed), m, K, ldw, _ptr(s), _ptr(a_lift), B, _ptr(out), _ptr(ws),
                        nws, _stream(stream)))
    return out


def gemv_parts(w_packed: torch.Tensor, s: torch.Tensor, parts: torch.Tensor, K: int, B: int,
               out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """out [B][m] = s * (sigma @ a_hat^T) from the image of lift_parts."""
    _dev(w_packed, s, parts)
    m, ldw = w_packed.shape
    if out is None:
        out = torch.empty((B, m), dtype=torch.float32, device=parts.device)
    n = _sz(0)
    check(lib().lq_gemv_parts_workspace_size(m, K, B, ctypes.byref(n)))
    ws = workspace(n.value, parts.device, -5, stream)
    check(lib().lq_gemv_parts(_ptr(w_packed), m, K, ldw, _ptr(s), _ptr(parts),
                              parts.numel() * parts.element_size(), B, _ptr(out), _ptr(ws),
                              n.value, _stream(stream)))
    return out


def gemv_noalloc(w_packed: torch.Tensor, s: torch.Tensor, a_lift: torch.Tensor,
                 out: torch.Tensor, stream=None) -> torch.Tensor:
    """lq_gemv without a workspace (the library's per-GPU scratch; calls on
    one GPU must not overlap); out [B][m] float32 must be given."""
    _dev(w_packed, s, a_lift, out)
    m, ldw = w_packed.shape
    B, K = a_lift.shape
    check(lib().lq_gemv_noalloc(_ptr(w_packed), m, K, ldw, _ptr(s), _ptr(a_lift), B, _ptr(out),
                                _stream(stream)))
    return out


def stream_read(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Read every byte of buf once (the HBM read-rate reference); sink: a
    device int32 tensor of at least 4 x compute units."""
    _dev(buf, sink)
    check(lib().lq_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                               _stream(stream)))


def gemm(w_packed: torch.Tensor, s: torch.Tensor, a_lift: torch.Tensor, K: Optional[int] = None,
         out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """out [B][m] on the matrix cores; a_lift float16 or bfloat16 [B][K]."""
    _dev(w_packed, s, a_lift)
    m, ldw = w_packed.shape
    B, Ka = a_lift.shape
    K = Ka if K is None else K
    if K != Ka:
        raise ValueError(f"K={K} differs from the lifted activations' row length {Ka}")
    if out is None:
        out = torch.empty((B, m), dtype=torch.float32, device=a_lift.device)
    check(lib().lq_gemm(_ptr(w_packed), m, K, ldw, _ptr(s), _ptr(a_lift), _dt(a_lift), B,
                        _ptr(out), _stream(stream)))
    return out


# ----------------------------------------------------------------- layer
class DeviceLayer:
    """A layer's stored arrays resident on the GPU (uploaded once)."""

    def __init__(self, packed, M, t_inv, s, d: int, D: int, n: int, act_dtype: str,
                 device="cuda"):
        import numpy as np
        self.d, self.D, self.n = d, D, n
        self.K = n // d * D
        self.m = packed.shape[0]
        self.act_dtype = act_dtype
        self.w = torch.from_numpy(np.ascontiguousarray(packed).view(np.int32)).to(device)
        self.M = torch.from_numpy(np.ascontiguousarray(M, dtype=np.float32)).to(device)
        self.t_inv = to_torch_16(t_inv, act_dtype).to(device)
        self.s = torch.from_numpy(np.ascontiguousarray(s, dtype=np.float32)).to(device)

    @classmethod
    def from_synth(cls, L, device="cuda") -> "DeviceLayer":
        return cls(L.packed, L.M, L.t_inv, L.s, L.d, L.D, L.n, L.dtype, device)

    def _parts_ok(self, a: torch.Tensor) -> bool:
        """The lift into the GEMV's operand image takes a and T^-1 of one
        16-bit type and d in {4, 8, 16, 32}."""
        return (a.dtype in (torch.float16, torch.bfloat16) and a.dtype == self.t_inv.dtype
                and self.d in (4, 8, 16, 32) and self.d <= self.D <= 256)

    def forward(self, a: torch.Tensor, gemm_dtype: torch.dtype = torch.float16,
                path: str = "auto") -> torch.Tensor:
        """o [B][m]: lift then the GEMV (B <= 16) or the GEMM (larger B), the
        faster paths at the workload shapes (6 - 16 tokens: the lift into the
        GEMV's operand image, when it takes the shape).  Paths: "gemv" / "gemm" force
        those; "fused" the one-token layer with the lift inside the GEMV
        (lq_layer_b1); "decoded" u = T^-1 a (the lift with M = I_4) then the
        decode-weights product; "parts" the lift into the GEMV's float8-part
        operand image, then the GEMV on it (lq_lift_parts, lq_gemv_parts)."""
        B = a.shape[0]
        if path == "fused":
            return layer_b1(a, self.t_inv, self.M, self.d, self.D, self.w, self.s)
        if path == "decoded":
            eye = torch.eye(4, dtype=torch.float32, device=a.device)
            u = lift(a, self.t_inv, eye, 4, 4, out_dtype=torch.float16)
            return gemm_decoded(self.w, self.s, self.M, self.d, self.D, u)
        if path == "auto" and 6 <= B <= 16 and self._parts_ok(a):
            path = "parts"
        if path == "parts":
            img = lift_parts(a, self.t_inv, self.M, self.d, self.D)
            return gemv_parts(self.w, self.s, img, self.K, B)
        use_gemm = path == "gemm" or (path == "auto" and B > 16)
        if use_gemm:
            al = lift(a, self.t_inv, self.M, self.d, self.D, out_dtype=gemm_dtype)
            return gemm(self.w, self.s, al, self.K)
        al = lift(a, self.t_inv, self.M, self.d, self.D, out_dtype=torch.float32)
        return gemv(self.w, self.s, al, self.K)


def to_torch_16(x, dtype: str) -> torch.Tensor:
    """Host array in storage format (float16, or bf16 bits as uint16) -> torch CPU tensor."""
    import numpy as np
    x = np.ascontiguousarray(x)
    if dtype == "f16":
        return torch.from_numpy(x.astype(np.float16))
    if dtype == "bf16":
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16)
    if dtype == "f32":
        return torch.from_numpy(x.astype(np.float32))
    raise ValueError(dtype)
