"""ctypes binding of libmoe_anyprec.so (argument marshalling only).

Every function mirrors one C entry point of include/moe_anyprec.h: it checks
that the torch tensors it is given live on the GPU with the expected dtype and
contiguity, passes their device pointers and the current HIP stream, and
raises MoeError on a non-zero status.  No step of the layer is computed here;
there is no fallback when the library is missing."""
from __future__ import annotations

import ctypes
import os
import re
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_anyprec.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "moe_anyprec.h")

STATUS = {0: "MOE_OK", 1: "MOE_ERR_NULL", 2: "MOE_ERR_SHAPE", 3: "MOE_ERR_ALIGN", 4: "MOE_ERR_RANGE",
          5: "MOE_ERR_WORKSPACE", 6: "MOE_ERR_UNSUPPORTED", 7: "MOE_ERR_HIP"}


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({detail})")


class ExpertBankC(ctypes.Structure):
    _fields_ = [("n_experts", ctypes.c_int32), ("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("group", ctypes.c_int32), ("b_max", ctypes.c_int32),
                ("w13_planes", ctypes.c_void_p), ("w13_sz", ctypes.c_void_p),
                ("w2_planes", ctypes.c_void_p), ("w2_sz", ctypes.c_void_p), ("plane_prefix", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m dynamic_any_precision_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
        bp = ctypes.POINTER(ExpertBankC)
        sig = {
            "moe_route_workspace_bytes": (sz, [i32, i32]),
            "moe_route": (i32, [vp, i32, i32, vp, i32, vp, i32, i32, vp, vp, vp, sz, vp]),
            "moe_alloc_bits": (i32, [vp, i32, i32, i32, f32, vp, vp, vp, vp]),
            "moe_budget_pairs": (i32, [i32, i32, i32, f32]),
            "moe_ffn_workspace_bytes": (sz, [bp, bp, i32, i32]),
            "moe_anyprec_ffn": (i32, [bp, bp, vp, i32, i32, vp, vp, vp, vp, i32, vp, sz, vp]),
            "moe_permute": (i32, [vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, sz, vp]),
            "moe_layer_workspace_bytes": (sz, [bp, bp, i32, i32]),
            "moe_layer": (i32, [bp, bp, vp, i32, i32, vp, vp, i32, i32, f32, vp, vp, vp, vp, i32, vp, sz, vp]),
            "moe_dequant": (i32, [bp, i32, i32, i32, vp, vp]),
            "moe_layer_static_scratch_bytes": (sz, []),
            "moe_layer_static": (i32, [bp, bp, vp, i32, i32, vp, vp, i32, i32, f32, vp, vp, vp, vp, i32, vp]),
            "moe_residual_to_bf16": (i32, [vp, vp, i64, vp]),
            "moe_rmsnorm_to_bf16": (i32, [vp, vp, i32, i32, f32, vp]),
            "moe_bits_from_threshold": (i32, [vp, i32, f32, i32, i32, vp, vp]),
            "moe_bits_from_threshold_device": (i32, [vp, i32, vp, i32, i32, vp, vp]),
            "moe_stream_read": (i32, [vp, i64, vp, vp]),
            "moe_duorate_bake": (i32, [bp, vp, vp]),
            "moe_duorate_profile": (i32, [vp, i32, i32, vp, i32, i32, vp, vp, vp]),
            "moe_duorate_solve": (i32, [vp, vp, vp, i32, i32, i32, i32, f32, vp, vp, vp, vp]),
            "moe_bits_from_expert_widths": (i32, [vp, i32, vp, i32, vp, vp]),
            "moe_dpa_residuals_workspace_bytes": (sz, [bp]),
            "moe_dpa_residuals": (i32, [bp, vp, vp, sz, vp]),
            "moe_dpa_alloc_workspace_bytes": (sz, [i32, i32, i32]),
            "moe_dpa_alloc": (i32, [vp, vp, i32, vp, i32, i32, i32, f32, vp, vp, vp, sz, vp]),
            "moe_status_string": (ctypes.c_char_p, [i32]),
            "moe_last_hip_error": (i32, []),
            "moe_set_kernel_events": (None, [vp, vp, vp, vp]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def header_functions() -> list:
    """Names of the functions declared in include/moe_anyprec.h."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def _check(status: int, where: str):
    if status != 0:
        detail = lib().moe_status_string(status).decode()
        if status == 7:
            detail += f", hipError={lib().moe_last_hip_error()}"
        raise MoeError(status, where, detail)


def _stream(stream=None) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _ptr(t: Optional[torch.Tensor], dtype=None, name="tensor"):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return t.data_ptr()


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)


# ---------------------------------------------------------------------------
# expert banks on the device


@dataclass
class DeviceBank:
    n_experts: int
    d: int
    f: int
    g: int
    b_max: int
    w13_planes: torch.Tensor
    w13_sz: torch.Tensor
    w2_planes: torch.Tensor
    w2_sz: torch.Tensor
    plane_prefix: Optional[torch.Tensor] = None   # ragged bank: int32 [E+1] (device)

    @classmethod
    def from_host(cls, bank, device="cuda") -> "DeviceBank":
        def up(a):
            a = np.ascontiguousarray(a)
            if a.dtype == np.uint32:
                a = a.view(np.int32)
            return torch.from_numpy(a).to(device)
        pp = getattr(bank, "plane_prefix", None)
        return cls(bank.n_experts, bank.d, bank.f, bank.g, bank.b_max,
                   up(bank.w13_planes), up(bank.w13_sz), up(bank.w2_planes), up(bank.w2_sz),
                   None if pp is None else up(np.asarray(pp, dtype=np.int32)))

    def clone(self) -> "DeviceBank":
        return DeviceBank(self.n_experts, self.d, self.f, self.g, self.b_max, self.w13_planes.clone(),
                          self.w13_sz.clone(), self.w2_planes.clone(), self.w2_sz.clone(),
                          None if self.plane_prefix is None else self.plane_prefix.clone())

    def struct(self) -> ExpertBankC:
        for t in (self.w13_planes, self.w13_sz, self.w2_planes, self.w2_sz):
            _ptr(t, name="bank")
        pp = None if self.plane_prefix is None else _ptr(self.plane_prefix, torch.int32, "plane_prefix")
        return ExpertBankC(self.n_experts, self.d, self.f, self.g, self.b_max,
                           self.w13_planes.data_ptr(), self.w13_sz.data_ptr(),
                           self.w2_planes.data_ptr(), self.w2_sz.data_ptr(), pp)

    def plane_bytes_per_expert(self, bits: int) -> int:
        """Bytes of the first `bits` planes of W13 and W2 of one expert."""
        return bits * 3 * self.d * self.f // 8

    def sz_bytes_per_expert(self) -> int:
        return 3 * self.d * self.f // self.g * 8


def _bank_struct(b: Optional[DeviceBank]):
    return None if b is None else ctypes.byref(b.struct())


# ---------------------------------------------------------------------------
# entry points


def route_workspace_bytes(T: int, E: int) -> int:
    return int(lib().moe_route_workspace_bytes(T, E))


def route_workspace(T: int, E: int, device="cuda") -> torch.Tensor:
    """Router workspace (any content: it receives the T x E float64 logits)."""
    n = route_workspace_bytes(T, E)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def route(x: torch.Tensor, w_router: torch.Tensor, logit_bias: Optional[torch.Tensor], top_k: int,
          renorm: bool = False, workspace: Optional[torch.Tensor] = None, idx: Optional[torch.Tensor] = None,
          gate: Optional[torch.Tensor] = None, stream=None):
    T, d = x.shape
    E = w_router.shape[0]
    if workspace is None:
        workspace = route_workspace(T, E, x.device)
    if idx is None:
        idx = torch.empty(T, top_k, dtype=torch.int32, device=x.device)
    if gate is None:
        gate = torch.empty(T, top_k, dtype=torch.float32, device=x.device)
    st = lib().moe_route(_ptr(x, _BF16, "x"), T, d, _ptr(w_router, torch.float32, "w_router"), E,
                         _ptr(logit_bias, torch.float32, "logit_bias"), top_k, int(renorm),
                         _ptr(idx, torch.int32, "topk_idx"), _ptr(gate, torch.float32, "topk_gate"),
                         _ptr(workspace, name="workspace"), workspace.numel() * workspace.element_size(),
                         _stream(stream))
    _check(st, "moe_route")
    return idx, gate


def budget_pairs(P: int, b_lo: int, b_max: int, target: float) -> int:
    return int(lib().moe_budget_pairs(P, b_lo, b_max, float(target)))


def alloc_bits(gate: torch.Tensor, b_lo: int, b_max: int, target: float, bits: Optional[torch.Tensor] = None,
               tau: Optional[torch.Tensor] = None, n_hi: Optional[torch.Tensor] = None, stream=None):
    P = gate.numel()
    if bits is None:
        bits = torch.empty(P, dtype=torch.uint8, device=gate.device)
    st = lib().moe_alloc_bits(_ptr(gate, torch.float32, "gate"), P, b_lo, b_max, float(target),
                              _ptr(bits, torch.uint8, "bits"), _ptr(tau, torch.float32, "tau"),
                              _ptr(n_hi, torch.int32, "n_hi"), _stream(stream))
    _check(st, "moe_alloc_bits")
    return bits


def bits_from_threshold(gate: torch.Tensor, tau: float, b_lo: int, b_max: int,
                        bits: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Widths from a fixed gate threshold (calibration-threshold mode)."""
    P = gate.numel()
    if bits is None:
        bits = torch.empty(P, dtype=torch.uint8, device=gate.device)
    st = lib().moe_bits_from_threshold(_ptr(gate, torch.float32, "gate"), P, float(tau), b_lo, b_max,
                                       _ptr(bits, torch.uint8, "bits"), _stream(stream))
    _check(st, "moe_bits_from_threshold")
    return bits


def bits_from_threshold_device(gate: torch.Tensor, tau: torch.Tensor, b_lo: int, b_max: int,
                               bits: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Widths from a gate threshold held on the device (float32 scalar tensor)."""
    P = gate.numel()
    if bits is None:
        bits = torch.empty(P, dtype=torch.uint8, device=gate.device)
    st = lib().moe_bits_from_threshold_device(_ptr(gate, torch.float32, "gate"), P, _ptr(tau, torch.float32, "tau"),
                                              b_lo, b_max, _ptr(bits, torch.uint8, "bits"), _stream(stream))
    _check(st, "moe_bits_from_threshold_device")
    return bits


class ThresholdController:
    """Calibration-threshold mode under a changing target: tau lives on the
    device and is re-bisected over the stored calibration gate scores
    (moe_alloc_bits) whenever the target changes; every step's widths come
    from it (moe_bits_from_threshold_device).  Only argument marshalling and
    the change test are done here."""

    def __init__(self, calib_gates: torch.Tensor, b_lo: int, b_max: int):
        self.cal = calib_gates.reshape(-1).contiguous()
        self.b_lo, self.b_max = b_lo, b_max
        self.tau = torch.empty(1, dtype=torch.float32, device=self.cal.device)
        self._scratch = torch.empty(self.cal.numel(), dtype=torch.uint8, device=self.cal.device)
        self.target = None

    def widths(self, gate: torch.Tensor, target: float, bits: Optional[torch.Tensor] = None, stream=None):
        if target != self.target:
            alloc_bits(self.cal, self.b_lo, self.b_max, target, bits=self._scratch, tau=self.tau, stream=stream)
            self.target = target
        return bits_from_threshold_device(gate.reshape(-1), self.tau, self.b_lo, self.b_max, bits=bits,
                                          stream=stream)


def ffn_workspace_bytes(routed: DeviceBank, shared: Optional[DeviceBank], T: int, top_k: int) -> int:
    return int(lib().moe_ffn_workspace_bytes(ctypes.byref(routed.struct()), _bank_struct(shared), T, top_k))


def ffn_workspace(routed: DeviceBank, shared: Optional[DeviceBank], T: int, top_k: int, device="cuda"):
    n = ffn_workspace_bytes(routed, shared, T, top_k)
    if n == 0 and T > 0:
        raise MoeError(2, "moe_ffn_workspace_bytes", "invalid bank or sizes")
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def anyprec_ffn(routed: DeviceBank, shared: Optional[DeviceBank], x: torch.Tensor, idx: torch.Tensor,
                gate: torch.Tensor, bits: torch.Tensor, y: Optional[torch.Tensor] = None, accumulate: bool = False,
                workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    T, d = x.shape
    k = idx.shape[1]
    if workspace is None:
        workspace = ffn_workspace(routed, shared, T, k, x.device)
    if y is None:
        y = torch.zeros(T, d, dtype=torch.float32, device=x.device)
    st = lib().moe_anyprec_ffn(ctypes.byref(routed.struct()), _bank_struct(shared), _ptr(x, _BF16, "x"), T, k,
                               _ptr(idx, torch.int32, "topk_idx"), _ptr(gate, torch.float32, "topk_gate"),
                               _ptr(bits, torch.uint8, "bits"), _ptr(y, torch.float32, "y"), int(accumulate),
                               _ptr(workspace, name="workspace"), workspace.numel() * workspace.element_size(),
                               _stream(stream))
    _check(st, "moe_anyprec_ffn")
    return y


def layer_workspace(routed: DeviceBank, shared: Optional[DeviceBank], T: int, top_k: int, device="cuda"):
    n = int(lib().moe_layer_workspace_bytes(ctypes.byref(routed.struct()), _bank_struct(shared), T, top_k))
    if n == 0 and T > 0:
        raise MoeError(2, "moe_layer_workspace_bytes", "invalid bank or sizes")
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def layer(routed: DeviceBank, shared: Optional[DeviceBank], x: torch.Tensor, w_router: torch.Tensor,
          logit_bias: Optional[torch.Tensor], top_k: int, b_lo: int, target: float, renorm: bool = False,
          y: Optional[torch.Tensor] = None, accumulate: bool = False, idx: Optional[torch.Tensor] = None,
          gate: Optional[torch.Tensor] = None, bits: Optional[torch.Tensor] = None,
          workspace: Optional[torch.Tensor] = None, stream=None):
    """The whole layer (route, allocate, FFN) in one call; returns y, idx, gate, bits."""
    T, d = x.shape
    dev = x.device
    if workspace is None:
        workspace = layer_workspace(routed, shared, T, top_k, dev)
    if y is None:
        y = torch.zeros(T, d, dtype=torch.float32, device=dev)
    if idx is None:
        idx = torch.empty(T, top_k, dtype=torch.int32, device=dev)
    if gate is None:
        gate = torch.empty(T, top_k, dtype=torch.float32, device=dev)
    if bits is None:
        bits = torch.empty(T * top_k, dtype=torch.uint8, device=dev)
    st = lib().moe_layer(ctypes.byref(routed.struct()), _bank_struct(shared), _ptr(x, _BF16, "x"), T, top_k,
                         _ptr(w_router, torch.float32, "w_router"), _ptr(logit_bias, torch.float32, "logit_bias"),
                         int(renorm), b_lo, float(target), _ptr(idx, torch.int32, "topk_idx"),
                         _ptr(gate, torch.float32, "topk_gate"), _ptr(bits, torch.uint8, "bits"),
                         _ptr(y, torch.float32, "y"), int(accumulate), _ptr(workspace, name="workspace"),
                         workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "moe_layer")
    return y, idx, gate, bits


def layer_static(routed: DeviceBank, shared: Optional[DeviceBank], x: torch.Tensor, w_router: torch.Tensor,
                 logit_bias: Optional[torch.Tensor], top_k: int, b_lo: int, target: float, renorm: bool = False,
                 y: Optional[torch.Tensor] = None, accumulate: bool = False, idx: Optional[torch.Tensor] = None,
                 gate: Optional[torch.Tensor] = None, bits: Optional[torch.Tensor] = None, stream=None):
    """moe_layer on the library's static scratch array (no workspace); returns y, idx, gate, bits."""
    T, d = x.shape
    dev = x.device
    if y is None:
        y = torch.zeros(T, d, dtype=torch.float32, device=dev)
    if idx is None:
        idx = torch.empty(T, top_k, dtype=torch.int32, device=dev)
    if gate is None:
        gate = torch.empty(T, top_k, dtype=torch.float32, device=dev)
    if bits is None:
        bits = torch.empty(T * top_k, dtype=torch.uint8, device=dev)
    st = lib().moe_layer_static(ctypes.byref(routed.struct()), _bank_struct(shared), _ptr(x, _BF16, "x"), T, top_k,
                                _ptr(w_router, torch.float32, "w_router"),
                                _ptr(logit_bias, torch.float32, "logit_bias"), int(renorm), b_lo, float(target),
                                _ptr(idx, torch.int32, "topk_idx"), _ptr(gate, torch.float32, "topk_gate"),
                                _ptr(bits, torch.uint8, "bits"), _ptr(y, torch.float32, "y"), int(accumulate),
                                _stream(stream))
    _check(st, "moe_layer_static")
    return y, idx, gate, bits


def permute(idx: torch.Tensor, bits: torch.Tensor, E: int, b_max: int, workspace: torch.Tensor, stream=None):
    T, k = idx.shape
    slot_pair = torch.empty(T * k, dtype=torch.int32, device=idx.device)
    eoff = torch.empty(E + 1, dtype=torch.int32, device=idx.device)
    emax = torch.empty(E, dtype=torch.int32, device=idx.device)
    st = lib().moe_permute(_ptr(idx, torch.int32, "topk_idx"), _ptr(bits, torch.uint8, "bits"), T, k, E, b_max,
                           slot_pair.data_ptr(), eoff.data_ptr(), emax.data_ptr(), _ptr(workspace, name="workspace"),
                           workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "moe_permute")
    return slot_pair, eoff, emax


def dequant(bank: DeviceBank, expert: int, matrix: int, bits: int, stream=None) -> torch.Tensor:
    shape = (2 * bank.f, bank.d) if matrix == 0 else (bank.d, bank.f)
    out = torch.empty(shape, dtype=torch.float32, device=bank.w13_planes.device)
    st = lib().moe_dequant(ctypes.byref(bank.struct()), expert, matrix, bits, out.data_ptr(), _stream(stream))
    _check(st, "moe_dequant")
    return out


def residual_to_bf16(h: torch.Tensor, x: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    if x is None:
        x = torch.empty(h.shape, dtype=torch.bfloat16, device=h.device)
    st = lib().moe_residual_to_bf16(_ptr(h, torch.float32, "h"), _ptr(x, _BF16, "x"), h.numel(), _stream(stream))
    _check(st, "moe_residual_to_bf16")
    return x


def rmsnorm_to_bf16(h: torch.Tensor, x: Optional[torch.Tensor] = None, eps: float = 1e-6,
                    stream=None) -> torch.Tensor:
    """Rows of h [T][d] fp32 scaled to unit root-mean-square, as bf16."""
    rows, d = h.shape
    if x is None:
        x = torch.empty(h.shape, dtype=torch.bfloat16, device=h.device)
    st = lib().moe_rmsnorm_to_bf16(_ptr(h, torch.float32, "h"), _ptr(x, _BF16, "x"), rows, d, float(eps),
                                   _stream(stream))
    _check(st, "moe_rmsnorm_to_bf16")
    return x


# ---------------------------------------------------------------------------
# DuoRate per-expert widths


def duorate_bake(bank: DeviceBank, stream=None) -> torch.Tensor:
    """Distortion tensor [E][b_max][d] float64 of a bank (offline bake)."""
    out = torch.empty(bank.n_experts, bank.b_max, bank.d, dtype=torch.float64, device=bank.w13_planes.device)
    st = lib().moe_duorate_bake(ctypes.byref(bank.struct()), out.data_ptr(), _stream(stream))
    _check(st, "moe_duorate_bake")
    return out


def duorate_profile(x: torch.Tensor, idx: torch.Tensor, E: int, stream=None):
    """Prefill profile: (act_energy [E][d] float64, pair_count [E] int32)."""
    T, d = x.shape
    k = idx.shape[1]
    a = torch.empty(E, d, dtype=torch.float64, device=x.device)
    n = torch.empty(E, dtype=torch.int32, device=x.device)
    st = lib().moe_duorate_profile(_ptr(x, _BF16, "x"), T, d, _ptr(idx, torch.int32, "topk_idx"), k, E,
                                   a.data_ptr(), n.data_ptr(), _stream(stream))
    _check(st, "moe_duorate_profile")
    return a, n


def duorate_solve(delta: torch.Tensor, act_energy: torch.Tensor, pair_count: torch.Tensor, b_lo: int, b_max: int,
                  target: float, stream=None):
    """Per-expert widths: (expert_bits [E] uint8, distortion [E][b_max] float64, lambda [1] float64)."""
    E, B, d = delta.shape
    D = torch.empty(E, B, dtype=torch.float64, device=delta.device)
    w = torch.empty(E, dtype=torch.uint8, device=delta.device)
    lam = torch.empty(1, dtype=torch.float64, device=delta.device)
    st = lib().moe_duorate_solve(_ptr(delta, torch.float64, "delta"), _ptr(act_energy, torch.float64, "act_energy"),
                                 _ptr(pair_count, torch.int32, "pair_count"), E, d, b_lo, b_max, float(target),
                                 D.data_ptr(), w.data_ptr(), lam.data_ptr(), _stream(stream))
    _check(st, "moe_duorate_solve")
    return w, D, lam


def bits_from_expert_widths(idx: torch.Tensor, expert_bits: torch.Tensor, bits: Optional[torch.Tensor] = None,
                            stream=None) -> torch.Tensor:
    P = idx.numel()
    if bits is None:
        bits = torch.empty(P, dtype=torch.uint8, device=idx.device)
    st = lib().moe_bits_from_expert_widths(_ptr(idx, torch.int32, "topk_idx"), P,
                                           _ptr(expert_bits, torch.uint8, "expert_bits"), expert_bits.numel(),
                                           _ptr(bits, torch.uint8, "bits"), _stream(stream))
    _check(st, "moe_bits_from_expert_widths")
    return bits


# ---------------------------------------------------------------------------
# DPA-MoE residual-aware chunk allocation


def dpa_residuals(bank: DeviceBank, workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Per-expert residuals [E][b_max] float64 of a bank (offline profile)."""
    dev = bank.w13_planes.device
    if workspace is None:
        n = int(lib().moe_dpa_residuals_workspace_bytes(ctypes.byref(bank.struct())))
        workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=dev)
    out = torch.empty(bank.n_experts, bank.b_max, dtype=torch.float64, device=dev)
    st = lib().moe_dpa_residuals(ctypes.byref(bank.struct()), out.data_ptr(), _ptr(workspace, name="workspace"),
                                 workspace.numel(), _stream(stream))
    _check(st, "moe_dpa_residuals")
    return out


def dpa_alloc(gate: torch.Tensor, idx: torch.Tensor, resid: torch.Tensor, b_lo: int, b_max: int, target: float,
              bits: Optional[torch.Tensor] = None, n_chunks: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Residual-aware per-pair widths in [b_lo, b_max]."""
    P = gate.numel()
    E = resid.shape[0]
    if workspace is None:
        n = int(lib().moe_dpa_alloc_workspace_bytes(P, b_lo, b_max))
        workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=gate.device)
    if bits is None:
        bits = torch.empty(P, dtype=torch.uint8, device=gate.device)
    st = lib().moe_dpa_alloc(_ptr(gate, torch.float32, "gate"), _ptr(idx, torch.int32, "topk_idx"), P,
                             _ptr(resid, torch.float64, "resid"), E, b_lo, b_max, float(target),
                             _ptr(bits, torch.uint8, "bits"), _ptr(n_chunks, torch.int32, "n_chunks"),
                             _ptr(workspace, name="workspace"), workspace.numel(), _stream(stream))
    _check(st, "moe_dpa_alloc")
    return bits


STREAM_SINK = 8192


def stream_read(buf: torch.Tensor, sink: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Pure streaming read of the whole of `buf` (a measurement helper)."""
    if sink is None:
        sink = torch.empty(STREAM_SINK, dtype=torch.int32, device=buf.device)
    nbytes = buf.numel() * buf.element_size()
    st = lib().moe_stream_read(_ptr(buf, name="buf"), nbytes, sink.data_ptr(), _stream(stream))
    _check(st, "moe_stream_read")
    return sink


def set_kernel_events(events=None):
    """Record four torch.cuda.Event objects (gate/up begin, end; down begin,
    end) around the FFN's streaming kernels of the following calls on this
    thread; None turns the marks off.  Each event must have been recorded
    once before (so that its HIP event exists)."""
    if events is None:
        lib().moe_set_kernel_events(None, None, None, None)
    else:
        lib().moe_set_kernel_events(*[ev.cuda_event for ev in events])


def bf16_tensor(bits_u16: np.ndarray, device="cuda") -> torch.Tensor:
    """Upload bf16 bit patterns (numpy uint16) as a torch bfloat16 tensor."""
    return torch.from_numpy(np.ascontiguousarray(bits_u16).view(np.int16)).to(device).view(torch.bfloat16)
