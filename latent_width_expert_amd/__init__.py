"""Python binding of libk3moe, the Kimi K3 LatentMoE layer forward for MI355X (gfx950).

Argument marshalling only: every step of the layer runs in the library's HIP kernels. torch
supplies device memory (tensors) and the stream (torch's current stream unless one is given).
The library must be built (``python latent_width_expert_amd/build.py``); importing works without
it, but any call that needs it raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libk3moe.so")

OK, EINVAL, ESTATE, ETOOBIG, EHIP, EUNSUPPORTED = 0, -1, -2, -3, -4, -5
ACT = {"bf16": 0, "mxfp8": 1}

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32


class Config(ctypes.Structure):
    _fields_ = [("d_model", _i32), ("latent", _i32), ("hidden", _i32), ("n_experts", _i32), ("top_k", _i32),
                ("n_shared", _i32), ("shared_hidden", _i32), ("latent_moe", _i32), ("act", _i32),
                ("max_tokens", _i32), ("rms_eps", ctypes.c_float), ("lora_rank", _i32)]


class MX(ctypes.Structure):
    _fields_ = [("codes", _vp), ("scales", _vp)]


class Lora(ctypes.Structure):
    _fields_ = [("a_gate", _vp), ("b_gate", _vp), ("a_up", _vp), ("b_up", _vp), ("a_down", _vp), ("b_down", _vp)]


LORA_FIELDS = [f for f, _ in Lora._fields_]


class Weights(ctypes.Structure):
    _fields_ = [("include_dense", _i32), ("w_router", MX), ("w_down", MX), ("w_up", MX),
                ("router_bias", _vp), ("rms_gamma", _vp),
                ("sh_gate", ctypes.POINTER(MX)), ("sh_up", ctypes.POINTER(MX)), ("sh_down", ctypes.POINTER(MX)),
                ("routed_first", _i32), ("routed_count", _i32),
                ("gate", ctypes.POINTER(MX)), ("up", ctypes.POINTER(MX)), ("down", ctypes.POINTER(MX)),
                ("lora", ctypes.POINTER(Lora))]


TAP_FIELDS = ["scores", "topk_idx", "topk_p", "counts", "offsets", "perm", "inv", "z", "z_scales", "z_f32",
              "h", "h_scales", "h_f32", "expert_out", "u", "n", "hs"]


class Taps(ctypes.Structure):
    _fields_ = [(f, _vp) for f in TAP_FIELDS]


class K3MoEError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"k3moe error {code}: {msg}")
        self.code = code


_lib = None


def lib():
    """Load libk3moe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with latent_width_expert_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        L.k3moe_create.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(_vp)]
        L.k3moe_create.restype = ctypes.c_int
        L.k3moe_destroy.argtypes = [_vp]
        L.k3moe_destroy.restype = None
        L.k3moe_last_error.argtypes = [_vp]
        L.k3moe_last_error.restype = ctypes.c_char_p
        L.k3moe_weight_bytes.argtypes = [_vp]
        L.k3moe_weight_bytes.restype = ctypes.c_size_t
        L.k3moe_workspace_bytes.argtypes = [_vp]
        L.k3moe_workspace_bytes.restype = ctypes.c_size_t
        L.k3moe_pack_weights.argtypes = [_vp, ctypes.POINTER(Weights), _vp, _vp]
        L.k3moe_pack_weights.restype = ctypes.c_int
        L.k3moe_forward.argtypes = [_vp, _vp, _i32, _vp, _vp, _vp]
        L.k3moe_forward.restype = ctypes.c_int
        L.k3moe_forward_ex.argtypes = [_vp, _vp, _i32, _vp, _vp, _vp, ctypes.POINTER(Taps)]
        L.k3moe_forward_ex.restype = ctypes.c_int
        L.k3moe_profile_begin.argtypes = [_vp, _i32]
        L.k3moe_profile_begin.restype = ctypes.c_int
        L.k3moe_quantile_bias.argtypes = [_vp, _vp, _i32, _vp, _vp]
        L.k3moe_quantile_bias.restype = ctypes.c_int
        L.k3moe_profile_end.argtypes = [_vp, ctypes.POINTER(ctypes.c_float), _i32, ctypes.POINTER(_i32)]
        L.k3moe_profile_end.restype = ctypes.c_int
        L.k3moe_stage_count.argtypes = []
        L.k3moe_stage_count.restype = _i32
        L.k3moe_stage_name.argtypes = [_i32]
        L.k3moe_stage_name.restype = ctypes.c_char_p
        L.k3moe_forward_head.argtypes = [_vp, _vp, _i32, _vp, _vp, _i32, _vp, _vp, _vp, _vp]
        L.k3moe_forward_head.restype = ctypes.c_int
        L.k3moe_experts_forward.argtypes = [_vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp]
        L.k3moe_experts_forward.restype = ctypes.c_int
        L.k3moe_forward_tail.argtypes = [_vp, _vp, _i32, _vp, _vp, _vp]
        L.k3moe_forward_tail.restype = ctypes.c_int
        L.k3moe_forward_noalloc.argtypes = [_vp, _vp, _i32, _vp, _vp]
        L.k3moe_forward_noalloc.restype = ctypes.c_int
        L.k3moe_scratch_fits.argtypes = [_vp, _i32]
        L.k3moe_scratch_fits.restype = ctypes.c_int
        L.k3moe_stream_read.argtypes = [_vp, ctypes.c_size_t, _vp, _vp]
        L.k3moe_stream_read.restype = ctypes.c_int
        _lib = L
    return _lib


def stage_names():
    L = lib()
    return [L.k3moe_stage_name(i).decode() for i in range(L.k3moe_stage_count())]


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    assert t.is_cuda and t.is_contiguous(), "device tensors must be contiguous CUDA/HIP tensors"
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _mx(pair):
    return MX(_ptr(pair[0]), _ptr(pair[1]))


@dataclass
class LayerConfig:
    d_model: int
    latent: int
    hidden: int
    n_experts: int
    top_k: int
    n_shared: int
    shared_hidden: int
    latent_moe: int = 1
    act: str = "bf16"
    max_tokens: int = 64
    rms_eps: float = 1e-6
    lora_rank: int = 0

    def c(self) -> Config:
        return Config(self.d_model, self.latent, self.hidden, self.n_experts, self.top_k, self.n_shared,
                      self.shared_hidden, self.latent_moe, ACT[self.act], self.max_tokens, self.rms_eps,
                      self.lora_rank)

    @property
    def expert_in(self) -> int:
        return self.latent if self.latent_moe else self.d_model


def _check_tensor(name, t, shape, dtypes):
    """Shape and dtype of a caller-supplied device tensor the library writes or reads."""
    if not (isinstance(t, torch.Tensor) and t.is_cuda and t.is_contiguous()):
        raise ValueError(f"{name}: a contiguous device tensor is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype}, expected one of {dtypes}")


class K3MoE:
    """One LatentMoE layer context. Owns nothing on the device: the packed weights and the
    workspace are torch tensors held by this object (allocate with `allocate`)."""

    def __init__(self, cfg: LayerConfig):
        self.cfg = cfg
        self._L = lib()
        h = _vp()
        rc = self._L.k3moe_create(ctypes.byref(cfg.c()), ctypes.byref(h))
        if rc != OK:
            raise K3MoEError(rc, self._L.k3moe_last_error(None).decode())
        self._h = h
        self.packed = None
        self.workspace = None

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._L.k3moe_destroy(h)
            self._h = None

    def _check(self, rc):
        if rc != OK:
            raise K3MoEError(rc, self._L.k3moe_last_error(self._h).decode())

    @property
    def weight_bytes(self) -> int:
        return int(self._L.k3moe_weight_bytes(self._h))

    @property
    def workspace_bytes(self) -> int:
        return int(self._L.k3moe_workspace_bytes(self._h))

    def allocate(self, device="cuda"):
        self.packed = torch.empty(self.weight_bytes, dtype=torch.uint8, device=device)
        self.workspace = torch.empty(self.workspace_bytes, dtype=torch.uint8, device=device)
        return self

    def tap_spec(self, T):
        """Expected (shape, dtypes) of every k3moe_taps field for a forward of T tokens."""
        c = self.cfg
        le, Tk = c.expert_in, T * c.top_k
        f8 = c.act == "mxfp8"
        act = (torch.uint8,) if f8 else (torch.bfloat16,)
        f32, i32 = (torch.float32,), (torch.int32,)
        spec = {"scores": ((T, c.n_experts), f32), "topk_idx": ((T, c.top_k), i32), "topk_p": ((T, c.top_k), f32),
                "counts": ((c.n_experts,), i32), "offsets": ((c.n_experts + 1,), i32), "perm": ((Tk,), i32),
                "inv": ((Tk,), i32), "h": ((Tk, c.hidden), act), "h_scales": ((Tk, c.hidden // 32), (torch.uint8,)),
                "h_f32": ((Tk, c.hidden), f32), "expert_out": ((Tk, le), f32), "u": ((T, le), f32),
                "hs": ((T, c.n_shared * c.shared_hidden), (torch.bfloat16,))}
        if c.latent_moe:
            spec.update(z=((T, c.latent), act), z_scales=((T, c.latent // 32), (torch.uint8,)),
                        z_f32=((T, c.latent), f32), n=((T, c.latent), (torch.bfloat16,)))
        return spec

    def pack(self, dense=None, routed=None, routed_first=0, stream=None, lora=None):
        """dense: dict with w_router, router_bias, [w_down, w_up, rms_gamma], shared (list of
        (gate, up, down)); routed: list of (gate, up, down) for experts routed_first.. .
        Matrices are (codes, scales) uint8 device tensors in the canonical MX layout. lora: with
        lora_rank > 0, a list (one per routed expert) of dicts a_gate, b_gate, a_up, b_up, a_down,
        b_down (bf16 device tensors)."""
        w = Weights()
        keep = []
        if dense is not None:
            w.include_dense = 1
            w.w_router = _mx(dense["w_router"])
            if "w_down" in dense:
                w.w_down = _mx(dense["w_down"])
                w.w_up = _mx(dense["w_up"])
                w.rms_gamma = _ptr(dense["rms_gamma"])
            w.router_bias = _ptr(dense["router_bias"])
            sh = dense.get("shared", [])
            if sh:
                arrs = [(MX * len(sh))(*[_mx(m[i]) for m in sh]) for i in range(3)]
                keep.append(arrs)
                w.sh_gate, w.sh_up, w.sh_down = [ctypes.cast(a, ctypes.POINTER(MX)) for a in arrs]
        if routed:
            arrs = [(MX * len(routed))(*[_mx(m[i]) for m in routed]) for i in range(3)]
            keep.append(arrs)
            w.routed_first = routed_first
            w.routed_count = len(routed)
            w.gate, w.up, w.down = [ctypes.cast(a, ctypes.POINTER(MX)) for a in arrs]
            if lora is not None:
                assert len(lora) == len(routed)
                la = (Lora * len(lora))(*[Lora(*[_ptr(m[f]) for f in LORA_FIELDS]) for m in lora])
                keep.append(la)
                w.lora = ctypes.cast(la, ctypes.POINTER(Lora))
        self._check(self._L.k3moe_pack_weights(self._h, ctypes.byref(w), _ptr(self.packed), _stream(stream)))

    def forward(self, x, y=None, taps=None, stream=None):
        """x: bf16 [T, d] device tensor. Returns y bf16 [T, d]. taps: optional dict name -> device
        tensor (fields of k3moe_taps) filled after the forward."""
        T = x.shape[0]
        _check_tensor("x", x, (T, self.cfg.d_model), (torch.bfloat16,))
        if y is None:
            y = torch.empty_like(x)
        _check_tensor("y", y, (T, self.cfg.d_model), (torch.bfloat16,))
        if taps:
            spec = self.tap_spec(T)
            for name, v in taps.items():
                if name not in spec:
                    raise ValueError(f"unknown tap {name}")
                if v is not None:
                    _check_tensor(name, v, *spec[name])
            t = Taps(*[_ptr(taps.get(f)) for f in TAP_FIELDS])
            rc = self._L.k3moe_forward_ex(self._h, _ptr(x), T, _ptr(y), _ptr(self.workspace), _stream(stream),
                                          ctypes.byref(t))
        else:
            rc = self._L.k3moe_forward(self._h, _ptr(x), T, _ptr(y), _ptr(self.workspace), _stream(stream))
        self._check(rc)
        return y

    def forward_raw(self, x_ptr, T, y_ptr, ws_ptr, stream=None):
        """Unchecked pointer-level call (for tests of the C-ABI error paths). Returns the status."""
        return self._L.k3moe_forward(self._h, x_ptr, T, y_ptr, ws_ptr, _stream(stream) if stream is not None else None)

    def last_error(self) -> str:
        return self._L.k3moe_last_error(self._h).decode()

    def quantile_bias(self, scores, stream=None):
        """Router bias b [E] (fp32, device) from router scores [T, E] (fp32, device) of a calibration
        batch: k3moe_quantile_bias."""
        if scores.dim() != 2:
            raise ValueError("scores must be [T, n_experts]")
        _check_tensor("scores", scores, (scores.shape[0], self.cfg.n_experts), (torch.float32,))
        bias = torch.empty(scores.shape[1], dtype=torch.float32, device=scores.device)
        self._check(self._L.k3moe_quantile_bias(self._h, _ptr(scores), scores.shape[0], _ptr(bias), _stream(stream)))
        return bias

    # ---- no device allocation: the library's static scratch replaces the workspace
    def scratch_fits(self, T: int) -> bool:
        return bool(self._L.k3moe_scratch_fits(self._h, T))

    def forward_noalloc(self, x, y, stream=None):
        """k3moe_forward_noalloc: y (preallocated bf16 [T, d]) = layer(x), no workspace."""
        T = x.shape[0]
        _check_tensor("x", x, (T, self.cfg.d_model), (torch.bfloat16,))
        _check_tensor("y", y, (T, self.cfg.d_model), (torch.bfloat16,))
        self._check(self._L.k3moe_forward_noalloc(self._h, _ptr(x), T, _ptr(y), _stream(stream)))
        return y

    # ---- expert-parallel split: head (origin) -> experts (each rank) -> tail (origin)
    def forward_head(self, x, n_ranks, stream=None):
        """Router, dispatch tables and the send side for n_ranks contiguous expert ranges. Returns
        (send_rows [T k, le], send_scales [T k, le / 32] or None, send_counts int32 [n_ranks],
        expert_counts int32 [E]); the workspace keeps the state forward_tail needs."""
        c = self.cfg
        T = x.shape[0]
        _check_tensor("x", x, (T, c.d_model), (torch.bfloat16,))
        le, Tk = c.expert_in, T * c.top_k
        f8 = c.act == "mxfp8" and c.latent_moe
        rows = torch.empty(Tk, le, dtype=torch.uint8 if f8 else torch.bfloat16, device=x.device)
        scales = torch.empty(Tk, le // 32, dtype=torch.uint8, device=x.device) if f8 else None
        send = torch.empty(n_ranks, dtype=torch.int32, device=x.device)
        counts = torch.empty(c.n_experts, dtype=torch.int32, device=x.device)
        self._check(self._L.k3moe_forward_head(self._h, _ptr(x), T, _ptr(self.workspace), _stream(stream), n_ranks,
                                               _ptr(rows), _ptr(scales), _ptr(send), _ptr(counts)))
        return rows, scales, send, counts

    def experts_forward(self, rows, scales, counts, out=None, stream=None):
        """This context's experts (one rank's range) on R received expert-contiguous rows
        (counts int32 [n_experts] rows each). Returns the expert outputs fp32 [R, le]."""
        c = self.cfg
        R = rows.shape[0]
        f8 = c.act == "mxfp8" and c.latent_moe
        _check_tensor("rows", rows, (R, c.expert_in), (torch.uint8,) if f8 else (torch.bfloat16,))
        if f8:
            _check_tensor("scales", scales, (R, c.expert_in // 32), (torch.uint8,))
        _check_tensor("counts", counts, (c.n_experts,), (torch.int32,))
        if out is None:
            out = torch.empty(R, c.expert_in, dtype=torch.float32, device=rows.device)
        _check_tensor("out", out, (R, c.expert_in), (torch.float32,))
        self._check(self._L.k3moe_experts_forward(self._h, _ptr(rows), _ptr(scales) if f8 else None, R, _ptr(counts),
                                                  _ptr(out), _ptr(self.workspace), _stream(stream)))
        return out

    def forward_tail(self, expert_out, T, y=None, stream=None):
        """Combine, RMSNorm, W_up and the shared experts' down projections on the expert outputs
        (fp32 [T k, le], in the order of the head's send rows) -> y bf16 [T, d]."""
        c = self.cfg
        _check_tensor("expert_out", expert_out, (T * c.top_k, c.expert_in), (torch.float32,))
        if y is None:
            y = torch.empty(T, c.d_model, dtype=torch.bfloat16, device=expert_out.device)
        _check_tensor("y", y, (T, c.d_model), (torch.bfloat16,))
        self._check(self._L.k3moe_forward_tail(self._h, _ptr(expert_out), T, _ptr(y), _ptr(self.workspace),
                                               _stream(stream)))
        return y

    def profile_begin(self, max_calls: int):
        self._check(self._L.k3moe_profile_begin(self._h, max_calls))

    def profile_end(self):
        n = self._L.k3moe_stage_count()
        ms = (ctypes.c_float * n)()
        calls = _i32()
        self._check(self._L.k3moe_profile_end(self._h, ms, n, ctypes.byref(calls)))
        return dict(zip(stage_names(), list(ms))), calls.value


def stream_read(buf, out=None, stream=None):
    """k3moe_stream_read over a device tensor (its bytes, a multiple of 16): xors a checksum into `out`
    (int32 [1], allocated if not given) and returns it; time it with events on the stream to get the
    read rate."""
    assert buf.is_cuda and buf.is_contiguous()
    nbytes = buf.numel() * buf.element_size()
    if out is None:
        out = torch.zeros(1, dtype=torch.int32, device=buf.device)
    _check_tensor("out", out, (1,), (torch.int32,))
    rc = lib().k3moe_stream_read(_ptr(buf), nbytes, _ptr(out), _stream(stream))
    if rc != OK:
        raise K3MoEError(rc, "stream_read failed")
    return out
