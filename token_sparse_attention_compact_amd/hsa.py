"""Python binding of libhsa (ctypes).  Argument marshalling only: every step of
the HSA iteration runs in the library's HIP kernels.  torch is used for device
memory and streams.

Function names mirror include/hsa.h.  Each wrapper takes torch tensors, checks
dtype, device, contiguity and shape (the C ABI sees raw pointers only, so a
tensor smaller than the sizes passed would be read or written out of
bounds), passes raw pointers and the current HIP stream, and raises HsaError
on a non-zero status.  If libhsa.so is missing the import
fails loudly: there is no fallback path.
"""
from __future__ import annotations

import ctypes as ct
import os
from typing import List, Optional, Sequence

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libhsa.so")

HSA_F32, HSA_BF16 = 0, 1
MAX_GROUPS = 8
ABI_VERSION = 4
NOALLOC_SCRATCH_BYTES = 64 << 20   # HSA_NOALLOC_SCRATCH_BYTES
# optional block features (hsa_dims.features)
FEAT_QK_NORM, FEAT_ROPE3D, FEAT_ADALN, FEAT_CFG = 1, 2, 4, 8
FEATURE_BITS = {"qk_norm": FEAT_QK_NORM, "rope3d": FEAT_ROPE3D, "adaln": FEAT_ADALN, "cfg": FEAT_CFG}
T_FREQ = 256   # width of the timestep sinusoid (t_w1 is [D][256])
EXPORTED = [
    "hsa_status_str", "hsa_abi_version", "hsa_workspace_size", "hsa_attn_workspace_size",
    "hsa_select_workspace_size", "hsa_n_active", "hsa_active_set", "hsa_select", "hsa_select_batch",
    "hsa_euler",
    "hsa_attn_active", "hsa_layernorm", "hsa_embed", "hsa_unembed", "hsa_linear",
    "hsa_linear_residual", "hsa_qkv_scatter", "hsa_qk_norm_rope", "hsa_time_embed", "hsa_guidance",
    "hsa_block_forward", "hsa_step", "hsa_attn_active_noalloc",
]


class HsaError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: status {status} ({msg})")
        self.status = status


# ---------------------------------------------------------------- C structs
class Dims(ct.Structure):
    _fields_ = [("N", ct.c_int32), ("C", ct.c_int32), ("D", ct.c_int32), ("H", ct.c_int32),
                ("Dh", ct.c_int32), ("F", ct.c_int32), ("L", ct.c_int32), ("n_text", ct.c_int32),
                ("dtype", ct.c_int), ("features", ct.c_int32), ("grid_f", ct.c_int32),
                ("grid_h", ct.c_int32), ("grid_w", ct.c_int32)]


class Schedule(ct.Structure):
    _fields_ = [("T", ct.c_int32), ("K", ct.c_int32), ("m", ct.c_int32),
                ("budget", ct.c_int32 * MAX_GROUPS), ("count", ct.c_int32 * MAX_GROUPS)]


BLOCK_FIELDS = ("w_qkv", "w_o", "w_1", "w_2", "w_qx", "w_ox", "k_cache", "v_cache", "k_text",
                "v_text", "q_gain", "k_gain", "mod", "k_text_u", "v_text_u", "k_cache_u", "v_cache_u")
TIME_FIELDS = ("t_w1", "t_b1", "t_w2", "t_b2", "t_w3", "t_b3", "head_mod")


class Block(ct.Structure):
    _fields_ = [(n, ct.c_void_p) for n in BLOCK_FIELDS]


class Model(ct.Structure):
    _fields_ = ([("dims", Dims), ("w_in", ct.c_void_p), ("w_out", ct.c_void_p),
                 ("blocks", ct.POINTER(Block))] + [(n, ct.c_void_p) for n in TIME_FIELDS]
                + [("cfg_scale", ct.c_float)])


class State(ct.Structure):
    _fields_ = [("x", ct.c_void_p), ("v_hat", ct.c_void_p), ("score", ct.c_void_p),
                ("group", ct.c_void_p), ("active_idx", ct.c_void_p), ("pos", ct.c_void_p),
                ("workspace", ct.c_void_p), ("workspace_bytes", ct.c_size_t)]


# ---------------------------------------------------------------- loading
_lib = None


def lib_path() -> str:
    return _LIB_PATH


def load() -> ct.CDLL:
    """Load libhsa.so (built in-tree by token_sparse_attention_compact_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"libhsa.so not found at {_LIB_PATH}: build it with "
                          f"`python -m token_sparse_attention_compact_amd.build`")
    L = ct.CDLL(_LIB_PATH)
    P, I, F, S = ct.c_void_p, ct.c_int32, ct.c_float, ct.c_size_t
    PS = ct.POINTER(ct.c_size_t)
    PI = ct.POINTER(ct.c_int32)
    sig = {
        "hsa_status_str": ([I], ct.c_char_p),
        "hsa_abi_version": ([], I),
        "hsa_workspace_size": ([ct.POINTER(Dims), PS], I),
        "hsa_attn_workspace_size": ([I, I, I, I, PS], I),
        "hsa_select_workspace_size": ([I, I, PS], I),
        "hsa_n_active": ([ct.POINTER(Schedule), I, PI], I),
        "hsa_active_set": ([P, I, ct.POINTER(Schedule), I, P, P, P, P], I),
        "hsa_select": ([P, I, PI, I, P, P, S, P], I),
        "hsa_select_batch": ([P, I, I, PI, I, P, P], I),
        "hsa_euler": ([P, P, P, P, P, I, I, F, F, I, P], I),
        "hsa_attn_active": ([P, P, P, P, I, I, I, I, F, ct.c_int, P, S, P], I),
        "hsa_attn_active_noalloc": ([P, P, P, P, I, I, I, I, F, ct.c_int, P], I),
        "hsa_layernorm": ([P, P, I, I, P, P, ct.c_int, P], I),
        "hsa_embed": ([P, P, P, P, I, I, I, ct.c_int, P], I),
        "hsa_unembed": ([P, P, P, I, I, I, P, P, ct.c_int, P], I),
        "hsa_linear": ([P, P, P, I, I, I, I, ct.c_int, P], I),
        "hsa_linear_residual": ([P, P, P, I, I, I, P, ct.c_int, P], I),
        "hsa_qkv_scatter": ([P, P, I, P, P, P, P, I, I, I, ct.c_int, P], I),
        "hsa_qk_norm_rope": ([P, P, P, I, ct.POINTER(Dims), P, P, P], I),
        "hsa_time_embed": ([ct.POINTER(Model), F, P, P, P], I),
        "hsa_guidance": ([P, P, I, I, F, P], I),
        "hsa_block_forward": ([ct.POINTER(Model), I, P, P, I, P, I, P, S, P], I),
        "hsa_step": ([ct.POINTER(Model), ct.POINTER(Schedule), ct.POINTER(State), I, F, F, I, P, P], I),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    if L.hsa_abi_version() != ABI_VERSION:
        raise ImportError(f"libhsa.so ABI version {L.hsa_abi_version()}, binding expects "
                          f"{ABI_VERSION}: rebuild with `python -m token_sparse_attention_compact_amd.build`")
    _lib = L
    return L


def status_str(status: int) -> str:
    return load().hsa_status_str(status).decode()


def _check(fn: str, status: int):
    if status != 0:
        raise HsaError(fn, status, status_str(status))


def _stream(stream=None) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return HSA_BF16
    if t.dtype == torch.float32:
        return HSA_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def _need(t: torch.Tensor, dtype, name: str):
    if t.dtype != dtype:
        raise ValueError(f"{name}: expected {dtype}, got {t.dtype}")


def _shape(t: torch.Tensor, shape, name: str):
    """Exact shape; None in `shape` accepts any size in that dimension."""
    if t.dim() != len(shape) or any(s is not None and d != s for d, s in zip(t.shape, shape)):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")


def _rows(t: torch.Tensor, rows: int, cols: Optional[int], name: str):
    """At least `rows` rows (and exactly `cols` columns when given)."""
    if t.dim() != (1 if cols is None else 2) or t.shape[0] < rows or (cols is not None and t.shape[1] != cols):
        want = f"[>={rows}]" if cols is None else f"[>={rows}, {cols}]"
        raise ValueError(f"{name}: expected shape {want}, got {tuple(t.shape)}")


# ---------------------------------------------------------------- structs from python
def make_dims(N, C, D, H, Dh, F, L, n_text=0, dtype=torch.bfloat16, features=0,
              grid=(0, 0, 0)) -> Dims:
    """`features`: OR of FEAT_* bits, or an iterable of feature names."""
    if not isinstance(features, int):
        features = sum(FEATURE_BITS[f] for f in set(features))
    return Dims(N, C, D, H, Dh, F, L, n_text, HSA_BF16 if dtype == torch.bfloat16 else HSA_F32,
                features, *grid)


def make_schedule(T: int, budgets: Sequence[int], counts: Sequence[int], m: int = 0) -> Schedule:
    if len(budgets) != len(counts) or not 1 <= len(budgets) <= MAX_GROUPS:
        raise ValueError("budgets/counts: 1..8 groups of equal length")
    s = Schedule()
    s.T, s.K, s.m = T, len(budgets), m
    for k, (b, c) in enumerate(zip(budgets, counts)):
        s.budget[k] = b
        s.count[k] = c
    return s


# ---------------------------------------------------------------- entry points
def hsa_abi_version() -> int:
    return load().hsa_abi_version()


def hsa_workspace_size(dims: Dims) -> int:
    n = ct.c_size_t()
    _check("hsa_workspace_size", load().hsa_workspace_size(ct.byref(dims), ct.byref(n)))
    return n.value


def hsa_attn_workspace_size(n_active: int, n_kv: int, H: int, Dh: int) -> int:
    n = ct.c_size_t()
    _check("hsa_attn_workspace_size", load().hsa_attn_workspace_size(n_active, n_kv, H, Dh, ct.byref(n)))
    return n.value


def hsa_n_active(sched: Schedule, it: int) -> int:
    n = ct.c_int32()
    _check("hsa_n_active", load().hsa_n_active(ct.byref(sched), it, ct.byref(n)))
    return n.value


def hsa_active_set(group: torch.Tensor, sched: Schedule, it: int, active_idx: torch.Tensor,
                   pos: torch.Tensor, n_active_dev: torch.Tensor, stream=None):
    _need(group, torch.uint8, "group")
    for t, n in ((active_idx, "active_idx"), (pos, "pos"), (n_active_dev, "n_active_dev")):
        _need(t, torch.int32, n)
    N = group.numel()
    _rows(active_idx, N, None, "active_idx")
    _rows(pos, N, None, "pos")
    _rows(n_active_dev, 1, None, "n_active_dev")
    _check("hsa_active_set", load().hsa_active_set(_ptr(group), group.numel(), ct.byref(sched), it,
                                                   _ptr(active_idx), _ptr(pos), _ptr(n_active_dev),
                                                   _stream(stream)))


def hsa_select(score: torch.Tensor, counts: Sequence[int], group_out: torch.Tensor, stream=None):
    _need(score, torch.float32, "score")
    _need(group_out, torch.uint8, "group_out")
    _shape(group_out, (score.numel(),), "group_out")
    arr = (ct.c_int32 * len(counts))(*counts)
    _check("hsa_select", load().hsa_select(_ptr(score), score.numel(), arr, len(counts),
                                           _ptr(group_out), None, 0, _stream(stream)))


def hsa_select_batch(score: torch.Tensor, counts: Sequence[int], group_out: torch.Tensor, stream=None):
    """score [B][N] float32 -> group_out [B][N] uint8, each row selected with the same counts."""
    _need(score, torch.float32, "score")
    _need(group_out, torch.uint8, "group_out")
    if score.dim() != 2:
        raise ValueError(f"score must be [B][N], got shape {tuple(score.shape)}")
    _shape(group_out, tuple(score.shape), "group_out")
    arr = (ct.c_int32 * len(counts))(*counts)
    _check("hsa_select_batch", load().hsa_select_batch(_ptr(score), score.shape[0], score.shape[1], arr,
                                                       len(counts), _ptr(group_out), _stream(stream)))


def hsa_euler(x, v_hat, score, v_new, pos, dsigma: float, update_score: bool, eps: float = 1e-6,
              stream=None):
    for t, n in ((x, "x"), (v_hat, "v_hat"), (score, "score")):
        _need(t, torch.float32, n)
    if v_new is not None:
        _need(v_new, torch.float32, "v_new")
    _need(pos, torch.int32, "pos")
    N, C = x.shape
    _shape(v_hat, (N, C), "v_hat")
    _shape(score, (N,), "score")
    _shape(pos, (N,), "pos")
    if v_new is not None:
        _shape(v_new, (None, C), "v_new")   # rows: every pos[n] >= 0 must index one
    _check("hsa_euler", load().hsa_euler(_ptr(x), _ptr(v_hat), _ptr(score), _ptr(v_new), _ptr(pos),
                                         N, C, dsigma, eps, int(update_score), _stream(stream)))


def hsa_attn_active(q, k, v, o, H: int, Dh: int, scale: Optional[float] = None,
                    ws: Optional[torch.Tensor] = None, stream=None):
    dt = _dt(q)
    for t in (k, v, o):
        _need(t, q.dtype, "k/v/o")
    nA, nkv = q.shape[0], k.shape[0]
    _shape(q, (nA, H * Dh), "q")
    _shape(k, (nkv, H * Dh), "k")
    _shape(v, (nkv, H * Dh), "v")
    _shape(o, (nA, H * Dh), "o")
    if scale is None:
        scale = Dh ** -0.5
    need = hsa_attn_workspace_size(nA, nkv, H, Dh)
    if need and (ws is None or ws.numel() * ws.element_size() < need):
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check("hsa_attn_active", load().hsa_attn_active(_ptr(q), _ptr(k), _ptr(v), _ptr(o), nA, nkv, H, Dh,
                                                     scale, dt, _ptr(ws), wsb, _stream(stream)))


def hsa_attn_active_noalloc(q, k, v, o, H: int, Dh: int, scale: Optional[float] = None,
                            stream=None):
    """hsa_attn_active without a workspace: the library's fixed per-device
    array holds the KV-split partials (nothing is allocated, here or in the
    library).  Calls that overlap on one GPU race on that array."""
    dt = _dt(q)
    for t in (k, v, o):
        _need(t, q.dtype, "k/v/o")
    nA, nkv = q.shape[0], k.shape[0]
    _shape(q, (nA, H * Dh), "q")
    _shape(k, (nkv, H * Dh), "k")
    _shape(v, (nkv, H * Dh), "v")
    _shape(o, (nA, H * Dh), "o")
    if scale is None:
        scale = Dh ** -0.5
    _check("hsa_attn_active_noalloc",
           load().hsa_attn_active_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), nA, nkv, H, Dh, scale,
                                          dt, _stream(stream)))


def _mod_pair(shift, scale, D: int, name: str):
    if (shift is None) != (scale is None):
        raise ValueError(f"{name}: shift and scale go together")
    for t, n in ((shift, "shift"), (scale, "scale")):
        if t is not None:
            _need(t, torch.float32, n)
            _shape(t, (D,), n)


def hsa_layernorm(h, out, shift=None, scale=None, stream=None):
    _need(h, torch.float32, "h")
    rows, D = h.shape
    _shape(out, (rows, D), "out")
    _mod_pair(shift, scale, D, "hsa_layernorm")
    _check("hsa_layernorm", load().hsa_layernorm(_ptr(h), _ptr(out), rows, D, _ptr(shift), _ptr(scale),
                                                 _dt(out), _stream(stream)))


def hsa_embed(x, active_idx, n_active: int, w_in, h, stream=None):
    _need(x, torch.float32, "x")
    _need(h, torch.float32, "h")
    _need(active_idx, torch.int32, "active_idx")
    D, C = w_in.shape
    _shape(x, (None, C), "x")
    _rows(active_idx, n_active, None, "active_idx")
    _rows(h, n_active, D, "h")
    _check("hsa_embed", load().hsa_embed(_ptr(x), _ptr(active_idx), _ptr(w_in), _ptr(h), n_active, C, D,
                                         _dt(w_in), _stream(stream)))


def hsa_unembed(h, w_out, v_new, n_active: int, shift=None, scale=None, stream=None):
    _need(h, torch.float32, "h")
    _need(v_new, torch.float32, "v_new")
    C, D = w_out.shape
    _rows(h, n_active, D, "h")
    _rows(v_new, n_active, C, "v_new")
    _mod_pair(shift, scale, D, "hsa_unembed")
    _check("hsa_unembed", load().hsa_unembed(_ptr(h), _ptr(w_out), _ptr(v_new), n_active, D, C,
                                             _ptr(shift), _ptr(scale), _dt(w_out), _stream(stream)))


def hsa_linear(a, w, out, act: int = 0, M: Optional[int] = None, stream=None):
    M = a.shape[0] if M is None else M
    Nout, K = w.shape
    _need(w, a.dtype, "w")
    _need(out, a.dtype, "out")
    _rows(a, M, K, "a")
    _rows(out, M, Nout, "out")
    _check("hsa_linear", load().hsa_linear(_ptr(a), _ptr(w), _ptr(out), M, Nout, K, act, _dt(a),
                                           _stream(stream)))


def hsa_linear_residual(a, w, h, M: Optional[int] = None, gate=None, stream=None):
    _need(h, torch.float32, "h")
    M = a.shape[0] if M is None else M
    Nout, K = w.shape
    _need(w, a.dtype, "w")
    _rows(a, M, K, "a")
    _rows(h, M, Nout, "h")
    if gate is not None:
        _need(gate, torch.float32, "gate")
        _shape(gate, (Nout,), "gate")
    _check("hsa_linear_residual", load().hsa_linear_residual(_ptr(a), _ptr(w), _ptr(h), M, Nout, K,
                                                             _ptr(gate), _dt(a), _stream(stream)))


def hsa_qkv_scatter(a, active_idx, n_active: int, w_qkv, q_out, k_cache, v_cache, gather: bool = False,
                    stream=None):
    """gather=False: row j of a ([>= n_active][D]) is active row j; gather=True:
    a is the [N][D] per-token matrix and active row j is a[active_idx[j]]."""
    _need(active_idx, torch.int32, "active_idx")
    N, D = k_cache.shape
    for t, n in ((w_qkv, "w_qkv"), (q_out, "q_out"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, a.dtype, n)
    _shape(v_cache, (N, D), "v_cache")
    _shape(w_qkv, (3 * D, D), "w_qkv")
    if gather:
        _shape(a, (N, D), "a")
    else:
        _rows(a, n_active, D, "a")
    _rows(q_out, n_active, D, "q_out")
    _rows(active_idx, n_active, None, "active_idx")
    _check("hsa_qkv_scatter", load().hsa_qkv_scatter(_ptr(a), _ptr(active_idx), int(bool(gather)), _ptr(w_qkv),
                                                     _ptr(q_out), _ptr(k_cache), _ptr(v_cache), n_active, N, D,
                                                     _dt(a), _stream(stream)))


def hsa_qk_norm_rope(q, k_cache, active_idx, n_active: int, dims: Dims, q_gain=None, k_gain=None,
                     stream=None):
    dt = torch.bfloat16 if dims.dtype == HSA_BF16 else torch.float32
    _need(q, dt, "q")
    _need(k_cache, dt, "k_cache")
    _need(active_idx, torch.int32, "active_idx")
    _rows(q, n_active, dims.D, "q")
    _shape(k_cache, (dims.N, dims.D), "k_cache")
    _rows(active_idx, n_active, None, "active_idx")
    for t, n in ((q_gain, "q_gain"), (k_gain, "k_gain")):
        if t is not None:
            _need(t, torch.float32, n)
            _shape(t, (dims.D,), n)
    _check("hsa_qk_norm_rope", load().hsa_qk_norm_rope(_ptr(q), _ptr(k_cache), _ptr(active_idx), n_active,
                                                       ct.byref(dims), _ptr(q_gain), _ptr(k_gain),
                                                       _stream(stream)))


def hsa_guidance(v_cond, v, rows: Optional[int] = None, g: float = 1.0, stream=None):
    _need(v_cond, torch.float32, "v_cond")
    _need(v, torch.float32, "v")
    C = v.shape[1]
    rows = v.shape[0] if rows is None else rows
    _rows(v, rows, C, "v")
    _rows(v_cond, rows, C, "v_cond")
    _check("hsa_guidance", load().hsa_guidance(_ptr(v_cond), _ptr(v), rows, C, float(g), _stream(stream)))


# ---------------------------------------------------------------- owning helpers
class DeviceModel:
    """Device weights + per-layer K/V caches, and the hsa_model struct over them.

    Weight layouts are those of include/hsa.h (out-major [out][in]).  Feature
    parameters are float32: per block q_gain, k_gain [D] (qk_norm), mod [6][D]
    (adaln); the unconditional branch's k_text_u, v_text_u, k_cache_u,
    v_cache_u in the model dtype (cfg); `time` holds t_w1 .. head_mod (adaln).
    Tensors are kept referenced here so the raw pointers in the struct stay
    valid."""

    def __init__(self, dims: Dims, w_in: torch.Tensor, w_out: torch.Tensor, blocks: List[dict],
                 time: Optional[dict] = None, cfg_scale: float = 1.0):
        self.dims = dims
        dt = torch.bfloat16 if dims.dtype == HSA_BF16 else torch.float32
        f32 = torch.float32
        N, C, D, F, T = dims.N, dims.C, dims.D, dims.F, dims.n_text
        feat = dims.features
        if len(blocks) != dims.L:
            raise ValueError(f"blocks: expected {dims.L}, got {len(blocks)}")
        shapes = {"w_qkv": ((3 * D, D), dt), "w_o": ((D, D), dt), "w_1": ((F, D), dt),
                  "w_2": ((D, F), dt), "k_cache": ((N, D), dt), "v_cache": ((N, D), dt)}
        if T > 0:
            shapes.update({"w_qx": ((D, D), dt), "w_ox": ((D, D), dt), "k_text": ((T, D), dt),
                           "v_text": ((T, D), dt)})
        if feat & FEAT_QK_NORM:
            shapes.update({"q_gain": ((D,), f32), "k_gain": ((D,), f32)})
        if feat & FEAT_ADALN:
            shapes["mod"] = ((6, D), f32)
        if feat & FEAT_CFG:
            shapes.update({"k_text_u": ((T, D), dt), "v_text_u": ((T, D), dt),
                           "k_cache_u": ((N, D), dt), "v_cache_u": ((N, D), dt)})
        for t, shp, n in ((w_in, (D, C), "w_in"), (w_out, (C, D), "w_out")):
            _need(t, dt, n)
            _shape(t, shp, n)
        for l, b in enumerate(blocks):
            for n, (shp, tdt) in shapes.items():
                if b.get(n) is None:
                    raise ValueError(f"block {l}: {n} missing")
                _need(b[n], tdt, f"block {l} {n}")
                _shape(b[n], shp, f"block {l} {n}")
        tshapes = {"t_w1": (D, T_FREQ), "t_b1": (D,), "t_w2": (D, D), "t_b2": (D,),
                   "t_w3": (6 * D, D), "t_b3": (6 * D,), "head_mod": (2, D)}
        self.time = None
        if feat & FEAT_ADALN:
            if time is None:
                raise ValueError("adaln: timestep weights missing")
            for n, shp in tshapes.items():
                if time.get(n) is None:
                    raise ValueError(f"time: {n} missing")
                _need(time[n], f32, f"time {n}")
                _shape(time[n], shp, f"time {n}")
            self.time = {n: time[n].contiguous() for n in tshapes}
        self.w_in, self.w_out = w_in.contiguous(), w_out.contiguous()
        self.blocks = [{k: (v.contiguous() if v is not None else None) for k, v in b.items()} for b in blocks]
        arr = (Block * dims.L)()
        for l, b in enumerate(self.blocks):
            for name in BLOCK_FIELDS:
                t = b.get(name) if name in shapes else None
                setattr(arr[l], name, None if t is None else _ptr(t))
        self._arr = arr
        tp = [None if self.time is None else _ptr(self.time[n]) for n in TIME_FIELDS]
        self.c = Model(dims, _ptr(self.w_in), _ptr(self.w_out), arr, *tp, float(cfg_scale))


class DeviceState:
    """Sampler state buffers and the workspace, plus the hsa_state struct."""

    def __init__(self, dims: Dims, x0: torch.Tensor, group0: torch.Tensor,
                 v_hat: Optional[torch.Tensor] = None, score: Optional[torch.Tensor] = None):
        dev = x0.device
        N, C = dims.N, dims.C
        _shape(x0, (N, C), "x0")
        _shape(group0, (N,), "group0")
        if v_hat is not None:
            _shape(v_hat, (N, C), "v_hat")
        if score is not None:
            _shape(score, (N,), "score")
        self.x = x0.to(torch.float32).contiguous().clone()
        self.v_hat = (torch.zeros(N, C, device=dev) if v_hat is None else v_hat.clone().contiguous())
        self.score = (torch.full((N,), float("inf"), device=dev) if score is None
                      else score.clone().contiguous())
        self.group = group0.to(torch.uint8).contiguous().clone()
        self.active_idx = torch.zeros(N, dtype=torch.int32, device=dev)
        self.pos = torch.zeros(N, dtype=torch.int32, device=dev)
        nbytes = hsa_workspace_size(dims)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        self.c = State(_ptr(self.x), _ptr(self.v_hat), _ptr(self.score), _ptr(self.group),
                       _ptr(self.active_idx), _ptr(self.pos), _ptr(self.workspace), nbytes)


def hsa_time_embed(model: DeviceModel, sigma: float, e, e0, stream=None):
    D = model.dims.D
    for t, shp, n in ((e, (D,), "e"), (e0, (6, D), "e0")):
        _need(t, torch.float32, n)
        _shape(t, shp, n)
    _check("hsa_time_embed", load().hsa_time_embed(ct.byref(model.c), float(sigma), _ptr(e), _ptr(e0),
                                                   _stream(stream)))


def hsa_block_forward(model: DeviceModel, layer: int, h, active_idx, n_active: int,
                      ws: torch.Tensor, e0=None, branch: int = 0, stream=None):
    _need(h, torch.float32, "h")
    _need(active_idx, torch.int32, "active_idx")
    _rows(h, n_active, model.dims.D, "h")
    _rows(active_idx, n_active, None, "active_idx")
    if e0 is not None:
        _need(e0, torch.float32, "e0")
        _shape(e0, (6, model.dims.D), "e0")
    _check("hsa_block_forward", load().hsa_block_forward(ct.byref(model.c), layer, _ptr(h), _ptr(active_idx),
                                                         n_active, _ptr(e0), branch, _ptr(ws), ws.numel(),
                                                         _stream(stream)))


def hsa_step(model: DeviceModel, sched: Schedule, state: DeviceState, it: int, sigma_i: float,
             sigma_next: float, regroup: bool, v_field: Optional[torch.Tensor] = None, stream=None):
    if v_field is not None:
        _need(v_field, torch.float32, "v_field")
        _shape(v_field, (model.dims.N, model.dims.C), "v_field")
    _check("hsa_step", load().hsa_step(ct.byref(model.c), ct.byref(sched), ct.byref(state.c), it,
                                       float(sigma_i), float(sigma_next), int(regroup), _ptr(v_field),
                                       _stream(stream)))
