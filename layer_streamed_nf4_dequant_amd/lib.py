"""ctypes binding to liblsnf4.so (the C ABI of include/lsnf4.h).

Argument marshalling only: every step of the path runs in the library's gfx950 kernels.
torch tensors are used as device memory (their data pointers are passed through) and torch
streams as HIP streams.  There is no fallback: if the library is missing or a call fails,
an exception is raised.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblsnf4.so")

LSN_OK, LSN_E_ARG, LSN_E_NOFIT, LSN_E_STATE, LSN_E_HIP, LSN_E_AUDIT = range(6)
STATUS_NAMES = {0: "LSN_OK", 1: "LSN_E_ARG", 2: "LSN_E_NOFIT", 3: "LSN_E_STATE", 4: "LSN_E_HIP",
                5: "LSN_E_AUDIT"}
W_NF4, W_BF16, W_BF16_T = 0, 1, 2
OUT_BF16, OUT_F32, OUT_BF16_T = 0, 1, 2
ADAPTERS_OFF, ADAPTERS_ON, ADAPTERS_U_READY = 0, 1, 2
DX_BF16_SET, DX_F32_ADD, DX_F32_SET = 0, 1, 2
GRAD_SET, GRAD_ADD = 0, 1
POOL_AUDIT, POOL_KEEP_AT_TURN, POOL_HOST_SIM, POOL_FILE_TIER, POOL_FILE_DIRECT = 1, 2, 4, 8, 16
FAULT_STALE_REFETCH, FAULT_WRONG_SLOT = 1 << 8, 1 << 9

EXPORTS = (
    "lsn_last_error", "lsn_abi_version", "lsn_nf4_codebook", "nf4_pack_ws_bytes", "nf4_pack",
    "nf4_dequant", "nf4_dequant_batch", "lora_down", "lora_linear_ws_bytes", "lora_linear_fwd", "lora_linear_fwd_group",
    "lora_linear_bwd", "lora_linear_group_ws_bytes", "lora_linear_bwd_group",
    "lora_linear_bwd_noalloc", "lora_linear_bwd_noalloc_max_ws_bytes",
    "lora_linear_fwd_group_epi", "lora_linear_fwd_swiglu", "lora_linear_bwd_swiglu",
    "layer_pool_create", "layer_pool_register", "layer_pool_register_file", "layer_pool_prefetch", "layer_pool_acquire",
    "layer_pool_release", "layer_pool_stats", "layer_pool_audit", "layer_pool_destroy",
    "lm_head_ce_ws_bytes", "lm_head_ce", "embedding_gather",
    "rmsnorm_fwd", "rmsnorm_bwd", "rope_apply", "rope_table", "swiglu_fwd", "swiglu_bwd",
    "attention_fwd", "attention_bwd_ws_bytes", "attention_bwd", "attention_bwd_rope",
    "add_bf16", "convert_f32_bf16", "convert_bf16_f32",
)


class LsnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class NF4Desc(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("codes", ctypes.c_void_p),
                ("qabsmax", ctypes.c_void_p), ("absmax2", ctypes.c_void_p), ("mean", ctypes.c_float)]


class WeightDesc(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("nf4", NF4Desc), ("bf16", ctypes.c_void_p)]


class LoraLinearDesc(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("K", ctypes.c_int64), ("N", ctypes.c_int64),
                ("r", ctypes.c_int64), ("scale", ctypes.c_float), ("W", WeightDesc),
                ("A", ctypes.c_void_p), ("B", ctypes.c_void_p)]


class RopeDesc(ctypes.Structure):
    """lsn_rope: a rope_table table, its rows and head width, and the rows' positions."""
    _fields_ = [("cs", ctypes.c_void_p), ("n_pos", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("positions", ctypes.c_void_p)]


class PoolStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in ("copies", "bytes_copied", "hits", "misses",
                                                "acquires", "releases", "audit_checks",
                                                "audit_failures")]

    def as_dict(self):
        return {n: int(getattr(self, n)) for n, _ in self._fields_}


_lib = None


class PoolBuffers(ctypes.Structure):
    """lsn_pool_buffers: the caller's checksum array (audit) and pinned bounce buffers (file tier)."""
    _fields_ = [("audit_sums", ctypes.c_void_p), ("audit_capacity", ctypes.c_size_t),
                ("bounce", ctypes.c_void_p * 2), ("direct_stage", ctypes.c_void_p * 2)]


def load():
    """Load liblsnf4.so once and declare its signatures. Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run python -m layer_streamed_nf4_dequant_amd.build")
    # One HIP runtime per process: torch ships its own copy of libamdhip64 under the same soname
    # as the system one this library links. Loaded after torch, the library binds to torch's
    # copy; loaded first, it would pull in the system copy and torch would later load its own,
    # and two runtimes in one process do not share devices or memory. So torch goes first.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    sig = {
        "lsn_last_error": (ctypes.c_char_p, []),
        "lsn_abi_version": (i32, []),
        "lsn_nf4_codebook": (None, [vp, vp]),
        "nf4_pack_ws_bytes": (sz, [i64, i64]),
        "nf4_pack": (i32, [vp, i64, i64, vp, vp, vp, vp, vp, sz, vp]),
        "nf4_dequant": (i32, [ctypes.POINTER(NF4Desc), vp, i32, vp]),
        "nf4_dequant_batch": (i32, [i32, ctypes.POINTER(NF4Desc), ctypes.POINTER(vp), i32, vp]),
        "lora_down": (i32, [i64, i64, vp, i32, ctypes.POINTER(vp), ctypes.POINTER(i32), ctypes.POINTER(vp), vp]),
        "lora_linear_ws_bytes": (sz, [i64, i64, i64, i64]),
        "lora_linear_fwd": (i32, [ctypes.POINTER(LoraLinearDesc), i32, vp, vp, vp, vp, sz, vp]),
        "lora_linear_fwd_group": (i32, [i32, ctypes.POINTER(LoraLinearDesc), i32, vp, ctypes.POINTER(vp),
                                        ctypes.POINTER(vp), vp, sz, vp]),
        "lora_linear_bwd": (i32, [ctypes.POINTER(LoraLinearDesc), vp, vp, vp, vp, i32, vp, vp, i32,
                                  vp, sz, vp]),
        "lora_linear_fwd_group_epi": (i32, [i32, ctypes.POINTER(LoraLinearDesc), i32, vp, ctypes.POINTER(vp),
                                            ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.c_uint32,
                                            ctypes.POINTER(RopeDesc), vp, sz, vp]),
        "lora_linear_fwd_swiglu": (i32, [ctypes.POINTER(LoraLinearDesc), ctypes.POINTER(LoraLinearDesc), i32, vp,
                                         vp, vp, vp, vp, vp, vp, sz, vp]),
        "lora_linear_bwd_swiglu": (i32, [ctypes.POINTER(LoraLinearDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp, i32,
                                         vp, sz, vp]),
        "lora_linear_bwd_noalloc": (i32, [ctypes.POINTER(LoraLinearDesc), vp, vp, vp, vp, i32, vp, vp, i32, vp]),
        "lora_linear_bwd_noalloc_max_ws_bytes": (sz, []),
        "lora_linear_group_ws_bytes": (sz, [i32, ctypes.POINTER(LoraLinearDesc)]),
        "lora_linear_bwd_group": (i32, [i32, ctypes.POINTER(LoraLinearDesc), vp, ctypes.POINTER(vp),
                                        ctypes.POINTER(vp), vp, i32, ctypes.POINTER(vp), ctypes.POINTER(vp), i32,
                                        vp, sz, vp]),
        "layer_pool_create": (i32, [i32, sz, ctypes.POINTER(vp), i32, vp, ctypes.c_uint32,
                                    ctypes.POINTER(PoolBuffers), ctypes.POINTER(vp)]),
        "layer_pool_register": (i32, [vp, i32, vp, sz]),
        "layer_pool_register_file": (i32, [vp, i32, ctypes.c_char_p, ctypes.c_uint64, sz]),
        "layer_pool_prefetch": (i32, [vp, i32]),
        "layer_pool_acquire": (i32, [vp, i32, vp, ctypes.POINTER(vp)]),
        "layer_pool_release": (i32, [vp, i32, vp]),
        "layer_pool_stats": (i32, [vp, ctypes.POINTER(PoolStats)]),
        "layer_pool_audit": (i32, [vp]),
        "layer_pool_destroy": (i32, [vp]),
        "lm_head_ce_ws_bytes": (sz, [i64, i64, i64]),
        "lm_head_ce": (i32, [i64, i64, i64, vp, vp, vp, f32, vp, vp, i64, vp, sz, vp]),
        "embedding_gather": (i32, [i64, i64, i64, vp, vp, vp, vp, vp]),
        "rmsnorm_fwd": (i32, [i64, i64, vp, vp, f32, vp, vp, vp]),
        "rmsnorm_bwd": (i32, [i64, i64, vp, vp, vp, vp, vp, i32, vp, vp]),
        "rope_apply": (i32, [i64, i32, i32, vp, i64, vp, f32, i32, vp]),
        "rope_table": (i32, [i32, i32, f32, vp, vp]),
        "swiglu_fwd": (i32, [i64, vp, vp, vp, vp]),
        "swiglu_bwd": (i32, [i64, vp, vp, vp, vp, vp, vp]),
        "attention_fwd": (i32, [i64, i64, i32, i32, i32, vp, i64, vp, i64, vp, i64, f32, vp, i64, vp, vp]),
        "attention_bwd_ws_bytes": (sz, [i64, i64, i32, i32, i32]),
        "add_bf16": (i32, [i64, vp, vp, vp, vp]),
        "convert_f32_bf16": (i32, [i64, vp, vp, vp]),
        "convert_bf16_f32": (i32, [i64, vp, vp, vp]),
        "attention_bwd": (i32, [i64, i64, i32, i32, i32, vp, i64, vp, i64, vp, i64, vp, i64, vp, vp, i64, f32,
                                vp, i64, vp, i64, vp, i64, vp, sz, vp]),
        "attention_bwd_rope": (i32, [i64, i64, i32, i32, i32, vp, i64, vp, i64, vp, i64, vp, i64, vp, vp, i64, f32,
                                     vp, i64, vp, i64, vp, i64, vp, sz, ctypes.POINTER(RopeDesc), vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != LSN_OK:
        raise LsnError(status, load().lsn_last_error().decode(errors="replace"))


def codebook() -> tuple[np.ndarray, np.ndarray]:
    """(levels[16], midpoints[15]) as the library's kernels use them (host call, no GPU)."""
    q = np.zeros(16, dtype=np.float32)
    m = np.zeros(15, dtype=np.float32)
    load().lsn_nf4_codebook(q.ctypes.data, m.ctypes.data)
    return q, m


# ---------------------------------------------------------------------------------------------
# torch-facing helpers (torch only owns memory and streams)
# ---------------------------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _stream_handle(stream=None) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _ptr(t) -> int | None:
    return None if t is None else int(t.data_ptr())


@dataclass
class NF4Tensor:
    """An NF4-packed weight W[rows][cols] whose arrays are torch device tensors."""
    rows: int
    cols: int
    codes: object      # uint8 [rows*cols/2]
    qabsmax: object    # int8 [rows*cols/64]
    absmax2: object    # float32 [rows*cols/16384]
    mean: float

    def desc(self) -> NF4Desc:
        return NF4Desc(self.rows, self.cols, _ptr(self.codes), _ptr(self.qabsmax),
                       _ptr(self.absmax2), float(self.mean))

    @staticmethod
    def nbytes_for(rows: int, cols: int) -> int:
        n = rows * cols
        return n // 2 + n // 64 + 4 * (n // 16384)


def nf4_pack(w, stream=None) -> NF4Tensor:
    """Pack fp32 device W[rows][cols] to NF4 (synchronises the stream)."""
    torch = _torch()
    assert w.dtype == torch.float32 and w.is_cuda and w.dim() == 2 and w.is_contiguous()
    rows, cols = w.shape
    n = rows * cols
    dev = w.device
    codes = torch.empty(n // 2, dtype=torch.uint8, device=dev)
    qabs = torch.empty(max(n // 64, 1), dtype=torch.int8, device=dev)
    abs2 = torch.empty(max(n // 16384, 1), dtype=torch.float32, device=dev)
    ws = torch.empty(max(load().nf4_pack_ws_bytes(rows, cols), 256), dtype=torch.uint8, device=dev)
    mean = ctypes.c_float(0.0)
    check(load().nf4_pack(_ptr(w), rows, cols, _ptr(codes), _ptr(qabs), _ptr(abs2),
                          ctypes.addressof(mean), _ptr(ws), ws.numel(), _stream_handle(stream)))
    return NF4Tensor(rows, cols, codes, qabs, abs2, float(mean.value))


def nf4_pack_into(w, codes, qabsmax, absmax2, ws, stream=None) -> float:
    """Pack into caller-provided device arrays; returns the per-tensor mean."""
    rows, cols = w.shape
    mean = ctypes.c_float(0.0)
    check(load().nf4_pack(_ptr(w), rows, cols, _ptr(codes), _ptr(qabsmax), _ptr(absmax2),
                          ctypes.addressof(mean), _ptr(ws), ws.numel() * ws.element_size(),
                          _stream_handle(stream)))
    return float(mean.value)


def nf4_dequant(w: NF4Tensor, out_dtype: str = "bf16", out=None, stream=None):
    """out_dtype: "bf16" ([rows][cols]), "f32" ([rows][cols]) or "bf16_t" (transposed, [cols][rows])."""
    torch = _torch()
    code = {"bf16": OUT_BF16, "f32": OUT_F32, "bf16_t": OUT_BF16_T}[out_dtype]
    if out is None:
        shape = (w.cols, w.rows) if code == OUT_BF16_T else (w.rows, w.cols)
        out = torch.empty(shape, dtype=torch.float32 if code == OUT_F32 else torch.bfloat16,
                          device=w.codes.device)
    d = w.desc()
    check(load().nf4_dequant(ctypes.byref(d), _ptr(out), code, _stream_handle(stream)))
    return out


def nf4_dequant_batch(descs, outs, out_dtype: str = "bf16", stream=None) -> None:
    """nf4_dequant of several NF4 tensors (NF4Desc list) into caller-allocated outputs, one launch."""
    code = {"bf16": OUT_BF16, "f32": OUT_F32, "bf16_t": OUT_BF16_T}[out_dtype]
    n = len(descs)
    arr = (NF4Desc * n)(*descs)
    ptrs = (ctypes.c_void_p * n)(*[o if isinstance(o, int) else _ptr(o) for o in outs])
    check(load().nf4_dequant_batch(n, arr, ptrs, code, _stream_handle(stream)))


def weight_desc(W, transposed: bool = False) -> WeightDesc:
    """W is an NF4Tensor or a bf16 device tensor: [N][K], or W^T [K][N] with transposed=True."""
    if isinstance(W, NF4Tensor):
        return WeightDesc(W_NF4, W.desc(), None)
    return WeightDesc(W_BF16_T if transposed else W_BF16, NF4Desc(), _ptr(W))


def linear_desc(T: int, K: int, N: int, r: int, scale: float, W, A, B, transposed: bool = False) -> LoraLinearDesc:
    return LoraLinearDesc(T, K, N, r, float(scale), weight_desc(W, transposed), _ptr(A), _ptr(B))


def ws_bytes(T: int, K: int, N: int, r: int) -> int:
    return int(load().lora_linear_ws_bytes(T, K, N, r))


def lora_down(X, A_list, U_list, stream=None) -> None:
    """U_g = bf16(X A_g^T) for all g, reading X once (linears that share the input X)."""
    T, K = X.shape
    n = len(A_list)
    A = (ctypes.c_void_p * n)(*[_ptr(a) for a in A_list])
    U = (ctypes.c_void_p * n)(*[_ptr(u) for u in U_list])
    r = (ctypes.c_int32 * n)(*[int(a.shape[0]) for a in A_list])
    check(load().lora_down(T, K, _ptr(X), n, A, r, U, _stream_handle(stream)))


def lora_linear_fwd(desc: LoraLinearDesc, X, Y, U=None, adapters=True, ws=None, stream=None) -> None:
    """adapters: True/False, or ADAPTERS_U_READY when U already holds bf16(X A^T)."""
    mode = adapters if isinstance(adapters, int) and not isinstance(adapters, bool) else (
        ADAPTERS_ON if adapters else ADAPTERS_OFF)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    check(load().lora_linear_fwd(ctypes.byref(desc), mode, _ptr(X), _ptr(Y), _ptr(U),
                                 _ptr(ws), nbytes, _stream_handle(stream)))


def lora_linear_fwd_group(descs, X, Y_list, U_list=None, adapters=True, ws=None, stream=None) -> None:
    """The forwards of linears sharing the input X (one GEMM launch for bf16 weights)."""
    mode = adapters if isinstance(adapters, int) and not isinstance(adapters, bool) else (
        ADAPTERS_ON if adapters else ADAPTERS_OFF)
    n = len(descs)
    arr = (LoraLinearDesc * n)(*descs)
    Y = (ctypes.c_void_p * n)(*[_ptr(y) for y in Y_list])
    U = (ctypes.c_void_p * n)(*[_ptr(u) for u in U_list]) if U_list is not None else None
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    check(load().lora_linear_fwd_group(n, arr, mode, _ptr(X), Y, U, _ptr(ws), nbytes, _stream_handle(stream)))


def _mode(adapters) -> int:
    return adapters if isinstance(adapters, int) and not isinstance(adapters, bool) else (
        ADAPTERS_ON if adapters else ADAPTERS_OFF)


def rope_desc(cs, n_pos: int, head_dim: int, positions) -> RopeDesc:
    """The rotation a fused epilogue applies: a rope_table table (fp32 [n_pos][head_dim/2][2])
    and the rows' positions (int32 [T])."""
    return RopeDesc(_ptr(cs), int(n_pos), int(head_dim), _ptr(positions))


def rope_table(n_pos: int, head_dim: int, theta: float, out=None, stream=None):
    """cs[p][i] = (cos, sin) of rope_apply's angle for position p, pair i (fp32 [n_pos][head_dim/2][2])."""
    torch = _torch()
    if out is None:
        out = torch.empty((n_pos, head_dim // 2, 2), dtype=torch.float32, device="cuda")
    check(load().rope_table(int(n_pos), int(head_dim), float(theta), _ptr(out), _stream_handle(stream)))
    return out


def lora_linear_fwd_group_epi(descs, X, Y_list, U_list=None, adapters=True, residual=None, rope_mask: int = 0,
                              rope: RopeDesc | None = None, ws=None, stream=None) -> None:
    """lora_linear_fwd_group with the residual add (residual: a list with None entries) and the
    rotary embedding (members in rope_mask) applied in the GEMM's epilogue."""
    n = len(descs)
    arr = (LoraLinearDesc * n)(*descs)
    Y = (ctypes.c_void_p * n)(*[_ptr(y) for y in Y_list])
    U = (ctypes.c_void_p * n)(*[_ptr(u) for u in U_list]) if U_list is not None else None
    R = (ctypes.c_void_p * n)(*[_ptr(r) for r in residual]) if residual is not None else None
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    check(load().lora_linear_fwd_group_epi(n, arr, _mode(adapters), _ptr(X), Y, U, R, int(rope_mask),
                                           ctypes.byref(rope) if rope is not None else None, _ptr(ws), nbytes,
                                           _stream_handle(stream)))


def lora_linear_fwd_swiglu(desc_gate: LoraLinearDesc, desc_up: LoraLinearDesc, X, M, gate=None, up=None, Ug=None,
                           Uu=None, adapters=True, ws=None, stream=None) -> None:
    """gate, up projections and M = bf16(silu(gate) up) in one launch (gate / up stored if given)."""
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    check(load().lora_linear_fwd_swiglu(ctypes.byref(desc_gate), ctypes.byref(desc_up), _mode(adapters), _ptr(X),
                                        _ptr(gate), _ptr(up), _ptr(M), _ptr(Ug), _ptr(Uu), _ptr(ws), nbytes,
                                        _stream_handle(stream)))


def lora_linear_bwd_swiglu(desc: LoraLinearDesc, X, dY, U, gate, up, dgate, dup, dA, dB, grad_mode: int = GRAD_SET,
                           ws=None, stream=None) -> None:
    """The down projection's backward with the SwiGLU backward in its epilogue: dgate, dup instead of dX."""
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    check(load().lora_linear_bwd_swiglu(ctypes.byref(desc), _ptr(X), _ptr(dY), _ptr(U), _ptr(gate), _ptr(up),
                                        _ptr(dgate), _ptr(dup), _ptr(dA), _ptr(dB), grad_mode, _ptr(ws), nbytes,
                                        _stream_handle(stream)))


def lora_linear_bwd(desc: LoraLinearDesc, X, dY, U, dX, dA, dB, dx_mode: int = DX_BF16_SET,
                    grad_mode: int = GRAD_SET, ws=None, stream=None) -> None:
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    check(load().lora_linear_bwd(ctypes.byref(desc), _ptr(X), _ptr(dY), _ptr(U), _ptr(dX), dx_mode,
                                 _ptr(dA), _ptr(dB), grad_mode, _ptr(ws), nbytes, _stream_handle(stream)))


def lora_linear_bwd_noalloc(desc: LoraLinearDesc, X, dY, U, dX, dA, dB, dx_mode: int = DX_BF16_SET,
                            grad_mode: int = GRAD_SET, stream=None) -> None:
    """lora_linear_bwd on the library's static per-GPU workspace (no workspace argument)."""
    check(load().lora_linear_bwd_noalloc(ctypes.byref(desc), _ptr(X), _ptr(dY), _ptr(U), _ptr(dX), dx_mode,
                                         _ptr(dA), _ptr(dB), grad_mode, _stream_handle(stream)))


def noalloc_max_ws_bytes() -> int:
    return int(load().lora_linear_bwd_noalloc_max_ws_bytes())


def group_ws_bytes(descs) -> int:
    n = len(descs)
    return int(load().lora_linear_group_ws_bytes(n, (LoraLinearDesc * n)(*descs)))


def lora_linear_bwd_group(descs, X, dY_list, U_list, dX, dA_list, dB_list, dx_mode: int = DX_F32_ADD,
                          grad_mode: int = GRAD_SET, ws=None, stream=None) -> None:
    """Backwards of linears sharing X whose input gradients add up in dX (one GEMM for
    transposed bf16 weights)."""
    n = len(descs)
    arr = (LoraLinearDesc * n)(*descs)
    ptrs = lambda ts: (ctypes.c_void_p * n)(*[_ptr(t) for t in ts])  # noqa: E731
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    check(load().lora_linear_bwd_group(n, arr, _ptr(X), ptrs(dY_list), ptrs(U_list), _ptr(dX), dx_mode,
                                       ptrs(dA_list), ptrs(dB_list), grad_mode, _ptr(ws), nbytes,
                                       _stream_handle(stream)))


class LayerPool:
    """Owner of an lsn_pool handle. Slots, the audit's checksum array and the file tier's bounce
    buffers are caller memory (torch tensors or host buffers), passed as addresses: audit_sums =
    (address, capacity in checksums), bounce = (address, address), direct_stage = (address,
    address) (plain host memory for the O_DIRECT reads)."""

    def __init__(self, slot_ptrs, slot_bytes: int, n_layers: int, copy_stream_handle: int | None,
                 flags: int = 0, audit_sums: tuple[int, int] | None = None, bounce: tuple[int, int] | None = None,
                 direct_stage: tuple[int, int] | None = None):
        arr = (ctypes.c_void_p * len(slot_ptrs))(*slot_ptrs)
        bufs = PoolBuffers()
        if audit_sums is not None:
            bufs.audit_sums, bufs.audit_capacity = audit_sums
        if bounce is not None:
            bufs.bounce[0], bufs.bounce[1] = bounce
        if direct_stage is not None:
            bufs.direct_stage[0], bufs.direct_stage[1] = direct_stage
        h = ctypes.c_void_p()
        check(load().layer_pool_create(len(slot_ptrs), slot_bytes, arr, n_layers, copy_stream_handle,
                                       flags, ctypes.byref(bufs), ctypes.byref(h)))
        self.h = h
        self.flags = flags

    def register(self, layer: int, host_ptr: int, nbytes: int) -> None:
        check(load().layer_pool_register(self.h, layer, host_ptr, nbytes))

    def register_file(self, layer: int, path: str, offset: int, nbytes: int) -> None:
        """File tier: the layer's image is nbytes at offset of the file at path."""
        check(load().layer_pool_register_file(self.h, layer, os.fsencode(path), offset, nbytes))

    def prefetch(self, layer: int) -> None:
        check(load().layer_pool_prefetch(self.h, layer))

    def acquire(self, layer: int, compute_stream_handle: int | None) -> int:
        out = ctypes.c_void_p()
        check(load().layer_pool_acquire(self.h, layer, compute_stream_handle, ctypes.byref(out)))
        return int(out.value)

    def release(self, layer: int, compute_stream_handle: int | None) -> None:
        check(load().layer_pool_release(self.h, layer, compute_stream_handle))

    def stats(self) -> dict:
        s = PoolStats()
        check(load().layer_pool_stats(self.h, ctypes.byref(s)))
        return s.as_dict()

    def audit(self) -> None:
        check(load().layer_pool_audit(self.h))

    def close(self) -> None:
        if self.h is not None and self.h.value:
            check(load().layer_pool_destroy(self.h))
        self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def lm_head_ce_ws_bytes(chunk_rows: int, H: int, V: int) -> int:
    return int(load().lm_head_ce_ws_bytes(chunk_rows, H, V))


def lm_head_ce(h, W, labels, grad_scale: float, loss, dh, chunk_rows: int, ws, stream=None) -> None:
    """loss[t] = logsumexp(h W^T)_t - (h W^T)_t,label (fp32) and dh = bf16(bf16(dlogits) W), chunked
    over rows (labels outside [0, V): ignored rows)."""
    T, H = h.shape
    V = W.shape[0]
    check(load().lm_head_ce(T, H, V, _ptr(h), _ptr(W), _ptr(labels), float(grad_scale), _ptr(loss), _ptr(dh),
                            chunk_rows, _ptr(ws), ws.numel() * ws.element_size(), _stream_handle(stream)))


def embedding_gather(ids, E, X, bad_ids=None, stream=None) -> None:
    """X[t] = E[ids[t]]; out-of-range ids give zero rows and are counted in bad_ids (int32)."""
    T = ids.shape[0]
    V, H = E.shape
    check(load().embedding_gather(T, H, V, _ptr(ids), _ptr(E), _ptr(X), _ptr(bad_ids), _stream_handle(stream)))


def rmsnorm_fwd(x, gain, eps: float, y, rstd, stream=None) -> None:
    """y = bf16(x * rstd * gain), rstd = 1 / sqrt(mean x^2 + eps) per row (fp32, kept for the backward)."""
    T, H = x.shape
    check(load().rmsnorm_fwd(T, H, _ptr(x), _ptr(gain), float(eps), _ptr(y), _ptr(rstd), _stream_handle(stream)))


def rmsnorm_bwd(x, gain, rstd, dy, dx, accumulate: bool = False, dx_bf16=None, stream=None) -> None:
    """dx (fp32) = gradient of rmsnorm_fwd with respect to x, stored or added into dx; dx_bf16 (optional)
    also receives bf16(dx)."""
    T, H = x.shape
    check(load().rmsnorm_bwd(T, H, _ptr(x), _ptr(gain), _ptr(rstd), _ptr(dy), _ptr(dx), int(bool(accumulate)),
                             _ptr(dx_bf16), _stream_handle(stream)))


def rope_apply(x, positions, n_heads: int, head_dim: int, theta: float, inverse: bool = False, stream=None) -> None:
    """Rotary embedding in place on the first n_heads * head_dim columns of each row of x (a 2-D
    bf16 tensor or a column slice of one); inverse turns the other way (the backward)."""
    T = x.shape[0]
    check(load().rope_apply(T, n_heads, head_dim, _ptr(x), x.stride(0), _ptr(positions), float(theta),
                            int(bool(inverse)), _stream_handle(stream)))


def swiglu_fwd(g, u, m, stream=None) -> None:
    """m = bf16(silu(g) u), elementwise."""
    check(load().swiglu_fwd(g.numel(), _ptr(g), _ptr(u), _ptr(m), _stream_handle(stream)))


def swiglu_bwd(g, u, dm, dg, du, stream=None) -> None:
    """dg, du = gradients of swiglu_fwd (bf16)."""
    check(load().swiglu_bwd(g.numel(), _ptr(g), _ptr(u), _ptr(dm), _ptr(dg), _ptr(du), _stream_handle(stream)))


def attention_fwd(q, k, v, o, lse, n_seq: int, n_q: int, n_kv: int, head_dim: int, scale: float | None = None,
                  stream=None) -> None:
    """Causal grouped-query attention over n_seq packed sequences of equal length: q, k, v and o are
    2-D bf16 tensors or column slices (head h in columns h*head_dim ..); lse [T][n_q] fp32."""
    T = q.shape[0]
    S = T // n_seq
    sc = 1.0 / float(head_dim) ** 0.5 if scale is None else float(scale)
    check(load().attention_fwd(n_seq, S, n_q, n_kv, head_dim, _ptr(q), q.stride(0), _ptr(k), k.stride(0),
                               _ptr(v), v.stride(0), sc, _ptr(o), o.stride(0), _ptr(lse), _stream_handle(stream)))


def attention_bwd_ws_bytes(n_seq: int, S: int, n_q: int, n_kv: int, head_dim: int) -> int:
    return int(load().attention_bwd_ws_bytes(n_seq, S, n_q, n_kv, head_dim))


def attention_bwd(q, k, v, o, lse, dO, dq, dk, dv, ws, n_seq: int, n_q: int, n_kv: int, head_dim: int,
                  scale: float | None = None, stream=None) -> None:
    """dq, dk, dv (bf16, stored) of attention_fwd for the upstream gradient dO."""
    T = q.shape[0]
    S = T // n_seq
    sc = 1.0 / float(head_dim) ** 0.5 if scale is None else float(scale)
    check(load().attention_bwd(n_seq, S, n_q, n_kv, head_dim, _ptr(q), q.stride(0), _ptr(k), k.stride(0),
                               _ptr(v), v.stride(0), _ptr(o), o.stride(0), _ptr(lse), _ptr(dO), dO.stride(0), sc,
                               _ptr(dq), dq.stride(0), _ptr(dk), dk.stride(0), _ptr(dv), dv.stride(0), _ptr(ws),
                               ws.numel() * ws.element_size(), _stream_handle(stream)))


def attention_bwd_rope(q, k, v, o, lse, dO, dq, dk, dv, ws, n_seq: int, n_q: int, n_kv: int, head_dim: int,
                       rope: RopeDesc, scale: float | None = None, stream=None) -> None:
    """attention_bwd with dq and dk rotated back by the inverse rotary embedding as they are stored."""
    T = q.shape[0]
    S = T // n_seq
    sc = 1.0 / float(head_dim) ** 0.5 if scale is None else float(scale)
    check(load().attention_bwd_rope(n_seq, S, n_q, n_kv, head_dim, _ptr(q), q.stride(0), _ptr(k), k.stride(0),
                                    _ptr(v), v.stride(0), _ptr(o), o.stride(0), _ptr(lse), _ptr(dO), dO.stride(0),
                                    sc, _ptr(dq), dq.stride(0), _ptr(dk), dk.stride(0), _ptr(dv), dv.stride(0),
                                    _ptr(ws), ws.numel() * ws.element_size(), ctypes.byref(rope),
                                    _stream_handle(stream)))


def add_bf16(a, b, out, stream=None) -> None:
    """out = bf16(a + b) elementwise (out may be a or b)."""
    check(load().add_bf16(a.numel(), _ptr(a), _ptr(b), _ptr(out), _stream_handle(stream)))


def convert(x, out, stream=None) -> None:
    """fp32 -> bf16 (nearest even) or bf16 -> fp32 (exact), by the dtypes of x and out."""
    torch = _torch()
    if x.dtype == torch.float32 and out.dtype == torch.bfloat16:
        check(load().convert_f32_bf16(x.numel(), _ptr(x), _ptr(out), _stream_handle(stream)))
    elif x.dtype == torch.bfloat16 and out.dtype == torch.float32:
        check(load().convert_bf16_f32(x.numel(), _ptr(x), _ptr(out), _stream_handle(stream)))
    else:
        raise TypeError(f"convert: {x.dtype} -> {out.dtype} not supported")
