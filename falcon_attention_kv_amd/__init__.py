"""Python binding of libunipin.so: M-FALCON masked attention over a slotted KV pool.

Argument marshalling only.  Every step of the computation runs in the library's HIP
kernels; PyTorch provides device memory and the current stream.  There is no CPU
fallback: if the library cannot be loaded, importing this package raises.

    pool = Pool.allocate(L, S, H, n_max, D, torch.bfloat16, device="cuda")
    slots = pool.acquire_many(B)                     # round-robin slot ids
    o = prefill(q, k, v, lens, pool, slots, layer)   # writes the slot's K/V rows
    oc = rank_decode(qc, kc, vc, pool, slots, lens, layer)
    o1 = ar_decode(q1, k1, v1, pool, slots, lens, layer)  # one retrieval step, row lens[b]

Functions mirror the C entry points of include/unipin.h (unipin_prefill,
unipin_rank_decode, unipin_ar_decode, unipin_pool_*), with the same argument meaning.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libunipin.so")

FP32, BF16, FP8_E4M3 = 0, 1, 2
OK, EINVAL, ERANGE, EDTYPE, EALIGN, EDEVICE, EHIP, ENOMEM, EPERM, EIO, ESCRATCH = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9, -10
FLAG_BAD_SLOT, FLAG_BAD_LEN, FLAG_DUP_SLOT = 1, 2, 4

# Every symbol include/unipin.h declares.
EXPORTS = ("unipin_pool_create", "unipin_pool_destroy", "unipin_pool_acquire",
           "unipin_pool_generation", "unipin_pool_dims", "unipin_pool_export",
           "unipin_pool_import", "unipin_prefill",
           "unipin_rank_decode", "unipin_rank_decode_split", "unipin_rank_decode_workspace_bytes", "unipin_ar_decode", "unipin_ar_decode_noalloc", "unipin_ar_decode_workspace_bytes",
           "unipin_pool_status", "unipin_strerror", "unipin_version",
           "unipin_block_ctx_create", "unipin_block_ctx_destroy", "unipin_block_workspace_bytes",
           "unipin_block_ctx_tune", "unipin_block_ctx_set_gemm", "unipin_block_fold_layernorm",
           "unipin_block_forward")


# Weights of one transformer block, in the order of unipin_block_weights_t.
BLOCK_WEIGHT_NAMES = ("ln1_w", "ln1_b", "w_qkv", "b_qkv", "w_o", "b_o", "ln2_w", "ln2_b", "w_fc", "b_fc",
                      "w_proj", "b_proj")
# The optional folded LayerNorm weights (fold_layernorm), after them in the struct.
BLOCK_FOLDED_NAMES = ("w_qkv_ln", "uv_qkv", "w_fc_ln", "uv_fc")
BLOCK_HISTORY, BLOCK_CANDIDATES = 0, 1
# unipin_block_ctx_set_gemm: AUTO, hipBLASLt only, or the library's kernel with tile 0, 1, 2, 3
GEMM_AUTO, GEMM_LIBRARY = -2, -1


class BlockWeights(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in BLOCK_WEIGHT_NAMES + BLOCK_FOLDED_NAMES]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python falcon_attention_kv_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    missing = [name for name in EXPORTS if not hasattr(lib, name)]
    if missing:
        raise ImportError(f"{LIB_PATH} lacks {', '.join(missing)}: it is stale, rebuild it with "
                          "`python falcon_attention_kv_amd/build.py`")
    vp, i32, i64p, u64p = ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_uint64)
    ip = ctypes.POINTER(ctypes.c_int)
    i32p = ctypes.POINTER(ctypes.c_int32)
    lib.unipin_pool_create.argtypes = [ctypes.POINTER(vp), vp, vp, i32, i32, i32, i32, i32, i32]
    lib.unipin_pool_destroy.argtypes = [vp]
    lib.unipin_pool_acquire.argtypes = [vp, i32p, u64p]
    lib.unipin_pool_generation.argtypes = [vp, ctypes.c_int32]
    lib.unipin_pool_dims.argtypes = [vp, ip, ip, ip, ip, ip, ip]
    lib.unipin_pool_export.argtypes = [vp, ctypes.c_char_p]
    lib.unipin_pool_import.argtypes = [ctypes.POINTER(vp), ctypes.c_char_p]
    lib.unipin_prefill.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, ctypes.c_float, vp, vp]
    lib.unipin_rank_decode.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, ctypes.c_float, vp, vp]
    lib.unipin_rank_decode_split.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, ctypes.c_float, vp, vp,
                                             ctypes.c_size_t, vp]
    lib.unipin_rank_decode_workspace_bytes.argtypes = [vp, i32, i32]
    lib.unipin_ar_decode.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, ctypes.c_float, vp, vp, ctypes.c_size_t, vp]
    lib.unipin_ar_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, ctypes.c_float, vp, vp]
    lib.unipin_ar_decode_workspace_bytes.argtypes = [vp, i32]
    lib.unipin_block_ctx_create.argtypes = [ctypes.POINTER(vp)]
    lib.unipin_block_ctx_destroy.argtypes = [vp]
    lib.unipin_block_workspace_bytes.argtypes = [vp, i32, i32]
    lib.unipin_block_ctx_tune.argtypes = [vp, vp, i32, i32, vp, ctypes.c_size_t, vp]
    lib.unipin_block_ctx_set_gemm.argtypes = [vp, i32]
    lib.unipin_block_forward.argtypes = [vp, ctypes.POINTER(BlockWeights), i32, vp, vp, vp, vp, i32, i32, i32,
                                         ctypes.c_float, vp, ctypes.c_size_t, vp]
    lib.unipin_block_fold_layernorm.argtypes = [ctypes.POINTER(BlockWeights), i32, vp, vp, vp, vp, vp]
    lib.unipin_pool_status.argtypes = [vp, vp, ip]
    lib.unipin_strerror.argtypes = [i32]
    lib.unipin_strerror.restype = ctypes.c_char_p
    lib.unipin_version.argtypes = []
    for name in EXPORTS:
        if name not in ("unipin_strerror", "unipin_ar_decode_workspace_bytes", "unipin_block_workspace_bytes",
                        "unipin_rank_decode_workspace_bytes",
                        "unipin_pool_generation"):
            getattr(lib, name).restype = ctypes.c_int
    lib.unipin_pool_generation.restype = ctypes.c_uint64
    lib.unipin_ar_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.unipin_rank_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.unipin_block_workspace_bytes.restype = ctypes.c_size_t
    return lib


lib = _load()


class UnipinError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        msg = lib.unipin_strerror(status).decode()
        super().__init__(f"{what}: {msg} (status {status})" if what else f"{msg} (status {status})")


def _check(status: int, what: str) -> None:
    if status != OK:
        raise UnipinError(status, what)


def _dtype_code(dtype: torch.dtype) -> int:
    if dtype == torch.bfloat16:
        return BF16
    if dtype == torch.float32:
        return FP32
    if dtype == torch.float8_e4m3fn:
        return FP8_E4M3
    raise UnipinError(EDTYPE, f"unsupported dtype {dtype}")


def _stream_handle(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


class Pool:
    """KV pool: K and V device tensors [L, S, H, n_max, D] plus the library descriptor.

    The tensors are float32, bfloat16 or float8_e4m3fn; calls on a float8_e4m3fn pool
    take bfloat16 activations (act_dtype).  A pool opened with Pool.import_shared has no
    tensors here (k and v are None): its memory belongs to the process that exported it."""

    _DTYPES = {FP32: torch.float32, BF16: torch.bfloat16, FP8_E4M3: torch.float8_e4m3fn}

    def __init__(self, k_pool: torch.Tensor, v_pool: torch.Tensor):
        if k_pool.shape != v_pool.shape or k_pool.dim() != 5:
            raise UnipinError(EINVAL, "k_pool and v_pool must both be [L, S, H, n_max, D]")
        if k_pool.dtype != v_pool.dtype or not k_pool.is_contiguous() or not v_pool.is_contiguous():
            raise UnipinError(EINVAL, "pool tensors must be contiguous and of one dtype")
        self.k, self.v = k_pool, v_pool
        self.device = k_pool.device
        h = ctypes.c_void_p()
        L, S, H, n_max, D = k_pool.shape
        _check(lib.unipin_pool_create(ctypes.byref(h), k_pool.data_ptr(), v_pool.data_ptr(),
                                      L, S, H, n_max, D, _dtype_code(k_pool.dtype)), "unipin_pool_create")
        self._h = h
        self._read_dims()

    def _read_dims(self) -> None:
        d = [ctypes.c_int() for _ in range(6)]
        _check(lib.unipin_pool_dims(self._h, *[ctypes.byref(x) for x in d]), "unipin_pool_dims")
        self.L, self.S, self.H, self.n_max, self.D, code = (x.value for x in d)
        self.dtype = self._DTYPES[code]
        # the element type of the tensors a call takes: an E4M3 pool works on bf16
        self.act_dtype = torch.bfloat16 if self.dtype == torch.float8_e4m3fn else self.dtype

    @classmethod
    def allocate(cls, L, S, H, n_max, D, dtype=torch.bfloat16, device="cuda") -> "Pool":
        shape = (L, S, H, n_max, D)
        return cls(torch.empty(shape, dtype=dtype, device=device),
                   torch.empty(shape, dtype=dtype, device=device))

    @classmethod
    def import_shared(cls, path: str, device=None) -> "Pool":
        """unipin_pool_import: a read-only view, in this process, of a pool that another
        process exported to `path` (rank_decode only)."""
        dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
        self = cls.__new__(cls)
        self.k = self.v = None
        self.device = dev
        h = ctypes.c_void_p()
        with torch.cuda.device(dev):
            _check(lib.unipin_pool_import(ctypes.byref(h), os.fsencode(path)), "unipin_pool_import")
        self._h = h
        self._read_dims()
        return self

    def export(self, path: str) -> None:
        """unipin_pool_export: writes the share file other processes import (IPC handles of
        the two arrays, the shared page of the slot generations)."""
        with torch.cuda.device(self.device):
            _check(lib.unipin_pool_export(self.handle, os.fsencode(path)), "unipin_pool_export")

    @property
    def handle(self) -> ctypes.c_void_p:
        if self._h is None:
            raise UnipinError(EINVAL, "pool already closed")
        return self._h

    def acquire(self):
        """Next slot, round-robin; returns (slot, generation)."""
        s, g = ctypes.c_int32(), ctypes.c_uint64()
        _check(lib.unipin_pool_acquire(self.handle, ctypes.byref(s), ctypes.byref(g)), "unipin_pool_acquire")
        return s.value, g.value

    def acquire_many(self, count: int) -> List[int]:
        return [self.acquire()[0] for _ in range(count)]

    def generation(self, slot: int) -> int:
        """unipin_pool_generation: hand-outs of `slot` so far (0 also for a slot outside [0, S))."""
        return int(lib.unipin_pool_generation(self.handle, int(slot)))

    def status(self, stream: Optional[torch.cuda.Stream] = None) -> int:
        """unipin_pool_status: the sticky flags (FLAG_BAD_SLOT | FLAG_BAD_LEN |
        FLAG_DUP_SLOT) that kernels of calls on this pool raised since the last call;
        clears them.  Synchronises `stream` (default: the current stream of the pool's
        device)."""
        st = stream.cuda_stream if stream is not None else _stream_handle(self.device)
        flags = ctypes.c_int()
        with torch.cuda.device(self.device):
            rc = lib.unipin_pool_status(self.handle, st, ctypes.byref(flags))
        if rc not in (OK, EDEVICE):
            raise UnipinError(rc, "unipin_pool_status")
        return flags.value

    def close(self) -> None:
        if getattr(self, "_h", None) is not None:
            lib.unipin_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _i32_on(x, device) -> torch.Tensor:
    t = torch.as_tensor(x, dtype=torch.int32)
    if t.device != device:
        t = t.to(device, non_blocking=True)
    return t.contiguous()


def _check_tensor(t: torch.Tensor, name: str, shape, dtype, device) -> None:
    if t.dtype != dtype:
        raise UnipinError(EDTYPE, f"{name} has dtype {t.dtype}, pool holds {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise UnipinError(EINVAL, f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise UnipinError(EINVAL, f"{name} must be contiguous")
    if t.device != device:
        raise UnipinError(EINVAL, f"{name} is on {t.device}, pool is on {device}")


def prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, lens, pool: Pool, slot,
            layer: int, o: Optional[torch.Tensor] = None, scale: Optional[float] = None) -> torch.Tensor:
    """unipin_prefill: causal attention over each history, K/V written to pool slots.

    q, k, v [B, H, n, D]; lens, slot: B ints (device tensor or anything torch.as_tensor takes).
    Returns o [B, H, n, D] (rows >= lens[b] are left as they were).
    """
    dev = pool.device
    B, H, n, D = q.shape
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(t, name, (B, pool.H, n, pool.D), pool.act_dtype, dev)
    if o is None:
        o = torch.empty_like(q)
    _check_tensor(o, "o", q.shape, pool.act_dtype, dev)
    lens_t, slot_t = _i32_on(lens, dev), _i32_on(slot, dev)
    if lens_t.numel() != B or slot_t.numel() != B:
        raise UnipinError(EINVAL, "lens and slot need one entry per user")
    _check(lib.unipin_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(), lens_t.data_ptr(),
                              pool.handle, slot_t.data_ptr(), layer, B, n,
                              0.0 if scale is None else float(scale), o.data_ptr(),
                              _stream_handle(dev)), "unipin_prefill")
    return o


def rank_decode_workspace_bytes(pool: Pool, B: int, k: int) -> int:
    """unipin_rank_decode_workspace_bytes: bytes rank_decode(split=True) uses for B users of
    k candidates (0: it runs the one-pass kernel)."""
    return int(lib.unipin_rank_decode_workspace_bytes(pool.handle, int(B), int(k)))


def rank_decode(qc: torch.Tensor, kc: torch.Tensor, vc: torch.Tensor, pool: Pool, slot, lens,
                layer: int, oc: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                split: bool = False, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """unipin_rank_decode: candidates attend to their slot's cached history plus themselves.

    qc, kc, vc [B, H, k, D]; slot, lens: B ints.  Returns oc [B, H, k, D].  split=True calls
    unipin_rank_decode_split, which splits each candidate tile's history over several
    workgroups when B*H pairs are too few to fill the GPU, with `workspace` (a device
    tensor of at least rank_decode_workspace_bytes(pool, B, k) bytes) or, when it is None,
    a buffer from torch's caching allocator.
    """
    dev = pool.device
    B, H, kk, D = qc.shape
    for name, t in (("qc", qc), ("kc", kc), ("vc", vc)):
        _check_tensor(t, name, (B, pool.H, kk, pool.D), pool.act_dtype, dev)
    if oc is None:
        oc = torch.empty_like(qc)
    _check_tensor(oc, "oc", qc.shape, pool.act_dtype, dev)
    lens_t, slot_t = _i32_on(lens, dev), _i32_on(slot, dev)
    if lens_t.numel() != B or slot_t.numel() != B:
        raise UnipinError(EINVAL, "lens and slot need one entry per user")
    sc = 0.0 if scale is None else float(scale)
    if not split:
        _check(lib.unipin_rank_decode(qc.data_ptr(), kc.data_ptr(), vc.data_ptr(), pool.handle,
                                      slot_t.data_ptr(), lens_t.data_ptr(), layer, B, kk, sc, oc.data_ptr(),
                                      _stream_handle(dev)), "unipin_rank_decode")
        return oc
    need = rank_decode_workspace_bytes(pool, B, kk)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        if workspace.device != dev or not workspace.is_contiguous():
            raise UnipinError(EINVAL, "workspace must be a contiguous tensor on the pool's device")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    _check(lib.unipin_rank_decode_split(qc.data_ptr(), kc.data_ptr(), vc.data_ptr(), pool.handle,
                                        slot_t.data_ptr(), lens_t.data_ptr(), layer, B, kk, sc, oc.data_ptr(),
                                        ws_ptr, ws_bytes, _stream_handle(dev)), "unipin_rank_decode_split")
    return oc


def ar_decode_workspace_bytes(pool: Pool, B: int) -> int:
    """unipin_ar_decode_workspace_bytes: scratch bytes ar_decode splits B users' rows with (0: none)."""
    return int(lib.unipin_ar_decode_workspace_bytes(pool.handle, int(B)))


def ar_decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, pool: Pool, slot, lens,
              layer: int, o: Optional[torch.Tensor] = None, scale: Optional[float] = None,
              workspace: Optional[torch.Tensor] = None, split: bool = True) -> torch.Tensor:
    """unipin_ar_decode: one autoregressive retrieval step on the pool.

    q, k, v [B, H, 1, D]: each user's new token; slot, lens: B ints, lens[b] = rows already
    in the slot at this layer (the new token's position).  Stores k/v at row lens[b] and
    returns o [B, H, 1, D].  lens is not advanced; the caller does that after the step.
    split=True lets the library split each user's rows across workgroups, with `workspace`
    (a device tensor of at least ar_decode_workspace_bytes(pool, B) bytes) or, when it is
    None, a buffer from torch's caching allocator; split=False runs the one-pass kernel.
    """
    dev = pool.device
    B = q.shape[0]
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(t, name, (B, pool.H, 1, pool.D), pool.act_dtype, dev)
    if o is None:
        o = torch.empty_like(q)
    _check_tensor(o, "o", q.shape, pool.act_dtype, dev)
    lens_t, slot_t = _i32_on(lens, dev), _i32_on(slot, dev)
    if lens_t.numel() != B or slot_t.numel() != B:
        raise UnipinError(EINVAL, "lens and slot need one entry per user")
    ws_ptr, ws_bytes = None, 0
    if split:
        need = ar_decode_workspace_bytes(pool, B)
        if workspace is None and need:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        if workspace is not None:
            if workspace.device != dev or not workspace.is_contiguous():
                raise UnipinError(EINVAL, "workspace must be a contiguous tensor on the pool's device")
            ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    _check(lib.unipin_ar_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), pool.handle,
                                slot_t.data_ptr(), lens_t.data_ptr(), layer, B,
                                0.0 if scale is None else float(scale), o.data_ptr(),
                                ws_ptr, ws_bytes, _stream_handle(dev)), "unipin_ar_decode")
    return o


class BlockContext:
    """unipin_block_ctx_create/destroy: GEMM plans for the current device."""

    def __init__(self):
        h = ctypes.c_void_p()
        _check(lib.unipin_block_ctx_create(ctypes.byref(h)), "unipin_block_ctx_create")
        self._h = h

    @property
    def handle(self):
        if self._h is None:
            raise UnipinError(EINVAL, "block context is closed")
        return self._h

    def set_gemm(self, kernel: int) -> None:
        """unipin_block_ctx_set_gemm: GEMM_AUTO, GEMM_LIBRARY (hipBLASLt) or the library's
        kernel with tile configuration 0, 1, 2 or 3; drops the plans made so far."""
        _check(lib.unipin_block_ctx_set_gemm(self.handle, int(kernel)), "unipin_block_ctx_set_gemm")

    def tune(self, pool: "Pool", B: int, rows: int, workspace: Optional[torch.Tensor] = None) -> None:
        """unipin_block_ctx_tune: time the candidate GEMM kernels (the library's own in each
        tile configuration, hipBLASLt's) for the block at B users x rows rows and keep the fastest
        (blocks until done)."""
        dev = pool.device
        if workspace is None:
            workspace = torch.empty(block_workspace_bytes(pool, B, rows), dtype=torch.uint8, device=dev)
        _check(lib.unipin_block_ctx_tune(self.handle, pool.handle, int(B), int(rows), workspace.data_ptr(),
                                         workspace.numel() * workspace.element_size(), _stream_handle(dev)),
               "unipin_block_ctx_tune")

    def close(self) -> None:
        if getattr(self, "_h", None) is not None:
            lib.unipin_block_ctx_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def block_workspace_bytes(pool: Pool, B: int, rows: int) -> int:
    """unipin_block_workspace_bytes."""
    return int(lib.unipin_block_workspace_bytes(pool.handle, int(B), int(rows)))


def _block_weights(weights, C: int, dev) -> BlockWeights:
    """The weights dict as unipin_block_weights_t, every tensor checked (the folded ones
    only when present)."""
    shapes = {"ln1_w": (C,), "ln1_b": (C,), "w_qkv": (C, 3 * C), "b_qkv": (3 * C,), "w_o": (C, C), "b_o": (C,),
              "ln2_w": (C,), "ln2_b": (C,), "w_fc": (C, 4 * C), "b_fc": (4 * C,), "w_proj": (4 * C, C),
              "b_proj": (C,)}
    folded = {"w_qkv_ln": ((C, 3 * C), torch.bfloat16), "uv_qkv": ((2, 3 * C), torch.float32),
              "w_fc_ln": ((C, 4 * C), torch.bfloat16), "uv_fc": ((2, 4 * C), torch.float32)}
    ptrs = []
    for name in BLOCK_WEIGHT_NAMES:
        if name not in weights:
            raise UnipinError(EINVAL, f"weights lack {name}")
        _check_tensor(weights[name], name, shapes[name], torch.bfloat16, dev)
        ptrs.append(weights[name].data_ptr())
    for name in BLOCK_FOLDED_NAMES:
        if name in weights:
            _check_tensor(weights[name], name, folded[name][0], folded[name][1], dev)
            ptrs.append(weights[name].data_ptr())
        else:
            ptrs.append(None)
    return BlockWeights(*ptrs)


def fold_layernorm(weights) -> dict:
    """unipin_block_fold_layernorm: a copy of the weights dict with the folded LayerNorm
    weights added (w_qkv_ln, uv_qkv, w_fc_ln, uv_fc; new device tensors, enqueued on the
    current stream).  block_forward then may run the QKV and MLP-up projections on the
    hidden state itself."""
    C = weights["ln1_w"].shape[0]
    dev = weights["ln1_w"].device
    bw = _block_weights({k: weights[k] for k in BLOCK_WEIGHT_NAMES}, C, dev)
    out = dict(weights)
    out["w_qkv_ln"] = torch.empty((C, 3 * C), dtype=torch.bfloat16, device=dev)
    out["uv_qkv"] = torch.empty((2, 3 * C), dtype=torch.float32, device=dev)
    out["w_fc_ln"] = torch.empty((C, 4 * C), dtype=torch.bfloat16, device=dev)
    out["uv_fc"] = torch.empty((2, 4 * C), dtype=torch.float32, device=dev)
    _check(lib.unipin_block_fold_layernorm(ctypes.byref(bw), C, out["w_qkv_ln"].data_ptr(), out["uv_qkv"].data_ptr(),
                                           out["w_fc_ln"].data_ptr(), out["uv_fc"].data_ptr(), _stream_handle(dev)),
           "unipin_block_fold_layernorm")
    return out


def block_forward(ctx: BlockContext, weights, mode: int, x: torch.Tensor, pool: Pool, slot, lens, layer: int,
                  scale: Optional[float] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """unipin_block_forward: one transformer block, in place on x [B, rows, C] (bf16).

    weights: a dict with the BLOCK_WEIGHT_NAMES keys (bf16 device tensors; matrices
    row-major [fan_in, fan_out]), and optionally the BLOCK_FOLDED_NAMES ones that
    fold_layernorm adds.  mode: BLOCK_HISTORY (causal over each user's lens[b]
    rows; their k, v go to the pool) or BLOCK_CANDIDATES (the candidates attend to the
    pool's lens[b] rows and themselves).  workspace: a device tensor of at least
    block_workspace_bytes(pool, B, rows) bytes, or None for one from torch's allocator.
    """
    dev = pool.device
    if x.dim() != 3:
        raise UnipinError(EINVAL, "x must be [B, rows, C]")
    B, rows, C = x.shape
    if C != pool.H * pool.D:
        raise UnipinError(EINVAL, f"x has width {C}, the pool's heads give {pool.H * pool.D}")
    _check_tensor(x, "x", (B, rows, C), torch.bfloat16, dev)
    bw = _block_weights(weights, C, dev)
    lens_t, slot_t = _i32_on(lens, dev), _i32_on(slot, dev)
    if lens_t.numel() != B or slot_t.numel() != B:
        raise UnipinError(EINVAL, "lens and slot need one entry per user")
    need = block_workspace_bytes(pool, B, rows)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace.device != dev or not workspace.is_contiguous():
        raise UnipinError(EINVAL, "workspace must be a contiguous tensor on the pool's device")
    _check(lib.unipin_block_forward(ctx.handle, ctypes.byref(bw), int(mode), x.data_ptr(), pool.handle,
                                    slot_t.data_ptr(), lens_t.data_ptr(), layer, B, rows,
                                    0.0 if scale is None else float(scale), workspace.data_ptr(),
                                    workspace.numel() * workspace.element_size(), _stream_handle(dev)),
           "unipin_block_forward")
    return x


def version() -> int:
    return lib.unipin_version()
