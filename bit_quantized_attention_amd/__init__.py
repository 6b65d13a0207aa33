"""Python binding of libqattn (8-bit quantized, optionally block-sparse attention
forward for MI355X / gfx950).

The functions ``qattn_smooth_quant``, ``qattn_block_mask``, ``qattn_fwd`` and the
size helpers carry the names of the C entry points declared in
``include/qattn.h`` and only marshal arguments: torch tensors supply device
memory, torch's current HIP stream supplies the stream, and every step of the
computation runs in the library's HIP kernels. There is no fallback: if the
shared library is not built, ``load()`` raises.

``attention(q, k, v, causal, sparse)`` chains the three calls with freshly
allocated intermediates; ``Plan`` does the same with intermediates allocated once
(for repeated calls on one shape).
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqattn.so")

QATTN_F16 = 0
QATTN_BF16 = 1
Q_BLOCK = 128
K_BLOCK = 64
KV_TILE = 64
# the attention kernel's online-softmax reference threshold
# (QATTN_SOFTMAX_REF_THRESHOLD in include/qattn.h)
SOFTMAX_REF_THRESHOLD = 8

_STATUS = {0: "QATTN_OK", 1: "QATTN_ERR_NULL", 2: "QATTN_ERR_SHAPE", 3: "QATTN_ERR_ALIGN",
           4: "QATTN_ERR_UNSUPPORTED", 5: "QATTN_ERR_ARG", 6: "QATTN_ERR_DEVICE",
           7: "QATTN_ERR_SCRATCH"}
# size of the allocation-free smoothing entry point's static scratch
# (QATTN_NOALLOC_SCRATCH_BYTES in include/qattn.h)
NOALLOC_SCRATCH_BYTES = 16 << 20
# Most vertical or slash lines per head (QATTN_MAX_PATTERN_LINES)
MAX_PATTERN_LINES = 64

_lib = None


class QattnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = qattn_status_str(status) if _lib is not None else ""
        super().__init__(f"{where}: {_STATUS.get(status, status)} ({msg})")


class qattn_problem_t(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("N", ctypes.c_int32), ("d", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("causal", ctypes.c_int32)]


def load(path: str = LIB_PATH):
    """Load libqattn.so (once). Raises ImportError when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m bit_quantized_attention_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    P = ctypes.POINTER(qattn_problem_t)
    lib.qattn_status_str.argtypes = [ctypes.c_int]
    lib.qattn_status_str.restype = ctypes.c_char_p
    lib.qattn_version.argtypes = []
    lib.qattn_version.restype = ctypes.c_char_p
    lib.qattn_workspace_bytes.argtypes = [P]
    lib.qattn_workspace_bytes.restype = sz
    lib.qattn_max_keep.argtypes = [P, i32, i32]
    lib.qattn_max_keep.restype = i32
    lib.qattn_smooth_quant.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.qattn_smooth_quant.restype = ctypes.c_int
    lib.qattn_smooth_quant_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.qattn_smooth_quant_noalloc.restype = ctypes.c_int
    lib.qattn_fwd_promoted_fp4.argtypes = [P, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, sz, vp]
    lib.qattn_fwd_promoted_fp4.restype = ctypes.c_int
    lib.qattn_block_mask.argtypes = [P, vp, vp, i32, i32, i32, vp, vp, vp, sz, vp]
    lib.qattn_block_mask.restype = ctypes.c_int
    lib.qattn_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp]
    lib.qattn_fwd.restype = ctypes.c_int
    lib.qattn_fwd_promoted.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp]
    lib.qattn_fwd_promoted.restype = ctypes.c_int
    lib.qattn_lowbit_workspace_bytes.argtypes = [P]
    lib.qattn_lowbit_workspace_bytes.restype = sz
    lib.qattn_block_mask_lowbit.argtypes = [P, vp, vp, vp, i32, i32, i32, vp, vp, vp, vp, sz, vp]
    lib.qattn_block_mask_lowbit.restype = ctypes.c_int
    lib.qattn_block_mask_patterns.argtypes = [P, vp, vp, i32, i32, i32, vp, vp, i32, vp, vp]
    lib.qattn_block_mask_patterns.restype = ctypes.c_int
    lib.qattn_stripe_select.argtypes = [P, vp, vp, vp, ctypes.c_float, i32, vp, vp, vp]
    lib.qattn_stripe_select.restype = ctypes.c_int
    lib.qattn_fwd_stripes.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp]
    lib.qattn_fwd_stripes.restype = ctypes.c_int
    lib.qattn_head_error.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp]
    lib.qattn_head_error.restype = ctypes.c_int
    lib.qattn_fwd_adaptive.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.qattn_fwd_adaptive.restype = ctypes.c_int
    _lib = lib
    return lib


# ---- marshalling helpers -------------------------------------------------------

def _ptr(t) -> Optional[int]:
    """Device address of a tensor (None -> NULL); ints pass through."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str):
    if status != 0:
        raise QattnError(status, where)


def problem(B: int, Hq: int, Hkv: int, N: int, d: int, dtype, causal: bool) -> qattn_problem_t:
    """Build a qattn_problem_t; dtype is "f16"/"bf16", a torch dtype, or 0/1."""
    if not isinstance(dtype, int):
        name = str(dtype)
        if "bfloat16" in name or name == "bf16":
            dtype = QATTN_BF16
        elif "float16" in name or name == "f16":
            dtype = QATTN_F16
        else:
            raise ValueError(f"unsupported dtype {dtype}")
    return qattn_problem_t(B, Hq, Hkv, N, d, dtype, int(bool(causal)) if causal in (0, 1, True, False) else causal)


def problem_of(q, k, causal: bool) -> qattn_problem_t:
    B, Hq, N, d = q.shape
    return problem(B, Hq, k.shape[1], N, d, q.dtype, causal)


# ---- the C entry points ----------------------------------------------------------

def qattn_status_str(status: int) -> str:
    return load().qattn_status_str(status).decode()


def qattn_version() -> str:
    return load().qattn_version().decode()


def qattn_workspace_bytes(p: qattn_problem_t) -> int:
    return load().qattn_workspace_bytes(ctypes.byref(p))


def qattn_max_keep(p: qattn_problem_t, keep_num: int, keep_den: int) -> int:
    return load().qattn_max_keep(ctypes.byref(p), keep_num, keep_den)


def qattn_smooth_quant(p, q, k, q_i8, q_scale, k_i8, k_scale, k_mean, q_pool, k_pool,
                       workspace, workspace_bytes=None, stream=None, check=True) -> int:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    st = load().qattn_smooth_quant(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(q_i8), _ptr(q_scale),
                                   _ptr(k_i8), _ptr(k_scale), _ptr(k_mean), _ptr(q_pool),
                                   _ptr(k_pool), _ptr(workspace), workspace_bytes,
                                   _stream(stream))
    if check:
        _check(st, "qattn_smooth_quant")
    return st


def qattn_smooth_quant_noalloc(p, q, k, q_i8, q_scale, k_i8, k_scale, k_mean, q_pool, k_pool,
                               stream=None, check=True) -> int:
    st = load().qattn_smooth_quant_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(q_i8),
                                           _ptr(q_scale), _ptr(k_i8), _ptr(k_scale), _ptr(k_mean),
                                           _ptr(q_pool), _ptr(k_pool), _stream(stream))
    if check:
        _check(st, "qattn_smooth_quant_noalloc")
    return st


def qattn_fwd_promoted_fp4(p, q, k, k_mean, v, kv_idx, kv_cnt, max_keep, o, lse, workspace,
                           workspace_bytes=None, stream=None, check=True) -> int:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    st = load().qattn_fwd_promoted_fp4(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(k_mean), _ptr(v),
                                       _ptr(kv_idx), _ptr(kv_cnt), max_keep, _ptr(o), _ptr(lse),
                                       _ptr(workspace), workspace_bytes, _stream(stream))
    if check:
        _check(st, "qattn_fwd_promoted_fp4")
    return st


def qattn_block_mask(p, q_pool, k_pool, keep_num, keep_den, max_keep, kv_idx, kv_cnt,
                     workspace, workspace_bytes=None, stream=None, check=True) -> int:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    st = load().qattn_block_mask(ctypes.byref(p), _ptr(q_pool), _ptr(k_pool), keep_num, keep_den,
                                 max_keep, _ptr(kv_idx), _ptr(kv_cnt), _ptr(workspace),
                                 workspace_bytes, _stream(stream))
    if check:
        _check(st, "qattn_block_mask")
    return st


def qattn_fwd(p, q_i8, q_scale, k_i8, k_scale, v, kv_idx, kv_cnt, max_keep, o, lse=None,
              stream=None, check=True) -> int:
    st = load().qattn_fwd(ctypes.byref(p), _ptr(q_i8), _ptr(q_scale), _ptr(k_i8), _ptr(k_scale),
                          _ptr(v), _ptr(kv_idx), _ptr(kv_cnt), max_keep, _ptr(o), _ptr(lse),
                          _stream(stream))
    if check:
        _check(st, "qattn_fwd")
    return st


def qattn_fwd_promoted(p, q_i8, q_scale, k_i8, k_scale, q, k, k_mean, v, kv_idx, kv_cnt,
                       max_keep, o, lse=None, stream=None, check=True) -> int:
    st = load().qattn_fwd_promoted(ctypes.byref(p), _ptr(q_i8), _ptr(q_scale), _ptr(k_i8),
                                   _ptr(k_scale), _ptr(q), _ptr(k), _ptr(k_mean), _ptr(v),
                                   _ptr(kv_idx), _ptr(kv_cnt), max_keep, _ptr(o), _ptr(lse),
                                   _stream(stream))
    if check:
        _check(st, "qattn_fwd_promoted")
    return st


def qattn_lowbit_workspace_bytes(p: qattn_problem_t) -> int:
    return int(load().qattn_lowbit_workspace_bytes(ctypes.byref(p)))


def qattn_block_mask_lowbit(p, q, k, k_mean, keep_num, keep_den, max_keep, kv_idx, kv_cnt,
                            scores, workspace, workspace_bytes=None, stream=None,
                            check=True) -> int:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    st = load().qattn_block_mask_lowbit(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(k_mean),
                                        keep_num, keep_den, max_keep, _ptr(kv_idx),
                                        _ptr(kv_cnt), _ptr(scores), _ptr(workspace),
                                        workspace_bytes, _stream(stream))
    if check:
        _check(st, "qattn_block_mask_lowbit")
    return st


def qattn_block_mask_patterns(p, kv_idx, kv_cnt, max_keep, n_vertical, n_slash, kv_idx_out,
                              kv_cnt_out, max_keep_out, lines, stream=None, check=True) -> int:
    st = load().qattn_block_mask_patterns(ctypes.byref(p), _ptr(kv_idx), _ptr(kv_cnt), max_keep,
                                          n_vertical, n_slash, _ptr(kv_idx_out), _ptr(kv_cnt_out),
                                          max_keep_out, _ptr(lines), _stream(stream))
    if check:
        _check(st, "qattn_block_mask_patterns")
    return st


def qattn_stripe_select(p, q_pool, k_i8, k_scale, theta, max_keys, key_idx, key_cnt,
                        stream=None, check=True) -> int:
    st = load().qattn_stripe_select(ctypes.byref(p), _ptr(q_pool), _ptr(k_i8), _ptr(k_scale),
                                    float(theta), max_keys, _ptr(key_idx), _ptr(key_cnt),
                                    _stream(stream))
    if check:
        _check(st, "qattn_stripe_select")
    return st


def qattn_fwd_stripes(p, q_i8, q_scale, k_i8, k_scale, v, key_idx, key_cnt, max_keys, o,
                      lse=None, stream=None, check=True) -> int:
    st = load().qattn_fwd_stripes(ctypes.byref(p), _ptr(q_i8), _ptr(q_scale), _ptr(k_i8),
                                  _ptr(k_scale), _ptr(v), _ptr(key_idx), _ptr(key_cnt), max_keys,
                                  _ptr(o), _ptr(lse), _stream(stream))
    if check:
        _check(st, "qattn_fwd_stripes")
    return st


def qattn_head_error(p, q_i8, q_scale, k_i8, k_scale, q, k, k_mean, threshold, head_err,
                     head_hi=None, stream=None, check=True) -> int:
    st = load().qattn_head_error(ctypes.byref(p), _ptr(q_i8), _ptr(q_scale), _ptr(k_i8),
                                 _ptr(k_scale), _ptr(q), _ptr(k), _ptr(k_mean), float(threshold),
                                 _ptr(head_err), _ptr(head_hi), _stream(stream))
    if check:
        _check(st, "qattn_head_error")
    return st


def qattn_fwd_adaptive(p, q_i8, q_scale, k_i8, k_scale, q, k, k_mean, v, head_hi, o, lse=None,
                       stream=None, check=True) -> int:
    st = load().qattn_fwd_adaptive(ctypes.byref(p), _ptr(q_i8), _ptr(q_scale), _ptr(k_i8),
                                   _ptr(k_scale), _ptr(q), _ptr(k), _ptr(k_mean), _ptr(v),
                                   _ptr(head_hi), _ptr(o), _ptr(lse), _stream(stream))
    if check:
        _check(st, "qattn_fwd_adaptive")
    return st


# ---- convenience: allocate intermediates and chain the calls ----------------------

@dataclass
class Plan:
    """Intermediates for one problem shape, allocated once on ``device``.

    ``sparse`` is None (dense) or a keep ratio (keep_num, keep_den). With
    ``promote`` the kept blocks are computed at 16-bit Q K^T and every other
    block through the INT8 path, instead of being skipped; ``low4`` (with
    ``promote``) takes those other blocks at MX FP4 Q K^T instead of INT8.
    ``patterns`` = (n_vertical, n_slash) extends the mask's kept lists with
    each head's predicted vertical and slash lines before the attention.
    """

    p: qattn_problem_t
    device: object
    sparse: Optional[Tuple[int, int]] = None
    with_lse: bool = False
    pools: Optional[bool] = None  # pooled block means; default: only when sparse
    promote: bool = False
    low4: bool = False
    patterns: Optional[Tuple[int, int]] = None

    def __post_init__(self):
        import torch
        if self.promote and self.sparse is None:
            raise ValueError("promote needs a keep ratio (the blocks to promote)")
        if self.low4 and not self.promote:
            raise ValueError("low4 is the low path of promote")
        p, dev = self.p, self.device
        B, Hq, Hkv, N, d = p.B, p.Hq, p.Hkv, p.N, p.d
        nqb, nkb = N // Q_BLOCK, N // K_BLOCK
        e = dict(device=dev)
        self.q_i8 = torch.empty((B, Hq, N, d), dtype=torch.int8, **e)
        self.q_scale = torch.empty((B, Hq, nqb), dtype=torch.float32, **e)
        self.k_i8 = torch.empty((B, Hkv, N, d), dtype=torch.int8, **e)
        self.k_scale = torch.empty((B, Hkv, nkb), dtype=torch.float32, **e)
        self.k_mean = torch.empty((B, Hkv, d), dtype=torch.float32, **e)
        self.workspace = torch.empty(max(16, qattn_workspace_bytes(p)), dtype=torch.uint8, **e)
        self.q_pool = self.k_pool = self.kv_idx = self.kv_cnt = None
        self.max_keep = 0
        if self.pools or (self.pools is None and self.sparse is not None):
            self.q_pool = torch.empty((B, Hq, nqb, d), dtype=torch.float32, **e)
            self.k_pool = torch.empty((B, Hkv, nkb, d), dtype=torch.float32, **e)
        if self.sparse is not None:
            if self.q_pool is None:
                raise ValueError("a sparse plan needs the pooled block means")
            num, den = self.sparse
            self.max_keep = qattn_max_keep(p, num, den)
            if self.max_keep < 0:
                raise ValueError(f"invalid keep ratio {self.sparse}")
            self.kv_idx = torch.empty((B, Hq, nqb, self.max_keep), dtype=torch.int32, **e)
            self.kv_cnt = torch.empty((B, Hq, nqb), dtype=torch.int32, **e)
        # the mask's own lists (the attention's lists unless patterns extend them)
        self.mask_keep, self.mask_idx, self.mask_cnt = self.max_keep, self.kv_idx, self.kv_cnt
        self.lines = None
        if self.patterns is not None:
            if self.sparse is None:
                raise ValueError("patterns extend a block mask: a keep ratio is needed")
            nv, ns = self.patterns
            self.lines = torch.empty((B, Hq, max(1, nv + ns)), dtype=torch.int32, **e)
            self.max_keep = min(nkb, self.mask_keep + nv + ns)
            self.kv_idx = torch.empty((B, Hq, nqb, self.max_keep), dtype=torch.int32, **e)
            self.kv_cnt = torch.empty((B, Hq, nqb), dtype=torch.int32, **e)
        self.lse = torch.empty((B, Hq, N), dtype=torch.float32, **e) if self.with_lse else None
        self.workspace4 = None
        if self.low4:
            self.workspace4 = torch.empty(max(16, qattn_lowbit_workspace_bytes(p)),
                                          dtype=torch.uint8, **e)

    def smooth_quant(self, q, k, stream=None):
        qattn_smooth_quant(self.p, q, k, self.q_i8, self.q_scale, self.k_i8, self.k_scale,
                           self.k_mean, self.q_pool, self.k_pool, self.workspace, stream=stream)

    def block_mask(self, stream=None):
        num, den = self.sparse
        qattn_block_mask(self.p, self.q_pool, self.k_pool, num, den, self.mask_keep,
                         self.mask_idx, self.mask_cnt, self.workspace, stream=stream)
        if self.patterns is not None:
            self.extend_patterns(stream)

    def extend_patterns(self, stream=None):
        """The mask's lists extended by each head's vertical and slash lines."""
        nv, ns = self.patterns
        qattn_block_mask_patterns(self.p, self.mask_idx, self.mask_cnt, self.mask_keep, nv, ns,
                                  self.kv_idx, self.kv_cnt, self.max_keep, self.lines,
                                  stream=stream)

    def fwd(self, v, o, stream=None):
        qattn_fwd(self.p, self.q_i8, self.q_scale, self.k_i8, self.k_scale, v, self.kv_idx,
                  self.kv_cnt, self.max_keep, o, self.lse, stream=stream)

    def fwd_promoted(self, q, k, v, o, stream=None):
        qattn_fwd_promoted(self.p, self.q_i8, self.q_scale, self.k_i8, self.k_scale, q, k,
                           self.k_mean, v, self.kv_idx, self.kv_cnt, self.max_keep, o, self.lse,
                           stream=stream)

    def fwd_promoted_fp4(self, q, k, v, o, stream=None):
        qattn_fwd_promoted_fp4(self.p, q, k, self.k_mean, v, self.kv_idx, self.kv_cnt,
                               self.max_keep, o, self.lse, self.workspace4, stream=stream)

    def run(self, q, k, v, o, stream=None):
        """The whole path: smooth + quantize, [block mask], attention."""
        self.smooth_quant(q, k, stream)
        if self.sparse is not None:
            self.block_mask(stream)
        if self.low4:
            self.fwd_promoted_fp4(q, k, v, o, stream)
        elif self.promote:
            self.fwd_promoted(q, k, v, o, stream)
        else:
            self.fwd(v, o, stream)
        return o


def attention(q, k, v, causal: bool = False, sparse: Optional[Tuple[int, int]] = None,
              return_plan: bool = False, with_lse: bool = False, promote: bool = False,
              low4: bool = False):
    """O = attention(Q, K, V) through the quantized path; Q [B,Hq,N,d], K/V [B,Hkv,N,d].

    ``sparse`` = (keep_num, keep_den) keeps the first, diagonal and top blocks
    per query block and skips the rest; with ``promote`` those blocks run at
    16-bit Q K^T and the rest through the INT8 path instead (``low4``: at MX
    FP4 Q K^T).
    """
    import torch
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be device tensors")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share one dtype")
    plan = Plan(problem_of(q, k, causal), q.device, sparse, with_lse, promote=promote, low4=low4)
    o = torch.empty_like(q)
    plan.run(q, k, v, o)
    return (o, plan) if return_plan else o
