"""One rank's shard of a tensor-parallel transformer layer on MI355X (gfx950).

Thin Python binding over the C ABI of ``libtpshard.so`` (include/tp_shard.h):
argument checking and marshalling only.  Every step of the layer runs in the
library's HIP kernels; PyTorch supplies device memory and streams.

    shard = Shard(4096, 32, 32, 11008, tp=2, rank=0)      # bf16, SwiGLU, RMSNorm, RoPE
    shard.load_weights(full_weights)                      # dict of FULL device tensors
    kv = shard.kv_cache(batch, max_seq)
    pa = shard.prefill(ATTN, x, kv)                       # fp32 partial [B, S, h]
    h = partial_reduce([pa, *other_ranks], residual=x)    # h = x + sum of partials
    pm = shard.prefill(MLP, h)
    y = partial_reduce([pm, *other_ranks], residual=h)
"""

from __future__ import annotations

import ctypes as C

import torch  # loaded first so that the library binds to torch's HIP runtime

from . import _native as N
from ._native import (TP_ACT_GELU, TP_ACT_SWIGLU, TP_BF16, TP_F32, TPError, TP_E_ARG, TP_E_DIVIDE,  # noqa: F401
                      TP_E_HIP, TP_E_KV_FULL, TP_E_NOMEM, TP_E_RANK, TP_E_STATE, TP_OK)

ATTN = N.TP_STAGE_ATTN
MLP = N.TP_STAGE_MLP
PRENORM = N.TP_STAGE_PRENORM   # OR into a stage whose input is already normalised

_DT = {"bf16": (N.TP_BF16, torch.bfloat16), "f32": (N.TP_F32, torch.float32)}


def _stream(stream) -> C.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None) -> C.c_void_p:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name}: expected a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    return C.c_void_p(t.data_ptr())


_hip = None


def _memcpy_d2d(dst_ptr: int, src_ptr: int, nbytes: int, stream=None) -> None:
    """Device-to-device copy on the stream (hipMemcpyAsync of the HIP runtime
    torch already loaded)."""
    global _hip
    if _hip is None:
        _hip = C.CDLL("libamdhip64.so.7")
        _hip.hipMemcpyAsync.restype = C.c_int
        _hip.hipMemcpyAsync.argtypes = [C.c_void_p, C.c_void_p, C.c_size_t, C.c_int, C.c_void_p]
    err = _hip.hipMemcpyAsync(C.c_void_p(dst_ptr), C.c_void_p(src_ptr), nbytes, 3, _stream(stream))
    if err != 0:
        raise RuntimeError(f"hipMemcpyAsync failed with HIP error {err}")


class KVCache:
    """K/V cache of one rank's KV heads: K and V [batch, kv_heads/t, max_seq, d],
    or (paged) pools [num_blocks, kv_heads/t, block_size, d] with a block table."""

    def __init__(self, shard: "Shard", batch: int, max_seq: int, block_size: int = 0, num_blocks: int = 0):
        h = C.c_void_p()
        if block_size:
            N.check(N.lib().tp_kv_create_paged(shard._h, batch, max_seq, block_size, num_blocks, C.byref(h)),
                    "tp_kv_create_paged")
            self.shape = (num_blocks, shard.kv_local, block_size, shard.head_dim)
            self.max_blocks = -(-max_seq // block_size)
        else:
            N.check(N.lib().tp_kv_create(shard._h, batch, max_seq, C.byref(h)), "tp_kv_create")
            self.shape = (batch, shard.kv_local, max_seq, shard.head_dim)
        self._h = h
        self.shard = shard
        self.batch, self.max_seq, self.block_size = batch, max_seq, block_size
        k, v = C.c_void_p(), C.c_void_p()
        N.check(N.lib().tp_kv_view(h, C.byref(k), C.byref(v)), "tp_kv_view")
        self._k, self._v = k.value, v.value

    def set_block_table(self, table) -> None:
        """Block ids [batch, ceil(max_seq / block_size)] (paged caches)."""
        import numpy as np
        t = np.ascontiguousarray(np.asarray(table, dtype=np.int32))
        if t.shape != (self.batch, self.max_blocks):
            raise ValueError(f"block table must be {(self.batch, self.max_blocks)}")
        N.check(N.lib().tp_kv_set_block_table(self._h, t.ctypes.data_as(C.c_void_p)), "tp_kv_set_block_table")

    @property
    def nbytes(self) -> int:
        n = 1
        for s in self.shape:
            n *= s
        return n * self.shard.elem_size

    @property
    def length(self) -> int:
        n = C.c_int()
        N.check(N.lib().tp_kv_get_len(self._h, C.byref(n)), "tp_kv_get_len")
        return n.value

    @length.setter
    def length(self, n: int) -> None:
        N.check(N.lib().tp_kv_set_len(self._h, int(n)), "tp_kv_set_len")

    def set_length_async(self, n: int, stream=None) -> None:
        """Set the length (and clear the overflow flag) in the stream's order."""
        N.check(N.lib().tp_kv_set_len_async(self._h, int(n), _stream(stream)), "tp_kv_set_len_async")

    def length_on(self, stream=None) -> int:
        """The length, waiting for the stream only."""
        n = C.c_int()
        N.check(N.lib().tp_kv_get_len_stream(self._h, C.byref(n), _stream(stream)), "tp_kv_get_len_stream")
        return n.value

    def write(self, k: torch.Tensor, v: torch.Tensor, stream=None) -> None:
        """Copy whole caches in (device tensors of the cache's shape and dtype)."""
        for name, src, dst in (("k", k, self._k), ("v", v, self._v)):
            _dev(src, name, self.shard.torch_dtype, self.shape)
            _memcpy_d2d(dst, src.data_ptr(), self.nbytes, stream)

    def copy_from(self, other: "KVCache", stream=None) -> None:
        """Copy another cache of the same shape (both K and V arrays)."""
        if other.shape != self.shape or other.shard.torch_dtype != self.shard.torch_dtype:
            raise ValueError("KV caches differ in shape or dtype")
        _memcpy_d2d(self._k, other._k, self.nbytes, stream)
        _memcpy_d2d(self._v, other._v, self.nbytes, stream)

    def read(self, stream=None):
        """Copies of the K and V arrays as device tensors."""
        out = []
        for src in (self._k, self._v):
            t = torch.empty(self.shape, dtype=self.shard.torch_dtype, device="cuda")
            _memcpy_d2d(t.data_ptr(), src, self.nbytes, stream)
            out.append(t)
        return tuple(out)

    def close(self) -> None:
        if self._h:
            N.lib().tp_kv_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Shard:
    """Rank ``rank`` of a layer split ``tp`` ways."""

    def __init__(self, hidden: int, heads: int, kv_heads: int, ffn: int, tp: int = 1, rank: int = 0, *,
                 dtype: str = "bf16", act: str = "swiglu", rmsnorm: bool = True, eps: float = 1e-5,
                 rope: bool = True, rope_theta: float = 10000.0, decode_fp8: bool = False):
        if dtype not in _DT:
            raise ValueError("dtype must be 'bf16' or 'f32'")
        if act not in ("swiglu", "gelu"):
            raise ValueError("act must be 'swiglu' or 'gelu'")
        code, tdt = _DT[dtype]
        opts = N.tp_opts(code, N.TP_ACT_SWIGLU if act == "swiglu" else N.TP_ACT_GELU, int(rmsnorm), eps,
                         int(rope), rope_theta, int(decode_fp8))
        h = C.c_void_p()
        N.check(N.lib().tp_shard_create(hidden, heads, kv_heads, ffn, tp, rank, C.byref(opts), C.byref(h)),
                "tp_shard_create")
        self._h = h
        self.hidden, self.heads, self.kv_heads, self.ffn, self.tp, self.rank = hidden, heads, kv_heads, ffn, tp, rank
        self.dtype, self.torch_dtype, self.elem_size = dtype, tdt, (2 if dtype == "bf16" else 4)
        self.act, self.rmsnorm, self.rope, self.decode_fp8 = act, rmsnorm, rope, decode_fp8
        self.head_dim = hidden // heads
        self.heads_local = heads // tp
        self.kv_local = kv_heads // tp
        self.ffn_local = ffn // tp

    # ---- setup
    def load_weights(self, W: dict, stream=None) -> None:
        """W: FULL unsharded weights as device tensors (wq, wk, wv, wo, w_gate
        for SwiGLU, w_up, w_down, g1/g2 with RMSNorm).  Waits for the copy."""
        d, h = self.head_dim, self.hidden
        shapes = {"wq": (self.heads * d, h), "wk": (self.kv_heads * d, h), "wv": (self.kv_heads * d, h),
                  "wo": (h, self.heads * d), "w_up": (self.ffn, h), "w_down": (h, self.ffn)}
        if self.act == "swiglu":
            shapes["w_gate"] = (self.ffn, h)
        if self.rmsnorm:
            shapes["g1"] = (h,)
            shapes["g2"] = (h,)
        w = N.tp_weights()
        for name, shp in shapes.items():
            if name not in W:
                raise ValueError(f"missing weight {name}")
            setattr(w, name, _dev(W[name], name, self.torch_dtype, shp))
        N.check(N.lib().tp_shard_load_weights(self._h, C.byref(w), _stream(stream)), "tp_shard_load_weights")
        (torch.cuda.current_stream() if stream is None else stream).synchronize()

    def reserve(self, max_tokens: int) -> None:
        N.check(N.lib().tp_shard_reserve(self._h, int(max_tokens)), "tp_shard_reserve")

    def kv_cache_paged(self, batch: int, max_seq: int, block_size: int, num_blocks: int) -> KVCache:
        return KVCache(self, batch, max_seq, block_size, num_blocks)

    def kv_cache(self, batch: int, max_seq: int) -> KVCache:
        return KVCache(self, batch, max_seq)

    # ---- forward
    def prefill(self, stage: int, x: torch.Tensor, kv: KVCache | None = None, out: torch.Tensor | None = None,
                stream=None) -> torch.Tensor:
        """x [B, S, hidden] (layer input for ATTN, reduced h for MLP) ->
        this rank's fp32 partial [B, S, hidden]."""
        if x.dim() != 3 or x.shape[2] != self.hidden:
            raise ValueError("x must be [batch, seq, hidden]")
        B, S = int(x.shape[0]), int(x.shape[1])
        if out is None:
            out = torch.empty((B, S, self.hidden), dtype=torch.float32, device=x.device)
        N.check(N.lib().tp_shard_forward_prefill(
            self._h, stage, _dev(x, "x", self.torch_dtype), B, S, kv._h if kv is not None else None,
            _dev(out, "partial", torch.float32, (B, S, self.hidden)), _stream(stream)), "tp_shard_forward_prefill")
        return out

    def prefill_reduce(self, stage: int, x: torch.Tensor, partials, residual: torch.Tensor | None = None,
                       kv: KVCache | None = None, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        """One prefill stage and the reduce of its partial with the other ranks'
        ``partials`` (a list of ``tp`` fp32 [B, S, hidden] tensors; entry ``rank``
        is not read and may be None), plus ``residual``: returns the reduced
        [B, S, hidden] in the shard's dtype."""
        if x.dim() != 3 or x.shape[2] != self.hidden:
            raise ValueError("x must be [batch, seq, hidden]")
        B, S = int(x.shape[0]), int(x.shape[1])
        if len(partials) != self.tp:
            raise ValueError("partials must hold one entry per rank")
        shape = (B, S, self.hidden)
        ptrs = (C.c_void_p * self.tp)()
        for r, p in enumerate(partials):
            ptrs[r] = None if (p is None or r == self.rank) else _dev(p, f"partials[{r}]", torch.float32, shape).value
        if out is None:
            out = torch.empty(shape, dtype=self.torch_dtype, device=x.device)
        res = None if residual is None else _dev(residual, "residual", self.torch_dtype, shape)
        N.check(N.lib().tp_shard_forward_prefill_reduce(
            self._h, stage, _dev(x, "x", self.torch_dtype), B, S, kv._h if kv is not None else None, ptrs, res,
            _dev(out, "out", self.torch_dtype, shape), _stream(stream)), "tp_shard_forward_prefill_reduce")
        return out

    def decode(self, stage: int, x: torch.Tensor, kv: KVCache | None = None, out: torch.Tensor | None = None,
               stream=None) -> torch.Tensor:
        """x [B, hidden] (one token per sequence) -> fp32 partial [B, hidden]."""
        if x.dim() != 2 or x.shape[1] != self.hidden:
            raise ValueError("x must be [batch, hidden]")
        B = int(x.shape[0])
        if out is None:
            out = torch.empty((B, self.hidden), dtype=torch.float32, device=x.device)
        N.check(N.lib().tp_shard_forward_decode(
            self._h, stage, _dev(x, "x", self.torch_dtype), B, kv._h if kv is not None else None,
            _dev(out, "partial", torch.float32, (B, self.hidden)), _stream(stream)), "tp_shard_forward_decode")
        return out

    def decode_reduce(self, stage: int, x: torch.Tensor, partials, residual: torch.Tensor | None = None,
                      kv: KVCache | None = None, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        """One decode stage and the reduce of its partial with the other ranks'
        ``partials`` (a list of ``tp`` fp32 [B, hidden] tensors; entry ``rank`` is
        not read and may be None), plus ``residual``: returns the reduced
        [B, hidden] in the shard's dtype."""
        if x.dim() != 2 or x.shape[1] != self.hidden:
            raise ValueError("x must be [batch, hidden]")
        B = int(x.shape[0])
        if len(partials) != self.tp:
            raise ValueError("partials must hold one entry per rank")
        ptrs = (C.c_void_p * self.tp)()
        for r, p in enumerate(partials):
            ptrs[r] = None if (p is None or r == self.rank) else _dev(p, f"partials[{r}]", torch.float32,
                                                                     (B, self.hidden)).value
        if out is None:
            out = torch.empty((B, self.hidden), dtype=self.torch_dtype, device=x.device)
        res = None if residual is None else _dev(residual, "residual", self.torch_dtype, (B, self.hidden))
        N.check(N.lib().tp_shard_forward_decode_reduce(
            self._h, stage, _dev(x, "x", self.torch_dtype), B, kv._h if kv is not None else None, ptrs, res,
            _dev(out, "out", self.torch_dtype, (B, self.hidden)), _stream(stream)), "tp_shard_forward_decode_reduce")
        return out

    def norm(self, which: int, x: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        """RMSNorm of rows of x [..., hidden] with the shard's gain g1 (which=1)
        or g2 (which=2): the per-rank norm of the sequence-parallel flow."""
        if x.shape[-1] != self.hidden:
            raise ValueError("x must end in hidden")
        if out is None:
            out = torch.empty_like(x)
        rows = x.numel() // self.hidden
        N.check(N.lib().tp_shard_norm(self._h, which, _dev(x, "x", self.torch_dtype),
                                      rows, _dev(out, "out", self.torch_dtype, tuple(x.shape)), _stream(stream)),
                "tp_shard_norm")
        return out

    def reduce_norm(self, which: int, partials, residual: torch.Tensor | None = None, out: torch.Tensor | None = None,
                    norm_out: torch.Tensor | None = None, stream=None):
        """out = (sum of the fp32 partials in rank order) + residual, and
        norm_out = RMSNorm(out) with gain g1 (which=1) or g2 (which=2), in one
        pass; partials [..., hidden].  Returns (out, norm_out)."""
        partials = list(partials)
        if not partials:
            raise ValueError("need at least one partial")
        shape = tuple(partials[0].shape)
        if shape[-1] != self.hidden:
            raise ValueError("partials must end in hidden")
        rows = partials[0].numel() // self.hidden
        ptrs = (C.c_void_p * len(partials))(*[_dev(p, f"partial[{i}]", torch.float32, shape).value
                                              for i, p in enumerate(partials)])
        if residual is not None:
            _dev(residual, "residual", self.torch_dtype)
            if residual.numel() != rows * self.hidden:
                raise ValueError("residual size differs from the partials")
        if out is None:
            out = torch.empty(shape, dtype=self.torch_dtype, device=partials[0].device)
        if norm_out is None:
            norm_out = torch.empty_like(out)
        N.check(N.lib().tp_shard_reduce_norm(self._h, which, ptrs, len(partials),
                                             C.c_void_p(residual.data_ptr()) if residual is not None else None,
                                             _dev(out, "out", self.torch_dtype, shape),
                                             _dev(norm_out, "norm_out", self.torch_dtype, shape), rows,
                                             _stream(stream)), "tp_shard_reduce_norm")
        return out, norm_out

    def fp8_weights(self, which: str, stream=None):
        """Copies of the E4M3 codes (uint8 [rows, cols], packed row order) and
        row scales (fp32 [rows]) of 'qkv', 'o', 'up' or 'down'."""
        code = {"qkv": 0, "o": 1, "up": 2, "down": 3}[which]
        q, sc, r, c = C.c_void_p(), C.c_void_p(), C.c_int(), C.c_int()
        N.check(N.lib().tp_shard_fp8_view(self._h, code, C.byref(q), C.byref(sc), C.byref(r), C.byref(c)),
                "tp_shard_fp8_view")
        codes = torch.empty((r.value, c.value), dtype=torch.uint8, device="cuda")
        scales = torch.empty((r.value,), dtype=torch.float32, device="cuda")
        _memcpy_d2d(codes.data_ptr(), q.value, codes.numel(), stream)
        _memcpy_d2d(scales.data_ptr(), sc.value, scales.numel() * 4, stream)
        return codes, scales

    def debug_tensor(self, which: str, shape, stream=None) -> torch.Tensor:
        """Copy of a workspace tensor of the last call: 'o' [tokens, heads/t*d],
        'act' [tokens, ffn/t] or 'n' [tokens, hidden]."""
        code = {"o": 0, "act": 1, "n": 2}[which]
        p = C.c_void_p()
        N.check(N.lib().tp_shard_debug_view(self._h, code, C.byref(p)), "tp_shard_debug_view")
        t = torch.empty(shape, dtype=self.torch_dtype, device="cuda")
        _memcpy_d2d(t.data_ptr(), p.value, t.numel() * self.elem_size, stream)
        return t

    def timing(self, enable, kinds=None) -> None:
        """Turn the per-kernel event timer on (resetting it) or off; ``kinds``
        limits it to the named kernel kinds (see _native.KERNEL_KINDS)."""
        mask = 0
        if enable:
            mask = -1 if kinds is None else sum(1 << N.KERNEL_KINDS.index(k) for k in kinds)
        N.check(N.lib().tp_shard_timing(self._h, mask), "tp_shard_timing")

    def timing_read(self) -> dict:
        """{kernel kind: (total ms, launches)} of the recorded launches."""
        out = {}
        for i, name in enumerate(N.KERNEL_KINDS):
            ms, n = C.c_double(), C.c_longlong()
            N.check(N.lib().tp_shard_timing_read(self._h, i, C.byref(ms), C.byref(n)), "tp_shard_timing_read")
            if n.value:
                out[name] = (ms.value, n.value)
        return out

    def close(self) -> None:
        if self._h:
            N.lib().tp_shard_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def partial_reduce(partials, residual: torch.Tensor | None = None, out: torch.Tensor | None = None,
                   dtype: str | None = None, stream=None) -> torch.Tensor:
    """out = (sum of fp32 partials in rank order) + residual, stored as the
    residual's dtype (or ``dtype``)."""
    partials = list(partials)
    if not partials:
        raise ValueError("need at least one partial")
    shape = tuple(partials[0].shape)
    n = partials[0].numel()
    ptrs = (C.c_void_p * len(partials))(*[_dev(p, f"partial[{i}]", torch.float32, shape).value
                                          for i, p in enumerate(partials)])
    if dtype is None:
        dtype = "bf16" if residual is None or residual.dtype == torch.bfloat16 else "f32"
    code, tdt = _DT[dtype]
    if residual is not None:
        _dev(residual, "residual", tdt)
        if residual.numel() != n:
            raise ValueError("residual size differs from the partials")
    if out is None:
        out = torch.empty(shape, dtype=tdt, device=partials[0].device)
    N.check(N.lib().tp_partial_reduce(ptrs, len(partials), C.c_void_p(residual.data_ptr()) if residual is not None
                                      else None, _dev(out, "out", tdt), n, code, _stream(stream)),
            "tp_partial_reduce")
    return out


def partial_reduce_scatter(partials, rank: int, residual_rows: torch.Tensor | None = None,
                           out: torch.Tensor | None = None, dtype: str | None = None, stream=None) -> torch.Tensor:
    """Rank ``rank``'s token rows of (sum of the fp32 partials in rank order)
    + residual_rows.  partials: t tensors [..., hidden] flattening to [T, hidden];
    returns [T/t, hidden]."""
    partials = list(partials)
    t = len(partials)
    if t == 0:
        raise ValueError("need at least one partial")
    shape = tuple(partials[0].shape)
    cols = shape[-1]
    rows = partials[0].numel() // cols
    ptrs = (C.c_void_p * t)(*[_dev(p, f"partial[{i}]", torch.float32, shape).value for i, p in enumerate(partials)])
    if dtype is None:
        dtype = "bf16" if residual_rows is None or residual_rows.dtype == torch.bfloat16 else "f32"
    code, tdt = _DT[dtype]
    if rows % t:
        raise ValueError("the token count must divide by the number of partials")
    if residual_rows is not None:
        _dev(residual_rows, "residual_rows", tdt)
        if residual_rows.numel() != rows // t * cols:
            raise ValueError("residual_rows must hold T/t rows")
    if out is None:
        out = torch.empty((rows // t, cols), dtype=tdt, device=partials[0].device)
    N.check(N.lib().tp_partial_reduce_scatter(ptrs, t, rank,
                                              C.c_void_p(residual_rows.data_ptr()) if residual_rows is not None
                                              else None, _dev(out, "out", tdt), rows, cols, code, _stream(stream)),
            "tp_partial_reduce_scatter")
    return out


def all_gather(pieces, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Rank-order concatenation of t equal [rows, cols] pieces into [t * rows, cols]."""
    pieces = list(pieces)
    t = len(pieces)
    shape = tuple(pieces[0].shape)
    dt = pieces[0].dtype
    code = N.TP_BF16 if dt == torch.bfloat16 else N.TP_F32
    cols = shape[-1]
    rows = pieces[0].numel() // cols
    ptrs = (C.c_void_p * t)(*[_dev(p, f"piece[{i}]", dt, shape).value for i, p in enumerate(pieces)])
    if out is None:
        out = torch.empty((t * rows, cols), dtype=dt, device=pieces[0].device)
    N.check(N.lib().tp_all_gather(ptrs, t, rows, cols, code, _dev(out, "out", dt), _stream(stream)), "tp_all_gather")
    return out


def set_gemm_config(cfg: int) -> None:
    """Tuning hook: force a projection tile configuration (-1 = automatic)."""
    N.check(N.lib().tp_tune_set_gemm_config(int(cfg)), "tp_tune_set_gemm_config")


def set_gemm_split(cfg0: int, cfg1: int, cols0: int) -> None:
    """Tuning hook: run every projection wider than cols0 columns as two
    launches (cfg0 on the first cols0 columns, cfg1 on the rest); cols0 = 0
    restores the planner."""
    N.check(N.lib().tp_tune_set_gemm_split(int(cfg0), int(cfg1), int(cols0)), "tp_tune_set_gemm_split")


def gemm_plan(M: int, N_: int, K: int, proj: str):
    """The planner's launch plan for an M x N x K projection ('partial',
    'qkv', 'swiglu' or 'gelu'): a list of (tile configuration, columns) per
    launch."""
    kind = {"partial": N.TP_PROJ_PARTIAL, "qkv": N.TP_PROJ_QKV, "swiglu": N.TP_PROJ_SWIGLU,
            "gelu": N.TP_PROJ_GELU}[proj]
    parts, cfg, cols = C.c_int(), (C.c_int * 2)(), (C.c_int * 2)()
    N.check(N.lib().tp_tune_gemm_plan(int(M), int(N_), int(K), kind, C.byref(parts), cfg, cols), "tp_tune_gemm_plan")
    return [(cfg[i], cols[i]) for i in range(parts.value)]


def set_decode_chunk(ch: int) -> None:
    """Tuning hook: decode attention positions per chunk for query groups (0 = automatic, 16, 32, 64)."""
    N.check(N.lib().tp_tune_set_decode_chunk(int(ch)), "tp_tune_set_decode_chunk")


def set_decode_attn(mode: int) -> None:
    """Tuning hook: decode attention merge (0 = automatic, 1 = a second launch,
    2 = in the same launch)."""
    N.check(N.lib().tp_tune_set_decode_attn(int(mode)), "tp_tune_set_decode_attn")


def set_attn_groups(kg: int) -> None:
    """Tuning hook: prefill attention key groups (0 = automatic, 1 or 2)."""
    N.check(N.lib().tp_tune_set_attn_groups(int(kg)), "tp_tune_set_attn_groups")


def set_attn_kernel(k: int) -> None:
    """Tuning hook: prefill attention kernel (0 = default, 1 one LDS stage
    per key group, 2 pipelined: the default)."""
    N.check(N.lib().tp_tune_set_attn_kernel(int(k)), "tp_tune_set_attn_kernel")
