"""Thin ctypes binding of librq (include/rq.h).

Argument marshalling only: every step of the ResidualQuant path runs in the
HIP library.  Tensors are torch tensors on the GPU; calls are enqueued on the
current torch stream (or the one given) and return before the GPU finishes.
Importing this module needs no GPU; the first call loads librq.so and fails
loudly if it has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# RQ_LIB selects another build of the same library (the host-sanitized one)
LIB_PATH = os.environ.get("RQ_LIB") or os.path.join(_PKG, "librq.so")

RQ_OK = 0
STATUS_NAMES = {0: "RQ_OK", 1: "RQ_ERR_INVALID_ARG", 2: "RQ_ERR_UNSUPPORTED",
                3: "RQ_ERR_CAPACITY", 4: "RQ_ERR_WORKSPACE", 5: "RQ_ERR_ALIGNMENT",
                6: "RQ_ERR_LAUNCH"}
MODE_RESIDUAL, MODE_DIRECT, MODE_CHAINED = 0, 1, 2
ALPHA_LS, ALPHA_NORM_RATIO, ALPHA_ONE = 0, 1, 2
ROT_NONE, ROT_HADAMARD = 0, 1
OUT_F32, OUT_BF16 = 0, 1

# Every symbol include/rq.h declares.
EXPORTS = (
    "rq_status_string", "rq_validate_desc", "rq_cache_bytes", "rq_cache_layout", "rq_cache_slot",
    "rq_quantize_append", "rq_quantize_append_ragged", "rq_reconstruct",
    "rq_decode_workspace_bytes", "rq_decode_splits", "rq_decode_attention",
    "rq_decode_attention_noalloc",
    "rq_decode_attention_ragged",
    "rq_bf16_decode_workspace_bytes", "rq_bf16_decode_attention",
    "rq_read_probe_sink_words", "rq_read_probe",
    "rq_paged_decode_workspace_bytes", "rq_paged_quantize_append", "rq_paged_decode_attention",
)


class RQError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS_NAMES.get(status, status)} "
                         f"({_status_string(status)})")


class CacheDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "loops", "layers", "kv_heads", "max_tokens", "head_dim", "loops_per_group",
        "anchor_bits", "residual_bits", "group_size", "mode", "alpha_mode", "rotation")]

    def __repr__(self):
        return "CacheDesc(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


class Slot(ctypes.Structure):
    _fields_ = [("codes_offset", ctypes.c_uint64), ("sz_offset", ctypes.c_uint64),
                ("alpha_offset", ctypes.c_uint64), ("slot_bytes", ctypes.c_uint64),
                ("bits", ctypes.c_int32), ("code_bytes", ctypes.c_int32)]


class Layout(ctypes.Structure):
    _fields_ = [("total_bytes", ctypes.c_uint64), ("layer_bytes", ctypes.c_uint64),
                ("group_bytes", ctypes.c_uint64), ("slot_bytes", ctypes.c_uint64 * 2),
                ("sz_offset", ctypes.c_uint64 * 2), ("alpha_offset", ctypes.c_uint64),
                ("alpha_row_bytes", ctypes.c_uint64),
                ("code_row_bytes", ctypes.c_int32 * 2), ("sz_row_bytes", ctypes.c_int32),
                ("token_tile", ctypes.c_int32)]


def make_desc(batch, loops, layers, kv_heads, max_tokens, head_dim, loops_per_group=4,
              anchor_bits=4, residual_bits=2, group_size=16, mode=MODE_RESIDUAL,
              alpha_mode=ALPHA_LS, rotation=ROT_HADAMARD) -> CacheDesc:
    return CacheDesc(batch, loops, layers, kv_heads, max_tokens, head_dim, loops_per_group,
                     anchor_bits, residual_bits, group_size, mode, alpha_mode, rotation)


_lib = None
_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_u64 = ctypes.c_uint64


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m decode_attention_int4_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        D = ctypes.POINTER(CacheDesc)
        L.rq_status_string.argtypes = [ctypes.c_int]
        L.rq_status_string.restype = ctypes.c_char_p
        L.rq_validate_desc.argtypes = [D]
        L.rq_cache_bytes.argtypes = [D, ctypes.POINTER(ctypes.c_uint64)]
        L.rq_cache_slot.argtypes = [D, _i32, _i32, _i32, _i32, _i32, ctypes.POINTER(Slot)]
        L.rq_cache_layout.argtypes = [D, ctypes.POINTER(Layout)]
        L.rq_quantize_append.argtypes = [D, _vp, _vp, _i32, _i32, _vp, _vp]
        L.rq_quantize_append_ragged.argtypes = [D, _vp, _vp, _vp, _i32, _vp, _vp]
        L.rq_reconstruct.argtypes = [D, _vp, _vp, _i32, _i32, _i32, _vp, _vp]
        L.rq_decode_workspace_bytes.argtypes = [D, _i32, _i32]
        L.rq_decode_workspace_bytes.restype = _u64
        L.rq_decode_splits.argtypes = [D, _i32, _i32, _i32]
        L.rq_decode_splits.restype = _i32
        L.rq_decode_attention.argtypes = [D, _vp, _vp, _i32, _i32, _vp, _i32, _i32,
                                          ctypes.c_float, _vp, _u64, _vp, _vp]
        L.rq_decode_attention_noalloc.argtypes = [D, _vp, _vp, _i32, _i32, _vp, _i32, _i32,
                                                  ctypes.c_float, _vp, _vp]
        L.rq_decode_attention_ragged.argtypes = [D, _vp, _vp, _i32, _i32, _vp, _i32, _vp, _i32,
                                                 ctypes.c_float, _vp, _u64, _vp, _vp]
        L.rq_bf16_decode_workspace_bytes.argtypes = [D, _i32, _i32]
        L.rq_bf16_decode_workspace_bytes.restype = _u64
        L.rq_bf16_decode_attention.argtypes = [D, _vp, _vp, _i32, _i32, _vp, _i32, _i32,
                                               ctypes.c_float, _vp, _u64, _vp, _vp]
        L.rq_paged_decode_workspace_bytes.argtypes = [D, _i32, _i32, _i32]
        L.rq_paged_decode_workspace_bytes.restype = _u64
        L.rq_paged_quantize_append.argtypes = [D, _vp, _vp, _i32, _vp, _i32, _vp, _i32, _vp, _vp]
        L.rq_paged_decode_attention.argtypes = [D, _vp, _vp, _i32, _i32, _vp, _i32, _i32, _vp,
                                                _i32, _vp, _i32, ctypes.c_float, _vp, _u64, _vp,
                                                _vp]
        L.rq_read_probe_sink_words.restype = ctypes.c_uint32
        L.rq_read_probe.argtypes = [_vp, _u64, _vp, _vp]
        for name in ("rq_validate_desc", "rq_cache_bytes", "rq_cache_layout", "rq_cache_slot",
                     "rq_quantize_append",
                     "rq_quantize_append_ragged", "rq_reconstruct", "rq_decode_attention",
                     "rq_decode_attention_noalloc",
                     "rq_decode_attention_ragged", "rq_bf16_decode_attention", "rq_read_probe",
                     "rq_paged_quantize_append", "rq_paged_decode_attention"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _status_string(s: int) -> str:
    try:
        return lib().rq_status_string(s).decode()
    except Exception:  # the library may be what failed to load
        return "?"


def _check(status: int, what: str):
    if status != RQ_OK:
        raise RQError(status, what)


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dev(t: torch.Tensor, dtype, name: str):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


# ---------------------------------------------------------------- host-only
def validate_desc(desc: CacheDesc) -> int:
    return lib().rq_validate_desc(ctypes.byref(desc))


def cache_bytes(desc: CacheDesc) -> int:
    n = ctypes.c_uint64()
    _check(lib().rq_cache_bytes(ctypes.byref(desc), ctypes.byref(n)), "rq_cache_bytes")
    return n.value


def cache_layout(desc: CacheDesc) -> Layout:
    out = Layout()
    _check(lib().rq_cache_layout(ctypes.byref(desc), ctypes.byref(out)), "rq_cache_layout")
    return out


def cache_slot(desc: CacheDesc, kv: int, batch: int, layer: int, loop: int, head: int) -> Slot:
    s = Slot()
    _check(lib().rq_cache_slot(ctypes.byref(desc), kv, batch, layer, loop, head, ctypes.byref(s)),
           "rq_cache_slot")
    return s


def decode_workspace_bytes(desc: CacheDesc, q_heads: int, max_n_tokens: int) -> int:
    return int(lib().rq_decode_workspace_bytes(ctypes.byref(desc), q_heads, max_n_tokens))


def decode_splits(desc: CacheDesc, loop: int, q_heads: int, n_tokens: int) -> int:
    return int(lib().rq_decode_splits(ctypes.byref(desc), loop, q_heads, n_tokens))


def bf16_decode_workspace_bytes(desc: CacheDesc, q_heads: int, max_n_tokens: int) -> int:
    return int(lib().rq_bf16_decode_workspace_bytes(ctypes.byref(desc), q_heads, max_n_tokens))


# ---------------------------------------------------------------- allocation helpers
def alloc_cache(desc: CacheDesc, device="cuda") -> torch.Tensor:
    """A uint8 tensor of rq_cache_bytes() bytes (torch's allocator aligns to 512 B)."""
    return torch.empty(cache_bytes(desc), dtype=torch.uint8, device=device)


def alloc_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """Workspace for split-K states, zero-filled once as the library requires
    (its split counters must start at zero; every call leaves them at zero)."""
    return torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------- device calls
def quantize_append(desc: CacheDesc, cache: torch.Tensor, kv_bf16: torch.Tensor, n_tokens: int,
                    signs: Optional[torch.Tensor], stream=None) -> None:
    """kv_bf16: [2, B, loops, layers, kv_heads, t_new, d] BF16; appends at n_tokens."""
    c = _dev(cache, torch.uint8, "cache")
    x = _dev(kv_bf16, torch.bfloat16, "kv_bf16")
    if kv_bf16.dim() != 7 or tuple(kv_bf16.shape[:5]) != (2, desc.batch, desc.loops, desc.layers,
                                                          desc.kv_heads) \
            or kv_bf16.shape[6] != desc.head_dim:
        raise ValueError(f"kv_bf16 shape {tuple(kv_bf16.shape)} does not match {desc}")
    s = _dev(signs, torch.int8, "signs") if signs is not None else None
    if cache.numel() < cache_bytes(desc):
        raise ValueError("cache tensor smaller than rq_cache_bytes()")
    _check(lib().rq_quantize_append(ctypes.byref(desc), c, x, n_tokens, kv_bf16.shape[5], s,
                                    _stream(stream)), "rq_quantize_append")


def quantize_append_ragged(desc: CacheDesc, cache: torch.Tensor, kv_bf16: torch.Tensor,
                           positions: torch.Tensor, signs: Optional[torch.Tensor],
                           stream=None) -> None:
    """kv_bf16: [2, B, loops, layers, kv_heads, t_new, d] BF16; batch row b is
    appended at positions[b] (device int32 [B])."""
    c = _dev(cache, torch.uint8, "cache")
    x = _dev(kv_bf16, torch.bfloat16, "kv_bf16")
    if kv_bf16.dim() != 7 or tuple(kv_bf16.shape[:5]) != (2, desc.batch, desc.loops, desc.layers,
                                                          desc.kv_heads) \
            or kv_bf16.shape[6] != desc.head_dim:
        raise ValueError(f"kv_bf16 shape {tuple(kv_bf16.shape)} does not match {desc}")
    if tuple(positions.shape) != (desc.batch,):
        raise ValueError(f"positions shape {tuple(positions.shape)} != ({desc.batch},)")
    s = _dev(signs, torch.int8, "signs") if signs is not None else None
    if cache.numel() < cache_bytes(desc):
        raise ValueError("cache tensor smaller than rq_cache_bytes()")
    _check(lib().rq_quantize_append_ragged(ctypes.byref(desc), c, x,
                                           _dev(positions, torch.int32, "positions"),
                                           kv_bf16.shape[5], s, _stream(stream)),
           "rq_quantize_append_ragged")


def reconstruct(desc: CacheDesc, cache: torch.Tensor, signs: Optional[torch.Tensor],
                tok_begin: int, tok_end: int, out: Optional[torch.Tensor] = None,
                out_dtype=torch.float32, stream=None) -> torch.Tensor:
    """Returns [2, B, loops, layers, kv_heads, tok_end - tok_begin, d] fp32 or BF16."""
    shape = (2, desc.batch, desc.loops, desc.layers, desc.kv_heads, tok_end - tok_begin,
             desc.head_dim)
    if out is None:
        out = torch.empty(shape, dtype=out_dtype, device=cache.device)
    if tuple(out.shape) != shape:
        raise ValueError("out has the wrong shape")
    code = OUT_F32 if out.dtype == torch.float32 else OUT_BF16
    o = _dev(out, out.dtype, "out")
    s = _dev(signs, torch.int8, "signs") if signs is not None else None
    _check(lib().rq_reconstruct(ctypes.byref(desc), _dev(cache, torch.uint8, "cache"), s,
                                tok_begin, tok_end, code, o, _stream(stream)), "rq_reconstruct")
    return out


def decode_attention(desc: CacheDesc, cache: torch.Tensor, signs: Optional[torch.Tensor],
                     loop: int, layer: int, q: torch.Tensor, n_tokens: int,
                     softmax_scale: float, workspace: torch.Tensor,
                     out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """q: [B, q_heads, d] BF16 -> out [B, q_heads, d] fp32."""
    if q.dim() != 3 or q.shape[0] != desc.batch or q.shape[2] != desc.head_dim:
        raise ValueError(f"q shape {tuple(q.shape)} does not match {desc}")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    s = _dev(signs, torch.int8, "signs") if signs is not None else None
    _check(lib().rq_decode_attention(
        ctypes.byref(desc), _dev(cache, torch.uint8, "cache"), s, loop, layer,
        _dev(q, torch.bfloat16, "q"), q.shape[1], n_tokens, float(softmax_scale),
        _dev(workspace, torch.uint8, "workspace"), workspace.numel(),
        _dev(out, torch.float32, "out"), _stream(stream)), "rq_decode_attention")
    return out


def decode_attention_noalloc(desc: CacheDesc, cache: torch.Tensor, signs: Optional[torch.Tensor],
                             loop: int, layer: int, q: torch.Tensor, n_tokens: int,
                             softmax_scale: float, out: Optional[torch.Tensor] = None,
                             stream=None) -> torch.Tensor:
    """As decode_attention, with the split-K workspace inside the library."""
    if q.dim() != 3 or q.shape[0] != desc.batch or q.shape[2] != desc.head_dim:
        raise ValueError(f"q shape {tuple(q.shape)} does not match {desc}")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    s = _dev(signs, torch.int8, "signs") if signs is not None else None
    _check(lib().rq_decode_attention_noalloc(
        ctypes.byref(desc), _dev(cache, torch.uint8, "cache"), s, loop, layer,
        _dev(q, torch.bfloat16, "q"), q.shape[1], n_tokens, float(softmax_scale),
        _dev(out, torch.float32, "out"), _stream(stream)), "rq_decode_attention_noalloc")
    return out


def decode_attention_ragged(desc: CacheDesc, cache: torch.Tensor, signs: Optional[torch.Tensor],
                            loop: int, layer: int, q: torch.Tensor, lengths: torch.Tensor,
                            max_n_tokens: int, softmax_scale: float, workspace: torch.Tensor,
                            out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """q: [B, q_heads, d] BF16, lengths: device int32 [B] -> out [B, q_heads, d] fp32."""
    if q.dim() != 3 or q.shape[0] != desc.batch or q.shape[2] != desc.head_dim:
        raise ValueError(f"q shape {tuple(q.shape)} does not match {desc}")
    if tuple(lengths.shape) != (desc.batch,):
        raise ValueError(f"lengths shape {tuple(lengths.shape)} != ({desc.batch},)")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    s = _dev(signs, torch.int8, "signs") if signs is not None else None
    _check(lib().rq_decode_attention_ragged(
        ctypes.byref(desc), _dev(cache, torch.uint8, "cache"), s, loop, layer,
        _dev(q, torch.bfloat16, "q"), q.shape[1], _dev(lengths, torch.int32, "lengths"),
        max_n_tokens, float(softmax_scale), _dev(workspace, torch.uint8, "workspace"),
        workspace.numel(), _dev(out, torch.float32, "out"), _stream(stream)),
        "rq_decode_attention_ragged")
    return out


def paged_decode_workspace_bytes(pool: CacheDesc, q_heads: int, n_seqs: int,
                                 max_n_tokens: int) -> int:
    return int(lib().rq_paged_decode_workspace_bytes(ctypes.byref(pool), q_heads, n_seqs,
                                                     max_n_tokens))


def _table(block_table: torch.Tensor, n_seqs: int):
    if block_table.dim() != 2 or block_table.shape[0] != n_seqs:
        raise ValueError(f"block_table shape {tuple(block_table.shape)} is not [n_seqs, max_blocks]")
    return _dev(block_table, torch.int32, "block_table"), block_table.shape[1]


def paged_quantize_append(pool: CacheDesc, cache: torch.Tensor, kv_bf16: torch.Tensor,
                          block_table: torch.Tensor, positions: torch.Tensor,
                          signs: Optional[torch.Tensor], stream=None) -> None:
    """Paged cache: pool.batch = blocks in the pool, pool.max_tokens = tokens per block.
    kv_bf16: [2, n_seqs, loops, layers, kv_heads, t_new, d] BF16; sequence s is
    appended at logical positions[s] through block_table[s] (device int32
    [n_seqs, max_blocks_per_seq])."""
    n = kv_bf16.shape[1]
    if kv_bf16.dim() != 7 or kv_bf16.shape[0] != 2 or \
            tuple(kv_bf16.shape[2:5]) != (pool.loops, pool.layers, pool.kv_heads) or \
            kv_bf16.shape[6] != pool.head_dim:
        raise ValueError(f"kv_bf16 shape {tuple(kv_bf16.shape)} does not match {pool}")
    if tuple(positions.shape) != (n,):
        raise ValueError(f"positions shape {tuple(positions.shape)} != ({n},)")
    if cache.numel() < cache_bytes(pool):
        raise ValueError("cache tensor smaller than rq_cache_bytes()")
    tab, mb = _table(block_table, n)
    s = _dev(signs, torch.int8, "signs") if signs is not None else None
    _check(lib().rq_paged_quantize_append(
        ctypes.byref(pool), _dev(cache, torch.uint8, "cache"),
        _dev(kv_bf16, torch.bfloat16, "kv_bf16"), n, tab, mb,
        _dev(positions, torch.int32, "positions"), kv_bf16.shape[5], s, _stream(stream)),
        "rq_paged_quantize_append")


def paged_decode_attention(pool: CacheDesc, cache: torch.Tensor, signs: Optional[torch.Tensor],
                           loop: int, layer: int, q: torch.Tensor, block_table: torch.Tensor,
                           lengths: torch.Tensor, max_n_tokens: int, softmax_scale: float,
                           workspace: torch.Tensor, out: Optional[torch.Tensor] = None,
                           stream=None) -> torch.Tensor:
    """q: [n_seqs, q_heads, d] BF16, block_table: device int32 [n_seqs, max_blocks],
    lengths: device int32 [n_seqs] -> out [n_seqs, q_heads, d] fp32."""
    if q.dim() != 3 or q.shape[2] != pool.head_dim:
        raise ValueError(f"q shape {tuple(q.shape)} does not match {pool}")
    n = q.shape[0]
    if tuple(lengths.shape) != (n,):
        raise ValueError(f"lengths shape {tuple(lengths.shape)} != ({n},)")
    tab, mb = _table(block_table, n)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    s = _dev(signs, torch.int8, "signs") if signs is not None else None
    _check(lib().rq_paged_decode_attention(
        ctypes.byref(pool), _dev(cache, torch.uint8, "cache"), s, loop, layer,
        _dev(q, torch.bfloat16, "q"), q.shape[1], n, tab, mb,
        _dev(lengths, torch.int32, "lengths"), max_n_tokens, float(softmax_scale),
        _dev(workspace, torch.uint8, "workspace"), workspace.numel(),
        _dev(out, torch.float32, "out"), _stream(stream)), "rq_paged_decode_attention")
    return out


def bf16_decode_attention(desc: CacheDesc, k_cache: torch.Tensor, v_cache: torch.Tensor,
                          loop: int, layer: int, q: torch.Tensor, n_tokens: int,
                          softmax_scale: float, workspace: torch.Tensor,
                          out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """k_cache, v_cache: [B, loops, layers, kv_heads, max_tokens, d] BF16."""
    shape = (desc.batch, desc.loops, desc.layers, desc.kv_heads, desc.max_tokens, desc.head_dim)
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} shape {tuple(t.shape)} != {shape}")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    _check(lib().rq_bf16_decode_attention(
        ctypes.byref(desc), _dev(k_cache, torch.bfloat16, "k_cache"),
        _dev(v_cache, torch.bfloat16, "v_cache"), loop, layer, _dev(q, torch.bfloat16, "q"),
        q.shape[1], n_tokens, float(softmax_scale), _dev(workspace, torch.uint8, "workspace"),
        workspace.numel(), _dev(out, torch.float32, "out"), _stream(stream)),
        "rq_bf16_decode_attention")
    return out


def read_probe_sink_words() -> int:
    return int(lib().rq_read_probe_sink_words())


def read_probe(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous GPU tensor")
    _check(lib().rq_read_probe(buf.data_ptr(), buf.numel() * buf.element_size(),
                               _dev(sink, torch.int32, "sink"), _stream(stream)), "rq_read_probe")
