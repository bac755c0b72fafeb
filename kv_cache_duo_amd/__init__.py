"""Python binding of libduo.so: DuoAttention mixed retrieval/streaming
attention over a head-split KV cache on AMD MI355X (gfx950).

Argument marshalling only.  Every step of prefill, decode and append runs in
the HIP kernels behind the C ABI of ``include/duo.h``; torch provides device
memory and the current stream.  There is no CPU fallback: if the library is
not built, importing the functions that need it raises.

    cfg = Config(batch=1, num_q_heads=32, num_kv_heads=32, head_dim=128,
                 max_len=33024, sink=64, recent=256,
                 kv_head_is_retrieval=mask)
    buf = torch.empty(required_bytes(cfg), dtype=torch.uint8, device="cuda")
    cache = duo_cache_init(cfg, buf)
    duo_prefill(cache, q, k, v, n_new, out)   # q/out [B,C,Hq,D], k/v [B,C,Hkv,D]
    duo_decode(cache, q1, k1, v1, out1)       # q1/out1 [B,Hq,D], k1/v1 [B,Hkv,D]
"""

from __future__ import annotations

import ctypes
import os
import re
from dataclasses import dataclass
from typing import Sequence

import torch  # noqa: F401  -- load torch's HIP runtime before libduo.so binds to it

_HERE = os.path.dirname(os.path.abspath(__file__))
# DUO_LIBRARY names another build of the same sources (the host-sanitized
# one of kv_cache_duo_amd.build.build_host_sanitized); default: the in-tree
# library.
LIB_PATH = os.environ.get("DUO_LIBRARY") or os.path.join(_HERE, "libduo.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "duo.h")

DUO_OK = 0
DUO_ERR_INVALID_ARG = 1
DUO_ERR_UNSUPPORTED = 2
DUO_ERR_BUFFER_TOO_SMALL = 3
DUO_ERR_CAPACITY = 4
DUO_ERR_HIP = 5
DUO_MAX_BATCH = 128


DUO_KV_BF16, DUO_KV_INT8, DUO_KV_FP8 = 0, 1, 2
DUO_ROPE_INTERLEAVED, DUO_ROPE_HALF = 0, 1
DUO_FP8_PREFILL_EXACT, DUO_FP8_PREFILL_MFMA = 0, 1
DUO_DECODE_STATIC, DUO_DECODE_DYNAMIC = 0, 1


class DuoError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class _Config(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("max_len", ctypes.c_int64), ("sink", ctypes.c_int32), ("recent", ctypes.c_int32),
        ("scale", ctypes.c_float), ("kv_head_is_retrieval", ctypes.POINTER(ctypes.c_uint8)),
        ("kv_format", ctypes.c_int32), ("rope_base", ctypes.c_float), ("rope_style", ctypes.c_int32),
        ("page_tokens", ctypes.c_int32), ("num_pages", ctypes.c_int64),
        ("kv_scale_k", ctypes.c_float), ("kv_scale_v", ctypes.c_float),
        ("fp8_prefill", ctypes.c_int32), ("decode_split", ctypes.c_int32),
        ("prefill_staging", ctypes.c_void_p), ("prefill_staging_bytes", ctypes.c_int64),
    ]


class Layout(ctypes.Structure):
    _fields_ = [
        ("lengths_offset", ctypes.c_int64), ("rk_offset", ctypes.c_int64),
        ("rv_offset", ctypes.c_int64), ("sk_offset", ctypes.c_int64),
        ("sv_offset", ctypes.c_int64), ("work_offset", ctypes.c_int64),
        ("work_bytes", ctypes.c_int64), ("total_bytes", ctypes.c_int64),
        ("n_retrieval", ctypes.c_int32), ("n_streaming", ctypes.c_int32),
        ("slots_per_streaming_head", ctypes.c_int32), ("kv_format", ctypes.c_int32),
        ("rks_offset", ctypes.c_int64), ("rvs_offset", ctypes.c_int64),
        ("page_table_offset", ctypes.c_int64), ("page_tokens", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32), ("num_pages", ctypes.c_int64),
        ("block_tokens", ctypes.c_int32), ("work_records_offset", ctypes.c_int64),
        ("prefill_staging_bytes", ctypes.c_int64),
    ]


_P = ctypes.c_void_p
_I32P = ctypes.POINTER(ctypes.c_int32)
_I64P = ctypes.POINTER(ctypes.c_int64)

_SIGNATURES = {
    "duo_cache_init": (ctypes.c_int, [ctypes.POINTER(_Config), _P, ctypes.c_size_t,
                                      ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(_P), _P]),
    "duo_cache_attach": (ctypes.c_int, [ctypes.POINTER(_Config), _P, ctypes.c_size_t, _I64P,
                                        ctypes.POINTER(_P)]),
    "duo_cache_destroy": (None, [_P]),
    "duo_cache_append": (ctypes.c_int, [_P, _P, _P, _I32P, ctypes.c_int32, _P]),
    "duo_prefill": (ctypes.c_int, [_P, _P, _P, _P, _I32P, ctypes.c_int32, _P, _P]),
    "duo_decode": (ctypes.c_int, [_P, _P, _P, _P, _P, _P]),
    "duo_decode_static_scratch": (ctypes.c_int, [_P, _P, _P, _P, _P, _P]),
    "duo_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "duo_cache_lengths": (ctypes.c_int, [_P, _I64P]),
    "duo_cache_layout": (ctypes.c_int, [_P, ctypes.POINTER(Layout)]),
    "duo_cache_head_index": (ctypes.c_int, [_P, _I32P]),
    "duo_cache_release": (ctypes.c_int, [_P, ctypes.c_int32, _P]),
    "duo_cache_append_varlen": (ctypes.c_int, [_P, _P, _P, _I32P, _P]),
    "duo_prefill_varlen": (ctypes.c_int, [_P, _P, _P, _P, _I32P, _P, _P]),
    "duo_cache_pages": (ctypes.c_int, [_P, ctypes.c_int32, _I32P, ctypes.c_int32, _I32P, _I64P]),
}

_lib = None


def _check_build_record() -> None:
    """Refuse a libduo.so built from other sources than the ones in the tree
    (the build writes a digest of its sources beside the library)."""
    import json

    from kv_cache_duo_amd.build import RECORD_NAME, source_digest
    record = os.path.join(os.path.dirname(LIB_PATH), RECORD_NAME)
    try:
        with open(record) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        raise RuntimeError(f"{LIB_PATH} has no build record ({record}): rebuild with "
                           "`python -m kv_cache_duo_amd.build`") from None
    if rec.get("sources_sha256") != source_digest():
        raise RuntimeError(f"{LIB_PATH} was built from other sources than kv_cache_duo_amd/csrc and "
                           "include/duo.h hold now: rebuild with `python -m kv_cache_duo_amd.build`")


def load_library() -> ctypes.CDLL:
    """Load libduo.so (built by ``kv_cache_duo_amd.build``); raise if it is
    absent or stale."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m kv_cache_duo_amd.build`")
        _check_build_record()
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def header_functions() -> list[str]:
    """Names of the functions declared in include/duo.h."""
    with open(HEADER_PATH) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(duo_[a-z_]+)\s*\(", text)))


def status_string(status: int) -> str:
    return load_library().duo_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != DUO_OK:
        raise DuoError(status, where)


@dataclass
class Config:
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    max_len: int
    sink: int
    recent: int
    kv_head_is_retrieval: Sequence[int]
    scale: float = 0.0
    kv_format: int = 0  # DUO_KV_BF16; DUO_KV_INT8 = 1 stores retrieval rows as int8 + fp32 row scales
    rope_base: float = 0.0  # > 0: rotary position embedding applied to q and k inside the library
    rope_style: int = 0     # DUO_ROPE_INTERLEAVED (pairs 2i, 2i+1) or DUO_ROPE_HALF (pairs i, i + D/2)
    page_tokens: int = 0    # > 0: paged retrieval cache, pages of this many positions
    num_pages: int = 0      # paged: pages in the pool
    kv_scale_k: float = 0.0  # DUO_KV_FP8: power-of-two K scale (0 = 1)
    kv_scale_v: float = 0.0  # DUO_KV_FP8: power-of-two V scale (0 = 1)
    fp8_prefill: int = 0     # DUO_FP8_PREFILL_EXACT (bf16 matrix cores) or DUO_FP8_PREFILL_MFMA (fp8 ones)
    decode_split: int = 0    # DUO_DECODE_STATIC (bitwise reproducible) or DUO_DECODE_DYNAMIC
    # DUO_KV_INT8 or rotary embedding: device workspace (a CUDA tensor, kept
    # alive with the config) where a prefill stages, once per call, the int8
    # rows it reads as bf16 and the streaming heads' turned chunk K rows; see
    # prefill_staging_bytes()
    prefill_staging: object = None

    def _c(self):
        mask = (ctypes.c_uint8 * max(len(self.kv_head_is_retrieval), 1))(
            *[1 if x else 0 for x in self.kv_head_is_retrieval])
        c = _Config(self.batch, self.num_q_heads, self.num_kv_heads, self.head_dim, self.max_len,
                    self.sink, self.recent, self.scale,
                    ctypes.cast(mask, ctypes.POINTER(ctypes.c_uint8)), self.kv_format, self.rope_base,
                    self.rope_style, self.page_tokens, self.num_pages, self.kv_scale_k, self.kv_scale_v,
                    self.fp8_prefill, self.decode_split, None, 0)
        if self.prefill_staging is not None:
            t = self.prefill_staging
            if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or not t.is_contiguous():
                raise ValueError("prefill_staging must be a contiguous CUDA tensor")
            c.prefill_staging = t.data_ptr()
            c.prefill_staging_bytes = t.numel() * t.element_size()
        return c, mask  # keep the mask alive for the call


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(getattr(stream, "cuda_stream", stream) or 0)


def _dev(t: torch.Tensor, shape, name: str) -> int:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != torch.bfloat16 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous bfloat16 tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def prefill_staging_bytes(cfg: Config) -> int:
    """Workspace bytes that let every prefill stage what it can: for an int8
    cache, and an fp8 cache with exact prefill, the retrieval rows as bf16 K
    and V (4 * batch * retrieval KV heads * head_dim * max_len), with rotary
    embedding the streaming heads' turned chunk K rows (2 * batch *
    streaming KV heads * head_dim * max_len)."""
    n_r = sum(1 for x in cfg.kv_head_is_retrieval if x)
    n_s = cfg.num_kv_heads - n_r
    out = 0
    if cfg.kv_format == DUO_KV_INT8 or (cfg.kv_format == DUO_KV_FP8 and cfg.fp8_prefill == DUO_FP8_PREFILL_EXACT):
        out += 4 * cfg.batch * n_r * cfg.head_dim * cfg.max_len
    if cfg.rope_base > 0:
        out += 2 * cfg.batch * n_s * cfg.head_dim * cfg.max_len
    return out


def required_bytes(cfg: Config) -> int:
    c, _m = cfg._c()
    req = ctypes.c_size_t(0)
    _check(load_library().duo_cache_init(ctypes.byref(c), None, 0, ctypes.byref(req), None, None),
           "duo_cache_init")
    return int(req.value)


class Cache:
    """Host handle of one cache laid out in a caller-owned device buffer."""

    def __init__(self, cfg: Config, handle: int, buf):
        self.cfg = cfg
        self._h = ctypes.c_void_p(handle)
        self.buf = buf  # keeps the device buffer alive as long as the handle

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.duo_cache_destroy(h)
            self._h = None

    @property
    def handle(self):
        return self._h

    def lengths(self) -> list[int]:
        out = (ctypes.c_int64 * self.cfg.batch)()
        _check(load_library().duo_cache_lengths(self._h, out), "duo_cache_lengths")
        return list(out)

    def layout(self) -> Layout:
        lay = Layout()
        _check(load_library().duo_cache_layout(self._h, ctypes.byref(lay)), "duo_cache_layout")
        return lay

    def head_index(self) -> list[int]:
        out = (ctypes.c_int32 * self.cfg.num_kv_heads)()
        _check(load_library().duo_cache_head_index(self._h, out), "duo_cache_head_index")
        return list(out)

    def pages(self, b: int) -> tuple[list[int], int]:
        """(pool pages of sequence b in position order, free pages left)."""
        n = ctypes.c_int32(0)
        free = ctypes.c_int64(0)
        lib = load_library()
        _check(lib.duo_cache_pages(self._h, b, None, 0, ctypes.byref(n), ctypes.byref(free)), "duo_cache_pages")
        out = (ctypes.c_int32 * max(n.value, 1))()
        _check(lib.duo_cache_pages(self._h, b, out, n.value, ctypes.byref(n), None), "duo_cache_pages")
        return list(out)[:n.value], int(free.value)


def duo_cache_init(cfg: Config, buf: torch.Tensor, stream=None) -> Cache:
    if buf.device.type != "cuda" or buf.dtype != torch.uint8 or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous uint8 CUDA (HIP) tensor")
    c, _m = cfg._c()
    req = ctypes.c_size_t(0)
    h = ctypes.c_void_p()
    _check(load_library().duo_cache_init(ctypes.byref(c), ctypes.c_void_p(buf.data_ptr()), buf.numel(),
                                         ctypes.byref(req), ctypes.byref(h), ctypes.c_void_p(_stream(stream))),
           "duo_cache_init")
    return Cache(cfg, h.value, buf)


def duo_cache_attach(cfg: Config, buf_ptr: int, buf_bytes: int, lengths: Sequence[int], keep=None) -> Cache:
    """Wrap an existing cache buffer (device address ``buf_ptr``); no device work."""
    c, _m = cfg._c()
    lens = (ctypes.c_int64 * max(cfg.batch, 1))(*[int(x) for x in lengths])
    h = ctypes.c_void_p()
    _check(load_library().duo_cache_attach(ctypes.byref(c), ctypes.c_void_p(buf_ptr), buf_bytes, lens,
                                           ctypes.byref(h)), "duo_cache_attach")
    return Cache(cfg, h.value, keep)


def _n_array(n_new, batch):
    arr = (ctypes.c_int32 * batch)(*[int(x) for x in n_new])
    if len(n_new) != batch:
        raise ValueError(f"n_new has {len(n_new)} entries, expected {batch}")
    return arr


def duo_cache_append(cache: Cache, k, v, n_new, stream=None) -> None:
    cfg = cache.cfg
    chunk = k.shape[1]
    shape = (cfg.batch, chunk, cfg.num_kv_heads, cfg.head_dim)
    pk, pv = _dev(k, shape, "k"), _dev(v, shape, "v")
    _check(load_library().duo_cache_append(cache.handle, pk, pv, _n_array(n_new, cfg.batch), chunk,
                                           _stream(stream)), "duo_cache_append")


def duo_prefill(cache: Cache, q, k, v, n_new, out, stream=None) -> None:
    cfg = cache.cfg
    chunk = q.shape[1]
    pq = _dev(q, (cfg.batch, chunk, cfg.num_q_heads, cfg.head_dim), "q")
    po = _dev(out, (cfg.batch, chunk, cfg.num_q_heads, cfg.head_dim), "out")
    kv_shape = (cfg.batch, chunk, cfg.num_kv_heads, cfg.head_dim)
    pk, pv = _dev(k, kv_shape, "k"), _dev(v, kv_shape, "v")
    _check(load_library().duo_prefill(cache.handle, pq, pk, pv, _n_array(n_new, cfg.batch), chunk, po,
                                      _stream(stream)), "duo_prefill")


def _cu_array(cu_seqlens, batch):
    if len(cu_seqlens) != batch + 1:
        raise ValueError(f"cu_seqlens has {len(cu_seqlens)} entries, expected {batch + 1}")
    return (ctypes.c_int32 * (batch + 1))(*[int(x) for x in cu_seqlens])


def duo_cache_append_varlen(cache: Cache, k, v, cu_seqlens, stream=None) -> None:
    """Packed rows: k, v [cu_seqlens[-1], Hkv, D]."""
    cfg = cache.cfg
    shape = (int(cu_seqlens[-1]), cfg.num_kv_heads, cfg.head_dim)
    pk, pv = _dev(k, shape, "k"), _dev(v, shape, "v")
    _check(load_library().duo_cache_append_varlen(cache.handle, pk, pv, _cu_array(cu_seqlens, cfg.batch),
                                                  _stream(stream)), "duo_cache_append_varlen")


def duo_prefill_varlen(cache: Cache, q, k, v, cu_seqlens, out, stream=None) -> None:
    """Packed rows: q, out [cu_seqlens[-1], Hq, D]; k, v [cu_seqlens[-1], Hkv, D]."""
    cfg = cache.cfg
    rows = int(cu_seqlens[-1])
    pq = _dev(q, (rows, cfg.num_q_heads, cfg.head_dim), "q")
    po = _dev(out, (rows, cfg.num_q_heads, cfg.head_dim), "out")
    kv_shape = (rows, cfg.num_kv_heads, cfg.head_dim)
    pk, pv = _dev(k, kv_shape, "k"), _dev(v, kv_shape, "v")
    _check(load_library().duo_prefill_varlen(cache.handle, pq, pk, pv, _cu_array(cu_seqlens, cfg.batch), po,
                                             _stream(stream)), "duo_prefill_varlen")


def duo_cache_release(cache: Cache, b: int, stream=None) -> None:
    _check(load_library().duo_cache_release(cache.handle, int(b), _stream(stream)), "duo_cache_release")


def duo_decode(cache: Cache, q, k, v, out, stream=None) -> None:
    cfg = cache.cfg
    pq = _dev(q, (cfg.batch, cfg.num_q_heads, cfg.head_dim), "q")
    po = _dev(out, (cfg.batch, cfg.num_q_heads, cfg.head_dim), "out")
    kv_shape = (cfg.batch, cfg.num_kv_heads, cfg.head_dim)
    pk, pv = _dev(k, kv_shape, "k"), _dev(v, kv_shape, "v")
    _check(load_library().duo_decode(cache.handle, pq, pk, pv, po, _stream(stream)), "duo_decode")


def duo_decode_static_scratch(cache: Cache, q, k, v, out, stream=None) -> None:
    """duo_decode with the split-K scratch in the library's static device
    array (for callers that cannot allocate; see include/duo.h)."""
    cfg = cache.cfg
    pq = _dev(q, (cfg.batch, cfg.num_q_heads, cfg.head_dim), "q")
    po = _dev(out, (cfg.batch, cfg.num_q_heads, cfg.head_dim), "out")
    kv_shape = (cfg.batch, cfg.num_kv_heads, cfg.head_dim)
    pk, pv = _dev(k, kv_shape, "k"), _dev(v, kv_shape, "v")
    _check(load_library().duo_decode_static_scratch(cache.handle, pq, pk, pv, po, _stream(stream)),
           "duo_decode_static_scratch")


def cache_views(cache: Cache):
    """Typed views of the regions of a cache's device buffer (for tests and
    checkpointing): lengths int32 [B], rk/rv [B,nR,max_len,D] (bf16, or uint8
    codes with rks/rvs fp32 [B,nR,max_len] row scales for DUO_KV_INT8), sk/sv
    [B,nS,sink+recent,D] as bf16.  rk/rv (rks/rvs) are views of the buffer
    for an unblocked contiguous cache and reordered copies for a blocked or
    paged one (whose raw regions are *_blocks or *_pool)."""
    cfg, lay, buf = cache.cfg, cache.layout(), cache.buf
    if buf is None:
        raise ValueError("cache has no torch buffer attached")
    d = cfg.head_dim

    def region(off, shape, dtype):
        nbytes = 1
        for s in shape:
            nbytes *= s
        nbytes *= torch.tensor([], dtype=dtype).element_size()
        return buf[off:off + nbytes].view(dtype).view(*shape)

    rdt = torch.uint8 if lay.kv_format in (DUO_KV_INT8, DUO_KV_FP8) else torch.bfloat16
    views = {"lengths": region(lay.lengths_offset, (cfg.batch,), torch.int32)}
    if lay.page_tokens > 0:
        # pools, the page table, and copies of every sequence's rows gathered
        # through the pages it holds: rk/rv [B, nR, pages held * P, D]
        pt = lay.page_tokens
        pshape = (lay.num_pages, lay.n_retrieval, pt, d)
        views["page_table"] = region(lay.page_table_offset, (cfg.batch, lay.max_pages_per_seq), torch.int32)
        names = [("rk", lay.rk_offset, pshape, rdt), ("rv", lay.rv_offset, pshape, rdt)]
        if lay.kv_format == DUO_KV_INT8:
            names += [("rks", lay.rks_offset, pshape[:3], torch.float32), ("rvs", lay.rvs_offset, pshape[:3], torch.float32)]
        held = [cache.pages(b)[0] for b in range(cfg.batch)]
        most = max([len(h) for h in held] + [1])
        for name, off, shape, dt in names:
            pool = region(off, shape, dt)
            views[name + "_pool"] = pool
            g = torch.zeros((cfg.batch, lay.n_retrieval, most * pt) + tuple(shape[3:]), dtype=dt, device=buf.device)
            for b, pages in enumerate(held):
                for j, page in enumerate(pages):
                    g[b, :, j * pt:(j + 1) * pt] = pool[page]
            views[name] = g
    elif lay.block_tokens > 0:
        # blocked contiguous rows [B][nblk][nR][block][D]: copies reordered to
        # rk/rv [B, nR, max_len, D] (rks/rvs [B, nR, max_len]); the raw
        # regions as *_blocks
        bt = lay.block_tokens
        nblk = (cfg.max_len + bt - 1) // bt
        bshape = (cfg.batch, nblk, lay.n_retrieval, bt, d)
        names = [("rk", lay.rk_offset, bshape, rdt), ("rv", lay.rv_offset, bshape, rdt)]
        if lay.kv_format == DUO_KV_INT8:
            names += [("rks", lay.rks_offset, bshape[:4], torch.float32),
                      ("rvs", lay.rvs_offset, bshape[:4], torch.float32)]
        for name, off, shape, dt in names:
            blocks = region(off, shape, dt)
            views[name + "_blocks"] = blocks
            flat = blocks.transpose(1, 2).reshape((cfg.batch, lay.n_retrieval, nblk * bt) + tuple(shape[4:]))
            views[name] = flat[:, :, :cfg.max_len].contiguous()
    else:
        rshape = (cfg.batch, lay.n_retrieval, cfg.max_len, d)
        views["rk"] = region(lay.rk_offset, rshape, rdt)
        views["rv"] = region(lay.rv_offset, rshape, rdt)
        if lay.kv_format == DUO_KV_INT8:
            views["rks"] = region(lay.rks_offset, rshape[:3], torch.float32)
            views["rvs"] = region(lay.rvs_offset, rshape[:3], torch.float32)
    views.update({
        "sk": region(lay.sk_offset, (cfg.batch, lay.n_streaming, lay.slots_per_streaming_head, d),
                     torch.bfloat16),
        "sv": region(lay.sv_offset, (cfg.batch, lay.n_streaming, lay.slots_per_streaming_head, d),
                     torch.bfloat16),
    })
    return views
