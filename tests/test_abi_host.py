"""Host-side checks of the C ABI (no GPU needed).

Every call here fails validation (or needs no device work), so nothing is
ever enqueued: handles come from duo_cache_attach over a fake, aligned
device address that is never dereferenced.
"""

import ctypes

import pytest

import kv_cache_duo_amd as duo
from workloads import WORKLOADS, workload_mask

FAKE = 0x7f0000000000  # 256-byte aligned, never dereferenced


def _cfg(**kw):
    base = dict(batch=2, num_q_heads=8, num_kv_heads=4, head_dim=128, max_len=1000,
                sink=4, recent=16, kv_head_is_retrieval=[1, 0, 1, 0])
    base.update(kw)
    return duo.Config(**base)


def _attach(cfg, lengths=None):
    req = duo.required_bytes(cfg)
    return duo.duo_cache_attach(cfg, FAKE, req, lengths or [0] * cfg.batch)


def test_library_exports_every_header_function():
    lib = duo.load_library()
    names = duo.header_functions()
    assert {"duo_cache_init", "duo_prefill", "duo_decode", "duo_cache_append"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(duo._SIGNATURES), "binding and header disagree"


def test_status_strings():
    for s in range(6):
        assert duo.status_string(s)
    assert duo.status_string(0) == "ok"


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_required_bytes_for_workloads(name):
    w = WORKLOADS[name]
    mask = workload_mask(w)
    cfg = duo.Config(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim,
                     w.prefill + w.decode_steps, w.sink, w.recent, list(mask))
    req = duo.required_bytes(cfg)
    nr = int(mask.sum())
    ns = w.num_kv_heads - nr
    kv_bytes = 2 * 2 * w.batch * w.head_dim * (nr * _rows(cfg.max_len) + ns * (w.sink + w.recent))
    assert req >= kv_bytes
    # the rest (lengths, tickets, split-K partials, alignment) stays small
    assert req - kv_bytes <= max(64 << 20, kv_bytes // 4)
    for extra in (1, 1024):
        m = cfg.max_len + extra
        bigger = duo.Config(**{**cfg.__dict__, "max_len": m})
        grow = 2 * 2 * w.batch * nr * w.head_dim * (_rows(m) - _rows(cfg.max_len))
        assert duo.required_bytes(bigger) >= req + grow - 4096


def _rows(max_len):
    """Retrieval rows per (sequence, head) of a contiguous cache: max_len, or
    whole 1024-position blocks past one block."""
    return max_len if max_len <= 1024 else -(-max_len // 1024) * 1024


def test_blocked_layout_reported():
    """Contiguous caches longer than 1024 positions report 1024-position
    blocks; shorter ones and paged ones report none."""
    assert _attach(_cfg(max_len=1024), [0, 0]).layout().block_tokens == 0
    lay = _attach(_cfg(max_len=1025), [0, 0]).layout()
    assert lay.block_tokens == 1024
    c = _cfg(max_len=5000)
    assert duo.required_bytes(c) >= 2 * 2 * c.batch * sum(c.kv_head_is_retrieval) * c.head_dim * 5120


@pytest.mark.parametrize("kw,status", [
    (dict(num_q_heads=6), duo.DUO_ERR_INVALID_ARG),       # Hq % Hkv != 0
    (dict(head_dim=96), duo.DUO_ERR_UNSUPPORTED),
    (dict(head_dim=256), duo.DUO_ERR_UNSUPPORTED),
    (dict(sink=-1), duo.DUO_ERR_INVALID_ARG),
    (dict(recent=0), duo.DUO_ERR_INVALID_ARG),
    (dict(batch=0), duo.DUO_ERR_INVALID_ARG),
    (dict(batch=129, kv_head_is_retrieval=[1, 0, 1, 0]), duo.DUO_ERR_UNSUPPORTED),
    (dict(max_len=0), duo.DUO_ERR_INVALID_ARG),
    (dict(scale=-1.0), duo.DUO_ERR_INVALID_ARG),
    (dict(scale=float("nan")), duo.DUO_ERR_INVALID_ARG),
    (dict(max_len=1 << 31), duo.DUO_ERR_UNSUPPORTED),
    (dict(rope_base=-1.0), duo.DUO_ERR_INVALID_ARG),
    (dict(rope_base=float("inf")), duo.DUO_ERR_INVALID_ARG),
    (dict(rope_base=10000.0, rope_style=2), duo.DUO_ERR_INVALID_ARG),
    (dict(page_tokens=256, num_pages=8), duo.DUO_ERR_INVALID_ARG),     # pages below 512 positions
    (dict(page_tokens=1000, num_pages=8), duo.DUO_ERR_INVALID_ARG),    # not a power of two
    (dict(page_tokens=131072, num_pages=8), duo.DUO_ERR_INVALID_ARG),  # above 65536
    (dict(page_tokens=512, num_pages=0), duo.DUO_ERR_INVALID_ARG),     # empty pool
])
def test_invalid_configs(kw, status):
    with pytest.raises(duo.DuoError) as e:
        duo.required_bytes(_cfg(**kw))
    assert e.value.status == status


def test_null_mask_and_null_outputs():
    lib = duo.load_library()
    c, _m = _cfg()._c()
    c.kv_head_is_retrieval = None
    req = ctypes.c_size_t(0)
    assert lib.duo_cache_init(ctypes.byref(c), None, 0, ctypes.byref(req), None, None) == duo.DUO_ERR_INVALID_ARG
    c2, _m2 = _cfg()._c()
    # no buffer and nowhere to write the size
    assert lib.duo_cache_init(ctypes.byref(c2), None, 0, None, None, None) == duo.DUO_ERR_INVALID_ARG
    assert lib.duo_cache_init(None, None, 0, ctypes.byref(req), None, None) == duo.DUO_ERR_INVALID_ARG


def test_attach_checks_buffer_and_lengths():
    cfg = _cfg()
    req = duo.required_bytes(cfg)
    with pytest.raises(duo.DuoError) as e:
        duo.duo_cache_attach(cfg, FAKE, req - 1, [0, 0])
    assert e.value.status == duo.DUO_ERR_BUFFER_TOO_SMALL
    with pytest.raises(duo.DuoError) as e:
        duo.duo_cache_attach(cfg, FAKE + 16, req, [0, 0])
    assert e.value.status == duo.DUO_ERR_INVALID_ARG
    with pytest.raises(duo.DuoError) as e:
        duo.duo_cache_attach(cfg, FAKE, req, [0, cfg.max_len + 1])
    assert e.value.status == duo.DUO_ERR_INVALID_ARG
    with pytest.raises(duo.DuoError) as e:
        duo.duo_cache_attach(cfg, 0, req, [0, 0])
    assert e.value.status == duo.DUO_ERR_INVALID_ARG


def test_layout_and_head_index():
    cfg = _cfg(kv_head_is_retrieval=[0, 1, 1, 0])
    c = _attach(cfg, [5, 7])
    assert c.lengths() == [5, 7]
    lay = c.layout()
    assert (lay.n_retrieval, lay.n_streaming) == (2, 2)
    assert lay.slots_per_streaming_head == cfg.sink + cfg.recent
    offs = [lay.lengths_offset, lay.work_offset, lay.rk_offset, lay.rv_offset, lay.sk_offset, lay.sv_offset]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    row = 2 * cfg.head_dim
    assert lay.rv_offset - lay.rk_offset >= cfg.batch * 2 * cfg.max_len * row
    assert lay.sv_offset - lay.sk_offset >= cfg.batch * 2 * (cfg.sink + cfg.recent) * row
    assert lay.total_bytes == duo.required_bytes(cfg)
    # retrieval heads 1,2 -> indices 0,1; streaming heads 0,3 -> indices 0,1
    assert c.head_index() == [0, 0, 1, 1]


def test_int8_layout():
    """DUO_KV_INT8: retrieval rows of D bytes plus fp32 row-scale regions;
    streaming regions unchanged; the bf16 layout reports no scale regions."""
    cfg = _cfg(kv_head_is_retrieval=[0, 1, 1, 0], kv_format=duo.DUO_KV_INT8)
    c = _attach(cfg, [5, 7])
    lay = c.layout()
    assert lay.kv_format == duo.DUO_KV_INT8
    offs = [lay.lengths_offset, lay.work_offset, lay.rk_offset, lay.rv_offset, lay.rks_offset, lay.rvs_offset,
            lay.sk_offset, lay.sv_offset]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert lay.rv_offset - lay.rk_offset >= cfg.batch * 2 * cfg.max_len * cfg.head_dim
    assert lay.rks_offset - lay.rv_offset >= cfg.batch * 2 * cfg.max_len * cfg.head_dim
    assert lay.sk_offset - lay.rvs_offset >= cfg.batch * 2 * cfg.max_len * 4
    bf = _attach(_cfg(kv_head_is_retrieval=[0, 1, 1, 0]), [5, 7]).layout()
    assert bf.kv_format == duo.DUO_KV_BF16 and bf.rks_offset == -1 and bf.rvs_offset == -1
    # retrieval bytes: D + 4 per row and tensor instead of 2 D
    r8 = (lay.sk_offset - lay.rk_offset)
    r16 = (bf.sk_offset - bf.rk_offset)
    assert r8 < r16 * 0.6
    with pytest.raises(duo.DuoError) as e:
        duo.required_bytes(_cfg(kv_format=3))
    assert e.value.status == duo.DUO_ERR_INVALID_ARG


def test_prefill_staging_workspace_size_and_checks():
    """The layout reports the staging workspace that serves every prefill:
    4 B nR D max_len bytes for an int8 cache and an fp8 one with exact
    prefill, plus 2 B nS D max_len with rotary embedding (0 otherwise); the
    configuration's workspace must be 16-byte aligned with a size >= 0."""
    for kw in (dict(kv_format=duo.DUO_KV_INT8), dict(kv_format=duo.DUO_KV_FP8)):
        cfg = _cfg(kv_head_is_retrieval=[0, 1, 1, 0], **kw)
        lay = _attach(cfg, [5, 7]).layout()
        assert lay.prefill_staging_bytes == duo.prefill_staging_bytes(cfg) == 4 * 2 * 2 * 128 * 1000
    for kw in (dict(kv_format=duo.DUO_KV_BF16), dict(kv_format=duo.DUO_KV_FP8, fp8_prefill=duo.DUO_FP8_PREFILL_MFMA)):
        other = _cfg(kv_head_is_retrieval=[0, 1, 1, 0], **kw)
        assert _attach(other, [5, 7]).layout().prefill_staging_bytes == 0 == duo.prefill_staging_bytes(other)
    # rotary embedding adds the streaming heads' turned chunk K rows (any format)
    for fmt, extra in ((duo.DUO_KV_BF16, 0), (duo.DUO_KV_INT8, 4 * 2 * 2 * 128 * 1000)):
        rope = _cfg(kv_head_is_retrieval=[0, 1, 1, 0], kv_format=fmt, rope_base=10000.0)
        want = extra + 2 * 2 * 2 * 128 * 1000
        assert _attach(rope, [5, 7]).layout().prefill_staging_bytes == want == duo.prefill_staging_bytes(rope)
    lib = duo.load_library()
    for ptr, nbytes, ok in ((FAKE, 1 << 20, True), (None, 0, True), (FAKE + 8, 1 << 20, False), (FAKE, -1, False)):
        c, _mask = cfg._c()
        c.prefill_staging = ptr
        c.prefill_staging_bytes = nbytes
        req = ctypes.c_size_t(0)
        st = lib.duo_cache_init(ctypes.byref(c), None, 0, ctypes.byref(req), None, None)
        assert (st == duo.DUO_OK) == ok, (ptr, nbytes, st)
        if not ok:
            assert st == duo.DUO_ERR_INVALID_ARG


def test_fp8_layout():
    """DUO_KV_FP8: retrieval rows of D bytes, no scale regions (one scale per
    tensor, in the configuration); streaming regions stay bf16."""
    cfg = _cfg(kv_head_is_retrieval=[0, 1, 1, 0], kv_format=duo.DUO_KV_FP8, kv_scale_k=0.5, kv_scale_v=2.0)
    c = _attach(cfg, [5, 7])
    lay = c.layout()
    assert lay.kv_format == duo.DUO_KV_FP8 and lay.rks_offset == -1 and lay.rvs_offset == -1
    assert lay.rv_offset - lay.rk_offset >= cfg.batch * 2 * cfg.max_len * cfg.head_dim
    assert lay.sk_offset - lay.rv_offset >= cfg.batch * 2 * cfg.max_len * cfg.head_dim
    bf = _attach(_cfg(kv_head_is_retrieval=[0, 1, 1, 0]), [5, 7]).layout()
    assert (lay.sk_offset - lay.rk_offset) * 2 <= (bf.sk_offset - bf.rk_offset) + 2 * 256
    assert lay.sv_offset - lay.sk_offset == bf.sv_offset - bf.sk_offset


@pytest.mark.parametrize("kw,status", [
    (dict(kv_format=2, kv_scale_k=0.3), duo.DUO_ERR_INVALID_ARG),            # not a power of two
    (dict(kv_format=2, kv_scale_v=-2.0), duo.DUO_ERR_INVALID_ARG),
    (dict(kv_format=2, kv_scale_k=float("inf")), duo.DUO_ERR_INVALID_ARG),
    (dict(kv_format=2, kv_scale_k=2.0 ** 40), duo.DUO_ERR_INVALID_ARG),       # outside [2^-32, 2^32]
])
def test_fp8_invalid_configs(kw, status):
    with pytest.raises(duo.DuoError) as e:
        duo.required_bytes(_cfg(**kw))
    assert e.value.status == status


@pytest.mark.parametrize("fmt", [duo.DUO_KV_INT8, duo.DUO_KV_FP8])
def test_rope_with_8bit_formats_needs_no_extra_bytes(fmt):
    plain = duo.required_bytes(_cfg(kv_format=fmt))
    for style in (duo.DUO_ROPE_INTERLEAVED, duo.DUO_ROPE_HALF):
        assert duo.required_bytes(_cfg(kv_format=fmt, rope_base=10000.0, rope_style=style)) == plain


def test_fp8_scale_zero_means_one():
    a = duo.required_bytes(_cfg(kv_format=duo.DUO_KV_FP8, kv_scale_k=0.0, kv_scale_v=0.0))
    b = duo.required_bytes(_cfg(kv_format=duo.DUO_KV_FP8, kv_scale_k=0.25, kv_scale_v=8.0))
    assert a == b > 0


def _raw(c):
    return duo.load_library(), c.handle


def test_call_validation_leaves_state_unchanged():
    cfg = _cfg()
    c = _attach(cfg, [3, 990])
    lib, h = _raw(c)
    A = FAKE + 4096  # aligned fake device pointers
    n_ok = (ctypes.c_int32 * 2)(1, 1)
    # null / misaligned pointers
    assert lib.duo_decode(h, None, A, A, A, None) == duo.DUO_ERR_INVALID_ARG
    assert lib.duo_decode(h, A + 2, A, A, A, None) == duo.DUO_ERR_INVALID_ARG
    assert lib.duo_decode(None, A, A, A, A, None) == duo.DUO_ERR_INVALID_ARG
    assert lib.duo_prefill(h, A, A, A, n_ok, 4, None, None) == duo.DUO_ERR_INVALID_ARG
    assert lib.duo_prefill(h, A, A + 8, A, n_ok, 4, A, None) == duo.DUO_ERR_INVALID_ARG
    assert lib.duo_prefill(h, A, A, A, None, 4, A, None) == duo.DUO_ERR_INVALID_ARG
    assert lib.duo_cache_append(h, None, A, n_ok, 4, None) == duo.DUO_ERR_INVALID_ARG
    # chunk and n_new ranges
    assert lib.duo_prefill(h, A, A, A, n_ok, 0, A, None) == duo.DUO_ERR_INVALID_ARG
    assert lib.duo_prefill(h, A, A, A, (ctypes.c_int32 * 2)(5, 1), 4, A, None) == duo.DUO_ERR_INVALID_ARG
    assert lib.duo_cache_append(h, A, A, (ctypes.c_int32 * 2)(-1, 0), 4, None) == duo.DUO_ERR_INVALID_ARG
    # row offsets b * chunk are int32: B * chunk past 2^31 - 1 is refused before any work
    big = 2**30 + 1
    assert lib.duo_cache_append(h, A, A, n_ok, big, None) == duo.DUO_ERR_UNSUPPORTED
    assert lib.duo_prefill(h, A, A, A, n_ok, big, A, None) == duo.DUO_ERR_UNSUPPORTED
    # capacity: sequence 1 holds 990 of 1000 tokens
    assert lib.duo_prefill(h, A, A, A, (ctypes.c_int32 * 2)(0, 11), 16, A, None) == duo.DUO_ERR_CAPACITY
    assert lib.duo_cache_append(h, A, A, (ctypes.c_int32 * 2)(0, 11), 16, None) == duo.DUO_ERR_CAPACITY
    assert c.lengths() == [3, 990]
    full = _attach(cfg, [10, cfg.max_len])
    lib, h2 = _raw(full)
    assert lib.duo_decode(h2, A, A, A, A, None) == duo.DUO_ERR_CAPACITY
    assert full.lengths() == [10, cfg.max_len]


def test_introspection_null_arguments():
    lib = duo.load_library()
    lay = duo.Layout()
    assert lib.duo_cache_layout(None, ctypes.byref(lay)) == duo.DUO_ERR_INVALID_ARG
    assert lib.duo_cache_lengths(None, None) == duo.DUO_ERR_INVALID_ARG
    c = _attach(_cfg())
    assert lib.duo_cache_head_index(c.handle, None) == duo.DUO_ERR_INVALID_ARG
    lib.duo_cache_destroy(None)  # no-op


def test_binding_rejects_cpu_tensors():
    import torch
    cfg = _cfg()
    with pytest.raises(ValueError):
        duo.duo_cache_init(cfg, torch.empty(16, dtype=torch.uint8))
    c = _attach(cfg)
    q = torch.zeros(2, 8, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        duo.duo_decode(c, q, q[:, :4], q[:, :4], q)


def test_rope_config_accepted_and_layout_unchanged():
    """Rotary embedding changes no region: the layout equals the plain one."""
    base = duo.Config(2, 8, 4, 128, 1000, 4, 64, [1, 0, 1, 0])
    for style in (duo.DUO_ROPE_INTERLEAVED, duo.DUO_ROPE_HALF):
        cfg = duo.Config(2, 8, 4, 128, 1000, 4, 64, [1, 0, 1, 0], rope_base=500000.0, rope_style=style)
        assert duo.required_bytes(cfg) == duo.required_bytes(base)
    # the style is not read without a base
    cfg = duo.Config(2, 8, 4, 128, 1000, 4, 64, [1, 0, 1, 0], rope_base=0.0, rope_style=7)
    assert duo.required_bytes(cfg) == duo.required_bytes(base)


def test_paged_layout_sizes_the_pool_not_the_batch():
    """A paged cache holds num_pages pages of every retrieval head instead of
    B * max_len rows: 32 sequences of up to 65536 positions in a pool of 100
    pages of 1024 positions."""
    pg = _cfg(batch=32, max_len=65536, page_tokens=1024, num_pages=100)
    flat = _cfg(batch=32, max_len=65536)
    c = _attach(pg)
    lay = c.layout()
    row = 2 * pg.head_dim
    assert (lay.page_tokens, lay.num_pages, lay.max_pages_per_seq) == (1024, 100, 64)
    assert lay.page_table_offset > lay.lengths_offset and lay.page_table_offset % 256 == 0
    assert lay.rv_offset - lay.rk_offset == 100 * 2 * 1024 * row  # pages * nR * P * row
    assert duo.required_bytes(pg) < duo.required_bytes(flat) / 15
    flay = _attach(flat).layout()
    assert flay.page_table_offset == -1 and flay.page_tokens == 0
    # int8 pools: codes and scales per page
    q8 = _cfg(batch=32, max_len=65536, page_tokens=1024, num_pages=100, kv_format=duo.DUO_KV_INT8)
    lay8 = _attach(q8).layout()
    assert lay8.rv_offset - lay8.rk_offset == 100 * 2 * 1024 * pg.head_dim
    assert lay8.rvs_offset - lay8.rks_offset == 100 * 2 * 1024 * 4


def test_paged_attach_needs_empty_sequences():
    cfg = _cfg(page_tokens=512, num_pages=4)
    with pytest.raises(duo.DuoError) as e:
        _attach(cfg, [0, 3])
    assert e.value.status == duo.DUO_ERR_INVALID_ARG
    assert _attach(cfg).pages(0) == ([], 4)


def test_paged_pool_exhaustion_is_checked_before_any_work():
    """Calls that would need more pages than the pool has free fail with
    CAPACITY and change nothing (no device work is enqueued)."""
    lib = duo.load_library()
    cfg = _cfg(max_len=4096, page_tokens=512, num_pages=3)
    c = _attach(cfg)
    A = ctypes.c_void_p(FAKE)
    # 2 sequences x 1000 tokens need 2 + 2 pages > 3
    n = (ctypes.c_int32 * 2)(1000, 1000)
    assert lib.duo_prefill(c.handle, A, A, A, n, 1000, A, None) == duo.DUO_ERR_CAPACITY
    assert lib.duo_cache_append(c.handle, A, A, n, 1000, None) == duo.DUO_ERR_CAPACITY
    cu = (ctypes.c_int32 * 3)(0, 1000, 2000)
    assert lib.duo_prefill_varlen(c.handle, A, A, A, cu, A, None) == duo.DUO_ERR_CAPACITY
    assert lib.duo_cache_append_varlen(c.handle, A, A, cu, None) == duo.DUO_ERR_CAPACITY
    assert c.lengths() == [0, 0] and c.pages(0) == ([], 3) and c.pages(1) == ([], 3)
    # decode needs one page per sequence: a pool of 1 is too small for 2
    one = _attach(_cfg(max_len=4096, page_tokens=512, num_pages=1))
    assert lib.duo_decode(one.handle, A, A, A, A, None) == duo.DUO_ERR_CAPACITY
    assert one.pages(0) == ([], 1)


def test_varlen_validation():
    lib = duo.load_library()
    c = _attach(_cfg())
    A = ctypes.c_void_p(FAKE)
    for cu in [(1, 2, 3), (0, 5, 3), (0, 600, 1601)]:  # cu[0] != 0, decreasing, over max_len
        arr = (ctypes.c_int32 * 3)(*cu)
        st = lib.duo_prefill_varlen(c.handle, A, A, A, arr, A, None)
        assert st in (duo.DUO_ERR_INVALID_ARG, duo.DUO_ERR_CAPACITY)
    assert lib.duo_prefill_varlen(c.handle, A, A, A, None, A, None) == duo.DUO_ERR_INVALID_ARG
    assert lib.duo_cache_append_varlen(c.handle, A, None, (ctypes.c_int32 * 3)(0, 1, 2), None) == duo.DUO_ERR_INVALID_ARG
    # no rows at all: nothing to do, null tensors accepted, nothing enqueued
    zero = (ctypes.c_int32 * 3)(0, 0, 0)
    assert lib.duo_prefill_varlen(c.handle, None, None, None, zero, None, None) == duo.DUO_OK
    assert lib.duo_cache_append_varlen(c.handle, None, None, zero, None) == duo.DUO_OK
    assert c.lengths() == [0, 0]


def test_release_checks_its_arguments():
    lib = duo.load_library()
    c = _attach(_cfg())
    assert lib.duo_cache_release(None, 0, None) == duo.DUO_ERR_INVALID_ARG
    assert lib.duo_cache_release(c.handle, 2, None) == duo.DUO_ERR_INVALID_ARG
    assert lib.duo_cache_release(c.handle, -1, None) == duo.DUO_ERR_INVALID_ARG


def test_failed_launch_keeps_pages_and_lengths():
    """A call whose kernel launch fails (DUO_ERR_HIP) gives back the pages it
    took and keeps every length.  Forced from the host: on a machine without
    a HIP device every launch fails, so the call gets past validation and
    fails at its first launch (the page-table write).  Where a device exists
    the launch would really write through the fake buffer address, so the
    test only runs without one."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("needs a host without a HIP device (every launch must fail)")
    lib = duo.load_library()
    cfg = _cfg(max_len=4096, page_tokens=512, num_pages=8)
    c = _attach(cfg, [0, 0])
    before = [c.pages(b) for b in range(cfg.batch)]
    n = (ctypes.c_int32 * 2)(600, 100)
    fake = ctypes.c_void_p(FAKE)
    assert lib.duo_cache_append(c.handle, fake, fake, n, 600, None) == duo.DUO_ERR_HIP
    assert lib.duo_prefill(c.handle, fake, fake, fake, n, 600, fake, None) == duo.DUO_ERR_HIP
    assert lib.duo_decode(c.handle, fake, fake, fake, fake, None) == duo.DUO_ERR_HIP
    assert [c.pages(b) for b in range(cfg.batch)] == before == [([], 8), ([], 8)]
    assert c.lengths() == [0, 0]


def test_stale_library_is_refused(tmp_path, monkeypatch):
    """load_library() checks the digest the build recorded against the
    sources in the tree and refuses a library built from other sources."""
    import json

    lib = tmp_path / "libduo.so"
    lib.write_bytes(b"not loaded: the record is checked first")
    monkeypatch.setattr(duo, "LIB_PATH", str(lib))
    monkeypatch.setattr(duo, "_lib", None)
    with pytest.raises(RuntimeError, match="no build record"):
        duo.load_library()
    (tmp_path / "libduo.build.json").write_text(json.dumps({"sources_sha256": "0" * 64, "arch": "gfx950"}))
    with pytest.raises(RuntimeError, match="other sources"):
        duo.load_library()


def test_static_scratch_decode_checks_its_size_first():
    """duo_decode_static_scratch refuses a handle whose decode needs more
    counters or partial results than the library's static array holds
    (UNSUPPORTED), before any device work."""
    lib = duo.load_library()
    big = _cfg(batch=128, num_q_heads=256, num_kv_heads=256, head_dim=128, max_len=1000,
               kv_head_is_retrieval=[1] * 256)
    c = _attach(big, [0] * 128)
    fake = ctypes.c_void_p(FAKE)
    assert lib.duo_decode_static_scratch(c.handle, fake, fake, fake, fake, None) == duo.DUO_ERR_UNSUPPORTED
    assert c.lengths() == [0] * 128
    assert lib.duo_decode_static_scratch(None, fake, fake, fake, fake, None) == duo.DUO_ERR_INVALID_ARG
