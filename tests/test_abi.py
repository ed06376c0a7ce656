"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before touching a device (runs without a GPU)."""
import ctypes
import subprocess

import pytest

from attention_reuse_amd import mac


@pytest.fixture(scope="module")
def lib():
    return mac.load()


def _params(**kw):
    base = dict(batch=2, n_q_heads=32, n_kv_heads=8, head_dim=128,
                kv_dtype=mac.MAC_DTYPE_BF16, ring_k=1024, band_r=256,
                kv_capacity=4096, tau=0.6)
    base.update(kw)
    return mac.make_params(**base)


def test_exports_every_declared_function(lib):
    names = mac.header_functions()
    assert len(names) >= 12
    out = subprocess.check_output(["nm", "-D", "--defined-only", mac.LIB_PATH]).decode()
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        assert hasattr(lib, n)


def test_struct_layout_matches_header():
    assert ctypes.sizeof(mac.mac_params) == 104
    assert mac.mac_params.kv_stride_b.offset == 48
    assert mac.mac_params.front_sink.offset == 72
    assert mac.mac_params.page_size.offset == 76
    assert mac.mac_params.max_pages.offset == 80
    assert mac.mac_params.page_table.offset == 88
    assert mac.mac_params.max_context.offset == 96
    assert mac.mac_params.min_context.offset == 100
    assert ctypes.sizeof(mac.mac_rings) == 32


@pytest.mark.parametrize("kw,ok", [
    (dict(page_size=16, max_pages=256, page_table=0x1000), True),
    (dict(page_size=64, max_pages=64, page_table=0x1000), True),
    (dict(page_size=64, max_pages=63, page_table=0x1000), False),   # pages do not cover T
    (dict(page_size=8, max_pages=512, page_table=0x1000), False),   # below 16 tokens
    (dict(page_size=48, max_pages=100, page_table=0x1000), False),  # not a power of two
    (dict(page_size=64, max_pages=64, page_table=None), False),
    (dict(page_size=64, max_pages=64, page_table=0x1002), False),   # misaligned table
    (dict(max_pages=64), False),                                    # table without pages
])
def test_paged_params(lib, kw, ok):
    assert (mac.mac_workspace_bytes(_params(**kw)) > 0) == ok


@pytest.mark.parametrize("kw,status", [
    (dict(max_context=4096), 0), (dict(max_context=0), 0), (dict(max_context=4095), -6),
    (dict(max_context=131072, kv_capacity=262144 + 512), -6), (dict(max_context=-1), -1),
    (dict(min_context=2048), 0), (dict(min_context=1 << 30), 0), (dict(min_context=-5), -1),
])
def test_context_limits(lib, kw, status):
    """max_context refuses a handle or call whose KV capacity exceeds it, on
    the host before any launch; min_context only has to be non-negative
    (it is applied on the device per request)."""
    p = _params(**kw)
    rc = lib.mac_full_decode(ctypes.byref(p), 0x1000, 0x2000, 0x3000, 0x4000,
                             None, None, None, 0, None)
    assert rc == (status if status != 0 else -1)
    assert (mac.mac_workspace_bytes(p) > 0) == (status == 0)
    if status != 0:
        # Refused before any device call (no handle is made).
        rings = mac.mac_rings(0x1000, 0x2000, 0x3000, 0x4000)
        h = ctypes.c_void_p()
        ctx = (ctypes.c_int32 * 2)(4096, 4096)
        rc = lib.mac_init_rings(ctypes.byref(p), ctypes.byref(rings), 0x6000, 1 << 40,
                                None, None, 0, ctx, None, None, None, ctypes.byref(h))
        assert rc == status and not h.value
    out = (ctypes.c_size_t * 4)()
    assert lib.mac_ring_bytes(ctypes.byref(p), out) == status


def test_front_sink_bounds(lib):
    assert mac.mac_workspace_bytes(_params(front_sink=4096)) > 0
    assert mac.mac_workspace_bytes(_params(front_sink=4097)) == 0
    assert mac.mac_workspace_bytes(_params(front_sink=-1)) == 0


def test_status_strings_and_chunk(lib):
    assert mac.mac_status_string(0) == "ok"
    assert "workspace" in mac.mac_status_string(-4)
    assert "max_context" in mac.mac_status_string(-6)
    assert "mac_init_rings" in mac.mac_status_string(-7)
    assert mac.mac_chunk_tokens(0, 63) == 64
    assert mac.mac_chunk_tokens(0, 64 * 128 - 1) == 64
    assert mac.mac_chunk_tokens(0, 64 * 128) == 128
    assert mac.mac_chunk_tokens(0, 128 * 128 - 1) == 128
    assert mac.mac_chunk_tokens(0, 128 * 128) == 256
    assert mac.mac_chunk_tokens(0, 65536) == 1024
    assert mac.mac_chunk_tokens(100, 65536) == 512
    assert mac.mac_chunk_tokens(0, 262399) == 4096
    assert mac.mac_chunk_tokens(5, 4) == -1
    # A 128-token minimum grid.
    assert mac.mac_chunk_tokens(0, 127, 128) == 128
    assert mac.mac_chunk_tokens(0, 128 * 128 - 1, 128) == 128
    assert mac.mac_chunk_tokens(0, 128 * 128, 128) == 256
    assert mac.mac_chunk_tokens(0, 65536, 128) == 1024
    assert mac.mac_chunk_tokens(0, 100, 96) == -1 and mac.mac_chunk_tokens(0, 100, 32) == -1


def test_min_chunk_by_shape(lib):
    """64-token grid up to 16 KV groups per layer, 256 above."""
    assert mac.mac_min_chunk_tokens(_params(batch=2)) == 64      # 16 groups
    assert mac.mac_min_chunk_tokens(_params(batch=1)) == 64
    assert mac.mac_min_chunk_tokens(_params(batch=3)) == 256     # 24 groups
    assert mac.mac_min_chunk_tokens(_params(batch=16)) == 256
    assert mac.mac_min_chunk_tokens(_params(batch=0)) == -1


def test_workspace_and_ring_sizes(lib):
    p = _params()
    ws = mac.mac_workspace_bytes(p)
    assert ws > 0
    # 2 x 32 heads x 1024 slots x 128 dims: bf16 query ring, fp32 summaries.
    assert mac.mac_ring_bytes(p) == (2 * 32 * 1024 * 128 * 2, 2 * 32 * 1024 * 128 * 4,
                                     2 * 32 * 1024 * 4, 2 * 8 * 1024 * 4)
    # The split-KV partials are bounded per KV group, so the workspace does
    # not grow with the KV capacity.
    assert mac.mac_workspace_bytes(_params(kv_capacity=65536)) == ws


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), -2), (dict(kv_dtype=7), -2), (dict(n_q_heads=48, n_kv_heads=3), -2),
    (dict(n_q_heads=30), -1), (dict(ring_k=0), -1), (dict(band_r=-1), -1),
    (dict(batch=0), -1), (dict(kv_capacity=0), -1), (dict(tau=float("nan")), -1),
    (dict(thresh_mode=2), -1), (dict(strides=(0, 0, 100)), -1), (dict(flags=32), -1),
    (dict(flags=6), -1), (dict(flags=18), -1), (dict(flags=20), -1), (dict(flags=1), 0),
    (dict(flags=3), 0), (dict(flags=5), 0), (dict(flags=17), 0), (dict(flags=24), 0),
    (dict(batch=300), -2),
    (dict(strides=(1 << 20, 4096 * 136, 136)), 0), (dict(strides=(1 << 20, 4096 * 132, 132)), -5),
])
def test_param_validation(lib, kw, status):
    p = _params(**kw)
    rc = lib.mac_full_decode(ctypes.byref(p), 0x1000, 0x2000, 0x3000, 0x4000,
                             None, None, None, 0, None)
    # Valid parameters then fail on the NULL output / workspace pointers.
    assert rc == (status if status != 0 else -1)
    assert (mac.mac_workspace_bytes(p) > 0) == (status == 0)


def test_pointer_validation_happens_before_any_device_call(lib):
    p = _params()
    ws = mac.mac_workspace_bytes(p)
    # Misaligned query pointer.
    rc = lib.mac_full_decode(ctypes.byref(p), 0x1004, 0x2000, 0x3000, 0x4000,
                             0x5000, None, 0x6000, ws, None)
    assert rc == -5
    # Workspace too small.
    rc = lib.mac_full_decode(ctypes.byref(p), 0x1000, 0x2000, 0x3000, 0x4000,
                             0x5000, None, 0x6000, ws - 1, None)
    assert rc == -4
    # Decode step with a NULL handle.
    assert lib.mac_decode_step(None, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000,
                               0x1000, None, None, None, None, None) == -7
    # Init: more warm positions than ring slots, and a prompt shorter than W.
    rings = mac.mac_rings(0x1000, 0x2000, 0x3000, 0x4000)
    h = ctypes.c_void_p()
    ctx = (ctypes.c_int32 * 2)(4096, 4096)
    rc = lib.mac_init_rings(ctypes.byref(p), ctypes.byref(rings), 0x6000, ws,
                            0x7000, 0x8000, 1025, ctx, 0x9000, 0xa000, None,
                            ctypes.byref(h))
    assert rc == -1
    ctx = (ctypes.c_int32 * 2)(4096, 100)
    rc = lib.mac_init_rings(ctypes.byref(p), ctypes.byref(rings), 0x6000, ws,
                            0x7000, 0x8000, 512, ctx, 0x9000, 0xa000, None,
                            ctypes.byref(h))
    assert rc == -1
    assert lib.mac_release(None) == -7
    assert lib.mac_profile_start(None, 3) == -7
    assert lib.mac_join_aux(None, None) == -7
    assert lib.mac_bind_epochs(None, None) == -7
    f = ctypes.c_int32()
    assert lib.mac_read_device_status(ctypes.byref(p), None, None, ctypes.byref(f)) == -1


def test_binding_raises_when_library_missing(monkeypatch, tmp_path):
    monkeypatch.setattr(mac, "_lib", None)
    monkeypatch.setattr(mac, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        mac.load()


@pytest.mark.parametrize("cmin", [64, 128, 256])
@pytest.mark.parametrize("s,e,r", [(0, 0, 0), (0, 127, 32), (0, 128, 32), (5, 1000, 256),
                                   (300, 1000, 256), (900, 1000, 256), (0, 262399, 256),
                                   (1000, 1000, 0), (0, 500, 1000), (640, 1000, 361)])
def test_partition_covers_range_on_the_grid(lib, s, e, r, cmin):
    """Items tile [s, e] in order; every interior boundary is a multiple of the
    chunk or the rectify split e - r + 1; no item crosses either."""
    C = mac.mac_chunk_tokens(s, e, cmin)
    assert C >= cmin
    items = mac.mac_partition(s, e, r, cmin)
    assert len(items) <= 130
    assert items[0][0] == s and items[-1][1] == e + 1
    for (a0, a1), (b0, _) in zip(items, items[1:]):
        assert a1 == b0
    sp = e - r + 1
    for t0, t1 in items:
        assert t0 < t1 <= t0 + C
        assert (t0 // C) == ((t1 - 1) // C)                  # inside one grid chunk
        assert not (t0 < sp < t1)                            # never straddles the split
        if t0 != s:
            assert t0 % C == 0 or t0 == sp
    # A miss head (s = 0) gets the same items as a full decode.
    if s == 0:
        assert items == mac.mac_partition(0, e, r, cmin)
    assert lib.mac_partition(5, 4, 0, cmin, None, None, 0) == -1
    assert lib.mac_partition(0, 4, 0, 100, None, None, 0) == -1


@pytest.mark.parametrize("cmin", [64, 128, 256])
@pytest.mark.parametrize("s,e,r,F", [(0, 0, 0, 64), (0, 63, 16, 64), (0, 200, 16, 64),
                                     (150, 3000, 256, 128), (0, 33000, 256, 128),
                                     (500, 600, 600, 4096), (0, 5000, 0, 1), (10, 90, 5, 0)])
def test_group_items_with_front_sink(lib, s, e, r, F, cmin):
    """Main items tile [max(s, F), e] as the plain partition does; the sink
    item [0, min(F, e + 1)) comes last; the rectify split counts only main
    items, and the items before it cover exactly [max(s, F), e - r]."""
    items, nb = mac.mac_group_items(s, e, r, F, cmin)
    ms = max(s, F)
    main = items[:-1] if F > 0 else items
    if F > 0:
        assert items[-1] == (0, min(F, e + 1))
    if ms <= e:
        assert main == mac.mac_partition(ms, e, r, cmin)
    else:
        assert main == []
    covered = [t for a, b in main[:nb] for t in range(a, b)]
    assert covered == list(range(ms, max(ms, e - r + 1)))
    assert nb <= len(main)
    # F = 0 is the plain partition.
    if F == 0:
        assert items == mac.mac_partition(s, e, r, cmin)
    assert lib.mac_group_items(5, 4, 0, 0, cmin, None, None, None, 0) == -1
    assert lib.mac_group_items(0, 4, 0, 4097, cmin, None, None, None, 0) == -1


def test_noalloc_full_decode_rejects_before_any_device_call(lib):
    """The allocation-free full decode checks its arguments and the scratch
    size on the host: a shape needing more than the static scratch is
    refused with its own status, before any launch."""
    big = _params(batch=48)   # 384 KV groups: ~100 MiB of partials
    assert mac.mac_workspace_bytes(big) > mac.MAC_NOALLOC_SCRATCH_BYTES
    rc = lib.mac_full_decode_noalloc(ctypes.byref(big), 0x1000, 0x2000, 0x3000, 0x4000,
                                     0x5000, None, None)
    assert rc == mac.MAC_ERR_SCRATCH_TOO_SMALL
    assert "scratch" in mac.mac_status_string(rc)
    p = _params()
    assert lib.mac_full_decode_noalloc(ctypes.byref(p), 0x1000, 0x2000, 0x3000, 0x4000,
                                       None, None, None) == -1
    assert lib.mac_full_decode_noalloc(ctypes.byref(p), 0x1004, 0x2000, 0x3000, 0x4000,
                                       0x5000, None, None) == -5


def test_timeline_summary_reads_the_latest_launch():
    """The timeline tool's host summary: workgroups of the latest launch are
    those that started within 20 us of its last start, and a point counts
    only when it was written after the workgroup's own start."""
    from attention_reuse_amd import timeline as tl
    W = [[0] * 32 for _ in range(8)]
    for w in range(4):                      # an earlier launch
        W[w][0], W[w][11] = 1000 + w, 5000
    for w in range(4, 8):                   # the latest launch: entries 100 us later
        W[w][0] = 11000 + 10 * w
        W[w][3] = W[w][0] + 300             # planned 3 us after start
        W[w][4] = W[w][0] + 400
        W[w][16], W[w][17] = 7, 7
    W[7][11] = 900                          # stale: before this launch's start
    lines = tl.summarize(W)
    assert lines[0].endswith(": 4")
    planned = [l for l in lines if l.startswith("group planned")][0].split()
    # planned 3.0, 3.1, 3.2, 3.3 us after the first start: min 3.0, median 3.2
    assert planned[2] == "4" and float(planned[3]) == 3.0 and float(planned[5]) == 3.2
    end = [l for l in lines if l.startswith("end (ran items)")][0].split()
    assert end[3] == "0"
