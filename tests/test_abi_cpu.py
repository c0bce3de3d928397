"""The C-ABI library on the CPU: it loads, exports every symbol the header declares,
and rejects bad arguments with the documented status before touching the GPU
(no compute call is made here)."""
import ctypes
import os
import re

import pytest

from exact_tiled_attention_pa_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pagedattn.h")

FAKE = 0x1000  # never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return B.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(B.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert lib.pa_version().decode().count(".") == 2
    for st in range(7):
        assert lib.pa_status_string(st).decode().startswith("PA_")
    assert "unknown" in lib.pa_status_string(99).decode()


def lay(num_pages=12, ps=256, hkv=1, d=64, maxp=3):
    return B.make_layout(num_pages, ps, hkv, d, maxp)


def prefill(lib, layout, *, q=FAKE, k=FAKE, v=FAKE, bt=FAKE, lens=FAKE, causal=1, scale=0.125,
            out=FAKE, qs=FAKE, batch=1, hq=1, max_q_len=600):
    return lib.pa_prefill(q, k, v, bt, lens, causal, scale, out, qs, batch, hq, max_q_len,
                          ctypes.byref(layout), None)


@pytest.mark.parametrize("kw,layout_kw,status", [
    (dict(q=None), {}, B.PA_ERR_NULL),
    (dict(out=None), {}, B.PA_ERR_NULL),
    (dict(qs=None), {}, B.PA_ERR_NULL),
    ({}, dict(d=96), B.PA_ERR_UNSUPPORTED),
    ({}, dict(ps=8), B.PA_ERR_UNSUPPORTED),
    ({}, dict(ps=512), B.PA_ERR_UNSUPPORTED),
    ({}, dict(ps=48), B.PA_ERR_UNSUPPORTED),
    ({}, dict(num_pages=0), B.PA_ERR_INVALID_ARG),
    (dict(batch=-1), {}, B.PA_ERR_INVALID_ARG),
    (dict(hq=3), dict(hkv=2), B.PA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), {}, B.PA_ERR_INVALID_ARG),
    (dict(scale=-1.0), {}, B.PA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), {}, B.PA_ERR_INVALID_ARG),
    (dict(max_q_len=769), {}, B.PA_ERR_INVALID_ARG),   # 3 pages of 256 hold 768 tokens
    (dict(max_q_len=-5), {}, B.PA_ERR_INVALID_ARG),
    (dict(q=FAKE + 2), {}, B.PA_ERR_INVALID_ARG),      # 16-byte pieces: aligned arrays
    (dict(k=FAKE + 8), {}, B.PA_ERR_INVALID_ARG),
    (dict(out=FAKE + 4), {}, B.PA_ERR_INVALID_ARG),
])
def test_prefill_rejects(lib, kw, layout_kw, status):
    st = prefill(lib, lay(**layout_kw), **kw)
    assert st == status, (st, B.last_error())
    assert B.last_error()


def test_window_argument_errors(lib):
    layout = lay()
    args = (FAKE, FAKE, FAKE, FAKE, FAKE)
    st = lib.pa_prefill_window(*args, 1, 0.125, FAKE, FAKE, 1, 1, 600, -1, ctypes.byref(layout), None)
    assert st == B.PA_ERR_INVALID_ARG
    st = lib.pa_prefill_window(*args, 0, 0.125, FAKE, FAKE, 1, 1, 600, 16, ctypes.byref(layout), None)
    assert st == B.PA_ERR_INVALID_ARG and "causal" in B.last_error()
    st = lib.pa_prefill_window(*args, 1, 0.125, FAKE, FAKE, 0, 1, 600, 16, ctypes.byref(layout), None)
    assert st == B.PA_OK
    dl = B.make_layout(100, 16, 4, 128, 10)
    need = lib.pa_decode_workspace_bytes(2, 4, ctypes.byref(dl))
    st = lib.pa_decode_window(*args, 0.1, FAKE, 2, 4, -3, FAKE, need, ctypes.byref(dl), None)
    assert st == B.PA_ERR_INVALID_ARG


def test_token_rows_above_32_mib_are_rejected(lib):
    layout = lay(hkv=131073, d=128)
    assert prefill(lib, layout, hq=131073) == B.PA_ERR_INVALID_ARG
    assert "2^24" in B.last_error()
    # exactly 2^24 elements per token row is accepted
    ok = lay(hkv=131072, d=128)
    assert lib.pa_decode_split_tokens(64, 131072, ctypes.byref(ok)) == 256
    assert lib.pa_decode_split_tokens(64, 131073, ctypes.byref(layout)) == 0


def test_prefill_empty_batch_is_ok_without_device(lib):
    assert prefill(lib, lay(), batch=0) == B.PA_OK
    assert prefill(lib, lay(), max_q_len=0) == B.PA_OK
    assert B.last_error() == ""


def test_decode_workspace_size_formula(lib):
    layout = B.make_layout(17000, 16, 32, 128, 512)
    # 512 pages x 16 tokens, 256-token splits -> 32 splits per sequence
    assert lib.pa_decode_split_tokens(64, 32, ctypes.byref(layout)) == 256
    o = 64 * 32 * 32 * 128 * 4
    ml = 64 * 32 * 32 * 2 * 4
    r = lambda n: (n + 255) // 256 * 256
    plan = (2 + 64 * 32) * 4  # claim counter, pair count, (sequence, split) pairs
    assert lib.pa_decode_workspace_bytes(64, 32, ctypes.byref(layout)) == r(o) + r(ml) + r(plan)
    big = B.make_layout(128, 256, 8, 128, 128)
    assert lib.pa_decode_split_tokens(64, 8, ctypes.byref(big)) == 256
    bad = B.make_layout(128, 24, 8, 128, 128)
    assert lib.pa_decode_workspace_bytes(1, 8, ctypes.byref(bad)) == 0
    assert lib.pa_decode_split_tokens(64, 8, ctypes.byref(bad)) == 0
    # grouped heads: 8 K/V heads, 2 query heads each keep 256-token splits; 4 or more
    # per K/V head walk 1024-token splits -> 8 splits of 8192 tokens
    gl = B.make_layout(17000, 16, 8, 128, 512)
    assert lib.pa_decode_split_tokens(64, 16, ctypes.byref(gl)) == 256
    assert lib.pa_decode_split_tokens(64, 64, ctypes.byref(gl)) == 1024
    assert lib.pa_decode_split_tokens(64, 12, ctypes.byref(gl)) == 0  # not a multiple of 8
    o = 64 * 64 * 8 * 128 * 4
    ml = 64 * 64 * 8 * 2 * 4
    plan = (2 + 64 * 8) * 4
    assert lib.pa_decode_workspace_bytes(64, 64, ctypes.byref(gl)) == r(o) + r(ml) + r(plan)


def test_decode_rejects(lib):
    layout = B.make_layout(100, 16, 4, 128, 10)
    need = lib.pa_decode_workspace_bytes(2, 4, ctypes.byref(layout))
    call = lambda **kw: lib.pa_decode(
        kw.get("q", FAKE), FAKE, FAKE, FAKE, kw.get("lens", FAKE), kw.get("scale", 0.1),
        kw.get("out", FAKE), kw.get("batch", 2), kw.get("hq", 4), kw.get("ws", FAKE),
        kw.get("ws_bytes", need), ctypes.byref(kw.get("layout", layout)), None)
    assert call(q=None) == B.PA_ERR_NULL
    assert call(out=None) == B.PA_ERR_NULL
    assert call(lens=None) == B.PA_ERR_NULL
    assert call(ws=None) == B.PA_ERR_WORKSPACE
    assert call(ws_bytes=need - 1) == B.PA_ERR_WORKSPACE
    assert call(scale=float("nan")) == B.PA_ERR_INVALID_ARG
    assert call(hq=6) == B.PA_ERR_INVALID_ARG
    assert call(layout=B.make_layout(100, 16, 4, 80, 10)) == B.PA_ERR_UNSUPPORTED
    assert call(q=FAKE + 2) == B.PA_ERR_INVALID_ARG
    assert call(ws=FAKE + 4) == B.PA_ERR_WORKSPACE
    assert "aligned" in B.last_error()
    assert call(batch=0) == B.PA_OK
    st = lib.pa_decode_partial(FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, 2, 4, None, need,
                               ctypes.byref(layout), None)
    assert st == B.PA_ERR_WORKSPACE
    st = lib.pa_decode_combine(FAKE, None, 2, 4, FAKE, need, ctypes.byref(layout), None)
    assert st == B.PA_ERR_NULL


def test_decode_noalloc_rejects_before_any_hip_call(lib):
    """The no-allocation decode checks every argument, and the size of the partials
    against its static workspace, before it looks the workspace up on a device."""
    layout = B.make_layout(100, 16, 4, 128, 10)
    call = lambda **kw: lib.pa_decode_noalloc(
        kw.get("q", FAKE), FAKE, FAKE, FAKE, kw.get("lens", FAKE), kw.get("scale", 0.1),
        kw.get("out", FAKE), kw.get("batch", 2), kw.get("hq", 4),
        ctypes.byref(kw.get("layout", layout)), None)
    assert call(q=None) == B.PA_ERR_NULL
    assert call(out=None) == B.PA_ERR_NULL
    assert call(lens=None) == B.PA_ERR_NULL
    assert call(scale=-1.0) == B.PA_ERR_INVALID_ARG
    assert call(hq=6) == B.PA_ERR_INVALID_ARG
    assert call(batch=-1) == B.PA_ERR_INVALID_ARG
    assert call(layout=B.make_layout(100, 16, 4, 80, 10)) == B.PA_ERR_UNSUPPORTED
    # 128 sequences x 32 heads over up to 32768 tokens: 272 MB of partials > 64 MiB
    mixed = B.make_layout(70000, 16, 32, 128, 2048)
    need = lib.pa_decode_workspace_bytes(128, 32, ctypes.byref(mixed))
    assert need > B.NOALLOC_SCRATCH_BYTES
    assert call(layout=mixed, batch=128, hq=32) == B.PA_ERR_WORKSPACE
    assert "static" in B.last_error() and str(B.NOALLOC_SCRATCH_BYTES) in B.last_error()
    # the 64-sequence decode batch (32 heads, up to 8192 tokens) fits
    dec = B.make_layout(20000, 16, 32, 128, 512)
    assert lib.pa_decode_workspace_bytes(64, 32, ctypes.byref(dec)) <= B.NOALLOC_SCRATCH_BYTES
    assert call(batch=0) == B.PA_OK


def test_noalloc_limit_matches_header():
    text = open(HEADER).read()
    assert "#define PA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)" in text
    assert B.NOALLOC_SCRATCH_BYTES == 64 << 20


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(4, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        B.pa_prefill(q, q, q, q, q, True, 0.1, q, q, 4)
    with pytest.raises(ValueError):  # a prepared call runs the same checks, once
        B.PreparedPrefill(q, q, q, q, q, True, 0.1, q, q, 4)
    with pytest.raises(ValueError):
        B.PreparedDecode(q, q, q, q, q, 0.1, q, q)


def test_kv_append_rejects(lib):
    layout = B.make_layout(100, 16, 4, 128, 10)
    call = lambda **kw: lib.pa_kv_append(
        kw.get("k", FAKE), FAKE, FAKE, kw.get("pos", FAKE), kw.get("n", 3), FAKE,
        kw.get("vp", FAKE), FAKE, kw.get("seqs", 2), ctypes.byref(kw.get("layout", layout)), None)
    assert call(k=None) == B.PA_ERR_NULL
    assert call(pos=None) == B.PA_ERR_NULL
    assert call(vp=None) == B.PA_ERR_NULL
    assert call(n=-1) == B.PA_ERR_INVALID_ARG
    assert call(seqs=-1) == B.PA_ERR_INVALID_ARG
    assert call(layout=B.make_layout(100, 12, 4, 128, 10)) == B.PA_ERR_UNSUPPORTED
    assert call(layout=B.make_layout(100, 16, 4, 96, 10)) == B.PA_ERR_UNSUPPORTED
    assert call(layout=B.make_layout(0, 16, 4, 128, 10)) == B.PA_ERR_INVALID_ARG
    assert lib.pa_kv_append(FAKE, FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, 1, None, None) \
        == B.PA_ERR_NULL
    assert call(k=FAKE + 2) == B.PA_ERR_INVALID_ARG and "aligned" in B.last_error()
    assert call(n=0) == B.PA_OK
    assert call(seqs=0) == B.PA_OK


def test_copy_pages_rejects(lib):
    layout = B.make_layout(100, 16, 4, 128, 1)
    call = lambda **kw: lib.pa_copy_pages(
        kw.get("k", FAKE), FAKE, kw.get("src", FAKE), FAKE, kw.get("n", 3),
        ctypes.byref(kw.get("layout", layout)), None)
    assert call(k=None) == B.PA_ERR_NULL
    assert call(src=None) == B.PA_ERR_NULL
    assert call(n=-2) == B.PA_ERR_INVALID_ARG
    assert call(layout=B.make_layout(100, 16, 4, 32, 1)) == B.PA_ERR_UNSUPPORTED
    # 256 tokens x 8192 heads x 128 x 2 bytes = 512 MiB per page
    assert call(layout=B.make_layout(4, 256, 8192, 128, 1)) == B.PA_ERR_INVALID_ARG
    assert call(k=FAKE + 8) == B.PA_ERR_INVALID_ARG
    assert call(n=0) == B.PA_OK


def test_prefill_path_override_is_checked(lib, monkeypatch):
    """PA_PREFILL_PATH forces one of the two prefill kernels; an unknown value is an
    argument error before anything is enqueued (also for an empty batch), and a forced
    split-key launch whose 32-row query tiles overflow the grid is refused."""
    monkeypatch.setenv("PA_PREFILL_PATH", "fastest")
    assert prefill(lib, lay()) == B.PA_ERR_INVALID_ARG
    assert "PA_PREFILL_PATH=fastest" in B.last_error()
    assert prefill(lib, lay(), batch=0) == B.PA_ERR_INVALID_ARG
    for ok in ("", "auto", "tiles", "split"):
        monkeypatch.setenv("PA_PREFILL_PATH", ok)
        assert prefill(lib, lay(), batch=0) == B.PA_OK, ok
    big = lay(num_pages=8700, ps=256, maxp=8700)
    monkeypatch.setenv("PA_PREFILL_PATH", "split")
    assert prefill(lib, big, max_q_len=32 * 65535 + 1) == B.PA_ERR_INVALID_ARG
    assert "split-key" in B.last_error()


def test_small_batches_take_shorter_decode_splits(lib):
    """One-head-per-row decode: 256-key splits unless the batch would give pass 1 fewer
    units (split x group of 4 heads at d = 128, 8 at d = 64) than the 256 CUs; then 128,
    then 64.  The workspace follows the split length; grouped heads keep 1024."""
    mha = B.make_layout(100, 16, 32, 128, 256)  # 4096 keys per sequence, 8 head groups
    st = lambda batch, hq=32, layout=mha: lib.pa_decode_split_tokens(batch, hq,
                                                                     ctypes.byref(layout))
    assert st(2) == 256      # 2 x 16 splits x 8 groups = 256 units
    assert st(1) == 128      # 1 x 16 x 8 = 128 < 256; 1 x 32 x 8 = 256
    four = B.make_layout(100, 16, 4, 128, 1024)  # 16384 keys, 4 heads: one group
    assert st(1, 4, four) == 64   # 64 and 128 units at 256 and 128 keys; 256 at 64
    assert st(4, 4, four) == 256  # 4 x 64 x 1 = 256
    d64 = B.make_layout(100, 16, 32, 64, 256)  # 8 heads per group: 4 groups
    assert st(1, 32, d64) == 64   # 1 x 16 x 4 = 64, x 32 = 128, x 64 = 256
    # grouped heads: 1024 keys, halved down to 128 while K/V heads x head blocks of 32 x
    # splits x batch < 256 workgroups
    gl = B.make_layout(100, 16, 8, 128, 256)   # 4096 keys, 8 K/V heads, g = 8: one block
    assert st(1, 64, gl) == 128    # 32 and 64 and 128 workgroups at 1024, 512, 256 keys
    assert st(8, 64, gl) == 1024   # 8 x 4 x 8 = 256
    assert st(2, 64, gl) == 256    # 2 x 16 x 8 = 256
    gl_long = B.make_layout(100, 16, 8, 128, 4096)  # 65536 keys
    assert st(1, 64, gl_long) == 1024  # 64 splits x 8 = 512
    assert st(-1) == 0
    # the workspace holds max_splits = 4096 / split partials per (sequence, head)
    r = lambda n: (n + 255) // 256 * 256
    need = r(1 * 32 * 32 * 128 * 4) + r(1 * 32 * 32 * 2 * 4) + r((2 + 32) * 4)
    assert lib.pa_decode_workspace_bytes(1, 32, ctypes.byref(mha)) == need
