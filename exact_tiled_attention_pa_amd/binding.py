"""Thin ctypes binding of libpagedattn (argument marshalling only).

Every function of the C ABI (include/pagedattn.h) is exposed under the same
name.  The tensor-level functions check shapes, dtypes and devices on the host,
pass raw device pointers and torch's current HIP stream, and raise
PagedAttnError on a non-zero status.  All attention arithmetic happens in the
HIP kernels of the library; nothing here computes a result, and there is no
fallback: if the library is missing or no GPU is present, calls fail loudly.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpagedattn.so")

PA_OK = 0
PA_ERR_NULL = 1
PA_ERR_INVALID_ARG = 2
PA_ERR_UNSUPPORTED = 3
PA_ERR_WORKSPACE = 4
PA_ERR_HIP = 5
PA_ERR_CAPACITY = 6

# Every symbol the header declares.
EXPORTED = (
    "pa_prefill", "pa_decode_workspace_bytes", "pa_decode_split_tokens", "pa_decode",
    "pa_decode_partial", "pa_decode_combine", "pa_prefill_window", "pa_decode_window",
    "pa_decode_noalloc",
    "pa_kv_append", "pa_copy_pages", "pa_bm_create", "pa_bm_destroy", "pa_bm_add_sequence",
    "pa_bm_fork", "pa_bm_free_sequence", "pa_bm_append", "pa_bm_seq_len",
    "pa_bm_free_page_count", "pa_bm_ref_count", "pa_bm_export", "pa_bm_validate",
    "pa_status_string", "pa_last_error", "pa_version",
)


class PagedAttnError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{status_string(status)} -- {detail}")
        self.status = status
        self.detail = detail


class ContractError(ValueError):
    """A block table, length or chunk offset breaks the device-array contract of
    pagedattn.h (raised by the opt-in host-side check, before anything is launched)."""


# Opt-in host-side check of the device-array contract before each attention launch
# (PA_CHECK_CONTRACT=1 in the environment, or set_contract_check(True)).  It copies
# the block table, lengths and chunk offsets to the host, which synchronises with
# the device: a debugging aid, not for timed or captured work.
_check_contract = os.environ.get("PA_CHECK_CONTRACT", "0") not in ("", "0")


def set_contract_check(enabled: bool) -> None:
    global _check_contract
    _check_contract = bool(enabled)


def _host_ints(x):
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu").numpy().astype(np.int64)
    return np.asarray(x, dtype=np.int64)


def contract_violations(block_table, seq_lens, num_pages: int, page_size: int,
                        q_start=None, max_q_len=None, total_q=None, max_report: int = 8):
    """Host-side check of the device-array contract stated in pagedattn.h: for each
    sequence b with KV length L_b, 0 <= L_b <= max_pages_per_seq * page_size and
    0 <= block_table[b, p] < num_pages for every p < ceil(L_b / page_size), the pages
    the kernels read ("What is Paged FlashAttention?", "Practical example": physical
    page = block_table[pos // page_size]).  With chunk offsets (prefill), q_start
    starts at 0, never decreases, stays within total_q rows, and every
    q_len_b = q_start[b+1] - q_start[b] is at most L_b and at most max_q_len.
    Accepts host arrays or tensors (copied to the host).  Returns a list of
    messages, empty when the arrays keep the contract."""
    bt = _host_ints(block_table)
    lens = _host_ints(seq_lens).reshape(-1)
    bad = []
    if bt.ndim != 2 or bt.shape[0] < lens.size:
        return [f"block_table has shape {bt.shape}, expected [>= {lens.size}, max_pages]"]
    max_pages = bt.shape[1]
    for b, L in enumerate(lens.tolist()):
        if L < 0 or L > max_pages * page_size:
            bad.append(f"sequence {b}: length {L} outside [0, {max_pages * page_size}] "
                       f"({max_pages} table entries of {page_size} tokens)")
            continue
        n = -(-L // page_size)
        row = bt[b, :n]
        out = np.nonzero((row < 0) | (row >= num_pages))[0]
        for p in out[:2].tolist():
            bad.append(f"sequence {b}: logical page {p} maps to physical page {int(row[p])}, "
                       f"outside the pool of {num_pages} pages")
    if q_start is not None:
        qs = _host_ints(q_start).reshape(-1)
        if qs.size != lens.size + 1:
            bad.append(f"q_start has {qs.size} entries, expected {lens.size + 1}")
        else:
            if qs[0] != 0:
                bad.append(f"q_start[0] is {int(qs[0])}, expected 0")
            if total_q is not None and qs[-1] > total_q:
                bad.append(f"q_start[{lens.size}] = {int(qs[-1])} exceeds the {total_q} "
                           "query rows")
            for b in range(lens.size):
                q_len = int(qs[b + 1] - qs[b])
                if q_len < 0:
                    bad.append(f"sequence {b}: q_start decreases ({int(qs[b])} -> "
                               f"{int(qs[b + 1])})")
                elif q_len > lens[b]:
                    bad.append(f"sequence {b}: {q_len} query rows over only {int(lens[b])} keys")
                elif max_q_len is not None and q_len > max_q_len:
                    bad.append(f"sequence {b}: {q_len} query rows exceed max_q_len {max_q_len}")
    return bad[:max_report]


def _enforce_contract(block_table, seq_lens, k_pool, **kw):
    if not _check_contract:
        return
    bad = contract_violations(block_table, seq_lens, int(k_pool.shape[0]),
                              int(k_pool.shape[1]), **kw)
    if bad:
        raise ContractError("device-array contract broken: " + "; ".join(bad))


class KVLayout(ctypes.Structure):
    _fields_ = [
        ("num_pages", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
    ]


_lib = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Loads libpagedattn.so (built in-tree by __graft_entry__.build or
    `python -m exact_tiled_attention_pa_amd.build`) and returns its handle; raises if it
    is missing.  Without `path` the in-tree library is loaded once and is the one every
    call of this module uses; with `path` that file is loaded and its handle returned,
    and the module's calls keep using their own library."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"libpagedattn.so not found at {p}; build it first "
                           "(python -m exact_tiled_attention_pa_amd.build)")
    lib = ctypes.CDLL(p)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    lay = ctypes.POINTER(KVLayout)
    lib.pa_prefill.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, f32, vp, vp, i32, i32, i32,
                               lay, vp]
    lib.pa_prefill.restype = ctypes.c_int
    lib.pa_decode_workspace_bytes.argtypes = [i32, i32, lay]
    lib.pa_decode_workspace_bytes.restype = sz
    lib.pa_decode_split_tokens.argtypes = [i32, i32, lay]
    lib.pa_decode_split_tokens.restype = i32
    lib.pa_decode.argtypes = [vp, vp, vp, vp, vp, f32, vp, i32, i32, vp, sz, lay, vp]
    lib.pa_decode.restype = ctypes.c_int
    lib.pa_decode_partial.argtypes = [vp, vp, vp, vp, vp, f32, i32, i32, vp, sz, lay, vp]
    lib.pa_decode_partial.restype = ctypes.c_int
    lib.pa_decode_combine.argtypes = [vp, vp, i32, i32, vp, sz, lay, vp]
    lib.pa_decode_combine.restype = ctypes.c_int
    lib.pa_prefill_window.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, f32, vp, vp, i32, i32,
                                      i32, i32, lay, vp]
    lib.pa_prefill_window.restype = ctypes.c_int
    lib.pa_decode_window.argtypes = [vp, vp, vp, vp, vp, f32, vp, i32, i32, i32, vp, sz, lay, vp]
    lib.pa_decode_window.restype = ctypes.c_int
    lib.pa_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, f32, vp, i32, i32, lay, vp]
    lib.pa_decode_noalloc.restype = ctypes.c_int
    lib.pa_kv_append.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, i32, lay, vp]
    lib.pa_kv_append.restype = ctypes.c_int
    lib.pa_copy_pages.argtypes = [vp, vp, vp, vp, i32, lay, vp]
    lib.pa_copy_pages.restype = ctypes.c_int
    i32p = ctypes.POINTER(ctypes.c_int32)
    lib.pa_bm_create.argtypes = [i32, i32, i32, i32, ctypes.POINTER(vp)]
    lib.pa_bm_create.restype = ctypes.c_int
    lib.pa_bm_destroy.argtypes = [vp]
    lib.pa_bm_destroy.restype = None
    lib.pa_bm_add_sequence.argtypes = [vp, i32p]
    lib.pa_bm_add_sequence.restype = ctypes.c_int
    lib.pa_bm_fork.argtypes = [vp, i32, i32, i32p]
    lib.pa_bm_fork.restype = ctypes.c_int
    lib.pa_bm_free_sequence.argtypes = [vp, i32]
    lib.pa_bm_free_sequence.restype = ctypes.c_int
    lib.pa_bm_append.argtypes = [vp, i32, i32, i32p, i32p, i32p]
    lib.pa_bm_append.restype = ctypes.c_int
    lib.pa_bm_seq_len.argtypes = [vp, i32]
    lib.pa_bm_seq_len.restype = i32
    lib.pa_bm_free_page_count.argtypes = [vp]
    lib.pa_bm_free_page_count.restype = i32
    lib.pa_bm_ref_count.argtypes = [vp, i32]
    lib.pa_bm_ref_count.restype = i32
    lib.pa_bm_export.argtypes = [vp, vp, vp]
    lib.pa_bm_export.restype = ctypes.c_int
    lib.pa_bm_validate.argtypes = [vp]
    lib.pa_bm_validate.restype = ctypes.c_int
    lib.pa_status_string.argtypes = [ctypes.c_int]
    lib.pa_status_string.restype = ctypes.c_char_p
    lib.pa_last_error.argtypes = []
    lib.pa_last_error.restype = ctypes.c_char_p
    lib.pa_version.argtypes = []
    lib.pa_version.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().pa_status_string(int(status)).decode()


def last_error() -> str:
    return load_library().pa_last_error().decode()


def _check(status: int):
    if status != PA_OK:
        raise PagedAttnError(status, last_error())


def make_layout(num_pages, page_size, num_kv_heads, head_dim, max_pages_per_seq) -> KVLayout:
    return KVLayout(int(num_pages), int(page_size), int(num_kv_heads), int(head_dim),
                    int(max_pages_per_seq))


def layout_of(k_pool: torch.Tensor, block_table: torch.Tensor) -> KVLayout:
    num_pages, page_size, num_kv_heads, head_dim = k_pool.shape
    return make_layout(num_pages, page_size, num_kv_heads, head_dim, block_table.shape[1])


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _require(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _check_device_tensors(**tensors):
    dev = None
    for name, t in tensors.items():
        _require(isinstance(t, torch.Tensor), f"{name} must be a torch.Tensor")
        _require(t.is_cuda, f"{name} must be on a GPU (got {t.device})")
        _require(t.is_contiguous(), f"{name} must be contiguous")
        dev = dev or t.device
        _require(t.device == dev, f"{name} is on {t.device}, expected {dev}")


def _prefill_args(q, k_pool, v_pool, block_table, seq_lens, causal, scale, out, q_start,
                  max_q_len, window):
    """Validates a prefill call and returns (C function, its arguments but the stream,
    the layout they point to)."""
    _enforce_contract(block_table, seq_lens, k_pool, q_start=q_start,
                      max_q_len=int(max_q_len), total_q=int(q.shape[0]))
    _check_device_tensors(q=q, k_pool=k_pool, v_pool=v_pool, block_table=block_table,
                          seq_lens=seq_lens, out=out, q_start=q_start)
    for name, t in (("q", q), ("k_pool", k_pool), ("v_pool", v_pool), ("out", out)):
        _require(t.dtype == torch.bfloat16, f"{name} must be bfloat16")
    for name, t in (("block_table", block_table), ("seq_lens", seq_lens), ("q_start", q_start)):
        _require(t.dtype == torch.int32, f"{name} must be int32")
    _require(k_pool.dim() == 4 and v_pool.shape == k_pool.shape, "k_pool/v_pool: [P, ps, Hkv, d]")
    _require(q.dim() == 3 and q.shape[2] == k_pool.shape[3], "q: [total_q, Hq, d]")
    _require(out.shape == q.shape, "out must have q's shape")
    batch = seq_lens.numel()
    _require(block_table.dim() == 2 and block_table.shape[0] >= batch, "block_table: [batch, maxp]")
    _require(q_start.numel() == batch + 1, "q_start: [batch + 1]")
    lay = layout_of(k_pool, block_table)
    head = (_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(seq_lens),
            int(bool(causal)), float(scale), _ptr(out), _ptr(q_start), batch, q.shape[1],
            int(max_q_len))
    lib = load_library()
    if window:
        return lib.pa_prefill_window, head + (int(window), ctypes.byref(lay)), lay
    return lib.pa_prefill, head + (ctypes.byref(lay),), lay


def pa_prefill(q, k_pool, v_pool, block_table, seq_lens, causal, scale, out, q_start,
               max_q_len: int, stream=None, window: int = 0):
    """Paged (chunked) prefill: out[q_start[b]:q_start[b+1]] = attention of sequence b's
    query rows over its L_b = seq_lens[b] paged keys.  See pa_prefill in pagedattn.h;
    window > 0 calls pa_prefill_window.  With the contract check on, the block table,
    lengths and chunk offsets are checked on the host first (ContractError)."""
    fn, args, _lay = _prefill_args(q, k_pool, v_pool, block_table, seq_lens, causal, scale,
                                   out, q_start, max_q_len, window)
    _check(fn(*args, _stream(stream)))
    return out


class PreparedPrefill:
    """A pa_prefill call validated and marshalled once, then launched any number of times
    on the same buffers (whose contents may change between launches): each launch is one
    C call, so a serving loop or a short prefill pays the checks once instead of per
    launch.  With the contract check on, it runs when the call is prepared.  The object
    keeps its tensors alive."""

    def __init__(self, q, k_pool, v_pool, block_table, seq_lens, causal, scale, out, q_start,
                 max_q_len: int, window: int = 0):
        self._fn, self._args, self._lay = _prefill_args(
            q, k_pool, v_pool, block_table, seq_lens, causal, scale, out, q_start, max_q_len,
            window)
        self._tensors = (q, k_pool, v_pool, block_table, seq_lens, out, q_start)
        self.out = out

    def launch(self, stream=None):
        """Enqueues the prefill on `stream` (default: torch's current stream); returns out."""
        st = self._fn(*self._args, _stream(stream))
        if st != PA_OK:
            raise PagedAttnError(st, last_error())
        return self.out


def pa_decode_workspace_bytes(batch: int, num_q_heads: int, layout: KVLayout) -> int:
    return int(load_library().pa_decode_workspace_bytes(int(batch), int(num_q_heads),
                                                        ctypes.byref(layout)))


def pa_decode_split_tokens(batch: int, num_q_heads: int, layout: KVLayout) -> int:
    return int(load_library().pa_decode_split_tokens(int(batch), int(num_q_heads),
                                                     ctypes.byref(layout)))


def decode_workspace(q, k_pool, block_table) -> torch.Tensor:
    """Allocates (through torch) a workspace large enough for pa_decode."""
    n = pa_decode_workspace_bytes(q.shape[0], q.shape[1], layout_of(k_pool, block_table))
    _require(n > 0, "invalid decode shapes")
    return torch.empty(n, dtype=torch.uint8, device=q.device)


def _decode_checks(q, k_pool, v_pool, block_table, seq_lens, workspace, out=None):
    _enforce_contract(block_table, seq_lens, k_pool)
    tensors = dict(q=q, k_pool=k_pool, v_pool=v_pool, block_table=block_table,
                   seq_lens=seq_lens, workspace=workspace)
    if out is not None:
        tensors["out"] = out
    _check_device_tensors(**tensors)
    for name, t in (("q", q), ("k_pool", k_pool), ("v_pool", v_pool)):
        _require(t.dtype == torch.bfloat16, f"{name} must be bfloat16")
    _require(out is None or (out.dtype == torch.bfloat16 and out.shape == q.shape),
             "out must be bfloat16 with q's shape")
    _require(block_table.dtype == torch.int32 and seq_lens.dtype == torch.int32,
             "block_table and seq_lens must be int32")
    _require(k_pool.dim() == 4 and v_pool.shape == k_pool.shape, "k_pool/v_pool: [P, ps, Hkv, d]")
    _require(q.dim() == 3 and q.shape[2] == k_pool.shape[3], "q: [batch, Hq, d]")
    _require(seq_lens.numel() == q.shape[0] and block_table.shape[0] >= q.shape[0],
             "seq_lens: [batch]; block_table: [batch, maxp]")


def pa_decode(q, k_pool, v_pool, block_table, seq_lens, scale, out, workspace, stream=None,
              window: int = 0):
    """One query token per sequence over all its L_b cached tokens (split-KV + combine);
    window > 0 calls pa_decode_window (only the last `window` tokens)."""
    _decode_checks(q, k_pool, v_pool, block_table, seq_lens, workspace, out)
    lay = layout_of(k_pool, block_table)
    nbytes = workspace.numel() * workspace.element_size()
    if window:
        st = load_library().pa_decode_window(
            _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(seq_lens),
            float(scale), _ptr(out), q.shape[0], q.shape[1], int(window), _ptr(workspace),
            nbytes, ctypes.byref(lay), _stream(stream))
    else:
        st = load_library().pa_decode(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
                                      _ptr(seq_lens), float(scale), _ptr(out), q.shape[0],
                                      q.shape[1], _ptr(workspace), nbytes, ctypes.byref(lay),
                                      _stream(stream))
    _check(st)
    return out


class PreparedDecode:
    """A pa_decode call (with its workspace) validated and marshalled once, then launched
    any number of times on the same buffers: each launch is one C call.  With the
    contract check on, it runs when the call is prepared.  Keeps its tensors alive."""

    def __init__(self, q, k_pool, v_pool, block_table, seq_lens, scale, out, workspace,
                 window: int = 0):
        _decode_checks(q, k_pool, v_pool, block_table, seq_lens, workspace, out)
        self._lay = layout_of(k_pool, block_table)
        nbytes = workspace.numel() * workspace.element_size()
        lib = load_library()
        head = (_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(seq_lens),
                float(scale), _ptr(out), q.shape[0], q.shape[1])
        tail = (_ptr(workspace), nbytes, ctypes.byref(self._lay))
        if window:
            self._fn, self._args = lib.pa_decode_window, head + (int(window),) + tail
        else:
            self._fn, self._args = lib.pa_decode, head + tail
        self._tensors = (q, k_pool, v_pool, block_table, seq_lens, out, workspace)
        self.out = out

    def launch(self, stream=None):
        """Enqueues both decode passes on `stream` (default: torch's current stream)."""
        st = self._fn(*self._args, _stream(stream))
        if st != PA_OK:
            raise PagedAttnError(st, last_error())
        return self.out


# size of the library's static decode workspace (PA_NOALLOC_SCRATCH_BYTES in pagedattn.h)
NOALLOC_SCRATCH_BYTES = 64 << 20


def pa_decode_noalloc(q, k_pool, v_pool, block_table, seq_lens, scale, out, stream=None):
    """pa_decode without a workspace argument: the library keeps the split partials in
    its own static device array (one per GPU), so the call allocates nothing.  Calls
    that overlap on one GPU race; requests needing more than NOALLOC_SCRATCH_BYTES of
    partials fail with PA_ERR_WORKSPACE."""
    _enforce_contract(block_table, seq_lens, k_pool)
    _check_device_tensors(q=q, k_pool=k_pool, v_pool=v_pool, block_table=block_table,
                          seq_lens=seq_lens, out=out)
    for name, t in (("q", q), ("k_pool", k_pool), ("v_pool", v_pool), ("out", out)):
        _require(t.dtype == torch.bfloat16, f"{name} must be bfloat16")
    _require(out.shape == q.shape, "out must have q's shape")
    _require(block_table.dtype == torch.int32 and seq_lens.dtype == torch.int32,
             "block_table and seq_lens must be int32")
    _require(k_pool.dim() == 4 and v_pool.shape == k_pool.shape, "k_pool/v_pool: [P, ps, Hkv, d]")
    _require(q.dim() == 3 and q.shape[2] == k_pool.shape[3], "q: [batch, Hq, d]")
    _require(seq_lens.numel() == q.shape[0] and block_table.shape[0] >= q.shape[0],
             "seq_lens: [batch]; block_table: [batch, maxp]")
    lay = layout_of(k_pool, block_table)
    _check(load_library().pa_decode_noalloc(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(seq_lens), float(scale),
        _ptr(out), q.shape[0], q.shape[1], ctypes.byref(lay), _stream(stream)))
    return out


def pa_decode_partial(q, k_pool, v_pool, block_table, seq_lens, scale, workspace, stream=None):
    _decode_checks(q, k_pool, v_pool, block_table, seq_lens, workspace)
    lay = layout_of(k_pool, block_table)
    st = load_library().pa_decode_partial(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(seq_lens), float(scale),
        q.shape[0], q.shape[1], _ptr(workspace), workspace.numel() * workspace.element_size(),
        ctypes.byref(lay), _stream(stream))
    _check(st)


def pa_decode_combine(seq_lens, out, workspace, layout: KVLayout, stream=None):
    _check_device_tensors(seq_lens=seq_lens, out=out, workspace=workspace)
    _require(out.dtype == torch.bfloat16 and out.dim() == 3, "out: bf16 [batch, Hq, d]")
    st = load_library().pa_decode_combine(
        _ptr(seq_lens), _ptr(out), out.shape[0], out.shape[1], _ptr(workspace),
        workspace.numel() * workspace.element_size(), ctypes.byref(layout), _stream(stream))
    _check(st)


def pa_kv_append(k_new, v_new, seq_ids, positions, k_pool, v_pool, block_table, stream=None):
    """Writes the K/V rows of new tokens into their pages (in place); token i goes to
    block_table[seq_ids[i], positions[i] // page_size], slot positions[i] % page_size."""
    _check_device_tensors(k_new=k_new, v_new=v_new, seq_ids=seq_ids, positions=positions,
                          k_pool=k_pool, v_pool=v_pool, block_table=block_table)
    for name, t in (("k_new", k_new), ("v_new", v_new), ("k_pool", k_pool), ("v_pool", v_pool)):
        _require(t.dtype == torch.bfloat16, f"{name} must be bfloat16")
    for name, t in (("seq_ids", seq_ids), ("positions", positions), ("block_table", block_table)):
        _require(t.dtype == torch.int32, f"{name} must be int32")
    _require(k_pool.dim() == 4 and v_pool.shape == k_pool.shape, "k_pool/v_pool: [P, ps, Hkv, d]")
    n = k_new.shape[0]
    _require(k_new.shape == (n,) + tuple(k_pool.shape[2:]) and v_new.shape == k_new.shape,
             "k_new/v_new: [num_tokens, Hkv, d]")
    _require(seq_ids.numel() == n and positions.numel() == n, "seq_ids/positions: [num_tokens]")
    _require(block_table.dim() == 2, "block_table: [num_seqs, maxp]")
    lay = layout_of(k_pool, block_table)
    _check(load_library().pa_kv_append(
        _ptr(k_new), _ptr(v_new), _ptr(seq_ids), _ptr(positions), n, _ptr(k_pool),
        _ptr(v_pool), _ptr(block_table), block_table.shape[0], ctypes.byref(lay),
        _stream(stream)))


def pa_copy_pages(k_pool, v_pool, src_pages, dst_pages, stream=None):
    """Copies page src_pages[i] to page dst_pages[i] in both pools (in place)."""
    _check_device_tensors(k_pool=k_pool, v_pool=v_pool, src_pages=src_pages,
                          dst_pages=dst_pages)
    _require(k_pool.dtype == torch.bfloat16 and v_pool.dtype == torch.bfloat16,
             "pools must be bfloat16")
    _require(k_pool.dim() == 4 and v_pool.shape == k_pool.shape, "k_pool/v_pool: [P, ps, Hkv, d]")
    _require(src_pages.dtype == torch.int32 and dst_pages.dtype == torch.int32,
             "src_pages/dst_pages must be int32")
    _require(src_pages.numel() == dst_pages.numel(), "src_pages and dst_pages differ in length")
    P, ps, hkv, d = k_pool.shape
    lay = make_layout(P, ps, hkv, d, 1)
    _check(load_library().pa_copy_pages(_ptr(k_pool), _ptr(v_pool), _ptr(src_pages),
                                        _ptr(dst_pages), src_pages.numel(), ctypes.byref(lay),
                                        _stream(stream)))


class BlockManager:
    """Host-side page manager of the library (pa_bm_* in pagedattn.h): block tables,
    on-demand pages, reference counts and copy-on-write prefix sharing.  Touches no
    device memory; the caller uploads the exported table and runs the page copies."""

    def __init__(self, num_pages: int, page_size: int, max_seqs: int, max_pages_per_seq: int):
        self._lib = load_library()
        h = ctypes.c_void_p()
        _check(self._lib.pa_bm_create(int(num_pages), int(page_size), int(max_seqs),
                                      int(max_pages_per_seq), ctypes.byref(h)))
        self._h = h
        self.num_pages = int(num_pages)
        self.page_size = int(page_size)
        self.max_seqs = int(max_seqs)
        self.max_pages_per_seq = int(max_pages_per_seq)

    def close(self):
        if self._h:
            self._lib.pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add_sequence(self) -> int:
        s = ctypes.c_int32()
        _check(self._lib.pa_bm_add_sequence(self._h, ctypes.byref(s)))
        return s.value

    def fork(self, parent: int, num_tokens: int) -> int:
        c = ctypes.c_int32()
        _check(self._lib.pa_bm_fork(self._h, int(parent), int(num_tokens), ctypes.byref(c)))
        return c.value

    def free_sequence(self, seq: int):
        _check(self._lib.pa_bm_free_sequence(self._h, int(seq)))

    def append(self, seq: int, num_tokens: int):
        """Reserves num_tokens more tokens; returns the [(src, dst)] page copies to run."""
        src, dst, n = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check(self._lib.pa_bm_append(self._h, int(seq), int(num_tokens), ctypes.byref(src),
                                      ctypes.byref(dst), ctypes.byref(n)))
        return [(src.value, dst.value)] if n.value else []

    def seq_len(self, seq: int) -> int:
        return int(self._lib.pa_bm_seq_len(self._h, int(seq)))

    def free_page_count(self) -> int:
        return int(self._lib.pa_bm_free_page_count(self._h))

    def ref_count(self, page: int) -> int:
        return int(self._lib.pa_bm_ref_count(self._h, int(page)))

    def export(self):
        """(block_table int32 [max_seqs, max_pages_per_seq], seq_lens int32 [max_seqs])."""
        import numpy as np
        table = np.empty((self.max_seqs, self.max_pages_per_seq), dtype=np.int32)
        lens = np.empty(self.max_seqs, dtype=np.int32)
        _check(self._lib.pa_bm_export(self._h, table.ctypes.data, lens.ctypes.data))
        return table, lens

    def validate(self):
        _check(self._lib.pa_bm_validate(self._h))
