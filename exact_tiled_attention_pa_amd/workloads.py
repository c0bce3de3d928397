"""Seeded synthetic inputs for paged attention.

This module only draws random numbers and lays pages out: sequence lengths,
the physical page assignment (block tables), and bf16 normal Q / K-pool /
V-pool contents.  It holds none of the attention arithmetic.  The parity tests
feed the same tensors to the HIP library and (copied to the host) to the CPU
oracle; the bench times the library on them.

Workload shapes (one GPU each):

  prefill_600      causal paged prefill, 1 sequence, 1 head, d=64, 600 tokens,
                   256-token pages, pool of 12 pages, block table [5, 1, 9]
                   (the page-size and table of "What is Paged FlashAttention?",
                   section "Practical example"), N(0, 1), scale 1/8
  decode_64        decode, 64 sequences x 1 query token, 32 heads, d=128,
                   lengths uniform on {512..8192}, 16-token pages, pool sized
                   exactly to the total context, pages a random permutation
  decode_64_gqa8   decode_64's lengths and page layout with grouped heads: 64
                   query heads over 8 K/V heads (8 query heads per K/V head)
  prefill_4096     prefill, 1 sequence, 32 heads, d=128, N=4096, identity table,
                   256-token pages; causal and non-causal variants
  prefill_32k      causal paged prefill, 1 sequence, 8 heads, d=128, N=32768,
                   256-token pages, shuffled pages, N(0, 0.5^2)
  mixed_128x4      128 decode sequences with lognormal lengths (median 4096,
                   sigma 1, clipped to [1024, 32768]) plus 4 causal prefill
                   chunks of 2048 tokens on top of 8192 cached tokens, 32 heads,
                   d=128, 16-token pages drawn without replacement from a pool
                   1.25x the pages needed (the rest are holes)

Draw order for a seed: lengths -> page assignment (both on a CPU generator, so
block tables do not depend on the device) -> Q -> K pool -> V pool (on a
generator of the target device).  Values are fp32 normals times sigma rounded
to bf16 (round to nearest even).  With poison=True every pool slot that no
sequence reads (tail slots of last pages, unused pages) holds bf16 NaN; table
entries past a sequence's last page are -1.
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

NAN_BF16 = 0x7FC0


@dataclass
class AttnCall:
    """One library call over the shared pools: a prefill or a decode batch."""
    kind: str                      # "prefill" | "decode"
    q: torch.Tensor                # bf16 [total_q, H, d] (prefill) or [batch, H, d] (decode)
    block_table: torch.Tensor      # int32 [batch, max_pages_per_seq] on the pool's device
    seq_lens: torch.Tensor         # int32 [batch] on the pool's device
    q_start: Optional[torch.Tensor]  # int32 [batch+1] (prefill only)
    max_q_len: int
    causal: bool
    # host copies for the oracle and for host-side sizing
    block_table_host: np.ndarray = None
    seq_lens_host: np.ndarray = None
    q_start_host: Optional[np.ndarray] = None

    @property
    def batch(self) -> int:
        return int(self.seq_lens_host.shape[0])


@dataclass
class Workload:
    name: str
    heads: int                     # K/V heads stored in the pools
    head_dim: int
    page_size: int
    num_pages: int
    max_pages_per_seq: int
    scale: float
    sigma: float
    k_pool: torch.Tensor           # bf16 [num_pages, page_size, H, d]
    v_pool: torch.Tensor
    calls: List[AttnCall] = field(default_factory=list)
    description: str = ""
    q_heads: int = 0               # query heads (0: same as heads)

    @property
    def num_q_heads(self) -> int:
        return self.q_heads or self.heads

    def digest(self) -> str:
        """SHA-256 over every input buffer (host copies, streamed in 128 MiB pieces),
        for the record: K pool, V pool, then each call's queries, block table, lengths
        and chunk offsets."""
        h = hashlib.sha256()
        for t in [self.k_pool, self.v_pool] + [c.q for c in self.calls]:
            flat = t.detach().contiguous().view(-1).view(torch.int16)
            step = 1 << 26
            for s in range(0, flat.numel(), step):
                h.update(flat[s:s + step].cpu().numpy().tobytes())
        for c in self.calls:
            h.update(c.block_table_host.tobytes())
            h.update(c.seq_lens_host.tobytes())
            if c.q_start_host is not None:
                h.update(c.q_start_host.tobytes())
        return h.hexdigest()


def _normal_bf16(shape, sigma, gen, device, chunk=1 << 26):
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    n = flat.numel()
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        x = torch.randn(e - s, generator=gen, device=device, dtype=torch.float32)
        if sigma != 1.0:
            x.mul_(sigma)
        flat[s:e] = x.to(torch.bfloat16)
    return out


def normal_bf16(shape, sigma: float, seed: int, device) -> torch.Tensor:
    """bf16 N(0, sigma^2) tensor from its own seeded generator on `device` (new K/V
    rows for cache appends, fresh pools)."""
    gen = torch.Generator(device=device).manual_seed(int(seed))
    return _normal_bf16(tuple(shape), sigma, gen, device)


def _pages_of(length: int, page_size: int) -> int:
    return -(-int(length) // int(page_size))


def _table_from_order(lens, page_size, order, max_pages):
    """Assigns physical pages to sequences in sequence order from `order`."""
    table = np.full((len(lens), max_pages), -1, dtype=np.int32)
    cursor = 0
    for b, L in enumerate(lens):
        n = _pages_of(L, page_size)
        table[b, :n] = order[cursor:cursor + n]
        cursor += n
    return table


def _poison(pool: torch.Tensor, tables, lens_list, page_size):
    """Writes NaN into every slot that no (table, length) pair reads."""
    num_pages = pool.shape[0]
    used = np.zeros((num_pages, page_size), dtype=bool)
    for table, lens in zip(tables, lens_list):
        for b, L in enumerate(lens):
            n = _pages_of(L, page_size)
            if n == 0:  # an empty sequence reads nothing
                continue
            pages = table[b, :n]
            used[pages[:-1], :] = True
            used[pages[-1], :int(L) - (n - 1) * page_size] = True
    bad = torch.from_numpy(~used).to(pool.device)
    view = pool.view(torch.int16)
    for p0 in range(0, num_pages, 4096):
        p1 = min(num_pages, p0 + 4096)
        m = bad[p0:p1]
        if bool(m.any()):
            chunk = view[p0:p1]
            chunk[m] = NAN_BF16
    return pool


def _make_call(kind, q, table, lens, q_lens, causal, device):
    lens = np.asarray(lens, dtype=np.int32)
    q_start_host = None
    q_start = None
    max_q_len = 1
    if kind == "prefill":
        q_start_host = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
        q_start = torch.from_numpy(q_start_host).to(device)
        max_q_len = int(max(q_lens)) if len(q_lens) else 0
    return AttnCall(kind=kind, q=q, block_table=torch.from_numpy(table).to(device),
                    seq_lens=torch.from_numpy(lens).to(device), q_start=q_start,
                    max_q_len=max_q_len, causal=causal, block_table_host=table,
                    seq_lens_host=lens, q_start_host=q_start_host)


def build(name: str, seed: int, heads: int, head_dim: int, page_size: int,
          lens, q_lens=None, causal=True, kind="prefill", sigma=1.0, pool_pages=None,
          table=None, shuffle=True, pool_slack=1.0, device="cpu", poison=False,
          scale=None, description="", tensors=True, q_heads=None) -> Workload:
    """Generic builder: one call over one pool.

    lens     KV length per sequence (L_b)
    q_lens   query rows per sequence (prefill); decode uses one per sequence
    table    explicit block table rows (list of lists) instead of a drawn one
    shuffle  draw the page assignment from a random permutation (else identity order)
    tensors  False: lay out lengths and tables only (q and pools are left None)
    q_heads  query heads (a multiple of heads, the K/V heads); default heads
    """
    cpu_gen = torch.Generator(device="cpu").manual_seed(seed)
    lens = [int(x) for x in lens]
    batch = len(lens)
    needed = sum(_pages_of(L, page_size) for L in lens)
    if table is not None:
        max_pages = max(len(r) for r in table)
        tbl = np.full((batch, max_pages), -1, dtype=np.int32)
        for b, row in enumerate(table):
            tbl[b, :len(row)] = row
        num_pages = pool_pages if pool_pages is not None else int(tbl.max()) + 1
    else:
        num_pages = pool_pages if pool_pages is not None else int(math.ceil(needed * pool_slack))
        max_pages = max(_pages_of(L, page_size) for L in lens)
        if shuffle:
            order = torch.randperm(num_pages, generator=cpu_gen).numpy()[:needed]
        else:
            order = np.arange(needed)
        tbl = _table_from_order(lens, page_size, order, max_pages)
    if kind == "prefill":
        q_lens = [int(x) for x in (q_lens if q_lens is not None else lens)]
    q = k_pool = v_pool = None
    if tensors:
        dev_gen = torch.Generator(device=device).manual_seed(seed)
        q_rows = sum(q_lens) if kind == "prefill" else batch
        q = _normal_bf16((q_rows, q_heads or heads, head_dim), sigma, dev_gen, device)
        k_pool = _normal_bf16((num_pages, page_size, heads, head_dim), sigma, dev_gen, device)
        v_pool = _normal_bf16((num_pages, page_size, heads, head_dim), sigma, dev_gen, device)
    if poison and tensors:
        _poison(k_pool, [tbl], [lens], page_size)
        _poison(v_pool, [tbl], [lens], page_size)
    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(head_dim)))
    call = _make_call(kind, q, tbl, lens, q_lens, causal if kind == "prefill" else False, device)
    return Workload(name=name, heads=heads, head_dim=head_dim, page_size=page_size,
                    num_pages=num_pages, max_pages_per_seq=tbl.shape[1], scale=scale,
                    sigma=sigma, k_pool=k_pool, v_pool=v_pool, calls=[call],
                    description=description, q_heads=int(q_heads or heads))


def prefill_600(device="cpu", poison=False, seed=1, tensors=True) -> Workload:
    return build("prefill_600", seed, heads=1, head_dim=64, page_size=256, lens=[600],
                 q_lens=[600], causal=True, table=[[5, 1, 9]], pool_pages=12,
                 device=device, poison=poison, tensors=tensors,
                 description="causal paged prefill, 600 tokens, d=64, pages of 256, table [5,1,9]")


def decode_64(device="cpu", poison=False, seed=2, tensors=True) -> Workload:
    g = torch.Generator(device="cpu").manual_seed(seed * 7919 + 1)
    lens = torch.randint(512, 8193, (64,), generator=g).tolist()
    return build("decode_64", seed, heads=32, head_dim=128, page_size=16, lens=lens,
                 kind="decode", shuffle=True, device=device, poison=poison, tensors=tensors,
                 description="decode, 64 seqs, 32 heads, d=128, L~U{512..8192}, pages of 16")


def decode_64_gqa8(device="cpu", poison=False, seed=2, tensors=True) -> Workload:
    """decode_64's lengths and pages with grouped heads: 64 query heads share 8 K/V heads."""
    g = torch.Generator(device="cpu").manual_seed(seed * 7919 + 1)
    lens = torch.randint(512, 8193, (64,), generator=g).tolist()
    return build("decode_64_gqa8", seed, heads=8, head_dim=128, page_size=16, lens=lens,
                 kind="decode", shuffle=True, device=device, poison=poison, tensors=tensors,
                 q_heads=64,
                 description="decode, 64 seqs, 64 query heads over 8 K/V heads, d=128, "
                             "L~U{512..8192}, pages of 16")


def prefill_4096(device="cpu", poison=False, causal=True, seed=3, tensors=True) -> Workload:
    return build("prefill_4096_" + ("causal" if causal else "noncausal"), seed, heads=32,
                 head_dim=128, page_size=256, lens=[4096], q_lens=[4096], causal=causal,
                 shuffle=False, device=device, poison=poison, tensors=tensors,
                 description="prefill N=4096, 32 heads, d=128, identity table, pages of 256")


def prefill_32k(device="cpu", poison=False, seed=4, tensors=True) -> Workload:
    return build("prefill_32k", seed, heads=8, head_dim=128, page_size=256, lens=[32768],
                 q_lens=[32768], causal=True, shuffle=True, sigma=0.5, device=device,
                 poison=poison, tensors=tensors,
                 description="causal paged prefill N=32768, 8 heads, d=128, shuffled pages of 256")


def mixed_lengths(seed=5):
    g = torch.Generator(device="cpu").manual_seed(seed * 7919 + 1)
    z = torch.randn(128, generator=g, dtype=torch.float64)
    lens = torch.exp(z * 1.0 + math.log(4096.0)).round().clamp(1024, 32768).to(torch.int64)
    return lens.tolist()


def mixed_128x4(device="cpu", poison=False, seed=5, tensors=True) -> Workload:
    """One pool shared by a decode call (128 sequences) and a prefill call (4 chunks)."""
    heads, d, ps = 32, 128, 16
    dec_lens = mixed_lengths(seed)
    pre_lens = [8192 + 2048] * 4
    pre_q = [2048] * 4
    lens = dec_lens + pre_lens
    cpu_gen = torch.Generator(device="cpu").manual_seed(seed)
    needed = sum(_pages_of(L, ps) for L in lens)
    num_pages = int(math.ceil(1.25 * needed))
    order = torch.randperm(num_pages, generator=cpu_gen).numpy()[:needed]
    max_pages = 32768 // ps
    tbl = _table_from_order(lens, ps, order, max_pages)
    q_dec = q_pre = k_pool = v_pool = None
    if tensors:
        dev_gen = torch.Generator(device=device).manual_seed(seed)
        q_dec = _normal_bf16((len(dec_lens), heads, d), 1.0, dev_gen, device)
        q_pre = _normal_bf16((sum(pre_q), heads, d), 1.0, dev_gen, device)
        k_pool = _normal_bf16((num_pages, ps, heads, d), 1.0, dev_gen, device)
        v_pool = _normal_bf16((num_pages, ps, heads, d), 1.0, dev_gen, device)
    if poison and tensors:
        _poison(k_pool, [tbl], [lens], ps)
        _poison(v_pool, [tbl], [lens], ps)
    nd = len(dec_lens)
    dec = _make_call("decode", q_dec, np.ascontiguousarray(tbl[:nd]), dec_lens, None, False, device)
    pre = _make_call("prefill", q_pre, np.ascontiguousarray(tbl[nd:]), pre_lens, pre_q, True,
                     device)
    return Workload(name="mixed_128x4", heads=heads, head_dim=d, page_size=ps,
                    num_pages=num_pages, max_pages_per_seq=max_pages,
                    scale=float(np.float32(1.0 / math.sqrt(d))), sigma=1.0, k_pool=k_pool,
                    v_pool=v_pool, calls=[dec, pre],
                    description="128 lognormal decode seqs + 4 causal chunks of 2048 on 8192 "
                                "cached tokens, 32 heads, d=128, pages of 16, 1.25x pool")


FULL_WORKLOADS = {
    "prefill_600": prefill_600,
    "decode_64": decode_64,
    "decode_64_gqa8": decode_64_gqa8,
    "prefill_4096_causal": lambda **kw: prefill_4096(causal=True, **kw),
    "prefill_4096_noncausal": lambda **kw: prefill_4096(causal=False, **kw),
    "prefill_32k": prefill_32k,
    "mixed_128x4": mixed_128x4,
}


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> host uint16 bit patterns (what the oracle consumes)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
