"""Seeded generators for the indexer workloads.

Layout of the paged index cache (one reading of the pages, kept identical on
both sides of the parity tests):

* The cache is ``uint8[num_pages, page_bytes]``; page ``p`` holds
  ``page_size`` (64) token rows back to back, token ``slot`` at byte
  ``slot * row_bytes`` (token-major rows, as in the 3-D
  ``(num_blocks, block_size, head_size)`` cache shape of the vLLM
  DeepSeek-V3.2 indexer backend, ``get_kv_cache_shape``).
* FP8 row: ``head_dim`` e4m3fn codes, then the fp32 per-token scale in 4
  little-endian bytes (the "128 fp8 bytes and 4 scale bytes" entry noted in
  ``get_max_prefill_buffer_size`` of that page).
* MXFP4 row: ``head_dim/2`` bytes of packed e2m1 (element ``2j`` in the low
  nibble of byte ``j``), then ``head_dim/32`` ue8m0 block scales (the
  ``head_dim // 2 + head_dim // MXFP4_BLOCK_SIZE`` width of
  ``kv_cache_as_quant_view`` on the glm5next sparse_indexer page).

Key values are drawn N(0,1) and quantised here, once, when the inputs are
made; the method itself only ever reads the quantised bytes.  Slots and
pages that no request references are filled with 0xFF bytes ("poison": NaN
codes / NaN scales) so that a read outside a request's live keys shows up as
NaN in a checked output.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

PAGE_SIZE = 64
FP8_MAX = 448.0
POISON = 0xFF


def row_bytes_for(fmt: str, head_dim: int) -> int:
    """Bytes of one token row in the paged cache."""
    if fmt == "fp8":
        return head_dim + 4
    if fmt == "mxfp4":
        return head_dim // 2 + head_dim // 32
    raise ValueError(fmt)


# ----------------------------------------------------------------------------
# Encoders (input production only)
# ----------------------------------------------------------------------------

def encode_fp8_rows(k: np.ndarray) -> np.ndarray:
    """fp32 keys [n, D] -> token rows [n, D+4]: e4m3fn codes at scale amax/448.

    The code conversion is torch's float -> float8_e4m3fn cast (round to
    nearest even) after clamping to the finite range.
    """
    k = np.ascontiguousarray(k, dtype=np.float32)
    n, d = k.shape
    amax = np.abs(k).max(axis=1)
    scale = np.where(amax > 0, amax / np.float32(FP8_MAX), np.float32(1.0)).astype(np.float32)
    x = np.clip(k / scale[:, None], -FP8_MAX, FP8_MAX).astype(np.float32)
    codes = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    out = np.empty((n, d + 4), dtype=np.uint8)
    out[:, :d] = codes
    out[:, d:] = scale.astype("<f4").view(np.uint8).reshape(n, 4)
    return out


_E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def _e2m1_code(mag: np.ndarray) -> np.ndarray:
    """Magnitudes (already divided by the block scale) -> 3-bit e2m1 codes,
    round to nearest, ties to the even code, saturating at 6.

    The grid is 0, .5, 1, 1.5, 2, 3, 4, 6 (codes 0..7).  The code is the
    number of midpoints below the magnitude; a magnitude exactly on the
    midpoint between codes i and i+1 rounds up only when i+1 is even."""
    mag = np.minimum(mag, 6.0)
    mids = ((_E2M1_GRID[:-1] + _E2M1_GRID[1:]) * 0.5).astype(mag.dtype)
    code = np.zeros(mag.shape, dtype=np.uint8)
    for i, m in enumerate(mids):
        up = (mag >= m) if (i + 1) % 2 == 0 else (mag > m)
        code += up.view(np.uint8)
    return code


def encode_mxfp4_rows(k: np.ndarray) -> np.ndarray:
    """fp32 keys [n, D] -> token rows [n, D/2 + D/32] in the OCP MX FP4 form:
    per 32-element block a shared power-of-two scale 2^(floor(log2 amax) - 2),
    elements rounded to e2m1 (nearest, ties to even, saturating).  (Bulk
    arithmetic on torch CPU tensors; every step is exact in fp32.)"""
    k = np.ascontiguousarray(k, dtype=np.float32)
    n, d = k.shape
    assert d % 32 == 0
    nb = d // 32
    blocks = torch.from_numpy(k).view(n, nb, 32)
    amax = blocks.abs().amax(dim=2)
    # floor(log2 amax) from the binary exponent (frexp: amax = m 2^ex, m in [.5, 1))
    _, ex = torch.frexp(amax)
    e = torch.where(amax > 0, ex.to(torch.int32) - 3, torch.full_like(ex, -127, dtype=torch.int32))
    e = e.clamp(-127, 127)
    scaled = blocks * torch.ldexp(torch.ones_like(amax), -e).unsqueeze(-1)   # exact: power of two
    mag = scaled.abs().clamp(max=6.0)
    code = torch.zeros(mag.shape, dtype=torch.uint8)
    for i, m in enumerate(((_E2M1_GRID[:-1] + _E2M1_GRID[1:]) * 0.5).tolist()):
        # midpoint between codes i and i+1: ties go up only to an even code
        code += (mag >= m) if (i + 1) % 2 == 0 else (mag > m)
    sign = (scaled < 0) & (code > 0)
    nib = (code | (sign.to(torch.uint8) << 3)).view(n, d)
    packed = nib[:, 0::2] | (nib[:, 1::2] << 4)
    out = np.empty((n, d // 2 + nb), dtype=np.uint8)
    out[:, : d // 2] = packed.numpy()
    out[:, d // 2 :] = (e + 127).to(torch.uint8).numpy()
    return out


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (torch's round-to-nearest-even cast), returned as uint16 bits."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


# ----------------------------------------------------------------------------
# Workload container
# ----------------------------------------------------------------------------

@dataclass
class Workload:
    name: str
    kind: str                     # "decode" | "prefill"
    fmt: str                      # "fp8" | "mxfp4"
    heads: int
    head_dim: int
    topk: int
    page_size: int
    page_bytes: int
    cache: np.ndarray             # uint8 [num_pages, page_bytes]
    block_table: np.ndarray       # int32 [num_req, width]
    seq_lens: np.ndarray          # int32 [num_req]
    q: np.ndarray                 # uint16 (bf16 bits) [rows, H, D]
    w: np.ndarray                 # float32 [rows, H]
    next_n: int = 1
    decode_lens: np.ndarray | None = None   # int32 [num_req], decode only
    q_packed: bool = False        # decode: q/w rows are packed tokens, not the grid
    query_lens: np.ndarray | None = None    # int32 [num_req], prefill only
    compress_ratio: int = 1       # keys stored per request: seq_lens // compress_ratio
    meta: dict = field(default_factory=dict)

    @property
    def num_req(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def num_pages(self) -> int:
        return int(self.cache.shape[0])

    @property
    def row_bytes(self) -> int:
        return row_bytes_for(self.fmt, self.head_dim)

    @property
    def grid_rows(self) -> int:
        """Output rows: the padded [num_req, next_n] grid (decode) or every
        query token (prefill)."""
        if self.kind == "decode":
            return self.num_req * self.next_n
        return int(self.query_lens.sum())


def _fill_cache(rng, fmt, head_dim, num_pages, page_bytes, block_table, seq_lens,
                chunk_keys=1 << 18, page_size=PAGE_SIZE):
    """Allocate the poisoned pool and write quantised N(0,1) keys into every
    referenced slot (key t of request b -> page block_table[b, t//page_size],
    slot t % page_size; seq_lens here are the stored key counts).  Keys are
    drawn request by request, token order."""
    PAGE_SIZE = page_size  # noqa: N806 (the loop below is written for any page size)
    rb = row_bytes_for(fmt, head_dim)
    cache = np.full((num_pages, page_bytes), POISON, dtype=np.uint8)
    enc = encode_fp8_rows if fmt == "fp8" else encode_mxfp4_rows
    assert chunk_keys % PAGE_SIZE == 0
    for b in range(len(seq_lens)):
        L = int(seq_lens[b])
        t0 = 0
        while t0 < L:
            t1 = min(L, t0 + chunk_keys)
            rows = enc(rng.standard_normal((t1 - t0, head_dim), dtype=np.float32))
            nfull = (t1 - t0) // PAGE_SIZE
            if nfull:
                pages = block_table[b, t0 // PAGE_SIZE : t0 // PAGE_SIZE + nfull]
                cache[pages, : PAGE_SIZE * rb] = rows[: nfull * PAGE_SIZE].reshape(nfull, PAGE_SIZE * rb)
            rest = (t1 - t0) - nfull * PAGE_SIZE
            if rest:
                page = block_table[b, t0 // PAGE_SIZE + nfull]
                cache[page, : rest * rb] = rows[nfull * PAGE_SIZE :].reshape(-1)
            t0 = t1
    return cache


def _deal_pages(rng, seq_lens, num_pages, width, page_size=PAGE_SIZE):
    """Disjoint random pages for every request, dealt from one permutation of
    the pool; unused table entries are 0 (as the pages' zero-filled tables)."""
    need = [-(-int(L) // page_size) for L in seq_lens]
    if sum(need) > num_pages:
        raise ValueError("pool too small")
    perm = rng.permutation(num_pages).astype(np.int32)
    bt = np.zeros((len(seq_lens), width), dtype=np.int32)
    pos = 0
    for b, n in enumerate(need):
        bt[b, :n] = perm[pos : pos + n]
        pos += n
    return bt


def build_decode(*, seed: int, seq_lens, heads: int, head_dim: int, topk: int,
                 fmt: str = "fp8", next_n: int = 1, decode_lens=None,
                 num_pages: int | None = None, pool_slack: float = 0.10,
                 width: int | None = None, w_std: float | None = None,
                 q_packed: bool = False, block_table=None, name: str = "decode",
                 page_bytes: int | None = None, page_size: int = PAGE_SIZE,
                 compress_ratio: int = 1) -> Workload:
    """A decode batch: ``num_req`` requests, the padded [num_req, next_n] grid of
    query rows.  With compress_ratio r, request b stores seq_lens[b] // r keys
    (a compressed index cache).  Draw order after the lengths: block table,
    keys, q, w."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return _build_decode_rng(rng, seq_lens=seq_lens, heads=heads, head_dim=head_dim,
                             topk=topk, fmt=fmt, next_n=next_n, decode_lens=decode_lens,
                             num_pages=num_pages, pool_slack=pool_slack, width=width,
                             w_std=w_std, q_packed=q_packed, block_table=block_table,
                             name=name, page_bytes=page_bytes, page_size=page_size,
                             compress_ratio=compress_ratio)


def _build_decode_rng(rng, *, seq_lens, heads, head_dim, topk, fmt, next_n, decode_lens,
                      num_pages, pool_slack, width, w_std, q_packed, block_table, name,
                      page_bytes, page_size=PAGE_SIZE, compress_ratio=1):
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    B = len(seq_lens)
    if decode_lens is not None:
        decode_lens = np.asarray(decode_lens, dtype=np.int32)
    stored = seq_lens // compress_ratio
    rb = row_bytes_for(fmt, head_dim)
    pb = page_bytes if page_bytes is not None else page_size * rb
    need_pages = sum(-(-int(L) // page_size) for L in stored)
    if num_pages is None:
        num_pages = max(1, int(math.ceil(need_pages * (1.0 + pool_slack))))
    if width is None:
        width = max(1, -(-int(stored.max(initial=1)) // page_size))
    if block_table is None:
        block_table = _deal_pages(rng, stored, num_pages, width, page_size)
    else:
        block_table = np.array(block_table, dtype=np.int32, order="C", copy=True)
    cache = _fill_cache(rng, fmt, head_dim, num_pages, pb, block_table, stored, page_size=page_size)
    if q_packed:
        rows = int(decode_lens.sum()) if decode_lens is not None else B * next_n
    else:
        rows = B * next_n
    q32 = rng.standard_normal((rows, heads, head_dim), dtype=np.float32)
    q = _bf16_bits(q32)
    if w_std is None:
        w_std = 1.0 / math.sqrt(heads)
    w = (rng.standard_normal((rows, heads), dtype=np.float32) * np.float32(w_std)).astype(np.float32)
    return Workload(name=name, kind="decode", fmt=fmt, heads=heads, head_dim=head_dim,
                    topk=topk, page_size=page_size, page_bytes=pb, cache=cache,
                    block_table=block_table, seq_lens=seq_lens, q=q, w=w, next_n=next_n,
                    decode_lens=decode_lens, q_packed=q_packed, compress_ratio=compress_ratio)


def build_prefill(*, seed: int, seq_lens, query_lens, heads: int, head_dim: int,
                  topk: int, fmt: str = "fp8", pool_slack: float = 0.10,
                  w_std: float | None = None, name: str = "prefill", page_size: int = PAGE_SIZE,
                  compress_ratio: int = 1) -> Workload:
    """Prefill requests: request b has query_lens[b] query tokens, the last
    ones of its seq_lens[b] tokens (seq_lens[b] // compress_ratio stored
    keys).  q/w rows are every query token in order."""
    rng = np.random.Generator(np.random.PCG64(seed))
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    query_lens = np.asarray(query_lens, dtype=np.int32)
    stored = seq_lens // compress_ratio
    rb = row_bytes_for(fmt, head_dim)
    pb = page_size * rb
    need_pages = sum(-(-int(L) // page_size) for L in stored)
    num_pages = max(1, int(math.ceil(need_pages * (1.0 + pool_slack))))
    width = max(1, -(-int(stored.max(initial=1)) // page_size))
    bt = _deal_pages(rng, stored, num_pages, width, page_size)
    cache = _fill_cache(rng, fmt, head_dim, num_pages, pb, bt, stored, page_size=page_size)
    rows = int(query_lens.sum())
    q = _bf16_bits(rng.standard_normal((rows, heads, head_dim), dtype=np.float32))
    if w_std is None:
        w_std = 1.0 / math.sqrt(heads)
    w = (rng.standard_normal((rows, heads), dtype=np.float32) * np.float32(w_std)).astype(np.float32)
    return Workload(name=name, kind="prefill", fmt=fmt, heads=heads, head_dim=head_dim,
                    topk=topk, page_size=page_size, page_bytes=pb, cache=cache,
                    block_table=bt, seq_lens=seq_lens, q=q, w=w, query_lens=query_lens,
                    compress_ratio=compress_ratio)


# ----------------------------------------------------------------------------
# The five named workloads
# ----------------------------------------------------------------------------

CONFIG_NAMES = ("C1", "C2", "C3", "C4", "C5")


def config(name: str) -> Workload:
    """The five synthetic workloads, seeds 0..4.

    C1 tiny decode: 1 request, L=300, 8-page pool whose block table is a
       random permutation of the 8 pages; H=4, D=32, k=64.
    C2 fp8 decode batch: 32 requests, L ~ U[4096, 32768], 20,000-page pool,
       H=64, D=128, k=2048, w ~ N(0,1)/8.
    C3 MTP non-uniform decode: 128 requests, decode_lens in {1,2} (p=1/2),
       next_n=2 padded grid, L = floor(exp(U(ln 512, ln 131072))).
    C4 MXFP4 long-context decode: 64 requests x L=131072, H=64, D=128, k=2048.
    C5 chunked prefill: 2 requests, query 16384 of seq 65536 each.
    V4 (beyond the five) compressed fp8 decode: 64 requests x 131072 tokens at
       compress ratio 4, 256-token pages, H=64, D=128, k=2048, seed 5.
    """
    if name == "C1":
        rng = np.random.Generator(np.random.PCG64(0))
        seq = np.array([300], dtype=np.int32)
        perm = rng.permutation(8).astype(np.int32).reshape(1, 8).copy()
        wl = _build_decode_rng(rng, seq_lens=seq, heads=4, head_dim=32, topk=64, fmt="fp8",
                               next_n=1, decode_lens=None, num_pages=8, pool_slack=0.0,
                               width=8, w_std=0.5, q_packed=False, block_table=perm,
                               name="C1", page_bytes=None)
        return wl
    if name == "C2":
        rng = np.random.Generator(np.random.PCG64(1))
        seq = rng.integers(4096, 32768, size=32, endpoint=True).astype(np.int32)
        return _build_decode_rng(rng, seq_lens=seq, heads=64, head_dim=128, topk=2048, fmt="fp8",
                                 next_n=1, decode_lens=None, num_pages=20000, pool_slack=0.0,
                                 width=512, w_std=1.0 / 8, q_packed=False, block_table=None,
                                 name="C2", page_bytes=None)
    if name == "C3":
        rng = np.random.Generator(np.random.PCG64(2))
        dl = rng.integers(1, 2, size=128, endpoint=True).astype(np.int32)
        seq = np.floor(np.exp(rng.uniform(math.log(512), math.log(131072), size=128))).astype(np.int32)
        return _build_decode_rng(rng, seq_lens=seq, heads=64, head_dim=128, topk=2048, fmt="fp8",
                                 next_n=2, decode_lens=dl, num_pages=None, pool_slack=0.10,
                                 width=2048, w_std=1.0 / 8, q_packed=False, block_table=None,
                                 name="C3", page_bytes=None)
    if name == "C4":
        rng = np.random.Generator(np.random.PCG64(3))
        seq = np.full(64, 131072, dtype=np.int32)
        return _build_decode_rng(rng, seq_lens=seq, heads=64, head_dim=128, topk=2048,
                                 fmt="mxfp4", next_n=1, decode_lens=None, num_pages=None,
                                 pool_slack=0.10, width=2048, w_std=1.0 / 8, q_packed=False,
                                 block_table=None, name="C4", page_bytes=None)
    if name == "C5":
        return build_prefill(seed=4, seq_lens=[65536, 65536], query_lens=[16384, 16384],
                             heads=64, head_dim=128, topk=2048, fmt="fp8", w_std=1.0 / 8,
                             name="C5")
    if name == "V4":
        # compressed index cache: C4's lengths at compress ratio 4 in fp8,
        # 256-token pages (32768 keys per request)
        rng = np.random.Generator(np.random.PCG64(5))
        seq = np.full(64, 131072, dtype=np.int32)
        return _build_decode_rng(rng, seq_lens=seq, heads=64, head_dim=128, topk=2048,
                                 fmt="fp8", next_n=1, decode_lens=None, num_pages=None,
                                 pool_slack=0.10, width=128, w_std=1.0 / 8, q_packed=False,
                                 block_table=None, name="V4", page_bytes=None, page_size=256,
                                 compress_ratio=4)
    raise KeyError(name)


# ----------------------------------------------------------------------------
# Cache-write inputs
# ----------------------------------------------------------------------------

@dataclass
class CacheWriteInputs:
    fmt: str
    head_dim: int
    k_bits: np.ndarray        # uint16 bf16 [T, k_stride] (first head_dim used)
    slots: np.ndarray         # int64 [T]
    num_pages: int
    page_bytes: int
    cache: np.ndarray         # uint8 [num_pages, page_bytes], the cache before the write
    page_size: int = PAGE_SIZE


def cache_write_inputs(*, seed: int, tokens: int, head_dim: int, fmt: str, num_pages: int,
                       k_stride: int | None = None, skip_frac: float = 0.05,
                       special_rows: bool = True, page_size: int = PAGE_SIZE) -> CacheWriteInputs:
    """New key tokens for an index-cache write: bf16 keys N(0,1) times a
    per-token power of two in [2^-20, 2^20], distinct random slots of the
    pool (a fraction set to -1, i.e. not stored) and a poisoned pool.  With
    `special_rows`, the first rows are edge cases: all zeros, signed zeros,
    a lone value, constant rows, values exactly halfway between fp8 / fp4
    codes after scaling, and bf16 subnormals next to a large absmax."""
    rng = np.random.default_rng(seed)
    D = head_dim
    stride = k_stride or D
    k = rng.standard_normal((tokens, D)).astype(np.float32) * np.exp2(rng.integers(-20, 21, (tokens, 1)))
    if special_rows:
        e4m3_ties = np.array([1.0625, 1.1875, 2.125, 3.25, 0.0029296875, 0.0087890625, 14.5, 416.0,
                              -1.0625, -2.125, -0.0029296875, -416.0], dtype=np.float32)   # halfway between codes
        fp4_ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, -0.25, -0.75, -2.5, -5.0], dtype=np.float32)
        specials = []
        specials.append(np.zeros(D, np.float32))
        z = np.zeros(D, np.float32)
        z[1::2] = -0.0
        specials.append(z)
        lone = np.zeros(D, np.float32)
        lone[D // 2] = -3.0
        specials.append(lone)
        specials.append(np.full(D, 2.0, np.float32))
        row = np.zeros(D, np.float32)
        row[0] = 448.0                                  # fp8 scale exactly 1
        row[1 : 1 + len(e4m3_ties)] = e4m3_ties
        specials.append(row)
        row = np.zeros(D, np.float32)
        for b in range(D // 32):                        # every block: amax 7 -> block exponent 0
            row[32 * b] = 7.0
            row[32 * b + 1 : 32 * b + 1 + len(fp4_ties)] = fp4_ties
        specials.append(row)
        row = np.zeros(D, np.float32)
        row[0] = 1024.0
        row[1:5] = [2.0 ** -133, -(2.0 ** -133), 2.0 ** -126, -(2.0 ** -130)]
        specials.append(row)
        n = min(len(specials), tokens)
        k[:n] = np.stack(specials[:n])
    bits = np.zeros((tokens, stride), dtype=np.uint16)
    bits[:, :D] = _bf16_bits(k)
    rb = row_bytes_for(fmt, D)
    page_bytes = (page_size * rb + 15) // 16 * 16
    cap = num_pages * page_size
    assert tokens <= cap
    slots = rng.permutation(cap)[:tokens].astype(np.int64)
    slots[rng.random(tokens) < skip_frac] = -1
    cache = np.full((num_pages, page_bytes), 0x5A, dtype=np.uint8)
    return CacheWriteInputs(fmt, D, bits, slots, num_pages, page_bytes, cache, page_size)
