"""GPU parity of idx_cache_write against the CPU oracle, through the C ABI:
every byte of the pool after the write, bit-exact."""

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_indexer_decode_amd as idx
from workloads import cache_write_inputs

pytestmark = pytest.mark.gpu

CASES = [
    # fmt, head_dim, tokens, num_pages, k_stride[, page_size]
    ("fp8", 128, 3001, 60, None),
    ("fp8", 128, 517, 9, 136),
    ("fp8", 64, 2003, 40, None),
    ("fp8", 32, 1999, 40, 40),
    ("mxfp4", 128, 3001, 60, None),
    ("mxfp4", 128, 7, 1, 144),
    ("fp8", 128, 1, 1, None),
    ("fp8", 128, 3001, 15, None, 256),
    ("mxfp4", 128, 1000, 5, 136, 256),
]


def _run(x, slots=None):
    dev = torch.device("cuda")
    pool = torch.from_numpy(x.cache.copy()).to(dev)
    cache = idx.Cache(pool, x.head_dim, x.fmt, x.page_size)
    k = torch.from_numpy(x.k_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    s = torch.from_numpy(x.slots if slots is None else slots).to(dev)
    ws = idx.new_workspace(idx.idx_workspace_bytes(idx.IDX_OP_CACHE_WRITE, cache, None, 0, 0), dev)
    idx.idx_cache_write(cache, k, s, ws)
    status = idx.idx_read_device_status(ws)
    return pool.cpu().numpy().reshape(-1), status


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_cache_write_bitexact(case):
    fmt, D, T, P, stride = case[:5]
    ps = case[5] if len(case) > 5 else 64
    x = cache_write_inputs(seed=500 + CASES.index(case), tokens=T, head_dim=D, fmt=fmt, num_pages=P,
                           k_stride=stride, page_size=ps)
    print(f"case {case} skipped slots {(x.slots < 0).sum()}", flush=True)
    got, status = _run(x)
    ref, bad = oracle.cache_write.write(x.cache, x.k_bits[:, :D], x.slots, fmt=fmt, page_size=ps,
                                        page_bytes=x.page_bytes)
    assert not bad and status == 0
    diff = np.nonzero(got != ref)[0]
    assert diff.size == 0, f"{diff.size} bytes differ, first at {diff[:8]}"


@pytest.mark.parametrize("ps", [64, 256])
def test_cache_write_bad_slots_skipped_and_flagged(ps):
    """Slots at or past num_pages * page_size are skipped and flagged; the
    last slot of the pool (num_pages * page_size - 1) is written."""
    x = cache_write_inputs(seed=77, tokens=400, head_dim=128, fmt="fp8", num_pages=10, page_size=ps)
    slots = x.slots.copy()
    cap = 10 * ps
    slots[slots == cap - 1] = -1
    slots[[3, 50, 399, 7]] = [cap, cap + 12345, 1 << 40, cap - 1]
    got, status = _run(x, slots)
    ref, bad = oracle.cache_write.write(x.cache, x.k_bits[:, :128], slots, fmt="fp8", page_size=ps,
                                        page_bytes=x.page_bytes)
    assert bad and status == idx.IDX_DEV_BAD_SLOT
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_cache_write_full_size_sampled(fmt):
    """The size the benchmark times: 64 x 131072 = 8,388,608 new tokens, a
    pool of exactly that many slots, one launch; 4096 sampled tokens are
    checked byte by byte against the oracle, and every slot is written."""
    dev = torch.device("cuda")
    T, D = 64 * 131072, 128
    P = T // 64
    g = torch.Generator(device=dev)
    g.manual_seed(900 if fmt == "fp8" else 901)
    print(f"full-size cache write {fmt}: {T} tokens", flush=True)
    k = torch.randn((T, D), generator=g, device=dev).to(torch.bfloat16)
    slots = torch.randperm(T, generator=g, device=dev)
    rb = D + 4 if fmt == "fp8" else D // 2 + D // 32
    page_bytes = (64 * rb + 15) // 16 * 16
    pool = torch.full((P, page_bytes), 0x5A, dtype=torch.uint8, device=dev)
    cache = idx.Cache(pool, D, fmt)
    ws = idx.new_workspace(256, dev)
    idx.idx_cache_write(cache, k, slots, ws)
    assert idx.idx_read_device_status(ws) == 0
    rng = np.random.default_rng(5)
    sample = np.sort(rng.choice(T, 4096, replace=False))
    ks = k[torch.from_numpy(sample).to(dev)].view(torch.int16).cpu().numpy().view(np.uint16)
    ss = slots[torch.from_numpy(sample).to(dev)].cpu().numpy()
    ref = oracle.cache_write.quantize_rows(ks, fmt)
    flat = pool.view(-1)
    starts = torch.from_numpy((ss // 64) * page_bytes + (ss % 64) * rb).to(dev)
    got = flat[starts[:, None] + torch.arange(rb, device=dev)[None, :]].cpu().numpy()
    assert np.array_equal(got, ref)
    # every slot was written: no row keeps the poison pattern in its scale bytes
    rows = pool[:, : 64 * rb].reshape(P * 64, rb)
    assert not bool(((rows[:, -4:] == 0x5A).all(dim=1)).any())


@pytest.mark.parametrize("fmt,ps,ratio", [("fp8", 64, 1), ("mxfp4", 64, 1), ("fp8", 256, 4)])
def test_written_cache_is_scored_like_the_oracles(fmt, ps, ratio):
    """Keys written by idx_cache_write at the slots a block table gives them,
    then scored by idx_logits_paged / idx_decode_topk, against the oracle's
    write followed by the oracle's scoring."""
    from tests.gpu_util import Dev, check_logits, check_topk_e2e
    from workloads import build_decode

    seqs = [70, 1000, 4100, 9000]
    H, D, k = 32, 128, 256
    wl = build_decode(seed=61, seq_lens=seqs, heads=H, head_dim=D, topk=k, fmt=fmt, page_size=ps,
                      compress_ratio=ratio, name=f"written-{fmt}-p{ps}")
    stored = np.asarray(seqs) // ratio
    rng = np.random.default_rng(62)
    T = int(stored.sum())
    keys = (rng.standard_normal((T, D)).astype(np.float32) * np.exp2(rng.integers(-3, 4, (T, 1))))
    kb = torch.from_numpy(keys).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    # slot of stored key t of request b: page block_table[b, t // ps], row t % ps
    slots = np.concatenate([wl.block_table[b, np.arange(n) // ps].astype(np.int64) * ps + np.arange(n) % ps
                            for b, n in enumerate(stored)])
    ref_pool, bad = oracle.cache_write.write(wl.cache, kb, slots, fmt=fmt, page_size=ps, page_bytes=wl.page_bytes)
    assert not bad
    dev = Dev(wl)
    ws = idx.new_workspace(256, dev.device)
    idx.idx_cache_write(dev.cache, torch.from_numpy(kb.view(np.int16)).to(dev.device).view(torch.bfloat16),
                        torch.from_numpy(slots).to(dev.device), ws)
    got_pool = dev.cache.pages.cpu().numpy().reshape(-1)
    assert np.array_equal(got_pool, ref_pool)
    wl.cache = ref_pool.reshape(wl.cache.shape)        # the oracle scores its own write
    ref = oracle.pipeline.decode_logits(wl)
    got, _ = dev.logits_decode()
    check_logits(got, {r: v for r, v in ref.items() if len(v)}, label=wl.name)
    L, _ = oracle.pipeline.decode_row_info(wl)
    out, _ = dev.decode_topk()
    check_topk_e2e(out, ref, L, k, label=wl.name)
