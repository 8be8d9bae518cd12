"""Helpers for the GPU parity tests: move a workload to the device, call the
library through its C ABI, compare with the oracle at the stated tolerances.

Tolerances (fixed by the method's definition of parity):
  logits   |gpu - oracle| <= 1e-4 + 2e-3 * |oracle|        elementwise, t < L
  top-k    on the oracle's fp32-rounded logits: bit-exact rows
           end to end: same set size, and every key in the symmetric
           difference has an oracle logit within the logits tolerance of
           the oracle's k-th largest value
"""

from __future__ import annotations

import numpy as np
import torch

import sparse_attention_indexer_decode_amd as idx

ATOL, RTOL = 1e-4, 2e-3


class Dev:
    """A workload's arrays on the GPU."""

    def __init__(self, wl, device="cuda"):
        self.wl = wl
        d = torch.device(device)
        self.device = d
        self.cache = idx.Cache(torch.from_numpy(wl.cache).to(d), wl.head_dim, wl.fmt, wl.page_size)
        self.ratio = getattr(wl, "compress_ratio", 1)
        self.bt = torch.from_numpy(np.ascontiguousarray(wl.block_table)).to(d)
        self.seq = torch.from_numpy(wl.seq_lens).to(d)
        self.dl = None if wl.decode_lens is None else torch.from_numpy(wl.decode_lens).to(d)
        self.q = torch.from_numpy(wl.q.view(np.int16)).to(d).view(torch.bfloat16)
        self.w = torch.from_numpy(wl.w).to(d)
        self.max_len = int(wl.seq_lens.max(initial=0))
        if wl.kind == "prefill":
            qsl = np.concatenate([[0], np.cumsum(wl.query_lens)]).astype(np.int32)
            self.qsl = torch.from_numpy(qsl).to(d)

    def decode_rows(self):
        wl = self.wl
        return idx.Rows.decode(self.bt, self.seq, self.max_len, next_n=wl.next_n, decode_lens=self.dl,
                               q_packed=wl.q_packed, compress_ratio=self.ratio)

    def prefill_rows(self, rec):
        """Rows of a chunk record (requests [req_begin, req_end), query slice)."""
        b0, b1 = rec["req_begin"], rec["req_end"]
        qsl = self.qsl[b0 : b1 + 1]
        return idx.Rows.prefill(self.bt[b0:b1], self.seq[b0:b1], qsl, rec["q_begin"], rec["q_end"],
                                int(self.wl.seq_lens[b0:b1].max(initial=0)), compress_ratio=self.ratio)

    def chunk_queries(self, rec):
        t0, t1 = rec["token_begin"], rec["token_end"]
        return self.q[t0:t1].contiguous(), self.w[t0:t1].contiguous()

    def logits_decode(self):
        rows = self.decode_rows()
        n = rows.num_rows
        logits = torch.full((n, max(self.max_len, 1)), float("nan"), device=self.device)
        ws = idx.new_workspace(idx.idx_workspace_bytes(idx.IDX_OP_LOGITS, self.cache, rows, self.wl.heads, 0),
                               self.device)
        idx.idx_logits_paged(self.cache, rows, self.q, self.w, logits, ws)
        torch.cuda.synchronize()
        return logits.cpu().numpy(), ws

    def decode_topk(self, ws=None):
        rows = self.decode_rows()
        k = self.wl.topk
        out = torch.full((rows.num_rows, k), -7, dtype=torch.int32, device=self.device)
        if ws is None:
            ws = idx.new_workspace(idx.idx_workspace_bytes(idx.IDX_OP_DECODE_TOPK, self.cache, rows,
                                                           self.wl.heads, k), self.device)
        idx.idx_decode_topk(self.cache, rows, self.q, self.w, k, out, ws)
        torch.cuda.synchronize()
        return out.cpu().numpy(), ws


def topk_workspace(rows, k, device="cuda"):
    """A zeroed workspace sized for idx_topk on these rows."""
    return idx.new_workspace(idx.idx_workspace_bytes(idx.IDX_OP_TOPK, None, rows, 0, k), device)


def check_logits(got_rows: np.ndarray, ref: dict, col0=None, check_untouched=True, label=""):
    """got_rows[r] is the GPU logits row; ref[r] the oracle's [L] logits."""
    for r, lg in ref.items():
        c0 = 0 if col0 is None else int(col0[r])
        L = len(lg)
        g = got_rows[r, c0 : c0 + L].astype(np.float64)
        err = np.abs(g - lg)
        bad = ~(err <= ATOL + RTOL * np.abs(lg))
        assert not bad.any(), (f"{label} row {r}: {bad.sum()} of {L} outside tolerance, first at "
                               f"t={int(np.argmax(bad))}: gpu {g[np.argmax(bad)]} oracle {lg[np.argmax(bad)]}")
        if check_untouched:
            assert np.isnan(got_rows[r, :c0]).all() and np.isnan(got_rows[r, c0 + L :]).all(), \
                f"{label} row {r}: wrote outside its window"


def check_topk_e2e(got: np.ndarray, ref_logits: dict, L: np.ndarray, k: int, label=""):
    """End-to-end top-k rows against the oracle's fp64 logits."""
    for r in range(got.shape[0]):
        row = got[r]
        Lr = int(L[r])
        valid = row[row >= 0]
        assert (row[len(valid):] == -1).all(), f"{label} row {r}: -1 padding not at the tail"
        assert len(valid) == min(Lr, k), f"{label} row {r}: {len(valid)} indices, want {min(Lr, k)}"
        assert (np.diff(valid) > 0).all(), f"{label} row {r}: not ascending / duplicates"
        assert (valid < max(Lr, 1)).all() if Lr > 0 else len(valid) == 0
        if Lr <= k:
            assert valid.tolist() == list(range(Lr)), f"{label} row {r}: not the causal fill"
            continue
        lg = ref_logits[r]
        order = np.lexsort((np.arange(Lr), -lg))
        ref_set = set(order[:k].tolist())
        diff = set(valid.tolist()) ^ ref_set
        if diff:
            kth = lg[order[k - 1]]
            tol = ATOL + RTOL * abs(kth)
            far = [t for t in diff if abs(lg[t] - kth) > tol]
            assert not far, f"{label} row {r}: {len(far)} selections differ beyond tolerance"


def fp32_rows(ref: dict, n_rows: int, stride: int, col0=None) -> np.ndarray:
    """Oracle logits rounded to fp32 in a [n_rows, stride] buffer (NaN elsewhere)."""
    buf = np.full((n_rows, stride), np.nan, dtype=np.float32)
    for r, lg in ref.items():
        c0 = 0 if col0 is None else int(col0[r])
        buf[r, c0 : c0 + len(lg)] = lg.astype(np.float32)
    return buf
