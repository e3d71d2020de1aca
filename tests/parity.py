"""Helpers for comparing the HIP path with the float64 oracle (tests only)."""
from __future__ import annotations

import numpy as np
import torch

import oracle

BF16_ATOL = 2e-2       # max-abs output error, bf16 inputs and outputs
F32_ATOL = 1e-4        # max-abs output error, fp32
# max-abs error of the natural-log LSE: the logits are exact bf16 products summed in fp32 and the row sum
# is a sum of P rounded to bf16 (relative error at most 2^-8 per term, so at most 2^-8 = 3.9e-3 on the
# sum and on its log); fp32 inputs keep every step in fp32
BF16_LSE_ATOL = 1e-2
F32_LSE_ATOL = 1e-4
SEL_REL = 1e-4         # selection exemption window around the top-p cutoff


def to_dev(x: np.ndarray, dtype: str, device) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)      # exact: the values are bf16-representable
    return t.to(device).contiguous()


def kept_lists(idx: torch.Tensor, cnt: torch.Tensor):
    """(batch, H, nq, nk) int32 lists -> nested python lists of arrays."""
    idx = idx.cpu().numpy()
    cnt = cnt.cpu().numpy()
    out = []
    for b in range(idx.shape[0]):
        out.append([[idx[b, g, i, :cnt[b, g, i]].astype(np.int64) for i in range(idx.shape[2])]
                    for g in range(idx.shape[1])])
    return out


def check_list_format(idx: torch.Tensor, cnt: torch.Tensor, n_cand):
    """Lists ascending, unique, in range, -1 padded.  n_cand(i) = #candidates."""
    idx = idx.cpu().numpy()
    cnt = cnt.cpu().numpy()
    nk = idx.shape[-1]
    for pos in np.ndindex(*cnt.shape):
        c = int(cnt[pos])
        row = idx[pos]
        n = n_cand(pos[-1])
        assert 1 <= c <= n, (pos, c, n)
        assert np.all(np.diff(row[:c]) > 0), pos
        assert row[0] >= 0 and row[c - 1] < n, pos
        assert np.all(row[c:] == -1), pos
        assert c <= nk


class SelectionReport:
    def __init__(self):
        self.rows = 0
        self.mismatched_rows = 0
        self.exempt = {"rel": 0, "abs": 0, "mass": 0}
        self.violations = []

    def __repr__(self):
        return (f"rows={self.rows} mismatched_rows={self.mismatched_rows} exempt={self.exempt} "
                f"violations={len(self.violations)}")


def compare_selection(rep: SelectionReport, gpu_kept, scores, forced, top_p, k_min, where):
    """Compare one row's kept set with the oracle's under the cutoff rule:
    a block on which the two disagree is allowed iff its oracle score is within
    1e-4 (relative, or absolute in logit units) of the oracle's cutoff score,
    or the oracle's cumulative mass just before or after it is within 1e-4 of p."""
    det = oracle.topp_detail(scores, forced, top_p, k_min)
    rep.rows += 1
    a = set(int(x) for x in det["kept"])
    bset = set(int(x) for x in gpu_kept)
    diff = a ^ bset
    if not diff:
        return
    rep.mismatched_rows += 1
    order = list(det["order"])
    kstar = det["kstar"]
    if kstar == 0:
        rep.violations.append((where, sorted(diff), "no residual kept"))
        return
    s_cut = scores[order[kstar - 1]]
    cum = det["cum"]
    for j in diff:
        if j not in order:  # a forced block missing / extra
            rep.violations.append((where, j, "forced block differs"))
            continue
        gap = abs(scores[j] - s_cut)
        if gap <= SEL_REL * abs(s_cut):
            rep.exempt["rel"] += 1
            continue
        if gap <= SEL_REL:
            rep.exempt["abs"] += 1
            continue
        k = order.index(j)
        before = cum[k - 1] if k > 0 else 0.0
        after = cum[k]
        if abs(before - top_p) <= SEL_REL or abs(after - top_p) <= SEL_REL:
            rep.exempt["mass"] += 1
            continue
        rep.violations.append((where, j, f"score {scores[j]:.6g} cut {s_cut:.6g} mass {before:.6g}/{after:.6g}"))


def max_abs(a, b, mask=None):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if mask is not None:
        a, b = a[mask], b[mask]
    if a.size == 0:
        return 0.0
    return float(np.nanmax(np.abs(a - b))) if not (np.isnan(a).any() or np.isnan(b).any()) else float("inf")
