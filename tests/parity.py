"""Comparison rules between the HIP path and the CPU oracle (shared by the GPU tests, the smoke check
and the benchmark's parity line).

Tolerances:
  * indexer scores: |gpu - oracle| <= 1e-3 * max(|oracle|, mag) + 1e-5 * absmag, with
    mag = sum_j |w_j| ReLU(q_j . k) (the magnitude the signed head sum is built from: scores that cancel
    to ~0 are judged against it) and absmag = sum_j |w_j| sum_i |q_ji k_i| (fp32 rounding of a dot
    product is relative to the magnitude of its terms, which also cancel); and the plain
    |gpu - oracle| <= 1e-3 * |oracle| on the well-conditioned entries, |oracle| >= 0.1 * mag and
    |oracle| >= 1e-3 * absmag (the head sum keeps a tenth of its magnitude and the result a thousandth
    of its terms' magnitude, so a plain relative error is meaningful there; an entry whose dot products
    cancel to ~0 cannot meet any relative bound in fp32); the share of entries this covers and the 99.9%
    quantile of the plain relative error over every entry are reported;
  * top-k: bit-exact when both sides see identical scores; end to end, positions whose oracle score is
    within 1e-3 relative of the row's k-th score (the band) may be exchanged for one another: outside
    the band the sets must be equal and inside it the counts must match;
  * attention outputs: |gpu - oracle| <= 2e-2 + 1e-2 * |oracle| (bf16 outputs); the log-sum-exp, kept in
    fp32, must be within 2e-4 absolute (a dropped or duplicated key moves it by about 1/k);
  * projections (bf16 products with fp32 accumulation): |gpu - oracle| <= 1e-3 + 8e-3 * |oracle|; bit-exact
    on exact-integer inputs whose sums bf16 represents;
  * sparse backward: |gpu - oracle| <= 2^-7 * M, elementwise, where M is the sum of the magnitudes of the
    terms that make the element (sparse_bwd_magnitudes): the GPU rounds P and sm_scale dS to bf16 before
    the second products (2^-9 relative each) and forms D = dout . out from the bf16 output (2^-9 of
    sum |dout out|), all summed in fp32; 2^-7 is that with a factor 2 of margin.  pbar (fp32 sums of
    fp32 P) within 1e-5 relative plus 1e-7.
"""
from __future__ import annotations

import numpy as np

IDX_REL = 1e-3
IDX_ROUND = 1e-5
ATT_ABS, ATT_REL = 2e-2, 1e-2
LSE_ABS = 2e-4
PROJ_ABS, PROJ_REL = 1e-3, 8e-3  # bf16 output of an fp32-accumulated product: rounding <= 2^-9 relative
BWD_REL = 2.0 ** -7


def indexer_errors(gpu_rows: np.ndarray, ora_rows: np.ndarray, mag_rows: np.ndarray, absmag_rows: np.ndarray,
                   pos: np.ndarray):
    """(worst |g-o| / bound, 99.9% quantile of |g-o| / |o|, entries compared) over the causal entries."""
    e = indexer_report(gpu_rows, ora_rows, mag_rows, absmag_rows, pos)
    return e["worst_bound_ratio"], e["rel_q999"], e["n"]


def indexer_report(gpu_rows: np.ndarray, ora_rows: np.ndarray, mag_rows: np.ndarray, absmag_rows: np.ndarray,
                   pos: np.ndarray) -> dict:
    """Indexer score errors over the causal entries of the given rows:
      worst_bound_ratio  max |g-o| / (1e-3 max(|o|, mag) + 1e-5 absmag)   (the asserted bound, <= 1)
      rel_wellcond       max |g-o| / |o| over the well-conditioned entries, |o| >= 0.1 mag and
                         |o| >= 1e-3 absmag: the plain relative error where neither the head sum nor the
                         dot products inside it cancel (asserted <= 1e-3)
      frac_wellcond      the share of entries that rel_wellcond covers
      rel_q999           99.9% quantile of the plain |g-o| / |o| over every entry (reported)
      rel_max            max plain |g-o| / |o| over every entry with o != 0 (reported; unbounded where the
                         weighted head sum cancels to about 0)
      n                  entries compared"""
    worst, rel_wc, n, n_wc = 0.0, 0.0, 0, 0
    rels = []
    for r in range(len(pos)):
        m = int(pos[r]) + 1
        g = gpu_rows[r, :m].astype(np.float64)
        o = ora_rows[r, :m].astype(np.float64)
        mg = mag_rows[r, :m].astype(np.float64)
        bound = IDX_REL * np.maximum(np.abs(o), mg) + IDX_ROUND * absmag_rows[r, :m].astype(np.float64)
        d = np.abs(g - o)
        with np.errstate(divide="ignore", invalid="ignore"):
            e1 = np.where(bound > 0, d / bound, np.where(d > 0, np.inf, 0.0))
            e2 = np.where(np.abs(o) > 0, d / np.abs(o), np.where(d > 0, np.inf, 0.0))
        wc = (np.abs(o) >= 0.1 * mg) & (np.abs(o) >= 1e-3 * absmag_rows[r, :m].astype(np.float64))
        worst = max(worst, float(e1.max()))
        if wc.any():
            rel_wc = max(rel_wc, float(e2[wc].max()))
        rels.append(e2)
        n += m
        n_wc += int(wc.sum())
    allr = np.concatenate(rels) if rels else np.zeros(1)
    finite = allr[np.isfinite(allr)]
    return dict(worst_bound_ratio=worst, rel_wellcond=rel_wc, frac_wellcond=n_wc / max(n, 1),
                rel_q999=float(np.quantile(allr, 0.999)), rel_max=float(finite.max()) if finite.size else 0.0, n=n)


def assert_indexer(report: dict, what: str = ""):
    """The asserted indexer bounds: the magnitude-relative bound everywhere, and the plain 1e-3 relative
    bound on the well-conditioned entries (|o| >= 0.1 mag and |o| >= 1e-3 absmag)."""
    assert report["worst_bound_ratio"] <= 1.0, (what, report)
    assert report["rel_wellcond"] <= IDX_REL, (what, report)


def assert_idx_wellformed(idx: np.ndarray, pos: np.ndarray, k: int):
    for r in range(len(pos)):
        n = min(k, int(pos[r]) + 1)
        row = idx[r]
        assert np.all(row[n:] == -1), f"row {r}: padding"
        sel = row[:n]
        assert np.all(sel >= 0) and np.all(sel <= pos[r]), f"row {r}: out of causal range"
        assert np.all(np.diff(sel) > 0), f"row {r}: not strictly ascending"


def topk_band_match(gpu_idx: np.ndarray, ora_idx: np.ndarray, ora_scores: np.ndarray, kth: np.ndarray,
                    pos: np.ndarray):
    """Rows where GPU and oracle selections agree under the band rule; returns (n_rows_ok, n_exact)."""
    ok, exact = 0, 0
    for r in range(len(pos)):
        g = set(int(s) for s in gpu_idx[r] if s >= 0)
        o = set(int(s) for s in ora_idx[r] if s >= 0)
        if g == o:
            ok += 1
            exact += 1
            continue
        tau = float(kth[r])
        if not np.isfinite(tau):
            continue
        sc = ora_scores[r]
        band = lambda s: abs(float(sc[s]) - tau) <= IDX_REL * abs(tau)
        g_out = {s for s in g if not band(s)}
        o_out = {s for s in o if not band(s)}
        if g_out == o_out and len(g) - len(g_out) == len(o) - len(o_out):
            ok += 1
    return ok, exact


def attention_errors(gpu_out: np.ndarray, ora_out: np.ndarray, gpu_lse: np.ndarray, ora_lse: np.ndarray):
    """(max violation ratio of the allclose bound, max abs err, max lse err)."""
    g = gpu_out.astype(np.float64)
    d = np.abs(g - ora_out)
    ratio = float((d / (ATT_ABS + ATT_REL * np.abs(ora_out))).max()) if d.size else 0.0
    lse_err = float(np.abs(gpu_lse.astype(np.float64) - ora_lse).max()) if ora_lse.size else 0.0
    return ratio, float(d.max()) if d.size else 0.0, lse_err


def sparse_bwd_magnitudes(q: np.ndarray, kv: np.ndarray, idx: np.ndarray, dout: np.ndarray, sm_scale: float,
                          d_v: int, rows=None):
    """Term magnitudes for the sparse backward tolerance (float64, numpy): for each (row, head) with P and
    dS = P (dP - D) over the valid entries and Dabs = sum_d |dout out|,
      Mq[r][h]  = sm_scale sum_j (|dS_j| + P_j Dabs) |kv_j|
      Mkv[s]   += sm_scale (|dS_j| + P_j Dabs) |q[r][h]| + P_j |[dout[r][h], 0]|
    over the given rows (all by default).  q [R, H, d], kv [S, d], idx [R, k], dout [R, H, d_v] float32."""
    R, H, d = q.shape
    rows = range(R) if rows is None else rows
    mq = np.zeros((len(list(rows)), H, d))
    mkv = np.zeros(kv.shape)
    for n, r in enumerate(rows):
        sel = idx[r][idx[r] >= 0]
        if len(sel) == 0:
            continue
        kr = kv[sel].astype(np.float64)
        qr = q[r].astype(np.float64)
        dr = dout[r].astype(np.float64)
        z = sm_scale * qr @ kr.T
        p = np.exp(z - z.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        dp = dr @ kr[:, :d_v].T
        dabs = np.abs(dr * (p @ kr[:, :d_v])).sum(axis=1, keepdims=True)   # [H, 1]
        ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
        t = sm_scale * (np.abs(ds) + p * dabs)                        # [H, n]
        mq[n] = t @ np.abs(kr)
        mkv[sel] += t.T @ np.abs(qr)
        mkv[sel, :d_v] += p.T @ np.abs(dr)
    return mq, mkv
