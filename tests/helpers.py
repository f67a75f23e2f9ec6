"""Shared test helpers: the oracle's version of a canvas step, the parity bar, device copies."""
from __future__ import annotations

import numpy as np

import oracle

# Parity bar for float32 outputs: |gpu - oracle| <= ATOL + RTOL * |oracle|, element-wise.
ATOL = 2e-4
RTOL = 1e-4


def assert_parity(gpu, ref, what="", atol=ATOL, rtol=RTOL):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), "%s: non-finite GPU output" % what
    err = np.abs(gpu - ref)
    bound = atol + rtol * np.abs(ref)
    bad = err > bound
    if np.any(bad):
        idx = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError("%s: %d of %d elements outside %.1e + %.1e*|ref|; worst at %s: "
                             "gpu %.8g ref %.8g (max abs err %.3e)"
                             % (what, int(bad.sum()), bad.size, atol, rtol, idx,
                                gpu[idx], ref[idx], float(err.max())))
    return float(err.max())


def oracle_prepare(case):
    """Set-up of a canvas block on the oracle side: rope table, roped cache keys."""
    cs = oracle.rope_table(case.ctx, case.T, case.hd, case.theta) if case.normed else None
    kc = case.kc
    if case.rope_cache and case.ctx > 0:
        csc = oracle.rope_table(0, case.ctx, case.hd, case.theta)
        kc = oracle.headnorm_rope(case.kc.reshape(case.B * case.nkv, case.ctx, case.hd), None,
                                  csc, 1, case.hd, oracle.NORM_ROPE | oracle.NORM_SKIP,
                                  0.0).reshape(case.kc.shape)
    return cs, kc


def oracle_step(case, q, k, v, cs, kc, rows=None):
    """One canvas step on the oracle: norms (if the case is normed), then attention."""
    if case.normed:
        q = oracle.headnorm_rope(q, case.wq, cs, case.nh, case.hd, 3, case.eps)
        k = oracle.headnorm_rope(k, case.wk, cs, case.nkv, case.hd, 3, case.eps)
        v = oracle.headnorm_rope(v, None, None, case.nkv, case.hd, 0, case.eps)
    out = oracle.attn_split_gqa(q, kc, case.vc, k, v, case.nh, case.nkv, case.hd, case.scale,
                                case.causal, rows=rows)
    return out, (q, k, v)


def sample_rows(nrows, count, seed):
    """Sorted distinct row indices: the first and last rows plus a seeded random draw."""
    rng = np.random.default_rng(seed)
    pick = set([0, nrows - 1])
    pick.update(rng.choice(nrows, size=min(count, nrows), replace=False).tolist())
    return np.array(sorted(pick), dtype=np.int64)
