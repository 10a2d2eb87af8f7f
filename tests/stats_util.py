"""Small statistics helpers for the distribution tests (no method arithmetic)."""
import numpy as np
from scipy import stats


def chisq_pvalue(observed_ids, probs, min_expected=5.0):
    """Chi-square goodness-of-fit p-value of observed category ids against probs.

    Categories with expected count below ``min_expected`` are pooled; an
    observation outside the support of ``probs`` gives p = 0."""
    probs = np.asarray(probs, dtype=np.float64)
    obs_ids = np.asarray(observed_ids)
    n = obs_ids.size
    assert n > 0
    if np.any(obs_ids < 0) or np.any(obs_ids >= probs.size):
        return 0.0
    counts = np.bincount(obs_ids, minlength=probs.size).astype(np.float64)
    if np.any((probs == 0) & (counts > 0)):
        return 0.0
    exp = probs * n
    big = exp >= min_expected
    o = list(counts[big])
    e = list(exp[big])
    if np.any(~big):
        o.append(counts[~big].sum())
        e.append(exp[~big].sum())
    o = np.array(o)
    e = np.array(e)
    keep = e > 0
    o, e = o[keep], e[keep]
    if o.size < 2:
        return 1.0
    e = e * (o.sum() / e.sum())
    return float(stats.chisquare(o, e).pvalue)


def mean_zscore(samples, expected_mean):
    s = np.asarray(samples, dtype=np.float64)
    sd = s.std(ddof=1)
    if sd == 0:
        return 0.0 if s.mean() == expected_mean else np.inf
    return float((s.mean() - expected_mean) / (sd / np.sqrt(s.size)))
