"""Pearson chi-square goodness of fit, used by the statistical pins."""
import numpy as np
from scipy import stats


def chi2_pvalue(observed: np.ndarray, probs: np.ndarray, min_expected: float = 5.0):
    """Pearson X^2 of ``observed`` counts against ``probs``; cells whose expected count is
    below ``min_expected`` are pooled into one cell.  Returns (p-value, X^2, df)."""
    observed = np.asarray(observed, dtype=np.float64)
    probs = np.asarray(probs, dtype=np.float64)
    n = observed.sum()
    exp = n * probs / probs.sum()
    big = exp >= min_expected
    o = list(observed[big])
    e = list(exp[big])
    if (~big).any():
        o.append(observed[~big].sum())
        e.append(exp[~big].sum())
    o, e = np.array(o), np.array(e)
    keep = e > 0
    # a count in a cell of zero expectation is an outright failure
    if (o[~keep] > 0).any():
        return 0.0, np.inf, 0
    o, e = o[keep], e[keep]
    x2 = float(((o - e) ** 2 / e).sum())
    df = len(o) - 1
    return float(stats.chi2.sf(x2, df)), x2, df
