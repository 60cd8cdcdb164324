"""The parity rules between the HIP path and the oracle.

* Greedy requests (T = 0, or the greedy entry point): every output slot and the accepted
  count are bit-exact.
* Sampled requests: outputs and accepted count identical, except for requests the oracle
  marks ambiguous: a decision margin |u - p(x)/q(x)| below 1e-6 at any position up to its
  stop, or a CDF gap below 1e-6 for the draw at the stop row.  Ambiguous requests are
  counted (and how many matched anyway) but still checked for the invariants.
* Probabilities: p(x), q(x), row sums and the residual mass agree to 1e-5 relative where
  the oracle's value is at least 1e-30 (absolute 1e-30 below: float32 exp underflows);
  row maxima are bit-equal.  The residual mass is held to this at every size: the library
  draws a small residual (below 5% of the mass) in a form accurate relative to itself.
* Invariants for every GPU request: 0 <= n <= gamma_b, the accepted prefix is the drafts,
  the stop slot holds an id in [0, V), the slots after it are -1.
"""
from __future__ import annotations

import numpy as np

AMBIGUOUS = 1e-6
REL = 1e-5
TINY = 1e-30


def _close(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    big = np.abs(b) >= TINY
    ok = np.ones_like(b, dtype=bool)
    ok[big] = np.abs(a[big] - b[big]) <= REL * np.abs(b[big])
    ok[~big] = np.abs(a[~big] - b[~big]) <= TINY
    return ok


def _margins(orc, db, g, on):
    """Oracle accept-test margins at the draft positions up to the oracle's stop row."""
    last = min(on, g - 1)
    return orc["margin"][db: db + last + 1] if g > 0 else np.array([])


def _ambiguous(orc, b, margins) -> bool:
    return bool((margins < AMBIGUOUS).any()) or orc["cdf_gap"][b] < AMBIGUOUS


def ambiguous_requests(w, orc: dict) -> np.ndarray:
    """Per request: sampled (T > 0) and, by the rule above, ambiguous."""
    out = np.zeros(w.B, dtype=bool)
    for b in range(w.B):
        if w.temperatures[b] > 0:
            g, db = int(w.gammas[b]), int(w.draft_base[b])
            out[b] = _ambiguous(orc, b, _margins(orc, db, g, int(orc["num_accepted"][b])))
    return out


def compare(w, gpu: dict, orc: dict, requests=None, greedy_call: bool = False,
            probes: bool = True) -> dict:
    """Check ``gpu`` against ``orc`` on ``requests`` (default all); returns a report and
    raises AssertionError listing every violation."""
    reqs = range(w.B) if requests is None else requests
    tb_all, db_all, g_all = w.target_base, w.draft_base, w.gammas
    rep = dict(requests=0, greedy=0, sampled=0, ambiguous=0, ambiguous_matched=0,
               max_rel_px=0.0, max_rel_rowsum=0.0, max_rel_resid=0.0, max_abs_resid=0.0)
    errors = []
    for b in reqs:
        tb, db, g = int(tb_all[b]), int(db_all[b]), int(g_all[b])
        rep["requests"] += 1
        gs = gpu["out_tokens"][tb: tb + g + 1]
        os_ = orc["out_tokens"][tb: tb + g + 1]
        gn, on = int(gpu["num_accepted"][b]), int(orc["num_accepted"][b])
        # invariants
        if not (0 <= gn <= g):
            errors.append(f"req {b}: accepted {gn} outside [0, {g}]")
            continue
        if not (gs[:gn] == w.draft_tokens[db: db + gn]).all():
            errors.append(f"req {b}: accepted prefix differs from the drafts")
        if not (0 <= gs[gn] < w.V):
            errors.append(f"req {b}: stop slot {gs[gn]} not a token id")
        if not (gs[gn + 1:] == -1).all():
            errors.append(f"req {b}: slots after the stop are not -1")
        equal = gn == on and (gs == os_).all()
        sampled = (not greedy_call) and w.temperatures[b] > 0
        if not sampled:
            rep["greedy"] += 1
            if not equal:
                errors.append(f"req {b} (greedy): gpu n={gn} {gs.tolist()} vs oracle n={on} "
                              f"{os_.tolist()}")
            if probes and "row_max_t" in gpu:
                stop = min(on, g)
                m_g = gpu["row_max_t"][tb: tb + stop + 1].astype(np.float64)
                m_o = orc["row_max_t"][tb: tb + stop + 1]
                if not (m_g == m_o).all():
                    errors.append(f"req {b}: row max differs")
            continue
        rep["sampled"] += 1
        margins = _margins(orc, db, g, on)
        ambiguous = _ambiguous(orc, b, margins)
        if ambiguous:
            rep["ambiguous"] += 1
            rep["ambiguous_matched"] += int(equal)
        elif not equal:
            errors.append(f"req {b}: gpu n={gn} {gs.tolist()} vs oracle n={on} {os_.tolist()} "
                          f"(margins {np.round(margins, 9).tolist()}, gap {orc['cdf_gap'][b]:.3g})")
        if not probes or "p_x" not in gpu:
            continue
        for name in ("p_x", "q_x"):
            a, o = gpu[name][db: db + g], orc[name][db: db + g]
            ok = _close(a, o)
            if not ok.all():
                errors.append(f"req {b}: {name} {a[~ok]} vs {o[~ok]}")
            big = np.abs(o) >= TINY
            if big.any():
                rep["max_rel_px"] = max(rep["max_rel_px"],
                                        float(np.max(np.abs(a[big] - o[big]) / np.abs(o[big]))))
        for name, lo, n in (("row_max_t", tb, g + 1), ("row_max_d", db, g)):
            if not (gpu[name][lo: lo + n].astype(np.float64) == orc[name][lo: lo + n]).all():
                errors.append(f"req {b}: {name} differs")
        for name, lo, n in (("row_sum_t", tb, g + 1), ("row_sum_d", db, g)):
            a, o = gpu[name][lo: lo + n], orc[name][lo: lo + n]
            if not _close(a, o).all():
                errors.append(f"req {b}: {name} {a} vs {o}")
            if n:
                rep["max_rel_rowsum"] = max(rep["max_rel_rowsum"],
                                            float(np.max(np.abs(a - o) / np.abs(o))))
        if gn == on and orc["fallback"][b] == 0:
            a, o = gpu["resid_mass"][b], orc["resid_mass"][b]
            if not _close([a], [o]).all():
                errors.append(f"req {b}: residual mass {a} vs {o}")
            rep["max_rel_resid"] = max(rep["max_rel_resid"], abs(a - o) / abs(o))
            rep["max_abs_resid"] = max(rep["max_abs_resid"], abs(a - o))
    if errors:
        raise AssertionError(f"{len(errors)} parity violations:\n" + "\n".join(errors[:40]))
    return rep
