"""Seeded synthetic inputs for the speculative-sampling verification step.

Both the HIP path and the oracle are fed from here; this module holds none of the
verifier's arithmetic.  It draws logits, noise, per-request settings and uniforms with
numpy's PCG64 ``default_rng`` and lays them out the way the library expects:

* target logits ``[R_t, V]``, one row per position ``0..gamma_b`` of each request
  (request ``b`` starts at row ``cu_draft[b] + b``, or ``b * (gamma + 1)`` when dense);
* draft logits ``[R_d, V]``, row ``i`` of request ``b`` aligned with its target row ``i``
  (request ``b`` starts at row ``cu_draft[b]``, or ``b * gamma`` when dense);
* draft token ids ``[R_d]`` int32, uniforms ``[R_t, 2]`` float32 in [0, 1), and one
  temperature per request.

Draft tokens are drawn the way a draft model draws them, which is the propose half of the
method and not part of verification: at temperature ``T > 0`` by the Gumbel-max trick on
the draft logits (argmax of ``z / T + G`` with standard Gumbel noise ``G``, an exact sampler
of the tempered softmax), at ``T = 0`` as the lowest-index argmax of the draft logits.

bf16 inputs are stored as their raw 16-bit patterns (``uint16``); values are generated in
float64, rounded to float32 and then to bf16, each step round-to-nearest-even.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

DTYPES = ("f32", "bf16")
ELEM_SIZE = {"f32": 4, "bf16": 2}


# ----------------------------------------------------------------------------- encoding

def bf16_bits(x) -> np.ndarray:
    """float64/float32 array -> bf16 bit patterns (uint16), via float32, both RNE."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(h) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 (exact)."""
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def encode(x, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def decode(a, dtype: str) -> np.ndarray:
    """Stored logits -> float64 (exact)."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_to_f32(a).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# ----------------------------------------------------------------------------- container

@dataclass
class Workload:
    name: str
    dtype: str
    B: int
    gamma: int                       # dense gamma, or max gamma_b when cu_draft is given
    V: int
    target: np.ndarray               # [R_t, V] float32, or uint16 bf16 bits
    draft: np.ndarray                # [R_d, V]
    draft_tokens: np.ndarray         # [R_d] int32
    uniforms: np.ndarray             # [R_t, 2] float32
    temperatures: np.ndarray         # [B] float32; 0 => greedy request
    cu_draft: Optional[np.ndarray] = None   # [B+1] int32 CSR offsets over draft rows
    meta: dict = field(default_factory=dict)

    # -- layout helpers (pure indexing)
    @property
    def gammas(self) -> np.ndarray:
        if self.cu_draft is None:
            return np.full(self.B, self.gamma, dtype=np.int64)
        return np.diff(self.cu_draft.astype(np.int64))

    @property
    def draft_base(self) -> np.ndarray:
        if self.cu_draft is None:
            return np.arange(self.B, dtype=np.int64) * self.gamma
        return self.cu_draft[:-1].astype(np.int64)

    @property
    def target_base(self) -> np.ndarray:
        return self.draft_base + np.arange(self.B, dtype=np.int64)

    @property
    def R_t(self) -> int:
        return int(self.target.shape[0])

    @property
    def R_d(self) -> int:
        return int(self.draft.shape[0])

    @property
    def positions(self) -> int:
        """Draft positions verified per call: sum of gamma_b."""
        return int(self.gammas.sum())

    @property
    def sampling(self) -> np.ndarray:
        return self.temperatures > 0

    @property
    def compulsory_bytes(self) -> int:
        """Every logit the step must read once: all target rows, plus the draft rows of
        requests with T > 0 (greedy requests never read draft logits)."""
        es = ELEM_SIZE[self.dtype]
        g = self.gammas
        rows = int((g + 1).sum()) + int(g[self.sampling].sum())
        return rows * self.V * es

    def requests(self, lo: int, hi: int) -> "Workload":
        """Requests [lo, hi) as a workload of their own (pure indexing: their target, draft,
        token, uniform rows and temperatures; CSR offsets rebased to 0). Requests are
        independent, so its results are the matching slice of the whole batch's."""
        assert 0 <= lo < hi <= self.B
        g = self.gammas
        t0 = int(self.target_base[lo])
        t1 = int(self.target_base[hi - 1] + g[hi - 1] + 1)
        d0 = int(self.draft_base[lo])
        d1 = int(self.draft_base[hi - 1] + g[hi - 1])
        cu = None
        if self.cu_draft is not None:
            cu = (self.cu_draft[lo:hi + 1] - self.cu_draft[lo]).astype(self.cu_draft.dtype)
        return Workload(f"{self.name} requests {lo}..{hi - 1}", self.dtype, hi - lo,
                        self.gamma if cu is None else int(g[lo:hi].max()), self.V,
                        self.target[t0:t1], self.draft[d0:d1], self.draft_tokens[d0:d1],
                        self.uniforms[t0:t1], self.temperatures[lo:hi], cu, dict(self.meta))

    def request_bytes(self) -> np.ndarray:
        """Logit bytes each request needs read (its target rows, and its draft rows if it
        samples): the per-request part of ``compulsory_bytes``."""
        g = self.gammas
        return ((g + 1) + np.where(self.sampling, g, 0)) * self.V * ELEM_SIZE[self.dtype]

    def as_greedy(self) -> "Workload":
        """Same tensors, every request at temperature 0."""
        return Workload(self.name + "-greedy", self.dtype, self.B, self.gamma, self.V,
                        self.target, self.draft, self.draft_tokens, self.uniforms,
                        np.zeros_like(self.temperatures), self.cu_draft, dict(self.meta))


# ----------------------------------------------------------------------------- generator

_BLOCK = 256   # rows generated at a time, bounds host memory


def _tempered(z: np.ndarray, T: float) -> np.ndarray:
    """z / T, with masked logits (-inf) staying -inf at every temperature (T = +inf too)."""
    with np.errstate(invalid="ignore"):
        return np.where(np.isneginf(z), -np.inf, z / T)


def _gumbel_max(z: np.ndarray, T: float, rng: np.random.Generator) -> int:
    u = rng.random(z.shape[-1])
    with np.errstate(divide="ignore"):
        g = -np.log(-np.log(u))
    return int(np.argmax(_tempered(z, T) + g))


def generate(*, name: str, B: int, V: int, dtype: str, gammas: Sequence[int], dense: bool,
             target_sigma: float, draft_sigma, temperatures, seed: int,
             uniform_seed: Optional[int] = None, peaks: int = 0, peak_height: float = 8.0,
             peak_rng_seed: Optional[int] = None, target_mean: float = 0.0,
             mask_frac: float = 0.0, mask_span: int = 0) -> Workload:
    """Generic seeded workload.

    ``mask_frac`` / ``mask_span``: masked vocabulary entries (logit -inf), the same for every
    row of a request, as a vocabulary constraint would set them: each entry with probability
    ``mask_frac`` plus one run of ``mask_span`` consecutive entries, drawn per request from
    the stream (``seed+6``, request); entry 0 stays unmasked if a mask would cover the row.
    Draft rows inherit the mask (-inf plus noise), so draft tokens never land on it.

    Streams: logits ``seed+1``, draft noise ``seed+2``, peak indices ``peak_rng_seed``
    (default ``seed+3``), draft-token draws ``seed+4``, uniforms ``uniform_seed``
    (default ``seed+5``).  ``draft_sigma`` and ``temperatures`` are scalars or per-request.
    """
    if dtype not in DTYPES:
        raise ValueError(dtype)
    gammas = np.asarray(gammas, dtype=np.int64)
    assert gammas.shape == (B,) and (gammas >= 1).all()
    if dense:
        assert (gammas == gammas[0]).all()
    sig_d = np.broadcast_to(np.asarray(draft_sigma, dtype=np.float64), (B,))
    temps = np.broadcast_to(np.asarray(temperatures, dtype=np.float32), (B,)).copy()
    cu = np.zeros(B + 1, dtype=np.int64)
    cu[1:] = np.cumsum(gammas)
    R_d = int(cu[-1])
    R_t = R_d + B
    dbase = cu[:-1]
    tbase = dbase + np.arange(B)

    rng_logit = np.random.default_rng(seed + 1)
    rng_noise = np.random.default_rng(seed + 2)
    rng_peak = np.random.default_rng(seed + 3 if peak_rng_seed is None else peak_rng_seed)
    rng_tok = np.random.default_rng(seed + 4)
    rng_unif = np.random.default_rng(seed + 5 if uniform_seed is None else uniform_seed)

    store_t = np.float32 if dtype == "f32" else np.uint16
    target = np.empty((R_t, V), dtype=store_t)
    req_of_t = np.repeat(np.arange(B), gammas + 1)

    def mask_of(b: int) -> np.ndarray:
        mrng = np.random.default_rng([seed + 6, b])
        m = mrng.random(V) < mask_frac
        if mask_span:
            start = int(mrng.integers(0, max(V - mask_span, 0) + 1))
            m[start: start + mask_span] = True
        if m.all():
            m[0] = False
        return m

    for r0 in range(0, R_t, _BLOCK):
        r1 = min(R_t, r0 + _BLOCK)
        blk = rng_logit.standard_normal((r1 - r0, V)) * target_sigma + target_mean
        if mask_frac > 0 or mask_span > 0:
            for r in range(r1 - r0):
                blk[r, mask_of(int(req_of_t[r0 + r]))] = -np.inf
        if peaks:
            for r in range(r1 - r0):
                idx = rng_peak.choice(V, size=peaks, replace=False)
                blk[r, idx] += peak_height
        target[r0:r1] = encode(blk, dtype)

    # request id of every draft row, and the target row it is aligned with
    req_of_d = np.repeat(np.arange(B), gammas)
    pos_of_d = np.arange(R_d) - dbase[req_of_d]
    trow_of_d = tbase[req_of_d] + pos_of_d

    draft = np.empty((R_d, V), dtype=store_t)
    tokens = np.empty(R_d, dtype=np.int32)
    for d0 in range(0, R_d, _BLOCK):
        d1 = min(R_d, d0 + _BLOCK)
        base = decode(target[trow_of_d[d0:d1]], dtype)
        noise = rng_noise.standard_normal((d1 - d0, V)) * sig_d[req_of_d[d0:d1], None]
        enc = encode(base + noise, dtype)
        draft[d0:d1] = enc
        zd = decode(enc, dtype)
        for k in range(d1 - d0):
            T = float(temps[req_of_d[d0 + k]])
            if T > 0:
                tokens[d0 + k] = _gumbel_max(zd[k], T, rng_tok)
            else:
                tokens[d0 + k] = int(np.argmax(zd[k]))

    uniforms = rng_unif.random((R_t, 2), dtype=np.float32)
    return Workload(name=name, dtype=dtype, B=B, gamma=int(gammas.max()), V=V,
                    target=target, draft=draft, draft_tokens=tokens, uniforms=uniforms,
                    temperatures=temps.astype(np.float32),
                    cu_draft=None if dense else cu.astype(np.int32),
                    meta=dict(seed=seed, target_sigma=target_sigma))


# ----------------------------------------------------------------------------- the five workloads

CONFIG_NAMES = {
    1: "tiny-sampling B=1 gamma=4 V=1000 f32 T=1.0",
    2: "greedy B=8 gamma=5 V=32000 bf16 T=0",
    3: "llama3-vocab-sampling B=64 gamma=4 V=128256 bf16 T=0.7 peaked",
    4: "large-batch-sampling B=256 gamma=8 V=151936 f32 T=1.0 mixed-sigma",
    5: "ragged-mix B=512 gamma_b=U{1..8} V=128256 bf16 T=U[0,1.2] 20%-greedy",
}


def shard_ranges(w: Workload, G: int) -> list:
    """Contiguous request ranges [lo, hi) for G GPUs, balanced by the logit bytes each request
    needs (not by request count: requests of a ragged batch differ in rows): range k ends
    at the first request where the running bytes reach (k + 1) / G of the total."""
    assert 1 <= G <= w.B
    c = np.cumsum(w.request_bytes())
    ends = [int(np.searchsorted(c, c[-1] * (k + 1) / G, side="left")) + 1 for k in range(G)]
    out, lo = [], 0
    for k, e in enumerate(ends):
        e = min(max(e, lo + 1), w.B - (G - 1 - k))  # every range non-empty
        out.append((lo, e))
        lo = e
    assert out[-1][1] == w.B
    return out


def config(cid: int) -> Workload:
    """The five named workloads.  Seeds for workload ``c``: logits ``10c+1``, draft noise
    ``10c+2``, per-request settings ``10c+3``, draft tokens ``10c+4``, uniforms ``10c+5``
    (workload 1 draws its uniforms from seed 0)."""
    s = 10 * cid
    if cid == 1:
        return generate(name=CONFIG_NAMES[1], B=1, V=1000, dtype="f32", gammas=[4], dense=True,
                        target_sigma=2.0, draft_sigma=0.5, temperatures=1.0, seed=s,
                        uniform_seed=0)
    if cid == 2:
        return generate(name=CONFIG_NAMES[2], B=8, V=32000, dtype="bf16", gammas=[5] * 8,
                        dense=True, target_sigma=3.0, draft_sigma=1.0, temperatures=0.0, seed=s)
    if cid == 3:
        return generate(name=CONFIG_NAMES[3], B=64, V=128256, dtype="bf16", gammas=[4] * 64,
                        dense=True, target_sigma=3.0, draft_sigma=1.0, temperatures=0.7,
                        seed=s, peaks=5, peak_height=8.0)
    if cid == 4:
        prng = np.random.default_rng(s + 3)
        sig = prng.uniform(0.2, 2.0, size=256)
        return generate(name=CONFIG_NAMES[4], B=256, V=151936, dtype="f32", gammas=[8] * 256,
                        dense=True, target_sigma=2.5, draft_sigma=sig, temperatures=1.0, seed=s)
    if cid == 5:
        B = 512
        prng = np.random.default_rng(s + 3)
        gam = prng.integers(1, 9, size=B)
        greedy = prng.permutation(B)[: round(0.2 * B)]
        temps = prng.uniform(0.0, 1.2, size=B)
        temps[greedy] = 0.0
        sig = prng.uniform(0.3, 1.5, size=B)
        return generate(name=CONFIG_NAMES[5], B=B, V=128256, dtype="bf16", gammas=gam,
                        dense=False, target_sigma=3.0, draft_sigma=sig, temperatures=temps,
                        seed=s)
    raise ValueError(f"no workload {cid}")


def to_torch(w: Workload, device="cuda") -> dict:
    """Copy a workload's arrays to ``device`` as torch tensors (bf16 bits reinterpreted as
    torch.bfloat16)."""
    import torch

    def logits(a):
        if w.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
        return torch.from_numpy(a).to(device)

    def ints(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(device)

    return dict(target=logits(w.target), draft=logits(w.draft), tokens=ints(w.draft_tokens),
                uniforms=torch.from_numpy(np.ascontiguousarray(w.uniforms, np.float32)).to(device),
                temps=torch.from_numpy(np.ascontiguousarray(w.temperatures, np.float32)).to(device),
                cu=ints(w.cu_draft))


def draw_draft_tokens(zd: np.ndarray, T: float, rng: np.random.Generator) -> np.ndarray:
    """Vectorised draft-model draw for rows ``zd [..., V]`` (float64): Gumbel-max at T > 0,
    lowest-index argmax at T = 0."""
    if T > 0:
        u = rng.random(zd.shape)
        with np.errstate(divide="ignore"):
            g = -np.log(-np.log(u))
        return np.argmax(_tempered(zd, T) + g, axis=-1).astype(np.int32)
    return np.argmax(zd, axis=-1).astype(np.int32)


def tiled(target_rows: np.ndarray, draft_rows: np.ndarray, n: int, *, T: float, seed: int,
          dtype: str = "f32") -> Workload:
    """``n`` independent trials of one request: every trial shares the same ``gamma + 1``
    target rows and ``gamma`` draft rows (float64, encoded to ``dtype``), and draws its own
    draft tokens (from the draft rows, as a draft model would) and its own uniforms."""
    tr = encode(np.asarray(target_rows, dtype=np.float64), dtype)
    dr = encode(np.asarray(draft_rows, dtype=np.float64), dtype)
    g1, V = tr.shape
    gamma = g1 - 1
    assert dr.shape == (gamma, V)
    rng_tok = np.random.default_rng(seed + 4)
    rng_unif = np.random.default_rng(seed + 5)
    zd = decode(dr, dtype)
    tokens = draw_draft_tokens(np.broadcast_to(zd, (n, gamma, V)), T, rng_tok).reshape(-1)
    return Workload(name=f"tiled n={n} gamma={gamma} V={V}", dtype=dtype, B=n, gamma=gamma,
                    V=V, target=np.tile(tr, (n, 1)), draft=np.tile(dr, (n, 1)),
                    draft_tokens=tokens,
                    uniforms=rng_unif.random((n * g1, 2), dtype=np.float32),
                    temperatures=np.full(n, T, dtype=np.float32), cu_draft=None,
                    meta=dict(seed=seed))


def small(*, B: int, gamma: int, V: int, dtype: str = "f32", seed: int = 0,
          temperatures=1.0, target_sigma: float = 2.0, draft_sigma=0.7,
          ragged: bool = False, peaks: int = 0, mask_frac: float = 0.0,
          mask_span: int = 0) -> Workload:
    """Small seeded workload of the same construction, for tests.  ``ragged`` draws
    gamma_b from U{1..gamma} and packs them as CSR offsets; ``mask_frac`` / ``mask_span`` as
    for ``generate``."""
    prng = np.random.default_rng(seed + 3)
    if ragged:
        gam = prng.integers(1, gamma + 1, size=B)
    else:
        gam = np.full(B, gamma)
    return generate(name=f"small B={B} gamma={gamma} V={V} {dtype}", B=B, V=V, dtype=dtype,
                    gammas=gam, dense=not ragged, target_sigma=target_sigma,
                    draft_sigma=draft_sigma, temperatures=temperatures, seed=seed,
                    peaks=peaks, peak_rng_seed=seed + 6, mask_frac=mask_frac,
                    mask_span=mask_span)


# ----------------------------------------------------------------------------- token contexts

def token_contexts(B: int, capacity: int, *, seed: int, alphabet: int = 32000,
                   copy_frac: float = 0.5, min_fill: float = 0.5, span=(8, 64)):
    """Seeded token histories that repeat themselves, as RAG answers and code edits do: each
    context is a run of spans, each span either fresh tokens drawn from ``alphabet`` or (with
    probability ``copy_frac``) a copy of an earlier stretch of the same context.  Returns
    ``seq [B, capacity]`` int32 (zeros past each length) and ``lengths [B]`` int32, lengths
    ~ U[min_fill * capacity, capacity]."""
    rng = np.random.default_rng(seed)
    seq = np.zeros((B, capacity), dtype=np.int32)
    lengths = rng.integers(int(min_fill * capacity), capacity + 1, size=B).astype(np.int32)
    for b in range(B):
        L, pos = int(lengths[b]), 0
        row = seq[b]
        while pos < L:
            n = min(int(rng.integers(span[0], span[1] + 1)), L - pos)
            if pos >= span[0] and rng.random() < copy_frac:
                src = int(rng.integers(0, pos - min(n, pos) + 1))
                n = min(n, pos - src)
                row[pos: pos + n] = row[src: src + n]
            else:
                row[pos: pos + n] = rng.integers(0, alphabet, size=n)
            pos += n
    return seq, lengths
