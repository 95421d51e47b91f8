"""Seeded synthetic inputs for the verify step (shared by tests, bench and smoke).

This module only draws random numbers and lays rows out; it holds none of the
method's arithmetic (no survival, ranking, budget, softmax, acceptance or
sampling of the verify step).  Both the oracle and the HIP library consume
what it produces.

Five workloads, shaped like the pages' serving setups (batch up to 256,
7-token draft blocks, DeepSeek-class vocabularies; agentlens page, section
"높은 동시성을 위한 추측적 디코딩 최적화"):

  tiny        4 requests, K=3, V=32, fp32.  z ~ N(0, 2^2), draft = z + N(0, 0.5^2).
              conf[r, j] = 0.8^j * U(0.9, 1).  raw cost 1 + 0.01 t.  tau 1.
  b16_v32000  16 requests, K=3, V=32000, bf16.  z ~ N(0, 3^2), draft = z + N(0, 1).
              conf = 0.75^j * U(0.8, 1).  flat cost (every draft is verified).
  b64_v128256 64 requests, K=7, V=128256, bf16.  z ~ N(0, 3^2), draft = z + N(0, 1).
              conf ~ U(0.5, 0.75) i.i.d. (survival at position 7 well under 10 %).
              raw cost max(1, t/256), t in [0, 512], T = 64.
  b256_v129280 256 requests, K=7, V=129280, bf16.  z ~ N(0, 3^2), draft = z + N(0, 1).
              conf = X^j with X ~ Beta(8, 2) per slot.  raw cost max(1, t/1024)
              padded to multiples of 16 up to 8 * 256 tokens, T = 256.
  b256_mix_v256000 256 requests, K_r ~ U{1..15}, V=256000, fp32, tau 0.7.
              conf = m_r * 0.85^j, m_r ~ U(0.5, 1).  raw cost
              max(1, t/1024) * (1 + 0.05 N(0, 1)), t in [0, 4096], T = 256.

Draft tokens: in stochastic mode the drafter samples from softmax(draft / tau)
by the exponential race argmax(draft/tau - log E), E ~ Exp(1) (equivalent to
the Gumbel-max trick); in greedy mode the drafter takes its own argmax.
Positions past K_r hold -1.

Every row is drawn from its own seed, numpy SeedSequence([1000 + i, r, ...]),
so any subset of rows is reproducible on its own.  bf16 workloads are drawn in
fp32 and rounded to bf16 (round to nearest even); rows are returned as fp32
arrays holding exactly the bf16 values.
"""

from dataclasses import dataclass, field

import numpy as np

CONFIG_NAMES = ["tiny", "b16_v32000", "b64_v128256", "b256_v129280", "b256_mix_v256000"]


def _round_bf16(x):
    """Round fp32 to the nearest bf16 (ties to even); returns fp32 holding bf16 values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    rounded = (bits + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)
    nan = np.isnan(x)
    out = rounded.astype(np.uint32).view(np.float32)
    out = np.where(nan, np.float32(np.nan), out)
    return out.astype(np.float32)


def bf16_bits(x):
    """Upper 16 bits of fp32 values that are exactly bf16 (as uint16)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


@dataclass
class Workload:
    name: str
    index: int
    n: int
    k_max: int
    vocab: int
    dtype: str
    tau: float
    z_sigma: float
    noise_sigma: float
    conf: np.ndarray
    draft_len: np.ndarray
    raw_cost: np.ndarray
    granule: int
    t_base: int
    n_bonus: int
    last_token: np.ndarray
    seed: int = 0
    step: int = 0
    _cache: dict = field(default_factory=dict, repr=False)

    @property
    def cost_len(self):
        return self.t_base + self.n * self.k_max + 1

    @property
    def capacity(self):
        return self.n * (self.k_max + 1)

    def request(self, r):
        """Rows of request r: target [K_r+1, V], draft [K_r, V], draft ids."""
        if r in self._cache:
            return self._cache[r]
        K = int(self.draft_len[r])
        V = self.vocab
        g = np.random.default_rng(np.random.SeedSequence([1000 + self.index, 7, r]))
        z = g.standard_normal((K + 1, V), dtype=np.float32) * np.float32(self.z_sigma)
        zd = z[:K] + g.standard_normal((K, V), dtype=np.float32) * np.float32(self.noise_sigma)
        if self.dtype == "bf16":
            z = _round_bf16(z)
            zd = _round_bf16(zd)
        gs = np.random.default_rng(np.random.SeedSequence([2000 + self.index, 7, r]))
        tok_s = np.full(self.k_max, -1, dtype=np.int32)
        tok_g = np.full(self.k_max, -1, dtype=np.int32)
        for j in range(K):
            e = gs.standard_exponential(V)
            race = zd[j].astype(np.float64) / self.tau - np.log(e)
            tok_s[j] = int(np.argmax(race))
            tok_g[j] = int(np.argmax(zd[j]))
        out = dict(target=z, draft=zd, tok_stochastic=tok_s, tok_greedy=tok_g)
        self._cache[r] = out
        return out

    def draft_tokens(self, mode):
        key = "tok_greedy" if mode == "greedy" else "tok_stochastic"
        return np.stack([self.request(r)[key] for r in range(self.n)]).astype(np.int32)

    def drop_cache(self):
        self._cache.clear()


def assemble_target(w, cu_rows, kept, rows=None, fill=np.nan):
    """Packed target logits [rows, V] with request r's rows 0..kept[r] placed at
    cu_rows[r] ..; every other row is ``fill`` (NaN by default, so that a read
    of an unused row shows up as a fault).  cu_rows comes from the caller."""
    rows = w.capacity if rows is None else rows
    out = np.full((rows, w.vocab), fill, dtype=np.float32)
    for r in range(w.n):
        b = int(kept[r])
        out[int(cu_rows[r]): int(cu_rows[r]) + b + 1] = w.request(r)["target"][: b + 1]
    return out


def assemble_draft(w, kept, fill=np.nan):
    """Padded draft logits [n * k_max, V]: row r*k_max + j holds draft row j of
    request r for j < kept[r]; every other row is ``fill``."""
    out = np.full((w.n * w.k_max, w.vocab), fill, dtype=np.float32)
    for r in range(w.n):
        b = int(kept[r])
        if b:
            out[r * w.k_max: r * w.k_max + b] = w.request(r)["draft"][:b]
    return out


def make(name_or_index):
    """Build one of the five workloads by name or by 1-based index."""
    if isinstance(name_or_index, int):
        i = name_or_index
        name = CONFIG_NAMES[i - 1]
    else:
        name = name_or_index
        i = CONFIG_NAMES.index(name) + 1
    rng = np.random.default_rng(1000 + i)
    if name == "tiny":
        n, k, V, dt, tau, zs, ns = 4, 3, 32, "fp32", 1.0, 2.0, 0.5
        pos = np.arange(1, k + 1, dtype=np.float64)
        conf = (0.8 ** pos)[None, :] * rng.uniform(0.9, 1.0, (n, k))
        dl = np.full(n, k)
        t_base = n
        raw = 1.0 + 0.01 * np.arange(0, t_base + n * k + 1)
        gran = 1
    elif name == "b16_v32000":
        n, k, V, dt, tau, zs, ns = 16, 3, 32000, "bf16", 1.0, 3.0, 1.0
        pos = np.arange(1, k + 1, dtype=np.float64)
        conf = (0.75 ** pos)[None, :] * rng.uniform(0.8, 1.0, (n, k))
        dl = np.full(n, k)
        t_base = n
        raw = np.ones(t_base + n * k + 1)
        gran = 1
    elif name == "b64_v128256":
        n, k, V, dt, tau, zs, ns = 64, 7, 128256, "bf16", 1.0, 3.0, 1.0
        conf = rng.uniform(0.5, 0.75, (n, k))
        dl = np.full(n, k)
        t_base = n
        raw = np.maximum(1.0, np.arange(0, 513) / 256.0)
        gran = 1
    elif name == "b256_v129280":
        n, k, V, dt, tau, zs, ns = 256, 7, 129280, "bf16", 1.0, 3.0, 1.0
        pos = np.arange(1, k + 1, dtype=np.float64)
        conf = rng.beta(8.0, 2.0, (n, k)) ** pos[None, :]
        dl = np.full(n, k)
        t_base = n
        raw = np.maximum(1.0, np.arange(0, (k + 1) * n + 1) / 1024.0)
        gran = 16
    elif name == "b256_mix_v256000":
        n, k, V, dt, tau, zs, ns = 256, 15, 256000, "fp32", 0.7, 3.0, 1.0
        pos = np.arange(1, k + 1, dtype=np.float64)
        dl = rng.integers(1, k + 1, n)
        m = rng.uniform(0.5, 1.0, n)
        conf = m[:, None] * (0.85 ** pos)[None, :]
        conf = np.where(pos[None, :] <= dl[:, None], conf, 0.0)
        t_base = n
        t = np.arange(0, 4097, dtype=np.float64)
        raw = np.maximum(1.0, t / 1024.0) * np.maximum(0.5, 1.0 + 0.05 * rng.standard_normal(len(t)))
        gran = 1
    else:
        raise KeyError(name)
    last = rng.integers(0, V, n).astype(np.int32)
    return Workload(name=name, index=i, n=n, k_max=k, vocab=V, dtype=dt, tau=tau,
                    z_sigma=zs, noise_sigma=ns, conf=conf.astype(np.float32),
                    draft_len=np.asarray(dl, dtype=np.int32),
                    raw_cost=np.asarray(raw, dtype=np.float32), granule=gran,
                    t_base=t_base, n_bonus=n, last_token=last)


def random_budget_case(rng, n, k_max, ties=False, zeros=False, flat_cost=False):
    """Small random budget-selection inputs for property tests.

    Confidences are multiples of 1/8 when ``ties`` (so survivals collide
    exactly); ``zeros`` sprinkles zero confidences.  Returns (conf, draft_len,
    cost, t_base, n_bonus) with a positive, random, not necessarily monotone
    cost table (the caller decides whether to shape it)."""
    if ties:
        conf = rng.integers(0, 9, (n, k_max)) / 8.0
    else:
        conf = rng.uniform(0.0, 1.0, (n, k_max))
    if zeros:
        conf = np.where(rng.uniform(size=(n, k_max)) < 0.2, 0.0, conf)
    dl = rng.integers(0, k_max + 1, n)
    t_base = int(rng.integers(0, 4))
    length = t_base + n * k_max + 1
    if flat_cost:
        cost = np.ones(length)
    else:
        cost = np.cumsum(rng.uniform(0.05, 1.0, length)) + rng.uniform(0.5, 2.0)
    return (conf.astype(np.float32), dl.astype(np.int32), cost.astype(np.float32),
            t_base, n)
