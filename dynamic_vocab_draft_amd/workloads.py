"""Seeded synthetic inputs for the dynamic-vocabulary draft head.

This module only *synthesises inputs*: LM-head weights, draft hidden states,
prompt ids, per-step draft-tree ids, verify ids and prefill logits.  It holds
none of the method's arithmetic (no stream update, no window, no unique, no
projection, no top-k); both the CPU oracle and the HIP path receive the arrays
it returns.

The pages' workloads (SpecBench / HumanEval prompts, Llama-3 and Qwen-2.5 LM
heads, EAGLE-2 draft trees) are not available, so these generators stand in
for them with the same shapes:

* token ids are Zipf(s=1.1) ranks mapped through a seeded permutation of the
  vocabulary (so popular ids are not clustered at low ids), optionally mixed
  with a small local pool (prompt) or resampled from the generator's own
  recent emissions (draft trees) to imitate the temporal locality the pages
  build on (NanoSpec, introduction: generation reuses recent context);
* weights ~ N(0, 0.02^2), hidden states ~ N(0, 1), prefill logits ~ N(0, 3^2)
  plus planted peaks, drawn in float32 and rounded to bfloat16 with
  round-to-nearest-even when the config is bf16.

Every array is a pure function of the config's seed: ``SeedSequence(seed)``
keys independent sequences for W, h, the id streams and the logits,
and large arrays are produced in fixed row blocks, each with its own child
seed, so the result does not depend on the number of threads used.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os
from typing import Iterator, List, Optional, Tuple

import numpy as np

# --------------------------------------------------------------------------
# Configurations (shapes of the Llama-3 / Qwen-2.5 / Qwen3 LM heads)
# --------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    V: int                 # vocabulary size (rows of W_head)
    d: int                 # hidden size (columns of W_head)
    dtype: str             # "bf16", "fp16" or "fp32" for W and h
    M: int                 # draft hidden rows per projection call
    k: int                 # draft top-k
    w_max: int             # sliding-window length W_max
    prompt_len: int
    prompt_kind: str       # "zipf" | "pool" | "uniform"
    steps: int             # decode steps
    n_tree: int            # raw draft-tree ids per step
    tree_resample: int     # of which resampled from the generator's recent emissions
    k_ver: int             # verify ids per step (distinct)
    seed: int
    # prefill-only fields
    L: int = 0             # prompt positions with target logits
    k_pre: int = 0
    sigma: float = 3.0     # std of the prefill logits
    n_peaks: int = 0       # planted peaks per prefill row
    peak: float = 0.0      # height added at each planted peak
    zipf_s: float = 1.1
    pool: int = 256        # local pool size ("pool" prompts)
    pool_p: float = 0.7    # probability of taking a prompt id from the pool
    recent: int = 128      # resampling horizon for draft-tree ids

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "fp32" else 2


CONFIGS = {
    "tiny": Config(name="tiny", V=2048, d=256, dtype="fp32", M=4, k=4, w_max=512,
                   prompt_len=512, prompt_kind="zipf", steps=8, n_tree=24,
                   tree_resample=12, k_ver=4, seed=1001),
    "llama3_8b": Config(name="llama3_8b", V=128256, d=4096, dtype="bf16", M=8, k=8,
                        w_max=3072, prompt_len=1024, prompt_kind="pool", steps=256,
                        n_tree=60, tree_resample=30, k_ver=8, seed=1002),
    "qwen25_7b": Config(name="qwen25_7b", V=151936, d=3584, dtype="bf16", M=60, k=10,
                        w_max=3072, prompt_len=2048, prompt_kind="pool", steps=256,
                        n_tree=60, tree_resample=30, k_ver=8, seed=1003),
    # Prefill candidate initialisation: target logits [L x V], then the first
    # active set at W_max, then one Llama-shaped projection (d, M, k below).
    "prefill": Config(name="prefill", V=128256, d=4096, dtype="bf16", M=8, k=8,
                      w_max=3072, prompt_len=4096, prompt_kind="zipf", steps=0,
                      n_tree=0, tree_resample=0, k_ver=0, seed=1004,
                      L=4096, k_pre=4, sigma=3.0, n_peaks=32, peak=8.0),
    "stress": Config(name="stress", V=151936, d=4096, dtype="bf16", M=64, k=16,
                     w_max=16384, prompt_len=16384, prompt_kind="uniform", steps=512,
                     n_tree=60, tree_resample=0, k_ver=8, seed=1005),
}


def get_config(name: str, **overrides) -> Config:
    cfg = CONFIGS[name]
    return dataclasses.replace(cfg, **overrides) if overrides else cfg


# --------------------------------------------------------------------------
# Low-level helpers
# --------------------------------------------------------------------------

_BLOCK_ROWS = 2048


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _seq(cfg: Config, *key: int) -> np.random.SeedSequence:
    """Independent seed sequence for one input stream of a config:
    (0,) weights, (1, step) hidden states, (2,) id script, (3,) prefill
    logits, (4,) prefill prompt."""
    return np.random.SeedSequence(entropy=cfg.seed, spawn_key=key)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns the
    16-bit patterns as uint16.  Inputs are finite (the generators never make
    NaN or Inf)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def f32_to_fp16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to IEEE binary16 (round to nearest, ties to even, by
    numpy's conversion); returns the 16-bit patterns as uint16.  Inputs stay
    within the binary16 range (the generators' values are small)."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 draws in the storage format of `dtype`: uint16 patterns for
    bf16 and fp16, float32 itself for fp32."""
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "fp16":
        return f32_to_fp16_bits(x)
    return np.ascontiguousarray(x, dtype=np.float32)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32 (input conversion for
    callers that want float views; not part of the method)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _blocked_normal(seed: np.random.SeedSequence, rows: int, cols: int, std: float,
                    fmt, post=None) -> np.ndarray:
    """rows x cols N(0, std^2) in fixed blocks of rows, each block with its own
    child seed (thread-count independent), stored as `fmt` ("bf16", "fp16" or
    "fp32"; True means "bf16").  ``post(block_index, r0, block)`` may modify
    the float32 block before rounding."""
    fmt = "bf16" if fmt is True else ("fp32" if fmt is False else fmt)
    nblk = (rows + _BLOCK_ROWS - 1) // _BLOCK_ROWS
    seeds = seed.spawn(nblk)
    out = np.empty((rows, cols), dtype=np.float32 if fmt == "fp32" else np.uint16)

    def work(b):
        r0 = b * _BLOCK_ROWS
        r1 = min(rows, r0 + _BLOCK_ROWS)
        g = np.random.default_rng(seeds[b])
        blk = g.standard_normal((r1 - r0, cols), dtype=np.float32)
        if std != 1.0:
            blk *= np.float32(std)
        if post is not None:
            post(b, r0, blk)
        out[r0:r1] = to_bits(blk, fmt)
        return None

    if nblk == 1:
        work(0)
    else:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nblk)))
    return out


class ZipfIds:
    """Draws token ids with P(rank r) proportional to r^-s over r = 1..V; the
    id of rank r is perm[r-1] for a seeded permutation of the vocabulary."""

    def __init__(self, V: int, s: float, rng: np.random.Generator):
        ranks = np.arange(1, V + 1, dtype=np.float64)
        w = ranks ** (-s)
        self.cdf = np.cumsum(w)
        self.cdf /= self.cdf[-1]
        self.perm = rng.permutation(V).astype(np.int32)
        self.V = V

    def draw(self, n: int, rng: np.random.Generator) -> np.ndarray:
        u = rng.random(n)
        r = np.searchsorted(self.cdf, u, side="right")
        r = np.minimum(r, self.V - 1)
        return self.perm[r]

    def draw_distinct(self, n: int, rng: np.random.Generator) -> np.ndarray:
        """n distinct ids, in the order they were first drawn."""
        got: List[int] = []
        seen = set()
        while len(got) < n:
            for x in self.draw(max(2 * n, 8), rng).tolist():
                if x not in seen:
                    seen.add(x)
                    got.append(x)
                    if len(got) == n:
                        break
        return np.asarray(got, dtype=np.int32)


def _uniform_distinct(V: int, n: int, rng: np.random.Generator) -> np.ndarray:
    got: List[int] = []
    seen = set()
    while len(got) < n:
        for x in rng.integers(0, V, size=max(2 * n, 8)).tolist():
            if x not in seen:
                seen.add(x)
                got.append(x)
                if len(got) == n:
                    break
    return np.asarray(got, dtype=np.int32)


# --------------------------------------------------------------------------
# Weights and hidden states
# --------------------------------------------------------------------------


def make_weights(cfg: Config, V: Optional[int] = None) -> np.ndarray:
    """W_head [V x d]: uint16 bf16 bits (bf16 configs) or float32."""
    V = cfg.V if V is None else V
    return _blocked_normal(_seq(cfg, 0), V, cfg.d, 0.02, cfg.dtype)


def make_hidden(cfg: Config, step: int, M: Optional[int] = None) -> np.ndarray:
    """Draft hidden states for one step [M x d], a fresh N(0,1) draw per step."""
    M = cfg.M if M is None else M
    g = np.random.default_rng(_seq(cfg, 1, step))
    x = g.standard_normal((M, cfg.d), dtype=np.float32)
    return to_bits(x, cfg.dtype)


# --------------------------------------------------------------------------
# Id streams
# --------------------------------------------------------------------------


@dataclasses.dataclass
class IdScript:
    """The per-sequence id inputs: the prompt, then per decode step the raw
    flattened draft-tree ids and the verify ids."""
    prompt: np.ndarray                      # int32 [prompt_len]
    tree: List[np.ndarray]                  # per step, int32 [n_tree] (raw, may repeat)
    ver: List[np.ndarray]                   # per step, int32 [k_ver] (distinct)


def make_id_script(cfg: Config, steps: Optional[int] = None) -> IdScript:
    """Prompt and per-step candidate ids.

    Draft-tree ids: ``tree_resample`` of them are drawn uniformly from the
    generator's own last ``recent`` emitted raw ids (prompt, earlier tree ids
    and verify ids, duplicates included), the rest from the id distribution;
    the two parts are interleaved by a seeded shuffle.  Verify ids are
    ``k_ver`` distinct draws from the id distribution."""
    steps = cfg.steps if steps is None else steps
    g = np.random.default_rng(_seq(cfg, 2))
    uniform = cfg.prompt_kind == "uniform"
    zipf = None if uniform else ZipfIds(cfg.V, cfg.zipf_s, g)

    def draw(n):
        return g.integers(0, cfg.V, size=n).astype(np.int32) if uniform else zipf.draw(n, g)

    if cfg.prompt_kind == "pool":
        pool = zipf.draw_distinct(cfg.pool, g)
        take = g.random(cfg.prompt_len) < cfg.pool_p
        from_pool = pool[g.integers(0, cfg.pool, size=cfg.prompt_len)]
        prompt = np.where(take, from_pool, draw(cfg.prompt_len)).astype(np.int32)
    else:
        prompt = draw(cfg.prompt_len).astype(np.int32)

    history = list(prompt.tolist())
    trees, vers = [], []
    for _ in range(steps):
        n_res = cfg.tree_resample
        recent = np.asarray(history[-cfg.recent:], dtype=np.int32)
        parts = [draw(cfg.n_tree - n_res)]
        if n_res:
            parts.append(recent[g.integers(0, len(recent), size=n_res)])
        tree = np.concatenate(parts).astype(np.int32)
        tree = tree[g.permutation(len(tree))]
        ver = (_uniform_distinct(cfg.V, cfg.k_ver, g) if uniform
               else zipf.draw_distinct(cfg.k_ver, g))
        trees.append(tree)
        vers.append(ver)
        history.extend(tree.tolist())
        history.extend(ver.tolist())
    return IdScript(prompt=prompt, tree=trees, ver=vers)


# --------------------------------------------------------------------------
# Prefill logits
# --------------------------------------------------------------------------


def make_prefill_logits(cfg: Config, L: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Target prefill logits Z [L x V] (bf16 bits, uint16): N(0, sigma^2) with
    ``peak`` added at ``n_peaks`` distinct Zipf-drawn ids per row.  Returns
    (Z, peak_ids [L x n_peaks])."""
    L = cfg.L if L is None else L
    g = np.random.default_rng(_seq(cfg, 2))
    zipf = ZipfIds(cfg.V, cfg.zipf_s, g)
    peaks = np.stack([zipf.draw_distinct(cfg.n_peaks, g) for _ in range(L)]) if cfg.n_peaks else \
        np.zeros((L, 0), np.int32)

    def post(b, r0, blk):
        rows = np.arange(blk.shape[0])[:, None]
        blk[rows, peaks[r0:r0 + blk.shape[0]]] += np.float32(cfg.peak)

    Z = _blocked_normal(_seq(cfg, 3), L, cfg.V, cfg.sigma, True, post=post)
    return Z, peaks


def make_prefill_prompt(cfg: Config) -> np.ndarray:
    """The prompt ids x_1..x_L of the prefill workload (Zipf)."""
    g = np.random.default_rng(_seq(cfg, 4))
    zipf = ZipfIds(cfg.V, cfg.zipf_s, g)
    return zipf.draw(cfg.prompt_len, g).astype(np.int32)


def iter_steps(cfg: Config, script: IdScript) -> Iterator[Tuple[int, np.ndarray, np.ndarray]]:
    for t, (tree, ver) in enumerate(zip(script.tree, script.ver)):
        yield t, tree, ver
