"""Seeded synthetic inputs for the MoE GroupGEMM + GLU workloads.

This module only draws random inputs; it holds none of the method's
arithmetic (no routing, GEMM, activation or quantisation).  Both the oracle
tests and the GPU tests/bench take their inputs from here, so they see
identical bytes.  Values are drawn in float32 with numpy's PCG64 and rounded
to bf16 (round-to-nearest-even, by torch's CPU cast) before anyone uses them.

Every large tensor is drawn per expert from its own stream
``SeedSequence([seed, tag, index])``, so any single expert can be regenerated
alone and the draws run in parallel threads.

Workloads (the model setups named on the pages; no public dataset is
involved -- these tensors stand in for trained weights and real routing):
  tiny      512 tokens, hidden 256, 4 experts, top-2 from Gaussian logits,
            intermediate 512, SwiGLU; "tiny_empty" forces one expert to 0 rows.
  dsv3      DeepSeek-V3-like one-GPU expert share: 32 experts, 16384 rows
            with Zipf(s=1.1) counts, hidden 7168, intermediate 2048.
  gptoss    GPT-OSS-like: 32 experts, top-4 of 8192 tokens, hidden = inter-
            mediate = 2880, bias ~N(0, 0.01), alpha 1.702, clamp +-7; one
            expert gets 0 rows and one more than twice the mean.
  dsv3_bwd  backward of dsv3's FC1: dY2 ~N(0, s) with s chosen so that
            dL/dy ~N(0, 1e-2) for W2 ~N(0, 0.02).
  dsv3_mx   dsv3 shapes with X = Student-t(3) * 0.5 (heavy tails for amax).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

TAGS = {"x": 1, "w1": 2, "w2": 3, "b1": 4, "logits": 5, "dy2": 6, "perm": 7, "misc": 8}


def rng(seed: int, tag: str, idx: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, TAGS[tag], idx])))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round-to-nearest-even (torch CPU cast)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_bf16(seed, tag, idx, shape, std=1.0) -> np.ndarray:
    a = rng(seed, tag, idx).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return to_bf16_bits(a)


def per_expert_normal_bf16(seed, tag, E, shape, std) -> np.ndarray:
    """[E, *shape] bf16 bits; expert e from stream (seed, tag, e)."""
    out = np.empty((E,) + tuple(shape), dtype=np.uint16)

    def fill(e):
        out[e] = normal_bf16(seed, tag, e, shape, std)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(E)))
    return out


def rows_normal_bf16(seed, tag, rows, cols, std=1.0, chunk=1024) -> np.ndarray:
    """[rows, cols] bf16 bits drawn in row chunks of ``chunk`` (stream index = chunk id)."""
    out = np.empty((rows, cols), dtype=np.uint16)
    n = (rows + chunk - 1) // chunk

    def fill(i):
        r0, r1 = i * chunk, min(rows, (i + 1) * chunk)
        out[r0:r1] = normal_bf16(seed, tag, i, (r1 - r0, cols), std)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(n)))
    return out


def zipf_counts(E: int, total: int, s: float, seed: int) -> np.ndarray:
    """Deterministic Zipf(s) counts over E experts summing exactly to ``total``.

    Rank r = 1..E gets a share proportional to r^-s, apportioned by largest
    remainder (ties to the lower rank); ranks are then assigned to expert ids
    by a seeded permutation so the hottest expert is not always id 0.
    """
    w = np.arange(1, E + 1, dtype=np.float64) ** (-s)
    quota = total * w / w.sum()
    base = np.floor(quota).astype(np.int64)
    rem = quota - base
    short = total - int(base.sum())
    order = sorted(range(E), key=lambda r: (-rem[r], r))
    for r in order[:short]:
        base[r] += 1
    perm = rng(seed, "perm").permutation(E)
    counts = np.empty(E, dtype=np.int32)
    counts[perm] = base          # rank r goes to expert perm[r]
    return counts


# ----------------------------------------------------------------------------- workloads

TINY = dict(name="tiny", seed=1, T=512, E=4, k=2, H=256, I=512)
DSV3 = dict(name="dsv3", seed=2, E=32, M=16384, H=7168, I=2048, zipf_s=1.1)
GPTOSS = dict(name="gptoss", seed=3, T=8192, E=32, k=4, H=2880, I=2880,
              alpha=1.702, limit=7.0, hot_expert_bias=0.75, cold_expert_bias=-1e4)
DSV3_BWD = dict(name="dsv3_bwd", seed=4)
DSV3_MX = dict(name="dsv3_mx", seed=5)


def tiny(empty_expert: bool = False) -> dict:
    """512 tokens, hidden 256, 4 experts, top-2 routing from N(0,1) logits.

    ``empty_expert`` sets expert 3's logits to -inf so it receives no rows
    (with 4 experts and top-2 an empty expert is otherwise vanishingly rare).
    """
    c = TINY
    seed, T, E, H, I = c["seed"], c["T"], c["E"], c["H"], c["I"]
    logits = rng(seed, "logits").standard_normal((T, E), dtype=np.float32)
    if empty_expert:
        logits[:, 3] = -np.inf
    return dict(name="tiny_empty" if empty_expert else "tiny", T=T, E=E, k=c["k"], H=H, I=I,
                logits=logits,
                x=normal_bf16(seed, "x", 0, (T, H)),
                w1=per_expert_normal_bf16(seed, "w1", E, (H, 2 * I), 0.02))


def dsv3_counts() -> np.ndarray:
    c = DSV3
    return zipf_counts(c["E"], c["M"], c["zipf_s"], c["seed"])


def dsv3(with_w2: bool = True, x_kind: str = "normal") -> dict:
    """DeepSeek-V3-like one-GPU expert share (32 of 256 routed experts)."""
    c = DSV3
    seed, E, M, H, I = c["seed"], c["E"], c["M"], c["H"], c["I"]
    d = dict(name="dsv3", E=E, M=M, H=H, I=I, counts=dsv3_counts())
    if x_kind == "normal":
        d["x"] = rows_normal_bf16(seed, "x", M, H)
    else:
        d["x"] = student_t_rows_bf16(DSV3_MX["seed"], M, H)
    d["w1"] = per_expert_normal_bf16(seed, "w1", E, (H, 2 * I), 0.02)
    if with_w2:
        d["w2"] = per_expert_normal_bf16(seed, "w2", E, (I, H), 0.02)
    return d


def dsv3_bwd_dy2_std() -> float:
    """Std of dY2 such that G = dY2 @ W2^T has std 1e-2 for W2 ~N(0, 0.02), K = 7168."""
    return 1e-2 / (0.02 * math.sqrt(DSV3["H"]))


def dsv3_dy2() -> np.ndarray:
    return rows_normal_bf16(DSV3_BWD["seed"], "dy2", DSV3["M"], DSV3["H"], dsv3_bwd_dy2_std())


def student_t_rows_bf16(seed, rows, cols, df=3.0, scale=0.5, chunk=1024) -> np.ndarray:
    out = np.empty((rows, cols), dtype=np.uint16)
    n = (rows + chunk - 1) // chunk

    def fill(i):
        r0, r1 = i * chunk, min(rows, (i + 1) * chunk)
        a = rng(seed, "x", i).standard_t(df, size=(r1 - r0, cols)).astype(np.float32)
        out[r0:r1] = to_bf16_bits(a * np.float32(scale))

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(n)))
    return out


def gptoss_logits() -> np.ndarray:
    """N(0,1) router logits plus a fixed per-expert bias: expert 0 is pushed to
    -1e4 (receives no rows) and expert 1 up by a constant chosen so that it
    receives more than twice the mean."""
    c = GPTOSS
    logits = rng(c["seed"], "logits").standard_normal((c["T"], c["E"]), dtype=np.float32)
    bias = np.zeros(c["E"], dtype=np.float32)
    bias[0] = c["cold_expert_bias"]
    bias[1] = c["hot_expert_bias"]
    return logits + bias[None, :]


def gptoss(with_weights: bool = True, with_w2: bool = False) -> dict:
    c = GPTOSS
    seed, T, E, H, I = c["seed"], c["T"], c["E"], c["H"], c["I"]
    d = dict(name="gptoss", T=T, E=E, k=c["k"], H=H, I=I, alpha=c["alpha"], limit=c["limit"],
             logits=gptoss_logits(), x=rows_normal_bf16(seed, "x", T, H))
    if with_weights:
        d["w1"] = per_expert_normal_bf16(seed, "w1", E, (H, 2 * I), 0.02)
        d["b1"] = normal_bf16(seed, "b1", 0, (E, 2 * I), 0.01)
    if with_w2:   # the optional FC2: W2 [E][I][H] bf16 ~N(0, 0.02)
        d["w2"] = per_expert_normal_bf16(seed, "w2", E, (I, H), 0.02)
    return d


def small_grouped(seed: int, counts, H: int, I: int, x_std=1.0, w_std=0.02, bias=False,
                  m_cap=None) -> dict:
    """Small grouped problem with explicit counts (parity cases: ragged tails,
    empty experts, several tiles)."""
    counts = np.asarray(counts, dtype=np.int32)
    E = len(counts)
    M = int(counts.sum())
    m_cap = M if m_cap is None else m_cap
    d = dict(E=E, M=M, M_cap=m_cap, H=H, I=I, counts=counts,
             x=normal_bf16(seed, "x", 0, (m_cap, H), x_std),
             w1=per_expert_normal_bf16(seed, "w1", E, (H, 2 * I), w_std),
             w2=per_expert_normal_bf16(seed, "w2", E, (I, H), w_std))
    if bias:
        d["b1"] = normal_bf16(seed, "b1", 0, (E, 2 * I), 0.01)
    return d


def ternary_bf16(seed: int, shape, density=1.0) -> np.ndarray:
    """Values in {-1, 0, +1} as bf16 bits; with density < 1 most entries are 0.

    Products and sums of these stay small integers, which fp32 accumulation
    and bf16 rounding represent exactly, so a GEMM over them has one correct
    bf16 result whatever the accumulation order.
    """
    g = rng(seed, "misc", 0)
    v = g.integers(-1, 2, size=shape).astype(np.float32)
    if density < 1.0:
        v *= (g.random(shape) < density).astype(np.float32)
    return to_bf16_bits(v)
