"""Seeded synthetic workloads (input generation only; no part of the method).

Every input is drawn from numpy's PCG64 generator.  The root
``SeedSequence(seed)`` of a workload is spawned into independent streams, one
per quantity (document lengths, x, dy, weight, bias, saturation mask), so a
quantity's values do not depend on what else is drawn.  Dense [S, C] normals
are drawn in float32 blocks of ``ROWS_PER_BLOCK`` rows, block i from the i-th
child of its stream, and rounded to bfloat16 (nearest, ties to even).
Parameters are drawn in float64, rounded to float32 and, for bfloat16
parameters, from float32 to bfloat16 (nearest, ties to even each time).

The five workloads mirror the shapes, dtypes and distributions the
documentation of ``flashinfer.cake_causal_conv1d_train`` prescribes for its
arguments (BF16 activations, FP32 or BF16 weight and bias, C a multiple of 8,
empty documents allowed); their sizes and distributions are this project's
choice and are listed in ``SPECS``.

BF16 arrays are returned as uint16 bit patterns.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROWS_PER_BLOCK = 1024
_STREAMS = ("docs", "x", "dy", "w", "b", "sat")


@dataclasses.dataclass(frozen=True)
class Spec:
    name: str
    seed: int
    S: int
    C: int
    docs: tuple           # ("fixed", lengths) | ("equal", n) | ("lognormal", median, sigma, lo, hi)
                          # | ("single",) | ("randint", n, lo, hi)
    w: tuple              # (dtype, "U", half_width)
    b: tuple | None       # (dtype, "N", std) or None
    policies: tuple
    sat: tuple | None = None   # (probability, magnitude) of saturated x entries


SPECS = {
    "tiny": Spec("tiny", 0, 1000, 64, ("fixed", (0, 1, 2, 3, 5, 17, 250, 722)),
                 ("f32", "U", 0.5), ("f32", "N", 0.1), ("bf16", "fp32")),
    "uniform": Spec("uniform", 1, 16384, 2048, ("equal", 4),
                    ("bf16", "U", 0.5), None, ("bf16",)),
    "headline": Spec("headline", 2, 65536, 4096, ("lognormal", 2048.0, 1.0, 1, 16384),
                     ("f32", "U", 0.5), ("f32", "N", 0.1), ("bf16",)),
    "long": Spec("long", 3, 131072, 8192, ("single",),
                 ("bf16", "U", 0.5), ("bf16", "N", 0.1), ("fp32",)),
    "stress": Spec("stress", 4, 262144, 520, ("randint", 19999, 0, 25),
                   ("f32", "U", 1.0), ("f32", "N", 0.5), ("bf16", "fp32"),
                   sat=(0.01, 60.0)),
}


@dataclasses.dataclass
class Workload:
    name: str
    S: int
    C: int
    x: np.ndarray          # uint16 [S, C] (bf16 bits)
    dy: np.ndarray         # uint16 [S, C] (bf16 bits)
    w: np.ndarray          # float32 [C, 4] or uint16 [C, 4] (bf16 bits)
    w_dtype: str           # "f32" | "bf16"
    b: np.ndarray | None   # float32 [C] or uint16 [C], or None
    b_dtype: str | None
    cu: np.ndarray         # int32 [D+1]
    policies: tuple

    @property
    def num_docs(self) -> int:
        return int(self.cu.size - 1)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, nearest with ties to even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
            >> np.uint32(16)).astype(np.uint16)


def _streams(seed: int):
    return dict(zip(_STREAMS, np.random.SeedSequence(seed).spawn(len(_STREAMS))))


def doc_lengths(spec: Spec, ss: np.random.SeedSequence) -> list:
    kind = spec.docs[0]
    S = spec.S
    if kind == "fixed":
        lengths = list(spec.docs[1])
    elif kind == "equal":
        n = spec.docs[1]
        lengths = [S // n] * n
        lengths[-1] += S - sum(lengths)
    elif kind == "single":
        lengths = [S]
    elif kind == "lognormal":
        # Draw clip(round(exp(N(ln median, sigma))), lo, hi) until the next
        # draw would reach S; the last document takes the remainder.
        _, median, sigma, lo, hi = spec.docs
        rng = np.random.Generator(np.random.PCG64(ss))
        lengths, total = [], 0
        while True:
            n = int(np.clip(np.round(np.exp(rng.normal(np.log(median), sigma))), lo, hi))
            if total + n >= S:
                lengths.append(S - total)
                break
            lengths.append(n)
            total += n
    elif kind == "randint":
        # n lengths uniform on {lo..hi}, then one document with the remainder.
        _, n, lo, hi = spec.docs
        rng = np.random.Generator(np.random.PCG64(ss))
        lengths = [int(v) for v in rng.integers(lo, hi + 1, size=n)]
        rest = S - sum(lengths)
        if rest < 0:
            raise ValueError("document lengths exceed S")
        lengths.append(rest)
    else:
        raise ValueError(kind)
    if sum(lengths) != S:
        raise ValueError("document lengths do not sum to S")
    return lengths


def cu_from_lengths(lengths) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32)


def _normal_block(args):
    child, rows, C, sat, sat_child = args
    rng = np.random.Generator(np.random.PCG64(child))
    bits = f32_to_bf16_bits(rng.standard_normal((rows, C), dtype=np.float32))
    if sat is not None:
        prob, mag = sat
        srng = np.random.Generator(np.random.PCG64(sat_child))
        hit = srng.random((rows, C)) < prob
        neg = srng.integers(0, 2, size=(rows, C)).astype(bool)
        pos_bits, neg_bits = f32_to_bf16_bits(np.array([mag, -mag], np.float32))
        bits[hit & ~neg] = pos_bits
        bits[hit & neg] = neg_bits
    return bits


def normal_bf16(S: int, C: int, ss, sat=None, sat_ss=None, workers: int = 8) -> np.ndarray:
    """[S, C] bf16 bits of N(0, 1), optionally with saturated entries."""
    nblk = (S + ROWS_PER_BLOCK - 1) // ROWS_PER_BLOCK
    children = ss.spawn(nblk) if nblk else []
    sat_children = sat_ss.spawn(nblk) if (sat is not None and nblk) else [None] * nblk
    out = np.empty((S, C), np.uint16)
    jobs = []
    for i in range(nblk):
        rows = min(ROWS_PER_BLOCK, S - i * ROWS_PER_BLOCK)
        jobs.append((children[i], rows, C, sat, sat_children[i]))
    with ThreadPoolExecutor(max_workers=max(1, workers)) as ex:
        for i, blk in enumerate(ex.map(_normal_block, jobs)):
            out[i * ROWS_PER_BLOCK:i * ROWS_PER_BLOCK + blk.shape[0]] = blk
    return out


def _param(desc, shape, ss):
    dtype, dist, scale = desc
    rng = np.random.Generator(np.random.PCG64(ss))
    if dist == "U":
        v64 = rng.uniform(-scale, scale, size=shape)
    elif dist == "N":
        v64 = rng.normal(0.0, scale, size=shape)
    else:
        raise ValueError(dist)
    v32 = v64.astype(np.float32)
    return (v32, "f32") if dtype == "f32" else (f32_to_bf16_bits(v32), "bf16")


def make(name_or_spec, *, with_dy: bool = True, workers: int = 8) -> Workload:
    spec = SPECS[name_or_spec] if isinstance(name_or_spec, str) else name_or_spec
    st = _streams(spec.seed)
    cu = cu_from_lengths(doc_lengths(spec, st["docs"]))
    x = normal_bf16(spec.S, spec.C, st["x"], spec.sat, st["sat"], workers)
    dy = normal_bf16(spec.S, spec.C, st["dy"], workers=workers) if with_dy else None
    w, w_dtype = _param(spec.w, (spec.C, 4), st["w"])
    if spec.b is not None:
        b, b_dtype = _param(spec.b, (spec.C,), st["b"])
    else:
        b, b_dtype = None, None
    return Workload(spec.name, spec.S, spec.C, x, dy, w, w_dtype, b, b_dtype, cu, spec.policies)


def random_case(seed: int, S: int, C: int, lengths=None, *, w_dtype="f32", b_dtype="f32",
                w_scale=0.5, b_scale=0.1, sat=None) -> Workload:
    """A small ad-hoc workload for tests (same recipe as the named ones)."""
    if lengths is None:
        lengths = [S]
    spec = Spec("case", seed, S, C, ("fixed", tuple(lengths)), (w_dtype, "U", w_scale),
                None if b_dtype is None else (b_dtype, "N", b_scale), ("bf16", "fp32"), sat)
    return make(spec)
