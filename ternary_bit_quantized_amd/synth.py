"""Seeded synthetic inputs for the Q2_0 hot path.

This module is shared by the tests, the benchmark and the CPU oracle's callers.
It draws random numbers and lays them out in the Q2_0 storage format; it holds
none of the method's arithmetic (no decoding, no dot products).

Storage format being produced (bisque.today "WebGPU: add Q2_0 support", the
paragraph on the format; aisvetem.cz, section "Osmnact bajtu na ctyriasedesat
vah"): a block is 18 bytes for 64 weights.  Bytes 0-1 hold the scale d as a
little-endian IEEE half; bytes 2-17 hold four little-endian 32-bit words, and
code i of word w sits in bits 2i..2i+1 and belongs to weight 16w+i.  On a
little-endian word that means byte j of the 16 code bytes carries the codes of
weights 4j..4j+3, lowest weight in the lowest two bits.

A weight matrix of M rows and K columns (K a multiple of 64) is stored row-major
as M rows of K/64 consecutive blocks, i.e. row m starts at byte m*(K/64)*18.

Seeds: every draw comes from
``np.random.default_rng(SeedSequence([seed, layer, matrix, stream]))`` where
``stream`` is 0 for codes, 1 for scales, 2 for activations, 3 for row ids and
4 for the zero-scale mask.
"""

from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
from typing import Iterable

import numpy as np

BLOCK_WEIGHTS = 64
BLOCK_BYTES = 18

STREAM_CODES, STREAM_SCALES, STREAM_X, STREAM_IDS, STREAM_ZERO = 0, 1, 2, 3, 4

# Matrix indices inside a transformer layer.
MATS = ("q", "k", "v", "o", "gate", "up", "down")


def rng_for(seed: int, layer: int, matrix: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, layer, matrix, stream]))


# ---------------------------------------------------------------------------
# Packing: codes (0..3) and half-precision scales -> Q2_0 bytes.
# ---------------------------------------------------------------------------

def pack_code_bytes(codes: np.ndarray) -> np.ndarray:
    """codes: (..., K) uint8 in 0..3, K % 4 == 0 -> (..., K/4) uint8.

    Byte j holds the codes of weights 4j..4j+3 at bit offsets 0, 2, 4, 6.
    """
    c = codes.reshape(codes.shape[:-1] + (codes.shape[-1] // 4, 4)).astype(np.uint8)
    return (c[..., 0] | (c[..., 1] << 2) | (c[..., 2] << 4) | (c[..., 3] << 6)).astype(np.uint8)


def assemble_blocks(scales_f16: np.ndarray, code_bytes: np.ndarray) -> np.ndarray:
    """scales_f16: (M, nb) float16; code_bytes: (M, nb*16) uint8 -> (M, nb*18) uint8."""
    M, nb = scales_f16.shape
    out = np.empty((M, nb, BLOCK_BYTES), dtype=np.uint8)
    out[:, :, 0:2] = np.ascontiguousarray(scales_f16.astype("<f2")).view(np.uint8).reshape(M, nb, 2)
    out[:, :, 2:] = code_bytes.reshape(M, nb, 16)
    return out.reshape(M, nb * BLOCK_BYTES)


def pack(codes: np.ndarray, scales_f16: np.ndarray) -> np.ndarray:
    """codes (M, K) in 0..3 and scales (M, K/64) float16 -> packed (M, K/64*18) uint8."""
    M, K = codes.shape
    assert K % BLOCK_WEIGHTS == 0 and scales_f16.shape == (M, K // BLOCK_WEIGHTS)
    return assemble_blocks(np.asarray(scales_f16, dtype=np.float16), pack_code_bytes(codes))


# 81-entry table: a uniform draw in [0, 81) read as four base-3 digits gives four
# i.i.d. uniform ternary codes; the entry is the byte those codes pack into.
_TERN_LUT = np.array(
    [(a | (b << 2) | (c << 4) | (d << 6))
     for v in range(81)
     for (a, b, c, d) in [(v % 3, (v // 3) % 3, (v // 9) % 3, (v // 27) % 3)]],
    dtype=np.uint8)


def code_bytes(rng: np.random.Generator, M: int, K: int, dist: str) -> np.ndarray:
    """Packed code bytes (M, K/4) for a code distribution.

    dist: "tern"    codes i.i.d. uniform in {0, 1, 2}
          "tern_c3" each code is 3 with probability 0.005, else uniform in {0, 1, 2}
          "quad"    codes i.i.d. uniform in {0, 1, 2, 3}
          "ones"    every code 1 (all-zero weights)
    """
    n = M * K // 4
    if dist == "tern":
        return _TERN_LUT[rng.integers(0, 81, size=n, dtype=np.uint8)].reshape(M, K // 4)
    if dist == "quad":
        return rng.integers(0, 256, size=n, dtype=np.uint8).reshape(M, K // 4)
    if dist == "tern_c3":
        c = rng.integers(0, 3, size=(M, K), dtype=np.uint8)
        c[rng.random(size=(M, K)) < 0.005] = 3
        return pack_code_bytes(c)
    if dist == "ones":
        return np.full((M, K // 4), 0x55, dtype=np.uint8)
    raise ValueError(dist)


@dataclasses.dataclass(frozen=True)
class ScaleDist:
    kind: str          # "uniform" or "loguniform"
    lo: float
    hi: float
    p_zero: float = 0.0  # probability that a block's scale is +0


def scales(rng: np.random.Generator, zrng: np.random.Generator | None, M: int, nb: int,
           dist: ScaleDist) -> np.ndarray:
    """(M, nb) float16 scales; drawn in float64 and rounded to half (nearest-even)."""
    if dist.kind == "uniform":
        v = rng.uniform(dist.lo, dist.hi, size=(M, nb))
    elif dist.kind == "loguniform":
        v = np.exp(rng.uniform(np.log(dist.lo), np.log(dist.hi), size=(M, nb)))
    else:
        raise ValueError(dist.kind)
    d = v.astype(np.float16)
    if dist.p_zero > 0:
        d[zrng.random(size=(M, nb)) < dist.p_zero] = np.float16(0.0)
    return d


def weight(seed: int, layer: int, matrix: int, M: int, K: int, codes: str,
           sdist: ScaleDist) -> np.ndarray:
    """A seeded packed Q2_0 weight, (M, K/64*18) uint8."""
    assert K % BLOCK_WEIGHTS == 0
    nb = K // BLOCK_WEIGHTS
    cb = code_bytes(rng_for(seed, layer, matrix, STREAM_CODES), M, K, codes)
    d = scales(rng_for(seed, layer, matrix, STREAM_SCALES), rng_for(seed, layer, matrix, STREAM_ZERO),
               M, nb, sdist)
    return assemble_blocks(d, cb)


def activations(seed: int, layer: int, matrix: int, N: int, K: int) -> np.ndarray:
    """x ~ N(0, 1) float32, N columns of K contiguous values, shape (N, K)."""
    return rng_for(seed, layer, matrix, STREAM_X).standard_normal((N, K), dtype=np.float32)


def to_f16(x: np.ndarray) -> np.ndarray:
    """Activations as IEEE half (round to nearest even), for the 16-bit activation inputs."""
    return np.asarray(x, dtype=np.float32).astype(np.float16)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Finite f32 activations rounded to bfloat16 (nearest, ties to even), as uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """The exact f32 value of bfloat16 bit patterns (the upper half of an IEEE single)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def row_ids(seed: int, layer: int, matrix: int, n: int, M: int) -> np.ndarray:
    return rng_for(seed, layer, matrix, STREAM_IDS).integers(0, M, size=n, dtype=np.int64).astype(np.int32)


def random_blocks(rng: np.random.Generator, M: int, nb: int) -> np.ndarray:
    """Fully random bytes: every scale bit pattern (subnormals, +-0, inf, NaN) can occur."""
    return rng.integers(0, 256, size=(M, nb * BLOCK_BYTES), dtype=np.uint8)


# ---------------------------------------------------------------------------
# The five workloads.
# ---------------------------------------------------------------------------

QWEN3_1P7B = {"q": (2048, 2048), "k": (1024, 2048), "v": (1024, 2048), "o": (2048, 2048),
              "gate": (6144, 2048), "up": (6144, 2048), "down": (2048, 6144)}
QWEN3_8B = {"q": (4096, 4096), "k": (1024, 4096), "v": (1024, 4096), "o": (4096, 4096),
            "gate": (12288, 4096), "up": (12288, 4096), "down": (4096, 12288)}
QWEN3_8B_LAYERS = 36
QWEN3_1P7B_LAYERS = 28
VOCAB, HIDDEN_8B = 151936, 4096


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    shapes: dict            # matrix name -> (M, K)
    codes: str
    sdist: ScaleDist
    ns: tuple               # activation column counts exercised
    layers: int = 1


TINY = Workload("tiny_256x512", 0, {"w": (256, 512)}, "tern", ScaleDist("uniform", 0.01, 0.1), (1,))
DECODE_1P7B = Workload("qwen3_1.7b_decode", 1, QWEN3_1P7B, "tern_c3",
                       ScaleDist("uniform", 0.005, 0.05), (1, 8))
PREFILL_1P7B = Workload("qwen3_1.7b_prefill", 2, QWEN3_1P7B, "tern",
                        ScaleDist("uniform", 0.005, 0.05), (512,))
STACK_8B = Workload("qwen3_8b_stack", 3, QWEN3_8B, "tern", ScaleDist("uniform", 0.002, 0.02),
                    (1, 512), layers=QWEN3_8B_LAYERS)
VOCAB_8B = Workload("vocab151936x4096", 4, {"emb": (VOCAB, HIDDEN_8B)}, "quad",
                    ScaleDist("loguniform", 1e-3, 1e-1, p_zero=0.01), (1, 4))

WORKLOADS = (TINY, DECODE_1P7B, PREFILL_1P7B, STACK_8B, VOCAB_8B)

# Row-id draws for the get_rows cases.
TINY_IDS = 4
VOCAB_IDS = 512


def workload_weight(wl: Workload, name: str, layer: int = 0) -> np.ndarray:
    M, K = wl.shapes[name]
    idx = MATS.index(name) if name in MATS else 0
    return weight(wl.seed, layer, idx, M, K, wl.codes, wl.sdist)


def stack_x_matrix_index(K: int) -> int:
    """The 36-layer stack uses one activation per distinct K (and per N): keyed 7 + K//4096."""
    return 7 + K // 4096


def stack_weights(wl: Workload, layers: Iterable[int], threads: int = 8) -> dict:
    """{(layer, name): packed weight} generated in parallel (numpy drops the GIL in its RNG)."""
    jobs = [(l, n) for l in layers for n in MATS]
    with ThreadPoolExecutor(max_workers=threads) as ex:
        res = ex.map(lambda j: workload_weight(wl, j[1], j[0]), jobs)
        return dict(zip(jobs, res))
