"""Seeded synthetic inputs for the rotated W4A16 linear.

This module is shared by the tests, the smoke check and the benchmark.  It
draws random tensors and encodes them in the stored formats (fp16 / bf16 bit
patterns, AWQ int32 packing) and nothing else: it holds none of the method's
arithmetic (no scaling, rotation, dequantization or contraction), so neither
the oracle nor the GPU path can inherit a mistake in the method from it.

Recipe (shapes and layouts from the "ParoQuant" GPTQModel wiki, Checkpoint and
inference implementation / Stored tensors; distributions chosen to stand in
for Llama-3-8B-shaped layers, since no trained weights or datasets are used):

  RNG        numpy Generator(PCG64) seeded by SeedSequence(base, spawn_key=
             (workload, layer, tensor_id)); tensor ids are fixed (TENSOR_IDS).
  x          N(0, 1), tokens x I; 4 distinct outlier channels scaled x20;
             cast to fp16 (round to nearest even) or to bf16 (nearest even on
             the fp32 bits).  The stored bit patterns define the input.
  pairs      per stage t and group g, a uniform random permutation of 0..G-1
             stored as consecutive (a, b) entries: a random perfect matching
             of the group's channels, all G/2 pairs active.
  theta      uniform(-pi/4, pi/4), (krot, I/2), fp32.
  cs         uniform(0.5, 2), (I,), fp32: the stored D^-1.
  q, z       integers 0..15, (I, O) and (I/G, O), AWQ-packed into int32.
  scales     uniform(0.005, 0.02), (I/G, O), fp16.
  bias       N(0, 0.01), (O,), fp16.
  w          (for the offline quantizer) a dense weight (O, I): N(0, 0.02)
             times a per-row factor uniform(0.5, 2), fp16/bf16/fp32.
  g          (for the rotation backward) an upstream gradient dL/dx_r,
             N(0, 1), (tokens, I), fp16/bf16 bits or fp32.
  MoE        E experts' q, z, scales, bias drawn as above with layer index
             e, stacked expert-major; the rotation (pairs, theta, cs) is
             expert 0's and shared.  Routing: each of T tokens is sent to
             k experts; the expert loads are a multinomial draw of T*k rows
             over expert probabilities from a flat Dirichlet, so loads are
             skewed and an expert may get no rows; rows are grouped by
             expert (offsets, E+1 int64).
"""
from __future__ import annotations

import dataclasses

import numpy as np

# Slot s (bits 4s..4s+3) of a packed int32 word holds column 8*w + AWQ_ORDER[s]
# (the AWQ GEMM interleave; the pages name the layout but do not print it).
AWQ_ORDER = (0, 2, 4, 6, 1, 3, 5, 7)

TENSOR_IDS = {"x": 0, "outliers": 1, "pairs": 2, "theta": 3, "cs": 4,
              "q": 5, "z": 6, "scales": 7, "bias": 8, "w": 9, "w_rows": 10, "g": 11, "route": 12}

F16, BF16, F32 = 0, 1, 2  # dtype codes shared by both C-ABIs' conventions

# The five workloads: seeded Llama-3-8B-shaped layers (synthetic weights).
WORKLOADS = {
    0: dict(name="rot-w4-linear-256x256-t4-f16", tokens=4, act=F16,
            layers=[("linear", 256, 256)]),
    1: dict(name="llama3-8b-q_proj-decode-t1-f16", tokens=1, act=F16,
            layers=[("q_proj", 4096, 4096)]),
    2: dict(name="llama3-8b-gate_proj-decode-t16-f16", tokens=16, act=F16,
            layers=[("gate_proj", 4096, 14336)]),
    3: dict(name="llama3-8b-down_proj-prefill-t2048-bf16", tokens=2048, act=BF16,
            layers=[("down_proj", 14336, 4096)]),
    4: dict(name="llama3-8b-decoder-layer-prefill-t4096-bf16", tokens=4096, act=BF16,
            layers=[("q_proj", 4096, 4096), ("k_proj", 4096, 1024),
                    ("v_proj", 4096, 1024), ("o_proj", 4096, 4096),
                    ("gate_proj", 4096, 14336), ("up_proj", 4096, 14336),
                    ("down_proj", 14336, 4096)]),
}


def rng_for(workload: int, layer: int, tensor: str, base: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence(base, spawn_key=(workload, layer, TENSOR_IDS[tensor]))
    return np.random.Generator(np.random.PCG64(ss))


def f32_to_bf16_bits(a) -> np.ndarray:
    """bf16 bit patterns of fp32 values, round to nearest even (finite inputs)."""
    # in 32 bits: the largest finite pattern, 0xFF7FFFFF, plus 0x8000 fits
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    b = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return b.astype(np.uint16)


def f16_bits(a) -> np.ndarray:
    """fp16 bit patterns (numpy's cast rounds to nearest even)."""
    return np.ascontiguousarray(a, dtype=np.float64).astype(np.float16).view(np.uint16)


def awq_pack(codes: np.ndarray) -> np.ndarray:
    """Pack (R, O) codes in 0..15 into (R, O/8) int32 words, AWQ order."""
    codes = np.asarray(codes)
    r, o = codes.shape
    if o % 8:
        raise ValueError("AWQ packing needs a column count divisible by 8")
    c = codes.astype(np.uint32).reshape(r, o // 8, 8)
    word = np.zeros((r, o // 8), dtype=np.uint32)
    for s, col in enumerate(AWQ_ORDER):
        word |= (c[:, :, col] & 0xF) << np.uint32(4 * s)
    return word.view(np.int32)


@dataclasses.dataclass
class Layer:
    """Host copies of one layer's stored tensors (numpy, C-contiguous)."""
    in_features: int
    out_features: int
    group_size: int
    krot: int
    pairs: np.ndarray           # int16  (krot, I)
    theta: np.ndarray           # float32 (krot, I/2)
    channel_scales: np.ndarray  # float32 (I,)
    qweight: np.ndarray         # int32  (I, O/8)
    qzeros: np.ndarray          # int32  (I/G, O/8)
    scales: np.ndarray          # uint16 fp16 bits (I/G, O)
    bias: np.ndarray | None     # uint16 fp16 bits (O,) or None
    q: np.ndarray | None = None  # uint8 codes (I, O), kept only on request
    z: np.ndarray | None = None  # uint8 zero codes (I/G, O), kept on request


def make_layer(workload: int, layer: int, in_features: int, out_features: int,
               group_size: int = 128, krot: int = 8, *, bias: bool = True,
               identity: bool = False, keep_codes: bool = False,
               base: int = 0) -> Layer:
    """Draw one layer.  identity=True gives zero angles and unit channel scales."""
    I, O, G = in_features, out_features, group_size
    if G == -1:
        G = I
    if I % G or G % 2 or O % 8:
        raise ValueError("need I % G == 0, even G and O % 8 == 0")
    r = rng_for(workload, layer, "pairs", base)
    pairs = np.empty((krot, I), dtype=np.int16)
    for t in range(krot):
        for g in range(I // G):
            pairs[t, g * G:(g + 1) * G] = r.permutation(G)
    if identity:
        theta = np.zeros((krot, I // 2), dtype=np.float32)
        cs = np.ones(I, dtype=np.float32)
    else:
        theta = rng_for(workload, layer, "theta", base).uniform(
            -np.pi / 4, np.pi / 4, size=(krot, I // 2)).astype(np.float32)
        cs = rng_for(workload, layer, "cs", base).uniform(0.5, 2.0, size=I).astype(np.float32)
    q = rng_for(workload, layer, "q", base).integers(0, 16, size=(I, O), dtype=np.uint8)
    z = rng_for(workload, layer, "z", base).integers(0, 16, size=(I // G, O), dtype=np.uint8)
    scales = f16_bits(rng_for(workload, layer, "scales", base).uniform(0.005, 0.02, size=(I // G, O)))
    b = f16_bits(rng_for(workload, layer, "bias", base).normal(0.0, 0.01, size=O)) if bias else None
    return Layer(I, O, group_size, krot, pairs, theta, cs, awq_pack(q), awq_pack(z),
                 scales, b, q if keep_codes else None, z if keep_codes else None)


def make_x(workload: int, layer: int, tokens: int, in_features: int, act: int,
           base: int = 0, outliers: int = 4) -> np.ndarray:
    """Activations as fp16/bf16 bit patterns (uint16) or fp32, (tokens, I)."""
    x = rng_for(workload, layer, "x", base).normal(0.0, 1.0, size=(tokens, in_features))
    if outliers:
        cols = rng_for(workload, layer, "outliers", base).choice(
            in_features, size=min(outliers, in_features), replace=False)
        x[:, cols] *= 20.0
    if act == F16:
        return f16_bits(x)
    if act == BF16:
        return f32_to_bf16_bits(x.astype(np.float32))
    if act == F32:
        return x.astype(np.float32)
    raise ValueError("unknown activation dtype code")


def make_w(workload: int, layer: int, out_features: int, in_features: int, dt: int,
           base: int = 0) -> np.ndarray:
    """A dense weight (out_features, in_features) for the offline quantizer:
    N(0, 0.02) scaled per output row by uniform[0.5, 2], as fp16/bf16 bits
    (uint16) or fp32."""
    w = rng_for(workload, layer, "w", base).normal(0.0, 0.02, size=(out_features, in_features))
    w *= rng_for(workload, layer, "w_rows", base).uniform(0.5, 2.0, size=(out_features, 1))
    if dt == F16:
        return f16_bits(w)
    if dt == BF16:
        return f32_to_bf16_bits(w.astype(np.float32))
    if dt == F32:
        return w.astype(np.float32)
    raise ValueError("unknown weight dtype code")


def make_g(workload: int, layer: int, tokens: int, in_features: int, dt: int,
           base: int = 0) -> np.ndarray:
    """An upstream gradient dL/dx_r (tokens, I): N(0, 1) as fp16/bf16 bits
    (uint16) or fp32."""
    g = rng_for(workload, layer, "g", base).normal(0.0, 1.0, size=(tokens, in_features))
    if dt == F16:
        return f16_bits(g)
    if dt == BF16:
        return f32_to_bf16_bits(g.astype(np.float32))
    if dt == F32:
        return g.astype(np.float32)
    raise ValueError("unknown gradient dtype code")


# Mixture-of-experts workloads: Mixtral-8x7B-shaped expert projections
# (hidden 4096, expert width 14336, 8 experts, top-2 routing), synthetic.
MOE_WORKLOADS = {
    5: dict(name="mixtral-8x7b-w1-experts-prefill-t2048-top2-bf16", experts=8, tokens=2048, top_k=2,
            act=BF16, layer=("w1", 4096, 14336)),
}


def make_moe_layer(workload: int, experts: int, in_features: int, out_features: int,
                   group_size: int = 128, krot: int = 8, bias: bool = True, base: int = 0) -> Layer:
    """E experts stacked in one Layer: qweight (E, I, O/8), qzeros (E, I/G, O/8),
    scales (E, I/G, O), bias (E, O); one shared rotation (expert 0's)."""
    parts = [make_layer(workload, e, in_features, out_features, group_size, krot, bias=bias, base=base)
             for e in range(experts)]
    p0 = parts[0]
    stack = lambda name: np.ascontiguousarray(np.stack([getattr(p, name) for p in parts]))
    return Layer(in_features, out_features, group_size, krot, p0.pairs, p0.theta, p0.channel_scales,
                 stack("qweight"), stack("qzeros"), stack("scales"), stack("bias") if bias else None)


def make_routing(workload: int, experts: int, tokens: int, top_k: int, base: int = 0) -> np.ndarray:
    """Expert row offsets (E+1,) int64 for T tokens routed to top_k experts each."""
    r = rng_for(workload, 0, "route", base)
    p = r.dirichlet(np.ones(experts))
    counts = r.multinomial(tokens * top_k, p)
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)


def workload_layers(workload: int, **kw):
    """(name, Layer, x) for every layer of a numbered workload."""
    spec = WORKLOADS[workload]
    for li, (lname, I, O) in enumerate(spec["layers"]):
        yield lname, make_layer(workload, li, I, O, **kw), make_x(workload, li, spec["tokens"], I, spec["act"])
