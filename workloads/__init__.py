"""Seeded synthetic inputs for the MXFP8 MoE expert layer.

This module is shared by the tests, the oracle's callers and the benchmark.
It holds none of the layer's arithmetic: it draws random numbers, rounds
float32 draws to bf16 with torch's own cast, and runs the router that
produces the top-k ids and weights the layer takes as inputs (the router is
not part of the layer: the layer's entry points receive ids and weights).

Five workloads, seed 0 unless stated (T tokens, hidden K, expert
intermediate I, E experts, top-k):

  tiny      T=64    K=256  I=128  E=8   k=2  plain softmax top-2
  decode    T=32    K=2048 I=768  E=128 k=8  renormalised top-8, 1% outlier channels x20
  mid       T=2048  K=2048 I=768  E=128 k=8  Zipf(1.1) gate bias, top-16 experts ~50% of assignments
  prefill   T=16384 K=2048 I=768  E=128 k=8  near-uniform routing, offline pre-quantised weights
  wide      T=16384 K=4096 I=1536 E=64  k=8  2 experts unreachable, 1 expert picked by ~20% of tokens

x is N(0,1) rounded to bf16; router gate and expert weights are N(0, 0.02)
rounded to bf16.  The "prefill" workload ships its expert weights already
quantised, as a checkpoint would: e4m3 bytes and e8m0 scale bytes drawn at
random (see ``_offline_checkpoint``), so no quantiser runs to make them.

The router (every workload): logits = x . Wg^T + bias in float64, softmax,
top-k by descending probability (ties to the lower expert id), the k
probabilities renormalised to sum to 1, cast to float32.
"""

from dataclasses import dataclass, field

import numpy as np
import torch

_TAGS = {"x": 1, "gate": 2, "w13": 3, "w2": 4, "outlier": 5, "bias": 6,
         "w13q": 7, "w13s": 8, "w2q": 9, "w2s": 10, "w13q4": 11, "w13s4": 12, "w2q4": 13, "w2s4": 14}


@dataclass(frozen=True)
class Config:
    name: str
    T: int
    K: int
    I: int
    E: int
    k: int
    outliers: bool = False
    routing: str = "plain"         # plain | zipf | hot_cold
    offline: bool = False          # weights shipped pre-quantised
    extra: dict = field(default_factory=dict)

    @property
    def M(self):
        return self.T * self.k


CONFIGS = {
    "tiny": Config("tiny", 64, 256, 128, 8, 2),
    "decode": Config("decode", 32, 2048, 768, 128, 8, outliers=True),
    "mid": Config("mid", 2048, 2048, 768, 128, 8, outliers=True, routing="zipf"),
    "prefill": Config("prefill", 16384, 2048, 768, 128, 8, offline=True),
    "wide": Config("wide", 16384, 4096, 1536, 64, 8, outliers=True, routing="hot_cold"),
}


def custom_config(name, T, K, I, E, k, **kw):
    """A workload with arbitrary sizes (small parity cases, edge cases)."""
    return Config(name, T, K, I, E, k, **kw)


def rng_for(seed, tag):
    """Independent PCG64 stream per (seed, tensor)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, _TAGS[tag]])))


def to_bf16_bits(a_f32):
    """float32 array -> bf16 bit patterns (uint16), rounded by torch's cast."""
    t = torch.from_numpy(np.ascontiguousarray(a_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f64(bits):
    """bf16 bit patterns -> float64 values (torch's widening cast)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def normal_bf16(rng, shape, std, chunk_rows=None):
    """N(0, std^2) draws in float32, rounded to bf16 bits."""
    if chunk_rows is None or shape[0] <= chunk_rows:
        return to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(std))
    out = np.empty(shape, np.uint16)
    for r in range(0, shape[0], chunk_rows):
        rr = min(chunk_rows, shape[0] - r)
        out[r:r + rr] = to_bf16_bits(
            rng.standard_normal((rr,) + tuple(shape[1:]), dtype=np.float32) * np.float32(std))
    return out


def make_x(cfg, seed=0):
    """Token activations [T, K] bf16 bits; outlier channels x20 when asked."""
    rng = rng_for(seed, "x")
    x = rng.standard_normal((cfg.T, cfg.K), dtype=np.float32)
    if cfg.outliers:
        n_out = -(-cfg.K // 100)           # ceil(1% of K)
        ch = rng_for(seed, "outlier").permutation(cfg.K)[:n_out]
        x[:, ch] *= np.float32(20.0)
    return to_bf16_bits(x)


def _softmax_topk(logits, k):
    z = logits - logits.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    order = np.argsort(-p, axis=1, kind="stable")[:, :k]     # ties -> lower id
    w = np.take_along_axis(p, order, axis=1)
    w = w / w.sum(axis=1, keepdims=True)
    return order.astype(np.int32), w.astype(np.float32)


def _topk_ids(logits, k):
    return np.argsort(-logits, axis=1, kind="stable")[:, :k]


def _zipf_bias(cfg, base_logits, seed, target=0.50, top=16, s=1.1):
    """bias_e = alpha * log(r_e^-s / H): ranks r from a seeded permutation,
    alpha bisected so the top-16 experts take ~50% of all assignments."""
    E = cfg.E
    ranks = np.empty(E, np.int64)
    ranks[rng_for(seed, "bias").permutation(E)] = np.arange(1, E + 1)
    H = np.sum(np.arange(1, E + 1, dtype=np.float64) ** -s)
    base = np.log(ranks.astype(np.float64) ** -s / H)
    top_experts = ranks <= top

    def share(alpha):
        ids = _topk_ids(base_logits + alpha * base[None, :], cfg.k)
        return np.isin(ids, np.nonzero(top_experts)[0]).mean()

    lo, hi = 0.0, 8.0
    for _ in range(40):
        mid = 0.5 * (lo + hi)
        if share(mid) < target:
            lo = mid
        else:
            hi = mid
    alpha = 0.5 * (lo + hi)
    return alpha * base, dict(alpha=alpha, top16_share=share(alpha))


def _hot_cold_bias(cfg, base_logits, seed, target=0.20):
    """Two seeded experts get bias -inf (never chosen); one seeded expert gets
    a bias beta bisected so ~20% of tokens choose it."""
    perm = rng_for(seed, "bias").permutation(cfg.E)
    cold, hot = perm[:2], perm[2]
    bias = np.zeros(cfg.E)
    bias[cold] = -np.inf

    def frac(beta):
        b = bias.copy()
        b[hot] = beta
        ids = _topk_ids(base_logits + b[None, :], cfg.k)
        return (ids == hot).any(axis=1).mean()

    lo, hi = -4.0, 8.0
    for _ in range(40):
        mid = 0.5 * (lo + hi)
        if frac(mid) < target:
            lo = mid
        else:
            hi = mid
    bias[hot] = 0.5 * (lo + hi)
    return bias, dict(cold=cold.tolist(), hot=int(hot), beta=float(bias[hot]),
                      hot_token_frac=frac(bias[hot]))


def router_inputs(cfg, x_bits, seed=0):
    """The router's inputs: bf16 gate bits [E, K] N(0,0.02) and the per-expert
    logit bias (float64 [E], None for plain routing), with an info dict."""
    gate = normal_bf16(rng_for(seed, "gate"), (cfg.E, cfg.K), 0.02)
    bias, info = None, {}
    if cfg.routing in ("zipf", "hot_cold"):
        logits = bf16_bits_to_f64(x_bits) @ bf16_bits_to_f64(gate).T
        fn = _zipf_bias if cfg.routing == "zipf" else _hot_cold_bias
        bias, info = fn(cfg, logits, seed)
    return gate, bias, info


def make_routing(cfg, x_bits, seed=0):
    """Router: bf16 gate [E, K] N(0,0.02); float64 logits; returns
    (topk_ids int32 [T,k], topk_w float32 [T,k], info dict)."""
    gate, bias, info = router_inputs(cfg, x_bits, seed)
    logits = bf16_bits_to_f64(x_bits) @ bf16_bits_to_f64(gate).T
    if bias is not None:
        logits = logits + bias[None, :]
    ids, w = _softmax_topk(logits, cfg.k)
    return ids, w, info


def _offline_checkpoint(rng_q, rng_s, shape):
    """Pre-quantised weights as a checkpoint ships them.

    Payload: random sign, magnitude code drawn uniformly from 0x30..0x7E
    (e4m3 values 1 .. 448, i.e. the top ten binades, as in MX blocks whose
    largest element sits near the top of the range).  Scales: bytes drawn
    uniformly from {113, 114, 115} (2^-14 .. 2^-12), one per 32 elements,
    in the pair-split [..., K/64, 2] layout.  Dequantised magnitudes fall in
    about [6e-5, 0.11], the range of N(0, 0.02) weights.
    """
    *lead, Kd = shape
    mag = rng_q.integers(0x30, 0x7F, size=shape, dtype=np.uint8)
    sign = rng_q.integers(0, 2, size=shape, dtype=np.uint8) << 7
    q = (mag | sign).astype(np.uint8)
    s = rng_s.integers(113, 116, size=tuple(lead) + (Kd // 64, 2), dtype=np.uint8)
    return q, s


def make_weights(cfg, seed=0):
    """Expert weights.  Online workloads: bf16 bits w13 [E,2I,K], w2 [E,K,I].
    Offline workload: e4m3 bytes + e8m0 scale bytes for both."""
    E, K, I = cfg.E, cfg.K, cfg.I
    if cfg.offline:
        w13q, w13s = _offline_checkpoint(rng_for(seed, "w13q"), rng_for(seed, "w13s"), (E, 2 * I, K))
        w2q, w2s = _offline_checkpoint(rng_for(seed, "w2q"), rng_for(seed, "w2s"), (E, K, I))
        return dict(w13q=w13q, w13s=w13s, w2q=w2q, w2s=w2s)
    w13 = normal_bf16(rng_for(seed, "w13"), (E, 2 * I, K), 0.02, chunk_rows=4)
    w2 = normal_bf16(rng_for(seed, "w2"), (E, K, I), 0.02, chunk_rows=4)
    return dict(w13=w13, w2=w2)


def make_inputs(cfg, seed=0, weights=True):
    """Everything one layer call needs, as NumPy arrays."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    x = make_x(cfg, seed)
    ids, w, info = make_routing(cfg, x, seed)
    d = dict(cfg=cfg, x=x, topk_ids=ids, topk_w=w, routing_info=info)
    if weights:
        d.update(make_weights(cfg, seed))
    return d


def dense_linear_inputs(T, K, N, seed=0):
    """A dense MXFP8 linear layer's inputs: x bf16 bits [T, K] N(0,1) and an
    offline-style pre-quantised weight [N, K] (e4m3 bytes + pair-split e8m0
    scale bytes, as ``_offline_checkpoint``)."""
    x = normal_bf16(rng_for(seed, "x"), (T, K), 1.0, chunk_rows=4096)
    wq, ws = _offline_checkpoint(rng_for(seed, "w2q"), rng_for(seed, "w2s"), (N, K))
    return x, wq, ws


def _offline_checkpoint_fp4(rng_q, rng_s, shape):
    """Pre-quantised MXFP4 weights (the W4A8 path) as a checkpoint ships them:
    packed e2m1 codes, two per byte, each code uniform over the 16 codes;
    scale bytes uniform over {120, 121, 122} (2^-7 .. 2^-5) in the pair-split
    [..., K/64, 2] layout, so magnitudes fall in about [4e-3, 0.19]."""
    *lead, Kd = shape
    q = rng_q.integers(0, 256, size=tuple(lead) + (Kd // 2,), dtype=np.uint8)
    s = rng_s.integers(120, 123, size=tuple(lead) + (Kd // 64, 2), dtype=np.uint8)
    return q, s


def make_weights_w4a8(cfg, seed=0):
    """Checkpoint-style MXFP4 expert weights for the W4A8 path:
    w13q4 [E, 2I, K/2], w13s4 [E, 2I, K/64, 2], w2q4 [E, K, I/2], w2s4."""
    E, K, I = cfg.E, cfg.K, cfg.I
    w13q, w13s = _offline_checkpoint_fp4(rng_for(seed, "w13q4"), rng_for(seed, "w13s4"), (E, 2 * I, K))
    w2q, w2s = _offline_checkpoint_fp4(rng_for(seed, "w2q4"), rng_for(seed, "w2s4"), (E, K, I))
    return dict(w13q4=w13q, w13s4=w13s, w2q4=w2q, w2s4=w2s)
