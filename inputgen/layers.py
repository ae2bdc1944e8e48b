"""Seeded synthetic MoE layers: shapes, value distributions and stored formats.

The layers follow the model shapes the pages analyse (Qwen3-235B-A22B, DeepSeek-V3,
DeepSeek-V4-Pro); the pages measure on no dataset, so every tensor here is synthetic:

* x ~ N(0, 1); the router matrix Wr[H, E] and the expert matrices ~ N(0, 1/fan_in), fan_in = H
  for Wr, W_gate and W_up, fan_in = I for W_down. Values are drawn in fp32 (inputgen.philox)
  and rounded into the stored format.
* "uniform" routing has no bias; "zipf" routing adds a per-expert bias calibrated so that the
  expected number of (token, expert) assignments of the expert of popularity rank r is
  proportional to r^-alpha, capped at one per token.
* The margin rule: a token whose k-th and (k+1)-th largest router logits (biased, fp64, from
  the stored x and Wr) differ by less than ``margin`` has its row of x redrawn from the next
  attempt's stream until it passes, so the selected set cannot flip under fp32 rounding.

Stored formats (logical row-major, the layout in which the pages write the matrices):

* ``f32``  : float32[K, N]
* ``bf16`` : uint16[K, N] (bit patterns)
* ``fp8``  : uint8[K, N] OCP E4M3FN codes + float32[K/128, N/128] scales (w = code * s)
* ``mxfp4``: uint8[K, N/2] e2m1 codes (even column in the low nibble) + uint8[K/32, N] e8m0
  exponents (w = e2m1 * 2^(E-127), one exponent per 32 consecutive K of a column)
* ``mxfp4a8``: stored as ``mxfp4``; the layer quantises the routed experts' activations to MXFP8
  for their products (W4A8)
* ``mxfp8a8``: uint8[K, N] E4M3FN codes + uint8[K/32, N] e8m0 exponents (w = e4m3 * 2^(E-127),
  one exponent per 32 consecutive K of a column); the layer quantises the expert's activations to
  MXFP8 for its products (W8A8 MXFP8, the shared expert of the hybrid MXFP8-MXFP4 layer)
* ``int8``: int8[K, N] codes + float32[N] scales, one per output column (w = code * s[n]); the layer
  quantises the expert's activations to int8 per token for its products (Int8 W8A8)

with (K, N) = (H, I) for gate and up and (I, H) for down.

Streams: key0 = seed, key1 = tensor id (``TID_*``), stream = expert index (or the redraw
attempt for x); value index = row-major element index.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass

import numpy as np

from . import philox as px

TID_X = 1
TID_WR = 2
TID_XCAL = 3
TID_RANK = 4
TID_TOKENS = 5
TID_HASH = 6
TID_ROUTED = {"gate": 16, "up": 17, "down": 18}
TID_SHARED = {"gate": 24, "up": 25, "down": 26}

ACT_DTYPES = ("f32", "bf16")
W_DTYPES = ("f32", "bf16", "fp8", "mxfp4", "mxfp4a8", "mxfp8a8", "int8")


@dataclass(frozen=True)
class LayerSpec:
    name: str
    T: int
    H: int
    E: int
    k: int
    I: int
    shared: bool = False
    act: str = "bf16"
    w_routed: str = "bf16"
    w_shared: str = "bf16"
    router: str = "uniform"  # "uniform" | "zipf"
    zipf_alpha: float = 0.0
    seed: int = 1
    margin: float = 1e-3
    calib_tokens: int = 4096

    def replace(self, **kw) -> "LayerSpec":
        return dataclasses.replace(self, **kw)

    @property
    def pairs(self) -> int:
        return self.T * self.k


CONFIGS = {
    "c1": LayerSpec("tiny-fp32", T=16, H=256, E=8, k=2, I=128, act="f32", w_routed="f32",
                    w_shared="f32", seed=1),
    "c2": LayerSpec("qwen3-235b-a22b-moe-decode-bf16", T=64, H=4096, E=128, k=8, I=1536, seed=2),
    "c3": LayerSpec("deepseek-v3-moe-decode-bf16", T=256, H=7168, E=256, k=8, I=2048,
                    shared=True, router="zipf", zipf_alpha=1.0, seed=3),
    "c4": LayerSpec("deepseek-v4-pro-moe-decode-mxfp4", T=32, H=7168, E=384, k=6, I=3072,
                    shared=True, w_routed="mxfp4", w_shared="bf16", seed=4),
    "c5": LayerSpec("deepseek-v3-moe-prefill-fp8", T=16384, H=7168, E=256, k=8, I=2048,
                    shared=True, w_routed="fp8", w_shared="fp8", router="zipf", zipf_alpha=1.2,
                    seed=5),
}

# Further workloads measured beside the configurations above: the DeepSeek-V4-Pro-shaped layer at a
# prefill batch (T * k = 64 E, where the path switches to the MFMA kernel), with MXFP4 routed
# experts and bf16 activations, with W4A8 routed experts (activations quantised to MXFP8), and in
# the hybrid MXFP8-MXFP4 scheme: W4A8 routed experts and a W8A8 MXFP8 shared expert. The
# DeepSeek-V3-shaped prefill layer with Int8 W8A8 routed and shared experts. The V4-Pro decode layer
# (T = 32) with W4A8 routed experts, and in the hybrid scheme; the DeepSeek-V3 decode layer with Int8
# W8A8 experts.
EXTRA = {
    "v4p": CONFIGS["c4"].replace(name="deepseek-v4-pro-moe-prefill-mxfp4", T=4096),
    "v4p-w4a8": CONFIGS["c4"].replace(name="deepseek-v4-pro-moe-prefill-w4a8", T=4096, w_routed="mxfp4a8"),
    "v4p-mx": CONFIGS["c4"].replace(name="deepseek-v4-pro-moe-prefill-hybrid-mxfp8-mxfp4", T=4096,
                                    w_routed="mxfp4a8", w_shared="mxfp8a8"),
    "v3-int8": CONFIGS["c5"].replace(name="deepseek-v3-moe-prefill-int8-w8a8", w_routed="int8", w_shared="int8"),
    "c4-w4a8": CONFIGS["c4"].replace(name="deepseek-v4-pro-moe-decode-w4a8", w_routed="mxfp4a8"),
    "c4-mx": CONFIGS["c4"].replace(name="deepseek-v4-pro-moe-decode-hybrid-mxfp8-mxfp4", w_routed="mxfp4a8",
                                   w_shared="mxfp8a8"),
    "c3-int8": CONFIGS["c3"].replace(name="deepseek-v3-moe-decode-int8-w8a8", w_routed="int8", w_shared="int8"),
}


def workload(name: str) -> LayerSpec:
    return CONFIGS[name] if name in CONFIGS else EXTRA[name]


# ----------------------------------------------------------------------------------------------
# dense draws and stored formats
# ----------------------------------------------------------------------------------------------

def sigma(fan_in: int) -> float:
    return float(np.float32(1.0 / math.sqrt(fan_in)))


def draw_f32(seed: int, tid: int, stream: int, shape, fan_in: int | None = None,
             start: int = 0) -> np.ndarray:
    n = int(np.prod(shape))
    s = 1.0 if fan_in is None else sigma(fan_in)
    return px.normal_f32(seed, tid, stream, start, n, s).reshape(shape)


def store_act(v: np.ndarray, act: str) -> np.ndarray:
    if act == "f32":
        return np.ascontiguousarray(v, np.float32)
    if act == "bf16":
        return px.f32_to_bf16_bits(v)
    raise ValueError(act)


def act_to_f64(v: np.ndarray, act: str) -> np.ndarray:
    if act == "f32":
        return np.asarray(v, np.float32).astype(np.float64)
    return px.bf16_bits_to_f32(v).astype(np.float64)


def store_matrix(w: np.ndarray, fmt: str) -> dict:
    """fp32 W[K, N] -> {'w': codes, 'scale': scales or None} in stored format ``fmt``."""
    if fmt == "f32":
        return {"w": np.ascontiguousarray(w, np.float32), "scale": None}
    if fmt == "bf16":
        return {"w": px.f32_to_bf16_bits(w), "scale": None}
    if fmt == "fp8":
        c, s = px.quantize_fp8_block128(w)
        return {"w": c, "scale": s}
    if fmt in ("mxfp4", "mxfp4a8"):
        c, s = px.quantize_mxfp4_k32(w)
        return {"w": c, "scale": s}
    if fmt == "mxfp8a8":
        c, s = px.quantize_mxfp8_k32(w)
        return {"w": c, "scale": s}
    if fmt == "int8":
        c, s = px.quantize_int8_per_channel(w)
        return {"w": c, "scale": s}
    raise ValueError(fmt)


def expert_weights(spec: LayerSpec, kind: str, e: int) -> dict:
    """Stored gate/up/down of routed expert ``e`` (kind='routed') or the shared expert."""
    tids = TID_ROUTED if kind == "routed" else TID_SHARED
    fmt = spec.w_routed if kind == "routed" else spec.w_shared
    H, I = spec.H, spec.I
    out = {}
    for name, (K, N, fan) in (("gate", (H, I, H)), ("up", (H, I, H)), ("down", (I, H, I))):
        st = store_matrix(draw_f32(spec.seed, tids[name], e, (K, N), fan), fmt)
        out[name] = st["w"]
        out[name + "_scale"] = st["scale"]
    return out


def stack_experts(spec: LayerSpec, experts=None) -> dict:
    """All routed experts stacked along a leading E axis (host memory; small layers only)."""
    experts = range(spec.E) if experts is None else experts
    per = [expert_weights(spec, "routed", e) for e in experts]
    out = {}
    for key in per[0]:
        out[key] = None if per[0][key] is None else np.stack([p[key] for p in per])
    return out


# ----------------------------------------------------------------------------------------------
# router inputs: Wr, bias, x with the margin rule
# ----------------------------------------------------------------------------------------------

def router_matrix(spec: LayerSpec) -> np.ndarray:
    return store_act(draw_f32(spec.seed, TID_WR, 0, (spec.H, spec.E), spec.H), spec.act)


def zipf_targets(E: int, k: int, T: int, alpha: float, order: np.ndarray) -> np.ndarray:
    """Expected assignments per expert: share ~ rank^-alpha, sum = T*k, each <= T (water-fill)."""
    share = np.arange(1, E + 1, dtype=np.float64) ** -alpha
    target = np.zeros(E)
    cap = np.zeros(E, bool)
    total = float(T * k)
    for _ in range(E + 1):
        free = ~cap
        rest = total - T * cap.sum()
        target[free] = rest * share[free] / share[free].sum()
        target[cap] = T
        over = free & (target > T)
        if not over.any():
            break
        cap |= over
    out = np.empty(E)
    out[order] = target  # order[r] = expert with rank r+1
    return out


def zipf_bias(spec: LayerSpec, Wr_stored: np.ndarray, iters: int = 50) -> np.ndarray:
    """Per-expert logit bias giving Zipf(alpha) popularity on a calibration draw.

    The calibration logits are drawn from the distribution of x @ Wr for x ~ N(0, I): a normal
    vector with covariance Wr^T Wr (via its Cholesky factor), so the calibration costs E, not
    H, draws per token. The bias is refined by b <- b + 0.5 (ln(c* + .5) - ln(c + .5)).
    """
    E, k = spec.E, spec.k
    Tc = spec.calib_tokens
    order = np.argsort(px.uniform_words(spec.seed, TID_RANK, 0, 0, E), kind="stable")
    target = zipf_targets(E, k, Tc, spec.zipf_alpha, order)
    W = act_to_f64(Wr_stored, spec.act)
    L = np.linalg.cholesky(W.T @ W)
    G = px.normal_f32(spec.seed, TID_XCAL, 0, 0, Tc * E).reshape(Tc, E).astype(np.float64)
    logits = G @ L.T
    b = np.zeros(E)
    for _ in range(iters):
        sel = np.argpartition(-(logits + b), k - 1, axis=1)[:, :k]
        cnt = np.bincount(sel.reshape(-1), minlength=E)
        b += 0.5 * (np.log(target + 0.5) - np.log(cnt + 0.5))
    b -= b.mean()
    return b.astype(np.float32)


def topk_gap(logits: np.ndarray, k: int) -> np.ndarray:
    """Per row: k-th largest minus (k+1)-th largest value (inf when k == E)."""
    E = logits.shape[1]
    if k >= E:
        return np.full(logits.shape[0], np.inf)
    part = -np.partition(-logits, (k - 1, k), axis=1)
    return part[:, k - 1] - part[:, k]


def activations(spec: LayerSpec, Wr_stored: np.ndarray, bias, max_attempts: int = 256, x0=None):
    """x[T, H] in the act format, with rows redrawn until the router margin holds.

    ``x0`` may hold the attempt-0 draw already (e.g. from the GPU fill, which is bit-identical).
    Returns (x_stored, attempts[T]) where attempts[t] is the stream x[t] finally came from.
    """
    T, H = spec.T, spec.H
    if x0 is None:
        x = store_act(draw_f32(spec.seed, TID_X, 0, (T, H)), spec.act)
    else:
        x = np.array(x0, copy=True)
    attempts = np.zeros(T, np.int32)
    W = act_to_f64(Wr_stored, spec.act)
    b = np.zeros(spec.E) if bias is None else np.asarray(bias, np.float64)
    rows = np.arange(T)
    for a in range(1, max_attempts + 1):
        logits = act_to_f64(x[rows], spec.act) @ W + b
        bad = rows[topk_gap(logits, spec.k) < spec.margin]
        if bad.size == 0:
            return x, attempts
        for t in bad:
            v = draw_f32(spec.seed, TID_X, a, (1, H), start=int(t) * H)
            x[t] = store_act(v, spec.act)[0]
            attempts[t] = a
        rows = bad
    raise RuntimeError("margin rule not met after %d attempts" % max_attempts)


def router_inputs(spec: LayerSpec) -> dict:
    Wr = router_matrix(spec)
    bias = zipf_bias(spec, Wr) if spec.router == "zipf" else None
    x, attempts = activations(spec, Wr, bias)
    return {"x": x, "Wr": Wr, "bias": bias, "attempts": attempts}


# ----------------------------------------------------------------------------------------------
# hash routing inputs
# ----------------------------------------------------------------------------------------------

def hash_inputs(spec: LayerSpec, vocab: int):
    """Token ids uniform in [0, vocab) and a [vocab][k] int32 table of k distinct experts per id.

    Token t's id is word t of stream 0 of (seed, TID_TOKENS) mod vocab; row v of the table takes
    words of stream v of (seed, TID_HASH) mod E in order, skipping experts already in the row.
    """
    ids = (px.uniform_words(spec.seed, TID_TOKENS, 0, 0, spec.T).astype(np.int64) % vocab).astype(np.int32)
    table = np.empty((vocab, spec.k), np.int32)
    for v in range(vocab):
        words = px.uniform_words(spec.seed, TID_HASH, v, 0, 8 * spec.k + 64).astype(np.int64) % spec.E
        row = []
        for e in words:
            if e not in row:
                row.append(int(e))
                if len(row) == spec.k:
                    break
        assert len(row) == spec.k, "hash table row %d: too few distinct draws" % v
        table[v] = row
    return ids, table

