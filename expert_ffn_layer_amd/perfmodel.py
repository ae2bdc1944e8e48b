"""Algorithmic bytes and FLOPs of one MoE expert-FFN layer (host-side closed forms).

These are the quantities the roofline is priced with: the bytes the method must move and the
FLOPs it must do, independent of how a kernel moves them.

* An expert is three matrices, H x I each (gate, up, down): 3 H I parameters
  (Chapter 6 'Supernodes', section 6.2.6; 'DeepSeek-V4-Pro on NVIDIA H200', section 3.2).
* One (token, expert) pair costs 6 H I FLOPs: two FLOPs per multiply-add over the three
  matrices ('DeepSeek-V4-Pro on NVIDIA H200', section 3.2).
* Within one batch every selected expert's weights are read from HBM once, so the weight
  bytes are the sum over the experts at least one token selected (Chapter 6, section 6.3.2).
* The roofline time is max(F/P, V/B) (Chapter 6, eq. (6-2)).
* With independent uniform choices the expected number of active experts is
  E (1 - (1 - k/E)^m) (Chapter 6, eq. (6-8)); the V4 report uses E (1 - (1 - 1/E)^(k B))
  (section 3.2).
"""
from __future__ import annotations

# bytes per parameter of each stored format, and bytes of block scales per parameter
PARAM_BYTES = {"f32": 4.0, "bf16": 2.0, "fp8": 1.0, "mxfp4": 0.5, "mxfp4a8": 0.5, "mxfp8a8": 1.0, "int8": 1.0}
ACT_BYTES = {"f32": 4, "bf16": 2}


def expert_params(H: int, I: int) -> int:
    return 3 * H * I


def matrix_bytes(K: int, N: int, fmt: str) -> int:
    """Stored bytes of one K x N matrix, including its block scales."""
    if fmt == "f32":
        return 4 * K * N
    if fmt == "bf16":
        return 2 * K * N
    if fmt == "fp8":  # one fp32 scale per 128 x 128 block
        return K * N + 4 * (K // 128) * (N // 128)
    if fmt in ("mxfp4", "mxfp4a8"):  # one e8m0 byte per 32 K-elements of a column (W4A8 stores MXFP4)
        return K * N // 2 + (K // 32) * N
    if fmt == "mxfp8a8":  # E4M3FN codes + one e8m0 byte per 32 K-elements of a column
        return K * N + (K // 32) * N
    if fmt == "int8":  # int8 codes + one fp32 scale per output column
        return K * N + 4 * N
    raise ValueError(fmt)


def expert_bytes(H: int, I: int, fmt: str) -> int:
    return 2 * matrix_bytes(H, I, fmt) + matrix_bytes(I, H, fmt)


def pair_flops(H: int, I: int) -> int:
    return 6 * H * I


def expected_active(E: int, k: int, m: int) -> float:
    """Expected number of experts some token of a batch of m selects (eq. (6-8))."""
    return E * (1.0 - (1.0 - k / E) ** m)


def touched_experts(E: int, k: int, B: int) -> float:
    """The V4 report's U(B) = E (1 - (1 - 1/E)^(k B))."""
    return E * (1.0 - (1.0 - 1.0 / E) ** (k * B))


def roofline_time(flops: float, peak_flops: float, bytes_: float, bw: float) -> float:
    return max(flops / peak_flops, bytes_ / bw)


def layer_traffic(spec, counts) -> dict:
    """Algorithmic bytes and FLOPs of one layer call, given the per-expert row counts.

    Bytes: active routed experts' weights (with scales), the shared expert, the router matrix,
    x read once, y written once, and the routing result (int32 index + fp32 weight per pair).
    FLOPs: 6 H I per (token, expert) pair, 6 H I per token for the shared expert, and
    2 H E per token for the router scores.
    """
    T, H, E, k, I = spec.T, spec.H, spec.E, spec.k, spec.I
    a = ACT_BYTES[spec.act]
    active = int(sum(1 for c in counts if c > 0))
    w_routed = active * expert_bytes(H, I, spec.w_routed)
    w_shared = expert_bytes(H, I, spec.w_shared) if spec.shared else 0
    other = a * H * E + 2 * a * T * H + 8 * T * k
    flops = 6 * H * I * T * k + (6 * H * I * T if spec.shared else 0) + 2 * T * H * E
    return {
        "active_experts": active,
        "weight_bytes": w_routed + w_shared,
        "other_bytes": other,
        "bytes": w_routed + w_shared + other,
        "flops": flops,
    }
