"""Operand-precision study for the Based forward: would fp8 MFMA operands hold the accuracy gate?

TEST INFRASTRUCTURE ONLY (a numerical study, like the rest of oracle/): nothing on the product path imports
it. It answers the question the page "Write a fast Based (Taylor linear attention) forward kernel" leaves
open in field precision_md (fp8 is allowed wherever the tolerance still holds) before any fp8 kernel is
written.

`emulate_forward` re-evaluates the chunked feature-map algorithm of field reference_src with the operands
of each of its three products rounded to a chosen format, the way a matrix-core kernel would feed them:
  * "intra"   - the causal Taylor weights A and the values v of a chunk (A [v | 1]);
  * "readout" - phi(scale q) and the state (S, z) of earlier chunks (phi(q) [S | z]);
  * "update"  - phi(k) and the values v folded into the state (phi(k)^T [v | 1]).
Products are accumulated exactly (float64, standing in for the fp32 accumulators), the state is kept in
float64 between chunks, and every operand block of 32 contraction entries gets a power-of-two scale that
puts its largest magnitude at the top of the format (per-block scaling as the fp8 MFMA forms allow).
The ones column of the normaliser is exact in every format. Formats: "f64" (no rounding), "bf16"
(8 significant bits), "e4m3" (OCP fp8: 4 significant bits, largest 448, subnormals from 2^-9) and "e5m2"
(3 significant bits, largest 57344, subnormals from 2^-16). Rounding is to nearest, ties to even.
"""
from __future__ import annotations

import numpy as np

from .based_oracle import DEN_GUARD, phi, resolve_scale, taylor_weight

FORMATS = {
    # name: (significant bits, smallest normal exponent, largest finite value)
    "bf16": (8, -126, 3.3895313892515355e38),
    "e4m3": (4, -6, 448.0),
    "e5m2": (3, -14, 57344.0),
}


def round_to_format(x, fmt: str):
    """Round to the nearest value of the format (ties to even); saturate at its largest finite value."""
    x = np.asarray(x, dtype=np.float64)
    if fmt == "f64":
        return x.copy()
    bits, emin, fmax = FORMATS[fmt]
    a = np.abs(x)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, emin)                    # below the smallest normal: fixed spacing (subnormals)
    ulp = np.exp2(e - (bits - 1))
    r = np.round(x / ulp) * ulp                # numpy rounds half to even
    return np.clip(r, -fmax, fmax)


def _blocks_scaled(x, fmt: str, axis: int, block: int = 32):
    """Round x with one power-of-two scale per block of `block` entries along `axis` (the contraction axis)
    and per position of every other axis, so that each block's largest magnitude lands in the top binade."""
    if fmt in ("f64", "bf16"):
        return round_to_format(x, fmt)
    x = np.moveaxis(np.asarray(x, dtype=np.float64), axis, -1)
    n = x.shape[-1]
    pad = (-n) % block
    xp = np.concatenate([x, np.zeros(x.shape[:-1] + (pad,))], axis=-1) if pad else x
    xb = xp.reshape(xp.shape[:-1] + (-1, block))
    amax = np.max(np.abs(xb), axis=-1, keepdims=True)
    fmax = FORMATS[fmt][2]
    scale = np.exp2(np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - np.floor(np.log2(fmax)))
    yb = round_to_format(xb / scale, fmt) * scale
    y = yb.reshape(xp.shape)[..., :n]
    return np.moveaxis(y, -1, axis)


def _features_rounded(f, fmt: str, feat_axis: int, contract_axis: int, block: int, K: int, quad_only: bool):
    """phi features (along feat_axis) rounded as a product operand with scale blocks along contract_axis;
    with quad_only the constant and linear features (the first 1 + K, whose range differs from the
    quadratic block's) stay bf16."""
    if not quad_only:
        return _blocks_scaled(f, fmt, contract_axis, block)
    f = np.asarray(f, dtype=np.float64)
    n = f.ndim
    fa = feat_axis % n
    ca = contract_axis % n
    idx = [slice(None)] * n
    idx[fa] = slice(0, 1 + K)
    head = round_to_format(f[tuple(idx)], "bf16")
    idx[fa] = slice(1 + K, None)
    quad = _blocks_scaled(f[tuple(idx)], fmt, ca, block)
    return np.concatenate([head, quad], axis=fa)


def emulate_forward(q, k, v, scale=None, chunk: int = 128, intra="bf16", readout="bf16", update="bf16",
                    block: int = 32, quad_only: bool = False):
    """The chunked algorithm with rounded operands (see the module text). Inputs as for the oracle routes:
    float arrays holding bf16 values, q, k (B, T, H, K), v (B, T, H, V). `block` is the number of
    contraction entries per scale; with quad_only only the quadratic feature block of phi(q) and phi(k) (and
    the matching rows of S) take the read-out's and update's format. Returns o (B, T, H, V) float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, T, H, K = q.shape
    V = v.shape[-1]
    P = 1 + K + K * K
    sigma = resolve_scale(scale, K)
    qh = np.transpose(q, (0, 2, 1, 3)) * sigma
    kh = np.transpose(k, (0, 2, 1, 3))
    vh = np.transpose(v, (0, 2, 1, 3))
    S = np.zeros((B, H, P, V))
    z = np.zeros((B, H, P))
    tri = np.tri(chunk, chunk)
    o = np.empty((B, H, T, V))
    for i in range(0, T, chunk):
        qc, kc, vc = qh[:, :, i:i + chunk], kh[:, :, i:i + chunk], vh[:, :, i:i + chunk]
        n = qc.shape[2]
        # read-out of earlier chunks: phi(q) against [S | z], contraction over the P features
        pq = _features_rounded(phi(qc), readout, -1, -1, block, K, quad_only)
        Sq = _features_rounded(S, readout, -2, -2, block, K, quad_only)
        zq = _features_rounded(z, readout, -1, -1, block, K, quad_only)
        num = pq @ Sq
        den = np.einsum("bhnp,bhp->bhn", pq, zq)
        # inside the chunk: the Taylor weights against [v | 1], contraction over the keys
        A = taylor_weight(qc @ np.swapaxes(kc, -1, -2)) * tri[:n, :n]
        Aq = _blocks_scaled(A, intra, axis=-1, block=block)
        vq = _blocks_scaled(vc, intra, axis=-2, block=block)
        num = num + Aq @ vq
        den = den + Aq.sum(-1)
        o[:, :, i:i + n] = num / (den + DEN_GUARD)[..., None]
        # fold the chunk into the state: phi(k)^T [v | 1], contraction over the chunk's tokens
        pk = _features_rounded(phi(kc), update, -1, -2, block, K, quad_only)
        vu = _blocks_scaled(vc, update, axis=-2, block=block)
        S = S + np.swapaxes(pk, -1, -2) @ vu
        z = z + pk.sum(axis=2)
    return np.ascontiguousarray(np.transpose(o, (0, 2, 1, 3)))


VARIANTS = (
    ("bf16 everywhere (the kernels)", dict(intra="bf16", readout="bf16", update="bf16")),
    ("e4m3 intra only", dict(intra="e4m3", readout="bf16", update="bf16")),
    ("e4m3 read-out only", dict(intra="bf16", readout="e4m3", update="bf16")),
    ("e4m3 update only", dict(intra="bf16", readout="bf16", update="e4m3")),
    ("e4m3 everywhere", dict(intra="e4m3", readout="e4m3", update="e4m3")),
    ("e5m2 everywhere", dict(intra="e5m2", readout="e5m2", update="e5m2")),
    # narrower ranges: one scale per 8 contraction entries, or fp8 only for the quadratic feature block
    ("e4m3 intra only, 8-entry scales", dict(intra="e4m3", readout="bf16", update="bf16", block=8)),
    ("e4m3 read-out only, 8-entry scales", dict(intra="bf16", readout="e4m3", update="bf16", block=8)),
    ("e4m3 read-out, quadratic features only", dict(intra="bf16", readout="e4m3", update="bf16", quad_only=True)),
    ("e4m3 update, quadratic features only", dict(intra="bf16", readout="bf16", update="e4m3", quad_only=True)),
)


def study(B=1, T=2048, H=2, K=16, V=64, seed=2):
    """Errors of every variant against the direct definition (fp64) on N(0, 1) bf16 inputs."""
    from taylor_feature_map_amd.inputs import make_qkv

    from .based_oracle import based_ref_direct, bf16_to_f64, errors
    qb, kb, vb = make_qkv(B, T, H, K, V, seed)
    q, k, v = bf16_to_f64(qb), bf16_to_f64(kb), bf16_to_f64(vb)
    ref = based_ref_direct(q, k, v)
    rows = []
    for name, kw in VARIANTS:
        o = emulate_forward(q, k, v, None, 128, **kw)
        o = round_to_format(o, "bf16")  # bf16 output, as the benchmark workloads
        m, r = errors(o, ref)
        rows.append((name, m, r))
    return rows


if __name__ == "__main__":
    import sys
    T = int(sys.argv[1]) if len(sys.argv) > 1 else 2048
    for name, m, r in study(T=T):
        print(f"{name:32s} max_abs {m:.3e}  rel_l2 {r:.3e}  {'passes' if m <= 2e-2 and r <= 5e-3 else 'FAILS'} the gate")
