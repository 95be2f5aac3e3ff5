"""CPU oracle for the causal Based forward (2nd-order Taylor linear attention).

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or run this module; only the tests,
the package's smoke check and the benchmark's CPU-baseline leg do. It shares no code with the HIP path.

Source: the page "Write a fast Based (Taylor linear attention) forward kernel" (KBench task spec
`based_forward.py`). Its fields are cited by name:
  * spec_md        - the definition: weights A[i,j] = 1 + s + s^2/2 for j <= i (else 0), s = scale*(q_i . k_j),
                     o_i = sum_j A[i,j] v_j / (sum_j A[i,j] + 1e-6); and the feature-map identity
                     phi(x) = [1, x, x (x) x / sqrt(2)], phi(q).phi(k) = 1 + (q.k) + (q.k)^2 / 2.
  * contract_md    - the default scale is the inverse square root of the key width K; the scale is applied
                     to the query side; the 1e-6 guard goes on after the row sum; the causal sum includes
                     the diagonal.
  * reference_src  - the chunked feature-map algorithm: per chunk, read out with the state of earlier chunks
                     plus the direct polynomial inside the chunk, then fold the chunk into the state.

Three independent routes are provided, all in float64 (or exact rationals):
  based_ref_direct    - the definition written out (library matmul for q.k and A@v).
  based_ref_chunked   - the page's chunked feature-map algorithm, in its order, explicit phi, float64 state.
  based_ref_rational  - the definition in exact rational arithmetic (fractions.Fraction), tiny shapes only.
The chunked route also runs with its state (S, z) carried in and out (`based_ref_chunked_state`), and the
same recurrence one token at a time (`based_ref_decode_step`): the steps on either side of the forward.

Inputs are float arrays already holding bfloat16 values (decode with `bf16_to_f64`), shapes
q, k: (B, T, H, K); v: (B, T, H, V). The result is float64 (B, T, H, V).

Readings taken where the page leaves a step open:
  * scale is rounded to float32 once (the reference multiplies an fp32 tensor by it), then used in float64.
  * the 1e-6 guard is applied in float64 (rational route: exactly 1/10**6).
  * T may be any positive length; the last chunk of the chunked route may be short.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

DEN_GUARD = 1e-6  # contract_md: fixed guard added to the denominator after the row sum


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bfloat16 bit patterns (uint16) exactly: a bfloat16 is the top half of a float32."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def resolve_scale(scale, K: int) -> float:
    """contract_md: no scale given means the inverse square root of the key width K (V does not enter).
    Rounded to float32 once."""
    if scale is None:
        scale = K ** -0.5
    return float(np.float32(scale))


def taylor_weight(s):
    """spec_md: the 2nd-order Taylor expansion of exp(s): 1 + s + s^2/2."""
    return 1.0 + s + 0.5 * s * s


# --------------------------------------------------------------------------------------------------------
# Route 1: the definition (spec_md), O(T^2) per (b, h)
# --------------------------------------------------------------------------------------------------------

def _direct_one_head(Q, Kk, Vv, sigma):
    """All rows of one (b, h): s = sigma * Q K^T, A = taylor(s) masked to j <= i, o = A V / (rowsum A + 1e-6)."""
    T = Q.shape[0]
    s = sigma * (Q @ Kk.T)
    A = taylor_weight(s)
    A = np.where(np.tri(T, T, dtype=bool), A, 0.0)  # causal, diagonal included (contract_md)
    num = A @ Vv
    den = A.sum(axis=1)
    return num / (den + DEN_GUARD)[:, None]


def based_ref_direct(q, k, v, scale=None):
    """The definition of spec_md, evaluated row by row in float64 for every (b, h)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, T, H, K = q.shape
    V = v.shape[-1]
    sigma = resolve_scale(scale, K)
    o = np.empty((B, T, H, V), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            o[b, :, h, :] = _direct_one_head(q[b, :, h, :], k[b, :, h, :], v[b, :, h, :], sigma)
    return o


def based_ref_direct_rows(q, k, v, scale, b: int, h: int, rows):
    """The same definition for selected output rows t of one (b, h): only j <= t enters row t.

    Used where a full O(T^2) evaluation would not finish in seconds (long sequences): each requested row is
    computed on its own from the inputs, so a sample of rows can be checked one by one.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    K = q.shape[-1]
    sigma = resolve_scale(scale, K)
    out = np.empty((len(rows), v.shape[-1]), dtype=np.float64)
    for n, t in enumerate(rows):
        t = int(t)
        qt = q[b, t, h, :].astype(np.float64)
        Kp = k[b, : t + 1, h, :].astype(np.float64)
        Vp = v[b, : t + 1, h, :].astype(np.float64)
        s = sigma * (Kp @ qt)
        A = taylor_weight(s)
        out[n] = (A @ Vp) / (A.sum() + DEN_GUARD)
    return out


# --------------------------------------------------------------------------------------------------------
# Route 2: the chunked feature-map algorithm (reference_src), float64 state
# --------------------------------------------------------------------------------------------------------

def phi(x):
    """spec_md: phi(x) = [1, x, vec(x (x) x) / sqrt(2)], length P = 1 + K + K*K, quadratic block row-major
    (entry a*K + b holds x_a x_b / sqrt(2)). x has shape (..., K)."""
    x = np.asarray(x, dtype=np.float64)
    K = x.shape[-1]
    ones = np.ones(x.shape[:-1] + (1,), dtype=np.float64)
    quad = (x[..., :, None] * x[..., None, :]).reshape(x.shape[:-1] + (K * K,)) / np.sqrt(2.0)
    return np.concatenate([ones, x, quad], axis=-1)


def feature_dim(K: int) -> int:
    """P = 1 + K + K*K, the length of phi(x) (spec_md)."""
    return 1 + K + K * K


def based_ref_chunked(q, k, v, scale=None, chunk: int = 256):
    """The chunked feature-map algorithm (reference_src) from empty sums, chunks of `chunk` tokens, every
    quantity float64: `based_ref_chunked_state` with no earlier tokens."""
    o, _ = based_ref_chunked_state(q, k, v, scale, None, chunk)
    return o


class _Carry:
    """The running sums of one (b, h) pair over the tokens already seen (reference_src's state): S = sum of
    phi(k_j) v_j^T (P x V) and z = sum of phi(k_j) (length P), in the layout of `phi`."""

    def __init__(self, S, z):
        self.S = np.array(S, dtype=np.float64)
        self.z = np.array(z, dtype=np.float64)

    def read(self, feats):
        """Numerator rows feats @ S and denominators feats @ z for feature rows `feats` (n x P)."""
        return feats @ self.S, feats @ self.z

    def fold(self, feats, values):
        """Add tokens with feature rows `feats` (n x P) and value rows `values` (n x V)."""
        self.S += feats.T @ values
        self.z += feats.sum(axis=0)


def based_ref_chunked_state(q, k, v, scale=None, state=None, chunk: int = 256):
    """The chunked feature-map algorithm of reference_src with its state carried across the call boundary.

    Each (b, h) pair is walked chunk by chunk. A chunk's outputs take the tokens before it through the
    carried sums (phi of the scaled queries against S and z) and the tokens inside it directly through the
    causal Taylor weights (diagonal included); then the chunk is folded into the sums. `state` = (S0, z0) of
    shapes (B, H, P, V) and (B, H, P), in the layout of `phi` (k unscaled, the scale being on the query side,
    contract_md), stands for tokens that came before this call; None means no earlier tokens. Returns
    (o, (S, z)) with the sums after the last token, so a sequence processed in pieces, each starting from the
    sums the previous piece returned, gives the same outputs as one call over the whole sequence."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, T, H, K = q.shape
    V = v.shape[-1]
    P = feature_dim(K)
    sigma = resolve_scale(scale, K)
    if state is None:
        S0, z0 = np.zeros((B, H, P, V)), np.zeros((B, H, P))
    else:
        S0 = np.asarray(state[0], dtype=np.float64).reshape(B, H, P, V)
        z0 = np.asarray(state[1], dtype=np.float64).reshape(B, H, P)
    o = np.empty((B, T, H, V))
    S_end, z_end = np.empty((B, H, P, V)), np.empty((B, H, P))
    for b in range(B):
        for h in range(H):
            carry = _Carry(S0[b, h], z0[b, h])
            for lo in range(0, T, chunk):
                hi = min(T, lo + chunk)
                qs = sigma * q[b, lo:hi, h]                      # scaled queries of the chunk (contract_md)
                kc, vc = k[b, lo:hi, h], v[b, lo:hi, h]
                numer, denom = carry.read(phi(qs))               # the tokens before the chunk
                w = np.tril(taylor_weight(qs @ kc.T))            # the chunk itself: row t sees keys j <= t
                numer = numer + w @ vc
                denom = denom + w.sum(axis=1)
                o[b, lo:hi, h] = numer / (denom + DEN_GUARD)[:, None]
                carry.fold(phi(kc), vc)
            S_end[b, h], z_end[b, h] = carry.S, carry.z
    return o, (S_end, z_end)


def based_ref_decode_step(q1, k1, v1, state, scale=None):
    """One token of the same recurrence: q1, k1 of shape (B, H, K) and v1 of shape (B, H, V) are the next
    token of every (b, h); state = (S, z) as in `based_ref_chunked_state`. The token is folded into the sums
    first (the diagonal j = i is part of the causal sum, contract_md), then read out:
    o = phi(scale q) S' / (phi(scale q) z' + 1e-6). Returns (o of shape (B, H, V), (S', z'))."""
    q1 = np.asarray(q1, dtype=np.float64)
    k1 = np.asarray(k1, dtype=np.float64)
    v1 = np.asarray(v1, dtype=np.float64)
    B, H, K = q1.shape
    sigma = resolve_scale(scale, K)
    S = np.array(state[0], dtype=np.float64)
    z = np.array(state[1], dtype=np.float64)
    o = np.empty(v1.shape)
    for b in range(B):
        for h in range(H):
            carry = _Carry(S[b, h], z[b, h])
            carry.fold(phi(k1[b, h])[None, :], v1[b, h][None, :])
            numer, denom = carry.read(phi(sigma * q1[b, h])[None, :])
            o[b, h] = numer[0] / (denom[0] + DEN_GUARD)
            S[b, h], z[b, h] = carry.S, carry.z
    return o, (S, z)


# --------------------------------------------------------------------------------------------------------
# Route 3: the definition in exact rationals (tiny shapes)
# --------------------------------------------------------------------------------------------------------

def based_ref_rational(q, k, v, scale=None):
    """Exact evaluation of spec_md with fractions.Fraction. bfloat16 values are dyadic rationals, the
    float32 scale is a dyadic rational and the guard is exactly 1/10**6, so the result is the true value of
    the definition for these inputs. Returns a nested list [b][t][h][v] of Fractions."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, T, H, K = q.shape
    V = v.shape[-1]
    sigma = Fraction(resolve_scale(scale, K))
    guard = Fraction(1, 10 ** 6)
    F = np.vectorize(Fraction, otypes=[object])
    qf, kf, vf = F(q), F(k), F(v)
    out = [[[[None] * V for _ in range(H)] for _ in range(T)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            for t in range(T):
                num = [Fraction(0)] * V
                den = Fraction(0)
                for j in range(t + 1):
                    s = sigma * sum(qf[b, t, h, a] * kf[b, j, h, a] for a in range(K))
                    A = 1 + s + s * s / 2
                    den += A
                    for c in range(V):
                        num[c] += A * vf[b, j, h, c]
                for c in range(V):
                    out[b][t][h][c] = num[c] / (den + guard)
    return out


def rational_to_f64(r) -> np.ndarray:
    return np.array([[[[float(x) for x in row] for row in th] for th in bt] for bt in r], dtype=np.float64)


# --------------------------------------------------------------------------------------------------------
# The acceptance gate
# --------------------------------------------------------------------------------------------------------

MAX_ABS_TOL = 2e-2   # max-abs error bound for bfloat16 inputs against the float32-or-better oracle
REL_L2_TOL = 5e-3    # relative-L2 (Frobenius over the whole output tensor) bound


def errors(o, ref):
    """Return (max |o - ref|, ||o - ref||_2 / ||ref||_2), both in float64 over the whole tensor."""
    o = np.asarray(o, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = o - ref
    max_abs = float(np.max(np.abs(d))) if d.size else 0.0
    nref = float(np.linalg.norm(ref.ravel()))
    rel = float(np.linalg.norm(d.ravel()) / nref) if nref > 0 else float(np.linalg.norm(d.ravel()))
    return max_abs, rel


def passes_gate(o, ref) -> bool:
    max_abs, rel = errors(o, ref)
    return max_abs <= MAX_ABS_TOL and rel <= REL_L2_TOL
