"""GPU parity of the state carried in and out of the forward and of the one-token recurrent step, against
the CPU oracle's state-carrying route (reference_src of the page "Write a fast Based (Taylor linear
attention) forward kernel", run in pieces) and the definition (spec_md).

Outputs use the forward's gate (max-abs 2e-2 and relative-L2 5e-3). A state is compared with relative-L2
5e-3 and max-abs 5e-3 of its largest entry: its entries grow with the number of tokens (the constant
feature of z counts them), so an absolute bound would mean different things at different lengths, and
the kernels accumulate bf16 products of phi(k) and v in fp32 as the forward does.
"""
import numpy as np
import pytest

from oracle import (MAX_ABS_TOL, REL_L2_TOL, based_ref_chunked_state, based_ref_decode_step, based_ref_direct,
                    bf16_to_f64, errors)
from taylor_feature_map_amd.inputs import make_qkv

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(_dev())


def _f32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(_dev())


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


def _gate(o, ref, what):
    m, r = errors(o, ref)
    print(f"{what}: max_abs={m:.3e} rel_l2={r:.3e}", flush=True)
    assert m <= MAX_ABS_TOL and r <= REL_L2_TOL, what


def _state_gate(st, ref, what):
    for name, a, b in (("S", st[0], ref[0]), ("z", st[1], ref[1])):
        m, r = errors(a, b)
        scale = float(np.max(np.abs(b)))
        print(f"{what} {name}: max_abs={m:.3e} (of {scale:.3e}) rel_l2={r:.3e}", flush=True)
        assert r <= 5e-3 and m <= 5e-3 * scale, f"{what} {name}"


@pytest.mark.parametrize("B,T,H,K,V", [(2, 777, 2, 16, 64), (1, 300, 3, 8, 128), (1, 5000, 1, 16, 64),
                                       (1, 1, 2, 16, 64), (1, 2100, 1, 8, 64)])
def test_final_state_matches_oracle(B, T, H, K, V):
    """State after the last token (ragged last chunk, several or many segments, a single token)."""
    from taylor_feature_map_amd import based_forward
    qb, kb, vb = make_qkv(B, T, H, K, V, seed=T + K)
    q, k, v = bf16_to_f64(qb), bf16_to_f64(kb), bf16_to_f64(vb)
    o_ref, st_ref = based_ref_chunked_state(q, k, v, None, None, chunk=256)
    o, (S, z) = based_forward(_to_dev(qb), _to_dev(kb), _to_dev(vb), return_state=True, out_dtype=torch.float32)
    torch.cuda.synchronize()
    _gate(_np(o), o_ref, f"o B{B} T{T} H{H} K{K} V{V}")
    _state_gate((_np(S), _np(z)), st_ref, f"state B{B} T{T} H{H} K{K} V{V}")


@pytest.mark.parametrize("K,V,T,cuts", [(16, 64, 777, [300]), (8, 128, 1000, [1, 450]), (16, 64, 5000, [2600])])
def test_split_and_carry(K, V, T, cuts):
    """Pieces of a sequence, each started from the state the previous piece returned, give the outputs of
    the definition on the whole sequence and the whole sequence's final state."""
    from taylor_feature_map_amd import based_forward
    B, H = 1, 2
    qb, kb, vb = make_qkv(B, T, H, K, V, seed=7 * K + T)
    q, k, v = bf16_to_f64(qb), bf16_to_f64(kb), bf16_to_f64(vb)
    o_ref, st_ref = based_ref_chunked_state(q, k, v, None, None, chunk=256)
    state, outs = None, []
    bounds = [0] + cuts + [T]
    for a, b in zip(bounds[:-1], bounds[1:]):
        sl = slice(a, b)
        o, state = based_forward(_to_dev(qb[:, sl]), _to_dev(kb[:, sl]), _to_dev(vb[:, sl]), initial_state=state,
                                 return_state=True, out_dtype=torch.float32)
        outs.append(_np(o))
    torch.cuda.synchronize()
    _gate(np.concatenate(outs, axis=1), o_ref, f"carried K{K} V{V} T{T} cuts{cuts}")
    _state_gate((_np(state[0]), _np(state[1])), st_ref, f"carried state K{K} V{V} T{T}")


def test_state_in_and_out_with_split_state_pass():
    """An automatic plan whose state pass sums each segment in two pieces (K = 8, V = 128, 128 heads,
    T = 4096: two segments of 2048 tokens, 256 state workgroups) with a state carried in and out; outputs
    and final states of six heads against the oracle started from the same state."""
    from taylor_feature_map_amd import based_forward, plan
    B, T, H, K, V = 1, 4096, 128, 8, 128
    G, L, ws = plan(B, T, H, K, V)
    slot_bytes = 3 * ((V // 16) * 4 * 64 // 2 + 16) * 4
    assert (G, L) == (2, 2048) and ws == B * H * (G - 1) * 2 * slot_bytes, "two pieces per segment"
    T0 = 300
    qb, kb, vb = make_qkv(B, T0 + T, H, K, V, seed=4242)
    q, k, v = bf16_to_f64(qb), bf16_to_f64(kb), bf16_to_f64(vb)
    _, st0 = based_ref_chunked_state(q[:, :T0], k[:, :T0], v[:, :T0], None, None)
    o, (S, z) = based_forward(_to_dev(qb[:, T0:]), _to_dev(kb[:, T0:]), _to_dev(vb[:, T0:]),
                              initial_state=(_f32(st0[0]), _f32(st0[1])), return_state=True,
                              out_dtype=torch.float32)
    torch.cuda.synchronize()
    heads = [0, 1, 37, 64, 101, 127]
    o_ref, st_ref = based_ref_chunked_state(q[:, T0:, heads], k[:, T0:, heads], v[:, T0:, heads], None,
                                            (st0[0][:, heads], st0[1][:, heads]))
    _gate(_np(o)[:, :, heads], o_ref, "split state pass, state in and out")
    _state_gate((_np(S)[:, heads], _np(z)[:, heads]), st_ref, "split state pass, final state")


@pytest.mark.parametrize("K,V", [(16, 64), (8, 64)])
def test_initial_state_only_symmetric_part_counts(K, V):
    """An antisymmetric matrix added to the quadratic block of the initial state changes no output."""
    from taylor_feature_map_amd import based_forward
    B, T, H = 1, 400, 2
    qb, kb, vb = make_qkv(B, T, H, K, V, seed=40 + K)
    q, k, v = bf16_to_f64(qb), bf16_to_f64(kb), bf16_to_f64(vb)
    _, st = based_ref_chunked_state(q[:, :150], k[:, :150], v[:, :150], None, None)
    o_ref, _ = based_ref_chunked_state(q[:, 150:], k[:, 150:], v[:, 150:], None, st)
    rng = np.random.default_rng(1)
    M = rng.standard_normal((B, H, K, K, V))
    S0 = st[0].copy()
    S0[:, :, 1 + K:] += (M - np.swapaxes(M, 2, 3)).reshape(B, H, K * K, V)
    o = based_forward(_to_dev(qb[:, 150:]), _to_dev(kb[:, 150:]), _to_dev(vb[:, 150:]),
                      initial_state=(_f32(S0), _f32(st[1])), out_dtype=torch.float32)
    torch.cuda.synchronize()
    _gate(_np(o), o_ref, f"antisymmetric initial state K{K}")


@pytest.mark.parametrize("K,V,out_dtype", [(16, 64, torch.float32), (8, 128, torch.bfloat16)])
def test_prefill_then_decode_steps(K, V, out_dtype):
    """Prefill on the GPU with the state carried out, then one decode step per token: every output equals
    the definition on the whole sequence, and the final state the oracle's."""
    from taylor_feature_map_amd import based_decode_step, based_forward
    B, T, H, T0 = 2, 300, 3, 260
    qb, kb, vb = make_qkv(B, T, H, K, V, seed=K + V)
    q, k, v = bf16_to_f64(qb), bf16_to_f64(kb), bf16_to_f64(vb)
    whole = based_ref_direct(q, k, v)
    _, st_ref = based_ref_chunked_state(q, k, v, None, None)
    o, state = based_forward(_to_dev(qb[:, :T0]), _to_dev(kb[:, :T0]), _to_dev(vb[:, :T0]), return_state=True,
                             out_dtype=out_dtype)
    outs = [_np(o)]
    for t in range(T0, T):
        o1 = based_decode_step(_to_dev(qb[:, t]), _to_dev(kb[:, t]), _to_dev(vb[:, t]), state, out_dtype=out_dtype)
        outs.append(_np(o1)[:, None])
    torch.cuda.synchronize()
    _gate(np.concatenate(outs, axis=1), whole, f"prefill+decode K{K} V{V}")
    _state_gate((_np(state[0]), _np(state[1])), st_ref, f"decode state K{K} V{V}")


def test_decode_from_empty_state_matches_oracle_step():
    from taylor_feature_map_amd import based_decode_step, feature_dim
    B, H, K, V = 3, 5, 16, 128
    P = feature_dim(K)
    qb, kb, vb = make_qkv(B, 4, H, K, V, seed=9)
    q, k, v = bf16_to_f64(qb), bf16_to_f64(kb), bf16_to_f64(vb)
    st = (np.zeros((B, H, P, V)), np.zeros((B, H, P)))
    state = (_f32(st[0]), _f32(st[1]))
    for t in range(4):
        o_ref, st = based_ref_decode_step(q[:, t], k[:, t], v[:, t], st, 0.3)
        o = based_decode_step(_to_dev(qb[:, t]), _to_dev(kb[:, t]), _to_dev(vb[:, t]), state, 0.3,
                              out_dtype=torch.float32)
        torch.cuda.synchronize()
        _gate(_np(o), o_ref, f"decode step {t}")
    _state_gate((_np(state[0]), _np(state[1])), st, "decode state")


@pytest.mark.parametrize("K,V", [(16, 512), (8, 320)])
def test_decode_steps_many_value_blocks(K, V):
    """Decode steps with many 64-column blocks per (b, h) (the kernel's partial numerators alternate between
    two LDS buffers, so eight and five blocks reuse each several times), from a state carried in from a
    prefix, against the oracle's steps."""
    from taylor_feature_map_amd import based_decode_step
    B, H, T0, steps = 2, 3, 40, 3
    qb, kb, vb = make_qkv(B, T0 + steps, H, K, V, seed=K * V)
    q, k, v = bf16_to_f64(qb), bf16_to_f64(kb), bf16_to_f64(vb)
    _, st = based_ref_chunked_state(q[:, :T0], k[:, :T0], v[:, :T0], None, None)
    state = (_f32(st[0]), _f32(st[1]))
    for t in range(T0, T0 + steps):
        o_ref, st = based_ref_decode_step(q[:, t], k[:, t], v[:, t], st, None)
        o = based_decode_step(_to_dev(qb[:, t]), _to_dev(kb[:, t]), _to_dev(vb[:, t]), state,
                              out_dtype=torch.float32)
        torch.cuda.synchronize()
        print(f"decode K{K} V{V} step {t}", flush=True)
        _gate(_np(o), o_ref, f"decode K{K} V{V} step {t}")
    _state_gate((_np(state[0]), _np(state[1])), st, f"decode state K{K} V{V}")


def test_decode_step_at_benchmark_batch():
    """The decode step at the batch the bench times (B = 64, H = 16, K = 16, V = 64: 1024 workgroups), from
    the state of a 4-token prefix, checked on every (b, h) pair against the oracle's step: the outputs and
    the updated state and normaliser."""
    from taylor_feature_map_amd import based_decode_step
    B, H, K, V, T0 = 64, 16, 16, 64, 4
    qb, kb, vb = make_qkv(B, T0 + 1, H, K, V, seed=4242)
    q, k, v = bf16_to_f64(qb), bf16_to_f64(kb), bf16_to_f64(vb)
    _, st = based_ref_chunked_state(q[:, :T0], k[:, :T0], v[:, :T0], None, None)
    state = (_f32(st[0]), _f32(st[1]))
    o = based_decode_step(_to_dev(qb[:, T0]), _to_dev(kb[:, T0]), _to_dev(vb[:, T0]), state, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, st_new = based_ref_decode_step(q[:, T0], k[:, T0], v[:, T0], st, None)
    print(f"decode B{B} H{H}: all {B * H} pairs", flush=True)
    _gate(_np(o), o_ref, "decode step at the benchmark batch")
    _state_gate((_np(state[0]), _np(state[1])), st_new, "decode state at the benchmark batch")
