"""Seeded random shapes through every entry point (MI355X).

Each case draws its shape, scale and output type from its own seed and takes one of four routes: the
default plan; a forced segment length (often more than 16 segments, which adds the scan kernel); a
sequence cut at a random token with the state carried from the first piece into the second; or decode
steps after a prefill state. Forwards run twice and must repeat bit for bit. Gate: max-abs 2e-2 and
relative-L2 5e-3 against the oracle (the page "Write a fast Based (Taylor linear attention) forward
kernel", field correctness_md); states within 5e-3 relative to their largest entry. The forward routes
draw shapes up to the size of those that showed the fp32 store overwrite: a build without the wait states
after wide stores fails four of the cases.
"""
import numpy as np
import pytest

from oracle import (MAX_ABS_TOL, REL_L2_TOL, based_ref_chunked, based_ref_chunked_state, based_ref_decode_step,
                    bf16_to_f64, errors)
from taylor_feature_map_amd.inputs import make_qkv

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

N_CASES = 32


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _to(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(_dev())


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


def _gate(o, ref, what):
    m, r = errors(o, ref)
    print(f"{what}: max_abs={m:.3e} rel_l2={r:.3e}", flush=True)
    assert np.isfinite(o).all() and m <= MAX_ABS_TOL and r <= REL_L2_TOL, (what, m, r)


def _state_gate(a, b, what):
    m, r = errors(a, b)
    assert r <= 5e-3 and m <= 5e-3 * float(np.max(np.abs(b))), (what, m, r)


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_case(case):
    from taylor_feature_map_amd import based_decode_step, based_forward, plan
    rng = np.random.default_rng(9000 + case)
    route = ("default", "segments", "state", "decode")[case % 4]
    K = int(rng.choice([8, 16]))
    V = int(rng.choice([64, 128, 192, 256, 320, 512]))
    scale = None if rng.random() < 0.5 else float(rng.uniform(-0.6, 0.6))
    out = torch.float32 if rng.random() < 0.5 else torch.bfloat16
    cap = 12_000_000 if route in ("default", "segments") else 2_500_000
    while True:
        B = int(rng.integers(1, 9))
        H = int(rng.choice([1, 2, 3, 4, 6, 8, 16]))
        T = int(rng.integers(2, 3000))
        if B * H * T * V <= cap:
            break
    what = f"case {case} {route}: B{B} T{T} H{H} K{K} V{V} scale={scale} out={out}"
    qb, kb, vb = make_qkv(B, T, H, K, V, seed=9000 + case)
    q, k, v = bf16_to_f64(qb), bf16_to_f64(kb), bf16_to_f64(vb)

    if route in ("default", "segments"):
        seg = 0 if route == "default" else 64 * int(rng.integers(1, max(2, T // 64 // 2 + 1)))
        print(f"{what} seg={seg} plan={plan(B, T, H, K, V, seg)[:2]}", flush=True)
        o1 = based_forward(_to(qb), _to(kb), _to(vb), scale, out_dtype=out, segment_len=seg)
        o2 = based_forward(_to(qb), _to(kb), _to(vb), scale, out_dtype=out, segment_len=seg)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2), f"{what}: outputs differ between runs"
        _gate(_np(o1), based_ref_chunked(q, k, v, scale, 256), what)
    elif route == "state":
        cut = int(rng.integers(1, T))
        print(f"{what} cut={cut}", flush=True)
        oa, st = based_forward(_to(qb[:, :cut]), _to(kb[:, :cut]), _to(vb[:, :cut]), scale, out_dtype=out,
                               return_state=True)
        ob, st2 = based_forward(_to(qb[:, cut:]), _to(kb[:, cut:]), _to(vb[:, cut:]), scale, out_dtype=out,
                                initial_state=st, return_state=True)
        ob2 = based_forward(_to(qb[:, cut:]), _to(kb[:, cut:]), _to(vb[:, cut:]), scale, out_dtype=out,
                            initial_state=st)
        torch.cuda.synchronize()
        assert torch.equal(ob, ob2), f"{what}: outputs differ between runs"
        o_ref, st_ref = based_ref_chunked_state(q, k, v, scale, None, 256)
        _gate(np.concatenate([_np(oa), _np(ob)], axis=1), o_ref, what)
        _state_gate(_np(st2[0]), st_ref[0], f"{what} S")
        _state_gate(_np(st2[1]), st_ref[1], f"{what} z")
    else:
        prefix = min(T - 1, int(rng.integers(1, 300)))
        steps = min(3, T - prefix)
        print(f"{what} prefix={prefix} steps={steps}", flush=True)
        _, st = based_ref_chunked_state(q[:, :prefix], k[:, :prefix], v[:, :prefix], scale, None, 256)
        S = torch.from_numpy(st[0].astype(np.float32)).to(_dev())
        z = torch.from_numpy(st[1].astype(np.float32)).to(_dev())
        ref = st
        for s in range(steps):
            t = prefix + s
            o = based_decode_step(_to(qb[:, t]), _to(kb[:, t]), _to(vb[:, t]), (S, z), scale, out_dtype=out)
            torch.cuda.synchronize()
            o_ref, ref = based_ref_decode_step(q[:, t], k[:, t], v[:, t], ref, scale)
            _gate(_np(o), o_ref, f"{what} step {s}")
        _state_gate(_np(S), ref[0], f"{what} S")
        _state_gate(_np(z), ref[1], f"{what} z")
