"""GPU parity on the shape lists the page gives for this task ("Write a fast Based (Taylor linear
attention) forward kernel", task spec shapes): its correctness and quick-measure shapes compared element by
element with the oracle, its measure and grader shapes (up to B=8, T=16384, H=32) at full size on eight
whole (b, h) sequences each, plus the convex-combination bound on every output.
Gate: max-abs 2e-2 and relative-L2 5e-3."""
import numpy as np
import pytest

from oracle import MAX_ABS_TOL, REL_L2_TOL, based_ref_chunked, based_ref_direct, bf16_to_f64, errors
from taylor_feature_map_amd.inputs import PAGE_SHAPES, make_workload

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _to_dev(bits):
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(_dev())


def _gate(o, ref, what):
    m, r = errors(o, ref)
    print(f"{what}: max_abs={m:.3e} rel_l2={r:.3e}", flush=True)
    assert m <= MAX_ABS_TOL and r <= REL_L2_TOL, what


def _shapes(role):
    return [w for w in PAGE_SHAPES if w.name.startswith(f"page_{role}_")]


@pytest.mark.parametrize("w", _shapes("correct") + _shapes("quick"), ids=lambda w: w.name)
def test_page_small_shapes_full(w):
    from taylor_feature_map_amd import based_forward
    qb, kb, vb = make_workload(w)
    o = based_forward(_to_dev(qb), _to_dev(kb), _to_dev(vb), w.scale)
    torch.cuda.synchronize()
    q, k, v = bf16_to_f64(qb), bf16_to_f64(kb), bf16_to_f64(vb)
    ref = based_ref_direct(q, k, v, w.scale) if w.T <= 512 else based_ref_chunked(q, k, v, w.scale)
    _gate(o.float().cpu().numpy().astype(np.float64), ref, w.name)


def _pairs(B, H, n=8):
    """n distinct (b, h) pairs spread over the batch and the heads: the corners, the middle, and pairs that
    land on different XCDs and segment positions."""
    cand = [(0, 0), (B - 1, H - 1), (B // 2, H // 2), (0, H - 1), (B - 1, 0), (B // 3, (2 * H) // 3),
            ((2 * B) // 3, 1 % H), (1 % B, H // 3), (B // 2, 0), (0, H // 2), (B - 1, H // 2)]
    out = []
    for p in cand:
        if p not in out:
            out.append(p)
    return out[:n]


@pytest.mark.parametrize("w", _shapes("measure") + _shapes("grader"), ids=lambda w: w.name)
def test_page_large_shapes_pairs(w):
    """The page's measure and grader shapes at full size, in the launch configuration the bench times.
    All inputs are seeded N(0, 1) bf16: eight (b, h) pairs are drawn on the host (numpy, the workload's
    seed) and written into tensors whose other pairs are drawn on the GPU (torch, same seed); every output
    of those eight pairs, the whole sequence and every value column, is compared with the chunked oracle,
    and every output of the tensor is held to the convex-combination bound."""
    from taylor_feature_map_amd import based_forward
    from taylor_feature_map_amd.inputs import make_qkv, make_qkv_device
    dev = _dev()
    print(f"{w.name}: generating inputs", flush=True)
    q, k, v = make_qkv_device(w.B, w.T, w.H, w.K, w.V, w.seed, dev)
    pairs = _pairs(w.B, w.H)
    assert len(pairs) == 8
    qb, kb, vb = make_qkv(len(pairs), w.T, 1, w.K, w.V, w.seed)
    for i, (b, h) in enumerate(pairs):
        q[b, :, h] = _to_dev(qb[i, :, 0])
        k[b, :, h] = _to_dev(kb[i, :, 0])
        v[b, :, h] = _to_dev(vb[i, :, 0])
    o = based_forward(q, k, v, w.scale)
    bound = torch.cummax(v.float().abs(), dim=1).values
    assert bool(torch.isfinite(o).all())
    assert bool((o.float().abs() <= bound * (1 + 2 ** -7) + 1e-6).all()), "convex-combination bound"
    del bound
    got = np.stack([o[b, :, h].float().cpu().numpy().astype(np.float64) for b, h in pairs])  # (8, T, V)
    torch.cuda.synchronize()
    del q, k, v, o
    ref = based_ref_chunked(bf16_to_f64(qb), bf16_to_f64(kb), bf16_to_f64(vb), w.scale)[:, :, 0]
    _gate(got, ref, f"{w.name}: 8 (b, h) pairs, whole sequence")
