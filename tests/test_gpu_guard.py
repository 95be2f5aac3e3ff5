"""Nothing is written outside the output tensor: the output lies inside a larger buffer whose other bytes
hold a fixed pattern, and after the forward those bytes are unchanged while the output itself passes the
parity gate. Sequence lengths are ragged (not a multiple of the chunk), so the last chunk of every sequence
reaches past its end and the rows past the end must be dropped, on every store path: whole-row stores
through LDS (K = 8, and K = 16 with 64-column items over several segments), 16-row tiles (one segment per
item, K = 16 with 128-column items) and the float32 tiles."""
import numpy as np
import pytest

from oracle import MAX_ABS_TOL, REL_L2_TOL, based_ref_direct, bf16_to_f64, errors
from taylor_feature_map_amd.inputs import make_qkv

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

PAD = 1 << 16  # bytes of pattern before and after the output
PATTERN = 0xA5


@pytest.mark.parametrize("B,T,H,K,V,out_dtype", [
    (1, 1000, 2, 16, 64, torch.bfloat16),    # several segments: whole-row stores
    (2, 999, 3, 8, 128, torch.bfloat16),     # K = 8, 128 columns: whole-row stores
    (1, 777, 2, 8, 64, torch.bfloat16),      # K = 8, 64 columns
    (1, 1001, 2, 16, 128, torch.bfloat16),   # K = 16, 128 columns
    (8, 200, 32, 16, 64, torch.bfloat16),    # 256 (b, h) pairs: one segment each, tile stores
    (1, 300, 2, 16, 64, torch.float32),      # float32 tiles
], ids=lambda x: str(x).replace("torch.", ""))
def test_no_write_outside_output(B, T, H, K, V, out_dtype):
    from taylor_feature_map_amd import based_forward
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda:0")
    qb, kb, vb = make_qkv(B, T, H, K, V, seed=11)
    to = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
    esize = torch.tensor([], dtype=out_dtype).element_size()
    n = B * T * H * V * esize
    buf = torch.full((PAD + n + PAD,), PATTERN, dtype=torch.uint8, device=dev)
    out = buf[PAD:PAD + n].view(out_dtype).view(B, T, H, V)
    print(f"guard B{B} T{T} H{H} K{K} V{V} {out_dtype}", flush=True)
    based_forward(to(qb), to(kb), to(vb), None, out=out)
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    assert np.all(host[:PAD] == PATTERN), "bytes before the output were written"
    assert np.all(host[PAD + n:] == PATTERN), "bytes after the output were written"
    o = out.float().cpu().numpy().astype(np.float64)
    ref = based_ref_direct(bf16_to_f64(qb), bf16_to_f64(kb), bf16_to_f64(vb), None)
    m, r = errors(o, ref)
    print(f"  max_abs={m:.3e} rel_l2={r:.3e}", flush=True)
    assert m <= MAX_ABS_TOL and r <= REL_L2_TOL
