"""The weight panel layout written by spa_pack_weights, byte for byte, against
the layout's definition computed here with numpy (a reshape and transpose of
the row-major bytes)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def expected_panels(src_bytes: np.ndarray, n_mats: int, n_rows: int, row_bytes: int) -> np.ndarray:
    ksteps = row_bytes // 64
    panels = (n_rows + 15) // 16
    a = src_bytes.reshape(n_mats, n_rows, ksteps, 64)
    pad = np.zeros((n_mats, panels * 16, ksteps, 64), np.uint8)
    pad[:, :n_rows] = a
    # [mat][panel][row16][kstep][64] -> [mat][panel][kstep][row16][64]
    return pad.reshape(n_mats, panels, 16, ksteps, 64).transpose(0, 1, 3, 2, 4).reshape(-1)


@pytest.mark.parametrize("dtype,esz,n_mats,n_rows,k", [
    ("bf16", 2, 3, 40, 96),     # padded last panel
    ("f32", 4, 1, 128, 48),
    ("e4m3", 1, 2, 33, 192),
    ("bf16", 2, 1, 5120, 2880),
])
def test_pack_matches_layout_definition(dtype, esz, n_mats, n_rows, k):
    from spatially_pipelined_attention_amd import binding as B
    code = {"f32": B.SPA_F32, "bf16": B.SPA_BF16, "e4m3": B.SPA_E4M3}[dtype]
    rng = np.random.default_rng(7)
    src = rng.integers(0, 256, size=n_mats * n_rows * k * esz, dtype=np.uint8)
    ctx = B.spa_init(0)
    src_d = torch.from_numpy(src).cuda()
    nb = B.spa_packed_bytes(code, n_mats, n_rows, k)
    assert nb == n_mats * ((n_rows + 15) // 16) * 16 * k * esz
    dst_d = torch.full((nb,), 0xAB, dtype=torch.uint8, device="cuda")
    B.spa_pack_weights(ctx, code, n_mats, n_rows, k, src_d, dst_d)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(dst_d.cpu().numpy(), expected_panels(src, n_mats, n_rows, k * esz))


def test_pack_rejects_bad_shapes():
    from spatially_pipelined_attention_amd import binding as B
    ctx = B.spa_init(0)
    a = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    b = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    assert B.spa_packed_bytes(B.SPA_BF16, 1, 16, 20) == 0          # 40-byte rows
    with pytest.raises(B.SpaError):
        B.spa_pack_weights(ctx, B.SPA_BF16, 1, 16, 20, a, b)
    with pytest.raises(B.SpaError):
        B.spa_pack_weights(ctx, B.SPA_BF16, 1, 16, 32, a, a)         # overlap
