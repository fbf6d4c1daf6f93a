"""The fragment-tiled weight layout produced by uno_pack_weight, checked element by
element against the layout's definition written out in numpy (16 x 32 blocks in
row-block-major order; element (r, c) of a block at ((c % 32) // 8 * 16 + r % 16)
* 8 + c % 8; with pair_hd, row i of a head in packed order is source row
8j + c (c < 8) or pair_hd/2 + 8j + c - 8 (c >= 8), j = i // 16, c = i % 16)."""
import numpy as np
import pytest

from diffusion_drafted_lora_amd import uno
from tests.gpu_util import host, require_gpu

pytestmark = pytest.mark.gpu


def _pack_ref(a, pair_hd):
    rows, cols = a.shape
    src_row = np.arange(rows)
    if pair_hd:
        i = src_row % pair_hd
        j, c = i // 16, i % 16
        src_row = src_row - i + np.where(c < 8, 8 * j + c, pair_hd // 2 + 8 * j + c - 8)
    a = a[src_row]
    out = np.empty(rows * cols, a.dtype)
    r = np.arange(rows)[:, None]
    c = np.arange(cols)[None, :]
    off = ((r // 16) * (cols // 32) + c // 32) * 512 + (((c % 32) // 8) * 16 + r % 16) * 8 + c % 8
    out[off.ravel()] = a.ravel()
    return out


@pytest.mark.parametrize("rows,cols,pair_hd", [(32, 64, 0), (48, 96, 16), (256, 128, 128),
                                               (16, 32, 0)])
def test_pack_matches_layout_definition(rows, cols, pair_hd):
    torch = require_gpu()
    g = torch.Generator().manual_seed(rows * 7 + cols)
    src = torch.randn(rows, cols, generator=g).to(torch.bfloat16)
    src_d = src.cuda()
    out = torch.empty_like(src_d)
    st = uno.lib().uno_pack_weight(uno._ptr(src_d), uno._ptr(out), rows, cols, pair_hd, None)
    assert st == uno.UNO_OK
    ref = _pack_ref(src.view(torch.int16).numpy(), pair_hd)
    got = host(out.view(torch.int16)).ravel()
    assert np.array_equal(got, ref)


def test_pack_rejects_bad_shapes():
    torch = require_gpu()
    a = torch.zeros(24, 64, dtype=torch.bfloat16, device="cuda")
    b = torch.empty_like(a)
    assert uno.lib().uno_pack_weight(uno._ptr(a), uno._ptr(b), 24, 64, 0, None) == 1
    a = torch.zeros(32, 48, dtype=torch.bfloat16, device="cuda")
    assert uno.lib().uno_pack_weight(uno._ptr(a), uno._ptr(b), 32, 48, 0, None) == 1
    assert uno.lib().uno_pack_weight(uno._ptr(a), uno._ptr(a), 32, 64, 0, None) == 1
