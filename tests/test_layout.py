"""The pair-interleaved code layout (host side): the binding's pack / unpack
helpers against the offset formula of the C header, written out here."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from mx_scaled_grouped_amd import api  # noqa: E402


def _offset(r, l, L):
    # rows 2p, 2p+1 share 2L bytes: 128-byte lines of 64 bytes of each row
    return (r // 2) * 2 * L + (l // 64) * 128 + (r % 2) * 64 + (l % 64)


@pytest.mark.parametrize("R,L", [(1, 64), (2, 128), (7, 256), (130, 384)])
def test_pack_matches_offset_formula(R, L):
    rng = np.random.default_rng(R * 1000 + L)
    x = rng.integers(0, 256, size=(R, L), dtype=np.uint8)
    p = api.pack_codes(torch.from_numpy(x)).numpy()
    assert p.shape == (R + R % 2, L)
    flat = p.reshape(-1)
    rr, ll = np.meshgrid(np.arange(R), np.arange(L), indexing="ij")
    assert np.array_equal(flat[_offset(rr, ll, L)], x)
    if R % 2:   # the added row of the last pair is zero
        assert not np.any(flat[_offset(np.full(L, R), np.arange(L), L)])


def test_unpack_inverts_pack_with_batch_dims():
    rng = np.random.default_rng(5)
    x = torch.from_numpy(rng.integers(0, 256, size=(3, 10, 192), dtype=np.uint8))
    p = api.pack_codes(x)
    assert torch.equal(api.unpack_codes(p), x)
    assert torch.equal(api.unpack_codes(p, 7), x[:, :7])
    # unpack is a permutation: pack(unpack(y)) == y for any even-row buffer
    y = torch.from_numpy(rng.integers(0, 256, size=(4, 128), dtype=np.uint8))
    assert torch.equal(api.pack_codes(api.unpack_codes(y)), y)


def test_shape_errors():
    with pytest.raises(ValueError):
        api.unpack_codes(torch.zeros(3, 64, dtype=torch.uint8))
    with pytest.raises(ValueError):
        api.pack_codes(torch.zeros(2, 96, dtype=torch.uint8))
