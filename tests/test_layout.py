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


# ---------------------------------------------------------------------------
# word-major MX (E8M0) scales

def _mx_offset(r, b, R):
    # word b//4 of every row, rows consecutive; byte b%4 of the row's word
    return ((b // 4) * R + r) * 4 + (b % 4)


@pytest.mark.parametrize("R,B", [(1, 4), (5, 8), (130, 12), (64, 128)])
def test_mx_pack_matches_offset_formula(R, B):
    rng = np.random.default_rng(R * 7 + B)
    x = rng.integers(0, 256, size=(R, B), dtype=np.uint8)
    p = api.pack_mx_scales(torch.from_numpy(x))
    assert tuple(p.shape) == (B // 4, R, 4)
    flat = p.numpy().reshape(-1)
    rr, bb = np.meshgrid(np.arange(R), np.arange(B), indexing="ij")
    assert np.array_equal(flat[_mx_offset(rr, bb, R)], x)


def test_mx_unpack_inverts_pack_with_expert_dim():
    rng = np.random.default_rng(11)
    x = torch.from_numpy(rng.integers(0, 256, size=(3, 9, 16), dtype=np.uint8))
    p = api.pack_mx_scales(x)
    assert tuple(p.shape) == (3, 4, 9, 4)
    assert torch.equal(api.unpack_mx_scales(p), x)
    # unpack is a permutation: pack(unpack(y)) == y
    y = torch.from_numpy(rng.integers(0, 256, size=(2, 6, 4), dtype=np.uint8))
    assert torch.equal(api.pack_mx_scales(api.unpack_mx_scales(y)), y)


def test_mx_shape_errors():
    with pytest.raises(ValueError):
        api.pack_mx_scales(torch.zeros(3, 6, dtype=torch.uint8))
    with pytest.raises(ValueError):
        api.unpack_mx_scales(torch.zeros(2, 3, 2, dtype=torch.uint8))


def test_batch_group_ends():
    # a 3-D [E, m, C] operand is E equal groups of its [E*m, C] view
    e = api.batch_group_ends(4, 200, "cpu")
    assert e.dtype == torch.int32
    assert e.tolist() == [200, 400, 600, 800]
    assert api.batch_group_ends(2, 0, "cpu").tolist() == [0, 0]
