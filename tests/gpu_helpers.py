"""Helpers shared by the GPU parity tests (host-side comparison only)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import formats as OF  # noqa: E402

FMT_OBJ = {0: OF.E4M3, 1: OF.E5M2, 2: OF.E2M1}

# group-size mixes covering empty, 1, block-1, block, block+1 and large groups
EDGE_SIZES = [0, 1, 31, 32, 33, 127, 128, 129, 255, 256, 257, 0, 5]


def gpu_available() -> bool:
    return torch.cuda.is_available()


def to_dev_u16(a: np.ndarray):
    """uint16 bf16 bits -> device int16 tensor with the same bits."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def to_dev(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t) -> np.ndarray:
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def scales_host(t, recipe) -> np.ndarray:
    """Host copy of device scales in their logical [..., rows, blocks]
    layout: MX (E8M0) scales are stored word-major and unpacked here."""
    if recipe == "mx":
        from mx_scaled_grouped_amd import api
        return host(api.unpack_mx_scales(t))
    return host(t)


def scales_dev(a: np.ndarray, recipe):
    """Device copy of host scales [..., rows, blocks] in the library's
    layout (word-major for MX)."""
    t = to_dev(a)
    if recipe == "mx":
        from mx_scaled_grouped_amd import api
        return api.pack_mx_scales(t)
    return t


def codes_host(t, rows=None) -> np.ndarray:
    """Row-major host copy of pair-interleaved device codes (the first `rows` rows)."""
    from mx_scaled_grouped_amd import api
    return host(api.unpack_codes(t, rows))


def codes_of(t, fmt, rows=None) -> np.ndarray:
    """Row-major codes, one per uint8, of pair-interleaved device codes; 4-bit
    e2m1 codes (fmt 2) are split out of their bytes."""
    c = codes_host(t, rows)
    return OF.unpack_nibbles(c) if fmt == 2 else c


def bf16_host_f64(t) -> np.ndarray:
    """A device bf16 tensor -> float64 numpy (exact)."""
    b = host(t.view(torch.int16)).view(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def assert_bits_equal(got: np.ndarray, want: np.ndarray, what: str):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if got.dtype == np.float32:
        got = got.view(np.uint32)
        want = want.astype(np.float32).view(np.uint32)
    bad = np.flatnonzero(got.reshape(-1) != want.reshape(-1))
    assert bad.size == 0, f"{what}: {bad.size} mismatches, first at {np.unravel_index(bad[0], got.shape)}: " \
                          f"got {got.reshape(-1)[bad[0]]:#x} want {want.reshape(-1)[bad[0]]:#x}"
