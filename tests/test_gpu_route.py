"""GPU parity of the routing permutation (mxsg_route) against the oracle's
stable grouping (oracle/routing.py): group ends, routed-row order and the
inverse map bit for bit on every workload's routing, on edge cases (no
tokens, one expert, repeated and invalid ids) and on a large random case;
and the routed rows feed the gathering quantizer exactly as the oracle's
gathered rows do."""
import numpy as np
import pytest

from tests.gpu_helpers import torch, gpu_available, to_dev, to_dev_u16, host, FMT_OBJ
from tests.test_gpu_quant import _compare_act
from oracle import routing as OR
from oracle import quant as OQ
from mx_scaled_grouped_amd import workloads as W

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="no GPU")]


def _api():
    from mx_scaled_grouped_amd import api
    return api


def _check(ids, E, expect_bad=False, offset_rows=0):
    """offset_rows > 0: the ids are a view that starts that many rows into a
    larger device array (not 16-byte aligned when rows * k * 4 is not)."""
    api = _api()
    ids = np.ascontiguousarray(ids, np.int32)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    if offset_rows:
        pad = np.zeros((offset_rows, ids.shape[1]), np.int32)
        dev = to_dev(np.concatenate([pad, ids]))[offset_rows:]
        assert dev.is_contiguous()
    else:
        dev = to_dev(ids)
    r = api.route(dev, E, slot_row=True, status=status)
    ref = OR.route(ids, E)
    assert np.array_equal(host(r.group_ends).astype(np.int64), ref["group_ends"]), "group ends"
    assert np.array_equal(host(r.row_index).astype(np.int64), ref["row_index"]), "row order"
    assert np.array_equal(host(r.slot_row).astype(np.int64), ref["slot_row"]), "inverse map"
    bad = int(host(status)[0])
    assert bad == (api.STATUS_BAD_EXPERT if expect_bad else 0), bad


@pytest.mark.parametrize("cid", [1, 2, 4, 5])
def test_workload_routing(cid):
    topk = W.routing_for(cid)
    print(f"route workload {cid}: T={topk.n_tokens} k={topk.k} E={topk.n_experts}", flush=True)
    _check(topk.expert_ids, topk.n_experts)


@pytest.mark.parametrize("T,k,E", [(0, 2, 4), (1, 1, 1), (7, 3, 1), (1000, 1, 3), (1025, 2, 8), (3000, 8, 257)])
def test_edge_shapes(T, k, E):
    rng = np.random.default_rng(T + k + E)
    _check(rng.integers(0, E, size=(T, k)), E)


def test_repeated_and_invalid_ids():
    rng = np.random.default_rng(3)
    ids = rng.integers(0, 6, size=(2049, 4))
    ids[5] = [2, 2, 2, 2]                        # a token routed to one expert four times
    ids[17, 1] = -1                              # invalid ids are not routed
    ids[300, 3] = 6
    ids[2048, 0] = 1 << 30
    _check(ids, 6, expect_bad=True)


def test_split_passes_with_invalid_ids():
    """Enough entries that each expert's rows are written by several
    workgroups (one per run of chunks), with invalid ids in several runs and
    an expert whose entries all sit in one run."""
    rng = np.random.default_rng(21)
    T, k, E = 20000, 4, 6
    ids = rng.integers(0, E - 1, size=(T, k))
    ids[12000:12100, 0] = E - 1                  # expert E-1: one run of entries only
    for t in (3, 4500, 9100, 15000, 19999):      # invalid ids spread over the runs
        ids[t, t % k] = -7 if t % 2 else E + 3
    print(f"route split: T={T} k={k} E={E}", flush=True)
    _check(ids, E, expect_bad=True)


@pytest.mark.parametrize("offset_rows", [1, 3])
def test_unaligned_ids(offset_rows):
    """Ids that do not start on a 16-byte boundary (a view one or three rows
    of three choices into a larger array) take the one-entry-at-a-time count."""
    rng = np.random.default_rng(30 + offset_rows)
    ids = rng.integers(0, 5, size=(11111, 3))
    ids[77, 2] = -1
    _check(ids, 5, expect_bad=True, offset_rows=offset_rows)


def test_large_random():
    rng = np.random.default_rng(9)
    T, k, E = 131072, 8, 256
    ids = np.argsort(rng.random((T // 64, E)), axis=1)[:, :k]
    ids = np.tile(ids, (64, 1))[rng.permutation(T)]
    print(f"route large: T={T} k={k} E={E}", flush=True)
    _check(ids, E)


@pytest.mark.parametrize("recipe,fmt", [("tw", 0), ("block", 0), ("mx", 0)])
def test_route_then_gather_quantize(recipe, fmt):
    """Device routing feeding the gathering quantizer gives the codes of the
    oracle's quantization of the oracle-gathered rows."""
    api = _api()
    topk = W.routing_for(1)
    x = W.token_activation(1)
    rt = api.route(to_dev(topk.expert_ids), topk.n_experts)
    ref_r = OR.route(topk.expert_ids, topk.n_experts)
    a = x[ref_r["row_index"]]
    ge = ref_r["group_ends"].astype(np.int32)
    q = api.quantize_act(to_dev_u16(x), recipe, fmt, rt.group_ends, rowwise=True, colwise=True,
                         row_index=rt.row_index)
    ref = OQ.quantize_act(a, recipe, FMT_OBJ[fmt], ge, rowwise=True, colwise=True)
    _compare_act(q, ref, recipe, a.shape[0], a.shape[1], True, True)
