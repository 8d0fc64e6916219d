"""The GPU parity checks are not vacuous: fed pools that the oracle wrote, with
one planted mistake each (a row at the wrong slot, K and V swapped, the
layers swapped, an extra slot written, a row left unwritten, an element off by
more than the tolerance, an element off by one ulp), the helpers the GPU
tests use (check_slot_sets, compare_rows) fail, and they pass on the
unchanged pools. Everything here runs on the CPU: the "device" is a stand-in
whose pools are host arrays.
"""

import numpy as np
import pytest

from oracle import ctx_kv_oracle as O
from speculative_decoding_draft_stacked_amd import workloads as W

from gpu_util import TOL, check_slot_sets, compare_rows


class HostPools:
    """The two methods of DeviceCase that the checks read, over host pools."""

    def __init__(self, case, pk, pv):
        self.case, self.pk, self.pv = case, pk, pv

    def touched_slots(self, layer, which):
        p = (self.pk if which == "k" else self.pv)[layer]
        return np.nonzero(np.any(p != W.SENTINEL, axis=(1, 2)))[0]

    def rows_at(self, layer, which, slots):
        return (self.pk if which == "k" else self.pv)[layer][np.asarray(slots)].copy()


def _oracle_pools(case):
    pk, pv = W.sentinel_pools(case)
    O.ctx_kv_write(case, pk, pv)
    return pk, pv


def _case():
    return W.make_case(T=24, H=64, L=2, NH=2, D=64, row_width=6, commit_range=(1, 7),
                       neg_loc_frac=0.1, slots=64, seed=17)


def _written(case):
    valid = O.valid_rows(case.locs, case.commit_lens, case.row_width)
    return case.locs[valid]


def _plant_move_row(case, pk, pv):
    s = _written(case)[0]
    free = np.setdiff1d(np.arange(case.slots), case.locs)[0]
    for p in pk + pv:
        p[free] = p[s]
        p[s] = W.SENTINEL


def _plant_kv_swap(case, pk, pv):
    s = _written(case)[1]
    pk[0][s], pv[0][s] = pv[0][s].copy(), pk[0][s].copy()


def _plant_layer_swap(case, pk, pv):
    pk[0], pk[1] = pk[1].copy(), pk[0].copy()


def _plant_extra_slot(case, pk, pv):
    free = np.setdiff1d(np.arange(case.slots), case.locs)[0]
    pv[1][free] = 0


def _plant_unwritten(case, pk, pv):
    pk[1][_written(case)[-1]] = W.SENTINEL


def _plant_far_element(case, pk, pv):
    s = _written(case)[2]
    rtol, atol = TOL[case.dtype]
    v = O.decode(pv[0][s, 1, 5:6], case.dtype)
    pv[0][s, 1, 5:6] = O.encode(v + 2 * (atol + rtol * np.abs(v)), case.dtype)


PLANTS = {
    "row at the wrong slot": _plant_move_row,
    "K and V swapped in one row": _plant_kv_swap,
    "layers swapped": _plant_layer_swap,
    "an extra slot written": _plant_extra_slot,
    "a valid row left unwritten": _plant_unwritten,
    "an element off by twice the tolerance": _plant_far_element,
}


def _checks(dc):
    check_slot_sets(dc)
    return compare_rows(dc, label="host")


def test_unchanged_oracle_pools_pass():
    case = _case()
    pk, pv = _oracle_pools(case)
    stats = _checks(HostPools(case, pk, pv))
    assert stats["rows"] == len(_written(case)) and stats["exact_frac"] == 1.0


@pytest.mark.parametrize("plant", list(PLANTS))
def test_planted_mistake_fails(plant):
    case = _case()
    pk, pv = _oracle_pools(case)
    PLANTS[plant](case, pk, pv)
    with pytest.raises(AssertionError):
        _checks(HostPools(case, pk, pv))


def test_one_ulp_passes_but_is_not_exact():
    """Within tolerance is not bit-exact: the reported exact fraction drops."""
    case = _case()
    pk, pv = _oracle_pools(case)
    s = _written(case)[0]
    pk[0][s, 0, 0] ^= 1  # one ulp
    stats = _checks(HostPools(case, pk, pv))
    assert stats["exact_frac"] < 1.0
