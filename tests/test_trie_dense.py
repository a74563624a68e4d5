"""Host-side dense child masks of the CSR trie (grw_trie_dense_build): every node with at
least min_fanout children gets a mask whose set bits are exactly its CSR codes; counting
mode, thresholds and invalid input.  Runs on the CPU (host code of the library)."""
import numpy as np
import pytest

from synth import build_trie_csr, catalog_items, workload


@pytest.fixture(scope="module")
def grw():
    import generative_recommendation_wide_amd as g
    return g


def _expand(masks, C):
    bits = np.unpackbits(masks.view(np.uint8), bitorder="little", axis=1)
    return bits[:, :C].astype(bool)


@pytest.mark.parametrize("name,min_fanout", [("tiny", 2), ("tiny", 100), ("qwen06b", 64)])
def test_masks_equal_csr_rows(grw, name, min_fanout):
    wl = workload(name)
    trie = build_trie_csr(catalog_items(wl), wl.C)
    rp, code, n = trie["row_ptr"], trie["code"], int(trie["n_internal"])
    slot, masks = grw.trie_dense_build(rp, code, n, wl.C, min_fanout)
    fan = np.diff(rp[: n + 1])
    assert np.array_equal(slot >= 0, fan >= min_fanout)
    dense = np.flatnonzero(slot >= 0)
    assert np.array_equal(slot[dense], np.arange(dense.size))        # masks in node order
    assert masks.shape == (dense.size, (wl.C + 31) // 32)
    bits = _expand(masks, wl.C)
    for v in dense[:: max(1, dense.size // 200)]:
        want = np.zeros(wl.C, bool)
        want[code[rp[v]:rp[v + 1]]] = True
        assert np.array_equal(bits[slot[v]], want)
    assert bits.sum() == fan[dense].sum()


def test_threshold_above_every_fanout_gives_no_masks(grw):
    wl = workload("tiny")
    trie = build_trie_csr(catalog_items(wl), wl.C)
    slot, masks = grw.trie_dense_build(trie["row_ptr"], trie["code"], trie["n_internal"], wl.C, wl.C + 1)
    assert (slot == -1).all() and masks.shape[0] == 0


def test_invalid_input_rejected(grw):
    rp = np.array([0, 2, 3], np.int32)
    code = np.array([1, 5, 2], np.int32)
    with pytest.raises(grw.GrwError):
        grw.trie_dense_build(rp, code, 2, 4, 1)          # code 5 outside [0, 4)
    with pytest.raises(grw.GrwError):
        grw.trie_dense_build(np.array([0, 3, 2], np.int32), np.array([0, 1, 2], np.int32), 2, 4, 1)
