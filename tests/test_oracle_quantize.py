"""Pins of the oracle's quantization ANN (CPU only).

* nearest codeword by explicit Euclidean distances (scipy's cdist, a library
  routine, instead of the inner-product form);
* codewords that are the inputs themselves: each input's id is its own index
  (distance 0, closed form);
* permuting the codebook permutes the ids;
* codewords of equal norm: the nearest codeword is the one of largest inner
  product (the cosine-nearest one, for a fixed input);
* one codeword: every id is 0;
* tie flags: an input exactly between two codewords is flagged and takes the
  lower index.
"""
import numpy as np
import pytest
from scipy.spatial.distance import cdist

from oracle import ann_quantize


@pytest.mark.parametrize("B", [2, 17, 128])
def test_nearest_by_cdist(B):
    rng = np.random.default_rng(B)
    x = rng.standard_normal((300, 16))
    C = rng.standard_normal((B, 16)) * rng.uniform(0.5, 2.0, (B, 1))
    ids, tie = ann_quantize(x, C)
    ref = np.argmin(cdist(x, C, "sqeuclidean"), axis=1)
    np.testing.assert_array_equal(ids[~tie], ref[~tie])
    assert tie.mean() < 0.01


def test_inputs_as_codewords():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((64, 8))
    ids, tie = ann_quantize(x, x)
    np.testing.assert_array_equal(ids, np.arange(64))
    assert not tie.any()


def test_codebook_permutation():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((200, 8))
    C = rng.standard_normal((40, 8))
    perm = rng.permutation(40)
    a, ta = ann_quantize(x, C)
    b, tb = ann_quantize(x, C[perm])
    ok = ~(ta | tb)
    np.testing.assert_array_equal(perm[b[ok]], a[ok])


def test_equal_norm_codewords_is_max_inner_product():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((200, 12))
    C = rng.standard_normal((30, 12))
    C = 2.5 * C / np.linalg.norm(C, axis=1, keepdims=True)
    ids, tie = ann_quantize(x, C)
    cosine = (x / np.linalg.norm(x, axis=1, keepdims=True)) @ (C / 2.5).T
    np.testing.assert_array_equal(ids[~tie], np.argmax(cosine, axis=1)[~tie])


def test_single_codeword_and_exact_tie():
    x = np.array([[0.0, 0.0], [1.0, 0.0], [-3.0, 2.0]])
    ids, tie = ann_quantize(x, np.array([[5.0, 5.0]]))
    assert ids.tolist() == [0, 0, 0] and not tie.any()
    # (0, 0) is equidistant from (1, 0) and (-1, 0): flagged, lower index
    ids, tie = ann_quantize(x, np.array([[1.0, 0.0], [-1.0, 0.0]]))
    assert ids.tolist() == [0, 0, 1] and tie.tolist() == [True, False, False]
