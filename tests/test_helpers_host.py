"""The comparison helpers themselves (CPU): the tolerance arithmetic that
every parity test relies on."""
import numpy as np

from tests.helpers import chunk_floor, error_ratio


def test_chunk_floor_restarts_at_chunks_and_sequences():
    x = np.zeros((1, 7, 1))
    x[0, :, 0] = [1, -5, 2, 3, -1, 4, 0.5]
    # sequences [0, 3) and [3, 7), chunks of 2 tokens
    f = chunk_floor(x, cu_seqlens=[0, 3, 7], chunk=2)[0, :, 0]
    assert f.tolist() == [5, 5, 2, 3, 3, 4, 4]
    # two batch rows, one sequence each
    y = np.stack([x[0], -2 * x[0]])
    g = chunk_floor(y, chunk=4)
    assert g[0, :, 0].tolist() == [5, 5, 5, 5, 4, 4, 4]
    assert g[1, :, 0].tolist() == [10, 10, 10, 10, 8, 8, 8]


def test_error_ratio_floor_only_widens_the_element_bound():
    ref = np.full(100, 1e-3)
    ref[0] = 1.0
    got = ref.copy()
    got[1] += 2e-6
    rms = np.sqrt(np.mean(ref ** 2))                 # ~0.1
    assert np.isclose(error_ratio(got, ref, "f32"), 2e-6 / rms / 1e-4)
    fl = np.zeros(100)
    fl[1] = 0.5
    assert np.isclose(error_ratio(got, ref, "f32", floor=fl), 2e-6 / 0.5 / 1e-4)
    # the norm-wise part is unchanged by the floor
    got2 = ref.copy()
    got2[0] += 5e-4
    assert np.isclose(error_ratio(got2, ref, "f32", floor=np.ones(100)), 5.0)
