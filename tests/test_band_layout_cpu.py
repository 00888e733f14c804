"""Address model of the unfused band-step layout (host logic, no GPU).

The sweeps of the unfused mode store at every step they run, columns outside
the grid included, so the band stride S of the arrays they write must keep
those stores off every other band's cells.  This model takes the cursor
formulas of the sweeps (forward: lane l of band k at step t holds cell
(64k + l, t - l); reverse: sweep row i is grid row N-1-i, the lane walks the
columns from the right) and the stride of the layout (sweep_steps(M), M + 63
rounded up to 16, for any N), and checks for every
lane of every band of both sweeps that a store inside the grid's columns
lands on its own cell, a store outside them on no cell at all, and every
access stays inside the array (the last band's frame spans skew_steps(M)
steps).  tests/test_abi_cpu.py checks that the library sizes its arrays
with the same stride."""
import numpy as np
import pytest

OFF = 80   # steps before a band's first cell


def skew_steps(M):
    return ((M + 2 * OFF + 46 + 15) // 16) * 16


def sweep_steps(M):
    return ((M + 63 + 15) // 16) * 16


def band_stride(N, M):
    return sweep_steps(M)


def check_layout(B, N, M):
    nb = (N + 63) // 64
    S = band_stride(N, M)
    G = B * nb
    elems = ((G - 1) * S + skew_steps(M)) * 64
    owner = np.full(elems, -1, dtype=np.int64)
    r = np.arange(nb * 64)[:, None]
    c = np.arange(M)[None, :]
    for b in range(B):
        idx = (((b * nb + (r >> 6)) * S + (c + (r & 63) + OFF)) * 64 + (r & 63)).ravel()
        assert idx.min() >= 0 and idx.max() < elems
        assert (owner[idx] == -1).all(), "two cells share an element"
        owner[idx] = ((b * nb * 64 + r) * M + c).ravel()
    t = np.arange(sweep_steps(M))[None, :]
    lane = np.arange(64)[:, None]
    for rev in (False, True):
        for b in range(B):
            for band in range(nb):
                i = band * 64 + lane
                if not rev:
                    row = i
                    base = ((b * nb + (row >> 6)) * S + OFF) * 64 + (row & 63)
                    idx = base + 64 * t
                    col = t - lane
                else:
                    row = np.where(i < N, N - 1 - i, i)
                    l = row & 63
                    base = ((b * nb + (row >> 6)) * S + (M - 1 + lane + l + OFF)) * 64 + l
                    idx = base - 64 * t
                    col = M - 1 - (t - lane)
                assert idx.min() >= 0 and idx.max() < elems, (B, N, M, rev, band)
                inside = (t - lane >= 0) & (t - lane < M)
                rows = np.broadcast_to(row, idx.shape)
                own = (b * nb * 64 + rows) * M + col
                assert (owner[idx[inside]] == own[inside]).all(), (B, N, M, rev, band)
                assert (owner[idx[~inside]] == -1).all(), ("store on a cell", B, N, M, rev, band)


@pytest.mark.parametrize("B,N,M", [(1, 1, 1), (1, 64, 1), (1, 64, 2), (2, 64, 17), (1, 5, 3),
                                   (3, 64, 64), (2, 65, 15), (2, 63, 100), (1, 128, 16),
                                   (2, 128, 47), (3, 200, 33), (2, 191, 300), (1, 70, 45),
                                   (2, 128, 1100), (1, 320, 200), (2, 192, 511),
                                   (2, 64, 513), (1, 256, 1000), (2, 127, 17), (2, 129, 64),
                                   (1, 97, 80), (2, 190, 79), (2, 255, 47), (1, 1000, 100),
                                   (2, 33, 513)])
def test_sweep_stores_stay_off_other_cells(B, N, M):
    check_layout(B, N, M)


def test_model_catches_a_too_small_stride():
    """The check fails for a stride one chunk short of the rule (so it is not
    vacuous)."""
    global band_stride
    keep = band_stride
    try:
        band_stride = lambda N, M: keep(N, M) - 16
        for shape in [(2, 128, 100), (2, 100, 100)]:
            with pytest.raises(AssertionError):
                check_layout(*shape)
    finally:
        band_stride = keep
