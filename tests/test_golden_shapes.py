"""The printed row counts are self-consistent and map onto pair counts T*k."""
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def load_rows():
    rows = []
    with open(os.path.join(HERE, "golden", "expert_gemm_row_counts.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                n, kind, _ = line.split(None, 2)
                rows.append((int(n), kind))
    return rows


def test_printed_counts_consistent():
    rows = dict(load_rows())
    assert rows[52752] == "wrong" and 8 * 1099 * 6 == 52752 and 52752 % 64 != 0
    assert rows[70336] == "right" and 8 * 1099 * 8 == 70336 and 70336 % 64 == 0
    for n, kind in rows.items():
        if kind == "wrong":
            assert n > 32768 and n % 64 != 0
        if kind == "right":
            assert n <= 32768 or n % 64 == 0
