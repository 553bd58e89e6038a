"""The room a QWHA forward plan reserves per row split (qwha_forward_plan_bytes)
must hold every chunk the forward's gather schedule produces.  This models
the chunking rule of the planned kernel on the host (a chunk takes at most
512 rows and ends early where the next row's segments would overflow the 112
partial-sum slots; a row of st 16-entry steps has ceil(st / 8) segments when
st > 8) and checks the documented bound (d_out / 512 rounded up) + nnz / 2048
+ 4 on synthetic supports of the benchmark's shape and on adversarial ones.
A plan that ran out of room would only be ignored (the forward prepares its
chunks itself), so this pins the sizing claim, not correctness."""
import numpy as np
import pytest

from wht_adapters_amd import synth

CHUNK, SEG, PSLOTS = 512, 8, 112


def steps_of(beg, end):
    return (end - (beg & ~3) + 15) >> 4 if end > beg else 0


def split_ranges(rp, splits):
    d_out, nnz = len(rp) - 1, int(rp[-1])
    bounds = []
    for s in range(1, splits):
        target = nnz * s // splits
        o = int(np.searchsorted(rp, target, side="left"))  # first row boundary >= target
        bounds.append(min(o & ~7, d_out) if o <= d_out else d_out)
    lo = [0] + bounds
    hi = bounds + [d_out]
    return [(lo[i], max(lo[i], hi[i])) for i in range(splits)]


def chunks_of(rp, r_lo, r_hi):
    n, base = 0, r_lo
    while base < r_hi:
        avail = min(CHUNK, r_hi - base)
        used, cn = 0, 0
        for r in range(base, base + avail):
            st = steps_of(int(rp[r]), int(rp[r + 1]))
            ns = -(-st // SEG) if st > SEG else 1
            dem = ns if 1 < ns <= PSLOTS else 0
            if used + dem > PSLOTS:
                break
            used += dem
            cn += 1
        assert cn >= 1
        base += cn
        n += 1
    return n


def cap(d_out, nnz):
    return -(-d_out // CHUNK) + nnz // 2048 + 4


def check(lens, splits=(1, 2, 8)):
    rp = np.r_[0, np.cumsum(lens)].astype(np.int64)
    d_out, nnz = len(lens), int(rp[-1])
    worst = 0
    for s in splits:
        for lo, hi in split_ranges(rp, s):
            worst = max(worst, chunks_of(rp, lo, hi))
    assert worst <= cap(d_out, nnz), (worst, cap(d_out, nnz))
    return worst


def test_benchmark_support():
    """The 4096 x 4096 support with 262,144 entries and log-normal row
    lengths: at most 11 chunks per split (6 and 6 with the two splits of 2048
    tokens, the count the GPU plan records) against a room of 140."""
    d = synth.qwha(tokens=16)
    lens = np.diff(d["row_ptr"])
    assert check(lens) <= 11
    rp = np.r_[0, np.cumsum(lens)]
    assert [chunks_of(rp, lo, hi) for lo, hi in split_ranges(rp, 2)] == [6, 6]


def test_rows_just_past_one_segment():
    """Every row two segments long (130 entries): chunks end on the slots."""
    worst = check(np.full(4096, 130))
    assert worst >= 4096 // (PSLOTS // 2)  # one split: 56 rows a chunk


@pytest.mark.parametrize("big", [33, 57, 111, 112])
def test_alternating_long_and_split_rows(big):
    """A row of `big` segments next to a two-segment row: with big >= 111
    every chunk holds a single row (rows longer than 4096 entries need
    repeated columns)."""
    long_len = 128 * big - 3
    lens = np.tile([long_len, 130], 300)
    check(lens)


def test_random_supports():
    rng = np.random.default_rng(0)
    for _ in range(20):
        d_out = int(rng.integers(1, 4097))
        kind = rng.integers(0, 3)
        if kind == 0:
            lens = rng.integers(0, 300, d_out)
        elif kind == 1:
            lens = np.minimum(rng.lognormal(3.5, 1.5, d_out).astype(np.int64), 4096)
        else:
            lens = rng.choice([0, 1, 126, 130, 1000, 4096, 14000], d_out)
        check(lens)
