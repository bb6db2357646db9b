"""CPU models of the decode kernels' work splits (the integer logic of Work::init and
VWork::init in csrc/pa_kernels.hip, restated in Python), checked against brute force.

Each wave of a stream kernel finds the first tile of its share from two cost thresholds
with closed-form arithmetic instead of a search; the reduce kernel then trusts that every
wave between a context's first and last piece holds a piece of it.  These tests compute
the cost position of every tile (and partition) one by one, assign it to the wave whose
share holds it, and check the kernels' formulas against that: the thresholds with their
die weights, the cursor each wave starts from, the inverse the segment descriptors use,
that every tile is taken once and in order, that with the default split every wave in a
context's range holds a piece of it, and that with fixed partitions none is split.
"""
import numpy as np
import pytest

ODD_DIE_WEIGHT = 60  # kOddDieWeight: an odd-numbered wave's share weight, of 64


def cum_weight(v, wo):
    """Summed share weights of waves 0 .. v - 1 (even waves 64, odd waves wo)."""
    return 64 * ((v + 1) // 2) + wo * (v // 2)


def thresholds(total, Wp, wo):
    Om = cum_weight(Wp, wo)
    return [-(-(cum_weight(w, wo) * total) // Om) for w in range(Wp)] + [total]


def wave_of(p, total, Wp, wo):
    """Work::wave_of_last: the wave whose share holds cost position p."""
    Om = cum_weight(Wp, wo)
    X = (p * Om) // total
    k = X // (64 + wo)
    return min(2 * k + (1 if X - k * (64 + wo) >= 64 else 0), Wp - 1)


def stream_split(nts, U, W, PT):
    """Work::init for every wave: (thresholds, [(first tile, tiles, cursor)] per wave)."""
    S = len(nts)
    nps = [((n + PT - 1) // PT if PT > 0 else (1 if n > 0 else 0)) for n in nts]
    T = sum(nts) * U
    total = T + sum(nps) * U
    Wp = min(W, total)
    wo = ODD_DIE_WEIGHT if total >= 2 * Wp else 64
    th = thresholds(total, Wp, wo)
    Gs = np.concatenate([[0], np.cumsum([n * U for n in nts])[:-1]]).astype(int)
    Js = np.concatenate([[0], np.cumsum([p * U for p in nps])[:-1]]).astype(int)

    def find(t_h):
        for s in range(S):
            nt, np_ = nts[s], nps[s]
            gj = int(Gs[s] + Js[s])
            last = gj + (U - 1) * (nt + np_) + (np_ - 1) * (PT + 1) + 1 if PT > 0 else \
                int(Gs[s]) + nt * U + int(Js[s]) + np_ * U - 1
            if nt > 0 and last >= t_h:
                if PT > 0:
                    ru = t_h - gj - (np_ - 1) * (PT + 1) - 1
                    u = (ru + nt + np_ - 1) // (nt + np_) if ru > 0 else 0
                    rj = t_h - gj - u * (nt + np_) - 1
                    t = ((rj + PT) // (PT + 1) if rj > 0 else 0) * PT
                else:
                    ru = t_h - gj + 1
                    u = max(0, (ru + nt) // (nt + 1) - 1) if ru > 0 else 0
                    rt = t_h - gj - u * (nt + 1) - 1
                    t = rt if rt > 0 else 0
                assert 0 <= u < U and 0 <= t < nt, (t_h, s, u, t)
                return int(Gs[s]) + u * nt + t, (s, u, t)
        return T, None

    shares = []
    for w in range(Wp):
        x0, cur = find(th[w])
        x1 = find(th[w + 1])[0] if w + 1 < Wp else T
        shares.append((x0, x1 - x0, cur))
    return dict(T=T, total=total, Wp=Wp, wo=wo, th=th, shares=shares, nps=nps)


def brute_force(nts, U, PT, th):
    """Every tile's (sequence, unit, tile) and the wave that takes it, one by one."""
    owner = lambda p: int(np.searchsorted(th, p, side="right") - 1)  # noqa: E731
    tiles, x, k = [], 0, 0
    for s, nt in enumerate(nts):
        for u in range(U):
            if nt == 0:
                continue
            if PT > 0:  # a partition goes whole to the wave of its first tile's position
                for j in range(0, nt, PT):
                    w = owner(x + j + k + 1)
                    tiles += [(s, u, t, w, k) for t in range(j, min(nt, j + PT))]
                    k += 1
            else:
                tiles += [(s, u, t, owner(x + t + k + 1), k) for t in range(nt)]
                k += 1
            x += nt
    return tiles


def check_stream(nts, U, W, PT):
    sp = stream_split(nts, U, W, PT)
    if sp["T"] == 0:
        return
    th, Wp = sp["th"], sp["Wp"]
    assert all(th[i + 1] - th[i] >= 1 for i in range(Wp)), "an empty threshold range"
    tiles = brute_force(nts, U, PT, th)
    assert len(tiles) == sp["T"]
    waves = [t[3] for t in tiles]
    assert waves == sorted(waves) and waves[-1] < Wp, "shares out of order"
    for w, (x0, n, cur) in enumerate(sp["shares"]):
        mine = [i for i, t in enumerate(tiles) if t[3] == w]
        assert n == len(mine), (w, n, len(mine))
        if mine:
            assert x0 == mine[0] and cur == tiles[x0][:3], (w, x0, cur, tiles[x0][:3])
    segs = {}
    for s, u, t, w, _ in tiles:
        segs.setdefault((s, u), []).append((t, w))
    for (s, u), tw in segs.items():
        ws = [w for _, w in tw]
        if PT == 0:
            # the merge reads the records of every wave from the segment's first to its last:
            # each must hold a piece (with partitions the records are per partition instead,
            # and a wave whose share lies inside one partition's span simply has no work)
            assert sorted(set(ws)) == list(range(ws[0], ws[-1] + 1)), "a wave in a segment's range holds none of it"
            # the descriptor's last wave, from the inverse of the thresholds
            x_last = next(i for i, t in enumerate(tiles) if t[:3] == (s, u, tw[-1][0]))
            p_last = x_last + tiles[x_last][4] + 1
            assert wave_of(p_last, sp["total"], Wp, sp["wo"]) == ws[-1]
        else:  # no partition is split between waves
            for j in range(0, len(tw), PT):
                assert len({w for _, w in tw[j:j + PT]}) == 1


@pytest.mark.parametrize("PT", [0, 1, 2, 3, 32])
def test_stream_split_against_brute_force(PT):
    rng = np.random.default_rng(10 + PT)
    for _ in range(150):
        S = int(rng.integers(1, 20))
        U = int(rng.integers(1, 9))
        W = int(rng.choice([1, 2, 3, 5, 64, 1024]))
        nts = [int(rng.integers(0, 3)) if rng.random() < 0.4 else int(rng.integers(0, 150)) for _ in range(S)]
        if rng.random() < 0.1:
            nts = [0] * S
        check_stream(nts, U, W, PT)


def test_die_weights_and_their_inverse():
    rng = np.random.default_rng(3)
    for _ in range(400):
        Wp = int(rng.integers(1, 3000))
        total = int(rng.integers(Wp, 40 * Wp + 2))
        wo = ODD_DIE_WEIGHT if total >= 2 * Wp else 64
        th = thresholds(total, Wp, wo)
        assert th[0] == 0 and all(th[i + 1] - th[i] >= 1 for i in range(Wp))
        for p in rng.integers(0, total, size=50):
            assert wave_of(int(p), total, Wp, wo) == int(np.searchsorted(th, p, side="right") - 1)
        if wo != 64 and total >= 64 * Wp:  # odd waves take about 60/64 of an even wave's share
            sizes = np.diff(th)
            ratio = sizes[1::2][: Wp // 2].mean() / sizes[0::2][: Wp // 2].mean()
            assert abs(ratio - 60 / 64) < 0.02


# -- the shared-prefix kernel's cost-weighted split (VWork::init) --------------------------
SH_TILE, SH_TILE2, SH_SEG = 4, 5, 6  # kShTileCost, kShTileCost2, kShSegCost


def check_shared(nts, rows, U, W):
    V = len(nts)
    wt = [SH_TILE2 if r > 16 else SH_TILE for r in rows]
    cost = [U * (SH_SEG + nt * w) if nt > 0 else 0 for nt, w in zip(nts, wt)]
    T, total = sum(nt * U for nt in nts), sum(cost)
    Wp = min(W, total // SH_TILE2)
    if T == 0:
        return
    Gv = np.concatenate([[0], np.cumsum([nt * U for nt in nts])[:-1]]).astype(int)
    Cv = np.concatenate([[0], np.cumsum(cost)[:-1]]).astype(int)
    pos, seg_of, cur = [], [], []
    for v in range(V):
        for u in range(U):
            c0 = int(Cv[v]) + u * (SH_SEG + nts[v] * wt[v])
            for t in range(nts[v]):
                pos.append(c0 + SH_SEG + t * wt[v])
                seg_of.append((v, u))
                cur.append((v, u, t))
    wave = (np.array(pos, dtype=np.int64) * Wp) // total
    assert np.all(np.diff(wave) >= 0) and wave.max() < Wp

    def find(th):
        for v in range(V):
            if nts[v] > 0 and Cv[v] + cost[v] - wt[v] >= th:
                nt, w_ = nts[v], wt[v]
                sz = SH_SEG + nt * w_
                rem = th - int(Cv[v]) - SH_SEG - (nt - 1) * w_
                u = -(-rem // sz) if rem > 0 else 0
                rt = th - (int(Cv[v]) + u * sz) - SH_SEG
                t = -(-rt // w_) if rt > 0 else 0
                return int(Gv[v]) + u * nt + t, (v, u, t)
        return T, None

    for w in range(Wp):
        x0, c = find(-(-(w * total) // Wp))
        x1 = find(-(-((w + 1) * total) // Wp))[0] if w + 1 < Wp else T
        idx = np.nonzero(wave == w)[0]
        assert x1 - x0 == len(idx)
        if len(idx):
            assert idx[0] == x0 and c == cur[x0]
    segs = {}
    for x, sg in enumerate(seg_of):
        segs.setdefault(sg, set()).add(int(wave[x]))
    for ws in segs.values():
        assert sorted(ws) == list(range(min(ws), max(ws) + 1))


def test_shared_split_against_brute_force():
    rng = np.random.default_rng(0)
    for _ in range(300):
        V = int(rng.integers(1, 30))
        U = int(rng.integers(1, 5))
        W = int(rng.choice([1, 2, 3, 7, 64, 768]))
        nts = [int(rng.integers(0, 3)) if rng.random() < 0.5 else int(rng.integers(0, 120)) for _ in range(V)]
        rows = [int(rng.choice([4, 8, 16, 24, 32])) for _ in range(V)]
        check_shared(nts, rows, U, W)
