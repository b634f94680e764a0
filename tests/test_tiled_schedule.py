"""The tiled kernel's DMA schedule (tq_tiled_sched.h), checked on the CPU.

The kernel keeps activations, weights and scales flowing into LDS with
global_load_lds and waits for them with explicit s_waitcnt vmcnt(n) counts; a
count that is too large reads LDS before the data lands.  This test compiles
the header's constexpr arithmetic with g++, then replays the kernel's issue
order instruction by instruction for every compiled tile and several round
counts, and checks that each wait covers the data its stage reads.  Both weight
sources are covered: 2-bit rows (one 16-byte copy per 16 weight rows, the next
round's weights read at the round's last stage) and 1.6-bit rows (four dword
copies per 16 rows and an LDS byte table, so 1 KB less for the rings; the
next round's weights read from the first stage at which they have landed).
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_mixed_precision_amd", "csrc")

# (MT, NR, NG, KG) of every compiled tile (NR weight-row groups of 16 per wave).
TILES = [(mt, 4, ng, kg) for mt in (2, 4) for ng, kg in ((4, 2), (2, 4), (2, 2), (1, 4))]
TILES += [(mt, 2, ng, 4) for mt in (2, 4) for ng in (1, 2)]
TILES += [(8, 2, 4, 2), (2, 2, 1, 8), (2, 4, 1, 8)]

DRIVER = r"""
#include <cstdio>
#include "tq_tiled_sched.h"
int main() {
  const int tiles[][4] = {%s};
  for (int t1 = 0; t1 < 2; ++t1)
  for (const auto& t : tiles) {
    const int mt = t[0], ng = t[1], kg = t[2], nr = t[3], wv = ng * kg;
    const int stage = kg * 16 * mt * 128, round = wv * (nr * 1024 + 256);
    const int budget = (wv == 8 ? 160 * 1024 : 80 * 1024) - (t1 ? 1024 : 0);
    const tq::RingPlan p = tq::ring_plan(stage, round, budget);
    const int kper = kg * 2 * mt / wv;
    const int w_issue = (t1 ? 4 : 1) * nr + 1;
    const int ready = t1 ? tq::w_ready_ch(p.xs, p.wd) : 3;
    std::printf("%%d %%d %%d %%d %%d %%d %%d %%d %%d", t1, mt, nr, ng, kg, p.xs, p.wd, kper, ready);
    for (int r0 = 1; r0 >= 0; --r0)
      for (int ch = 0; ch < 4; ++ch)
        std::printf(" %%d", tq::vm_younger(p.xs, kper, w_issue, ch, r0, tq::w_issue_ch(p.wd)));
    std::printf("\n");
  }
}
"""


@pytest.fixture(scope="module")
def plans(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    d = tmp_path_factory.mktemp("sched")
    src = d / "drv.cpp"
    src.write_text(DRIVER % ", ".join("{%d, %d, %d, %d}" % (t[0], t[2], t[3], t[1]) for t in TILES))
    exe = d / "drv"
    subprocess.run([gxx, "-std=c++17", "-O1", f"-I{CSRC}", str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout
    rows = {}
    for line in out.strip().splitlines():
        v = [int(x) for x in line.split()]
        t1, mt, nr, ng, kg, xs, wd, kper, ready = v[:9]
        rows[(bool(t1), (mt, nr, ng, kg))] = dict(xs=xs, wd=wd, kper=kper, ready=ready,
                                                  r0=v[9:13], rn=v[13:17],
                                                  w_issue=(4 if t1 else 1) * nr + 1)
    assert set(rows) == {(t1, t) for t1 in (False, True) for t in TILES}
    return rows


KINDS = [False, True]  # 2-bit rows, 1.6-bit rows


def replay(xs, wd, kper, r0, rn, rounds, w_issue, ready=3):
    """Issue order of one wave; returns the first uncovered read, else None.
    w_issue: the weight DMAs of a round plus one scale DMA.  The weights of
    round rd + wd go out at stage ch = 1 of round rd with two weight slots, at
    ch = 0 with one (its slot's round was read in the round before); the next
    round's weights are read at every stage from ch = ready on."""
    wch = 1 if wd == 2 else 0
    q = []  # (kind, id)
    for rd in range(wd):
        q += [("W", rd)] * w_issue
    S = 4 * rounds
    for s in range(xs - 1):
        q += [("X", min(s, S - 1))] * kper
    for rd in range(rounds):
        for ch in range(4):
            s = 4 * rd + ch
            n = (r0 if rd == 0 else rn)[ch]
            landed = len(q) - n  # instructions 0 .. landed-1 have completed
            # every instruction of stage s's first issue (later ones past the
            # end refill the same bytes)
            group = [i for i, e in enumerate(q) if e == ("X", s)][:kper]
            if max(group) >= landed:
                return ("X", rd, ch)
            if ch >= ready:  # the next round's weights are read here
                last_w = max(i for i, e in enumerate(q) if e == ("W", rd + 1))
                if last_w >= landed:
                    return ("W", rd, ch)
            if ch == wch:
                q += [("W", rd + wd)] * w_issue
            q += [("X", min(s + xs - 1, S - 1))] * kper
    return None


@pytest.mark.parametrize("t1", KINDS)
@pytest.mark.parametrize("tile", TILES)
def test_every_wait_covers_its_data(plans, tile, t1):
    p = plans[(t1, tile)]
    assert 3 <= p["xs"] <= 6 and p["wd"] in (1, 2)
    assert p["xs"] <= 4 * p["wd"] - (1 if p["wd"] == 2 else 0)
    assert 0 <= p["ready"] <= 3
    for rounds in (1, 2, 3, 5, 8, 32):
        assert replay(p["xs"], p["wd"], p["kper"], p["r0"], p["rn"], rounds,
                      p["w_issue"], p["ready"]) is None, (tile, t1, rounds)


def test_t1_ready_stage_is_the_earliest(plans):
    """For the 1.6-bit rows, one stage earlier than w_ready_ch would read the
    next round's weights before they land (in some tile and round count)."""
    early = 0
    for tile in TILES:
        p = plans[(True, tile)]
        if p["ready"] == 0:
            continue
        early += 1
        assert any(replay(p["xs"], p["wd"], p["kper"], p["r0"], p["rn"], r, p["w_issue"],
                          p["ready"] - 1) for r in (2, 3, 8)), tile
    assert early > 0


@pytest.mark.parametrize("t1", KINDS)
@pytest.mark.parametrize("tile", TILES)
def test_ring_fits_lds(plans, tile, t1):
    mt, nr, ng, kg = tile
    p, wv = plans[(t1, tile)], ng * kg
    lut = 1024 if t1 else 0
    ring = p["xs"] * kg * 16 * mt * 128 + p["wd"] * wv * (nr * 1024 + 256)
    red = (kg - 1) * ng * mt * nr * 256 * 4
    budget = (160 * 1024 if wv == 8 else 80 * 1024) - lut
    assert max(ring + lut, red) <= 160 * 1024
    order = ((6, 2), (5, 2), (4, 2), (4, 1), (3, 2), (3, 1))
    if ring <= budget:  # the plan is the deepest candidate that fits
        deeper = [(x, w) for x, w in order
                  if x * kg * 16 * mt * 128 + w * wv * (nr * 1024 + 256) <= budget]
        assert (p["xs"], p["wd"]) == deeper[0]


def test_a_count_one_too_large_is_caught(plans):
    """Mutation check of the replay itself: raising any single wait count by one
    (waiting for one instruction less) must leave some read uncovered in some tile."""
    caught = 0
    for key in plans:
        p = plans[key]
        for which in ("r0", "rn"):
            for ch in range(4):
                bad = dict(p)
                bad[which] = list(p[which])
                bad[which][ch] += 1
                if any(replay(bad["xs"], bad["wd"], bad["kper"], bad["r0"], bad["rn"], r,
                              p["w_issue"], p["ready"]) for r in (1, 2, 3, 8)):
                    caught += 1
    # every count of every tile is tight
    assert caught == len(plans) * 8
