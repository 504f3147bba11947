"""The varlen tile schedule's clamping, checked on the CPU.

``tests/tilemap_check.cpp`` compiles the header the device pre-pass uses
(``fa_tilemap.h``) with g++ and prints the tile list for given cumulative
lengths.  For well-formed lengths the list must be exactly the query tiles of
every sequence; for malformed ones (decreasing, negative, past T) every entry
must still stay inside [0, T) for q and [0, Tkv) for k, and the list never
outgrows the grid (ceil(T / BM) + B entries per head).
"""
import os
import random
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def exe(tmp_path_factory):
    # one binary per test process (parallel runs must not overwrite a binary another one executes)
    out = str(tmp_path_factory.mktemp("tilemap") / "tilemap_check")
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-I", os.path.join(ROOT, "attention_forward_fa_amd", "csrc"),
                    os.path.join(ROOT, "tests", "tilemap_check.cpp"), "-o", out], check=True)
    return out


def run(exe, cq, ck, bm, tq, tkv, reverse):
    inp = f"{len(cq) - 1} {bm} {tq} {tkv} {reverse}\n" + " ".join(map(str, cq)) + "\n" + " ".join(map(str, ck)) + "\n"
    r = subprocess.run([exe], input=inp, stdout=subprocess.PIPE, text=True, check=True)
    lines = r.stdout.split("\n")
    ntiles, tph = map(int, lines[0].split())
    entries = [tuple(map(int, l.split())) for l in lines[1:1 + tph]]
    return ntiles, tph, entries


@pytest.mark.parametrize("reverse", [0, 1])
def test_well_formed_lengths_give_every_tile_once(exe, reverse):
    lens = [300, 0, 17, 260, 1, 128, 129]
    cq = [0]
    for n in lens:
        cq.append(cq[-1] + n)
    T, bm = cq[-1], 128
    ntiles, tph, entries = run(exe, cq, cq, bm, T, T, reverse)
    want = sorted((b, t) for b, n in enumerate(lens) for t in range(-(-n // bm)))
    got = [(e[0], e[1]) for e in entries if e[6]]
    assert sorted(got) == want and ntiles == len(want) <= tph
    if reverse:  # the heaviest (last) tiles of the list come first
        assert got == sorted(got, reverse=True)
    for b, qt, q0, k0, sq, skv, valid in entries:
        if valid:
            assert (q0, sq) == (cq[b], lens[b]) and (k0, skv) == (cq[b], lens[b])


def test_malformed_lengths_stay_inside_the_tensors(exe):
    rng = random.Random(5)
    bm = 128
    for _ in range(400):
        B = rng.randint(1, 9)
        T = rng.randint(0, 2000)
        Tk = rng.randint(0, 2000)
        pick = lambda top: [rng.choice([rng.randint(-300, top + 300), rng.randint(0, top), 0, top])
                            for _ in range(B + 1)]
        cq, ck = pick(T), pick(Tk)
        ntiles, tph, entries = run(exe, cq, ck, bm, T, Tk, rng.randint(0, 1))
        assert len(entries) == tph == -(-T // bm) + B
        for b, qt, q0, k0, sq, skv, valid in entries:
            if not valid:
                assert (b, qt, q0, k0, sq, skv) == (0, 0, 0, 0, 0, 0)
                continue
            assert 0 <= b < B and 0 <= qt and qt * bm < sq
            assert 0 <= q0 and q0 + sq <= T and sq > 0
            assert 0 <= k0 and k0 + skv <= Tk and skv >= 0
