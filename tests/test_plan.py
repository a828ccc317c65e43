"""The launch planner (vlm_vision_patch_amd/csrc/pe_plan.cpp) built on the host with g++ under
-fsanitize=address,undefined, fed random and edge-case requests, and compared with a Python model of
the planning rules. No GPU.

The model restates the rules the planner implements: the grid checks and their error codes; patch
rows split at one launch's 4 GiB buffer range; frames grouped greedily into launches of at most 64
items (any number of identical ones), at most 4 GiB of input, and, with the image fold, runs of
single images kept apart from videos; the tile choice (fewest rounds x measured round cost:
256 x 256 ~30, 256 x 128 ~18, split-k ~8; ties to the larger tile); and the LDS-staged image path
(single images, bf16 input and weight, P = 14, large tiles) with its grouped weight. The sanitizers
catch what a model cannot: reads past the caller's grid and frame arrays, signed overflow in the
int64 size arithmetic at the int32 limits.
"""
import os
import random
import subprocess

import pytest

from conftest import ROOT

CSRC = os.path.join(ROOT, "vlm_vision_patch_amd", "csrc")
PE_OK, PE_ERR_INVALID_ARG, PE_ERR_SHAPE, PE_ERR_UNSUPPORTED = 0, -1, -2, -3
KMAX, MAXB = 64, 0xFFFFFFF0
I31 = 2 ** 31


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("plan") / "plan_fuzz")
    subprocess.check_call(["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-Wall", "-Wextra", "-Werror",
                           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                           os.path.join(CSRC, "pe_plan.cpp"), os.path.join(ROOT, "tests", "plan_fuzz.cpp"),
                           "-o", exe])
    return exe


def run_driver(exe, reqs):
    lines = []
    for r in reqs:
        head = [r["P"], r["E"], r["m"], r["wesz"], r["iesz"], r["oesz"], r["merge"], r["fold"], r["stage"], r["ncu"],
                r["kind"], len(r["grid"]), 1 if r["frames"] is not None else 0]
        body = []
        for i, g in enumerate(r["grid"]):
            body += list(g) + ([r["frames"][i]] if r["frames"] is not None else [])
        lines.append(" ".join(str(v) for v in head + body))
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    p = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True, env=env, timeout=300)
    assert p.returncode == 0 and "runtime error" not in p.stderr and "ERROR" not in p.stderr, p.stderr[-3000:]
    out, cur = [], None
    for ln in p.stdout.splitlines():
        f = ln.split()
        if f[0] == "R":
            cur = {"rc": int(f[1]), "launches": []}
            out.append(cur)
        elif f[0] == "L":
            v = [int(x) for x in f[1:]]
            keys = ("row0 n_rows in_off in_bytes n_items tile bm bn wg tiles_m tiles_n img fold mixg uni colmajor "
                    "wmap u_rows u_elems plane rstr kind order staged").split()
            cur["launches"].append(dict(zip(keys, v), items=[]))
        elif f[0] == "I":
            cur["launches"][-1]["items"].append(tuple(int(x) for x in f[1:]))
    assert len(out) == len(reqs)
    return out


def cdiv(a, b):
    return -(-a // b)


def model_tiles(n_rows, E, wesz, ncu):
    skn = 160 if E % 160 == 0 else 128
    if wesz == 4:
        return (3, 32, skn)
    ncu = ncu if ncu > 0 else 256
    rounds = lambda t: cdiv(t, ncu)
    rt = cdiv(n_rows, 256)
    c256 = rounds(rt * cdiv(E, 256)) * 30
    c128 = rounds(rt * cdiv(E, 128)) * 18
    csk = rounds(cdiv(n_rows, 32) * cdiv(E, skn)) * 8
    if c256 <= c128 and c256 <= csk:
        return (0, 256, 256)
    if c128 <= csk:
        return (1, 256, 128)
    return (2, 32, skn)


def model_plan(r):
    """(status, launches) by the rules stated in the module docstring."""
    P, E, m, iesz = r["P"], r["E"], r["m"], r["iesz"]
    grid, frames = r["grid"], r["frames"]
    n = len(grid)
    if n == 0:
        return PE_ERR_SHAPE, []
    K = 6 * P * P
    fr_in = r["kind"] == 1
    merge = fr_in and r["merge"]
    F, elems, row0, N = [], [], [], 0
    for i, (t, h, w) in enumerate(grid):
        if t <= 0 or h <= 0 or w <= 0:
            return PE_ERR_SHAPE, []
        if t * h >= I31 or t * h * w >= I31:
            return PE_ERR_SHAPE, []
        if fr_in:
            f = frames[i] if frames is not None else (1 if t == 1 else 2 * t)
            if f <= 0 or (f + 1) // 2 != t:
                return PE_ERR_SHAPE, []
            if merge and (h % m or w % m):
                return PE_ERR_SHAPE, []
            e = f * 3 * h * P * w * P
            if e * iesz > MAXB:
                return PE_ERR_UNSUPPORTED, []
            F.append(f)
            elems.append(e)
        row0.append(N)
        N += t * h * w
    row0.append(N)
    if N >= I31:
        return PE_ERR_SHAPE, []
    pcols = cdiv(E, 32 if iesz == 2 else 16) * (32 if iesz == 2 else 16)
    out = []

    def tiles(L, nr):
        tid, bm, bn = model_tiles(nr, E, r["wesz"], r["ncu"])
        L.update(tile=tid, bm=bm, bn=bn, tiles_m=cdiv(nr, bm), tiles_n=cdiv(E, bn), wg=cdiv(nr, bm) * cdiv(E, bn))

    if not fr_in:
        per = MAXB // (K * iesz)
        for s in range(0, N, per):
            nr = min(per, N - s)
            L = dict(row0=s, n_rows=nr, in_off=s * K * iesz, in_bytes=nr * K * iesz, n_items=0, img=0, fold=0, mixg=0,
                     uni=0, colmajor=int(nr * K * iesz < pcols * K * iesz), wmap=1 if r["wesz"] == 2 else 0,
                     u_rows=0, u_elems=0, plane=2 * P * P, rstr=P, kind=0, order=0, staged=0, items=[])
            tiles(L, nr)
            out.append(L)
        return PE_OK, out
    i0, x0 = 0, 0
    while i0 < n:
        i1, span, same, mixed, imgs = i0, 0, True, False, True
        while i1 < n and (not r["fold"] or (F[i1] == 1) == (F[i0] == 1)) and (span + elems[i1]) * iesz <= MAXB:
            still = same and F[i1] == F[i0] and tuple(grid[i1]) == tuple(grid[i0])
            if i1 - i0 >= KMAX and not still:
                break
            span += elems[i1]
            mixed = mixed or grid[i1][1:] != grid[i0][1:]
            imgs = imgs and F[i1] == 1
            same = still
            i1 += 1
        items, off = [], 0
        for i in range(i0, min(i1, i0 + KMAX)):
            items.append((row0[i] - row0[i0], grid[i][0], grid[i][1], grid[i][2], F[i], off))
            off += elems[i]
        fold = int(imgs and bool(r["fold"]))
        L = dict(row0=row0[i0], n_rows=row0[i1] - row0[i0], in_off=x0 * iesz, in_bytes=span * iesz, n_items=i1 - i0,
                 img=int(imgs), fold=fold, mixg=int(mixed), uni=int(same),
                 colmajor=int(span * iesz < pcols * K * iesz), wmap=2 if fold else 0,
                 u_rows=row0[i0 + 1] - row0[i0], u_elems=elems[i0], plane=grid[i0][1] * P * grid[i0][2] * P,
                 rstr=grid[i0][2] * P, kind=1, order=int(merge), items=items)
        tiles(L, L["n_rows"])
        # single images, bf16, P = 14, large tiles: pixel rows staged through LDS, grouped weight
        L["staged"] = int(bool(r["stage"]) and bool(imgs) and not fold and not mixed and P == 14 and r["wesz"] == 2
                          and iesz == 2 and L["tile"] in (0, 1))
        if L["staged"]:
            L["wmap"] = 3
        out.append(L)
        x0 += span
        i0 = i1
    return PE_OK, out


def req(grid, frames=None, P=14, E=1280, m=2, wesz=2, iesz=2, oesz=2, merge=1, fold=0, ncu=256, kind=1, stage=0):
    return dict(grid=[tuple(g) for g in grid], frames=frames, P=P, E=E, m=m, wesz=wesz, iesz=iesz, oesz=oesz,
                merge=merge, fold=fold, ncu=ncu, kind=kind, stage=stage)


def compare(got, want, r):
    rc, launches = want
    assert got["rc"] == rc, (r, got["rc"], rc)
    assert len(got["launches"]) == len(launches), (r, len(got["launches"]), len(launches))
    for g, w in zip(got["launches"], launches):
        for k, v in w.items():
            if k == "items":
                assert g["items"] == v, (r, k)
            else:
                assert g[k] == v, (r, k, g[k], v)


def edge_requests():
    big = [1, 1, I31 - 1]
    rs = [
        # the workloads' shapes
        req([[1, 16, 64]], [1]),                                     # one 224 x 896 image: split-k
        req([[1, 28, 28]], [1], P=16, E=1152, merge=0),
        req([[8, 32, 32]], [16]),
        req([[1, 72, 72]] * 64, [1] * 64),                           # 64 identical images: one launch
        req([[1, 32, 32], [1, 48, 64], [2, 32, 32], [1, 24, 40], [1, 32, 32]], [1, 1, 4, 1, 1], P=16, E=1024),
        req([[1, 32, 32]], None, kind=0, wesz=4, iesz=4, oesz=4, merge=0),   # fp32 patch rows
        # the 4 GiB split: 720 images of 1008^2 split after 704; 1.9M patch rows after 1,826,091
        req([[1, 72, 72]] * 720, [1] * 720),
        req([[1, 1, 1900000]], None, kind=0, merge=0),
        req([[1, 1, 1900000]], None, kind=0, merge=0, iesz=4),
        # more than 64 items: identical (one launch), and runs of identical items with changes
        req([[1, 4, 4]] * 200, [1] * 200),
        req([[1, 4, 4]] * 70 + [[1, 4, 6]] + [[1, 4, 4]] * 70, [1] * 141),
        req([[1, 4, 4]] * 63 + [[2, 4, 4]] * 5, [1] * 63 + [4] * 5),
        req([[1, 4, 4]] * 63 + [[2, 4, 4]] * 5, [1] * 63 + [4] * 5, fold=1),
        req([[2, 4, 4], [1, 4, 4], [2, 4, 4], [1, 4, 4]], [3, 1, 4, 2], fold=1),
        # errors and the int32 / int64 limits
        req([[0, 2, 2]], [1]), req([[1, -2, 2]], [1]), req([[1, 2, 2]], [0]), req([[2, 2, 2]], [1]),
        req([[1, 3, 2]], [1]), req([[1, 3, 2]], [1], merge=0),
        req([big], None, kind=0, merge=0),                            # N just below 2^31, too many bytes per row? no: rows split
        req([big, [1, 1, 1]], None, kind=0, merge=0),                  # N = 2^31
        req([[I31 - 1, I31 - 1, I31 - 1]], None, kind=0),
        req([[1, 46341, 46341]], None, kind=0),                        # t*h*w just above 2^31
        req([[1, 46340, 46340]], None, kind=0, merge=0),
        req([[1, 1000, 1000]], [1]),                                   # one item's frames beyond 4 GiB
        req([[I31 - 1, 1, 1]], [I31 - 1]),
        req([[I31 - 1, 1, 1]], [-(I31)]),
        req([], None),
    ]
    for ncu in (0, 80, 304):
        rs.append(req([[1, 72, 72]] * 64, [1] * 64, ncu=ncu))
        rs.append(req([[1, 16, 64]], [1], ncu=ncu))
    # the opt-in LDS-staged images: both large tiles, and the launches it leaves alone (split-k,
    # P = 16, fp32 input, mixed frame sizes, videos, the fold)
    for g, f, kw in (([[1, 72, 72]] * 64, [1] * 64, {}), ([[1, 64, 64]], [1], {}), ([[1, 16, 64]], [1], {}),
                     ([[1, 64, 64]], [1], {"P": 16}), ([[1, 64, 64]], [1], {"iesz": 4}),
                     ([[1, 64, 64], [1, 60, 70]], [1, 1], {}), ([[2, 64, 64]], [4], {}),
                     ([[1, 72, 72]] * 64, [1] * 64, {"fold": 1}), ([[1, 64, 64]], [1], {"merge": 0})):
        rs.append(req(g, f, stage=1, **kw))
    return rs


def random_requests(seed, count):
    rng = random.Random(seed)
    rs = []
    for _ in range(count):
        P = rng.choice([14, 16])
        E = rng.choice([16, 128, 160, 1024, 1152, 1280, 2304, 4096, 16 * rng.randint(1, 300)])
        wesz = rng.choice([2, 2, 2, 4])
        iesz = 4 if wesz == 4 else rng.choice([2, 4])
        kind = rng.choice([0, 1, 1, 1])
        m = rng.choice([1, 2, 2, 3])
        merge = rng.choice([0, 1])
        fold = rng.choice([0, 1]) if wesz == 2 else 0
        stage = rng.choice([0, 1])
        ncu = rng.choice([0, 256, 256, 80, 304])
        n = rng.choice([1, 2, 3, 5, 17, 64, 65, 130, rng.randint(1, 300)])
        grid, frames = [], []
        style = rng.choice(["mixed", "runs", "same", "bad"])
        base = None
        for i in range(n):
            if style == "same" and base is not None:
                g, f = base
            elif style == "runs" and base is not None and rng.random() < 0.85:
                g, f = base
            else:
                t = rng.choice([1, 1, 2, 3, 8])
                h = rng.choice([2, 4, 6, 16, 36, 72, rng.randint(1, 90)])
                w = rng.choice([2, 4, 8, 64, 72, rng.randint(1, 90)])
                f = 1 if t == 1 and rng.random() < 0.7 else rng.choice([2 * t, 2 * t - 1])
                g = (t, h, w)
                if style == "bad" and rng.random() < 0.05:
                    g = rng.choice([(0, h, w), (t, -1, w), (t, h, I31 - 1), (I31 - 1, I31 - 1, 1)])
                    f = rng.choice([f, 0, -1, 2 * t + 1, I31 - 1])
            base = (g, f)
            grid.append(g)
            frames.append(f)
        use_frames = kind == 1 and rng.random() < 0.8
        rs.append(req(grid, frames if use_frames else None, P=P, E=E, m=m, wesz=wesz, iesz=iesz, oesz=rng.choice([2, 4]),
                      merge=merge, fold=fold, ncu=ncu, kind=kind, stage=stage))
    return rs


def test_plan_edge_cases_match_model(driver):
    rs = edge_requests()
    for got, r in zip(run_driver(driver, rs), rs):
        compare(got, model_plan(r), r)


def test_plan_known_answers(driver):
    """Facts the GPU tests and the bench also rely on, written out by hand."""
    rs = [req([[1, 72, 72]] * 64, [1] * 64), req([[1, 16, 64]], [1]), req([[1, 72, 72]] * 720, [1] * 720),
          req([[1, 1, 1900000]], None, kind=0, merge=0), req([[8, 32, 32]], [16]),
          req([[1, 72, 72]] * 64, [1] * 64, stage=1)]
    got = run_driver(driver, rs)
    w5 = got[0]["launches"]
    assert len(w5) == 1 and (w5[0]["bm"], w5[0]["bn"], w5[0]["wg"]) == (256, 256, 1296 * 5)
    assert w5[0]["uni"] == 1 and w5[0]["img"] == 1 and w5[0]["n_rows"] == 331776
    w2 = got[1]["launches"]
    assert len(w2) == 1 and (w2[0]["tile"], w2[0]["bm"], w2[0]["bn"], w2[0]["wg"]) == (2, 32, 160, 256)
    split = got[2]["launches"]
    assert [L["n_items"] for L in split] == [704, 16] and split[1]["in_off"] == 704 * 3 * 1008 * 1008 * 2
    rows = got[3]["launches"]
    assert [L["n_rows"] for L in rows] == [1826091, 1900000 - 1826091]
    assert got[4]["launches"][0]["wg"] == 32 * 5 and got[4]["launches"][0]["img"] == 0
    # the default gathers in registers from the temporal-split weight; stage_images switches the
    # batch to the LDS-staged kernel and the grouped weight, same tiles
    assert (w5[0]["staged"], w5[0]["wmap"]) == (0, 0)
    st = got[5]["launches"]
    assert len(st) == 1 and (st[0]["staged"], st[0]["wmap"], st[0]["wg"]) == (1, 3, 1296 * 5)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_plan_random_requests_match_model(driver, seed):
    rs = random_requests(seed, 400)
    for got, r in zip(run_driver(driver, rs), rs):
        compare(got, model_plan(r), r)
