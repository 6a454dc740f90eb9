"""The LDS bank model of gfx950, pinned to hardware counters, and the
kernels' LDS access patterns checked against it (CPU only).

tests/golden/gfx950_lds_measured.json holds SQ_LDS_BANK_CONFLICT per
dispatch of tests/lds_geometry/lds_probe.hip on an MI355X: for every
address pattern of make_patterns.py (--no-pairs) and, for each access width,
the lane pairs that conflict when they hit one bank.  From that data alone
this module derives the model (bank line = the smallest conflicting stride;
lane phases = groups of lanes that conflict with one another), checks that
the oracle's bank simulator then reproduces every measured counter exactly,
and finally checks that every LDS instruction the GEMM kernels issue --
operand reads of the 16-bit (32x32x16 and 16x16x32) and MX kernels (the
MXFP6 8-byte reads on their own layout), K-major
and MN-major loader stores -- has degree 1 (no conflict) under that model, using the kernels'
own LDS map exported through the C ABI.
"""
import importlib.util
import json
import os

import numpy as np
import pytest

import dense_gemm_swizzled_amd as sg
from oracle import banks

HERE = os.path.dirname(os.path.abspath(__file__))
FIX = os.path.join(HERE, "golden", "gfx950_lds_measured.json")
WIDTH = {"r32": 4, "r64": 8, "r128": 16, "w128": 16}


def _patterns_module():
    spec = importlib.util.spec_from_file_location(
        "make_patterns", os.path.join(HERE, "lds_geometry", "make_patterns.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


@pytest.fixture(scope="module")
def measured():
    with open(FIX) as f:
        return json.load(f)


@pytest.fixture(scope="module")
def patterns(tmp_path_factory):
    p = tmp_path_factory.mktemp("lds") / "p.txt"
    _patterns_module().main(str(p), pairs=False)
    out = {}
    for line in open(p):
        f = line.split()
        out[f"{f[0]} {f[1]}"] = [None if int(a) < 0 else int(a) for a in f[2:]]
    return out


def _phases(pairs):
    parent = list(range(64))

    def find(x):
        while parent[x] != x:
            parent[x] = parent[parent[x]]
            x = parent[x]
        return x
    for i, j in pairs:
        parent[find(i)] = find(j)
    groups = {}
    for lane in range(64):
        groups.setdefault(find(lane), []).append(lane)
    return sorted(groups.values())


@pytest.fixture(scope="module")
def model(measured):
    m = {}
    for op in ("r64", "r128", "w128"):
        phases = _phases(measured["pairs_conflicting"][op])
        line = min(int(k.split()[0].split("_")[1]) for k, v in measured["patterns"].items()
                   if k.startswith("line_") and k.endswith(" " + op) and v > 0)
        m[op] = dict(nbanks=line // 4, phases=phases)
    return m


def test_derived_model_shape(model, measured):
    # Every pair inside a phase conflicts (the phases are cliques).
    for op in model:
        s = {tuple(p) for p in measured["pairs_conflicting"][op]}
        for ph in model[op]["phases"]:
            for a in ph:
                for b in ph:
                    if a < b:
                        assert (a, b) in s
    assert model["r128"]["nbanks"] == 64 and model["r64"]["nbanks"] == 64
    assert model["w128"]["nbanks"] == 32
    assert [len(p) for p in model["r128"]["phases"]] == [16] * 4
    assert model["r128"]["phases"][0] == [0, 1, 2, 3, 12, 13, 14, 15,
                                          20, 21, 22, 23, 24, 25, 26, 27]
    assert model["w128"]["phases"] == [list(range(s, s + 8)) for s in range(0, 64, 8)]
    assert model["r64"]["phases"] == [list(range(32)), list(range(32, 64))]


def test_simulator_reproduces_every_measured_counter(model, measured, patterns):
    n_instr = measured["instructions_per_dispatch"]
    checked = 0
    for key, counter in measured["patterns"].items():
        op = key.split()[1]
        if op not in model:
            continue
        sim = banks.extra_cycles(patterns[key], WIDTH[op], nbanks=model[op]["nbanks"],
                                 phases=model[op]["phases"])
        assert sim * n_instr == counter, (key, sim, counter)
        checked += 1
    assert checked > 100


# ----------------------------------------------- the kernels' LDS patterns

def _degree(model, op, addrs):
    return banks.conflict_degree(addrs, WIDTH[op], nbanks=model[op]["nbanks"],
                                 phases=model[op]["phases"])


@pytest.mark.parametrize("tile", [128, 256])
def test_kernel_operand_reads_conflict_free(model, tile):
    lds = sg.gemm_lds_layout(tile, 128)   # the kernels' own map (C ABI)
    half = tile // 2
    worst = 0
    for w in range(2):                    # wave row / column in the 2x2 grid
        for f in range(half // 32):
            base = w * half + f * 32
            # 16-bit MFMA 32x32x16: lane l -> row l%32, chunk 2*kk + l/32.
            for kk in range(4):
                a = [int(lds[base + l % 32, 2 * kk + l // 32]) for l in range(64)]
                worst = max(worst, _degree(model, "r128", a))
            # 16-bit MFMA 16x16x32 (256x256 tiles): lane l -> row l%16 of a
            # 16-row block, chunk 4*kk + l/16.
            for sub in range(2):
                for kk in range(2):
                    a = [int(lds[base + 16 * sub + l % 16, 4 * kk + l // 16])
                         for l in range(64)]
                    worst = max(worst, _degree(model, "r128", a))
            # MXFP8 32x32x64: two reads, chunks 4*kk + 2*h + l/32.
            for kk in range(2):
                for h in range(2):
                    a = [int(lds[base + l % 32, 4 * kk + 2 * h + l // 32])
                         for l in range(64)]
                    worst = max(worst, _degree(model, "r128", a))
    assert worst == 1


@pytest.mark.parametrize("tile", [128, 256])
def test_kernel_loader_stores_conflict_free(model, tile):
    lds = sg.gemm_lds_layout(tile, 128)
    worst = 0
    for wave in range(4):
        tids = [64 * wave + l for l in range(64)]
        # K-major loader: step i, thread t -> row 32*i + t/8, chunk t%8.
        for i in range(tile * 8 // 256):
            a = [int(lds[32 * i + t // 8, t % 8]) for t in tids]
            worst = max(worst, _degree(model, "w128", a))
        # MN-major loader after the register transpose: thread t -> rows
        # 8*(t/8) + c, chunk t%8 (threads beyond the tile's rows idle).
        for c in range(8):
            a = [int(lds[8 * (t // 8) + c, t % 8]) if t < tile else None for t in tids]
            if any(x is not None for x in a):
                worst = max(worst, _degree(model, "w128", a))
    assert worst == 1


@pytest.mark.parametrize("unshifted", [32, 7, 30])
def test_mxfp6_operand_reads_conflict_free(model, unshifted):
    # The MXFP6 fragment read: lane l -> row l%32 of a 32-row block, bytes
    # [24(2kk + h) + 8q, +8) with h = l/32, one ds_read_b64 per piece q.  With
    # every odd row shifted the reads are conflict-free; the block position
    # left unshifted in the tile that holds an operand's last row costs at
    # most one 2-way conflict.
    lds = sg.gemm_lds_layout_mxfp6(256, unshifted)
    worst = 0
    for base in range(0, 256, 32):
        for kk in range(2):
            for q in range(3):
                a = [int(lds[base + l % 32, (24 * (2 * kk + l // 32) + 8 * q) // 8])
                     for l in range(64)]
                worst = max(worst, _degree(model, "r64", a))
    # (an even position changes nothing: even rows are never shifted)
    assert worst == (2 if unshifted % 2 else 1)


def test_mxfp6_reads_without_the_shift_would_conflict(model):
    # The same reads on the plain XOR layout: the 16-byte units alone give 32
    # rows only 16 distinct 8-byte bank slots.
    lds = sg.gemm_lds_layout(32, 128)
    a = [int(lds[l % 32, (24 * (l // 32)) // 16]) + (24 * (l // 32)) % 16 for l in range(64)]
    assert _degree(model, "r64", a) == 2


def test_cblock_map_fits_the_loads_it_rides_on():
    # The 256x256 kernel's C block: each wave's 128 x 8 chunks fill exactly
    # its own 1 KiB regions 4q + w of the four 16 KiB quarters, and load q of
    # quarter Q (lane l -> byte 16 l of region 4q + w) carries row 32Q + 8q +
    # l/8 -- the rows the load's lanes are given.
    m = sg.gemm_lds_layout_cblock()
    flat = m.reshape(-1)
    assert len(set(flat.tolist())) == flat.size and flat.min() >= 0 and flat.max() < 65536
    assert (flat % 16 == 0).all()
    for w in range(4):
        for r in range(128):
            for c in range(8):
                off = int(m[w, r, c])
                Q, inq = divmod(off, 16384)
                region, byte = divmod(inq, 1024)
                assert Q == r // 32 and region == 4 * ((r // 8) % 4) + w
                assert byte // 128 == r % 8   # lane l = byte / 16 covers row l / 8
    # every lane's 16 bytes receive exactly one chunk of the row it loads
    for w in range(4):
        for Q in range(4):
            for q in range(4):
                got = sorted(int(m[w, 32 * Q + 8 * q + l // 8, c]) % 1024
                             for l in range(0, 64, 8) for c in range(8))
                assert got == list(range(0, 1024, 16))


def test_cblock_epilogue_reads_conflict_free(model):
    # Lane l of accumulator block (i, jn) reads C row 16i + l%16, columns
    # 16jn + 4(l/16) .. +3: 8 bytes at half (l/16)%2 of chunk 2jn + l/32.
    m = sg.gemm_lds_layout_cblock()
    worst = 0
    for w in range(4):
        for i in range(8):
            for jn in range(4):
                a = [int(m[w, 16 * i + l % 16, 2 * jn + l // 32]) + 8 * ((l // 16) % 2)
                     for l in range(64)]
                worst = max(worst, _degree(model, "r64", a))
    assert worst == 1
    # the same reads with the chunks left in place would conflict
    a = [(l % 16) * 128 + 16 * (l // 32) + 8 * ((l // 16) % 2) for l in range(64)]
    assert _degree(model, "r64", a) > 1


def test_16x16_d_staging_conflict_free(model):
    # The 256x256 kernel of 16x16x32 MFMAs stages a 16-bit D in the wave's C
    # block regions: row r of its 128 x 64 block in quarter r/32, region
    # 4((r/8)%4) + w, 128-byte row r%8, chunk c at c XOR r%8.  After
    # v_permlane16_swap, lane l (rho = l/16) of block row i and block pair jp
    # writes chunk 4jp + 2(rho%2) + rho/2 of row 16i + l%16 (ds_write_b128);
    # the store pass reads row 8s + l/8, chunk l%8.
    place = lambda w, r, c: ((r // 32) * 16384 + (4 * ((r // 8) % 4) + w) * 1024
                             + (r % 8) * 128 + 16 * (c ^ (r % 8)))
    m = sg.gemm_lds_layout_cblock()
    for w in range(4):   # the same bytes as the wave's C block
        assert ({place(w, r, c) for r in range(128) for c in range(8)}
                == set(m[w].reshape(-1).tolist()))
    wr = max(_degree(model, "w128", [place(w, 16 * i + l % 16,
                                           4 * jp + 2 * ((l // 16) % 2) + l // 32)
                                     for l in range(64)])
             for w in range(4) for i in range(8) for jp in range(2))
    rd = max(_degree(model, "r128", [place(w, 8 * s + l // 8, l % 8) for l in range(64)])
             for w in range(4) for s in range(16))
    assert (wr, rd) == (1, 1)


def test_mn_major_transposing_reads_conflict_free(model):
    # The 64x64 deep-ring kernel keeps an MN-major operand one 128-byte row
    # per k, chunks of rows with bit 1 set rotated by 64 bytes.  A fragment
    # (columns c0..c0+31, 16 wide K step kk) is two ds_read_b64_tr_b16: lane
    # l (group G = l/16, i = l%16) reads 8 bytes of row 16kk + 8(G/2) + 4r +
    # i/4 at column c0 + 16(G%2) + 4(i%4).
    off = lambda k, byte: k * 128 + ((byte + 64 * ((k >> 1) & 1)) % 128)
    worst = 0
    for c0 in (0, 32):
        for kk in range(4):
            for r in range(2):
                a = [off(16 * kk + 8 * ((l // 16) // 2) + 4 * r + (l % 16) // 4,
                         2 * (c0 + 16 * ((l // 16) % 2) + 4 * ((l % 16) % 4)))
                     for l in range(64)]
                worst = max(worst, _degree(model, "r64", a))
    assert worst == 1
    # with the rotation on bit 3 instead, rows k0 and k0+2 share their banks
    off3 = lambda k, byte: k * 128 + ((byte + 64 * ((k >> 3) & 1)) % 128)
    a = [off3(8 * ((l // 16) // 2) + (l % 16) // 4, 2 * (16 * ((l // 16) % 2) + 4 * (l % 4)))
         for l in range(64)]
    assert _degree(model, "r64", a) == 2


def test_mn_major_128_tiles_deep_ring_conflict_free(model):
    # The 128x128 deep ring's MN-major operand: 256-byte rows, 32-byte unit u
    # of row k at u XOR 2(k % 4).  Lane l (group c = l/16, i = l%16) reads 8
    # bytes of row 16kk + 8(c/2) + 4r + i/4 at column col0 + 16(c%2) + 4(i%4),
    # col0 = 32 x (wave block) (ds_read_b64_tr_b16).
    off = lambda k, byte: k * 256 + 32 * ((byte >> 5) ^ (2 * (k % 4))) + byte % 32
    assert sorted(off(k, b) for k in range(64) for b in range(0, 256, 16)) == \
        list(range(0, 16384, 16))
    worst = 0
    for col0 in range(0, 128, 32):
        for kk in range(4):
            for r in range(2):
                a = [off(16 * kk + 8 * ((l // 16) // 2) + 4 * r + (l % 16) // 4,
                         2 * (col0 + 16 * ((l // 16) % 2) + 4 * (l % 4))) for l in range(64)]
                worst = max(worst, _degree(model, "r64", a))
    assert worst == 1


def test_mn_major_b_256_tiles_conflict_free(model):
    # The 256x256 kernel's MN-major B half: one 256-byte row per k, 32-byte
    # unit u of row k at u XOR ((k % 4) + 4 ((k / 8) % 2)).  Lane l (group c =
    # l/16, i = l%16) of wave w4 reads 8 bytes of row 32kh + 8c + 4r + i/4 at
    # column 64(w4%2) + 16j + 4(i%4) (ds_read_b64_tr_b16).
    key = lambda k: (k % 4) | (((k >> 3) & 1) << 2)
    off = lambda k, byte: k * 256 + 32 * ((byte >> 5) ^ key(k)) + byte % 32
    assert sorted(off(k, b) for k in range(64) for b in range(0, 256, 16)) == \
        list(range(0, 16384, 16))
    worst = 0
    for w4 in range(4):
        for j in range(4):
            for kh in range(2):
                for r in range(2):
                    a = [off(32 * kh + 8 * (l // 16) + 4 * r + (l % 16) // 4,
                             2 * (64 * (w4 % 2) + 16 * j + 4 * (l % 4))) for l in range(64)]
                    worst = max(worst, _degree(model, "r64", a))
    assert worst == 1


@pytest.mark.parametrize("kfm,kfn", [(1, 1), (2, 2)])
def test_fp32_d_staging_conflict_free(model, kfm, kfn):
    # The deep-ring kernels' fp32 D (64x64 tiles: a 32x32 block per wave;
    # 128x128: 64x64): lane l of accumulator block (fm, fn) writes 16 bytes
    # of row 32fm + l%32, chunk 8fn + 2q + l/32, to row * 128kfn + 16 (chunk
    # XOR row%8) with ds_write_b128; the store pass reads one contiguous KiB
    # per instruction (row 8s/kfn + l/(8kfn), chunk l%(8kfn)).
    rb = 128 * kfn
    place = lambda r, c: r * rb + 16 * (c ^ (r & 7))
    assert len({place(r, c) for r in range(32 * kfm) for c in range(8 * kfn)}) == 32 * kfm * 8 * kfn
    w = max(_degree(model, "w128", [place(32 * fm + l % 32, 8 * fn + 2 * q + l // 32)
                                    for l in range(64)])
            for fm in range(kfm) for fn in range(kfn) for q in range(4))
    lpr = rb // 16
    r = max(_degree(model, "r128", [place((64 // lpr) * s + l // lpr, l % lpr) for l in range(64)])
            for s in range(32 * kfm * rb // 1024))
    assert (w, r) == (1, 1)


def test_mx_d_staging_conflict_free(model):
    # The MX kernels' 16-bit D: after v_permlane32_swap, lane l holds chunk
    # 4fn + 2p + l/32 of row 32fm + l%32 of its 128 x 64 block (128-byte
    # rows), written at chunk XOR row%8; the store pass reads row 8s + l/8,
    # chunk l%8.
    place = lambda r, c: r * 128 + 16 * (c ^ (r & 7))
    w = max(_degree(model, "w128", [place(32 * fm + l % 32, 4 * fn + 2 * p + l // 32)
                                    for l in range(64)])
            for fm in range(4) for fn in range(2) for p in range(2))
    r = max(_degree(model, "r128", [place(8 * s + l // 8, l % 8) for l in range(64)])
            for s in range(16))
    assert (w, r) == (1, 1)
    # 8-byte halves written straight from the accumulator layout (32 rows,
    # one half each per 32 lanes) find only 16 places in a 256-byte line:
    # even the C block map, built for 8-byte accesses, leaves them 2-way.
    m = sg.gemm_lds_layout_cblock()
    a = [int(m[0, l % 32, 0]) % 16384 + 8 * (l // 32) for l in range(64)]
    assert _degree(model, "r64", a) == 2


def test_padded_layout_is_conflict_free(model):
    # The padded layout of the layout ablation (144-byte rows, no XOR): the
    # 32x32x16 fragment reads and the register-staged ds_write_b128 stores
    # (thread t -> row t/8 + 32 i, chunk t%8) of the 128x128 kernel.
    pad = lambda r, c: r * 144 + 16 * c
    worst = 0
    for base in range(0, 128, 32):
        for kk in range(4):
            worst = max(worst, _degree(model, "r128",
                                       [pad(base + l % 32, 2 * kk + l // 32) for l in range(64)]))
    for wave in range(4):
        for i in range(4):
            tids = [64 * wave + l for l in range(64)]
            worst = max(worst, _degree(model, "w128", [pad(32 * i + t // 8, t % 8) for t in tids]))
    assert worst == 1


def test_unswizzled_layout_would_conflict(model):
    # The same 16-bit operand read on an unswizzled 128-byte-pitch tile.
    a = [(l % 32) * 128 + 16 * (l // 32) for l in range(64)]
    assert _degree(model, "r128", a) == 8
