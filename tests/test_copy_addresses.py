"""Every memory address the attention kernel computes, emulated on the CPU.

The kernel's tile copies are inline-assembly direct-to-LDS loads
(global_load_lds_dwordx4): lane l copies 16 bytes from its own global
address to LDS address M0 + 16 l, and a paired copy adds the instruction
offset (-2048 / +2048) to both.  The compiler checks none of this address
arithmetic, so this test recomputes it for every workgroup of a launch, from
the kernel's own rules restated here: the schedule (the library's host build of
decode_tile, via attn_sched_tile), the per-head valid key length and causal
end, the full-tile and clamped copy sources with their unsigned 32-bit
offsets, the LDS destination of every copy, the per-wave Q slab copies, the
epilogue's LDS staging and global row stores, and the split-state writes.
Each address is asserted to lie inside its tensor's head (and, for K/V, below
the valid key count: rows past it are never read) and each LDS write inside
its stage of the workgroup's LDS, which must fit the CU's 160 KB.

It covers every shape the GPU tests launch, and also the copy form of an
earlier build (commit caccbdf: a scalar base per super-tile plus a 32-bit
per-lane offset; copy i of wave w at stage rows 8(4*KS*i + w)) on the shape
whose first calls faulted the GPU in a development sweep (B=8, H=8, S=1000,
causal, bf16, keys split between two wave groups): its addresses are in bounds
too, so that fault did not come from the copy arithmetic as written."""
import itertools

import numpy as np
import pytest

import transformer_attention_04_amd as A

BM, BN, N_CU, LDS_CU = 128, 64, 256, 160 * 1024
LANE = np.arange(64)


class Geometry:
    """Compile-time constants of one kernel instance (QG: 32-row query groups
    per workgroup: 4, or 2 or 1 with the key split's 64- and 32-row tiles)."""

    def __init__(self, esz, KS, QG=4):
        self.esz, self.KS, self.QG = esz, KS, QG
        self.ROWB = 64 * esz
        self.TILE = 64 * self.ROWB
        self.STAGE = 2 * KS * self.TILE
        self.NS = 3 if KS == 1 else 2
        self.LPR = self.ROWB // 16
        self.RPC = 64 // self.LPR
        self.NCP = 64 // (QG * self.RPC)
        self.CSTEP = self.RPC * QG * self.ROWB
        # copies PG apart (rows a multiple of the 16-row swizzle period apart) go in pairs
        self.PG = 1 if (QG * self.RPC) % 16 == 0 else 16 // (QG * self.RPC)
        self.PSTEP = self.PG * self.CSTEP
        assert self.PSTEP in (2048, 4096) and self.NCP % (2 * self.PG) == 0
        assert QG == 4 or (QG in (1, 2) and KS == 2)
        assert QG * KS * 32 * self.ROWB <= self.STAGE   # the Q slabs fit a stage
        sizes = [self.STAGE, self.STAGE, self.STAGE if self.NS == 3 else 16]
        self.stage_base = [0, sizes[0], sizes[0] + sizes[1]]
        self.stage_size = sizes
        self.lds_bytes = sum(sizes)

    def kswz(self, row, ph):
        if self.esz == 4:
            return 16 * (ph ^ (row & 15))
        return 16 * (ph ^ ((row & 7) ^ ((row >> 3) & 1)))

    def vswz(self, row, ph):
        return 16 * ph if self.esz == 4 else 16 * (ph ^ ((row & 3) << 1))

    def copy_row(self, i, wave):
        """Stage row of copy i for every lane of `wave` (the current kernel)."""
        QG = self.QG
        return 64 * (wave // QG) + self.RPC * (QG * i + wave % QG) + LANE // self.LPR

    def wgs_per_cu(self):
        return 3 if (self.esz == 2 and self.KS == 1) else (2 if (self.QG <= 2 and self.esz == 2) else 1)


class Box:
    """Accumulates the byte ranges one launch touches and checks them."""

    def __init__(self, what):
        self.what = what
        self.n = 0

    def inside(self, lo_hi, lo, hi, label):
        a, b = lo_hi
        self.n += 1
        assert lo <= a and b <= hi, f"{self.what}: {label} bytes [{a}, {b}) outside [{lo}, {hi})"


def u32(x):
    x = np.asarray(x, dtype=np.int64)
    assert (x >= 0).all() and (x < 2 ** 32).all(), "32-bit offset overflows"
    return x


def stage_of(j, NS):
    return j % NS


def launch_params(B, H, S_q, S_kv, causal, esz, chunk=None, kv_len=None, n_split=1, lens=None):
    """The launch the library makes on a 256-CU device: the split path always
    takes 128-row tiles with one wave group; otherwise the library's own rule
    (attn_sched_rows) gives the tile height and the key split."""
    kv_len = S_kv if kv_len is None else kv_len
    chunk = S_q if chunk is None else chunk
    if n_split > 1:
        rows, KS = (32, 2) if S_q <= 32 else (BM, 1)
    else:
        rows, KS = A.sched_rows(B, H, S_q, causal, "bf16" if esz == 2 else "f32", N_CU)
        tiles = B * H * -(-S_q // BM)
        if S_q <= 32:
            assert (rows, KS) == (32, 2)
        else:
            if esz == 4:
                fine = 2 * tiles <= N_CU
            else:
                fine = KS == 2 and (tiles < 2 * N_CU if causal else tiles % N_CU != 0 and 2 * (tiles % N_CU) <= N_CU)
            assert KS == (2 if tiles <= 2 * N_CU else 1) and rows == (64 if fine else 128)
    return dict(B=B, H=H, S_q=S_q, S_kv=S_kv, causal=causal, esz=esz, chunk=chunk, kv_len=kv_len,
                n_split=n_split, lens=lens, KS=KS, rows=rows, QG=rows // 32)


def blocks_to_check(grid, limit=600):
    """Every workgroup of grids up to `limit`; otherwise the first and last
    200 (the heaviest and lightest windows) and 200 drawn at random."""
    if grid <= limit:
        return range(grid)
    r = np.random.default_rng(grid)
    pick = set(range(0, 200)) | set(range(grid - 200, grid)) | set(r.choice(grid, 200).tolist())
    return sorted(pick)


def emulate_current(P, box):
    """The current kernel: VGPR 64-bit copy addresses, paired copies, Q slabs,
    epilogue staging and stores, split states."""
    g = Geometry(P["esz"], P["KS"], P["QG"])
    assert g.lds_bytes * g.wgs_per_cu() <= LDS_CU
    B, H, S_q, S_kv, causal = P["B"], P["H"], P["S_q"], P["S_kv"], P["causal"]
    ROWB, KS, QG, rows_wg = g.ROWB, P["KS"], P["QG"], P["rows"]
    base_grid = A.sched_grid(B, H, S_q, P["chunk"] if P["n_split"] == 1 else S_q, P["kv_len"], causal, rows_wg)
    n_split = P["n_split"]
    span = 0
    if n_split > 1:
        per = -(-(-(-P["kv_len"] // BN)) // n_split)
        span = per * BN
    head_q = S_q * ROWB           # bytes of one head of q / o
    head_kv = S_kv * ROWB
    for blk in blocks_to_check(base_grid * n_split):
        split, tile = divmod(blk, base_grid)
        head, row0, row1 = A.sched_tile(B, H, S_q, P["chunk"] if n_split == 1 else S_q, tile, P["kv_len"], causal,
                                        rows_wg)
        assert 0 <= head < B * H and 0 <= row0 < row1 <= S_q and row1 - row0 <= rows_wg
        if P["lens"] is not None:
            kv_full = min(max(int(P["lens"][head // H]), 0), S_kv)
        else:
            kv_full = P["kv_len"]
        k_start = split * span
        kv_len = max(0, min(kv_full, k_start + span) - k_start) if n_split > 1 else kv_full
        shift = kv_full - S_q - k_start
        kv_end = min(kv_len, row1 + shift) if causal else kv_len
        if P["lens"] is not None or n_split > 1:
            kv_end = max(0, kv_end)
        n_tiles = -(-kv_end // BN)
        n_super = -(-n_tiles // KS)
        # valid K/V bytes of this head: rows [0, kv_full); this workgroup's
        # base is k_start rows in
        kv_lo = head * head_kv
        kv_hi = kv_lo + kv_full * ROWB
        kbase = kv_lo + k_start * ROWB
        for wave in range(QG * KS):
            qg, kh = wave % QG, wave // QG
            wrow0 = row0 + 32 * qg
            # Q slab: whole rows, K's swizzle, clamped to the tile's last row,
            # in the stage the first step refills (the last of the NS stages)
            sb = g.stage_base[g.NS - 1]
            for i in range(32 * ROWB // 1024):
                row = g.RPC * i + LANE // g.LPR
                cb = g.kswz(row, LANE % g.LPR)
                src = head * head_q + np.minimum(wrow0 + row, row1 - 1) * ROWB + cb
                box.inside((src.min(), src.max() + 16), head * head_q, (head + 1) * head_q, "Q slab source")
                dst = sb + wave * 32 * ROWB + i * 1024 + 16 * LANE
                box.inside((dst.min(), dst.max() + 16), sb, sb + g.STAGE, "Q slab LDS")
            # K/V tile copies
            rows = [g.copy_row(i, wave) for i in range(g.NCP)]
            kc = [g.kswz(r, LANE % g.LPR) for r in rows]
            vc = [g.vswz(r, LANE % g.LPR) for r in rows]
            kof = [u32(r * ROWB + c) for r, c in zip(rows, kc)]
            vof = [u32(r * ROWB + c) for r, c in zip(rows, vc)]
            for i in range(g.NCP):   # a pair shares one address: copy i+PG lies PSTEP bytes on
                if (i // g.PG) % 2 == 0:
                    j = i + g.PG
                    assert (kof[j] - kof[i] == g.PSTEP).all() and (vof[j] - vof[i] == g.PSTEP).all()
                    # and the stage rows are the same distance apart
                    assert ((rows[j] - rows[i]) * ROWB == g.PSTEP).all()
            wdst = (64 * kh + g.RPC * qg) * ROWB
            n_full = min(n_super, kv_len // (KS * BN))    # super-tiles wholly below the cache end
            full_supers = [0, n_full - 1] if n_full > 0 else []
            part_supers = range(n_full, n_super)
            for j in full_supers:   # sources grow with j: the first and last bound them
                off = j * KS * BN * ROWB
                for i in range(g.NCP):
                    for ofs, name in ((kof, "K"), (vof, "V")):
                        src = kbase + ofs[i] + off
                        box.inside((src.min(), src.max() + 16), kv_lo, kv_hi, f"{name} full-tile copy")
            for j in part_supers:
                kv0 = j * KS * BN
                for i in range(g.NCP):
                    rb = u32(np.minimum(kv0 + rows[i], kv_len - 1) * ROWB)
                    for c, name in ((kc[i], "K"), (vc[i], "V")):
                        src = kbase + u32(rb + c)
                        box.inside((src.min(), src.max() + 16), kv_lo, kv_hi, f"{name} clamped copy")
            for j in range(min(n_super, 3)):   # LDS destinations: every stage, every copy
                sb = g.stage_base[stage_of(j, g.NS)]
                for i in range(g.NCP):
                    for m in (sb + wdst, sb + wdst + KS * g.TILE):
                        dst = m + i * g.CSTEP + 16 * LANE
                        box.inside((dst.min(), dst.max() + 16), sb, sb + g.STAGE, "K/V copy LDS")
            # epilogue
            if n_split > 1:
                qrow = wrow0 + (LANE & 31)
                ok = qrow < row1
                prow = (split * B * H + head) * S_q + qrow[ok]
                if ok.any():
                    box.inside((prow.min() * 256, prow.max() * 256 + 256), 0, n_split * B * H * S_q * 256,
                               "split acc state")
                continue
            if KS == 1:
                sb = g.stage_base[(n_super + 1) % 3]
                ot = sb + wave * 32 * ROWB
            else:
                sb = g.stage_base[0]
                ot = sb + qg * 8 * 64 * 16
            box.inside((ot, ot + 32 * ROWB), sb, sb + g.STAGE, "O staging LDS")
            lanes_per_row = ROWB // 16
            for k in range(32 // (64 // lanes_per_row)):
                row = (64 // lanes_per_row) * k + LANE // lanes_per_row
                ch = LANE % lanes_per_row
                ok = wrow0 + row < row1
                if ok.any():
                    dst = head * head_q + (wrow0 + row[ok]) * ROWB + 16 * ch[ok]
                    box.inside((dst.min(), dst.max() + 16), head * head_q, (head + 1) * head_q, "O store")
    return g


def emulate_caccbdf(P, box):
    """The copy form of commit caccbdf: K/V copies from a scalar base (the head
    base, advanced to the super-tile for full tiles) plus a 32-bit per-lane
    offset; copy i of wave w fills stage rows 8(4*KS*i + w) .. +7 (16-bit)."""
    g = Geometry(P["esz"], P["KS"])
    B, H, S_q, S_kv, causal, KS, ROWB = P["B"], P["H"], P["S_q"], P["S_kv"], P["causal"], P["KS"], g.ROWB
    grid = A.sched_grid(B, H, S_q, P["chunk"], P["kv_len"], causal)
    head_kv = S_kv * ROWB
    for blk in blocks_to_check(grid):
        head, row0, row1 = A.sched_tile(B, H, S_q, P["chunk"], blk, P["kv_len"], causal)
        kv_len = P["kv_len"]
        shift = kv_len - S_q
        kv_end = min(kv_len, row1 + shift) if causal else kv_len
        n_super = -(-(-(-kv_end // BN)) // KS)
        kbase = head * head_kv
        for wave in range(4 * KS):
            crow = [g.RPC * (4 * KS * i + wave) + LANE // g.LPR for i in range(g.NCP)]
            kcb = [g.kswz(r, LANE % g.LPR) for r in crow]
            vcb = [g.vswz(r, LANE % g.LPR) for r in crow]
            kof = [u32(r * ROWB + c) for r, c in zip(crow, kcb)]
            vof = [u32(r * ROWB + c) for r, c in zip(crow, vcb)]
            wdst = g.RPC * wave * ROWB
            n_full = min(n_super, kv_len // (KS * BN))
            for j in sorted({0, 1, 2, max(0, n_full - 1)} | set(range(n_full, n_super))):
                if j >= n_super:
                    continue
                kv0 = j * KS * BN
                sb = g.stage_base[stage_of(j, g.NS)]
                for i in range(g.NCP):
                    for m in (sb + wdst, sb + wdst + KS * g.TILE):
                        dst = m + i * (g.RPC * 4 * KS * ROWB) + 16 * LANE
                        box.inside((dst.min(), dst.max() + 16), sb, sb + g.STAGE, "K/V copy LDS (caccbdf)")
                    if kv0 + KS * BN <= kv_len:
                        for o, name in ((kof[i], "K"), (vof[i], "V")):
                            src = kbase + kv0 * ROWB + o
                            box.inside((src.min(), src.max() + 16), kbase, kbase + kv_len * ROWB,
                                       f"{name} full copy (caccbdf)")
                    else:
                        rb = u32(np.minimum(kv0 + crow[i], kv_len - 1) * ROWB)
                        for c, name in ((kcb[i], "K"), (vcb[i], "V")):
                            src = kbase + u32(rb + c)
                            box.inside((src.min(), src.max() + 16), kbase, kbase + kv_len * ROWB,
                                       f"{name} clamped copy (caccbdf)")


ES = {"bf16": 2, "f16": 2, "f32": 4}

# Every launch shape of the GPU tests: (B, H, S_q, S_kv, causal, chunk, kv_len, n_split, lens)
EDGE = [(1, 1, 1, 1, False), (1, 1, 1, 1, True), (1, 1, 2, 3, False), (1, 1, 3, 5, True), (1, 2, 5, 17, True),
        (2, 1, 17, 17, True), (1, 1, 63, 64, False), (1, 1, 64, 64, True), (1, 1, 65, 65, True),
        (1, 3, 127, 129, False), (1, 1, 129, 129, True), (2, 2, 200, 200, True), (1, 1, 200, 63, False),
        (1, 1, 1, 200, False), (1, 1, 1, 200, True), (1, 2, 33, 300, True), (2, 4, 257, 257, True),
        (1, 8, 130, 70, False), (3, 1, 300, 301, True), (1, 1, 512, 1000, True)]
SHAPES = [dict(B=b, H=h, S_q=sq, S_kv=skv, causal=c) for b, h, sq, skv, c in EDGE]
SHAPES += [
    dict(B=16, H=16, S_q=300, S_kv=333, causal=True), dict(B=16, H=16, S_q=300, S_kv=333, causal=False),
    dict(B=16, H=16, S_q=300, S_kv=333, causal=True, chunk=100, kv_len=320),
    dict(B=32, H=16, S_q=200, S_kv=200, causal=True), dict(B=64, H=8, S_q=130, S_kv=70, causal=False),
    dict(B=64, H=16, S_q=130, S_kv=40, causal=False), dict(B=16, H=16, S_q=600, S_kv=1000, causal=True, chunk=250,
                                                          kv_len=900),
    dict(B=7, H=13, S_q=700, S_kv=700, causal=True),
    dict(B=2, H=2, S_q=96, S_kv=700, causal=True, chunk=32, kv_len=97),
    dict(B=2, H=2, S_q=96, S_kv=700, causal=True, chunk=96, kv_len=640),
    dict(B=2, H=2, S_q=96, S_kv=700, causal=False, chunk=50, kv_len=333),
    dict(B=2, H=4, S_q=1500, S_kv=1500, causal=True, chunk=7), dict(B=8, H=16, S_q=700, S_kv=700, causal=True,
                                                                     chunk=300),
    dict(B=1, H=8, S_q=512, S_kv=3000, causal=True, chunk=512, kv_len=3000),
    dict(B=1, H=1, S_q=128, S_kv=128, causal=False), dict(B=8, H=8, S_q=512, S_kv=512, causal=False),
    dict(B=4, H=8, S_q=2048, S_kv=2048, causal=True), dict(B=32, H=16, S_q=1024, S_kv=1024, causal=False),
    dict(B=16, H=16, S_q=98304, S_kv=98304, causal=True, chunk=4096),
    dict(B=16, H=16, S_q=4096, S_kv=98304, causal=True, chunk=4096, kv_len=8192),
    dict(B=1, H=4, S_q=1100, S_kv=1100, causal=True), dict(B=8, H=8, S_q=1100, S_kv=1100, causal=True),
    dict(B=8, H=8, S_q=1000, S_kv=1000, causal=True),
]
SHAPES += [dict(B=2, H=3, S_q=200, S_kv=200 + off, causal=True) for off in (1, 2, 31, 32, 33, 63, 64, 65, 100)]
SPLIT = [(1, 1, 1, 5000, 5000, True, (2, 7, 40, 79)), (2, 3, 1, 777, 700, False, (2, 3, 16)),
         (1, 2, 3, 4100, 4100, True, (4, 9)), (1, 1, 128, 128, 128, False, (2,)),
         (2, 2, 200, 3000, 2900, True, (3, 6)), (1, 4, 16, 1030, 1030, False, (5,)),
         (1, 4, 130, 1100, 1100, True, (2, 3, 7)), (16, 16, 1, 98304, 98304, True, (2,))]
for b, h, sq, skv, kvl, c, ns in SPLIT:
    SHAPES += [dict(B=b, H=h, S_q=sq, S_kv=skv, causal=c, kv_len=kvl, n_split=n) for n in ns]
VARLEN = [(4, 2, 1100, [1100, 700, 333, 1050]), (8, 3, 333, [333, 1, 0, 65, 200, 12, 300, 129]),
          (32, 16, 1024, list(range(256, 1025, 24))), (4, 8, 2048, [1055, 527, 1450, 1221])]
for b, h, s, lens in VARLEN:
    for c in (False, True):
        SHAPES.append(dict(B=b, H=h, S_q=s, S_kv=s, causal=c, lens=lens[:b]))


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_random_launch_shape_plan_in_bounds(dtype):
    """Every case of the GPU launch-shape test's plan (all tile heights, key
    split or not, each entry point with its drawn window, cache length,
    per-sequence lengths or range count)."""
    from launch_plan import plan
    esz = 4 if dtype == "f32" else 2
    for label, entry, B, H, S_q, S_kv, causal, _, args in plan(dtype, N_CU):
        kw = {k: (v.tolist() if hasattr(v, "tolist") else v) for k, v in args.items()}
        P = launch_params(B, H, S_q, S_kv, causal, esz, **kw)
        box = Box(f"{label} entry {entry} {kw}")
        emulate_current(P, box)
        assert box.n > 0


@pytest.mark.parametrize("esz", [2, 4])
@pytest.mark.parametrize("n", range(len(SHAPES)))
def test_every_address_in_bounds(n, esz):
    s = dict(SHAPES[n])
    P = launch_params(s.pop("B"), s.pop("H"), s.pop("S_q"), s.pop("S_kv"), s.pop("causal"), esz, **s)
    box = Box(f"shape {SHAPES[n]} esz {esz}")
    emulate_current(P, box)
    assert box.n > 0


def test_caccbdf_copies_of_the_faulting_shape_are_in_bounds():
    """B=8, H=8, S=1000, causal, bf16: 64 heads x 8 tiles = 512 query tiles,
    so the keys are split between two wave groups (KS = 2, two stages); the
    last super-tile of a tile crosses the cache end and takes the clamped
    copies."""
    P = launch_params(8, 8, 1000, 1000, True, 2)
    assert P["KS"] == 2
    box = Box("caccbdf B8 H8 S1000 causal bf16")
    emulate_caccbdf(P, box)
    assert box.n > 1000
    for s in SHAPES[:20]:
        if s.get("n_split", 1) == 1 and s.get("lens") is None:
            P = launch_params(s["B"], s["H"], s["S_q"], s["S_kv"], s["causal"], 2, chunk=s.get("chunk"),
                              kv_len=s.get("kv_len"))
            emulate_caccbdf(P, Box(f"caccbdf {s}"))


def test_emulation_catches_a_planted_overrun():
    """The checks bite: a copy row one past the clamp is outside the head."""
    g = Geometry(2, 2)
    box = Box("planted")
    kv_len, kv0 = 1000, 960
    rows = g.copy_row(1, 4)   # wave 4 (second key half), copy 1: stage rows 96 .. 103
    rb = u32(np.minimum(kv0 + rows, kv_len) * g.ROWB)   # clamp to kv_len, not kv_len - 1
    with pytest.raises(AssertionError):
        src = rb + g.kswz(rows, LANE % g.LPR)
        box.inside((src.min(), src.max() + 16), 0, kv_len * g.ROWB, "planted")
