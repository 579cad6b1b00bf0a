"""Host model of the 16-bit kernel's LDS layouts (CPU only).

Restates the slot formulas of mha_fwd16.hpp and checks, for D = 32, 64,
128 and 256:
  - the global -> LDS copy maps (lane l of a copy fills 16-byte slot l of a
    1 KiB key-group block) cover every (key, 16-byte chunk) of a tile once;
  - every operand read of a tile is one per-lane base plus an immediate;
  - reads hit distinct banks in each 16-lane (64-bank) cycle;
  - the transposing V reads, with ds_read_b64_tr_b16's lane mapping (per 16
    lanes: lane i gets element i%4 of the 8 bytes lane 4k + i/4 addresses,
    k = 0..3, as measured on gfx950), deliver V[key][d] in exactly the key
    order of P's accumulator layout: element e of lane (c, g) in PV step s
    is key 16s + 8(e//4) + 4g + e%4, dim 32t + c.
The GPU parity tests check the kernel itself; this pins the layout algebra.
"""
import pytest


DIMS = [32, 64, 128, 256]
TILE_KEYS = {32: 128, 64: 64, 128: 64, 256: 64}
K_BASES = {32: 1, 64: 1, 128: 2, 256: 4}      # k-step period of the K read bases
V_BASES = {32: (1, 2), 64: (1, 1), 128: (1, 1), 256: (2, 1)}  # (sub-tile, half) periods


def cfg(D):
    return 512 // D, D // 8, TILE_KEYS[D]  # keys per 1 KiB group, chunks per row, keys per tile


def swK(D, kg):
    return kg & (D // 32 - 1)


def swVc(D, kg):
    return 4 * (kg & 1) if D == 256 else 0


def swVk(D, c):
    if D == 32:
        return (4 * ((c >> 1) & 1)) ^ (8 * (c & 1))
    return 4 * ((c >> 1) & 1) if D == 64 else 0


def k_byte(D, key, c):
    G = cfg(D)[0]
    kg, ks = divmod(key, G)
    return kg * 1024 + ((c ^ swK(D, kg)) * G + ks) * 16


def v_byte(D, key, c):
    G = cfg(D)[0]
    kg, ks = divmod(key, G)
    return kg * 1024 + ((c ^ swVc(D, kg)) * G + (ks ^ swVk(D, c))) * 16


def bank_ways(addrs, nbytes, banks=64):
    per = banks * 4 // nbytes
    worst = 1
    for g0 in range(0, 64, per):
        used = {}
        for a in addrs[g0:g0 + per]:
            for w in range(a // 4, (a + nbytes) // 4):
                used.setdefault(w % banks, set()).add(a)
        worst = max(worst, max(len(v) for v in used.values()))
    return worst


@pytest.mark.parametrize("D", DIMS)
def test_copy_maps_cover_the_tile_once(D):
    G, CPR, BN = cfg(D)
    for name, f in (("K", k_byte), ("V", v_byte)):
        seen = set()
        for kg in range(BN // G):
            for lane in range(64):
                c_phys, ks_phys = divmod(lane, G)
                if name == "K":
                    key, c = kg * G + ks_phys, c_phys ^ swK(D, kg)
                else:
                    c = c_phys ^ swVc(D, kg)
                    key = kg * G + (ks_phys ^ swVk(D, c))
                assert f(D, key, c) == kg * 1024 + lane * 16
                seen.add((key, c))
        assert seen == {(k, c) for k in range(BN) for c in range(CPR)}


@pytest.mark.parametrize("D", DIMS)
def test_k_reads_are_immediates_and_conflict_free(D):
    G, CPR, BN = cfg(D)
    KP = K_BASES[D]
    for t in range(BN // 32):
        for s in range(D // 16):
            addrs = [k_byte(D, 32 * t + l % 32, 2 * s + l // 32) for l in range(64)]
            base = [k_byte(D, 32 * t + l % 32, 2 * (s % KP) + l // 32) for l in range(64)]
            assert len({a - b for a, b in zip(addrs, base)}) == 1
            assert addrs[0] - base[0] == (s // KP) * 2 * KP * G * 16
            assert bank_ways(addrs, 16) == 1


def tr16(sup):
    return [[sup[16 * (L // 16) + 4 * k + (L % 16) // 4][L % 4] for k in range(4)] for L in range(64)]


def v_read_addrs(D, s, t, half):
    out = []
    for L in range(64):
        q, j = divmod(L, 16)
        key = 16 * s + 8 * half + 4 * (q // 2) + j // 4
        d = 32 * t + 16 * (q % 2) + 4 * (j % 4)
        out.append(v_byte(D, key, d // 8) + (d % 8) * 2)
    return out


@pytest.mark.parametrize("D", DIMS)
def test_transposing_v_reads_give_p_key_order(D):
    G, CPR, BN = cfg(D)
    VT, VH = V_BASES[D]
    for s in range(BN // 16):
        for t in range(D // 32):
            got = [[None] * 8 for _ in range(64)]
            for half in range(2):
                sup = []
                for L in range(64):
                    q, j = divmod(L, 16)
                    key = 16 * s + 8 * half + 4 * (q // 2) + j // 4
                    d = 32 * t + 16 * (q % 2) + 4 * (j % 4)
                    sup.append([(key, d + e) for e in range(4)])
                addrs = v_read_addrs(D, s, t, half)
                assert bank_ways(addrs, 8) == 1
                base = v_read_addrs(D, 0, t % VT, half % VH)
                off = {a - b for a, b in zip(addrs, base)}
                assert off == {(16 * s + 8 * (half - half % VH)) // G * 1024 + (t - t % VT) * 64 * G}
                for L, r in enumerate(tr16(sup)):
                    got[L][4 * half:4 * half + 4] = r
            for L in range(64):
                g, c = divmod(L, 32)
                assert got[L] == [(16 * s + 8 * (e // 4) + 4 * g + e % 4, 32 * t + c) for e in range(8)]
