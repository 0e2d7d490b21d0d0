"""The TileLayout helper against the worked values printed on the TIRx layout
pages (tests/golden/layout_worked_examples.json, each entry cited), plus the
invariants the pages state: apply() does not enumerate replicas, shape= may
differ from the shard extents, the swizzle keeps the element set (a
bijection) and needs atom_len >= swizzle_len."""
import json
import os

import pytest

lay = pytest.importorskip("dense_fp16_gemm_02_amd.layout")

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "layout_worked_examples.json")


@pytest.fixture(scope="module")
def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_worked_apply_values(golden):
    for case in golden["apply"]:
        got = lay.apply(case["spec"], *case["coord"], shape=case["shape"])
        assert got == case["expect"], case["cite"]


def test_apply_does_not_enumerate_replicas(golden):
    spec = golden["apply"][0]["spec"]
    got = lay.apply(spec, 1, 3, shape=[8, 16])
    assert got["warpid"] == 5  # base position only; the copy at warp 9 is not returned
    assert lay.replicas(spec) == [{}, {"warpid": 4}]


def test_full_tile_closed_form(golden):
    case = golden["closed_forms"][0]
    spec = case["spec"]
    warps = set()
    for i in range(8):
        for j in range(16):
            got = lay.apply(spec, i, j, shape=case["shape"])
            assert got == {"laneid": 4 * i + (j // 2) % 4, "warpid": j // 8 + 5, "m": j % 2}
            warps.add(got["warpid"])
    assert sorted(warps) == case["warps_base"]
    reps = [r.get("warpid", 0) for r in lay.replicas(spec)]
    assert sorted(w + r for w in warps for r in reps) == case["warps_with_replica"]


def test_shape_may_differ_from_shard_extents(golden):
    spec = golden["apply"][0]["spec"]
    want = lay.apply(spec, 19)
    assert lay.apply(spec, 0, 19, shape=[1, 128]) == want
    assert lay.apply(spec, 2, 3, shape=[4, 8]) == want
    assert lay.apply(spec, 1, 0, 3, shape=[2, 4, 4]) == want
    with pytest.raises(lay.LayoutError):
        lay.apply(spec, 128)  # flat index beyond the shard's 128 elements


def test_tmem_accumulator_layout(golden):
    case = golden["closed_forms"][1]
    cols = set()
    for a in range(2):
        for l in (0, 1, 63, 127):
            for c in (0, 1, 57, 111):
                got = lay.apply(case["spec"], a, l, c, shape=case["shape"])
                assert got == {"TLane": l, "TCol": 112 * a + c}
    for a in range(2):
        for c in range(112):
            cols.add(lay.apply(case["spec"], a, 0, c, shape=case["shape"])["TCol"])
    lo, hi = case["tcol_range"]
    assert cols == set(range(lo, hi))
    assert lay.size(case["spec"]) == 2 * 128 * 112


def test_scale_factor_replica_layout(golden):
    case = golden["closed_forms"][2]
    for sf in case["sf_values"]:
        spec = case["spec_template"].format(sf=sf)
        for r in range(32):
            for s in range(sf):
                assert lay.apply(spec, r, s, shape=[32, sf]) == {"TLane": r, "TCol": s}
        reps = lay.replicas(spec)
        assert [x.get("TLane", 0) for x in reps] == [o["TLane"] for o in case["replica_offsets"]]
        lanes = sorted({r + x.get("TLane", 0) for r in range(32) for x in reps})
        assert lanes == list(range(128))


def test_128b_swizzle_formula(golden):
    case = golden["swizzle"][0]
    addrs = set()
    for i in range(8):
        for j in range(64):
            got = lay.compose_apply(case["per_element"], case["swizzle_len"], case["atom_len"],
                                    case["tile_spec"], i * 64 + j)
            assert got == 64 * i + 8 * ((j // 8) ^ i) + j % 8
            addrs.add(got)
    assert addrs == set(range(512))  # the swizzle keeps the element set


def test_128b_swizzle_bank_spread(golden):
    case = golden["swizzle"][1]
    sw = golden["swizzle"][0]
    addr = [lay.compose_apply(3, 3, 3, sw["tile_spec"], 64 * i) for i in range(8)]
    assert addr == case["column0_addr"]
    bm = case["bank_model"]
    banks = [(a // 2) % bm["n_banks"] for a in addr]
    assert banks == case["column0_banks_swizzled"]
    plain = [(64 * i // 2) % bm["n_banks"] for i in range(8)]
    assert plain == case["column0_banks_plain"]
    # in the bank model the swizzled column costs one cycle, the plain one eight
    assert lay.lds_access_cycles([2 * a for a in addr], 2, 32, 4, 8) == 1
    assert lay.lds_access_cycles([2 * 64 * i for i in range(8)], 2, 32, 4, 8) == 8


def test_swizzle_needs_atom_len_at_least_swizzle_len():
    assert lay.swizzle(3, 3, 3, 100) >= 0
    with pytest.raises(lay.LayoutError):
        lay.swizzle(3, 3, 2, 100)
    with pytest.raises(lay.LayoutError):
        lay.compose_apply(3, 3, 3, "S[(8,64):(64@m,1@laneid)]", 0)  # tile must only produce m


@pytest.mark.parametrize("mbs", [(3, 3, 3), (3, 2, 3), (3, 1, 3), (3, 3, 4), (2, 2, 5)])
@pytest.mark.parametrize("inner", [True, False])
def test_swizzle_is_a_bijection_per_period(mbs, inner):
    M, B, S = mbs
    period = 1 << (M + S + B)
    out = sorted(lay.swizzle(M, B, S, a, inner) for a in range(period))
    assert out == list(range(period))


def test_offset_and_replica_notation():
    # R[2 : 4@warpid] places two copies four warps apart; 5@warpid shifts by five
    spec = "S[4:1@laneid] + R[2 : 4@warpid] + 5@warpid"
    assert lay.apply(spec, 3) == {"laneid": 3, "warpid": 5}
    assert lay.replicas(spec) == [{}, {"warpid": 4}]
    # an untagged stride goes to the default axis m; an axis may repeat
    assert lay.apply("S[(2,3):(3,1)]", 1, 2, shape=[2, 3]) == {"m": 5}
    assert lay.apply("S[(2,2):(1@laneid,2@laneid)]", 3) == {"laneid": 3}
    for bad in ["S[(2,3):(1)]", "S[(2):(1@nosuchaxis)]", "R[2:1]", "S[(0):(1)]", "S[(2):(1)] + S[2:1]"]:
        with pytest.raises(lay.LayoutError):
            lay.size(bad)


def test_mfma_fragment_specs_parse_as_documented():
    """The gfx950 fragment maps the kernels assume, written in the pages'
    notation.  The pages do not cover AMD matrix cores: these maps are pinned
    on the device by the one-hot and integer-pattern GEMM tests, not here."""
    op = "S[(32,2,8):(1@laneid,32@laneid,1@m)]"
    for row in range(32):
        for k in range(16):
            assert lay.apply(op, row, k, shape=[32, 16]) == {"laneid": row + 32 * (k // 8), "m": k % 8}
    acc = "S[(4,2,4,32):(4@m,32@laneid,1@m,1@laneid)]"
    seen = set()
    for r in range(32):
        for c in range(32):
            got = lay.apply(acc, r, c, shape=[32, 32])
            v, l = got["m"], got["laneid"]
            assert r == 8 * (v // 4) + 4 * (l // 32) + v % 4 and c == l % 32
            seen.add((l, v))
    assert len(seen) == 1024
    # the 16×16×32 shape of the 256×256 kernel: operand lane = row + 16·(k/8),
    # element k mod 8; accumulator (inputs swapped) D row = lane mod 16,
    # D col = 4·(lane/16) + register
    op16 = "S[(16,4,8):(1@laneid,16@laneid,1@m)]"
    for row in range(16):
        for k in range(32):
            assert lay.apply(op16, row, k, shape=[16, 32]) == {"laneid": row + 16 * (k // 8), "m": k % 8}
    acc16 = "S[(16,4,4):(1@laneid,16@laneid,1@m)]"
    seen = set()
    for r in range(16):
        for c in range(16):
            got = lay.apply(acc16, r, c, shape=[16, 16])
            v, l = got["m"], got["laneid"]
            assert r == l % 16 and c == 4 * (l // 16) + v
            seen.add((l, v))
    assert len(seen) == 256


def _fragment_read_addrs(compose, rows_base=0, kk=0):
    """Byte addresses of one 128-bit MFMA fragment read: lane l reads row
    (l & 31) at K-chunk 2·kk + (l >> 5) of a (rows × 64) fp16 LDS tile."""
    M, B, S = compose
    out = []
    for l in range(64):
        r = rows_base + (l & 31)
        c = 2 * kk + (l >> 5)
        out.append(2 * lay.compose_apply(M, B, S, "S[(256,64):(64@m,1@m)]", r * 64 + 8 * c))
    return out


@pytest.mark.parametrize("rows_base", [0, 32, 96])
@pytest.mark.parametrize("kk", [0, 1, 3])
def test_operand_swizzle_choice_under_bank_models(rows_base, kk):
    """Why the kernels use ComposeLayout(3, 3, 4) rather than the pages'
    128-byte mode (3, 3, 3): a 128-bit LDS read served 16 lanes per pass by 64
    four-byte banks (the model gfx950's bank-conflict counter confirmed: 2-way
    conflicts with (3,3,3), none with (3,3,4)) needs 16 consecutive rows on 16
    distinct 16-byte slots of a 256-byte bank line.  Under the pages' own
    32-bank, 8-lanes-per-pass model both are conflict-free."""
    pages = _fragment_read_addrs((3, 3, 3), rows_base, kk)
    pairs = _fragment_read_addrs((3, 3, 4), rows_base, kk)
    assert lay.lds_access_cycles(pages, 16, 64, 4, 16) == 8   # 4 passes × 2-way
    assert lay.lds_access_cycles(pairs, 16, 64, 4, 16) == 4   # 4 passes, no conflict
    assert lay.lds_access_cycles(pages, 16, 32, 4, 8) == 8    # 8 passes, no conflict
    # the direct-to-LDS copy writes 64 consecutive 16-byte slots per wave
    # instruction: conflict-free whatever the swizzle
    linear = [16 * l for l in range(64)]
    assert lay.lds_access_cycles(linear, 16, 64, 4, 16) == 4
