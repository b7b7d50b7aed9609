"""The host planner (through rr_plan_query, no GPU needed): every supported N gets
a compiled configuration that holds the row, the grid path appears only past
one workgroup's capacity, workspace sizes follow the documented layout, and the
test-only overrides reach every path."""
import pytest

import memory_bound_row_softmax_amd as rr

ROW_OPS = (rr.RR_OP_SOFTMAX, rr.RR_OP_RMSNORM, rr.RR_OP_XENT_GRAD, rr.RR_OP_SOFTMAX_BWD)
NS = [1, 2, 3, 7, 100, 255, 256, 257, 1000, 1024, 2048, 4095, 4096, 4097, 8192, 16384, 32768,
      65535, 65536, 65537, 131072, 200000, 262144, 524288, 1 << 20]


@pytest.mark.parametrize("op", ROW_OPS)
@pytest.mark.parametrize("dt", (rr.RR_F32, rr.RR_BF16))
@pytest.mark.parametrize("vec", (True, False))
def test_row_plans_hold_the_row(op, dt, vec):
    for N in NS:
        if N > 262144:  # beyond the guaranteed range: either a plan that holds it, or refused
            try:
                p = rr.rr_plan_query(op, 16384, N, dt, vec)
            except rr.RRError as e:
                assert e.status == rr.RR_ERR_UNSUPPORTED
                continue
        else:
            p = rr.rr_plan_query(op, 16384, N, dt, vec)
        P, R, G = p["vals_per_lane"], p["lanes_per_row"], p["groups_per_row"]
        if p["path"] == 4:  # past every on-chip plan: the two-pass long-row kernel
            assert N > 262144
            assert p["max_n"] == 1 << 28 and G in (16, 32, 64) and p["ws_bytes"] > 0
            continue
        assert p["max_n"] == P * R * G >= N
        assert p["vectorized"] == int(vec)
        if p["path"] == 0:  # block kernel: a few rows per workgroup, one workgroup per row
            assert G == 1 and N <= 65536
            assert p["block_threads"] == max(R, 256) and p["rows_per_block"] * R == p["block_threads"]
            # the narrowest lane group that holds the row (at least 16 lanes)
            assert R == 16 or (R // 2) * P < N
            assert p["ws_bytes"] == 0
        else:  # stream kernel: one row per workgroup at a time, at least half full
            assert p["path"] == (1 if G > 1 else 3) and N >= 2048
            assert 2 * N >= P * R or not vec
            assert p["block_threads"] == R and p["rows_per_block"] == 1
            # a row is split only over as many workgroups as it needs
            assert G == 1 or (G // 2) * P * R < N
            assert p["ws_bytes"] == (256 + 1024 * (64 + 64 * G) if G > 1 else 0)
    if op in (rr.RR_OP_SOFTMAX, rr.RR_OP_RMSNORM):  # long rows: read twice, up to 2^28
        q = rr.rr_plan_query(op, 16, (1 << 22) + 1, dt, vec)
        if op == rr.RR_OP_RMSNORM and vec:  # on chip at any fill, to 2^23 (packed bf16 2^24)
            cap = 1 << (24 if dt == rr.RR_BF16 else 23)
            assert q["path"] == 1 and q["vals_per_lane"] == (128 if dt == rr.RR_BF16 else 64)
            assert rr.rr_plan_query(op, 16, cap, dt, vec)["path"] == 1
            assert rr.rr_plan_query(op, 16, cap + 1, dt, vec)["path"] == 4
        else:
            assert q["path"] == 4
        with pytest.raises(rr.RRError):
            rr.rr_plan_query(op, 16, (1 << 28) + 1, dt, vec)
    else:  # backward ops: read twice past the on-chip plans, up to 2^28
        assert rr.rr_plan_query(op, 16, (1 << 21) + 1, dt, vec)["path"] == 4
        with pytest.raises(rr.RRError):
            rr.rr_plan_query(op, 16, (1 << 28) + 1, dt, vec)


def test_rows_up_to_8m_elements_stay_on_chip():
    """Aligned rows of 2^21 to 2^22 elements are split over 128 workgroups (64 values
    on 512 lanes; bf16 RMSNorm packed, 64 workgroups of 128 values), rows of 2^22 to
    2^23 over 256 (packed bf16 RMSNorm: 128), and read once; the softmax on 128 and
    on 256 only from 9/10 full, the RMSNorm at any fill; the per-element path past
    2^18 reads twice."""
    def cap_ok(N, cap):
        return 10 * N >= 9 * cap
    for N in ((1 << 21) + 1, 3_000_000, 3_774_874, 1 << 22, (1 << 22) + 1, 6_000_000,
              7_549_747, 7_549_748, 1 << 23):
        big = N > 1 << 22
        G = 256 if big else 128
        for dt in (rr.RR_F32, rr.RR_BF16):
            for op in (rr.RR_OP_SOFTMAX, rr.RR_OP_RMSNORM):
                p = rr.rr_plan_query(op, 256, N, dt)
                packed = op == rr.RR_OP_RMSNORM and dt == rr.RR_BF16
                g = G // 2 if packed else G
                vals = 128 if packed else 64
                if op == rr.RR_OP_SOFTMAX and not cap_ok(N, vals * 512 * g):
                    assert p["path"] == 4, (op, dt, N, p)
                    continue
                assert (p["path"], p["vals_per_lane"], p["lanes_per_row"], p["groups_per_row"]) == \
                    (1, vals, 512, g), (op, dt, N, p)
                assert p["ws_bytes"] == 256 + 256 * (64 + 64 * g)
        # the backward ops read their rows twice past their on-chip plans
        for op in (rr.RR_OP_XENT_GRAD, rr.RR_OP_SOFTMAX_BWD):
            assert rr.rr_plan_query(op, 256, N, rr.RR_F32)["path"] == 4
    for dt in (rr.RR_F32, rr.RR_BF16):
        assert rr.rr_plan_query(rr.RR_OP_SOFTMAX, 256, 1 << 22, dt, False)["path"] == 4
        assert rr.rr_plan_query(rr.RR_OP_SOFTMAX, 256, (1 << 23) + 1, dt)["path"] == 4
    # bf16 softmax on 64 workgroups only from 9/10 full; fp32 at any fill
    assert rr.rr_plan_query(rr.RR_OP_SOFTMAX, 256, 1_500_000, rr.RR_BF16)["path"] == 4
    assert rr.rr_plan_query(rr.RR_OP_SOFTMAX, 256, 1_900_000, rr.RR_BF16)["groups_per_row"] == 64
    assert rr.rr_plan_query(rr.RR_OP_SOFTMAX, 256, 1_500_000, rr.RR_F32)["groups_per_row"] == 64


def test_bf16_softmax_rows_take_exactly_the_workgroups_they_need():
    """bf16 softmax rows that need 3, 5 or 6 workgroups of 64 values x 512 lanes get
    exactly that many (seven take eight, four keep the table's 64 x 256 x 8); fp32
    softmax rows that need 5 or 6 too; bf16 cross-entropy gradient rows of 32769 to
    262144 elements take exactly ceil(N / 16384) workgroups of 64 x 256; other fp32
    rows and forced plans keep powers of two."""
    for N, (P, R, G) in ((70000, (64, 512, 3)), (100000, (64, 256, 8)), (151936, (64, 512, 5)),
                         (180000, (64, 512, 6)), (200000, (64, 512, 8)), (262144, (64, 512, 8))):
        p = rr.rr_plan_query(rr.RR_OP_SOFTMAX, 16384, N, rr.RR_BF16)
        assert (p["vals_per_lane"], p["lanes_per_row"], p["groups_per_row"]) == (P, R, G), (N, p)
        assert p["ws_bytes"] == 256 + 1024 * (64 + 64 * G)
        f32 = rr.rr_plan_query(rr.RR_OP_SOFTMAX, 16384, N, rr.RR_F32)
        want = {151936: 5, 180000: 6}.get(N)
        if want:
            assert (f32["vals_per_lane"], f32["lanes_per_row"], f32["groups_per_row"]) == (64, 512, want)
        else:
            assert f32["groups_per_row"] in (2, 4, 8), (N, f32)
        # the fp32 cross-entropy gradient keeps powers of two
        assert rr.rr_plan_query(rr.RR_OP_XENT_GRAD, 8192, N, rr.RR_F32)["groups_per_row"] in (2, 4, 8, 16)
    for N, G in ((32768, None), (32769, 3), (49152, 3), (65536, 4), (70000, 5), (90000, 6),
                 (100000, 7), (131072, 8), (151936, 10), (180000, 11), (200000, 13),
                 (262144, 16), (262145, None)):
        p = rr.rr_plan_query(rr.RR_OP_XENT_GRAD, 16384, N, rr.RR_BF16)
        if G is None:
            assert (p["lanes_per_row"], p["groups_per_row"]) != (256, (N + 16383) // 16384), (N, p)
        else:
            assert (p["path"], p["vals_per_lane"], p["lanes_per_row"], p["groups_per_row"]) == \
                (1, 64, 256, G), (N, p)
            assert p["ws_bytes"] == 256 + 1024 * (64 + 64 * G)
    # also with few rows
    for M, N, G in ((512, 40000, 3), (4096, 65536, 4), (256, 151936, 10)):
        p = rr.rr_plan_query(rr.RR_OP_XENT_GRAD, M, N, rr.RR_BF16)
        assert (p["path"], p["lanes_per_row"], p["groups_per_row"]) == (1, 256, G), (M, N, p)
    # the per-element path has no such plans
    assert rr.rr_plan_query(rr.RR_OP_SOFTMAX, 16384, 151935, rr.RR_BF16, False)["groups_per_row"] in (4, 8, 16)


@pytest.mark.parametrize("dt", (rr.RR_F32, rr.RR_BF16))
def test_cross_entropy_gradient_runs_the_softmax_kernels(dt):
    """The fused gradient runs the softmax kernels with its own measured plans: the
    same kinds of plan, never fp32 with 32 values on 1024 lanes (it would not fit
    the registers), and the same workspace layout."""
    for N in NS[:-2]:
        for vec in (True, False):
            b = rr.rr_plan_query(rr.RR_OP_XENT_GRAD, 8192, N, dt, vec)
            assert b["max_n"] >= N and b["path"] in (0, 1, 3)
            if dt == rr.RR_F32 and b["path"] != 0:
                assert (b["vals_per_lane"], b["lanes_per_row"]) != (32, 1024)


def test_workspace_scales_with_rows_up_to_the_group_cap():
    N = 131072
    small = rr.workspace_bytes(rr.RR_OP_SOFTMAX, 3, N, rr.RR_F32)
    big = rr.workspace_bytes(rr.RR_OP_SOFTMAX, 100000, N, rr.RR_F32)
    # the larger of the 128-bit and the per-element plans
    G = max(rr.rr_plan_query(rr.RR_OP_SOFTMAX, 3, N, rr.RR_F32, v)["groups_per_row"]
            for v in (True, False))
    assert small == 256 + 3 * (64 + 64 * G)
    assert big == 256 + 1024 * (64 + 64 * G)
    assert rr.workspace_bytes(rr.RR_OP_SOFTMAX, 0, N, rr.RR_F32) == 0
    assert rr.workspace_bytes(rr.RR_OP_XENT, 8192, N, rr.RR_F32) == 0


@pytest.mark.parametrize("dt", (rr.RR_F32, rr.RR_BF16))
def test_cross_entropy_streams(dt):
    for N in NS + [(1 << 22) + 3]:
        p = rr.rr_plan_query(rr.RR_OP_XENT, 8192, N, dt)
        assert p["path"] == 2 and p["groups_per_row"] == 1 and p["ws_bytes"] == 0
        assert p["vals_per_lane"] in (16, 32) and 16 <= p["lanes_per_row"] <= (512 if dt else 256)
    # bf16 rows of 1025..32767 elements take the least padding in two to eight steps; f32 one
    for N, lanes in ((2048, 64 >> dt), (3000, 128 >> (2 * dt)), (4096, 128 >> dt), (8192, 256 >> dt), (16384, 256)):
        assert rr.rr_plan_query(rr.RR_OP_XENT, 8192, N, dt)["lanes_per_row"] == lanes, N


def test_forced_configurations(overrides):
    overrides.set(P=64)
    overrides.set(R=256)
    overrides.set(G=4)
    p = rr.rr_plan_query(rr.RR_OP_SOFTMAX, 50, 3000, rr.RR_F32)
    assert (p["vals_per_lane"], p["lanes_per_row"], p["groups_per_row"], p["path"]) == (64, 256, 4, 1)
    assert p["ws_bytes"] == 256 + 50 * (64 + 64 * 4)
    # too small for the row
    with pytest.raises(rr.RRError):
        rr.rr_plan_query(rr.RR_OP_SOFTMAX, 50, 70000, rr.RR_F32)
    # a stream kernel with one workgroup per row
    overrides.set(kind="stream")
    overrides.set(G=1)
    p = rr.rr_plan_query(rr.RR_OP_RMSNORM, 50, 3000, rr.RR_BF16)
    assert (p["path"], p["groups_per_row"], p["block_threads"], p["ws_bytes"]) == (3, 1, 256, 0)
    # not compiled for RMSNorm (would not fit in registers): 64 values x 1024 lanes
    overrides.set(kind="block")
    overrides.set(R=1024)
    with pytest.raises(rr.RRError):
        rr.rr_plan_query(rr.RR_OP_RMSNORM, 50, 3000, rr.RR_F32)
    # no block kernel splits a row
    overrides.set(G=2)
    with pytest.raises(rr.RRError):
        rr.rr_plan_query(rr.RR_OP_SOFTMAX, 50, 3000, rr.RR_F32)
    overrides.set(kind=None)
    overrides.set(G=None)
    overrides.set(P=16)
    overrides.set(R=64)
    p = rr.rr_plan_query(rr.RR_OP_XENT, 50, 3000, rr.RR_F32)
    assert (p["vals_per_lane"], p["lanes_per_row"]) == (16, 64)


def test_short_unaligned_rows_take_small_lane_groups(overrides):
    """Unaligned bf16 rows shorter than 16 bytes are read element by element, which
    only lane groups of fewer than 64 lanes compile: default plans use those (for
    fp32 too), and forced bf16 plans with whole waves per row are refused."""
    ops = (rr.RR_OP_SOFTMAX, rr.RR_OP_RMSNORM, rr.RR_OP_XENT, rr.RR_OP_XENT_GRAD,
           rr.RR_OP_SOFTMAX_BWD, rr.RR_OP_RMSNORM_BWD)
    for dt, size in ((rr.RR_F32, 4), (rr.RR_BF16, 2)):
        for N in range(1, 16 // size):
            for op in ops:
                p = rr.rr_plan_query(op, 100, N, dt, False)
                assert p["lanes_per_row"] < 64, (op, N, dt, p)
    overrides.set(kind="long")
    with pytest.raises(rr.RRError):
        rr.rr_plan_query(rr.RR_OP_SOFTMAX, 70, 7, rr.RR_BF16, False)
    assert rr.rr_plan_query(rr.RR_OP_SOFTMAX, 70, 9, rr.RR_BF16, False)["path"] == 4
    assert rr.rr_plan_query(rr.RR_OP_SOFTMAX, 70, 3, rr.RR_F32, False)["path"] == 4
    overrides.set(kind="stream")
    overrides.set(P=16)
    overrides.set(R=1024)
    with pytest.raises(rr.RRError):
        rr.rr_plan_query(rr.RR_OP_RMSNORM, 70, 7, rr.RR_BF16, False)
    assert rr.rr_plan_query(rr.RR_OP_RMSNORM, 70, 9, rr.RR_BF16, False)["lanes_per_row"] == 1024


def test_unaligned_bf16_split_rows_take_wide_lanes():
    """Unaligned bf16 softmax and RMSNorm rows split over 2 to 8 workgroups take 32
    values on 512 lanes up to 81920 elements, and cross-entropy gradient rows past
    32768 elements; other ops, fp32 and longer rows keep 16 values per lane on the
    per-element path."""
    for op in (rr.RR_OP_SOFTMAX, rr.RR_OP_RMSNORM):
        for N in (16385, 32001, 50257, 65537, 81920):
            p = rr.rr_plan_query(op, 8192, N, rr.RR_BF16, False)
            assert (p["vals_per_lane"], p["lanes_per_row"]) == (32, 512), (op, N, p)
            assert 2 <= p["groups_per_row"] <= 8
        for N in (81921, 100001, 151935):
            assert rr.rr_plan_query(op, 8192, N, rr.RR_BF16, False)["vals_per_lane"] == 16
        for N in (32001, 50257):
            assert rr.rr_plan_query(op, 8192, N, rr.RR_F32, False)["vals_per_lane"] <= 16
    for N in (32769, 50257, 81920):
        p = rr.rr_plan_query(rr.RR_OP_XENT_GRAD, 8192, N, rr.RR_BF16, False)
        assert (p["vals_per_lane"], p["lanes_per_row"]) == (32, 512), (N, p)
        assert 2 <= p["groups_per_row"] <= 8
    assert rr.rr_plan_query(rr.RR_OP_XENT_GRAD, 8192, 100001, rr.RR_BF16, False)["vals_per_lane"] == 16
    assert rr.rr_plan_query(rr.RR_OP_SOFTMAX_BWD, 8192, 50257, rr.RR_BF16, False)["vals_per_lane"] <= 16


def test_invalid_plan_arguments():
    for args in ((rr.RR_OP_SOFTMAX, -1, 10, rr.RR_F32), (rr.RR_OP_SOFTMAX, 4, 0, rr.RR_F32),
                 (7, 4, 10, rr.RR_F32), (rr.RR_OP_SOFTMAX, 4, 10, 3),
                 (rr.RR_OP_XENT, 4, 1 << 31, rr.RR_F32)):
        with pytest.raises(rr.RRError) as e:
            rr.rr_plan_query(*args)
        assert e.value.status == rr.RR_ERR_INVALID_ARGUMENT


def test_workspace_covers_the_element_path():
    # N * 4 bytes not a multiple of 16: the per-element plan splits the row further
    for op in (rr.RR_OP_SOFTMAX, rr.RR_OP_RMSNORM):
        for N in (40000, 65537, 131072):
            need = rr.workspace_bytes(op, 6, N, rr.RR_F32)
            for vec in (True, False):
                assert rr.rr_plan_query(op, 6, N, rr.RR_F32, vec)["ws_bytes"] <= need


@pytest.mark.parametrize("dt", (rr.RR_F32, rr.RR_BF16))
@pytest.mark.parametrize("vec", (True, False))
def test_rmsnorm_bwd_plans(dt, vec):
    """Persistent kernels: one workgroup per row up to 16384 elements, then split;
    the workspace holds the exchange area and one fp32 partial row per row group.
    Unaligned fp32 rows keep at most 16 values per lane."""
    for N in NS:
        lim = 262144
        if N > lim:
            with pytest.raises(rr.RRError):
                rr.rr_plan_query(rr.RR_OP_RMSNORM_BWD, 16384, N, dt, vec)
            continue
        p = rr.rr_plan_query(rr.RR_OP_RMSNORM_BWD, 16384, N, dt, vec)
        P, R, G = p["vals_per_lane"], p["lanes_per_row"], p["groups_per_row"]
        assert P * R * G == p["max_n"] >= N and P in (8, 16, 32) and (vec or dt == rr.RR_BF16 or P <= 16)
        assert p["path"] == (1 if G > 1 else 3)
        assert G == 1 or (N > 8192 and (G // 2) * P * R < N)
        assert p["rows_per_block"] == (max(256, R) // R if G == 1 else 1)
        parts = min(1024 // G, -(-16384 // p["rows_per_block"]))
        assert p["ws_bytes"] >= parts * N * 4
    # a handful of rows: as many partial rows as row blocks
    p = rr.rr_plan_query(rr.RR_OP_RMSNORM_BWD, 3, 4096, dt, vec)
    blocks = -(-3 // p["rows_per_block"])
    assert p["ws_bytes"] >= blocks * 4096 * 4 and p["ws_bytes"] < 16 * 4096 * 4


def test_long_rows_take_the_two_pass_kernel(overrides):
    for op in (rr.RR_OP_SOFTMAX, rr.RR_OP_RMSNORM):
        for dt in (rr.RR_F32, rr.RR_BF16):
            for n in (1 << 20, 1 << 21, 1 << 22, 1 << 23):
                on_chip = rr.rr_plan_query(op, 1000, n, dt)
                G = on_chip["groups_per_row"]
                assert on_chip["path"] == 1 and G in (16, 32, 64, 128, 256)
                assert on_chip["vals_per_lane"] * on_chip["lanes_per_row"] * G == n
                assert on_chip["ws_bytes"] == 256 + min(1000, 512 if G > 128 else 1024) * (64 + 64 * G)
            for n in ((1 << 22) + 8, 5_000_000, (1 << 23) + 8, (1 << 24) + 8, 1 << 26):
                p = rr.rr_plan_query(op, 1000, n, dt)
                if op == rr.RR_OP_RMSNORM and n <= 1 << (24 if dt == rr.RR_BF16 else 23):
                    assert p["path"] == 1  # on chip at any fill
                    continue
                # enough workgroups that a workgroup's share of the row is at most
                # 512 KiB (16 to 64)
                G = 16
                while G < 64 and n * (4 if dt == rr.RR_F32 else 2) > G * 512 * 1024:
                    G *= 2
                assert p["path"] == 4 and p["lanes_per_row"] == 512 and p["groups_per_row"] == G
                assert p["ws_bytes"] == 256 + 1000 * (64 + 64 * G)
            # the per-element path holds 16 * 1024 * 16 elements on chip
            assert rr.rr_plan_query(op, 10, 262144, dt, False)["path"] == 1
            q = rr.rr_plan_query(op, 10, 262145, dt, False)
            assert q["path"] == 4 and q["vals_per_lane"] == 16
    overrides.set(kind="long")
    assert rr.rr_plan_query(rr.RR_OP_SOFTMAX, 8, 1000, rr.RR_F32)["path"] == 4
    assert rr.rr_plan_query(rr.RR_OP_SOFTMAX_BWD, 8, 1000, rr.RR_F32)["path"] == 4
    assert rr.rr_plan_query(rr.RR_OP_XENT_GRAD, 8, 1000, rr.RR_F32)["path"] == 4
    # the cross-entropy forward streams any row in its own kernel
    assert rr.rr_plan_query(rr.RR_OP_XENT, 8, (1 << 21) + 4, rr.RR_F32)["path"] == 2
    # the per-element path keeps the two-pass kernel past 262144 elements


def test_cross_entropy_gradient_long_rows_take_the_two_pass_kernel():
    """Cross-entropy gradient rows past the on-chip plans (2^21 elements on the 128-bit
    path, 262144 on the per-element path) read the logits twice, up to 2^28 elements,
    on 16 to 64 workgroups per row (the softmax's rule)."""
    for dt, size in ((rr.RR_F32, 4), (rr.RR_BF16, 2)):
        assert rr.rr_plan_query(rr.RR_OP_XENT_GRAD, 64, 1 << 21, dt)["path"] == 1
        assert rr.rr_plan_query(rr.RR_OP_XENT_GRAD, 64, 262144, dt, False)["path"] == 1
        for vec, N in ((True, (1 << 21) + 8), (True, 3_000_000), (True, 1 << 28),
                       (False, 262145), (False, 1_000_003)):
            p = rr.rr_plan_query(rr.RR_OP_XENT_GRAD, 64, N, dt, vec)
            G = 16
            while G < 64 and N * size > G * 512 * 1024:
                G *= 2
            assert (p["path"], p["lanes_per_row"], p["groups_per_row"]) == (4, 512, G), (N, p)
        with pytest.raises(rr.RRError):
            rr.rr_plan_query(rr.RR_OP_XENT_GRAD, 64, (1 << 28) + 1, dt)


def test_softmax_backward_long_rows_take_the_two_pass_kernel():
    """Softmax backward rows past the on-chip plans (2^20 elements on the 128-bit path,
    262144 on the per-element path) read y and dy twice, up to 2^28 elements, on 16 to
    64 workgroups per row: as many as keep a workgroup's share of the two rows at
    about 512 KiB or less."""
    for dt, size in ((rr.RR_F32, 4), (rr.RR_BF16, 2)):
        assert rr.rr_plan_query(rr.RR_OP_SOFTMAX_BWD, 64, 1 << 20, dt)["path"] == 1
        assert rr.rr_plan_query(rr.RR_OP_SOFTMAX_BWD, 64, 262144, dt, False)["path"] == 1
        for vec, N in ((True, (1 << 20) + 8), (True, 3_000_000), (True, 1 << 28),
                       (False, 262145), (False, 1_000_003)):
            p = rr.rr_plan_query(rr.RR_OP_SOFTMAX_BWD, 64, N, dt, vec)
            G = 16
            while G < 64 and 2 * N * size > G * 512 * 1024:
                G *= 2
            assert (p["path"], p["lanes_per_row"], p["groups_per_row"]) == (4, 512, G), (N, p)
            assert p["vals_per_lane"] == (32 if vec else 16)
            assert p["ws_bytes"] == 256 + 64 * (64 + 64 * G)
        with pytest.raises(rr.RRError):
            rr.rr_plan_query(rr.RR_OP_SOFTMAX_BWD, 64, (1 << 28) + 1, dt)


def test_packed_bf16_rmsnorm_stays_on_chip_to_16m_elements():
    """Aligned bf16 RMSNorm rows keep the packed plans at any fill: 128 workgroups up
    to 2^23 elements, 256 (one on every CU) up to 2^24, then the two-pass kernel; the
    per-element path and fp32 take the two-pass kernel past 2^23."""
    for N, G in ((2_200_000, 64), (4_500_000, 128), (6_000_000, 128), (1 << 23, 128),
                 ((1 << 23) + 8, 256), (9_000_000, 256), (15_000_000, 256), (1 << 24, 256)):
        p = rr.rr_plan_query(rr.RR_OP_RMSNORM, 128, N, rr.RR_BF16)
        assert (p["path"], p["vals_per_lane"], p["lanes_per_row"], p["groups_per_row"]) == \
            (1, 128, 512, G), (N, p)
        assert p["ws_bytes"] == 256 + 128 * (64 + 64 * G)
    for M in (1, 300, 1 << 20):  # row groups capped per G: the workspace stays small
        assert rr.rr_plan_query(rr.RR_OP_RMSNORM, M, 1 << 24, rr.RR_BF16)["ws_bytes"] <= \
            (8 << 20) + (256 << 10)
    assert rr.rr_plan_query(rr.RR_OP_RMSNORM, 128, (1 << 24) + 8, rr.RR_BF16)["path"] == 4
    assert rr.rr_plan_query(rr.RR_OP_RMSNORM, 128, (1 << 23) + 8, rr.RR_F32)["path"] == 4
    assert rr.rr_plan_query(rr.RR_OP_RMSNORM, 128, (1 << 23) + 8, rr.RR_BF16, False)["path"] == 4
    # fp32 RMSNorm rows on 256 workgroups at any fill
    assert rr.rr_plan_query(rr.RR_OP_RMSNORM, 128, 4_500_000, rr.RR_F32)["groups_per_row"] == 256
    # the softmax keeps the fill rule on its largest plan
    assert rr.rr_plan_query(rr.RR_OP_SOFTMAX, 128, 6_000_000, rr.RR_F32)["path"] == 4


def test_few_rows_keep_a_row_on_one_workgroup():
    """With few rows, a row one workgroup holds is not split (its exchange would not
    be hidden behind other rows); with many rows the measured split plan stays."""
    for op in (rr.RR_OP_SOFTMAX, rr.RR_OP_RMSNORM):
        few = rr.rr_plan_query(op, 4096, 32768, rr.RR_F32)
        assert few["path"] == 3 and few["groups_per_row"] == 1
        assert few["vals_per_lane"] * few["lanes_per_row"] >= 32768
        many = rr.rr_plan_query(op, 16384, 32768, rr.RR_F32)
        assert many["groups_per_row"] == 2
        # rows one workgroup cannot hold are split whatever M is
        assert rr.rr_plan_query(op, 64, 65536, rr.RR_F32)["groups_per_row"] > 1
        # the per-element path keeps its plan
        assert rr.rr_plan_query(op, 64, 32768, rr.RR_F32, False)["vals_per_lane"] <= 16


def test_every_softmax_plan_fits_the_static_workspace():
    """rr_softmax_fwd_static exchanges through a library array of 8 MiB + 256 KiB per
    GPU: every on-chip softmax plan's workspace fits it, at any number of rows (the
    row groups are capped per G)."""
    limit = (8 << 20) + (256 << 10)
    for dt in (rr.RR_F32, rr.RR_BF16):
        for N in (65536, 1 << 20, 1 << 21, 1 << 22, 1 << 23):
            for M in (1, 300, 1 << 20):
                p = rr.rr_plan_query(rr.RR_OP_SOFTMAX, M, N, dt)
                assert p["ws_bytes"] <= limit, (dt, N, M, p)
