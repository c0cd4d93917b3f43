"""GPU parity of paro_w4a16_moe_linear (experts stacked in one tensor, one
rotation shared by all experts) against the oracle's composition of
per-expert linears, through the C-ABI.

Each expert's rows must meet the linear gate (5e-3 of the largest |Y| of that
expert's rows, plus one output rounding for a 16-bit y).  Cases: skewed
routing with an empty expert, experts of one row, expert boundaries inside a
16-row tile and inside a 256-row tile, all rows to one expert, no rows routed
at all, more tiles than the persistent workgroups, G = 64, and the
Mixtral-8x7B-shaped expert projection at 2048 tokens x top-2 on sampled rows.
Rows outside every expert's range must stay untouched, and offsets past the
row count are clamped.
"""
import numpy as np
import pytest

import synth
from _helpers import LIN_TOL, U, bits_to_f64, sample_rows, say, to_host_bits, torch_dtype, x_to_device
from oracle import ref

torch = pytest.importorskip("torch")
paro = pytest.importorskip("rotation_int4_weight_amd")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    paro.load()
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    yield
    torch.cuda.synchronize()


def run_moe(D, E, offs, x, dt, y_dt, rows_total=None):
    M = x.shape[0]
    xd = x_to_device(x, dt)
    od = torch.from_numpy(np.asarray(offs, dtype=np.int64)).cuda()
    y = torch.full((M, D.out_features), float("nan"), dtype=torch_dtype(y_dt), device="cuda")
    ws = paro.make_workspace(paro.paro_w4a16_moe_linear_workspace_bytes(D, M, dt))
    paro.paro_w4a16_moe_linear(D, E, od, xd, y, ws)
    torch.cuda.synchronize()
    return to_host_bits(y)


def check_moe(Lm, E, offs, x, dt, rows=None, label=""):
    D = paro.DeviceLayer(Lm)
    M = x.shape[0]
    say(f"moe {label} E={E} I={Lm.in_features} O={Lm.out_features} rows={M} offsets={list(offs)[:9]}")
    for y_dt in (synth.F32, dt):
        yh = run_moe(D, E, offs, x, dt, y_dt)
        for e in range(E):
            lo, hi = int(offs[e]), int(offs[e + 1])
            if hi <= lo:
                continue
            r = np.arange(lo, hi) if rows is None else np.array([m for m in rows if lo <= m < hi])
            if r.size == 0:
                continue
            rc, err, mref, _ = ref.paro_linear_ref_check(ref.expert_layer(Lm, e), np.ascontiguousarray(x[r]), dt,
                                                         np.ascontiguousarray(yh[r]), y_dt,
                                                         LIN_TOL + (U[y_dt] if y_dt != synth.F32 else 0.0))
            assert rc == ref.OK, f"expert {e} rows {lo}..{hi}: off by {err / mref:.3e} of max|Y|"
    return yh


@pytest.mark.parametrize("I,O,E,offs,dt", [
    (256, 136, 4, [0, 100, 100, 101, 300], synth.F16),           # empty expert, a one-row expert
    (512, 256, 3, [0, 7, 263, 300], synth.BF16),                 # boundaries inside 16- and 256-row tiles
    (384, 64, 2, [0, 0, 90], synth.BF16),                        # all rows to one expert
    (256, 200, 5, [0, 17, 34, 51, 68, 85], synth.F16),
])
def test_moe_matches_oracle(I, O, E, offs, dt):
    Lm = synth.make_moe_layer(610, E, I, O)
    x = synth.make_x(610, 1, offs[-1], I, dt)
    check_moe(Lm, E, np.array(offs), x, dt)


def test_moe_group_64_and_random_routing():
    E, I, O = 6, 512, 264
    Lm = synth.make_moe_layer(611, E, I, O, group_size=64)
    offs = synth.make_routing(611, E, 300, 2)
    x = synth.make_x(611, 1, int(offs[-1]), I, synth.BF16)
    check_moe(Lm, E, offs, x, synth.BF16, label="G=64")


def test_moe_uncovered_rows_untouched_and_offsets_clamped():
    """Offsets end before the last row: those rows keep their contents; a
    final offset past the row count is clamped to it."""
    E, I, O, M = 3, 256, 64, 80
    Lm = synth.make_moe_layer(612, E, I, O)
    x = synth.make_x(612, 1, M, I, synth.F16)
    D = paro.DeviceLayer(Lm)
    yh = run_moe(D, E, [0, 20, 50, 60], x, synth.F16, synth.F32)
    assert np.isnan(yh[60:]).all() and np.isfinite(yh[:60]).all()
    y_clamped = run_moe(D, E, [0, 20, 50, 10 ** 9], x, synth.F16, synth.F32)
    want = ref.moe_linear(Lm, [0, 20, 50, 80], x, synth.F16)
    rc, err, mref, _ = ref.paro_linear_ref_check(ref.expert_layer(Lm, 2), np.ascontiguousarray(x[50:]), synth.F16,
                                                 np.ascontiguousarray(y_clamped[50:]), synth.F32, LIN_TOL)
    assert rc == ref.OK and np.isfinite(want).all()


def test_moe_single_expert_equals_the_linear():
    I, O, M = 512, 256, 300
    L = synth.make_layer(613, 0, I, O)
    Lm = synth.Layer(I, O, 128, L.krot, L.pairs, L.theta, L.channel_scales, L.qweight[None], L.qzeros[None],
                     L.scales[None], L.bias[None])
    x = synth.make_x(613, 0, M, I, synth.BF16)
    y_moe = run_moe(paro.DeviceLayer(Lm), 1, [0, M], x, synth.BF16, synth.F32)
    D = paro.DeviceLayer(L)
    y = torch.empty((M, O), dtype=torch.float32, device="cuda")
    paro.paro_w4a16_linear(D, x_to_device(x, synth.BF16), y,
                           paro.make_workspace(paro.paro_w4a16_linear_workspace_bytes(D, M, synth.BF16, 3)), path=3)
    torch.cuda.synchronize()
    assert np.array_equal(y_moe.view(np.uint32), y.cpu().numpy().view(np.uint32))


def test_moe_full_size_sampled():
    spec = synth.MOE_WORKLOADS[5]
    _, I, O = spec["layer"]
    E = spec["experts"]
    Lm = synth.make_moe_layer(5, E, I, O)
    offs = synth.make_routing(5, E, spec["tokens"], spec["top_k"])
    x = synth.make_x(5, 0, int(offs[-1]), I, spec["act"])
    rows = np.unique(np.concatenate([sample_rows(int(offs[-1]), 40), offs[1:-1], offs[1:-1] - 1]))
    rows = rows[(rows >= 0) & (rows < offs[-1])]
    check_moe(Lm, E, offs, x, spec["act"], rows=rows, label="mixtral w1")


def test_moe_all_experts_empty():
    """Offsets that give no expert any row: the launch has no tile, every
    workgroup leaves at once, and y keeps its contents."""
    E, I, O, M = 4, 256, 128, 40
    Lm = synth.make_moe_layer(614, E, I, O)
    x = synth.make_x(614, 1, M, I, synth.BF16)
    yh = run_moe(paro.DeviceLayer(Lm), E, [0, 0, 0, 0, 0], x, synth.BF16, synth.F32)
    assert np.isnan(yh).all()


def test_moe_more_tiles_than_workgroups():
    """More (expert block, column tile) pairs than the 256 persistent
    workgroups: each workgroup takes several tiles, across expert boundaries,
    in turn."""
    E, I, O = 5, 256, 4096
    Lm = synth.make_moe_layer(615, E, I, O)
    offs = synth.make_routing(615, E, 1300, 2)
    x = synth.make_x(615, 1, int(offs[-1]), I, synth.BF16)
    items = sum(-(-(int(offs[e + 1]) - (int(offs[e]) & ~15)) // 256) for e in range(E) if offs[e + 1] > offs[e])
    assert items * (O // 128) > 256
    rows = np.unique(np.concatenate([sample_rows(int(offs[-1]), 64, seed=615), offs[1:-1], offs[1:-1] - 1]))
    rows = rows[(rows >= 0) & (rows < offs[-1])]
    check_moe(Lm, E, offs, x, synth.BF16, rows=rows, label="persistent")
