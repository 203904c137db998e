"""GPU parity of quantize_rows_e4m3 against the oracle's quantiser: bit-exact codes and scales."""
import numpy as np
import pytest
import torch

import attention_flash_attn_fwd_amd as fa
import oracle
from tests.helpers import dev, say
from workloads import make_quantize, make_mla_prefill, workload

pytestmark = pytest.mark.gpu

QZ = "quantize_e4m3_rows_b1_s8192_h128_d128"


def _check(x: np.ndarray, what: str):
    say(f"case quantize {what} shape={x.shape}")
    codes, scale = fa.quantize_rows_e4m3(dev(x))
    torch.cuda.synchronize()
    rc, rs = oracle.quantize_rows(x)
    got_s = scale.cpu().numpy()
    got_c = codes.cpu().numpy()
    bad_s = np.flatnonzero(got_s.view(np.uint32).ravel() != rs.view(np.uint32).ravel())
    assert bad_s.size == 0, f"{what}: {bad_s.size} scales differ, first row {bad_s[0]}"
    bad = np.flatnonzero(got_c.ravel() != rc.ravel())
    assert bad.size == 0, (f"{what}: {bad.size} codes differ; first at {bad[0]}: "
                           f"x={x.ravel()[bad[0]]!r} got {got_c.ravel()[bad[0]]:#x} want {rc.ravel()[bad[0]]:#x}")


@pytest.mark.parametrize("rows,cols", [(1, 4), (3, 8), (37, 64), (1000, 128), (5, 132), (17, 256), (9, 1000), (4, 4096)])
def test_quantize_random_rows(rows, cols):
    rng = np.random.default_rng(rows * 7919 + cols)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x *= np.exp2(rng.uniform(-40, 40, (rows, 1))).astype(np.float32)   # row magnitudes over 80 binades
    _check(x, f"random {rows}x{cols}")


def test_quantize_edge_rows():
    cols = 128
    rows = []
    rows.append(np.zeros(cols))                                     # all zero: scale 1, codes 0
    r = np.zeros(cols); r[5] = -3.0; rows.append(r)                 # one non-zero
    r = np.full(cols, -0.0); r[0] = 1.0; rows.append(r)             # negative zeros
    rows.append(np.full(cols, 7.25))                                # constant row: every code is 448
    r = np.linspace(-1, 1, cols); rows.append(r)
    rows.append(np.float32(1e-38) * np.linspace(-1, 1, cols))       # subnormal fp32 inputs
    rows.append(np.float32(3e38) * np.linspace(-1, 1, cols))        # near the fp32 maximum
    # amax 448 makes the scale exactly 1: put every e4m3 midpoint and code point in the row
    grid = oracle.E4M3_TABLE[:0x7F]
    mids = (grid[:-1] + grid[1:]) / 2
    r = np.zeros(cols); r[0] = 448.0; r[1:1 + 126] = mids[:126]; rows.append(r)
    r = np.zeros(cols); r[:127] = grid; r[127] = -448.0; rows.append(r)
    # quotients just around the subnormal / normal boundary of e4m3
    r = np.full(cols, 2.0 ** -6) * np.linspace(0.5, 1.5, cols); r[0] = 448.0; rows.append(r)
    x = np.asarray(rows, dtype=np.float32)
    _check(x, "edge rows")


def test_quantize_full_workload_sampled():
    """The full workload (8192 tokens x 128 heads rows of 128) in one launch; every code and
    scale of sampled token blocks against the oracle, and the whole output against the MLA
    prefill workload's stored q_nope codes, which are quantised from the same draws."""
    w = workload(QZ)
    say(f"case {w.name}")
    d = make_quantize(w)
    x = d["x"]
    codes, scale = fa.quantize_rows_e4m3(dev(x))
    torch.cuda.synchronize()
    got_c, got_s = codes.cpu().numpy(), scale.cpu().numpy()
    for t0 in (0, 4096 - 16, 8192 - 16):
        rc, rs = oracle.quantize_rows(x[:, t0:t0 + 16])
        assert (got_c[:, t0:t0 + 16] == rc).all(), t0
        assert (got_s[:, t0:t0 + 16].view(np.uint32) == rs.view(np.uint32)).all(), t0
    m = make_mla_prefill(workload("mla_prefill_fp8_causal_b1_h128_s8192", Skv=16))
    assert (got_c == m["q_nope"]).all()
    assert (got_s == m["q_scale"]).all()


def test_quantize_empty():
    x = torch.empty((0, 128), dtype=torch.float32, device="cuda")
    codes, scale = fa.quantize_rows_e4m3(x)
    assert codes.shape == (0, 128) and scale.shape == (0,)
