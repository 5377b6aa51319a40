"""GPU checks of the chained plans' failure reporting and of launches on a stream that is not the current one.

A chained plan hands states (or adjoints) between pieces of a sequence through ready flags in the workspace.
Here the test hook SSM_TEST_NEVER_READY=1 makes every wait poll a word that no one sets, with a spin limit of 64
polls, so every wait runs out quickly and every kernel still ends normally: the call must report
SSM_ERR_HANDOFF_TIMEOUT through ssm_workspace_status, the pieces that depend on a lost hand-off must be NaN,
and everything else must equal the normal run.  SSM_NUM_CU plans the small layers as for a small device, so
that they take the chained plan.
"""
import numpy as np
import pytest
import torch

from oracle import bwd as OB
from oracle import ssd as S
from selective_state_space_33_amd import inputs as I
from selective_state_space_33_amd import ops

from .gpu_util import TOL, _Env, oracle_scan, rel_err, say, to_dev, to_dev_f32

pytestmark = pytest.mark.gpu


class _Timeouts:
    def __enter__(self):
        self.a = _Env("SSM_TEST_NEVER_READY", "1")
        self.b = _Env("SSM_TEST_SPIN_LIMIT", "64")
        self.a.__enter__()
        self.b.__enter__()

    def __exit__(self, *e):
        self.b.__exit__(*e)
        self.a.__exit__(*e)


def _fwd(x, ws):
    y, fs = ops.ssm_scan_fwd(to_dev(x["u"], "f32"), to_dev(x["delta"], "f32"), to_dev_f32(x["A"]),
                             to_dev(x["B"], "f32"), to_dev(x["C"], "f32"), D=to_dev_f32(x["D"]),
                             z=to_dev(x["z"], "f32"), delta_bias=to_dev_f32(x["delta_bias"]), workspace=ws)
    return y, fs


def test_forward_handoff_timeout_is_reported(monkeypatch):
    """10 tiles on an '8-CU' plan: 8 whole, 2 cut into 4 chunks of 256 tokens."""
    monkeypatch.setenv("SSM_NUM_CU", "8")
    rng = np.random.default_rng(700)
    x = I.random_scan_inputs(rng, 1, 1024, 640, 16, dtype="f32")
    need = ops.ssm_scan_workspace_size(1, 1024, 640, 16, torch.float32)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    say("fwd chained for 8 CUs, normal")
    y, fs = _fwd(x, ws)
    assert ops.ssm_workspace_status(ws) == ops.SSM_OK
    yo, fo = oracle_scan(x)
    ey, ef = rel_err(y.cpu().numpy(), yo), rel_err(fs.cpu().numpy(), fo)
    print(f"[parity] fwd chained for 8 CUs: y {ey:.2e} state {ef:.2e}", flush=True)
    assert ey <= TOL["f32"] and ef <= TOL["f32"]
    say("fwd chained for 8 CUs, every hand-off lost")
    with _Timeouts():
        y2, fs2 = _fwd(x, ws)
        assert ops.ssm_workspace_status(ws) == ops.SSM_ERR_HANDOFF_TIMEOUT
    y2, fs2 = y2.cpu(), fs2.cpu()
    yc, fsc = y.cpu(), fs.cpu()
    assert torch.equal(y2[:, :, :512], yc[:, :, :512])          # whole tiles: as before
    assert torch.equal(y2[:, :256, 512:], yc[:, :256, 512:])     # chunk 0 of the cut tiles: as before
    assert torch.isnan(y2[:, 256:, 512:]).all()                  # the chunks after a lost hand-off
    assert torch.equal(fs2[:, :512], fsc[:, :512]) and torch.isnan(fs2[:, 512:]).all()
    say("fwd chained for 8 CUs, normal again")
    y3, _ = _fwd(x, ws)
    assert ops.ssm_workspace_status(ws) == ops.SSM_OK             # each call resets the status word
    assert torch.equal(y3.cpu(), yc)
    with pytest.raises(ops.SSMError, match="HANDOFF_TIMEOUT"):
        with _Timeouts():
            ops.ssm_scan_fwd(to_dev(x["u"], "f32"), to_dev(x["delta"], "f32"), to_dev_f32(x["A"]),
                             to_dev(x["B"], "f32"), to_dev(x["C"], "f32"), check_status=True)


def test_backward_handoff_timeout_is_reported(monkeypatch):
    monkeypatch.setenv("SSM_NUM_CU", "8")
    rng = np.random.default_rng(701)
    x = I.random_scan_inputs(rng, 1, 600, 640, 16, dtype="f32")
    dy = np.asarray(rng.standard_normal((1, 600, 640)), np.float32).astype(np.float64)
    args = (to_dev(x["u"], "f32"), to_dev(x["delta"], "f32"), to_dev_f32(x["A"]), to_dev(x["B"], "f32"),
            to_dev(x["C"], "f32"), to_dev(dy, "f32"))
    kw = dict(D=to_dev_f32(x["D"]), z=to_dev(x["z"], "f32"), delta_bias=to_dev_f32(x["delta_bias"]))
    need = ops.ssm_scan_bwd_workspace_size(1, 600, 640, 16, torch.float32)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    say("bwd chained for 8 CUs, normal")
    g = ops.ssm_scan_bwd(*args, workspace=ws, **kw)
    assert ops.ssm_workspace_status(ws) == ops.SSM_OK
    o = OB.scan_bwd(x["u"], x["delta"], x["A"], x["B"], x["C"], dy, D=x["D"], z=x["z"], delta_bias=x["delta_bias"])
    for k in ("du", "ddelta", "dz", "dB", "dC", "dA", "dD", "ddelta_bias"):
        e = rel_err(g[k].cpu().numpy(), o[k])
        assert e <= TOL["f32"], (k, e)
    say("bwd chained for 8 CUs, every hand-off lost")
    with _Timeouts():
        g2 = ops.ssm_scan_bwd(*args, workspace=ws, **kw)
        assert ops.ssm_workspace_status(ws) == ops.SSM_ERR_HANDOFF_TIMEOUT
    for k in ("du", "ddelta", "dz"):
        assert torch.equal(g2[k][:, :, :512].cpu(), g[k][:, :, :512].cpu()), k   # whole tiles unaffected
    assert torch.isnan(g2["du"][:, :, 512:].cpu()).any()
    g3 = ops.ssm_scan_bwd(*args, workspace=ws, **kw)
    assert ops.ssm_workspace_status(ws) == ops.SSM_OK
    assert torch.equal(g3["du"].cpu(), g["du"].cpu())


def test_ssd_handoff_timeout_is_reported(monkeypatch):
    """10 (row, head) units on an '8-CU' plan: 8 whole, 2 cut into 4 segments of 2 chunks."""
    monkeypatch.setenv("SSM_NUM_CU", "8")
    xs = I.random_ssd_inputs(np.random.default_rng(702), 1, 512, 10, 64, 64)
    bf = lambda a: to_dev(a, "bf16")  # noqa: E731
    args = (bf(xs["x"]), bf(xs["delta"]), to_dev_f32(xs["A"]), bf(xs["B"]), bf(xs["C"]))
    kw = dict(D=to_dev_f32(xs["D"]), z=bf(xs["z"]), delta_bias=to_dev_f32(xs["delta_bias"]))
    need = ops.ssm_ssd_fwd_workspace_size(1, 512, 10, 64, 64, torch.bfloat16)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    say("ssd chained for 8 CUs, normal")
    y, fs = ops.ssm_ssd_fwd(*args, workspace=ws, **kw)
    assert ops.ssm_workspace_status(ws) == ops.SSM_OK
    yo, fo = S.ssd_fwd(xs["x"], xs["delta"], xs["A"], xs["B"], xs["C"], D=xs["D"], z=xs["z"],
                       delta_bias=xs["delta_bias"])
    ey, ef = rel_err(y.float().cpu().numpy(), yo), rel_err(fs.cpu().numpy(), fo)
    print(f"[parity] ssd chained for 8 CUs: y {ey:.2e} state {ef:.2e}", flush=True)
    assert ey <= TOL["bf16"] and ef <= TOL["bf16"]
    say("ssd chained for 8 CUs, every hand-off lost")
    with _Timeouts():
        y2, fs2 = ops.ssm_ssd_fwd(*args, workspace=ws, **kw)
        assert ops.ssm_workspace_status(ws) == ops.SSM_ERR_HANDOFF_TIMEOUT
    y2c, yc = y2.cpu(), y.cpu()
    assert torch.equal(y2c[:, :, :8], yc[:, :, :8])              # whole units
    assert torch.equal(y2c[:, :128, 8:], yc[:, :128, 8:])        # segment 0 of the cut units
    assert torch.isnan(y2c[:, 128:, 8:].float()).all()
    assert torch.isnan(fs2[:, 8:].cpu()).all()


def test_launch_on_a_side_stream():
    """A call on a stream that is not the current one, with outputs and workspace allocated by the binding, while
    the current stream keeps allocating and writing: equal to the same call on the current stream."""
    rng = np.random.default_rng(703)
    x = I.random_scan_inputs(rng, 5, 700, 64 * 64, 16, dtype="bf16")   # 320 tiles: the chained plan
    args = (to_dev(x["u"], "bf16"), to_dev(x["delta"], "bf16"), to_dev_f32(x["A"]), to_dev(x["B"], "bf16"),
            to_dev(x["C"], "bf16"))
    kw = dict(D=to_dev_f32(x["D"]), z=to_dev(x["z"], "bf16"), delta_bias=to_dev_f32(x["delta_bias"]))
    say("fwd on the current stream")
    y0, f0 = ops.ssm_scan_fwd(*args, **kw)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    say("fwd on a side stream, three calls, current stream busy")
    for _ in range(3):
        outs.append(ops.ssm_scan_fwd(*args, stream=side, **kw))
        junk = torch.full((64 << 20,), 7.0, device="cuda")   # reuses whatever the allocator frees
        del junk
    side.synchronize()
    torch.cuda.synchronize()
    for y, f in outs:
        assert torch.equal(y, y0) and torch.equal(f, f0)
