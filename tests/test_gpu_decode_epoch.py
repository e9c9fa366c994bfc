"""The decode kernel's epochs and its bounded wait.

* A wait that gives up, forced from the host with the test-only plan flag
  under which routing items are never published, leaves every column of y
  NaN; the kernel still ends normally, path_out is still written, and the
  next ordinary call on the same workspace is correct.
* A decode call captured into a HIP graph takes its epoch from the workspace
  header: replays with new inputs between them, with ordinary calls on the
  same workspace and other GPU work in between, each match an ordinary call
  on the same input bit for bit (the kernel reduces in a fixed order).
* A captured call that gives up poisons the header: later captured calls on
  that workspace write NaN to all of y until an ordinary call resets it.
"""
import dataclasses

import numpy as np
import pytest
import torch

import workloads
from gpu_helpers import check, to_device, to_f64
import sparse_tree_structured_amd as fff

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="no GPU")

# The decode workload's layer (d 2048, 32 trees of depth 6, h 128).
D_MODEL, P, DEPTH, H = 2048, 32, 6, 128


def _inputs(T, seed):
    inp = workloads.random_inputs(T, D_MODEL, P, DEPTH, H, "bf16", seed=seed, unit_rms_x=True)
    return inp, to_device(inp)


def _workspace(dev):
    shape = fff.shape_of(dev["x"], dev["W_node"], dev["V_node"])
    ws, _ = fff.alloc_workspace(shape, fff.make_plan("decode"), dev["x"].device)
    return ws


def _fwd(dev, x=None, **kw):
    return fff.forward(dev["x"] if x is None else x, dev["W_node"], dev["b_node"], dev["V_node"],
                       dev["W_out"], algo="decode", **kw)


@needs_gpu
@pytest.mark.parametrize("T", [1, 8, 64])
def test_give_up_is_visible(T):
    inp, dev = _inputs(T, seed=90 + T)
    ws = _workspace(dev)
    print(f"[gpu] decode T={T}: forced give-up", flush=True)
    y_bad, p_bad = _fwd(dev, workspace=ws, plan_flags=fff.PLAN_TEST_DECODE_NO_PUBLISH)
    torch.cuda.synchronize()
    assert torch.isnan(y_bad.float()).all(), "a wait that gave up must leave y NaN"
    print(f"[gpu] decode T={T}: ordinary call on the same workspace", flush=True)
    y_ok, p_ok = _fwd(dev, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(p_bad, p_ok)  # routing itself ran and wrote its paths
    assert not torch.isnan(y_ok.float()).any()
    print(check(inp, to_f64(y_ok), p_ok.cpu().numpy()))


def _capture(dev, x, y, path, ws, **kw):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _fwd(dev, x=x, y=y, path_out=path, workspace=ws, **kw)
    return g


@needs_gpu
@pytest.mark.parametrize("T", [1, 64])
def test_captured_replays_take_fresh_epochs(T):
    inp, dev = _inputs(T, seed=110 + T)
    ws = _workspace(dev)
    x = dev["x"].clone()
    y = torch.empty((T, D_MODEL), dtype=x.dtype, device=x.device)
    path = torch.empty((T, P), dtype=torch.int32, device=x.device)
    print(f"[gpu] decode T={T}: eager warm-up, then capture", flush=True)
    _fwd(dev, x=x, y=y, path_out=path, workspace=ws)
    torch.cuda.synchronize()
    g = _capture(dev, x, y, path, ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(T)
    for i in range(6):
        xi = torch.randn((T, D_MODEL), generator=torch.Generator().manual_seed(1000 * T + i))
        xi = xi.to(torch.bfloat16).to(x.device)
        x.copy_(xi)
        print(f"[gpu] decode T={T}: replay {i}", flush=True)
        g.replay()
        # Other work on the stream between replays, and at i == 3 an ordinary
        # call on the same workspace (its epoch comes from the host; the next
        # replay continues from the header it leaves).
        junk = torch.randn(int(rng.integers(1, 1 << 16)), device=x.device).sum()
        if i == 3:
            _fwd(dev, x=xi, workspace=ws)
        torch.cuda.synchronize()
        y_ref, p_ref = _fwd(dev, x=xi)
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        assert torch.equal(path, p_ref), f"replay {i}: paths differ from an ordinary call"
        assert torch.equal(y, y_ref), f"replay {i}: y differs from an ordinary call"
    # The last replay's input against the oracle.
    last = dataclasses.replace(inp, x=x.cpu().view(torch.int16).numpy().view(np.uint16).copy())
    print(check(last, to_f64(y), path.cpu().numpy()))


@needs_gpu
def test_captured_give_up_poisons_until_reset():
    T = 8
    inp, dev = _inputs(T, seed=130)
    ws = _workspace(dev)
    x = dev["x"]
    y_ok = torch.empty((T, D_MODEL), dtype=x.dtype, device=x.device)
    p_ok = torch.empty((T, P), dtype=torch.int32, device=x.device)
    y_bad = torch.empty_like(y_ok)
    p_bad = torch.empty_like(p_ok)
    print("[gpu] decode: eager warm-up, then capture an ordinary and a give-up call", flush=True)
    y_ref, path_ref = _fwd(dev)
    torch.cuda.synchronize()
    g_ok = _capture(dev, x, y_ok, p_ok, ws)
    g_bad = _capture(dev, x, y_bad, p_bad, ws, plan_flags=fff.PLAN_TEST_DECODE_NO_PUBLISH)
    torch.cuda.synchronize()

    def replay_ok(expect_ok):
        y_ok.zero_()
        g_ok.replay()
        torch.cuda.synchronize()
        if expect_ok:
            assert torch.equal(y_ok, y_ref) and torch.equal(p_ok, path_ref)
        else:
            assert torch.isnan(y_ok.float()).all()

    print("[gpu] replay ordinary", flush=True)
    replay_ok(True)
    print("[gpu] replay give-up", flush=True)
    g_bad.replay()
    torch.cuda.synchronize()
    assert torch.isnan(y_bad.float()).all()
    print("[gpu] replay ordinary on the poisoned workspace (twice)", flush=True)
    replay_ok(False)
    replay_ok(False)
    print("[gpu] ordinary uncaptured call resets the header", flush=True)
    y_e, p_e = _fwd(dev, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y_e, y_ref) and torch.equal(p_e, path_ref)
    replay_ok(True)
    replay_ok(True)
    print(check(inp, to_f64(y_ok), p_ok.cpu().numpy()))
