"""GPU: the measurement support beside the hot path, and writes that must
stay inside the caller's D.

* gemm_clock_trace: every workgroup of a traced launch writes its four
  counters once, into its own slot; slots past the grid and every byte past
  the buffer stay as they were; an untraced launch writes nothing.
* gemm_clock_probe: the shader-clock counter and the MFMA count give the same
  clock (the counter counts core clocks, the probe keeps the MFMA pipes
  busy), and the clock lies in the chip's range.
* Guard bands around D: the headline kernels (256x256 ping-pong with C, the
  64x64 ring, the MXFP8 ping-pong, the grouped ping-pong) write no byte
  before or after their output.
"""
import sys

import numpy as np
import pytest
import torch

import dense_gemm_swizzled_amd as sg
import synth_inputs as si

pytestmark = pytest.mark.gpu

SENTINEL = -0x5A5A5A5A5A5A5A5B   # an int64 no counter pair takes


def say(msg):
    print(f"[gpu-measure] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sg.load()
    return torch.device("cuda:0")


def _traced(dev, launch, grid, slots):
    buf = torch.full((4 * (slots + 64),), SENTINEL, dtype=torch.int64, device=dev)
    khz = sg.gemm_clock_trace(buf.data_ptr(), slots)
    try:
        launch()
        torch.cuda.synchronize()
    finally:
        sg.gemm_clock_trace(None, 0)
    return khz, buf


@pytest.mark.parametrize("shape,kern,grid", [
    ((4100, 4104, 192), "pingpong16_gemm_kernel<bf16,k,k", 17 * 17),
    ((1024, 1024, 1024), "deep_gemm_kernel<64,bf16,k,mn", 256),
])
def test_clock_trace_one_slot_per_workgroup(dev, shape, kern, grid):
    M, N, K = shape
    b_major = "mn" if "mn" in kern else "k"
    case = si.dense_case(M, N, K, 301, ab_dtype="bf16", b_major=b_major, d_dtype="f32",
                         scale=1.0 / np.sqrt(K))
    A, B = case.A.to(dev), case.B.to(dev)
    D = torch.empty(M, N, device=dev)
    say(f"clock trace {kern}> grid {grid}")
    launch = lambda: sg.gemm(A, B, b_major=b_major, out=D)
    slots = grid + 10
    khz, buf = _traced(dev, launch, grid, slots)
    v = buf.view(-1, 4).cpu().numpy()
    assert sg.gemm_last_kernel().startswith(kern), sg.gemm_last_kernel()
    assert khz > 0
    rec, rest = v[:grid], v[grid:]
    assert (rec[:, 0] > 0).all() and (rec[:, 1] > rec[:, 0]).all(), "shader-clock counter"
    assert (rec[:, 2] > 0).all() and (rec[:, 3] > rec[:, 2]).all(), "real-time counter"
    assert (rest == SENTINEL).all(), f"{int((rest != SENTINEL).any(axis=1).sum())} extra slots"
    ghz = (rec[:, 1] - rec[:, 0]).sum() / (rec[:, 3] - rec[:, 2]).sum() * khz / 1e6
    say(f"  {kern}> ran at {ghz:.3f} GHz (real-time counter {khz} kHz)")
    assert 0.3 < ghz < 3.0
    # Only `slots` workgroups are recorded when the grid is larger.
    khz, buf7 = _traced(dev, launch, grid, 7)
    assert (buf7.view(-1, 4).cpu().numpy()[7:] == SENTINEL).all()
    # Trace off: the last traced buffer is left alone.
    before = buf.clone()
    launch()
    torch.cuda.synchronize()
    assert torch.equal(buf, before)


def test_clock_probe_counts_core_clocks(dev):
    import bench
    waves = sg.gemm_clock_probe_waves()
    khz = sg.gemm_clock_trace(None, 0)
    out = torch.full((5 * waves + 64,), SENTINEL, dtype=torch.int64, device=dev)
    rc = sg.gemm_clock_probe(20000, out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == 0, sg.gemm_last_error()
    torch.cuda.synchronize()
    assert (out[5 * waves:].cpu().numpy() == SENTINEL).all()
    v = out[:4 * waves].view(-1, 8, 4).cpu().numpy()
    assert (v[:, :, 1] > v[:, :, 0]).all() and (v[:, :, 3] > v[:, :, 2]).all()
    mfma_ghz, counter_ghz = bench.probe_ghz(v, 20000, khz)
    say(f"clock probe: counter {counter_ghz:.3f} GHz, MFMA count {mfma_ghz:.3f} GHz")
    assert 0.3 < counter_ghz < 3.0
    # The MFMA pipes are busy for nearly the whole span: the MFMA-count clock
    # is at most the counter's and not far below it.
    assert 0.85 * counter_ghz < mfma_ghz < 1.02 * counter_ghz


# ---------------------------------------------------- guard bands around D

GUARD = 1 << 20   # elements on each side


def _guarded(dev, rows, cols, dtype, fill):
    buf = torch.full((2 * GUARD + rows * cols,), fill, dtype=dtype, device=dev)
    return buf, buf[GUARD:GUARD + rows * cols].view(rows, cols)


def _guards_intact(buf, rows, cols, fill):
    return bool((buf[:GUARD] == fill).all()) and bool((buf[GUARD + rows * cols:] == fill).all())


def test_dense_8192_writes_only_d(dev):
    case = si.dense_8192(seed=3)
    say("guard bands: 8192^3 bf16 + C")
    buf, D = _guarded(dev, case.M, case.N, torch.bfloat16, 3.0)
    sg.gemm(case.A.to(dev), case.B.to(dev), C=case.C.to(dev), out=D)
    torch.cuda.synchronize()
    assert sg.gemm_last_kernel().startswith("pingpong16_gemm_kernel<bf16,k,k")
    assert _guards_intact(buf, case.M, case.N, 3.0)


def test_dense_1024_writes_only_d(dev):
    case = si.dense_1024(seed=2)
    say("guard bands: 1024^3 fp32 D")
    buf, D = _guarded(dev, case.M, case.N, torch.float32, 3.0)
    sg.gemm(case.A.to(dev), case.B.to(dev), b_major="mn", out=D)
    torch.cuda.synchronize()
    assert sg.gemm_last_kernel().startswith("deep_gemm_kernel<64,bf16,k,mn")
    assert _guards_intact(buf, case.M, case.N, 3.0)


def test_mxfp8_writes_only_d(dev):
    case = si.mx_case(4100, 4104, 256, 311)
    say("guard bands: MXFP8 4100x4104x256 bf16 D")
    buf, D = _guarded(dev, case.M, case.N, torch.bfloat16, 3.0)
    sg.mx_gemm(case.A.to(dev), case.SFA.to(dev), case.B.to(dev), case.SFB.to(dev), out=D)
    torch.cuda.synchronize()
    assert sg.gemm_last_kernel().startswith("pingpong_mx_kernel<e4m3")
    assert _guards_intact(buf, case.M, case.N, 3.0)


def test_grouped_writes_only_d(dev):
    case = si.grouped_case([300, 1, 0, 777, 2000, 513, 1200], 4096, 192, 321)
    say("guard bands: grouped, bf16 D")
    rows = case.m_offsets[-1]
    buf, D = _guarded(dev, rows, case.N, torch.bfloat16, 3.0)
    sg.grouped_gemm(case.A.to(dev), case.B.to(dev), case.m_offsets, out=D)
    torch.cuda.synchronize()
    assert sg.gemm_last_kernel().startswith("pingpong16_grouped_kernel<bf16")
    assert _guards_intact(buf, rows, case.N, 3.0)
