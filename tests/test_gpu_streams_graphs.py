"""The library's calls under concurrent streams and inside a captured HIP
graph: they hold no global state, clear their own scalars with a fill kernel
(no memset node) and enqueue everything on the caller's stream, so results
equal the eager, single-stream ones bit for bit."""
import numpy as np
import pytest

from gpu_util import q_to_host, say, to_device, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp4():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import fp4_fully_quantized_amd as m
    m.lib()
    return m


def _data(shape, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    from oracle.oracle import f32_to_bf16_bits
    return f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


def _same(a, b):
    for k in ("codes", "scales"):
        assert np.array_equal(a[k], b[k]), k
    if a["fmt"] == 0:
        assert a["amax"] == b["amax"] and a["sg"] == b["sg"]


def test_concurrent_streams_match_one_stream(fp4):
    """Two streams quantize and multiply different tensors at the same time."""
    import torch
    say("two streams")
    xs = [to_device(_data((1024, 2048), 1 + i)) for i in range(2)]
    ws = [to_device(_data((768, 2048), 11 + i, 0.02)) for i in range(2)]
    ref = []
    for x, w in zip(xs, ws):
        qx, qxt = fp4.quantize_dual(x, rnd_rows=1, seed_rows=5)
        qw = fp4.quantize(w)
        ref.append((q_to_host(qx), q_to_host(qxt), to_host(fp4.gemm(qx, qw))))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    out = [None, None]
    for i, s in enumerate(streams):
        with torch.cuda.stream(s):
            qx, qxt = fp4.quantize_dual(xs[i], rnd_rows=1, seed_rows=5, stream=s)
            qw = fp4.quantize(ws[i], stream=s)
            y = fp4.gemm(qx, qw, stream=s)
            out[i] = (qx, qxt, y)
    torch.cuda.synchronize()
    for i in range(2):
        _same(q_to_host(out[i][0]), ref[i][0])
        _same(q_to_host(out[i][1]), ref[i][1])
        assert np.array_equal(to_host(out[i][2]), ref[i][2])


def test_graph_replays_match_eager(fp4):
    """A layer step (NVFP4 dual quantization of X, W and dY, the three GEMMs)
    captured once and replayed three times, with eager work and
    synchronizations between the replays; every replay equals the eager run.
    The inputs are overwritten in place between replays, so each replay
    recomputes the amax and the codes."""
    import torch
    say("graph capture")
    T, D, F = 512, 1024, 768
    X = to_device(_data((T, D), 21))
    W = to_device(_data((F, D), 22, 0.02))
    dY = to_device(_data((T, F), 23, 1e-3))
    Q = fp4.QTensor
    q = {"X": Q(T, D, 0), "Xt": Q(D, T, 0), "W": Q(F, D, 0), "Wt": Q(D, F, 0),
         "dY": Q(T, F, 0), "dYt": Q(F, T, 0)}
    for a, b in (("Xt", "X"), ("Wt", "W"), ("dYt", "dY")):
        q[a].amax = q[b].amax
    Y = torch.empty((T, F), dtype=torch.bfloat16, device="cuda")
    dX = torch.empty((T, D), dtype=torch.float32, device="cuda")
    dW = torch.empty((F, D), dtype=torch.float32, device="cuda")

    def step(s=None):
        fp4.fp4_quantize_dual(X, 0, 0, 0, 1, 3, 0, False, q["X"], q["Xt"], stream=s)
        fp4.fp4_quantize_dual(W, 0, 0, 0, 1, 4, 0, False, q["W"], q["Wt"], stream=s)
        fp4.fp4_gemm(q["X"], q["W"], Y, stream=s)
        fp4.fp4_quantize_dual(dY, 1, 1, 0, 1, 2, 0, False, q["dY"], q["dYt"], stream=s)
        fp4.fp4_gemm(q["dY"], q["Wt"], dX, stream=s)
        fp4.fp4_gemm(q["dYt"], q["Xt"], dW, stream=s)

    def snapshot():
        torch.cuda.synchronize()
        return ({k: q_to_host(v) for k, v in q.items()}, to_host(Y), to_host(dX), to_host(dW))

    inputs = [(_data((T, D), 31 + r), _data((F, D), 41 + r, 0.02), _data((T, F), 51 + r, 1e-3))
              for r in range(3)]
    # eager results for each input set
    eager = []
    for xh, wh, dyh in inputs:
        X.copy_(to_device(xh)); W.copy_(to_device(wh)); dY.copy_(to_device(dyh))
        step()
        eager.append(snapshot())
    # capture (on a side stream, as torch requires)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(s)                      # warm-up on the capture stream
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        step(s)
    torch.cuda.synchronize()
    for r, (xh, wh, dyh) in enumerate(inputs):
        X.copy_(to_device(xh)); W.copy_(to_device(wh)); dY.copy_(to_device(dyh))
        torch.cuda.synchronize()
        junk = torch.randn(1 << 20, device="cuda").sum()   # eager work between replays
        g.replay()
        got = snapshot()
        assert float(junk.cpu()) == float(junk.cpu())
        for k in q:
            _same(got[0][k], eager[r][0][k])
        for a, b in zip(got[1:], eager[r][1:]):
            assert np.array_equal(a, b), f"replay {r}"


def test_graph_replays_noise_monitor(fp4):
    """The noise-monitored dual pass (its grid sized from the kernel's
    occupancy at launch) captured with a fill kernel that clears the four
    sums, replayed three times on new inputs: codes and scales equal the
    eager run's bit for bit, the FP64 sums (added by atomics in any order)
    to 1e-12 relative."""
    import torch
    say("graph capture, noise monitor")
    T, F = 4096, 4096    # 1024 tiles of 128 x 128: more than run at once, so workgroups loop
    dY = to_device(_data((T, F), 61, 1e-3))
    Q = fp4.QTensor
    qc, qr = Q(T, F, 0), Q(F, T, 0)
    qr.amax = qc.amax
    noise = torch.zeros(4, dtype=torch.float64, device="cuda")

    def step(s=None):
        noise.zero_()
        fp4.fp4_quantize_dual_noise(dY, 1, 7, 0, 1, 8, 0, False, qc, qr, noise[0:2], noise[2:4], stream=s)

    def snapshot():
        torch.cuda.synchronize()
        return q_to_host(qc), q_to_host(qr), noise.cpu().numpy().copy()

    inputs = [_data((T, F), 71 + r, 1e-3) for r in range(3)]
    eager = []
    for h in inputs:
        dY.copy_(to_device(h))
        step()
        eager.append(snapshot())
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        step(s)
    torch.cuda.synchronize()
    for r, h in enumerate(inputs):
        dY.copy_(to_device(h))
        torch.cuda.synchronize()
        g.replay()
        got = snapshot()
        _same(got[0], eager[r][0])
        _same(got[1], eager[r][1])
        assert np.all(got[2] > 0)
        np.testing.assert_allclose(got[2], eager[r][2], rtol=1e-12, atol=0)
