"""Calls captured into a HIP graph and replayed (torch.cuda.graph on the
caller's stream).  The library keeps no per-call host state in a captured
call, so a replay recomputes the call on whatever the captured buffers then
hold.  Each replay follows new inputs copied into those buffers and eager
work with synchronizations, and must equal an eager call on the same inputs.

The elementwise look-back schedule carries a tile-counter base and epoch
from the host, which a replay would reuse: under capture the automatic
schedule takes the stream schedule, and a forced look-back is refused
without capturing anything or disturbing later eager calls.
"""
import pytest
import torch

from linear_recurrence_scan_fma_amd import binding, inputs
from _helpers import rel, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ctx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    c = binding.Context(0)
    yield c
    c.close()


def _replay_matches(run, bufs, fresh, outs, n=3):
    """Capture run() once, then n times: copy fresh(i) into bufs, replay, and
    compare outs with an eager run() on the same inputs."""
    torch.cuda.synchronize()
    run()                                   # warm-up: sizes the context's workspaces
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            run()
    torch.cuda.synchronize()
    for i in range(n):
        for dst, src in zip(bufs, fresh(i)):
            dst.copy_(src)
        junk = torch.randn(1 << 20, device="cuda:0").sum()   # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outs]
        run()
        torch.cuda.synchronize()
        for a, b in zip(got, outs):
            assert torch.equal(a, b), f"replay {i}"
        del junk


def test_graph_diag_outer(ctx):
    B, T, H, K, V = 1, 300, 2, 128, 128
    d = inputs.gla(B=B, T=T, H=H, K=K, V=V, seed=1201)
    q, k, v, g = (d[n].to("cuda:0") for n in ("q", "k", "v", "g"))
    o = torch.empty((B, T, H, V), device="cuda:0")
    fin = torch.empty((B, H, K, V), device="cuda:0")
    binding.lrs_context_set_param(ctx, binding.LRS_PARAM_DIAG_SEGMENTS, 3)
    try:
        say("graph: diag outer, 3 segments")
        run = lambda: binding.lrs_scan_diag_outer(ctx, q, k, v, g, 1, None, d["scale"], None, o, fin)  # noqa: E731
        fresh = lambda i: [inputs.gla(B=B, T=T, H=H, K=K, V=V, seed=1300 + i)[n].to("cuda:0")  # noqa: E731
                           for n in ("q", "k", "v", "g")]
        _replay_matches(run, [q, k, v, g], fresh, [o, fin])
    finally:
        binding.lrs_context_set_param(ctx, binding.LRS_PARAM_DIAG_SEGMENTS, 0)


@pytest.mark.parametrize("decay", [False, True])
def test_graph_delta(ctx, decay):
    B, T, H, K, V = 1, 200, 2, 64, 64
    gen = inputs.rwkv7 if decay else inputs.deltanet
    d = gen(B=B, T=T, H=H, K=K, V=V, seed=1401)
    names = ("q", "k", "v", "g", "beta") if decay else ("q", "k", "v", "beta")
    x = [d[n].to("cuda:0") for n in names]
    o = torch.empty((B, T, H, V), device="cuda:0")
    fin = torch.empty((B, H, K, V), device="cuda:0")
    say(f"graph: delta decay={decay}")
    if decay:
        run = lambda: binding.lrs_scan_delta_decay(ctx, *x, 1.0, None, o, fin)  # noqa: E731
    else:
        run = lambda: binding.lrs_scan_delta(ctx, *x, 1.0, None, o, fin)  # noqa: E731
    fresh = lambda i: [gen(B=B, T=T, H=H, K=K, V=V, seed=1500 + i)[n].to("cuda:0") for n in names]  # noqa: E731
    _replay_matches(run, x, fresh, [o, fin])


def test_graph_delta_out_bf16_decay_k128(ctx):
    # the decayed delta rule at K = 128 (half-key prep tiles, single-buffered
    # scan operands, L2 touches) with a bf16 output
    B, T, H, K, V = 1, 200, 2, 128, 64
    d = inputs.rwkv7(B=B, T=T, H=H, K=K, V=V, seed=1601)
    names = ("q", "k", "v", "g", "beta")
    x = {n: d[n].to("cuda:0") for n in names}
    o = torch.empty((B, T, H, V), device="cuda:0", dtype=torch.bfloat16)
    fin = torch.empty((B, H, K, V), device="cuda:0")
    say("graph: delta decay K=128, bf16 out")
    run = lambda: binding.lrs_scan_delta_out(ctx, x["q"], x["k"], x["v"], x["g"], x["beta"], 1.0, None,  # noqa: E731
                                             binding.LRS_DTYPE_BF16, o, fin)
    fresh = lambda i: [inputs.rwkv7(B=B, T=T, H=H, K=K, V=V, seed=1700 + i)[n].to("cuda:0")  # noqa: E731
                       for n in names]
    _replay_matches(run, [x[n] for n in names], fresh, [o, fin])


def test_graph_delta_time_segments(ctx):
    # the delta rule in time segments (segment pass, prefix, output pass)
    B, T, H, K, V = 1, 1300, 2, 128, 128
    d = inputs.deltanet(B=B, T=T, H=H, K=K, V=V, seed=1611)
    names = ("q", "k", "v", "beta")
    x = {n: d[n].to("cuda:0") for n in names}
    o = torch.empty((B, T, H, V), device="cuda:0")
    fin = torch.empty((B, H, K, V), device="cuda:0")
    binding.lrs_context_set_param(ctx, binding.LRS_PARAM_DELTA_SEGMENTS, 3)
    try:
        say("graph: delta rule, 3 time segments")
        run = lambda: binding.lrs_scan_delta(ctx, x["q"], x["k"], x["v"], x["beta"], 1.0, None, o, fin)  # noqa: E731
        fresh = lambda i: [inputs.deltanet(B=B, T=T, H=H, K=K, V=V, seed=1710 + i)[n].to("cuda:0")  # noqa: E731
                           for n in names]
        _replay_matches(run, [x[n] for n in names], fresh, [o, fin])
    finally:
        binding.lrs_context_set_param(ctx, binding.LRS_PARAM_DELTA_SEGMENTS, 0)


def test_graph_elementwise_stream_schedule(ctx):
    B, T, N = 2, 500, 256
    d = inputs.elementwise_small(B, T, N, seed=1601)
    a, u = d["a"].to("cuda:0"), d["u"].to("cuda:0")
    s = torch.empty_like(a)
    fin = torch.empty((B, N), device="cuda:0")
    binding.lrs_context_set_param(ctx, binding.LRS_PARAM_ELEM_SCHEDULE, binding.LRS_ELEM_SCHEDULE_STREAM)
    try:
        say("graph: gated scan, stream schedule")
        run = lambda: binding.lrs_scan_gated(ctx, a, u, None, s, fin)  # noqa: E731
        fresh = lambda i: [inputs.elementwise_small(B, T, N, seed=1700 + i)[n].to("cuda:0")  # noqa: E731
                           for n in ("a", "u")]
        _replay_matches(run, [a, u], fresh, [s, fin])
    finally:
        binding.lrs_context_set_param(ctx, binding.LRS_PARAM_ELEM_SCHEDULE, binding.LRS_ELEM_SCHEDULE_AUTO)


def test_graph_elementwise_automatic_schedule_under_capture(ctx):
    # a shape whose eager automatic schedule is the look-back: captured, the
    # call takes the (deterministic) stream schedule, so replays equal an
    # eager stream-schedule call bit for bit
    B, T, N = 2, 500, 256
    d = inputs.elementwise_small(B, T, N, seed=1801)
    a, u = d["a"].to("cuda:0"), d["u"].to("cuda:0")
    s = torch.empty_like(a)
    fin = torch.empty((B, N), device="cuda:0")
    s_ref = torch.empty_like(a)
    f_ref = torch.empty_like(fin)
    say("graph: gated scan, automatic schedule")
    run = lambda: binding.lrs_scan_gated(ctx, a, u, None, s, fin)  # noqa: E731
    run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            run()
    torch.cuda.synchronize()
    for i in range(3):
        fresh = inputs.elementwise_small(B, T, N, seed=1900 + i)
        a.copy_(fresh["a"].to("cuda:0"))
        u.copy_(fresh["u"].to("cuda:0"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        binding.lrs_context_set_param(ctx, binding.LRS_PARAM_ELEM_SCHEDULE, binding.LRS_ELEM_SCHEDULE_STREAM)
        try:
            binding.lrs_scan_gated(ctx, a, u, None, s_ref, f_ref)
            torch.cuda.synchronize()
        finally:
            binding.lrs_context_set_param(ctx, binding.LRS_PARAM_ELEM_SCHEDULE, binding.LRS_ELEM_SCHEDULE_AUTO)
        assert torch.equal(s, s_ref) and torch.equal(fin, f_ref), i
    assert binding.lib().lrs_context_check(ctx.handle) == binding.LRS_OK


def test_graph_forced_lookback_is_refused(ctx):
    B, T, N = 2, 500, 256
    d = inputs.elementwise_small(B, T, N, seed=2001)
    a, u = d["a"].to("cuda:0"), d["u"].to("cuda:0")
    s = torch.empty_like(a)
    fin = torch.empty((B, N), device="cuda:0")
    L = binding.lib()
    binding.lrs_context_set_param(ctx, binding.LRS_PARAM_ELEM_SCHEDULE, binding.LRS_ELEM_SCHEDULE_LOOKBACK)
    try:
        say("graph: forced look-back under capture")
        binding.lrs_scan_gated(ctx, a, u, None, s, fin)
        torch.cuda.synchronize()
        want_s, want_f = s.clone(), fin.clone()
        g = torch.cuda.CUDAGraph()
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            with torch.cuda.graph(g, stream=st):
                rc = L.lrs_scan_gated(ctx.handle, a.data_ptr(), u.data_ptr(), None, s.data_ptr(),
                                      fin.data_ptr(), B, T, N, st.cuda_stream)
                fin.add_(0.0)                   # the graph captures something
        assert rc == binding.LRS_E_UNSUPPORTED
        torch.cuda.synchronize()
        # later eager look-back calls are unaffected
        s.fill_(-7.0)
        fin.fill_(-7.0)
        binding.lrs_scan_gated(ctx, a, u, None, s, fin)
        torch.cuda.synchronize()
        assert rel(s, want_s) <= 1e-6 and rel(fin, want_f) <= 1e-6
        assert L.lrs_context_check(ctx.handle) == binding.LRS_OK
    finally:
        binding.lrs_context_set_param(ctx, binding.LRS_PARAM_ELEM_SCHEDULE, binding.LRS_ELEM_SCHEDULE_AUTO)


def test_graph_capture_refuses_workspace_growth():
    """A captured matrix-scan call that would have to grow the context's
    workspace (allocate and wait) is refused with nothing captured; the same
    call made eagerly afterwards sizes the workspace and matches the oracle's
    shape of result (the eager path is unaffected)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B, T, H, K, V = 1, 200, 2, 64, 64
    d = inputs.deltanet(B=B, T=T, H=H, K=K, V=V, seed=1207)
    q, k, v, beta = (d[n].to("cuda:0") for n in ("q", "k", "v", "beta"))
    o = torch.empty((B, T, H, V), device="cuda:0")
    fin = torch.empty((B, H, K, V), device="cuda:0")
    L = binding.lib()
    with binding.Context(0) as fresh:   # empty workspace
        say("graph: capture on a context whose workspace must grow")
        g = torch.cuda.CUDAGraph()
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            with torch.cuda.graph(g, stream=st):
                rc = L.lrs_scan_delta(fresh.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(), beta.data_ptr(),
                                      1.0, None, o.data_ptr(), fin.data_ptr(), B, T, H, K, V, st.cuda_stream)
                fin.add_(0.0)                   # the graph captures something
        assert rc == binding.LRS_E_UNSUPPORTED
        torch.cuda.synchronize()
        o2, fin2 = binding.scan_delta(fresh, q, k, v, beta, 1.0)
        o3, fin3 = binding.scan_delta(fresh, q, k, v, beta, 1.0)
        torch.cuda.synchronize()
        assert torch.isfinite(o2).all() and torch.equal(o2, o3) and torch.equal(fin2, fin3)


@pytest.mark.parametrize("kind", ["delta", "diag"])
def test_graph_replay_after_eager_workspace_growth(kind):
    """A graph captured on a context keeps the workspace it was captured with.
    An eager call that then grows the context's workspace must not free it:
    replaying the graph afterwards still equals an eager call on the captured
    shape (and the grown, eager path is unaffected)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    with binding.Context(0) as c:
        small = dict(B=1, T=200, H=2, K=64, V=64)
        large = dict(B=2, T=900, H=4, K=64, V=64)
        if kind == "delta":
            gen, names = inputs.deltanet, ("q", "k", "v", "beta")
        else:
            gen, names = inputs.gla, ("q", "k", "v", "g")
            binding.lrs_context_set_param(c, binding.LRS_PARAM_DIAG_SEGMENTS, 3)
        d = gen(**small, seed=1901)
        x = [d[n].to("cuda:0") for n in names]
        B, T, H, K, V = (small[n] for n in ("B", "T", "H", "K", "V"))
        o = torch.empty((B, T, H, V), device="cuda:0")
        fin = torch.empty((B, H, K, V), device="cuda:0")
        if kind == "delta":
            run = lambda: binding.lrs_scan_delta(c, *x, 1.0, None, o, fin)  # noqa: E731
        else:
            run = lambda: binding.lrs_scan_diag_outer(c, *x, 1, None, d["scale"], None, o, fin)  # noqa: E731
        say(f"graph: {kind}, capture then grow the workspace eagerly, then replay")
        run()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            with torch.cuda.graph(g, stream=st):
                run()
        torch.cuda.synchronize()
        # an eager call on a larger shape grows the workspace
        dl = gen(**large, seed=1902)
        xl = [dl[n].to("cuda:0") for n in names]
        if kind == "delta":
            ol, fl = binding.scan_delta(c, *xl, 1.0)
        else:
            ol, fl = binding.scan_diag_outer(c, *xl, 1, None, dl["scale"])
        torch.cuda.synchronize()
        assert torch.isfinite(ol).all() and torch.isfinite(fl).all()
        for i in range(3):
            for dst, n in zip(x, names):
                dst.copy_(gen(**small, seed=1910 + i)[n])
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            got = (o.clone(), fin.clone())
            run()
            torch.cuda.synchronize()
            assert torch.equal(got[0], o) and torch.equal(got[1], fin), f"replay {i}"
        del g
        torch.cuda.synchronize()


def test_graph_diag_outer_keyscale(ctx):
    B, T, H, K, V = 1, 300, 2, 64, 64
    names = ("q", "k", "v", "g", "k_scale_key")
    d = inputs.assoc_memory(B=B, T=T, H=H, K=K, V=V, seed=1211)
    x = [d[n].to("cuda:0") for n in names]
    o = torch.empty((B, T, H, V), device="cuda:0")
    fin = torch.empty((B, H, K, V), device="cuda:0")
    say("graph: diag outer with a per-key kappa")
    run = lambda: binding.lrs_scan_diag_outer_keyscale(ctx, *x, d["scale"], None, o, fin)  # noqa: E731
    fresh = lambda i: [inputs.assoc_memory(B=B, T=T, H=H, K=K, V=V, seed=1311 + i)[n].to("cuda:0")  # noqa: E731
                       for n in names]
    _replay_matches(run, x, fresh, [o, fin])


def test_graph_diag_outer_epilogue(ctx):
    B, T, H, K, V = 1, 300, 2, 128, 128
    d = inputs.gla(B=B, T=T, H=H, K=K, V=V, seed=1221)
    e = inputs.norm_gate_epilogue(B, T, H, V, seed=1222)
    x = [d[n].to("cuda:0") for n in ("q", "k", "v", "g")] + [e["gate"].to("cuda:0")]
    w = e["norm_weight"].to("cuda:0")
    o = torch.empty((B, T, H, V), dtype=torch.bfloat16, device="cuda:0")
    fin = torch.empty((B, H, K, V), device="cuda:0")
    say("graph: diag outer with the norm-gate epilogue, bf16 output")
    run = lambda: binding.lrs_scan_diag_outer_epilogue(  # noqa: E731
        ctx, x[0], x[1], x[2], x[3], 1, None, d["scale"], None, binding.LRS_EPILOGUE_NORM_GATE, None, x[4], w,
        e["eps"], binding.LRS_DTYPE_BF16, o, fin)

    def fresh(i):
        f = inputs.gla(B=B, T=T, H=H, K=K, V=V, seed=1321 + i)
        z = inputs.norm_gate_epilogue(B, T, H, V, seed=1421 + i)["gate"]
        return [f[n].to("cuda:0") for n in ("q", "k", "v", "g")] + [z.to("cuda:0")]

    _replay_matches(run, x, fresh, [o, fin])


def test_graph_elementwise_backward(ctx):
    B, T, N = 2, 500, 256
    d = inputs.elementwise_small(B, T, N, seed=2101)
    a, u = d["a"].to("cuda:0"), d["u"].to("cuda:0")
    s = inputs.random_normal((B, T, N), 2102).to("cuda:0")
    ds = inputs.random_normal((B, T, N), 2103).to("cuda:0")
    s0 = inputs.random_state((B, N), 2104).to("cuda:0")
    dsf = inputs.random_state((B, N), 2105).to("cuda:0")
    da, du = torch.empty_like(a), torch.empty_like(a)
    ds0 = torch.empty((B, N), device="cuda:0")
    binding.lrs_context_set_param(ctx, binding.LRS_PARAM_ELEM_SCHEDULE, binding.LRS_ELEM_SCHEDULE_STREAM)
    try:
        say("graph: gated gradient pass, stream schedule")
        run = lambda: binding.lrs_scan_gated_backward(ctx, a, u, s0, s, ds, dsf, da, du, ds0)  # noqa: E731

        def fresh(i):
            f = inputs.elementwise_small(B, T, N, seed=2200 + i)
            return [f["a"].to("cuda:0"), f["u"].to("cuda:0"),
                    inputs.random_normal((B, T, N), 2300 + i).to("cuda:0"),
                    inputs.random_normal((B, T, N), 2400 + i).to("cuda:0")]

        _replay_matches(run, [a, u, s, ds], fresh, [da, du, ds0])
    finally:
        binding.lrs_context_set_param(ctx, binding.LRS_PARAM_ELEM_SCHEDULE, binding.LRS_ELEM_SCHEDULE_AUTO)


def test_graph_step(ctx):
    # the step updates s in place: each replay and the eager call it is
    # compared with start from the same fresh state
    B, N = 4, 4096
    d = inputs.elementwise_small(B, 1, N, seed=2501)
    a, u = d["a"][:, 0].contiguous().to("cuda:0"), d["u"][:, 0].contiguous().to("cuda:0")
    s = inputs.random_state((B, N), 2502).to("cuda:0")
    say("graph: gated single step")
    run = lambda: binding.lrs_step_gated(ctx, a, u, s)  # noqa: E731
    run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            run()
    torch.cuda.synchronize()
    for i in range(3):
        f = inputs.elementwise_small(B, 1, N, seed=2600 + i)
        fs = inputs.random_state((B, N), 2700 + i).to("cuda:0")
        a.copy_(f["a"][:, 0].to("cuda:0"))
        u.copy_(f["u"][:, 0].to("cuda:0"))
        s.copy_(fs)
        junk = torch.randn(1 << 20, device="cuda:0").sum()   # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = s.clone()
        s.copy_(fs)
        run()
        torch.cuda.synchronize()
        assert torch.equal(got, s), f"replay {i}"
        del junk
