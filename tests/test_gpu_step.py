"""GPU parity of the persistent decode-step kernel (spectra_step_*).

Each phase's outputs must equal, bit for bit, the single-product GEMV run on
the same input (the grouped launch for phases of several containers), and
meet the oracle's per-element bound |y - y_ref| <= 1e-3 (|W_hat| |x|) + 1e-6
with y_ref the oracle's float64 product.  A phase that reads an earlier
phase's output is checked on the input the GPU staged for it: that output
times the phase's power-of-two scale, rounded to fp16 (exact).
"""
import numpy as np
import pytest

from dequant_gemv_spectra_amd import decoder, synth
from oracle import spectra_oracle as O

pytestmark = pytest.mark.gpu


def _sp():
    from dequant_gemv_spectra_amd import spectra
    return spectra


def _torch():
    import torch
    return torch


def staged_input(phases, outs, p):
    """x of phase p as the kernel stages it (host float16 [K])."""
    ph = phases[p]
    if ph["input"] < 0:
        x = ph["x"].cpu().numpy().reshape(-1)
    else:
        x = outs[ph["input"]][0]
    return (x.astype(np.float64) * ph["x_scale"]).astype(np.float16)


def check_phases(phases, imgs=None, rows=None, which=None):
    """Bit equality with the GEMV on the staged inputs for every phase, and
    the oracle bound for the phases in `which` (all by default); `imgs` maps
    a container handle to its exported image, `rows` samples output rows."""
    sp, torch = _sp(), _torch()
    torch.cuda.synchronize()
    outs = [[y.cpu().numpy().reshape(-1) for y in ph["ys"]] for ph in phases]
    for p, ph in enumerate(phases):
        x = staged_input(phases, outs, p)
        xd = torch.from_numpy(x.reshape(1, -1)).cuda()
        if len(ph["containers"]) == 1:
            ref = [sp.spectra_gemm(ph["containers"][0], xd, kernel="gemv")]
        else:
            ref = sp.spectra_gemm_grouped(ph["containers"], xd)
        torch.cuda.synchronize()
        for i, r in enumerate(ref):
            got, want = outs[p][i], r.cpu().numpy().reshape(-1)
            nd = int((got.view(np.uint16) != want.view(np.uint16)).sum())
            assert nd == 0, f"phase {p} task {i}: {nd} outputs differ from the GEMV's"
        if which is not None and p not in which:
            continue
        for i, c in enumerate(ph["containers"]):
            img = imgs[c.handle.value] if imgs else sp.spectra_export(c)
            if rows is None:
                W_hat = O.unpack(img)["W_hat"]
                sel = slice(None)
            else:
                N = c.info()["N"]
                sel = np.unique(np.concatenate([rows[rows < N], [0, N - 1]]))
                W_hat = O.reconstruct_rows(img, sel)
            yr = O.matmul_ref(W_hat, x.reshape(1, -1))[0]
            tol = O.tolerance(W_hat, x.reshape(1, -1))[0]
            err = np.abs(outs[p][i][sel].astype(np.float64) - yr)
            bad = err > tol
            assert not bad.any(), (f"phase {p} task {i}: {bad.sum()} of {bad.size} outside the bound, "
                                   f"worst ratio {(err / tol).max():.3g}")
    return outs


def small_chain(seed=0):
    """Phases over small containers: three tasks sharing an external input,
    ragged K (K % 8 != 0), no heavy-tailed channels, many, and a row count
    below the number of blocks."""
    sp, torch = _sp(), _torch()
    shapes = [  # (phase tasks [(N, planted heavy-tailed)], K, input, scale)
        ([(520, 6), (131, 3), (97, 0)], 384, -1, 1.0),
        ([(384, 40)], 520, 0, 0.5),
        ([(1000, 0), (1000, 12)], 384, 1, 0.25),
        ([(97, 9)], 1000, 2, 1.0),
        ([(2600, 2), (64, 1)], 97, 3, 2.0),
        ([(384, 30)], 2600, 4, 0.125),
    ]
    phases, keep = [], []
    for p, (tasks, K, inp, sc) in enumerate(shapes):
        cs, ys = [], []
        for i, (N, n_out) in enumerate(tasks):
            W, g, _ = synth.random_case(N, K, n_out, seed=seed * 100 + 10 * p + i)
            cs.append(sp.spectra_pack(W, g))
            ys.append(torch.full((N,), 7.0, dtype=torch.float16, device="cuda"))
        x = None
        if inp < 0:
            x = torch.from_numpy(synth.random_case(1, K, 0, seed=seed * 100 + 99)[2].reshape(-1)).cuda()
        phases.append({"containers": cs, "ys": ys, "input": inp, "x": x, "x_scale": sc})
        keep.append(cs)
    return phases


def test_step_small_chain():
    sp = _sp()
    phases = small_chain()
    plan = sp.StepPlan(phases)
    plan.run()
    assert plan.status() == sp.SPECTRA_OK
    check_phases(phases)
    plan.close()


def test_step_repeated_runs_and_graph_replays():
    sp, torch = _sp(), _torch()
    phases = small_chain(seed=1)
    plan = sp.StepPlan(phases)
    plan.run()
    torch.cuda.synchronize()
    first = [[y.cpu().clone() for y in ph["ys"]] for ph in phases]
    for _ in range(3):  # later runs carry new launch tags and must give the same outputs
        for ph in phases:
            for y in ph["ys"]:
                y.fill_(0.0)
        plan.run()
        torch.cuda.synchronize()
        for p, ph in enumerate(phases):
            for i, y in enumerate(ph["ys"]):
                assert torch.equal(y.cpu(), first[p][i]), f"run differs at phase {p} task {i}"
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        plan.run(stream=s)
    for rep in range(3):
        for ph in phases:
            for y in ph["ys"]:
                y.fill_(0.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for p, ph in enumerate(phases):
            for i, y in enumerate(ph["ys"]):
                assert torch.equal(y.cpu(), first[p][i]), f"replay {rep} differs at phase {p} task {i}"
    assert plan.status() == sp.SPECTRA_OK
    check_phases(phases)
    plan.close()


def test_step_bounded_wait_reports_timeout():
    """A wait forced never to be satisfied (host-set tag skew, 8 polls) gives
    up, the kernel still completes, the status reports it once, and the plan
    then runs correctly again."""
    sp, torch = _sp(), _torch()
    phases = small_chain(seed=2)
    plan = sp.StepPlan(phases)
    plan.test_hooks(poll_limit=8, tag_skew=1)
    plan.run()
    assert plan.status() == sp.SPECTRA_E_TIMEOUT
    plan.test_hooks(0, 0)
    plan.run()
    assert plan.status() == sp.SPECTRA_OK
    check_phases(phases)
    plan.close()


def test_step_rejects_bad_plans():
    sp, torch = _sp(), _torch()
    W, g, x = synth.random_case(64, 128, 2, seed=5)
    c = sp.spectra_pack(W, g)
    y = torch.empty(64, dtype=torch.float16, device="cuda")
    xd = torch.from_numpy(x.reshape(-1)).cuda()
    good = {"containers": [c], "ys": [y], "input": -1, "x": xd}
    with pytest.raises(sp.SpectraError) as e:
        sp.StepPlan([good, {"containers": [c], "ys": [y], "input": 0}])  # K 128 != N 64
    assert e.value.status == sp.SPECTRA_E_INVAL
    with pytest.raises(sp.SpectraError) as e:
        sp.StepPlan([dict(good, x_scale=0.3)])
    assert e.value.status == sp.SPECTRA_E_INVAL
    with pytest.raises(sp.SpectraError) as e:
        sp.StepPlan([dict(good, input=0)])  # a phase cannot read itself
    assert e.value.status == sp.SPECTRA_E_INVAL
    Wb, gb, _ = synth.random_case(8, 12000, 0, seed=6)  # G = 375 > 320
    cb = sp.spectra_pack(Wb, gb)
    with pytest.raises(sp.SpectraError) as e:
        sp.StepPlan([{"containers": [cb], "ys": [torch.empty(8, dtype=torch.float16, device="cuda")],
                      "input": -1, "x": torch.zeros(12000, dtype=torch.float16, device="cuda")}])
    assert e.value.status == sp.SPECTRA_E_UNSUPPORTED
    c2 = sp.spectra_pack(W, g)
    h = c2.handle.value
    c2.close()
    with pytest.raises(sp.SpectraError):
        bad = sp.Container(h)  # a freed handle is rejected, not dereferenced
        sp.StepPlan([{"containers": [bad], "ys": [y], "input": -1, "x": xd}])
    bad.ptr = 0


def decoder_stack(layer_ids, cfg=3):
    """Containers and outputs of config-3 decoder layers, with the chain's
    power-of-two input scales from the weights' row norms."""
    sp, torch = _sp(), _torch()
    wl = synth.workload(cfg)
    by = {}
    for lin in wl.linears:
        if lin.layer in layer_ids:
            by.setdefault(lin.layer, {})[lin.name.split(".")[-1]] = lin
    layers, gains = [], []
    for l in layer_ids:
        L = {}
        for nm, lin in by[l].items():
            W = synth.weights(lin, cfg)
            c = sp.spectra_pack(W, synth.gamma(lin, cfg))
            L[nm] = (c, torch.zeros(lin.N, dtype=torch.float16, device="cuda"))
            if nm in ("q", "o", "gate", "down"):
                w = W.astype(np.float32).ravel()
                L["gain_" + nm] = float(np.sqrt(np.dot(w, w) / lin.N))
        layers.append(L)
        gains += [L["gain_q"], L["gain_o"], L["gain_gate"], L["gain_down"]]
    x0 = torch.from_numpy(synth.activations(by[layer_ids[0]]["q"], cfg, 1).reshape(-1)).cuda()
    phases = decoder.layer_phases(layers, x0, decoder.chain_scales(gains))
    return phases


def test_step_decoder_layers_at_bench_shapes():
    """Two 4B-class layers (hidden 2560, MLP 9728; grouped q/k/v and gate/up)
    through the persistent kernel: every output of every phase against the
    oracle and bit-equal to the grouped / single GEMV launches."""
    sp = _sp()
    phases = decoder_stack([0, 35])
    plan = sp.StepPlan(phases)
    plan.run()
    assert plan.status() == sp.SPECTRA_OK
    outs = check_phases(phases)
    for p, o in enumerate(outs):  # the chain stays finite and away from zero
        for v in o:
            f = v.astype(np.float64)
            assert np.isfinite(f).all() and 0.05 < np.sqrt((f * f).mean()) < 20, f"phase {p} rms {np.sqrt((f * f).mean())}"
    plan.close()


def test_step_decoder_36_layers_sampled():
    """The benchmark's whole 36-layer step: bit-equal to the GEMV launches on
    every phase, oracle bound on sampled rows of every container of layers
    0, 17 and 35."""
    sp = _sp()
    phases = decoder_stack(list(range(36)))
    plan = sp.StepPlan(phases)
    for _ in range(2):
        plan.run()
    assert plan.status() == sp.SPECTRA_OK
    rng = np.random.default_rng(36)
    rows = rng.integers(0, 9728, 24)
    which = {p for p, ph in enumerate(phases) if ph["layer"] in (0, 17, 35)}
    check_phases(phases, rows=rows, which=which)
    plan.close()
