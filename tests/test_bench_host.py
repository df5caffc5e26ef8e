"""Host logic of bench.py (no GPU): the partition of the timed steps into captured HIP graphs, the
host CPU record and the step budget of the oracle baseline, the hot-prefix length, the traffic
records and the kernel names of the roofline line."""
import pytest

import bench


@pytest.mark.parametrize("steps", [1, 5, 20, 63, 64, 65, 128, 1000, 1024])
@pytest.mark.parametrize("graph_steps", [1, 7, 64, 2048])
def test_graph_plan_covers_every_step_once(steps, graph_steps):
    plan = bench.graph_plan(steps, graph_steps)
    covered = [t for g0, n in plan for t in range(g0, g0 + n)]
    assert covered == list(range(steps))
    assert all(1 <= n <= graph_steps for _, n in plan)
    # only the last graph may be shorter
    assert all(n == graph_steps for _, n in plan[:-1])


def test_graph_plan_driver_command():
    # `bench.py --gpus 1 --steps 20 --warmup 5` with the default graph size: one graph of 20 steps
    assert bench.graph_plan(20, 64) == [(0, 20)]
    assert bench.graph_plan(1024, 64) == [(64 * k, 64) for k in range(16)]
    assert bench.graph_plan(100, 64) == [(0, 64), (64, 36)]


def test_graph_plan_eager_and_errors():
    assert bench.graph_plan(20, 0) == []
    with pytest.raises(ValueError):
        bench.graph_plan(0, 64)


def test_host_cpu_record():
    n, model = bench.host_cpu()
    assert n >= 1 and isinstance(model, str) and model


def test_hot_prefix_len_from_profile_counts():
    import torch
    counts = torch.tensor([512, 512, 511, 507, 506, 300, 2, 0], dtype=torch.int32)
    assert bench.hot_prefix_len(counts, 512, 0.99) == 4  # ceil(0.99 * 512) = 507
    assert bench.hot_prefix_len(counts, 512, 1.0) == 2
    assert bench.hot_prefix_len(counts, 512, 0.001) == 7
    assert bench.hot_prefix_len(torch.zeros(5, dtype=torch.int32), 512, 0.5) == 0
    with pytest.raises(ValueError):
        bench.hot_prefix_len(torch.tensor([1, 9], dtype=torch.int32), 10, 0.5)  # not hot-first
    with pytest.raises(ValueError):
        bench.hot_prefix_len(counts, 512, 0.0)


def test_traffic_hash_ignores_comments_only(tmp_path, monkeypatch):
    # the traffic figures stay valid across comment edits and are dropped by any code edit
    code = "int f(int x) { return x + 1; }\n"
    for f in bench.TRAFFIC_SOURCES:
        p = tmp_path / f
        p.parent.mkdir(parents=True, exist_ok=True)
        p.write_text(code)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.sources_hash()
    first = tmp_path / bench.TRAFFIC_SOURCES[0]
    first.write_text("// a comment\nint f(int x) {  /* another */ return x + 1; }\n")
    assert bench.sources_hash() == h0
    first.write_text("int f(int x) { return x + 2; }\n")
    assert bench.sources_hash() != h0
    monkeypatch.setattr(bench, "TRAFFIC", {("w", 1): {"sources": h0, "bytes": 7}})
    assert bench.measured_traffic("w", 1) is None
    first.write_text(code)
    assert bench.measured_traffic("w", 1) == 7


def test_traffic_record_with_its_own_sources(tmp_path, monkeypatch):
    # a record that names its own kernel sources is dropped by an edit to those files only
    for f in bench.TRAFFIC_SOURCES + bench.BATCH_TRAFFIC_SOURCES:
        p = tmp_path / f
        p.parent.mkdir(parents=True, exist_ok=True)
        p.write_text("int %s;\n" % p.stem)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    hb = bench.sources_hash(bench.BATCH_TRAFFIC_SOURCES)
    monkeypatch.setattr(bench, "TRAFFIC", {("w", 8): {"files": bench.BATCH_TRAFFIC_SOURCES, "sources": hb, "bytes": 9}})
    assert bench.measured_traffic("w", 8) == 9
    only_b1 = [f for f in bench.TRAFFIC_SOURCES if f not in bench.BATCH_TRAFFIC_SOURCES][0]
    (tmp_path / only_b1).write_text("int changed;\n")
    assert bench.measured_traffic("w", 8) == 9
    (tmp_path / bench.BATCH_TRAFFIC_SOURCES[-1]).write_text("int changed;\n")
    assert bench.measured_traffic("w", 8) is None


def test_layer_kernels_names_the_pipeline():
    import synth
    S = synth.CONFIGS
    assert bench.layer_kernels(S["opt30b_relu_f16"], 1) == "k_h1, k_qu, k_dn"
    assert bench.layer_kernels(S["opt175b_relu_i4"], 8).startswith("MFMA batch kernels: k_bh, k_bhred, k_bq_full, k_bscan")
    assert "k_bup (orders the list)" in bench.layer_kernels(S["opt30b_relu_f16"], 4)
    assert bench.layer_kernels(S["falcon40b_stack_f16"], 1, ln=True) == "k_h with the LayerNorm, k_qu, k_dn"
    assert bench.layer_kernels(S["falcon40b_stack_f16"], 32, ln=True).startswith("the LayerNorm kernel, then MFMA batch kernels")


def test_cpu_baseline_budget_and_cap():
    """The oracle baseline times decode steps until its CPU-time budget is spent (at least one),
    at most the given number of steps (0: every token of the workload)."""
    import synth

    spec = synth.CONFIGS["tiny_relu_f32"]
    L = synth.make_layer(spec, seed=1)
    X = synth.make_tokens(spec, 6, seed=2).reshape(6, 1, spec.d)
    r = bench.cpu_baseline(spec, (L, L), X, 1, 4, 100.0)
    assert r["sample"].startswith("4 decode steps") and r["value"] > 0 and r["kind"] == "oracle"
    assert bench.cpu_baseline(spec, (L, L), X, 1, 0, 0.0)["sample"].startswith("1 decode steps")
    assert bench.cpu_baseline(spec, (L, L), X, 1, 0, 100.0)["sample"].startswith("6 decode steps")
