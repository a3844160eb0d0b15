"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Expert ids and route buckets must match bit for bit; gate weights within 1e-6;
the bf16 output within max|err| <= 2e-2 * rms(ref).  The five workloads run at
their full sizes in the same launch configuration the benchmark times; the
oracle computes every output of every workload (every route column of the
128-route MFMA chunks that occurs is covered).  Edge
cases: ragged token counts, k = E, all tokens on the same experts, all
routes on distinct experts, zero input, guard regions around the output and
workspace, bitwise run-to-run determinism, and graph replays with changed
inputs.
"""

import numpy as np
import pytest
import torch

import oracle
import sparse_moe_expert_amd as sme
from gpu_harness import (
    DEV,
    assert_buckets,
    assert_output,
    assert_route,
    chunk_columns,
    collect,
    device_packed,
    device_weights,
    oracle_all,
    run_gpu,
    shared_decoder,
    to_dev,
    x_bits,
)
from moe_inputs import make_workload
from moe_inputs.configs import CONFIG_ORDER

pytestmark = pytest.mark.gpu


# Every workload is compared on every output (the whole [T, H] output, rms
# over all of it).  The oracle decodes each expert of the shared bank once
# per session.
def _parity_tokens(wl, idx):
    return list(range(wl.T))


_REFS = {}


def _workload_reference(name):
    """Routing, buckets, compared tokens and the oracle's output on them, once
    per workload (shared by the three paths)."""
    if name not in _REFS:
        wl = make_workload(name)
        idx, w = oracle.route_topk(wl.logits, wl.bias, wl.k)
        b = oracle.bucket_routes(idx, wl.E)
        tokens = _parity_tokens(wl, idx)
        y = oracle.moe_output(wl.x, wl.bank, idx, w, tokens=tokens, decoder=shared_decoder(wl.bank))
        _REFS[name] = (wl, idx, w, b, tokens, y)
    return _REFS[name]


PATHS = ["step", "packed", "calls"]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("name", CONFIG_ORDER)
def test_workload_parity(name, path):
    print(f"[parity] {name} path={path}", flush=True)
    wl, idx, w, b, tokens, y_ref = _workload_reference(name)
    g = run_gpu(wl.x, wl.logits, wl.bias, wl.bank, wl.k, path=path)
    assert_route(g, idx, w)
    assert_buckets(g, b)
    pairs, cols = chunk_columns(idx, b, tokens)
    if wl.T >= 64:
        # every route column that occurs in the 128-route chunks of the
        # matrix-core kernels (route tile col // 32, lane col % 32) is compared
        # somewhere
        _, all_cols = chunk_columns(idx, b, range(wl.T))
        assert cols == all_cols, sorted(all_cols - cols)[:8]
    err, rms = assert_output(g["y"][tokens], y_ref, name)
    over = int(np.sum(np.abs(g["y"][tokens] - y_ref) > 2e-2 * rms))
    print(f"[parity] {name} path={path}: tokens={len(tokens)}/{wl.T} routes={len(tokens) * wl.k} "
          f"expert_column_pairs={len(pairs)} chunk_columns={len(cols)} max_err={err:.3e} rms={rms:.3e} "
          f"ratio={err / rms if rms else 0.0:.4f} elements_over_plain_2e-2_rms={over}", flush=True)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("T", [1, 5, 12, 33])
@pytest.mark.parametrize("shape", ["tiny", "decode_t4"])
def test_ragged_token_counts(shape, T, path):
    wl = make_workload(shape, T=T, x_seed=100 + T)
    print(f"[ragged] {shape} T={T} path={path}", flush=True)
    g = run_gpu(wl.x, wl.logits, wl.bias, wl.bank, wl.k, path=path)
    idx, w, b, y = oracle_all(wl.x, wl.logits, wl.bias, wl.bank, wl.k)
    assert_route(g, idx, w)
    assert_buckets(g, b)
    assert_output(g["y"], y, f"{shape} T={T}")


# Shapes whose row tiles run past the matrix: with H = 256 a gate/up tile
# spans 128 rows of I and a down tile 512-1024 rows of H, so rows past I (or
# H) must read as zeros and never be stored.  T picks the kernels: 8 tokens
# the fused down/unroute kernel, 40 the per-expert down tiles (R > 128; with
# E = 4 each expert's row tiles loop over ~40 routes), 128 the MFMA tiles as
# well (128 weight rows per tile against I = 64).
RAGGED_TILE_SHAPES = [
    # (H, I, E, k, T)
    (256, 64, 16, 4, 8),
    (256, 64, 16, 4, 40),
    (256, 64, 16, 4, 128),
    (128, 32, 8, 2, 70),
    (128, 64, 8, 2, 70),     # the packed down kernel's second 128-row tile lies past H
    (32, 32, 4, 2, 10),
    (32, 64, 6, 3, 50),
    (256, 64, 4, 4, 40),     # ~40 routes per expert in a batch under 64 tokens
]


@pytest.mark.parametrize("path", ["step", "packed"])
@pytest.mark.parametrize("shape", RAGGED_TILE_SHAPES, ids=lambda s: "H%d_I%d_E%d_k%d_T%d" % s)
def test_ragged_row_tiles(shape, path):
    from dataclasses import replace
    from moe_inputs.configs import get_config
    H, I, E, k, T = shape
    cfg = replace(get_config("tiny"), name="ragged_tiles", H=H, I=I, E=E, k=k, T=T)
    wl = make_workload(cfg, x_seed=11 + T)
    if path == "packed" and (H % 64 or I % 64):
        pytest.skip("packed weights need H and I multiples of 64")
    print(f"[ragged tiles] H={H} I={I} E={E} k={k} T={T} path={path}", flush=True)
    g = run_gpu(wl.x, wl.logits, wl.bias, wl.bank, wl.k, path=path)
    idx, w, b, y = oracle_all(wl.x, wl.logits, wl.bias, wl.bank, wl.k)
    assert_route(g, idx, w)
    assert_buckets(g, b)
    # shapes this small have max|y| up to ~6 * rms: the output's own bf16
    # rounding alone can exceed 2e-2 * rms here
    assert_output(g["y"], y, f"ragged tiles {shape}")


@pytest.mark.parametrize("path", PATHS)
def test_k_equals_E(path):
    wl = make_workload("tiny", T=6, x_seed=7)
    g = run_gpu(wl.x, wl.logits, None, wl.bank, wl.E, path=path)
    idx, w, b, y = oracle_all(wl.x, wl.logits, None, wl.bank, wl.E)
    assert_route(g, idx, w)
    assert_buckets(g, b)
    assert_output(g["y"], y, "k=E")


@pytest.mark.parametrize("path", ["step", "packed"])
@pytest.mark.parametrize("T", [12, 33, 300])
def test_all_tokens_on_same_experts(T, path):
    """Every token routed to the same 10 experts: T routes per expert, so the
    kernels loop over the expert's tokens (T = 12: the small-batch routing
    kernel and the fused down/unroute kernel; T = 33: the larger-batch
    kernels; T = 300: the matrix-core kernels with two full 128-route chunks
    and a partial one per expert, each chunk its own work item), on both
    weight layouts."""
    wl = make_workload("decode_t4", T=T, x_seed=3)
    chosen = [7, 100, 101, 250, 311, 312, 400, 450, 500, 511]
    bias = np.zeros(wl.E, np.float32)
    bias[chosen] = 50.0
    g = run_gpu(wl.x, wl.logits, bias, wl.bank, wl.k, path=path)
    idx, w, b, y = oracle_all(wl.x, wl.logits, bias, wl.bank, wl.k)
    assert int(b["n_active"]) == 10 and sorted(np.unique(idx)) == chosen
    assert_route(g, idx, w)
    assert_buckets(g, b)
    err, rms = assert_output(g["y"], y, "all-equal experts")
    print(f"[same experts] T={T} path={path}: every token, max_err={err:.3e} rms={rms:.3e}", flush=True)


@pytest.mark.parametrize("path", ["step", "packed"])
@pytest.mark.parametrize("T", [12, 40])
def test_all_routes_on_distinct_experts(T, path):
    wl = make_workload("decode_t4", T=T, x_seed=4)
    k, E = 10, 512
    logits = np.zeros((T, E), np.float32)
    rng = np.random.default_rng(0)
    perm = rng.permutation(E)[: T * k].reshape(T, k)
    for t in range(T):
        logits[t, perm[t]] = 10.0 - np.arange(k, dtype=np.float32) * 0.5
    g = run_gpu(wl.x, logits, None, wl.bank, k, path=path)
    idx, w, b, y = oracle_all(wl.x, logits, None, wl.bank, k)
    assert np.all(b["expert_count"][b["expert_count"] > 0] == 1) and int(b["n_active"]) == T * k
    assert_route(g, idx, w)
    assert_buckets(g, b)
    assert_output(g["y"], y, "all-disjoint experts")


def test_zero_input_gives_exact_zero():
    wl = make_workload("decode_t4")
    x = np.zeros_like(wl.x)
    logits = np.zeros_like(wl.logits)
    g = run_gpu(x, logits, None, wl.bank, wl.k)
    assert np.array_equal(g["idx"], np.tile(np.arange(wl.k, dtype=np.int32), (wl.T, 1)))
    assert np.all(g["w"] == np.float32(1.0 / wl.k))
    assert np.all(g["y_bits"] == 0)


@pytest.mark.parametrize("path", PATHS)
def test_guard_regions_untouched(path):
    wl = make_workload("decode_t4", T=5, x_seed=9)
    T, H, I, E, k = wl.T, wl.H, wl.I, wl.E, wl.k
    W = device_weights(wl.bank)
    step = sme.MoeStep(T, H, I, E, k, DEV, path=path)
    ws_bytes = sme.moe_step_workspace_size(T, H, I, E, k)
    big_ws = torch.zeros(ws_bytes + 512, dtype=torch.uint8, device=DEV)
    big_ws[:256] = 0xA5
    big_ws[256 + ws_bytes:] = 0x5A
    step.workspace = big_ws[256: 256 + ws_bytes]
    big_y = torch.full((T + 2, H), 3.0, dtype=torch.bfloat16, device=DEV)
    step.y = big_y[1: T + 1]
    step.run(x_bits(wl.x), to_dev(wl.logits), None, W, packed=device_packed(wl.bank) if path == "packed" else None)
    torch.cuda.synchronize()
    assert torch.all(big_ws[:256] == 0xA5) and torch.all(big_ws[256 + ws_bytes:] == 0x5A)
    assert torch.all(big_y[0] == 3.0) and torch.all(big_y[T + 1] == 3.0)
    idx, w, b, y = oracle_all(wl.x, wl.logits, None, wl.bank, k)
    assert_output(big_y[1: T + 1].float().cpu().numpy().astype(np.float64), y, "guarded")


@pytest.mark.parametrize("name", ["decode_t4", "decode_t256_zipf"])
def test_bitwise_determinism(name):
    wl = make_workload(name)
    a = run_gpu(wl.x, wl.logits, wl.bias, wl.bank, wl.k)
    b = run_gpu(wl.x, wl.logits, wl.bias, wl.bank, wl.k)
    for key in ("idx", "route_src", "route_pos", "y_bits"):
        assert np.array_equal(a[key], b[key]), key
    assert np.array_equal(a["w"].view(np.uint32), b["w"].view(np.uint32))


@pytest.mark.parametrize("path", PATHS)
def test_graph_replays_with_changed_inputs(path):
    """Capture the step once; replay with inputs A, B, A, B with eager work
    and synchronisation between replays; each replay must match the oracle
    for its inputs (the workspace needs no reset between replays)."""
    A = make_workload("decode_t4", x_seed=11)
    B = make_workload("decode_t4", x_seed=12)
    T, H, I, E, k = A.T, A.H, A.I, A.E, A.k
    W = device_weights(A.bank)
    step = sme.MoeStep(T, H, I, E, k, DEV, path=path)
    pk = device_packed(A.bank) if path == "packed" else None
    x_s = x_bits(A.x)
    l_s = to_dev(A.logits)
    step.run(x_s, l_s, None, W, packed=pk)          # warm-up outside capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step.run(x_s, l_s, None, W, packed=pk)
    torch.cuda.synchronize()
    refs = {}
    for wl in (A, B):
        idx, w, b, y = oracle_all(wl.x, wl.logits, None, wl.bank, k)
        refs[id(wl)] = (idx, w, b, y)
    for rep, wl in enumerate([A, B, A, B]):
        x_s.copy_(x_bits(wl.x))
        l_s.copy_(to_dev(wl.logits))
        junk = torch.randn(1024, device=DEV).sum()   # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        g = collect(step)
        idx, w, b, y = refs[id(wl)]
        assert_route(g, idx, w)
        assert_buckets(g, b)
        assert_output(g["y"], y, f"replay {rep}")
        del junk


def test_hand_worked_cases_on_gpu():
    """The closed-form golden FFN cases (H = I = 32) through the GPU path."""
    import math
    import pins
    from nvfp4_testlib import bank_from_case, x_from_case
    for case in pins.load_golden("ffn_hand_worked.json")["cases"]:
        bank = bank_from_case(case)
        x = x_from_case(case)
        logits = np.array(case["logits"], dtype=np.float32)
        g = run_gpu(x, logits, None, bank, case["k"])
        assert g["idx"].tolist() == case["idx"]
        ev = lambda s: float(eval(s, {"math": math, "__builtins__": {}}))  # noqa: E731
        ref = np.empty((case["T"], case["H"]))
        ref[:, 0::2] = ev(case["y"]["even"])
        ref[:, 1::2] = ev(case["y"]["odd"])
        assert_output(g["y"], ref, case["name"])


@pytest.mark.parametrize("name", CONFIG_ORDER)
def test_fused_routing_matches_two_calls(name):
    """moe_route_bucket and moe_step give exactly the routing outputs of
    moe_route_topk + moe_bucket_routes."""
    wl = make_workload(name)
    logits = to_dev(wl.logits)
    bias = None if wl.bias is None else to_dev(wl.bias)
    a = sme.MoeStep(wl.T, wl.H, wl.I, wl.E, wl.k, DEV, path="calls")
    b = sme.MoeStep(wl.T, wl.H, wl.I, wl.E, wl.k, DEV, path="calls_unfused")
    c = sme.MoeStep(wl.T, wl.H, wl.I, wl.E, wl.k, DEV, path="step")
    a.routing(logits, bias)
    b.routing(logits, bias)
    c.run(x_bits(wl.x), logits, bias, device_weights(wl.bank))
    torch.cuda.synchronize()
    for s in (a, c):
        assert torch.equal(s.topk_idx, b.topk_idx)
        assert torch.equal(s.topk_w.view(torch.int32), b.topk_w.view(torch.int32))
        for ta, tb in zip(s.buckets, b.buckets):
            assert torch.equal(ta, tb)


# (T, E, k, ties, bias): batches on both sides of the one-workgroup routing
# limit (16 tokens), expert counts that are not a multiple of 64, k = E,
# k = 32, k = 1, the unrolled k = 10 and other k, and heavy ties; then the
# chunked bucketing (one workgroup per 1024 routes): 1023, 1024 and 1025
# routes, 1030 routes over 100 experts, k = E = 8 (every expert in every
# chunk, 64 routes of one expert in a wavefront), 65536 routes (its limit)
# and 65568 (past it: the one-workgroup bucketing).
ROUTING_EDGE_CASES = [
    (1, 512, 10, False, False), (4, 512, 10, False, True), (6, 512, 10, True, False),
    (16, 512, 4, False, False), (7, 100, 9, True, True), (13, 100, 5, False, False),
    (16, 1000, 4, True, False), (3, 64, 10, False, False), (5, 8, 8, False, False),
    (2, 1024, 32, True, False), (16, 1024, 1, False, False), (8, 200, 8, True, False),
    (17, 512, 10, False, True), (40, 100, 3, True, False), (64, 512, 10, False, False),
    (1023, 512, 1, False, False), (1024, 512, 1, True, False), (205, 512, 5, False, True),
    (103, 100, 10, True, False), (400, 8, 8, False, False), (2048, 512, 32, False, True),
    (2049, 512, 32, True, False),
]


@pytest.mark.parametrize("case", ROUTING_EDGE_CASES, ids=lambda c: "T%d_E%d_k%d_ties%d_bias%d" % c)
def test_fused_routing_edges(case):
    """moe_route_bucket against the oracle (bit-exact ids and buckets, weights
    within 1e-6) and against the two separate calls, bit for bit."""
    T, E, k, ties, with_bias = case
    rng = np.random.default_rng(1000 + T * 7 + E + k)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    if ties:
        logits = (np.round(logits * 2.0) / 2.0).astype(np.float32)   # few distinct scores
    bias = (0.5 * rng.standard_normal(E)).astype(np.float32) if with_bias else None
    idx_ref, w_ref = oracle.route_topk(logits, bias, k)
    b_ref = oracle.bucket_routes(idx_ref, E)
    ld = to_dev(logits)
    bd = None if bias is None else to_dev(bias)
    fused = sme.MoeStep(T, 64, 64, E, k, DEV, path="calls")
    split = sme.MoeStep(T, 64, 64, E, k, DEV, path="calls_unfused")
    fused.routing(ld, bd)
    split.routing(ld, bd)
    torch.cuda.synchronize()
    g = collect(fused, with_y=False)
    assert_route(g, idx_ref, w_ref)
    assert_buckets(g, b_ref)
    assert torch.equal(fused.topk_idx, split.topk_idx)
    assert torch.equal(fused.topk_w.view(torch.int32), split.topk_w.view(torch.int32))
    for ta, tb in zip(fused.buckets, split.buckets):
        assert torch.equal(ta, tb)


@pytest.mark.parametrize("name", ["tiny", "decode_t4", "verify_t32", "decode_t256_zipf"])
def test_stages_compose_to_full_call(name):
    """moe_expert_ffn_stage 1 then 2 equals moe_expert_ffn bit for bit
    (decode_t256_zipf: the matrix-core kernels, whose work list stage 2
    rebuilds on its own)."""
    wl = make_workload(name)
    W = device_weights(wl.bank)
    st = sme.MoeStep(wl.T, wl.H, wl.I, wl.E, wl.k, DEV)
    x = x_bits(wl.x)
    st.routing(to_dev(wl.logits), None if wl.bias is None else to_dev(wl.bias))
    st.ffn(x, W)
    torch.cuda.synchronize()
    full = st.y.clone()
    st.y.zero_()
    st.ffn(x, W, stage=1)
    st.ffn(x, W, stage=2)
    torch.cuda.synchronize()
    assert torch.equal(full.view(torch.int16), st.y.view(torch.int16))


def _pack_reference(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """The packed layout of one matrix, written out in numpy from its
    definition: 128-row tiles t, 64-wide steps s, 32-row groups w, lanes l
    (row 128t + 32w + l%32, half l//32); 16 code bytes and 2 scale bytes per
    (t, s, w, l) in that order, rows past N zero, each expert padded to 256."""
    E, N, K2 = codes.shape
    K = 2 * K2
    tiles, steps = (N + 127) // 128, K // 64
    out = []
    for e in range(E):
        c = np.zeros((tiles * 128, K2), np.uint8)
        c[:N] = codes[e]
        sc = np.zeros((tiles * 128, K // 16), np.uint8)
        sc[:N] = scales[e]
        cb, sb = [], []
        for t in range(tiles):
            for st in range(steps):
                for w in range(4):
                    for l in range(64):
                        r, h = 128 * t + 32 * w + (l % 32), l // 32
                        cb.append(c[r, 32 * st + 16 * h: 32 * st + 16 * h + 16])
                        sb.append(sc[r, 4 * st + 2 * h: 4 * st + 2 * h + 2])
        m = np.concatenate([np.concatenate(cb), np.concatenate(sb)])
        out.append(np.concatenate([m, np.zeros((-m.size) % 256, np.uint8)]))
    return np.concatenate(out)


@pytest.mark.parametrize("shape", [(3, 256, 128), (2, 128, 64), (2, 64, 192)])
def test_packed_weights_layout(shape):
    """moe_pack_weights is the byte permutation its header defines (bit-exact)."""
    from dataclasses import replace
    from moe_inputs.configs import get_config
    E, H, I = shape
    wl = make_workload(replace(get_config("tiny"), name="pack", H=H, I=I, E=E, k=1, T=1))
    b = wl.bank
    packed = device_packed(b).cpu().numpy()
    ref = np.concatenate([_pack_reference(b.w_gate, b.s_gate), _pack_reference(b.w_up, b.s_up),
                          _pack_reference(b.w_down, b.s_down)])
    assert packed.shape == ref.shape
    assert np.array_equal(packed, ref)
