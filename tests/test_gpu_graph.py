"""A decode step captured into a HIP graph (torch.cuda.CUDAGraph) and replayed.

mla_decode enqueues its two kernels on the caller's stream, allocates nothing
and synchronises nothing, so a serving loop can capture it once and replay it.
Every replay here runs on new query values (copied into the captured buffer
by eager work between replays) and is compared bitwise with an eager call on
the same inputs; one replay per case is also checked against the oracle.
"""
import numpy as np
import pytest

import oracle
import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_paged_latent_decode_amd as m
    m.load_library()
    return m


@pytest.mark.parametrize("mode,splits", [(None, None), (0, 1), (0, 4)])
def test_captured_decode_replays_match_eager(mla, mode, splits):
    sl = (37, 700, 1031, 5)
    inp = W.small_case(seed=600, batch=len(sl), num_heads=128, head_size=576, kv_lora_rank=512,
                       page_size=64, seq_lens=sl)
    w = inp.workload
    q = torch.from_numpy(inp.q_bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    kv = torch.from_numpy(inp.kv_bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    bt = torch.from_numpy(inp.block_table).to(DEV)
    sl_d = torch.from_numpy(inp.seq_lens).to(DEV)
    shape = mla.shape_of(q, kv, bt)
    if mode is None:
        mode, splits, _ = mla.mla_plan(shape, int(max(sl)), int(sum(sl)), 256)
    need = mla.mla_workspace_size(shape, mode, splits)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=DEV)
    o = torch.empty((len(sl), 128, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((len(sl), 128), dtype=torch.float32, device=DEV)
    print(f"[graph] mode={mode} S={splits}", flush=True)

    def step(stream):
        mla.mla_decode(q, kv, bt, sl_d, w.scale, w.page_size, w.k_scale, splits, o, lse,
                       split_mode=mode, workspace=ws, stream=stream)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(side)  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(torch.cuda.current_stream())
    torch.cuda.synchronize()

    rng = np.random.default_rng(601)
    for rep in range(4):
        q_new = W.f32_to_bf16_bits(rng.standard_normal(inp.q_bits.shape, dtype=np.float32))
        q.copy_(torch.from_numpy(q_new.view(np.int16)).view(torch.bfloat16).to(DEV))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o_g, l_g = o.clone(), lse.clone()
        step(torch.cuda.current_stream())  # eager, same inputs
        torch.cuda.synchronize()
        assert torch.equal(o_g, o) and torch.equal(l_g, lse), f"replay {rep}"
        if rep == 3:
            ro, rl = oracle.decode(q_new, inp.kv_bits, inp.block_table, inp.seq_lens,
                                   scale=w.scale, k_scale=w.k_scale, kv_dtype=w.kv_dtype,
                                   kv_lora_rank=w.kv_lora_rank)
            o_np = o_g.float().cpu().numpy().astype(np.float64)
            ax = np.maximum(np.abs(ro), 2.0 ** -126)
            slack = np.exp2(np.floor(np.log2(ax)) - 8)  # bf16 output rounding
            assert (np.abs(o_np - ro) - slack).max() <= 1e-2
            assert np.abs(l_g.cpu().numpy() - rl).max() <= 1e-3
            # the same launch configuration with fp32 output, at the plain tolerances
            o32, l32 = mla.mla_decode(q, kv, bt, sl_d, w.scale, w.page_size, w.k_scale, splits,
                                      split_mode=mode, workspace=ws, o_dtype=torch.float32)
            torch.cuda.synchronize()
            assert np.abs(o32.cpu().numpy().astype(np.float64) - ro).max() <= 1e-2
            assert np.abs(l32.cpu().numpy().astype(np.float64) - rl).max() <= 1e-3


@pytest.mark.parametrize("kind", ["int4_per_token", "mtp", "sparse"])
def test_other_entry_points_replay_like_eager(mla, kind):
    """Per-token int4 cache, multi-token decode (q_len 3) and sparse decode,
    each captured once and replayed on new queries, bitwise equal to eager
    calls on the same inputs."""
    sl = (37, 700, 1031, 5)
    dt = W.INT4_PER_TOKEN if kind == "int4_per_token" else W.BF16
    inp = W.small_case(seed=610, batch=len(sl), num_heads=128, head_size=576, kv_lora_rank=512,
                       page_size=64, seq_lens=sl, kv_dtype=dt,
                       q_len=3 if kind == "mtp" else 1, topk=256 if kind == "sparse" else None)
    w = inp.workload
    q = torch.from_numpy(inp.q_bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    if dt == W.BF16:
        kv = torch.from_numpy(inp.kv_bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    else:
        kv = torch.from_numpy(np.ascontiguousarray(inp.kv_bits)).to(DEV)
    bt = torch.from_numpy(inp.block_table).to(DEV)
    B, H = len(sl), 128
    rows = (B, 3, H) if kind == "mtp" else (B, H)
    o = torch.empty(rows + (512,), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(rows, dtype=torch.float32, device=DEV)
    shape = mla.shape_of(q, kv, bt, kv_dtype=w.kv_dtype)
    splits, mode = 9, mla.SPLIT_BALANCED
    ws = torch.empty(max(mla.mla_workspace_size(shape, mode, splits,
                                                3 if kind == "mtp" else 1), 256),
                     dtype=torch.uint8, device=DEV)
    if kind == "sparse":
        idx = torch.from_numpy(inp.topk_indices).to(DEV)
        lens = torch.from_numpy(inp.topk_lens).to(DEV)
    else:
        sl_d = torch.from_numpy(inp.seq_lens).to(DEV)
    print(f"[graph] {kind}", flush=True)

    def step(stream):
        if kind == "sparse":
            mla.mla_decode_sparse(q, kv, bt, idx, lens, w.scale, w.page_size, w.k_scale, splits,
                                  o, lse, split_mode=mode, workspace=ws, stream=stream)
        else:
            mla.mla_decode(q, kv, bt, sl_d, w.scale, w.page_size, w.k_scale, splits, o, lse,
                           split_mode=mode, workspace=ws, kv_dtype=w.kv_dtype, stream=stream)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    rng = np.random.default_rng(611)
    for rep in range(3):
        q_new = W.f32_to_bf16_bits(rng.standard_normal(inp.q_bits.shape, dtype=np.float32))
        q.copy_(torch.from_numpy(q_new.view(np.int16)).view(torch.bfloat16).to(DEV))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o_g, l_g = o.clone(), lse.clone()
        step(torch.cuda.current_stream())
        torch.cuda.synchronize()
        assert torch.equal(o_g, o) and torch.equal(l_g, lse), f"{kind} replay {rep}"
