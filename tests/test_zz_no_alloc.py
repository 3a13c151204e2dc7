"""GPU test of the allocation-free entry point mla_decode_noalloc (C ABI,
through the ctypes binding): its stage-1 partials live in the library's
built-in per-device scratch instead of a caller's workspace, so its output
must be bitwise that of mla_decode (the workspace entry point) with the same
split plan.  Two calls in a row, the second on a smaller batch (the scratch
keeps the first call's contents: nothing may leak into the second), in the
balanced and per-sequence split modes, single-token and multi-token decode;
and a plan too large for the scratch is refused before any launch."""
import numpy as np
import pytest

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


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def case(seed, sl, H=128, q_len=1):
    inp = W.small_case(seed=seed, batch=len(sl), num_heads=H, head_size=576, kv_lora_rank=512,
                       page_size=64, seq_lens=sl, q_len=q_len)
    q = dev(inp.q_bits.view(np.int16)).view(torch.bfloat16)
    kv = dev(inp.kv_bits.view(np.int16)).view(torch.bfloat16)
    return inp, q, kv, dev(inp.block_table), dev(inp.seq_lens)


@pytest.mark.parametrize("q_len", [1, 2])
def test_noalloc_matches_workspace_entry_point(mla, q_len):
    big = case(900 + q_len, (4000, 1031, 7000, 300, 2500, 64, 5000, 1), q_len=q_len)
    small = case(910 + q_len, (700, 33, 1500), q_len=q_len)
    for label, (inp, q, kv, bt, sl) in (("big", big), ("small", small)):
        w = inp.workload
        shape = mla.shape_of(q, kv, bt)
        mode, units, ws_bytes = mla.mla_plan(shape, int(inp.seq_lens.max()),
                                             int(inp.seq_lens.sum()), 256, q_len=q_len)
        assert 0 < ws_bytes <= mla.mla_noalloc_scratch_bytes()
        for m, s in ((mode, units), (mla.SPLIT_PER_SEQUENCE, 5), (mla.SPLIT_PER_SEQUENCE, 1)):
            print(f"[noalloc] {label} q_len={q_len} mode={m} S={s}", flush=True)
            rows = tuple(q.shape[:-1])
            o1 = torch.empty(rows + (512,), dtype=torch.bfloat16, device=DEV)
            l1 = torch.empty(rows, dtype=torch.float32, device=DEV)
            o2, l2 = torch.full_like(o1, float("nan")), torch.full_like(l1, float("nan"))
            mla.mla_decode(q, kv, bt, sl, w.scale, 64, 1.0, s, o1, l1, split_mode=m)
            mla.mla_decode_noalloc(q, kv, bt, sl, w.scale, 64, 1.0, s, m, o2, l2)
            torch.cuda.synchronize()
            assert torch.equal(o1, o2) and torch.equal(l1, l2), (label, m, s)


def test_noalloc_refuses_a_plan_beyond_its_scratch(mla):
    inp, q, kv, bt, sl = case(920, (100, 200))
    w = inp.workload
    shape = mla.shape_of(q, kv, bt)
    splits = 65536  # per-sequence: 2 x 65536 partial rows of 128 heads, far above 64 MiB
    assert mla.mla_workspace_size(shape, mla.SPLIT_PER_SEQUENCE, splits) > \
        mla.mla_noalloc_scratch_bytes()
    o = torch.zeros((2, 128, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros((2, 128), dtype=torch.float32, device=DEV)
    with pytest.raises(mla.MlaError, match="MLA_ERR_SCRATCH"):
        mla.mla_decode_noalloc(q, kv, bt, sl, w.scale, 64, 1.0, splits,
                               mla.SPLIT_PER_SEQUENCE, o, lse)
    torch.cuda.synchronize()
    assert (o == 0).all()  # nothing was enqueued
