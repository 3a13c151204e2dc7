"""The Python binding refuses buffers the kernels would index past: the C ABI
takes raw pointers, so the binding checks that block_table, the sequence
lengths and o / lse hold B sequences before anything is enqueued."""
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


@pytest.fixture(scope="module")
def case():
    sl = (37, 100, 5)
    inp = W.small_case(seed=620, batch=3, num_heads=16, head_size=576, kv_lora_rank=512,
                       page_size=16, seq_lens=sl, topk=32)
    q = torch.from_numpy(inp.q_bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    kv = torch.from_numpy(inp.kv_bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    bt = torch.from_numpy(inp.block_table).to(DEV)
    sl_d = torch.from_numpy(inp.seq_lens).to(DEV)
    idx = torch.from_numpy(inp.topk_indices).to(DEV)
    lens = torch.from_numpy(inp.topk_lens).to(DEV)
    return inp.workload, q, kv, bt, sl_d, idx, lens


def test_decode_refuses_short_buffers(mla, case):
    w, q, kv, bt, sl, _, _ = case
    o = torch.empty((3, 16, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((3, 16), dtype=torch.float32, device=DEV)
    args = (w.scale, w.page_size, 1.0, 2)
    with pytest.raises(ValueError):
        mla.mla_decode(q, kv, bt, sl[:2].contiguous(), *args, o, lse)
    with pytest.raises(ValueError):
        mla.mla_decode(q, kv, bt[:2].contiguous(), sl, *args, o, lse)
    with pytest.raises(ValueError):
        mla.mla_decode(q, kv, bt, sl, *args, o[:2].contiguous(), lse)
    with pytest.raises(ValueError):
        mla.mla_decode(q, kv, bt, sl, *args, o, lse[:, :8].contiguous())
    mla.mla_decode(q, kv, bt, sl, *args, o, lse)  # the right sizes go through
    torch.cuda.synchronize()


def test_sparse_and_prepared_calls_refuse_short_buffers(mla, case):
    w, q, kv, bt, sl, idx, lens = case
    o = torch.empty((3, 16, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((3, 16), dtype=torch.float32, device=DEV)
    args = (w.scale, w.page_size, 1.0, 2)
    with pytest.raises(ValueError):
        mla.mla_decode_sparse(q, kv, bt, idx, lens[:2].contiguous(), *args, o, lse)
    with pytest.raises(ValueError):
        mla.mla_decode_sparse(q, kv, bt, idx[:2].contiguous(), lens, *args, o, lse)
    with pytest.raises(ValueError):
        mla.mla_decode_sparse(q, kv, bt, idx, lens, *args, o[:, :8].contiguous(), lse)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError):
        mla.PreparedDecode(q, kv, bt, sl, w.scale, w.page_size, 1.0, 2, mla.SPLIT_PER_SEQUENCE,
                           o[:2].contiguous(), lse, ws)
    mla.mla_decode_sparse(q, kv, bt, idx, lens, *args, o, lse)
    torch.cuda.synchronize()


def test_kernel_timing_events_bracket_one_launch(mla, case):
    """mla_time_next_launch: the next stage-1 and stage-2 launches record their
    own start and end into the events, then the setting clears (a later launch
    leaves them as they are)."""
    w, q, kv, bt, sl, _, _ = case
    shape = mla.shape_of(q, kv, bt)
    splits = 3
    need = mla.mla_workspace_size(shape, mla.SPLIT_PER_SEQUENCE, splits)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    o = torch.empty((3, 16, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((3, 16), dtype=torch.float32, device=DEV)
    call = mla.PreparedDecode(q, kv, bt, sl, w.scale, w.page_size, w.k_scale, splits,
                              mla.SPLIT_PER_SEQUENCE, o, lse, ws)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in ev:
        e.record()  # torch creates an event at its first record
    mla.mla_time_next_launch(1, ev[0], ev[1])
    mla.mla_time_next_launch(2, ev[2], ev[3])
    call("both")
    torch.cuda.synchronize()
    t1, t2 = ev[0].elapsed_time(ev[1]), ev[2].elapsed_time(ev[3])
    gap = ev[1].elapsed_time(ev[2])  # stage 2 starts after stage 1 ends
    assert 0 < t1 < 100 and 0 < t2 < 100 and gap >= 0
    call("both")  # the setting was cleared: the events keep the first launch's times
    torch.cuda.synchronize()
    assert ev[0].elapsed_time(ev[1]) == t1 and ev[2].elapsed_time(ev[3]) == t2
