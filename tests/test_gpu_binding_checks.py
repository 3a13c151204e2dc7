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
