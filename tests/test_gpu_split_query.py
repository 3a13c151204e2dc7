"""GPU parity of the split query: q given as the pair (q_nope, q_pe) of
separate, strided tensors ("Triton と MLA" page, データフロー: forward_mqa
accepts q whole or as that tuple and joins it on the last axis, q_nope first).
The C ABI's mla_decode_split_q reads both parts in place; its result must be
bitwise that of mla_decode on the concatenated query (same kernels, same
values), and within the stated tolerance of the oracle."""
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


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def strided_parts(q, D_v):
    """q_nope as a head-major buffer viewed sequence-major (as a per-head
    up-projection leaves it: strides (row pad, B * row pad, 1)) and q_pe as a
    slice of a padded buffer; neither part is contiguous."""
    B, H, D = q.shape
    pad = D_v + 8
    hm = torch.full((H, B, pad), float("nan"), dtype=q.dtype, device=q.device)
    hm[:, :, :D_v] = q[:, :, :D_v].transpose(0, 1)
    q_nope = hm.transpose(0, 1)[:, :, :D_v]
    pe_buf = torch.full((B, H, (D - D_v) + 16), float("nan"), dtype=q.dtype, device=q.device)
    pe_buf[:, :, 8:8 + D - D_v] = q[:, :, D_v:]
    q_pe = pe_buf[:, :, 8:8 + D - D_v]
    assert not q_nope.is_contiguous() and not q_pe.is_contiguous()
    return q_nope, q_pe


@pytest.mark.parametrize("H,D,P,sl", [(128, 576, 64, (37, 700, 1031, 5)),
                                      (16, 320, 16, (1, 250, 513)),
                                      (48, 576, 16, (3, 129, 40))])
@pytest.mark.parametrize("mode,splits", [(0, 1), (1, 5)])
def test_tuple_query_is_the_concatenated_query(mla, H, D, P, sl, mode, splits):
    inp = W.small_case(seed=700 + H, batch=len(sl), num_heads=H, head_size=D,
                       kv_lora_rank=D - 64, page_size=P, seq_lens=sl)
    w = inp.workload
    q = dev(inp.q_bits.view(np.int16)).view(torch.bfloat16)
    kv = dev(inp.kv_bits.view(np.int16)).view(torch.bfloat16)
    bt, sl_d = dev(inp.block_table), dev(inp.seq_lens)
    q_nope, q_pe = strided_parts(q, D - 64)
    print(f"[split-q] H={H} D={D} mode={mode} S={splits}", flush=True)
    for o_dtype in (torch.float32, torch.bfloat16):
        o1, l1 = mla.mla_decode(q, kv, bt, sl_d, w.scale, P, 1.0, splits, split_mode=mode,
                                o_dtype=o_dtype)
        o2, l2 = mla.mla_decode((q_nope, q_pe), kv, bt, sl_d, w.scale, P, 1.0, splits,
                                split_mode=mode, o_dtype=o_dtype)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
    ro, rl = oracle.decode(inp.q_bits, inp.kv_bits, inp.block_table, inp.seq_lens,
                           scale=w.scale, k_scale=1.0, kv_dtype="bf16", kv_lora_rank=D - 64)
    o32, l32 = mla.mla_decode((q_nope, q_pe), kv, bt, sl_d, w.scale, P, 1.0, splits,
                              split_mode=mode, o_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.abs(o32.cpu().numpy() - ro).max() <= 1e-2
    assert np.abs(l32.cpu().numpy() - rl).max() <= 1e-3


def test_tuple_query_multi_token(mla):
    """q_len = 3: the parts are [B, q_len, H, *] slices of one buffer."""
    sl = (2, 40, 700)
    inp = W.small_case(seed=710, batch=len(sl), num_heads=128, head_size=576, kv_lora_rank=512,
                       page_size=64, seq_lens=sl, q_len=3)
    w = inp.workload
    q = dev(inp.q_bits.view(np.int16)).view(torch.bfloat16)
    kv = dev(inp.kv_bits.view(np.int16)).view(torch.bfloat16)
    bt, sl_d = dev(inp.block_table), dev(inp.seq_lens)
    wide = torch.zeros(q.shape[:-1] + (576 + 64,), dtype=q.dtype, device=DEV)
    wide[..., :512] = q[..., :512]
    wide[..., 576:] = q[..., 512:]
    parts = (wide[..., :512], wide[..., 576:])
    for mode, splits in ((0, 1), (1, 4)):
        o1, l1 = mla.mla_decode(q, kv, bt, sl_d, w.scale, 64, 1.0, splits, split_mode=mode)
        o2, l2 = mla.mla_decode(parts, kv, bt, sl_d, w.scale, 64, 1.0, splits, split_mode=mode)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_tuple_query_rejections(mla):
    inp = W.small_case(seed=720, batch=2, num_heads=16, head_size=576, kv_lora_rank=512,
                       page_size=16, seq_lens=(5, 9))
    w = inp.workload
    q = dev(inp.q_bits.view(np.int16)).view(torch.bfloat16)
    kv = dev(inp.kv_bits.view(np.int16)).view(torch.bfloat16)
    bt, sl_d = dev(inp.block_table), dev(inp.seq_lens)
    with pytest.raises(ValueError):  # q_pe of the wrong width
        mla.mla_decode((q[..., :512], q[..., 500:]), kv, bt, sl_d, w.scale, 16, 1.0, 1)
    with pytest.raises(ValueError):  # a last axis that is not unit-stride
        wide = torch.zeros((2, 16, 128), dtype=torch.bfloat16, device=DEV)
        mla.mla_decode((q[..., :512], wide[..., ::2]), kv, bt, sl_d, w.scale, 16, 1.0, 1)
    with pytest.raises(mla.MlaError):  # a row stride that is not a multiple of 8 elements
        odd = torch.zeros((2, 16, 516), dtype=torch.bfloat16, device=DEV)
        mla.mla_decode((odd[..., :512], q[..., 512:]), kv, bt, sl_d, w.scale, 16, 1.0, 1)
