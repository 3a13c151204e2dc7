"""Out-of-range tables stay inside every buffer ("vLLM 中 Attention Kernel 如何
并行处理多个请求", section 十一: a request reaches the cache only through its own
table row).  The kernels clamp each length to what its table (or index) row
can address and read a page number outside the pool as a page of zero rows,
so such a call computes a well-defined result instead of reading foreign
memory:

* a block-table entry outside [0, num_blocks) gives bitwise the result of the
  same entry pointing at an all-zero page;
* a length above max_blocks_per_seq * page_size gives bitwise the result of
  that maximum length;
* sparse decode: a listed position outside the table's reach is a zero row,
  a list length above topk is topk.

Every access of these cases was checked against the buffers by reading the
kernel's address arithmetic; they run on the GPU like any other parity case.
mla_check_inputs rejects all of these inputs on the host (tests/test_host_abi.py)."""
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


def with_zero_page(inp):
    """The pool with one extra all-zero page appended (index num_blocks)."""
    kv = inp.kv_bits
    zero = np.zeros((1,) + kv.shape[1:], dtype=kv.dtype)
    return np.concatenate([kv, zero], axis=0)


@pytest.mark.parametrize("mode,splits", [(0, 1), (0, 3), (1, 5)])
@pytest.mark.parametrize("H", [16, 128])
def test_bad_pages_read_as_zero_rows(mla, mode, splits, H):
    sl = (40, 100, 77)
    inp = W.small_case(seed=800 + H, batch=len(sl), num_heads=H, head_size=576,
                       kv_lora_rank=512, page_size=16, seq_lens=sl, table_pad=1)
    w = inp.workload
    nb = inp.kv_bits.shape[0]
    bad = inp.block_table.copy()
    bad[1, 2] = nb + 1000          # past the pool
    bad[2, 0] = -5                 # negative
    bad[2, 4] = 2 ** 31 - 1        # the largest int32
    zero_tab = inp.block_table.copy()
    zero_tab[1, 2] = zero_tab[2, 0] = zero_tab[2, 4] = nb
    q = dev(inp.q_bits.view(np.int16)).view(torch.bfloat16)
    kv = dev(inp.kv_bits.view(np.int16)).view(torch.bfloat16)
    kvz = dev(with_zero_page(inp).view(np.int16)).view(torch.bfloat16)
    sl_d = dev(inp.seq_lens)
    print(f"[table-safety] bad pages H={H} mode={mode} S={splits}", flush=True)
    o1, l1 = mla.mla_decode(q, kv, dev(bad), sl_d, w.scale, 16, 1.0, splits, split_mode=mode)
    o2, l2 = mla.mla_decode(q, kvz, dev(zero_tab), sl_d, w.scale, 16, 1.0, splits,
                            split_mode=mode)
    torch.cuda.synchronize()
    assert torch.isfinite(o1).all() and torch.equal(o1, o2) and torch.equal(l1, l2)
    with pytest.raises(ValueError, match="MLA_ERR_TABLE"):
        mla.mla_decode(q, kv, dev(bad), sl_d, w.scale, 16, 1.0, splits, split_mode=mode,
                       check=True)


@pytest.mark.parametrize("mode,splits", [(0, 1), (1, 4)])
def test_lengths_past_the_table_are_clamped(mla, mode, splits):
    W_, P = 3, 16
    sl = (20, 48, 5)
    inp = W.small_case(seed=810, batch=len(sl), num_heads=32, head_size=576, kv_lora_rank=512,
                       page_size=P, seq_lens=sl)
    assert inp.block_table.shape[1] == W_
    w = inp.workload
    q = dev(inp.q_bits.view(np.int16)).view(torch.bfloat16)
    kv = dev(inp.kv_bits.view(np.int16)).view(torch.bfloat16)
    bt = dev(inp.block_table)
    long = np.array([20, 10 ** 9, 5], dtype=np.int32)   # beyond the 48 positions a row holds
    print(f"[table-safety] long lengths mode={mode} S={splits}", flush=True)
    o1, l1 = mla.mla_decode(q, kv, bt, dev(long), w.scale, P, 1.0, splits, split_mode=mode)
    o2, l2 = mla.mla_decode(q, kv, bt, dev(inp.seq_lens), w.scale, P, 1.0, splits,
                            split_mode=mode)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    neg = np.array([20, -7, 5], dtype=np.int32)           # a negative length is empty
    o3, l3 = mla.mla_decode(q, kv, bt, dev(neg), w.scale, P, 1.0, splits, split_mode=mode)
    zero = np.array([20, 0, 5], dtype=np.int32)
    o4, l4 = mla.mla_decode(q, kv, bt, dev(zero), w.scale, P, 1.0, splits, split_mode=mode)
    torch.cuda.synchronize()
    assert torch.equal(o3, o4) and torch.equal(l3, l4)
    assert (o3[1] == 0).all() and torch.isneginf(l3[1]).all()


@pytest.mark.parametrize("mode,splits", [(0, 1), (1, 3)])
def test_sparse_bad_entries(mla, mode, splits):
    sl = (300, 200)
    inp = W.small_case(seed=820, batch=len(sl), num_heads=128, head_size=576, kv_lora_rank=512,
                       page_size=16, seq_lens=sl, topk=64, table_pad=2)
    w = inp.workload
    nb = inp.kv_bits.shape[0]
    idx = inp.topk_indices.copy()
    lens = inp.topk_lens.copy()
    cap = inp.block_table.shape[1] * 16
    bad_idx = idx.copy()
    bad_idx[0, 3] = cap + 5        # past what the table row addresses
    bad_idx[1, 0] = -1             # negative
    # the same list entries read through an all-zero page: table slot 19 (two
    # padding slots past the 19 pages of the longest sequence) points at the zero
    # page, and the reference lists a position in it where the bad run has a bad one
    assert inp.block_table.shape[1] == 21 and idx.max() < 19 * 16
    zt = inp.block_table.copy()
    zt[:, 19] = nb
    ref_idx = idx.copy()
    ref_idx[0, 3] = 19 * 16 + 1
    ref_idx[1, 0] = 19 * 16
    q = dev(inp.q_bits.view(np.int16)).view(torch.bfloat16)
    kv = dev(inp.kv_bits.view(np.int16)).view(torch.bfloat16)
    kvz = dev(with_zero_page(inp).view(np.int16)).view(torch.bfloat16)
    print(f"[table-safety] sparse mode={mode} S={splits}", flush=True)
    o1, l1 = mla.mla_decode_sparse(q, kv, dev(inp.block_table), dev(bad_idx), dev(lens),
                                   w.scale, 16, 1.0, splits, split_mode=mode)
    o2, l2 = mla.mla_decode_sparse(q, kvz, dev(zt), dev(ref_idx), dev(lens), w.scale, 16, 1.0,
                                   splits, split_mode=mode)
    # a list length above topk is topk
    o3, l3 = mla.mla_decode_sparse(q, kv, dev(inp.block_table), dev(idx),
                                   dev(np.array([64, 10 ** 6], dtype=np.int32)), w.scale, 16,
                                   1.0, splits, split_mode=mode)
    o4, l4 = mla.mla_decode_sparse(q, kv, dev(inp.block_table), dev(idx),
                                   dev(np.array([64, 64], dtype=np.int32)), w.scale, 16, 1.0,
                                   splits, split_mode=mode)
    torch.cuda.synchronize()
    assert torch.isfinite(o1).all() and torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o3, o4) and torch.equal(l3, l4)
