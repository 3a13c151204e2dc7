"""Pins of the float64 oracle against facts that do not come from the oracle.

Each test checks the oracle against something fixed by the pages or by
mathematics: a worked example the pages print, a closed form, a library
routine (torch's float64 SDPA, torch's bf16/fp8 decoders), exact rational
arithmetic, or a brute-force loop.  The last group plants mistakes in the
oracle and checks that at least one pin catches each of them.
"""
import dataclasses
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
import oracle.mla_oracle as OM
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_worked_examples.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def run(inp, **kw):
    w = inp.workload
    return O.decode(inp.q_bits, inp.kv_bits, inp.block_table, inp.seq_lens, scale=w.scale,
                    k_scale=w.k_scale, kv_dtype=w.kv_dtype, kv_lora_rank=w.kv_lora_rank, **kw)


def small(seed=11, seq_lens=(37, 100, 1, 64), H=16, D=576, DV=512, P=16, kv="bf16",
          k_scale=1.0):
    return W.small_case(seed=seed, batch=len(seq_lens), num_heads=H, head_size=D,
                        kv_lora_rank=DV, page_size=P, seq_lens=seq_lens, kv_dtype=kv,
                        k_scale=k_scale)


def dense_keys(inp, b):
    """K rows of sequence b, gathered with numpy fancy indexing (independent of
    the oracle's own per-token lookup)."""
    w = inp.workload
    n = int(inp.seq_lens[b])
    P = w.page_size
    pos = np.arange(n)
    rows = inp.block_table[b][pos // P] * P + pos % P
    flat = inp.kv_bits.reshape(-1, inp.kv_bits.shape[-1])[rows]
    if w.kv_dtype == "bf16":
        t = torch.from_numpy(flat.view(np.int16).copy()).view(torch.bfloat16)
        return t.to(torch.float64)
    if w.kv_dtype in ("fp8_per_token", "int8_per_token"):
        D = w.head_size
        code_t = torch.float8_e4m3fn if w.kv_dtype == "fp8_per_token" else torch.int8
        codes = torch.from_numpy(flat[:, :D].copy()).view(code_t).to(torch.float64)
        scale = torch.from_numpy(flat[:, D:D + 4].copy()).view(torch.float32).to(torch.float64)
        return codes * scale
    if w.kv_dtype == "int4_per_token":
        # nibbles with torch integer ops: sign-extend by shifting into an int8's top bits
        nb = w.head_size // 2
        b = torch.from_numpy(flat[:, :nb].copy()).view(torch.int8)
        lo = torch.bitwise_left_shift(b, 4) >> 4
        hi = b >> 4
        codes = torch.stack([lo, hi], dim=-1).reshape(b.shape[0], 2 * nb).to(torch.float64)
        scale = torch.from_numpy(flat[:, nb:nb + 4].copy()).view(torch.float32).to(torch.float64)
        return codes * scale
    t = torch.from_numpy(flat.copy()).view(torch.float8_e4m3fn)
    return t.to(torch.float64) * float(np.float32(w.k_scale))


def q_of(inp, b):
    return torch.from_numpy(inp.q_bits[b].view(np.int16).copy()).view(torch.bfloat16).to(
        torch.float64)


# ---------------------------------------------------------------- storage formats

def test_bf16_decoder_matches_torch_on_every_code():
    codes = np.arange(65536, dtype=np.uint16)
    mine = O.bf16_bits_to_f64(codes)
    ref = torch.from_numpy(codes.view(np.int16).copy()).view(torch.bfloat16).to(
        torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])


def test_e4m3fn_decoder_matches_torch_on_every_code():
    codes = np.arange(256, dtype=np.uint8)
    mine = O.e4m3fn_bits_to_f64(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2  # S.1111.111 only: e4m3fn has no infinity
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])
    assert mine[0x7E] == 448.0 and mine[0x01] == 2.0 ** -9


# ---------------------------------------------------------------- worked examples

def test_paged_address_worked_example():
    g = golden()["paged_address"]
    P = g["block_size"]
    pos = g["logical_position"]
    for blk, slot in ((g["physical_block_request_A"], g["physical_slot_A"]),
                      (g["physical_block_request_B"], g["physical_slot_B"])):
        row = np.zeros(g["logical_block"] + 1, dtype=np.int32)
        row[g["logical_block"]] = blk
        assert pos // P == g["logical_block"] and pos % P == g["offset_in_block"]
        assert O.physical_slot(row, pos, P) == slot


def test_kv_segments_worked_example():
    g = golden()["kv_segments"]
    C = g["segment_length"]
    n = g["segments"][-1][1] + 1
    got = O.segment_bounds(n, C)
    assert [(s, e - 1) for (s, e) in got] == [tuple(x) for x in g["segments"]]
    # a short tail segment
    assert O.segment_bounds(n + 5, C)[-1] == (n, n + 5)


def test_split_count_rule_cases():
    g = golden()["split_count_rule"]
    for c in g["cases"]:
        assert O.pages_split_count(c["max_seq_len"], c["sm_count"]) == c["splits"], c


# ---------------------------------------------------------------- brute force

def _python_attention(q, K, d_v, scale):
    """Per-element loops with math.exp / math.fsum; plain full softmax."""
    H, n = len(q), len(K)
    o = [[0.0] * d_v for _ in range(H)]
    lse = []
    for h in range(H):
        s = [scale * math.fsum(q[h][d] * K[t][d] for d in range(len(q[h]))) for t in range(n)]
        mx = max(s)
        z = math.fsum(math.exp(x - mx) for x in s)
        L = mx + math.log(z)
        lse.append(L)
        for j in range(d_v):
            o[h][j] = math.fsum(math.exp(s[t] - L) * K[t][j] for t in range(n))
    return o, lse


def test_brute_force_python_loops_small_dims():
    inp = small(seed=3, seq_lens=(5, 9, 1), H=3, D=8, DV=4, P=4)
    o, lse = run(inp)
    for b in range(3):
        K = dense_keys(inp, b).tolist()
        q = q_of(inp, b).tolist()
        ro, rl = _python_attention(q, K, 4, float(np.float32(inp.workload.scale)))
        assert np.allclose(o[b], ro, rtol=0, atol=1e-13)
        assert np.allclose(lse[b], rl, rtol=0, atol=1e-13)


def test_matches_torch_sdpa_float64():
    inp = small(seed=5, seq_lens=(37, 100, 1, 64, 17))
    o, lse = run(inp)
    sc = float(np.float32(inp.workload.scale))
    for b in range(len(inp.seq_lens)):
        K = dense_keys(inp, b)
        q = q_of(inp, b)
        H = q.shape[0]
        ref = torch.nn.functional.scaled_dot_product_attention(
            q[:, None, :], K.expand(H, -1, -1), K[:, :512].expand(H, -1, -1), scale=sc)[:, 0]
        ref_lse = torch.logsumexp((q @ K.T) * sc, dim=-1)
        assert np.max(np.abs(o[b] - ref.numpy())) < 1e-12
        assert np.max(np.abs(lse[b] - ref_lse.numpy())) < 1e-12


def test_fp8_cache_matches_torch_sdpa_with_k_scale():
    inp = small(seed=7, seq_lens=(50, 130), kv="fp8_e4m3", k_scale=float(np.float32(0.05)))
    o, lse = run(inp)
    sc = float(np.float32(inp.workload.scale))
    for b in range(2):
        K = dense_keys(inp, b)
        q = q_of(inp, b)
        H = q.shape[0]
        ref = torch.nn.functional.scaled_dot_product_attention(
            q[:, None, :], K.expand(H, -1, -1), K[:, :512].expand(H, -1, -1), scale=sc)[:, 0]
        ref_lse = torch.logsumexp((q @ K.T) * sc, dim=-1)
        assert np.max(np.abs(o[b] - ref.numpy())) < 1e-12
        assert np.max(np.abs(lse[b] - ref_lse.numpy())) < 1e-12


# ---------------------------------------------------------------- closed forms

def _exact(bits_f64):
    return [Fraction(float(x)) for x in bits_f64]


def test_one_token_sequence_returns_its_row_and_score():
    inp = small(seed=9, seq_lens=(1, 1, 1))
    o, lse = run(inp)
    sc = Fraction(float(np.float32(inp.workload.scale)))
    for b in range(3):
        row = dense_keys(inp, b)[0].numpy()
        assert np.array_equal(o[b], np.broadcast_to(row[:512], o[b].shape))
        for h in range(inp.workload.num_heads):
            q = _exact(q_of(inp, b)[h].numpy())
            k = _exact(row)
            exact = sc * sum(a * c for a, c in zip(q, k))
            assert abs(lse[b, h] - float(exact)) <= 1e-12 * max(1.0, abs(float(exact)))


def test_zero_query_gives_log_n_and_the_mean_row():
    inp = small(seed=13, seq_lens=(1, 2, 37, 100, 255))
    inp.q_bits[:] = 0
    o, lse = run(inp)
    for b, n in enumerate(inp.seq_lens):
        K = dense_keys(inp, b).numpy()
        mean = np.array([float(sum(_exact(K[:, j])) / int(n)) for j in range(512)])
        assert np.max(np.abs(lse[b] - math.log(int(n)))) < 1e-13
        assert np.max(np.abs(o[b] - mean[None, :])) < 1e-13


def test_equal_scores_from_equal_rope_keys():
    """q_nope = 0 and every k_pe equal: all scores are s = scale*q_pe.k_pe, so
    lse = s + ln n and o is the mean of kv_c."""
    inp = small(seed=17, seq_lens=(40, 77))
    inp.q_bits[:, :, :512] = 0
    P = inp.workload.page_size
    inp.kv_bits[:, :, 512:] = inp.kv_bits[0, 0, 512:]
    o, lse = run(inp)
    sc = Fraction(float(np.float32(inp.workload.scale)))
    kpe = _exact(dense_keys(inp, 0)[0, 512:].numpy())
    for b, n in enumerate(inp.seq_lens):
        K = dense_keys(inp, b).numpy()
        mean = np.array([float(sum(_exact(K[:, j])) / int(n)) for j in range(512)])
        for h in range(inp.workload.num_heads):
            qpe = _exact(q_of(inp, b)[h, 512:].numpy())
            s = float(sc * sum(a * c for a, c in zip(qpe, kpe)))
            assert abs(lse[b, h] - (s + math.log(int(n)))) < 1e-12
        assert np.max(np.abs(o[b] - mean[None, :])) < 1e-12


def test_empty_sequence_gives_zero_output_and_minus_inf():
    inp = small(seed=19, seq_lens=(0, 5))
    o, lse = run(inp)
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))
    assert np.all(np.isfinite(lse[1]))


def test_normalisation_and_convexity():
    inp = small(seed=23, seq_lens=(3, 64, 129))
    o, lse = run(inp)
    sc = float(np.float32(inp.workload.scale))
    for b in range(3):
        K = dense_keys(inp, b).numpy()
        q = q_of(inp, b).numpy()
        w = np.exp(q @ K.T * sc - lse[b][:, None])
        assert np.max(np.abs(w.sum(axis=1) - 1.0)) < 1e-12
        lo, hi = K[:, :512].min(axis=0), K[:, :512].max(axis=0)
        assert np.all(o[b] >= lo - 1e-12) and np.all(o[b] <= hi + 1e-12)


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("normalised", [False, True])
def test_split_merge_equals_single_pass(normalised):
    inp = small(seed=29, seq_lens=(37, 100, 1, 64, 300, 0))
    w = inp.workload
    full_o, full_l = run(inp)
    rng = np.random.default_rng(0)

    def uniform(b, n):            # one chunk length for the whole batch
        C = 32
        return [(s, min(s + C, n)) for s in range(0, max(n, 1), C)] if n else []

    def per_seq(b, n):            # S segments per sequence, some empty
        S = 4
        C = max(1, -(-n // S))
        return [(min(s * C, n), min((s + 1) * C, n)) for s in range(S)]

    def random_cuts(b, n):
        cuts = sorted(set(rng.integers(0, n + 1, size=5).tolist()) | {0, n})
        return list(zip(cuts[:-1], cuts[1:])) + [(n, n)]

    for rule in (uniform, per_seq, random_cuts):
        o, l = O.decode_split(inp.q_bits, inp.kv_bits, inp.block_table, inp.seq_lens,
                              scale=w.scale, k_scale=w.k_scale, kv_dtype=w.kv_dtype,
                              kv_lora_rank=w.kv_lora_rank, bounds_of=rule,
                              normalised=normalised)
        live = np.asarray(inp.seq_lens) > 0
        assert np.max(np.abs(o - full_o)) < 1e-12
        assert np.max(np.abs(l[live] - full_l[live])) < 1e-12
        assert np.all(np.isneginf(l[~live])) and np.all(o[~live] == 0)


def test_physical_page_permutation_is_bitwise_invariant():
    inp = small(seed=31, seq_lens=(37, 100, 64, 65))
    o, l = run(inp)
    o2, l2 = run(W.permute_pages(inp, seed=99))
    assert np.array_equal(o, o2) and np.array_equal(l, l2)


def test_poisoned_unreferenced_rows_are_never_read():
    inp = small(seed=37, seq_lens=(37, 100, 5))
    o, l = run(inp)
    pois = W.poison_unreferenced(inp)
    assert np.isnan(O.decode_kv(pois.kv_bits, "bf16", 1.0)).any()
    o2, l2 = run(pois)
    assert np.all(np.isfinite(o2)) and np.array_equal(o, o2) and np.array_equal(l, l2)


def test_k_scale_has_no_effect_on_bf16_cache():
    inp = small(seed=41, seq_lens=(37, 100))
    o, l = O.decode(inp.q_bits, inp.kv_bits, inp.block_table, inp.seq_lens,
                    scale=inp.workload.scale, k_scale=1.0, kv_dtype="bf16", kv_lora_rank=512)
    o2, l2 = O.decode(inp.q_bits, inp.kv_bits, inp.block_table, inp.seq_lens,
                      scale=inp.workload.scale, k_scale=0.05, kv_dtype="bf16",
                      kv_lora_rank=512)
    assert np.array_equal(o, o2) and np.array_equal(l, l2)


def test_head_size_320_variant_matches_sdpa():
    inp = small(seed=43, seq_lens=(20, 257), H=16, D=320, DV=256)
    o, lse = run(inp)
    sc = float(np.float32(inp.workload.scale))
    for b in range(2):
        K = dense_keys(inp, b)
        q = q_of(inp, b)
        ref = torch.nn.functional.scaled_dot_product_attention(
            q[:, None, :], K.expand(16, -1, -1), K[:, :256].expand(16, -1, -1), scale=sc)[:, 0]
        assert np.max(np.abs(o[b] - ref.numpy())) < 1e-12


def test_generator_is_deterministic():
    a = W.generate("tiny")
    b = W.generate("tiny")
    for x, y in ((a.q_bits, b.q_bits), (a.kv_bits, b.kv_bits),
                 (a.block_table, b.block_table), (a.seq_lens, b.seq_lens)):
        assert np.array_equal(x, y)
    # each sequence gets its own pages
    P = a.workload.page_size
    used = np.concatenate([a.block_table[i, :(int(n) + P - 1) // P]
                           for i, n in enumerate(a.seq_lens)])
    assert len(set(used.tolist())) == used.size


# ---------------------------------------------------------------- planted mistakes

def _pins_fail(monkeypatch, name, fake):
    """Plant ``fake`` as oracle function ``name`` and report whether any of a
    set of pins fails."""
    monkeypatch.setattr(OM, name, fake)
    pins = [test_matches_torch_sdpa_float64, test_one_token_sequence_returns_its_row_and_score,
            test_zero_query_gives_log_n_and_the_mean_row, test_paged_address_worked_example,
            test_fp8_cache_matches_torch_sdpa_with_k_scale, test_head_size_320_variant_matches_sdpa]
    failed = 0
    for p in pins:
        try:
            p()
        except AssertionError:
            failed += 1
    monkeypatch.undo()
    return failed


def test_planted_mistakes_are_caught(monkeypatch):
    real_attend = OM.attend
    real_slot = OM.physical_slot
    real_decode_kv = OM.decode_kv

    def log2_lse(q, K, d_v, scale):
        o, l = real_attend(q, K, d_v, scale)
        return o, l / math.log(2.0)

    def no_rope(q, K, d_v, scale):
        K2 = K.copy()
        K2[:, d_v:] = 0
        return real_attend(q, K2, d_v, scale)

    def v_from_wrong_columns(q, K, d_v, scale):
        o, l = real_attend(q, K, d_v, scale)
        o2, _ = real_attend(q, np.roll(K, -1, axis=1), d_v, scale)
        return o2, l

    def scale_squared(q, K, d_v, scale):
        return real_attend(q, K, d_v, scale * scale)

    def slot_off_by_one(row, pos, bs):
        return real_slot(row, pos, bs) + (1 if pos % bs == 0 else 0)

    def slot_transposed(row, pos, bs):
        return int(row[pos % bs if pos % bs < len(row) else 0]) * bs + pos // bs

    def k_scale_ignored(bits, dt, ks):
        return real_decode_kv(bits, dt, 1.0)

    for name, fake in (("attend", log2_lse), ("attend", no_rope),
                       ("attend", v_from_wrong_columns), ("attend", scale_squared),
                       ("physical_slot", slot_off_by_one), ("physical_slot", slot_transposed),
                       ("decode_kv", k_scale_ignored)):
        assert _pins_fail(monkeypatch, name, fake) > 0, (name, fake.__name__)


# ---------------------------------------------------------------- multi-token decode
# (lshu.cn article, section 10: q_len new positions verified at once; query i
# sees the whole context and new positions 0..i)

def mtp_case(seed, seq_lens, q_len, H=16, D=576, DV=512, P=16, kv="bf16", k_scale=1.0):
    return W.small_case(seed=seed, batch=len(seq_lens), num_heads=H, head_size=D,
                        kv_lora_rank=DV, page_size=P, seq_lens=seq_lens, kv_dtype=kv,
                        k_scale=k_scale, q_len=q_len)


def run_mtp(inp, **kw):
    w = inp.workload
    return O.decode_mtp(inp.q_bits, inp.kv_bits, inp.block_table, inp.seq_lens, scale=w.scale,
                        k_scale=w.k_scale, kv_dtype=w.kv_dtype, kv_lora_rank=w.kv_lora_rank,
                        **kw)


def test_visibility_matches_the_pages_worked_example():
    g = golden()["multi_token_verification"]
    n, ql, ctx = g["kv_length"], g["query_length"], g["history_tokens"]
    assert ctx == n - ql
    for i in range(ql):
        vis = O.visible_keys(n, ql, i)
        assert vis == g["visible_keys_per_query"][i]
        assert vis >= ctx  # the whole history is visible to every query
        for j in range(ql):
            assert (ctx + j < vis) == bool(g["new_position_visibility"][i][j])


@pytest.mark.parametrize("kv,D,DV,lens,ql", [
    ("bf16", 576, 512, (9, 40, 3), 3),
    ("bf16", 576, 512, (17, 64), 8),
    ("fp8_e4m3", 576, 512, (33, 8), 4),
    ("bf16", 320, 256, (21, 2, 50), 2),
])
def test_mtp_matches_causal_sdpa(kv, D, DV, lens, ql):
    """torch float64 SDPA with an explicit boolean mask key_t <= n - q_len + i."""
    inp = mtp_case(seed=41, seq_lens=lens, q_len=ql, D=D, DV=DV, kv=kv,
                   k_scale=float(np.float32(0.05)) if kv != "bf16" else 1.0)
    o, lse = run_mtp(inp)
    sc = float(np.float32(inp.workload.scale))
    H = inp.workload.num_heads
    for b, n in enumerate(lens):
        K = dense_keys(inp, b)
        q = q_of(inp, b).reshape(ql * H, D)  # row = token * H + head
        tok = torch.arange(ql * H) // H
        mask = torch.arange(n)[None, :] <= (n - ql + tok)[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            q[None], K[None], K[None, :, :DV], attn_mask=mask[None], scale=sc)[0]
        s = (q @ K.T) * sc
        ref_lse = torch.logsumexp(s.masked_fill(~mask, -math.inf), dim=1)
        assert np.abs(o[b].reshape(ql * H, DV) - ref.numpy()).max() < 1e-12
        assert np.abs(lse[b].reshape(ql * H) - ref_lse.numpy()).max() < 1e-12


def test_mtp_with_one_token_is_plain_decode():
    flat = mtp_case(seed=42, seq_lens=(37, 100, 1), q_len=1)  # q [B, H, D]
    o0, l0 = run(flat)
    inp = W.DecodeInputs(workload=flat.workload, q_bits=flat.q_bits[:, None].copy(),
                         kv_bits=flat.kv_bits, block_table=flat.block_table,
                         seq_lens=flat.seq_lens)  # the same query as [B, 1, H, D]
    o1, l1 = run_mtp(inp)
    assert np.array_equal(o1[:, 0], o0) and np.array_equal(l1[:, 0], l0)


def test_mtp_rows_reduce_to_single_token_decode_at_the_visible_length():
    lens, ql = (12, 70), 5
    inp = mtp_case(seed=43, seq_lens=lens, q_len=ql)
    o, lse = run_mtp(inp)
    for i in range(ql):
        vis = [O.visible_keys(n, ql, i) for n in lens]
        one = W.DecodeInputs(workload=inp.workload, q_bits=inp.q_bits[:, i].copy(),
                             kv_bits=inp.kv_bits, block_table=inp.block_table,
                             seq_lens=np.asarray(vis, dtype=np.int32))
        oi, li = run(one)
        assert np.array_equal(o[:, i], oi) and np.array_equal(lse[:, i], li)


def test_mtp_identical_keys_closed_form():
    """Every key equal: each query's weights are uniform over its visible keys,
    so o is that row and lse = s + ln(visible)."""
    lens, ql = (11,), 4
    inp = mtp_case(seed=44, seq_lens=lens, q_len=ql)
    P = inp.workload.page_size
    kv = inp.kv_bits.copy()
    row = kv[inp.block_table[0, 0], 0].copy()
    kv[:] = row
    inp = W.DecodeInputs(workload=inp.workload, q_bits=inp.q_bits, kv_bits=kv,
                         block_table=inp.block_table, seq_lens=inp.seq_lens)
    o, lse = run_mtp(inp)
    v = O.bf16_bits_to_f64(row)
    sc = float(np.float32(inp.workload.scale))
    for i in range(ql):
        s = (O.bf16_bits_to_f64(inp.q_bits[0, i]) @ v) * sc
        assert np.abs(o[0, i] - v[None, :512]).max() < 1e-12
        assert np.abs(lse[0, i] - (s + math.log(11 - ql + i + 1))).max() < 1e-12


def test_mtp_rows_that_see_no_key():
    """seq_len < q_len: the first q_len - n queries see nothing (o = 0,
    lse = -inf, the empty sum); the others see 1..n keys."""
    inp = mtp_case(seed=45, seq_lens=(2,), q_len=5)
    o, lse = run_mtp(inp)
    assert [O.visible_keys(2, 5, i) for i in range(5)] == [0, 0, 0, 1, 2]
    assert np.all(o[0, :3] == 0) and np.all(np.isneginf(lse[0, :3]))
    assert np.all(np.isfinite(lse[0, 3:]))


def test_planted_visibility_mistakes_are_caught(monkeypatch):
    """An off-by-one or a mirrored triangle in the causal rule of section 10
    makes the SDPA-with-mask pin fail."""
    def excludes_own_position(n, q_len, i):
        return max(0, min(n, n - q_len + i))

    def mirrored(n, q_len, i):
        return max(0, min(n, n - i))

    def no_mask(n, q_len, i):
        return n

    for fake in (excludes_own_position, mirrored, no_mask):
        monkeypatch.setattr(OM, "visible_keys", fake)
        with pytest.raises(AssertionError):
            test_mtp_matches_causal_sdpa("bf16", 576, 512, (9, 40, 3), 3)
        monkeypatch.undo()


# ---------------------------------------------------------------- sparse decode
# (lshu.cn article, section 13: each query attends only to its selected
# positions, still reached through the request's own block table)

def sparse_case(seed, seq_lens, topk, H=16, P=16):
    return W.small_case(seed=seed, batch=len(seq_lens), num_heads=H, head_size=576,
                        kv_lora_rank=512, page_size=P, seq_lens=seq_lens, topk=topk)


def run_sparse(inp, idx=None, lens=None):
    w = inp.workload
    return O.decode_sparse(inp.q_bits, inp.kv_bits, inp.block_table,
                           inp.topk_indices if idx is None else idx,
                           inp.topk_lens if lens is None else lens, scale=w.scale,
                           k_scale=w.k_scale, kv_dtype=w.kv_dtype, kv_lora_rank=w.kv_lora_rank)


def test_sparse_matches_sdpa_over_the_selected_keys_at_the_pages_size():
    """The page's example size (k = 2048 keys of dimension 576): torch float64
    SDPA over the selected rows, gathered with numpy fancy indexing."""
    g = golden()["sparse_topk"]
    inp = sparse_case(seed=51, seq_lens=(4096, 2100), topk=g["topk"])
    assert inp.q_bits.shape[-1] == g["query_dim"]
    o, lse = run_sparse(inp)
    sc = float(np.float32(inp.workload.scale))
    for b in range(2):
        K = dense_keys(inp, b)[torch.from_numpy(inp.topk_indices[b, :inp.topk_lens[b]].astype(
            np.int64))]
        assert K.shape[0] == g["score_shape"][1]
        q = q_of(inp, b)
        ref = torch.nn.functional.scaled_dot_product_attention(q[None], K[None],
                                                               K[None, :, :512], scale=sc)[0]
        ref_lse = torch.logsumexp((q @ K.T) * sc, dim=1)
        assert np.abs(o[b] - ref.numpy()).max() < 1e-12
        assert np.abs(lse[b] - ref_lse.numpy()).max() < 1e-12


def test_sparse_over_every_position_in_order_is_dense_decode():
    lens = (37, 100, 1)
    inp = sparse_case(seed=52, seq_lens=lens, topk=128)
    idx = np.zeros((3, 128), np.int32)
    for b, n in enumerate(lens):
        idx[b, :n] = np.arange(n)
    o, lse = run_sparse(inp, idx, np.asarray(lens, np.int32))
    od, ld = run(inp)
    assert np.array_equal(o, od) and np.array_equal(lse, ld)


def test_sparse_is_order_invariant_and_counts_duplicates_twice():
    inp = sparse_case(seed=53, seq_lens=(300,), topk=64)
    o, lse = run_sparse(inp)
    rng = np.random.default_rng(0)
    shuf = inp.topk_indices.copy()
    shuf[0] = rng.permutation(shuf[0])
    o2, l2 = run_sparse(inp, shuf)
    assert np.abs(o - o2).max() < 1e-12 and np.abs(lse - l2).max() < 1e-12
    # one position listed twice: exactly a key set in which that row appears twice
    dup = inp.topk_indices.copy()
    dup[0, 1] = dup[0, 0]
    o3, l3 = run_sparse(inp, dup)
    K = dense_keys(inp, 0)[torch.from_numpy(dup[0].astype(np.int64))]
    q = q_of(inp, 0)
    sc = float(np.float32(inp.workload.scale))
    ref = torch.nn.functional.scaled_dot_product_attention(q[None], K[None], K[None, :, :512],
                                                           scale=sc)[0]
    assert np.abs(o3[0] - ref.numpy()).max() < 1e-12


def test_sparse_empty_list_is_the_empty_sum():
    inp = sparse_case(seed=54, seq_lens=(50, 20), topk=8)
    o, lse = run_sparse(inp, lens=np.asarray([0, 8], np.int32))
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0])) and np.all(np.isfinite(lse[1]))


def test_planted_sparse_mistakes_are_caught(monkeypatch):
    """Reading the listed positions as physical slots (skipping the block
    table), or attending to the first k positions instead of the listed ones,
    fails the SDPA pin."""
    real = OM.decode_sparse

    def no_table(q_bits, kv_bits, block_table, topk_indices, topk_lens, **kw):
        ident = np.tile(np.arange(block_table.shape[1], dtype=np.int32), (block_table.shape[0], 1))
        return real(q_bits, kv_bits, ident, topk_indices, topk_lens, **kw)

    def first_k(q_bits, kv_bits, block_table, topk_indices, topk_lens, **kw):
        firsts = np.tile(np.arange(topk_indices.shape[1], dtype=np.int32),
                         (topk_indices.shape[0], 1))
        return real(q_bits, kv_bits, block_table, firsts, topk_lens, **kw)

    for fake in (no_table, first_k):
        monkeypatch.setattr(O, "decode_sparse", fake)
        with pytest.raises(AssertionError):
            test_sparse_matches_sdpa_over_the_selected_keys_at_the_pages_size()
        monkeypatch.undo()


# ---------------------------------------------------------------- per-token quantised cache
# (Triton MLA page, key files: per-token-head modes pad head_dim to hold an
# inline scale; rows here are [e4m3fn codes (D) | fp32 scale | 12 pad bytes])

def pt_case(seed, seq_lens, H=16, D=576, P=16):
    return W.small_case(seed=seed, batch=len(seq_lens), num_heads=H, head_size=D,
                        kv_lora_rank=D - 64, page_size=P, seq_lens=seq_lens,
                        kv_dtype=W.FP8_PER_TOKEN)


def test_per_token_rows_decode_like_torch_times_their_scale():
    inp = pt_case(seed=61, seq_lens=(40, 7))
    rows = inp.kv_bits.reshape(-1, inp.kv_bits.shape[-1])
    mine = O.decode_kv(rows, "fp8_per_token", 1.0)
    D = inp.workload.head_size
    codes = torch.from_numpy(rows[:, :D].copy()).view(torch.float8_e4m3fn).to(torch.float64)
    scale = torch.from_numpy(rows[:, D:D + 4].copy()).view(torch.float32).to(torch.float64)
    assert np.array_equal(mine, (codes * scale).numpy())
    assert rows.shape[-1] == O.row_width("fp8_per_token", D) == D + 16


def test_per_token_row_maximum_round_trips():
    """The largest element of each token's row is quantised to +-448 exactly,
    so it decodes to the row's max|x| (to the fp32 rounding of the scale)."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((64, 576), dtype=np.float32) * rng.uniform(0.01, 100, (64, 1)).astype(
        np.float32)
    rows = W.per_token_fp8_rows(x)
    dec = O.decode_kv(rows, "fp8_per_token", 1.0)
    amax = np.abs(x).max(axis=1).astype(np.float64)
    got = np.abs(dec).max(axis=1)
    assert np.all(np.abs(got - amax) <= amax * 2.0 ** -22)
    assert np.all(np.abs(dec - x) <= amax[:, None] * 2.0 ** -4)  # e4m3: 3 mantissa bits


@pytest.mark.parametrize("D", [576, 320])
def test_per_token_cache_matches_torch_sdpa(D):
    inp = pt_case(seed=62, seq_lens=(37, 100, 1), D=D)
    w = inp.workload
    o, lse = run(inp)
    sc = float(np.float32(w.scale))
    for b in range(3):
        K = dense_keys(inp, b)
        q = q_of(inp, b)
        ref = torch.nn.functional.scaled_dot_product_attention(q[None], K[None],
                                                               K[None, :, :D - 64], scale=sc)[0]
        ref_lse = torch.logsumexp((q @ K.T) * sc, dim=1)
        assert np.abs(o[b] - ref.numpy()).max() < 1e-12
        assert np.abs(lse[b] - ref_lse.numpy()).max() < 1e-12


def test_per_token_cache_ignores_k_scale():
    inp = pt_case(seed=63, seq_lens=(20, 64))
    a = run(inp)
    w = dataclasses.replace(inp.workload, k_scale=0.05)
    b = run(dataclasses.replace(inp, workload=w))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_planted_per_token_mistakes_are_caught(monkeypatch):
    """Dropping the per-token scale, or reading it from the wrong bytes, fails
    the SDPA pin."""
    real = OM.decode_kv

    def scale_dropped(bits, dt, ks):
        if dt != "fp8_per_token":
            return real(bits, dt, ks)
        D = bits.shape[-1] - 16
        return O.e4m3fn_bits_to_f64(np.asarray(bits)[..., :D])

    def scale_misread(bits, dt, ks):
        if dt != "fp8_per_token":
            return real(bits, dt, ks)
        b2 = np.array(bits, copy=True)
        D = b2.shape[-1] - 16
        b2[..., D:D + 4] = b2[..., D - 4:D]  # the last four codes taken as the scale
        return real(b2, dt, ks)

    for fake in (scale_dropped, scale_misread):
        monkeypatch.setattr(OM, "decode_kv", fake)
        with pytest.raises(AssertionError):
            test_per_token_cache_matches_torch_sdpa(576)
        monkeypatch.undo()


# ---------------------------------------------------------------- per-token int8 cache
# (the same pages list int8 among the per-token-head modes; rows here are
# [signed int8 codes (D) | fp32 scale | 12 pad bytes], value = code * scale)

def test_int8_rows_decode_like_torch_times_their_scale():
    inp = W.small_case(seed=71, batch=2, num_heads=16, head_size=576, kv_lora_rank=512,
                       page_size=16, seq_lens=(40, 7), kv_dtype=W.INT8_PER_TOKEN)
    rows = inp.kv_bits.reshape(-1, inp.kv_bits.shape[-1])
    D = 576
    mine = O.decode_kv(rows, "int8_per_token", 1.0)
    codes = torch.from_numpy(rows[:, :D].copy()).view(torch.int8).to(torch.float64)
    scale = torch.from_numpy(rows[:, D:D + 4].copy()).view(torch.float32).to(torch.float64)
    assert np.array_equal(mine, (codes * scale).numpy())
    assert O.row_width("int8_per_token", D) == D + 16


def test_int8_every_code_decodes_to_itself():
    """All 256 byte values with scale 1 give -128..127 (two's complement):
    a reading of the bytes as unsigned, or as sign-magnitude, fails."""
    rows = np.zeros((1, 256 + 16), dtype=np.uint8)
    rows[0, :256] = np.arange(256, dtype=np.uint8)
    rows[0, 256:260] = np.array([1.0], dtype="<f4").view(np.uint8)
    got = O.decode_kv(rows, "int8_per_token", 1.0)[0]
    want = np.array([b if b < 128 else b - 256 for b in range(256)], dtype=np.float64)
    assert np.array_equal(got, want)


def test_int8_quantisation_round_trips_within_half_a_step():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((64, 320), dtype=np.float32) * rng.uniform(0.01, 100, (64, 1)).astype(
        np.float32)
    rows = W.per_token_int8_rows(x)
    dec = O.decode_kv(rows, "int8_per_token", 1.0)
    amax = np.abs(x).max(axis=1).astype(np.float64)
    step = amax / 127.0
    assert np.all(np.abs(np.abs(dec).max(axis=1) - amax) <= amax * 2.0 ** -22)
    assert np.all(np.abs(dec - x) <= step[:, None] * (0.5 + 2.0 ** -20))


@pytest.mark.parametrize("D", [576, 320])
def test_int8_cache_matches_torch_sdpa(D):
    inp = W.small_case(seed=72, batch=3, num_heads=16, head_size=D, kv_lora_rank=D - 64,
                       page_size=16, seq_lens=(37, 100, 1), kv_dtype=W.INT8_PER_TOKEN)
    w = inp.workload
    o, lse = run(inp)
    sc = float(np.float32(w.scale))
    for b in range(3):
        K = dense_keys(inp, b)
        q = q_of(inp, b)
        ref = torch.nn.functional.scaled_dot_product_attention(q[None], K[None],
                                                               K[None, :, :D - 64], scale=sc)[0]
        ref_lse = torch.logsumexp((q @ K.T) * sc, dim=1)
        assert np.abs(o[b] - ref.numpy()).max() < 1e-12
        assert np.abs(lse[b] - ref_lse.numpy()).max() < 1e-12


def test_planted_int8_mistakes_are_caught(monkeypatch):
    """Reading the int8 codes as unsigned bytes, or as fp8 codes, fails the
    SDPA pin."""
    real = OM.decode_kv

    def unsigned(bits, dt, ks):
        if dt != "int8_per_token":
            return real(bits, dt, ks)
        b = np.asarray(bits)
        D = b.shape[-1] - 16
        scale = b[..., D:D + 4].copy().view("<f4")[..., 0].astype(np.float64)
        return b[..., :D].astype(np.float64) * scale[..., None]

    def as_fp8(bits, dt, ks):
        return real(bits, "fp8_per_token" if dt == "int8_per_token" else dt, ks)

    for fake in (unsigned, as_fp8):
        monkeypatch.setattr(OM, "decode_kv", fake)
        with pytest.raises(AssertionError):
            test_int8_cache_matches_torch_sdpa(576)
        monkeypatch.undo()


# ---------------------------------------------------------------- cross-shard (DCP) merge
# (Triton MLA page, design motivation: decode always returns lse because the
# shards of a context-parallel decode are merged through it; AttentionBackend
# page, limits: reading an lse in the wrong base corrupts that merge)

def shard_results(inp, G):
    """Oracle decode of each round-robin page shard of the batch."""
    outs = [run(W.shard_pages(inp, G, r)) for r in range(G)]
    return np.stack([o for o, _ in outs]), np.stack([l for _, l in outs])


@pytest.mark.parametrize("G", [2, 3, 4, 8])
def test_shard_merge_equals_unsharded_decode(G):
    """Every key lies in exactly one shard, so merging the shards' (o, lse)
    must give the single-pass decode of the whole batch (to rounding)."""
    inp = small(seed=81, seq_lens=(1, 15, 16, 17, 100, 257), P=16)
    o_p, l_p = shard_results(inp, G)
    o, lse = O.merge_shards(o_p, l_p)
    ro, rl = run(inp)
    assert np.abs(o - ro).max() < 1e-12 and np.abs(lse - rl).max() < 1e-12


def test_shard_pages_cover_every_position_once():
    inp = small(seed=82, seq_lens=(1, 16, 33, 100), P=16)
    for G in (2, 3, 5):
        seen = {b: [] for b in range(4)}
        for r in range(G):
            sh = W.shard_pages(inp, G, r)
            for b in range(4):
                n = int(sh.seq_lens[b])
                pos_pages = [int(sh.block_table[b, t // 16]) * 16 + t % 16 for t in range(n)]
                seen[b] += pos_pages
        for b in range(4):
            n = int(inp.seq_lens[b])
            full = [int(inp.block_table[b, t // 16]) * 16 + t % 16 for t in range(n)]
            assert sorted(seen[b]) == sorted(full)


def test_shard_merge_log2_base_and_empty_shards():
    """A sequence shorter than a page lives in shard 0 only: the other shards
    carry lse = -inf and must get weight 0.  The same lse given in base 2
    merges to the same result when declared as such, and to a wrong one when
    declared as natural log."""
    inp = small(seed=83, seq_lens=(5, 40, 16), P=16)
    o_p, l_p = shard_results(inp, 4)
    assert np.all(np.isneginf(l_p[1:, 0]))  # sequence 0: one page, shard 0 only
    ro, rl = run(inp)
    o, lse = O.merge_shards(o_p, l_p / math.log(2.0), lse_base="log2")
    assert np.abs(o - ro).max() < 1e-12 and np.abs(lse - rl).max() < 1e-12
    o_bad, _ = O.merge_shards(o_p, l_p / math.log(2.0), lse_base="ln")
    assert np.abs(o_bad - ro).max() > 1e-3
    # no shard saw anything: o = 0, lse = -inf
    o0, l0 = O.merge_shards(np.ones((3, 2, 4)), np.full((3, 2), -np.inf))
    assert np.all(o0 == 0) and np.all(np.isneginf(l0))


def test_shard_merge_closed_form():
    """Two shards with lse a and b: weights e^a / (e^a + e^b) exactly."""
    o_p = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])
    l_p = np.array([[math.log(3.0)], [math.log(1.0)]])
    o, lse = O.merge_shards(o_p, l_p)
    assert np.allclose(o[0], [0.75, 0.25], atol=1e-15, rtol=0)
    assert abs(lse[0] - math.log(4.0)) < 1e-15


# ---------------------------------------------------------------- per-token int4 cache
# (the same pages list int4 among the per-token-head modes; rows here are
# [two signed 4-bit codes per byte, element 2i low nibble (D/2 bytes) |
#  fp32 scale | 12 pad bytes], value = code * scale)

def test_int4_every_byte_decodes_to_its_two_nibbles():
    rows = np.zeros((1, 256 + 16), dtype=np.uint8)
    rows[0, :256] = np.arange(256, dtype=np.uint8)
    rows[0, 256:260] = np.array([1.0], dtype="<f4").view(np.uint8)
    got = O.decode_kv(rows, "int4_per_token", 1.0)[0]
    signed = lambda v: v - 16 if v >= 8 else v
    want = np.array([f(b) for b in range(256) for f in (lambda b: signed(b & 15),
                                                        lambda b: signed(b >> 4))],
                    dtype=np.float64)
    assert np.array_equal(got, want)
    assert O.row_width("int4_per_token", 576) == 288 + 16


def test_int4_quantisation_round_trips_within_half_a_step():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((64, 320), dtype=np.float32) * rng.uniform(0.01, 100, (64, 1)).astype(
        np.float32)
    rows = W.per_token_int4_rows(x)
    assert rows.shape == (64, 160 + 16)
    dec = O.decode_kv(rows, "int4_per_token", 1.0)
    amax = np.abs(x).max(axis=1).astype(np.float64)
    step = amax / 7.0
    assert np.all(np.abs(np.abs(dec).max(axis=1) - amax) <= amax * 2.0 ** -22)
    assert np.all(np.abs(dec - x) <= step[:, None] * (0.5 + 2.0 ** -20))


@pytest.mark.parametrize("D", [576, 320])
def test_int4_cache_matches_torch_sdpa(D):
    inp = W.small_case(seed=73, batch=3, num_heads=16, head_size=D, kv_lora_rank=D - 64,
                       page_size=16, seq_lens=(37, 100, 1), kv_dtype=W.INT4_PER_TOKEN)
    w = inp.workload
    o, lse = run(inp)
    sc = float(np.float32(w.scale))
    for b in range(3):
        K = dense_keys(inp, b)
        q = q_of(inp, b)
        ref = torch.nn.functional.scaled_dot_product_attention(q[None], K[None],
                                                               K[None, :, :D - 64], scale=sc)[0]
        ref_lse = torch.logsumexp((q @ K.T) * sc, dim=1)
        assert np.abs(o[b] - ref.numpy()).max() < 1e-12
        assert np.abs(lse[b] - ref_lse.numpy()).max() < 1e-12


def test_planted_int4_mistakes_are_caught(monkeypatch):
    """Swapping the nibble order, or reading the nibbles unsigned, fails the
    SDPA pin."""
    real = OM.int4_bits_to_f64

    def swapped(packed):
        v = real(packed)
        out = v.copy()
        out[..., 0::2], out[..., 1::2] = v[..., 1::2], v[..., 0::2]
        return out

    def unsigned(packed):
        b = np.asarray(packed, dtype=np.uint8)
        out = np.empty(b.shape[:-1] + (2 * b.shape[-1],))
        out[..., 0::2] = b & 15
        out[..., 1::2] = b >> 4
        return out

    for fake in (swapped, unsigned):
        monkeypatch.setattr(OM, "int4_bits_to_f64", fake)
        with pytest.raises(AssertionError):
            test_int4_cache_matches_torch_sdpa(576)
        monkeypatch.undo()
