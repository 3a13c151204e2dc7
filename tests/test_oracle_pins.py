"""Pins of the float64 oracle against facts that do not come from the oracle.

Each test checks the oracle against something fixed by the pages or by
mathematics: a worked example the pages print, a closed form, a library
routine (torch's float64 SDPA, torch's bf16/fp8 decoders), exact rational
arithmetic, or a brute-force loop.  The last group plants mistakes in the
oracle and checks that at least one pin catches each of them.
"""
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
    flat = inp.kv_bits.reshape(-1, w.head_size)[rows]
    if w.kv_dtype == "bf16":
        t = torch.from_numpy(flat.view(np.int16).copy()).view(torch.bfloat16)
        return t.to(torch.float64)
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
