"""Pins that tie the CPU oracle to something other than itself (CPU only).

Each test names what fixes the expected value: an independent brute force
(multiset of pool rows in 50-digit arithmetic), a closed form, an invariant
of the definition, or torch's float64 scaled_dot_product_attention.  They are
chosen so that a dropped term, a wrong sign or index, or a transposed operand
anywhere in the oracle fails one of them.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle.formats import decode_bits

D = 512
LOG2E = 1.0 / math.log(2.0)


# ---------------------------------------------------------------------------
# tiny input builders (stored bit patterns, like the real inputs)
# ---------------------------------------------------------------------------

def bf16_bits(x):
    t = torch.as_tensor(np.asarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def fp8_bits(x):
    t = torch.as_tensor(np.asarray(x, np.float32)).clamp(-448, 448)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def tiny_case(seed, T=3, H=3, K=150, swa_rows=40, comp_rows=60, dtype="bf16",
              neg=6, dup=True, sinks=True, lens="random", qscale=0.15):
    rng = np.random.default_rng(seed)
    enc = bf16_bits if dtype == "bf16" else fp8_bits
    kscale = 1.0 if dtype == "bf16" else 1 / 0.08
    q = enc(rng.standard_normal((T, H, D)) * qscale * (1 if dtype == "bf16" else 8))
    swa = enc(rng.standard_normal((swa_rows, D)) * kscale)
    comp = enc(rng.standard_normal((comp_rows, D)) * kscale)
    idx = np.empty((T, K), np.int32)
    for t in range(T):
        idx[t, :128] = rng.integers(0, swa_rows, 128)
        idx[t, 128:] = rng.integers(0, comp_rows, K - 128)
        if not dup:
            idx[t, :128] = rng.permutation(swa_rows)[:128] if swa_rows >= 128 \
                else idx[t, :128]
        idx[t, rng.choice(K, neg, replace=False)] = -1
    if lens == "random":
        topk = rng.integers(0, K + 1, T).astype(np.int32)
        topk[0] = K
    elif lens is None:
        topk = None
    else:
        topk = np.asarray(lens, np.int32)
    sk = rng.standard_normal(H).astype(np.float32) if sinks else None
    return dict(q_bits=q, q_dtype=dtype, swa_bits=swa, comp_bits=comp,
                kv_dtype=dtype, indices=idx, topk_lens=topk, sinks=sk)


def run(case, b1=0.07, b2=1.0, g=1.0, **kw):
    return oracle.sparse_mla_decode(bmm1_scale=b1, bmm2_scale=b2, lse_scale=g,
                                    **case, **kw)


# ---------------------------------------------------------------------------
# P1: independent brute force (multiset, mpmath)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed,dtype,sinks,lens", [
    (0, "bf16", True, "random"), (1, "bf16", False, "random"),
    (2, "fp8_e4m3fn", True, "random"), (3, "bf16", True, None),
    (4, "bf16", True, [0, 127, 128]), (5, "bf16", False, [129, 150, 1]),
])
def test_p1_brute_force_multiset(seed, dtype, sinks, lens):
    case = tiny_case(seed, dtype=dtype, sinks=sinks, lens=lens)
    b1, b2, g = 0.0625, 0.75, 1.5
    ref = run(case, b1, b2, g)
    out, lse = oracle.brute_force_decode(
        case["q_bits"], dtype, case["swa_bits"], case["comp_bits"], dtype,
        case["indices"], case["topk_lens"], case["sinks"], b1, b2, g)
    fin = np.isfinite(lse)
    assert np.array_equal(fin, np.isfinite(ref["lse"]))
    np.testing.assert_allclose(ref["lse"][fin], lse[fin], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ref["out"], out, rtol=1e-11, atol=1e-13)


# ---------------------------------------------------------------------------
# P2-P4: closed forms
# ---------------------------------------------------------------------------

def single_slot_case(col, sink=None, H=2):
    rng = np.random.default_rng(7)
    q = bf16_bits(rng.standard_normal((1, H, D)) * 0.05)
    swa = bf16_bits(rng.standard_normal((4, D)))
    comp = bf16_bits(rng.standard_normal((4, D)))
    idx = np.full((1, 200), -1, np.int32)
    idx[0, col] = 3
    sk = None if sink is None else np.full(H, sink, np.float32)
    return dict(q_bits=q, q_dtype="bf16", swa_bits=swa, comp_bits=comp,
                kv_dtype="bf16", indices=idx, topk_lens=None, sinks=sk)


@pytest.mark.parametrize("col", [0, 127, 128, 199])
def test_p2_single_slot_returns_the_row(col):
    case = single_slot_case(col)
    pool = case["swa_bits"] if col < 128 else case["comp_bits"]
    row = decode_bits(pool[3], "bf16")
    b1, b2, g = 0.09, 0.5, 2.0
    r = run(case, b1, b2, g)
    q = decode_bits(case["q_bits"][0], "bf16")
    s = float(np.float32(b1)) * (q @ row)
    assert np.array_equal(r["out"][0], np.tile(b2 * row, (2, 1)))
    np.testing.assert_allclose(r["lse"][0], g * s * LOG2E, rtol=1e-15)
    assert r["n_active"][0] == 1


def test_p3_equal_logits_mean_of_rows():
    case = tiny_case(11, sinks=False, lens=None)
    case["q_bits"][:] = 0                       # every logit is 0
    r = run(case, 0.3, 1.25, 0.5)
    for t in range(case["indices"].shape[0]):
        slots = oracle.active_slots(case["indices"][t], None)
        rows = np.stack([decode_bits((case["swa_bits"] if p == 0 else
                                      case["comp_bits"])[i], "bf16")
                         for _, p, i in slots])
        mean = rows.sum(0) / len(slots)
        np.testing.assert_allclose(r["out"][t], np.tile(1.25 * mean, (3, 1)),
                                   rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(r["lse"][t], 0.5 * math.log2(len(slots)),
                                   rtol=1e-15)


def test_p3_equal_logits_with_sink():
    case = tiny_case(12, sinks=True, lens=None)
    case["q_bits"][:] = 0
    r = run(case, 0.3, 1.0, 1.0)
    nosink = run(dict(case, sinks=None), 0.3, 1.0, 1.0)
    for t in range(case["indices"].shape[0]):
        n = r["n_active"][t]
        for h in range(3):
            es = math.exp(float(case["sinks"][h]))
            np.testing.assert_allclose(
                r["out"][t, h], nosink["out"][t, h] * n / (n + es), rtol=1e-13,
                atol=1e-15)
            np.testing.assert_allclose(r["lse"][t, h], math.log2(n + es),
                                       rtol=1e-14)


@pytest.mark.parametrize("col,sink", [(5, 0.7), (150, -1.3), (0, 3.0)])
def test_p4_sink_and_single_slot_is_logistic(col, sink):
    case = single_slot_case(col, sink=sink)
    pool = case["swa_bits"] if col < 128 else case["comp_bits"]
    row = decode_bits(pool[3], "bf16")
    b1, b2, g = 0.2, 1.0, 1.0
    q = decode_bits(case["q_bits"][0], "bf16")
    s = float(np.float32(b1)) * (q @ row)
    r = run(case, b1, b2, g)
    sink = float(np.float32(sink))          # sinks are fp32 on the pages
    sig = 1.0 / (1.0 + np.exp(-(s - sink)))
    np.testing.assert_allclose(r["out"][0], sig[:, None] * row[None, :],
                               rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(r["lse"][0],
                               np.log2(np.exp(s) + math.exp(sink)), rtol=1e-14)


def test_closed_form_two_one_hot_rows():
    # q = e_0, rows 2*e_0 and 2*e_1, beta1 = 1: logits 2 and 0
    q = np.zeros((1, 1, D)); q[0, 0, 0] = 1.0
    swa = np.zeros((2, D)); swa[0, 0] = 2.0; swa[1, 1] = 2.0
    case = dict(q_bits=bf16_bits(q), q_dtype="bf16", swa_bits=bf16_bits(swa),
                comp_bits=bf16_bits(swa), kv_dtype="bf16",
                indices=np.array([[0, 1]], np.int32), topk_lens=None, sinks=None)
    r = run(case, 1.0, 1.0, 1.0)
    e2 = math.exp(2.0)
    assert r["out"][0, 0, 0] == pytest.approx(2 * e2 / (e2 + 1), rel=1e-15)
    assert r["out"][0, 0, 1] == pytest.approx(2 / (e2 + 1), rel=1e-15)
    assert not np.any(r["out"][0, 0, 2:])
    assert r["lse"][0, 0] == pytest.approx(math.log2(e2 + 1), rel=1e-15)


# ---------------------------------------------------------------------------
# P5, P6: -1 is removal; permutation invariance
# ---------------------------------------------------------------------------

def test_p5_minus_one_equals_removal_compressed_segment():
    case = tiny_case(21, lens=None, neg=0)
    base = run(case)
    masked = dict(case, indices=case["indices"].copy())
    masked["indices"][:, 140] = -1
    removed = dict(case, indices=np.concatenate(
        [case["indices"][:, :140], case["indices"][:, 141:],
         np.full((3, 1), 7, np.int32)], axis=1),
        topk_lens=np.full(3, 149, np.int32))
    a, b = run(masked), run(removed)
    np.testing.assert_allclose(a["out"], b["out"], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(a["lse"], b["lse"], rtol=1e-13)
    assert not np.allclose(a["out"], base["out"])


def test_p5_minus_one_in_swa_segment_matches_multiset_without_slot():
    case = tiny_case(22, T=1, lens=None, neg=0)
    masked = dict(case, indices=case["indices"].copy())
    masked["indices"][0, 17] = -1
    out, lse = oracle.brute_force_decode(
        case["q_bits"], "bf16", case["swa_bits"], case["comp_bits"], "bf16",
        masked["indices"], None, case["sinks"], 0.07, 1.0, 1.0)
    r = run(masked)
    np.testing.assert_allclose(r["out"], out, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(r["lse"], lse, rtol=1e-12)
    assert r["n_active"][0] == case["indices"].shape[1] - 1


def test_p6_permutation_invariance():
    case = tiny_case(31, lens=[150, 150, 150], neg=9)
    rng = np.random.default_rng(5)
    idx = case["indices"].copy()
    for t in range(idx.shape[0]):
        idx[t, :128] = idx[t, rng.permutation(128)]
        idx[t, 128:] = idx[t, 128 + rng.permutation(idx.shape[1] - 128)]
    a, b = run(case), run(dict(case, indices=idx))
    np.testing.assert_allclose(a["out"], b["out"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(a["lse"], b["lse"], rtol=1e-13)


def test_swa_boundary_is_column_127_128():
    # the same row number read through column 127 (SWA pool) and through
    # column 128 (compressed pool); a single slot with no sink returns it
    case = tiny_case(33, T=1, lens=None, neg=0, sinks=False)
    for col, pool in [(127, case["swa_bits"]), (128, case["comp_bits"])]:
        idx = np.full((1, 129), -1, np.int32)
        idx[0, col] = 5
        r = run(dict(case, indices=idx))
        want = decode_bits(pool[5], "bf16")
        assert np.array_equal(r["out"][0], np.tile(want, (3, 1)))
    assert not np.array_equal(case["swa_bits"][5], case["comp_bits"][5])


# ---------------------------------------------------------------------------
# P7: split form + combine equals the unsplit result
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("S,chunk", [(1, 64), (2, 64), (3, 32), (5, 16),
                                     (16, 8), (7, 64)])
@pytest.mark.parametrize("sinks", [True, False])
def test_p7_split_combine_equals_unsplit(S, chunk, sinks):
    case = tiny_case(41 + S, K=180, lens=[180, 40, 0], sinks=sinks)
    b1, b2, g = 0.05, 0.8, 0.7
    ref = run(case, b1, b2, g)
    K = case["indices"].shape[1]
    ranges = oracle.split_columns(K, S, chunk)
    assert ranges[0][0] == 0 and ranges[-1][1] <= K
    assert all(a[1] == b[0] for a, b in zip(ranges, ranges[1:]))
    for t in range(3):
        slots = oracle.active_slots(case["indices"][t], case["topk_lens"][t])
        rows = oracle.sparse_mla.gather_rows(slots, case["swa_bits"],
                                             case["comp_bits"], "bf16")
        q_t = decode_bits(case["q_bits"][t], "bf16")
        mo, ml = oracle.split_partials(q_t, slots, rows, ranges,
                                       float(np.float32(b1)),
                                       float(np.float32(b2)))
        out, lse = oracle.combine(mo, ml, case["sinks"], g)
        fin = np.isfinite(ref["lse"][t])
        assert np.array_equal(fin, np.isfinite(lse))
        np.testing.assert_allclose(lse[fin], ref["lse"][t][fin], rtol=1e-12,
                                   atol=1e-12)
        np.testing.assert_allclose(out, ref["out"][t], rtol=1e-11, atol=1e-14)


def test_p7_combine_all_empty():
    mo = np.zeros((2, 4, D))
    ml = np.full((2, 4), -np.inf)
    out, lse = oracle.combine(mo, ml)
    assert not out.any() and np.all(np.isneginf(lse))
    sk = np.array([0.5, -2.0], np.float32)
    out, lse = oracle.combine(mo, ml, sk, 1.0)
    assert not out.any()
    np.testing.assert_allclose(lse, sk.astype(np.float64) * LOG2E, rtol=1e-15)


# ---------------------------------------------------------------------------
# P8: textbook routine (torch SDPA in float64 on the CPU)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "fp8_e4m3fn"])
def test_p8_matches_torch_sdpa_float64(dtype):
    case = tiny_case(51, T=2, H=4, K=170, swa_rows=200, comp_rows=300,
                     dtype=dtype, neg=0, sinks=False, lens=None, dup=False)
    # make rows unique inside each token
    rng = np.random.default_rng(3)
    for t in range(2):
        case["indices"][t, :128] = rng.permutation(200)[:128]
        case["indices"][t, 128:] = rng.permutation(300)[:42]
    b1, b2 = 0.04, 0.6
    r = run(case, b1, b2, 1.0)
    for t in range(2):
        slots = oracle.active_slots(case["indices"][t], None)
        rows = torch.from_numpy(oracle.sparse_mla.gather_rows(
            slots, case["swa_bits"], case["comp_bits"], dtype))
        q = torch.from_numpy(decode_bits(case["q_bits"][t], dtype))
        k = rows[None].expand(4, -1, -1)[None]
        o = torch.nn.functional.scaled_dot_product_attention(
            q[None, :, None, :], k, k, scale=float(np.float32(b1)))
        o = o[0, :, 0, :].numpy() * float(np.float32(b2))
        lse = torch.logsumexp(float(np.float32(b1)) * (q @ rows.T), -1) \
            / math.log(2.0)
        np.testing.assert_allclose(r["out"][t], o, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(r["lse"][t], lse.numpy(), rtol=1e-13)


# ---------------------------------------------------------------------------
# P9: selection probe with one-hot rows (exact counts)
# ---------------------------------------------------------------------------

def test_p9_selection_probe_counts():
    rng = np.random.default_rng(61)
    T, K, H = 6, 300, 2
    swa = np.zeros((512, D)); comp = np.zeros((700, D))
    swa[np.arange(512), np.arange(512)] = 1.0
    comp[np.arange(700), np.arange(700) % 512] = 1.0
    idx = np.empty((T, K), np.int32)
    for t in range(T):
        idx[t, :128] = rng.integers(0, 512, 128)
        idx[t, 128:] = rng.integers(0, 700, K - 128)
        idx[t, rng.choice(K, 20, replace=False)] = -1
    idx[5, :] = -1                              # all masked
    lens = np.array([127, 128, 129, K, 0, K], np.int32)
    case = dict(q_bits=bf16_bits(np.zeros((T, H, D))), q_dtype="bf16",
                swa_bits=bf16_bits(swa), comp_bits=bf16_bits(comp),
                kv_dtype="bf16", indices=idx, topk_lens=lens, sinks=None)
    r = run(case, 0.1, 1.0, 1.0)
    for t in range(T):
        want = np.zeros(D)
        n = 0
        for c in range(lens[t]):
            if idx[t, c] == -1:
                continue
            want[idx[t, c] % 512] += 1
            n += 1
        if n == 0:
            assert np.all(np.isneginf(r["lse"][t])) and not r["out"][t].any()
            continue
        assert np.all(np.rint(2.0 ** r["lse"][t]) == n)
        assert np.array_equal(np.rint(n * r["out"][t]), np.tile(want, (H, 1)))


# ---------------------------------------------------------------------------
# P10-P12: normalisation, FP8 folding, linearity and head permutation
# ---------------------------------------------------------------------------

def test_p10_probabilities_sum_to_one():
    case = tiny_case(71, sinks=True, lens=None)
    b1, g = 0.05, 1.3
    r = run(case, b1, 1.0, g)
    for t in range(3):
        slots = oracle.active_slots(case["indices"][t], None)
        rows = oracle.sparse_mla.gather_rows(slots, case["swa_bits"],
                                             case["comp_bits"], "bf16")
        q = decode_bits(case["q_bits"][t], "bf16")
        s = float(np.float32(b1)) * (q @ rows.T) * LOG2E
        ln = r["lse"][t] / float(np.float32(g))
        tot = np.exp2(s - ln[:, None]).sum(1) + np.exp2(
            case["sinks"].astype(np.float64) * LOG2E - ln)
        np.testing.assert_allclose(tot, 1.0, rtol=1e-13)


def test_p11_fp8_scale_folding():
    # power-of-two scales make the folded binary32 scale exact
    sm, qs, ks = 2.0 ** -5, 2.0 ** -4, 2.0 ** -3
    case = tiny_case(81, dtype="fp8_e4m3fn", lens=None)
    folded = run(case, sm * qs * ks, ks, 1.0)
    for t in range(3):
        slots = oracle.active_slots(case["indices"][t], None)
        rows = oracle.sparse_mla.gather_rows(slots, case["swa_bits"],
                                             case["comp_bits"], "fp8_e4m3fn")
        q = decode_bits(case["q_bits"][t], "fp8_e4m3fn") * qs
        o, l, _ = oracle.decode_token(q, rows * ks,
                                      case["sinks"].astype(np.float64),
                                      sm, 1.0, 1.0)
        np.testing.assert_allclose(folded["out"][t], o, rtol=1e-13, atol=1e-16)
        np.testing.assert_allclose(folded["lse"][t], l, rtol=1e-14)


def test_p12_linearity_and_head_permutation():
    case = tiny_case(91, H=4, lens=None)
    a = run(case, 0.05, 1.0, 1.0)
    b = run(case, 0.05, 0.375, 1.0)
    np.testing.assert_allclose(b["out"], 0.375 * a["out"], rtol=1e-15, atol=0)
    perm = np.array([2, 0, 3, 1])
    pc = dict(case, q_bits=case["q_bits"][:, perm], sinks=case["sinks"][perm])
    c = run(pc, 0.05, 1.0, 1.0)
    np.testing.assert_allclose(c["out"], a["out"][:, perm], rtol=1e-15, atol=0)
    np.testing.assert_allclose(c["lse"], a["lse"][:, perm], rtol=1e-15)


def test_lse_scale_ln2_gives_natural_log():
    case = tiny_case(92, lens=None)
    a = run(case, 0.05, 1.0, 1.0)
    b = run(case, 0.05, 1.0, math.log(2.0))
    np.testing.assert_allclose(b["lse"], a["lse"] * float(np.float32(
        math.log(2.0))), rtol=1e-15)


def test_empty_token_with_and_without_sink():
    case = tiny_case(93, lens=[0, 0, 0], sinks=True)
    r = run(case, 0.05, 1.0, 2.0)
    assert not r["out"].any()
    np.testing.assert_allclose(
        r["lse"], np.tile(2.0 * case["sinks"].astype(np.float64) * LOG2E,
                          (3, 1)), rtol=1e-15)
    r2 = run(dict(case, sinks=None), 0.05, 1.0, 2.0)
    assert not r2["out"].any() and np.all(np.isneginf(r2["lse"]))
