"""Pins of the fp64 oracle against things other than itself.

Every check compares the oracle with a closed form, an invariant, a library
routine (transformers' half-split RoPE, torch's scaled-dot-product attention,
torch's float32->bfloat16 conversion, numpy sorting) or brute force on tiny
inputs.  A plausible slip anywhere in the oracle -- wrong rotation sign or
pairing, a dropped 1/sqrt(d), HF/LF swapped, an off-by-half representative
position, a wrong window bound, a transposed operand, a wrong GQA head
mapping -- fails at least one of them.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle
from synth import bf16_bits, bf16_to_f32

RNG = np.random.default_rng(12345)


def cfg(d=64, hq=1, hkv=1, C=64, G=4, ns=1, nl=2, kc=2, kg=4, theta=1e4, hf=64.0, bf16=False,
        rep_integer=False, interleaved=False):
    return oracle.make_cfg(d, hq, hkv, C, G, ns, nl, kc, kg, theta, hf, bf16, rep_integer,
                           interleaved)


def omegas(c):
    return np.array([oracle.omega(c, j) for j in range(c.d // 2)])


def lib_rope(x, pos, c):
    """Half-split RoPE through transformers' apply_rotary_pos_emb (fp64).

    x [..., n, d], pos [n]."""
    mod = pytest.importorskip("transformers.models.llama.modeling_llama")
    w = torch.tensor(omegas(c), dtype=torch.float64)
    ang = torch.tensor(np.asarray(pos, dtype=np.float64))[:, None] * w[None, :]
    emb = torch.cat([ang, ang], dim=-1)
    xt = torch.tensor(np.asarray(x, dtype=np.float64))
    out, _ = mod.apply_rotary_pos_emb(xt, xt, emb.cos(), emb.sin(), unsqueeze_dim=0)
    return out.numpy().reshape(xt.shape)


def as_complex(x):
    h = x.shape[-1] // 2
    return x[..., :h] + 1j * x[..., h:]


def from_complex(z):
    return np.concatenate([z.real, z.imag], axis=-1)


# ------------------------------------------------------------------ RoPE
def test_omega_matches_library_frequencies():
    mod = pytest.importorskip("transformers.models.llama.modeling_llama")
    from types import SimpleNamespace
    for d, theta in [(64, 1e4), (128, 1e6)]:
        conf = SimpleNamespace(rope_parameters={"rope_theta": theta}, head_dim=d,
                               hidden_size=d, num_attention_heads=1)
        inv, _ = mod.LlamaRotaryEmbedding.compute_default_rope_parameters(conf)
        c = cfg(d=d, theta=theta)
        np.testing.assert_allclose(omegas(c), inv.double().numpy(), rtol=2e-6)


def test_rope_matches_library_half_split():
    c = cfg(d=128, theta=1e6)
    x = RNG.standard_normal((7, 128))
    pos = np.array([0, 1, 5, 63, 1000, 32767, 65535])
    ref = lib_rope(x, pos, c)
    got = np.stack([oracle.rope(c, x[i], pos[i]) for i in range(7)])
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_rope_interleaved_matches_library():
    """The interleaved variant against transformers' GPT-J rotary embedding
    (pairs (x_2j, x_2j+1)), fp64."""
    mod = pytest.importorskip("transformers.models.gptj.modeling_gptj")
    c = cfg(d=128, theta=1e6, interleaved=True)
    x = RNG.standard_normal((7, 128))
    pos = np.array([0, 1, 5, 63, 1000, 32767, 65535], dtype=np.float64)
    ang = torch.tensor(pos)[:, None] * torch.tensor(omegas(c))[None, :]  # [n][d/2]
    xt = torch.tensor(x)[None, :, None, :]                                # [1][n][1][d]
    ref = mod.apply_rotary_pos_emb(xt, ang.sin()[None], ang.cos()[None])[0, :, 0].numpy()
    got = np.stack([oracle.rope(c, x[i], pos[i]) for i in range(7)])
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_interleaved_is_a_permutation_of_half_split():
    """Rotating, summarising and routing with interleaved pairs equals the
    half-split path on inputs whose dims are permuted (2j, 2j+1) -> (j, j+d/2),
    permuted back."""
    d = 128
    perm = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])  # interleaved dim of half-split dim
    ci = cfg(d=d, theta=1e6, interleaved=True)
    ch = cfg(d=d, theta=1e6)
    x = RNG.standard_normal(d)
    np.testing.assert_array_equal(oracle.rope(ci, x, 4321)[perm], oracle.rope(ch, x[perm], 4321))
    k = RNG.standard_normal((64, d))
    np.testing.assert_array_equal(oracle.span_summary(ci, k, 640)[perm],
                                  oracle.span_summary(ch, k[:, perm], 640))


def test_rope_invariants():
    c = cfg(d=128, theta=1e6)
    x = RNG.standard_normal(128)
    y = RNG.standard_normal(128)
    np.testing.assert_array_equal(oracle.rope(c, x, 0), x)
    r = oracle.rope(c, x, 40000)
    np.testing.assert_allclose(np.abs(as_complex(r)), np.abs(as_complex(x)), rtol=1e-13)
    for t, p in [(65535, 1234), (100, 99), (7, 60000)]:
        lhs = oracle.rope(c, x, t) @ oracle.rope(c, y, p)
        rhs = x @ oracle.rope(c, y, p - t)
        assert abs(lhs - rhs) < 1e-9 * (1 + abs(lhs))


def test_hf_classification_closed_form():
    # wavelength 2*pi*theta^(2j/d) < C  <=>  j < (d/2) ln(C / 2 pi) / ln(theta)
    for d, theta, n_hf in [(64, 1e4, 9), (128, 1e6, 11)]:
        c = cfg(d=d, theta=theta, hf=64.0)
        flags = [oracle.is_hf(c, j) for j in range(d // 2)]
        assert flags == [j < n_hf for j in range(d // 2)]
        bound = (d / 2) * math.log(64 / (2 * math.pi)) / math.log(theta)
        assert n_hf == math.floor(bound) + 1
    assert not any(oracle.is_hf(cfg(hf=0.0), j) for j in range(32))
    assert all(oracle.is_hf(cfg(hf=math.inf), j) for j in range(32))


def test_hf_classification_at_group_wavelength():
    """The variant lambda_hf = g = 16: 4 HF pairs at d = 64, theta = 1e4 and 5
    at d = 128, theta = 1e6 (the closed form of the bound)."""
    for d, theta, n_hf in [(64, 1e4, 4), (128, 1e6, 5)]:
        c = cfg(d=d, theta=theta, hf=16.0)
        flags = [oracle.is_hf(c, j) for j in range(d // 2)]
        assert flags == [j < n_hf for j in range(d // 2)]
        bound = (d / 2) * math.log(16 / (2 * math.pi)) / math.log(theta)
        assert n_hf == math.floor(bound) + 1


# ------------------------------------------------------------- summaries
@pytest.mark.parametrize("rep_integer", [False, True])
@pytest.mark.parametrize("n,a", [(64, 0), (16, 48), (64, 65472), (16, 1000)])
def test_summary_all_lowfreq_is_rotated_mean(n, a, rep_integer):
    """All pairs low-frequency: the raw mean rotated to the representative
    position, the midpoint a + (n-1)/2 or, in the variant, a + n/2."""
    c = cfg(d=128, theta=1e6, hf=0.0, rep_integer=rep_integer)
    k = RNG.standard_normal((n, 128))
    r = a + (n / 2 if rep_integer else (n - 1) / 2)
    want = from_complex(as_complex(k.mean(axis=0)) * np.exp(1j * r * omegas(c)))
    np.testing.assert_allclose(oracle.span_summary(c, k, a), want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("n,a", [(64, 64 * 37), (16, 16 * 5)])
def test_summary_all_highfreq_scores_are_mean_token_logits(n, a):
    c = cfg(d=128, theta=1e6, hf=math.inf)
    k = RNG.standard_normal((n, 128))
    qbar = RNG.standard_normal(128)
    s = oracle.span_summary(c, k, a)
    rot = lib_rope(k, np.arange(a, a + n), c)
    np.testing.assert_allclose(qbar @ s / math.sqrt(128), np.mean(rot @ qbar) / math.sqrt(128),
                               rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("d,theta", [(64, 1e4), (128, 1e6)])
@pytest.mark.parametrize("n,a", [(64, 960), (16, 65520), (64, 0)])
def test_summary_constant_key_dirichlet_closed_form(d, theta, n, a):
    c = cfg(d=d, theta=theta, hf=64.0)
    k0 = RNG.standard_normal(d)
    k = np.tile(k0, (n, 1))
    w = omegas(c)
    r = a + (n - 1) / 2
    dn = np.sin(n * w / 2) / (n * np.sin(w / 2))
    hf = 2 * np.pi / w < 64.0
    factor = np.where(hf, dn, 1.0)
    want = from_complex(as_complex(k0) * factor * np.exp(1j * r * w))
    # fp64 angles near 65535 rad carry ~1e-11 rad of rounding
    np.testing.assert_allclose(oracle.span_summary(c, k, a), want, rtol=0, atol=1e-10)


def test_representative_position_moves_only_lowfreq_pairs():
    """The variant changes LF pairs by a half-step rotation (omega_j / 2) and
    leaves HF pairs exactly as they were."""
    d, a, n = 128, 64 * 77, 64
    k = RNG.standard_normal((n, d))
    mid = oracle.span_summary(cfg(d=d, theta=1e6, hf=64.0), k, a)
    intg = oracle.span_summary(cfg(d=d, theta=1e6, hf=64.0, rep_integer=True), k, a)
    w = omegas(cfg(d=d, theta=1e6))
    hf = 2 * np.pi / w < 64.0
    zm, zi = as_complex(mid), as_complex(intg)
    np.testing.assert_array_equal(zi[hf], zm[hf])
    np.testing.assert_allclose(zi[~hf], zm[~hf] * np.exp(0.5j * w[~hf]), rtol=0, atol=1e-12)


def test_summary_mixed_is_per_pair_choice():
    d = 128
    k = RNG.standard_normal((64, d))
    a = 64 * 123
    mixed = oracle.span_summary(cfg(d=d, theta=1e6, hf=64.0), k, a)
    hf = oracle.span_summary(cfg(d=d, theta=1e6, hf=math.inf), k, a)
    lf = oracle.span_summary(cfg(d=d, theta=1e6, hf=0.0), k, a)
    pick = np.array([j < 11 for j in range(d // 2)] * 2)
    np.testing.assert_array_equal(mixed, np.where(pick, hf, lf))


def test_summary_linear_and_shift_equivariant():
    c = cfg(d=128, theta=1e6, hf=64.0)
    ka = RNG.standard_normal((64, 128))
    kb = RNG.standard_normal((64, 128))
    sa = oracle.span_summary(c, ka, 640)
    sb = oracle.span_summary(c, kb, 640)
    np.testing.assert_allclose(oracle.span_summary(c, 2.5 * ka - 0.75 * kb, 640), 2.5 * sa - 0.75 * sb,
                               atol=1e-12)
    shift = 64 * 311
    moved = oracle.span_summary(c, ka, 640 + shift)
    want = from_complex(as_complex(sa) * np.exp(1j * shift * omegas(c)))
    np.testing.assert_allclose(moved, want, atol=1e-11)


def test_summaries_table_layout():
    c = cfg(d=64, theta=1e4, hf=64.0)
    k = RNG.standard_normal((256, 64))
    cs, gs = oracle.summaries(c, k)
    assert cs.shape == (4, 64) and gs.shape == (16, 64)
    np.testing.assert_array_equal(cs[2], oracle.span_summary(c, k[128:192], 128))
    np.testing.assert_array_equal(gs[9], oracle.span_summary(c, k[144:160], 144))


# ------------------------------------------------------------------ pool
def test_round_bf16_matches_torch_on_float32_values():
    x = (RNG.standard_normal(20000) * np.exp(RNG.uniform(-20, 20, 20000))).astype(np.float32)
    want = torch.tensor(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.round_bf16(x.astype(np.float64)), want)
    np.testing.assert_array_equal(bf16_to_f32(bf16_bits(x)).astype(np.float64), want)


def test_round_bf16_direct_from_fp64():
    e = 2.0 ** -8
    cases = {1 + e: 1.0,                     # tie -> even
             1 + 3 * e: 1 + 4 * e,           # tie -> even (up)
             1 + e + 2.0 ** -40: 1 + 2 * e,  # just above the tie: up (no double rounding)
             -(1 + e - 2.0 ** -40): -1.0,
             0.0: 0.0, 3.0: 3.0}
    for x, want in cases.items():
        assert oracle.round_bf16([x])[0] == want, x


@pytest.mark.parametrize("bf16", [True, False])
def test_pool_is_rounded_rotation(bf16):
    c = cfg(d=128, theta=1e6, bf16=bf16)
    k = RNG.standard_normal((32, 128))
    pos0 = 65500
    rot = lib_rope(k, np.arange(pos0, pos0 + 32), c)
    want = oracle.round_bf16(rot) if bf16 else rot.astype(np.float32).astype(np.float64)
    got = oracle.pool(c, k, pos0)
    # the library rotation and the oracle rotation agree to ~1e-15; a
    # rounding-boundary straddle would show as a 1-ulp difference
    diff = np.abs(got - want)
    ulp = np.abs(want) * (2.0 ** -7 if bf16 else 2.0 ** -23)
    assert np.all(diff <= ulp)
    assert np.mean(diff > 0) < 1e-3


# ----------------------------------------------------- windows, candidates
@pytest.mark.parametrize("ns,nl", [(1, 2), (1, 4), (0, 3), (2, 0), (3, 5)])
def test_windows_brute_force(ns, nl):
    c = cfg(ns=ns, nl=nl)
    for ct in range(0, 25):
        win, lo, hi = oracle.windows(c, ct)
        want = sorted({ch for ch in range(ct) if ch < ns} | {ch for ch in range(ct) if ct - nl <= ch})
        assert list(win) == want
        cands = [ch for ch in range(ct) if ch not in want and ch >= ns]
        assert list(range(lo, hi)) == cands, (ct, lo, hi)


# -------------------------------------------------------------- selection
def tiny_state(T=1024, d=64, hq=1, hkv=1, theta=1e4, seed=0):
    r = np.random.default_rng(seed)
    k = r.standard_normal((T, d))
    c = cfg(d=d, hq=hq, hkv=hkv, theta=theta)
    cs, gs = oracle.summaries(c, k)
    return c, k, cs, gs, r


def test_selection_matches_numpy_sort_and_brute_force():
    c, k, cs, gs, r = tiny_state()
    for t in range(1016, 1024):
        q = r.standard_normal((1, 1, 64))
        sel, margins, scores = oracle.select(c, q, t, cs, gs)
        ct = t // 64
        qbar = oracle.rope(c, q[0, 0], t)
        cand = np.arange(1, ct - 2)
        s1 = cs[cand] @ qbar / 8.0
        np.testing.assert_allclose(scores, s1, rtol=1e-13, atol=1e-15)
        order = np.lexsort((cand, -s1))
        top1 = set(cand[order[:2]])
        # brute force: the top-2 set maximises the score sum over all pairs
        best = max(itertools.combinations(range(len(cand)), 2), key=lambda ij: s1[list(ij)].sum())
        assert top1 == set(cand[list(best)])
        groups = np.array([ch * 4 + j for ch in sorted(top1) for j in range(4)])
        s2 = gs[groups] @ qbar / 8.0
        top2 = set(groups[np.lexsort((groups, -s2))[:4]])
        want = sorted(set(range(0, 4)) | set(range((ct - 2) * 4, ct * 4)) |
                      set(range(ct * 4, t // 16 + 1)) | top2)
        assert list(sel) == want
        ss = np.sort(s1)[::-1]
        assert margins[0] == pytest.approx(ss[1] - ss[2], abs=1e-15)


def test_selection_nesting_and_level2_subset():
    _, k, cs, gs, r = tiny_state(T=4096, d=64, seed=3)
    q = r.standard_normal((1, 1, 64))
    t = 4095
    prev = None
    for kc in range(1, 12):
        c = cfg(kc=kc, kg=4 * kc)
        sel, _, scores = oracle.select(c, q, t, cs, gs)
        s = set(sel)
        if prev is not None:
            assert prev <= s
        prev = s
    c = cfg(kc=6, kg=1)
    prev = None
    for kg in range(1, 25):
        c = cfg(kc=6, kg=kg)
        sel, _, scores = oracle.select(c, q, t, cs, gs)
        cand = np.arange(1, 63 - 2)
        l1 = set(cand[np.lexsort((cand, -scores))[:6]])
        routed = [g for g in sel if 1 <= g // 4 < 61]
        assert {g // 4 for g in routed} <= l1
        assert len(routed) == kg
        s = set(sel)
        if prev is not None:
            assert prev <= s
        prev = s


@pytest.mark.parametrize("t", [0, 5, 63, 64, 100, 200, 255, 1023])
def test_select_all_gives_every_group_up_to_t(t):
    _, k, cs, gs, r = tiny_state(seed=7)
    c = cfg(kc=10 ** 6, kg=10 ** 6)
    q = r.standard_normal((1, 1, 64))
    sel, margins, _ = oracle.select(c, q, t, cs, gs)
    assert list(sel) == list(range(t // 16 + 1))
    assert margins[0] == math.inf and margins[1] == math.inf


def test_windows_always_present():
    _, k, cs, gs, r = tiny_state(seed=11)
    for ns, nl in [(1, 2), (2, 1), (0, 3)]:
        c = cfg(ns=ns, nl=nl, kc=1, kg=1)
        for t in [64, 129, 500, 1000, 1023]:
            q = r.standard_normal((1, 1, 64))
            sel, _, _ = oracle.select(c, q, t, cs, gs)
            ct = t // 64
            for ch in list(range(min(ns, ct))) + list(range(max(0, ct - nl), ct)):
                assert all(ch * 4 + j in sel for j in range(4))
            assert all(g in sel for g in range(ct * 4, t // 16 + 1))
            assert list(sel) == sorted(set(sel))


def test_pooled_query_scores_equal_mean_head_token_logits():
    # all-HF summaries: pooled-query score == mean over heads, query tokens
    # and span tokens of the exact rotated logits (scores are linear)
    d, hg, lq = 64, 4, 3
    c = oracle.make_cfg(d, hg, 1, 64, 4, 1, 1, 3, 6, 1e4, math.inf, False)
    k = RNG.standard_normal((64 * 20, d))
    cs, gs = oracle.summaries(c, k)
    q = RNG.standard_normal((hg, lq, d))
    pos0 = 64 * 19 + 10
    _, _, scores = oracle.select(c, q, pos0, cs, gs)
    qrot = np.stack([lib_rope(q[h], np.arange(pos0, pos0 + lq), c) for h in range(hg)])
    krot = lib_rope(k, np.arange(k.shape[0]), c)
    for i, ch in enumerate(range(1, 19 - 1)):
        logits = qrot.reshape(-1, d) @ krot[ch * 64:(ch + 1) * 64].T / math.sqrt(d)
        assert scores[i] == pytest.approx(logits.mean(), rel=1e-11, abs=1e-13)


# -------------------------------------------------------------- attention
def sdpa_dense(q_rot, k, v, q_pos, hg):
    """Dense causal attention through torch SDPA (fp64, CPU).

    q_rot [Hq][lq][d] rotated; k, v [Hkv][T][d]; q_pos [lq]."""
    T = k.shape[1]
    kk = torch.tensor(k).repeat_interleave(hg, dim=0)
    vv = torch.tensor(v).repeat_interleave(hg, dim=0)
    mask = torch.tensor(np.arange(T)[None, :] <= np.asarray(q_pos)[:, None])
    return torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q_rot), kk, vv, attn_mask=mask).numpy()


@pytest.mark.parametrize("hq,hkv,lq,pos0", [(1, 1, 1, 1023), (8, 2, 1, 777), (4, 2, 64, 640),
                                            (6, 3, 5, 130)])
def test_select_all_equals_dense_causal_attention(hq, hkv, lq, pos0):
    d, T = 64, 1024
    c = oracle.make_cfg(d, hq, hkv, 64, 4, 1, 2, 10 ** 6, 10 ** 6, 1e4, 64.0, True)
    hg = hq // hkv
    kraw = RNG.standard_normal((hkv, T, d))
    v = RNG.standard_normal((hkv, T, d))
    q = RNG.standard_normal((hq, lq, d))
    kpool = np.stack([oracle.pool(c, kraw[h], 0) for h in range(hkv)])
    qpos = np.arange(pos0, pos0 + lq)
    q_rot = np.stack([lib_rope(q[h], qpos, c) for h in range(hq)])
    want = sdpa_dense(q_rot, kpool, v, qpos, hg)
    for h in range(hkv):
        cs, gs = oracle.summaries(c, kraw[h])
        qh = q[h * hg:(h + 1) * hg]
        sel, _, _ = oracle.select(c, qh, pos0, cs, gs)
        out, lse = oracle.attend(c, qh, pos0, kpool[h], v[h], sel)
        np.testing.assert_allclose(out, want[h * hg:(h + 1) * hg], rtol=0, atol=1e-12)
        logits = np.einsum("hld,td->hlt", q_rot[h * hg:(h + 1) * hg], kpool[h]) / math.sqrt(d)
        logits = np.where(np.arange(T)[None, None, :] <= qpos[None, :, None], logits, -np.inf)
        np.testing.assert_allclose(lse, torch.logsumexp(torch.tensor(logits), -1).numpy(),
                                   rtol=1e-13)


def test_lse_merge_of_disjoint_parts_equals_union():
    c = oracle.make_cfg(64, 4, 1, 64, 4, 1, 2, 2, 4, 1e4, 64.0, False)
    k = RNG.standard_normal((1024, 64))
    v = RNG.standard_normal((1024, 64))
    q = RNG.standard_normal((4, 1, 64))
    kp = oracle.pool(c, k, 0)
    sel = np.array([0, 1, 2, 3, 9, 17, 40, 41, 55, 56, 57, 58, 59, 60, 61, 62, 63])
    a, b = sel[::2], sel[1::2]
    oa, la = oracle.attend(c, q, 1023, kp, v, a)
    ob, lb = oracle.attend(c, q, 1023, kp, v, b)
    om, lm = oracle.merge(oa, la, ob, lb)
    ou, lu = oracle.attend(c, q, 1023, kp, v, sel)
    np.testing.assert_allclose(om, ou, atol=1e-13)
    np.testing.assert_allclose(lm, lu, rtol=1e-14)


def test_gather_is_a_copy():
    c = cfg()
    pool = RNG.standard_normal((1024, 64))
    sel = np.array([0, 5, 6, 63])
    got = oracle.gather(c, pool, sel)
    want = pool.reshape(64, 16, 64)[sel].reshape(-1, 64)
    np.testing.assert_array_equal(got, want)


def test_exact_ties_break_by_ascending_id():
    # identical summary rows give bit-identical scores; the kept items must
    # be the lowest ids among the tied ones at both levels
    c = cfg(kc=2, kg=3)
    q = RNG.standard_normal((1, 1, 64))
    t = 1023
    qbar = oracle.rope(c, q[0, 0], t)
    cs = np.zeros((16, 64))
    gs = np.zeros((64, 64))
    for ch in (3, 5, 8, 11):
        cs[ch] = qbar / np.linalg.norm(qbar)
    for ch in (1, 2, 4, 6, 7, 9, 10, 12):
        cs[ch] = -qbar / np.linalg.norm(qbar)
    gs[:] = -qbar
    for gid in (13, 14, 15, 20, 22):
        gs[gid] = qbar
    sel, margins, _ = oracle.select(c, q, t, cs, gs)
    assert margins[0] == 0.0 and margins[1] == 0.0
    routed = [g for g in sel if 1 <= g // 4 < 13]
    assert routed == [13, 14, 15]


# ------------------------------------------------------------- fp8 pool
def test_fp8_decode_matches_torch_e4m3fn():
    """Every E4M3FN code decodes as torch's float8_e4m3fn does."""
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.fp8_decode(c) for c in range(256)])
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])


def test_fp8_encode_matches_torch_rounding():
    """Round to nearest even into E4M3FN, against torch's float32 ->
    float8_e4m3fn conversion, on random values across the normal and
    subnormal ranges and on exact halfway points."""
    rng = np.random.default_rng(8)
    y = np.concatenate([rng.uniform(-448, 448, 4000),
                        rng.uniform(-2.0 ** -5, 2.0 ** -5, 2000),
                        rng.standard_normal(2000) * 3.0]).astype(np.float32)
    vals = np.array([oracle.fp8_decode(c) for c in range(256)])
    fin = np.sort(np.unique(vals[np.isfinite(vals)]))
    halfway = ((fin[1:] + fin[:-1]) / 2).astype(np.float32)  # exact in fp32
    y = np.concatenate([y, halfway, -halfway, np.float32([0.0, 448.0, -448.0, 2.0 ** -9])])
    ref = torch.tensor(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy().astype(int)
    got = np.array([oracle.fp8_encode(float(v)) for v in y])
    neg_zero = (y == 0) & np.signbit(y)
    np.testing.assert_array_equal(got[~neg_zero], ref[~neg_zero])


def test_fp8_row_scale_is_the_smallest_fitting_power_of_two():
    rng = np.random.default_rng(9)
    for amax in np.concatenate([rng.uniform(1e-6, 1e6, 500), [448.0, 448.0 * 2 ** -20, 1.0, 0.0]]):
        s = oracle.fp8_scale(amax)
        assert s > 0 and math.frexp(s)[0] == 0.5  # a power of two
        if amax == 0:
            assert s == 1.0
            continue
        assert amax / s <= 448.0 and amax / (s / 2) > 448.0
    x = rng.standard_normal((5, 128)) * np.array([1e-3, 1.0, 30.0, 500.0, 1e4])[:, None]
    codes, scales, deq = oracle.fp8_rows(x)
    for i in range(5):
        assert scales[i] == oracle.fp8_scale(np.abs(x[i]).max())
        want = np.array([oracle.fp8_decode(oracle.fp8_encode(v / scales[i])) for v in x[i]]) * scales[i]
        np.testing.assert_array_equal(deq[i], want)
        # within half a quantum of the rounded binade (3 mantissa bits)
        assert np.all(np.abs(deq[i] - x[i]) <= np.maximum(np.abs(x[i]) * 2.0 ** -4, 2.0 ** -10 * scales[i]))


def test_pool_fp8_quantises_the_library_rotation():
    """FP8 pool keys: each row of transformers' half-split RoPE at its own
    position, divided by the smallest power of two that brings its largest
    magnitude within 448, converted by torch to float8_e4m3fn.  Quantising
    before the rotation, or rotating to the wrong first position, fails."""
    c = cfg(d=128, theta=1e6, bf16=True)
    rng = np.random.default_rng(21)
    kraw = rng.standard_normal((48, 128)) * np.geomspace(1e-3, 3e3, 48)[:, None]
    pos0 = 40000
    codes, scales, deq = oracle.pool_fp8(c, kraw, pos0)
    rot = lib_rope(kraw, np.arange(pos0, pos0 + 48), c)
    amax = np.abs(rot).max(axis=1)
    want_scale = 2.0 ** np.ceil(np.log2(amax / 448.0))
    np.testing.assert_array_equal(scales, want_scale)
    y = torch.tensor(rot / want_scale[:, None])
    want = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy().astype(np.int64)
    np.testing.assert_array_equal(codes, want)
    np.testing.assert_array_equal(
        deq, y.to(torch.float8_e4m3fn).to(torch.float64).numpy() * want_scale[:, None])
    # the same rows quantised at another first position differ
    other, _, _ = oracle.pool_fp8(c, kraw, pos0 + 1)
    assert (other != codes).mean() > 0.3


def test_group_scores_rank_level2_and_equal_mean_token_logits():
    """Level-2 scores: the groups ora_select routes are the top-k_g of
    ora_group_scores over the groups of its level-1 chunks (numpy lexsort);
    with all-HF summaries a group's score is the mean over the query heads,
    query tokens and the group's tokens of the exact rotated logits."""
    d, hg, lq = 64, 4, 3
    c = oracle.make_cfg(d, hg, 1, 64, 4, 1, 1, 3, 6, 1e4, 64.0, False)
    k = RNG.standard_normal((64 * 20, d))
    cs, gs = oracle.summaries(c, k)
    q = RNG.standard_normal((hg, lq, d))
    pos0 = 64 * 19 + 10
    sel, _, s1 = oracle.select(c, q, pos0, cs, gs)
    g_sc = oracle.group_scores(c, q, pos0, gs)
    assert g_sc.shape == (19 * 4,)
    cand = np.arange(1, 18)
    l1 = cand[np.lexsort((cand, -s1))[:3]]
    groups = np.array([ch * 4 + j for ch in l1 for j in range(4)])
    top = set(groups[np.lexsort((groups, -g_sc[groups]))[:6]])
    assert top == {g for g in sel if 1 <= g // 4 < 18}
    ch = oracle.make_cfg(d, hg, 1, 64, 4, 1, 1, 3, 6, 1e4, math.inf, False)
    cs, gs = oracle.summaries(ch, k)
    g_sc = oracle.group_scores(ch, q, pos0, gs)
    qrot = np.stack([lib_rope(q[h], np.arange(pos0, pos0 + lq), ch) for h in range(hg)])
    krot = lib_rope(k, np.arange(k.shape[0]), ch)
    for gid in (0, 5, 33, 75):
        logits = qrot.reshape(-1, d) @ krot[gid * 16:(gid + 1) * 16].T / math.sqrt(d)
        assert g_sc[gid] == pytest.approx(logits.mean(), rel=1e-11, abs=1e-13)


@pytest.mark.parametrize("lq", [1, 3])
def test_step_equals_per_unit_select_and_attend(lq):
    """The batched driver gives, unit by unit, the bits of ora_select then
    ora_attend on that unit's own slices (distinct content and positions per
    unit, so a wrong per-unit stride shows)."""
    d, hq, hkv, T = 64, 4, 2, 1024
    hg = hq // hkv
    c = oracle.make_cfg(d, hq, hkv, 64, 4, 1, 2, 2, 4, 1e4, 64.0, True)
    rng = np.random.default_rng(31)
    U = 5
    kraw = rng.standard_normal((U, T, d))
    v = rng.standard_normal((U, T, d))
    q = rng.standard_normal((U, hg, lq, d))
    pos = np.array([1021, 700, 64 * 9 + 3, 960, 129])
    cs = np.stack([oracle.summaries(c, kraw[u])[0] for u in range(U)])
    gs = np.stack([oracle.summaries(c, kraw[u])[1] for u in range(U)])
    kp = np.stack([oracle.pool(c, kraw[u], 0) for u in range(U)])
    max_sel = 40
    sel, nsel, out = oracle.step(c, q, pos, cs, gs, kp, v, max_sel)
    for u in range(U):
        s_u, _, _ = oracle.select(c, q[u], pos[u], cs[u], gs[u])
        assert nsel[u] == s_u.size
        np.testing.assert_array_equal(sel[u, :nsel[u]], s_u)
        o_u, _ = oracle.attend(c, q[u], pos[u], kp[u], v[u], s_u)
        np.testing.assert_array_equal(out[u], o_u)


# ------------------------------------------------------------- warm tier
def _warm_brute(tags, used, routed):
    """Every assignment of the misses to slots that are not hits, kept when
    the taken slots are the least recently used ones by (stamp, slot index)
    and the misses take them in list order."""
    W = len(tags)
    where = {int(t): s for s, t in enumerate(tags) if t >= 0}
    hits = {where[g] for g in routed if g in where}
    misses = [g for g in routed if g not in where]
    free = [s for s in range(W) if s not in hits]
    key = lambda s: (used[s], s)
    found = []
    for perm in itertools.permutations(free, len(misses)):
        taken = set(perm)
        least = all(key(a) < key(b) for a in taken for b in free if b not in taken)
        ordered = all(key(perm[i]) < key(perm[i + 1]) for i in range(len(perm) - 1))
        if least and ordered:
            found.append(perm)
    return found, hits


def test_warm_policy_brute_force():
    rng = np.random.default_rng(41)
    for trial in range(300):
        W = int(rng.integers(1, 7))
        universe = rng.permutation(20)[:W + 4]
        n_cached = int(rng.integers(0, W + 1))
        tags = np.full(W, -1)
        tags[rng.permutation(W)[:n_cached]] = universe[:n_cached]
        used = np.where(tags >= 0, rng.integers(1, 4, W), 0)
        n = int(rng.integers(0, W + 1))
        routed = [int(x) for x in rng.permutation(universe)[:n]]
        found, hits = _warm_brute(tags, used, routed)
        misses = [g for g in routed if g not in set(tags.tolist())]
        if len(misses) > W - len(hits):
            with pytest.raises(ValueError):
                oracle.warm_step(tags, used, routed, 5)
            continue
        assert len(found) == 1, (tags, used, routed, found)
        t2, u2, slot, hit, nh = oracle.warm_step(tags, used, routed, 5)
        assert nh == len(hits) == int(hit.sum())
        assert tuple(int(slot[i]) for i, g in enumerate(routed) if g in misses) == found[0]
        for i, g in enumerate(routed):
            assert t2[slot[i]] == g and u2[slot[i]] == 5
        kept = [s for s in range(W) if s not in set(slot.tolist())]
        np.testing.assert_array_equal(t2[kept], tags[kept])
        np.testing.assert_array_equal(u2[kept], used[kept])


def test_warm_policy_is_textbook_lru_for_one_access_per_step():
    """With one routed group per step the policy is the textbook LRU cache
    (move to the most recent end on a hit; on a miss with the cache full,
    evict the least recent): the same set of cached groups after every step."""
    from collections import OrderedDict
    rng = np.random.default_rng(43)
    W = 6
    tags, used = np.full(W, -1), np.zeros(W, dtype=int)
    ref = OrderedDict()
    for step in range(1, 400):
        g = int(rng.zipf(1.5)) % 25
        tags, used, _, hit, _ = oracle.warm_step(tags, used, [g], step)
        if g in ref:
            ref.move_to_end(g)
            assert hit[0] == 1
        else:
            if len(ref) == W:
                ref.popitem(last=False)
            ref[g] = True
            assert hit[0] == 0
        assert set(int(t) for t in tags if t >= 0) == set(ref)


def test_warm_policy_invariants_over_many_steps():
    rng = np.random.default_rng(47)
    W = 16
    tags, used = np.full(W, -1), np.zeros(W, dtype=int)
    seen = set()
    for step in range(1, 80):
        routed = [int(x) for x in rng.permutation(40)[:int(rng.integers(1, 9))]]
        before = set(int(t) for t in tags if t >= 0)
        tags, used, slot, hit, nh = oracle.warm_step(tags, used, routed, step)
        assert nh == len(before & set(routed))
        assert len(set(int(t) for t in tags if t >= 0)) == int((tags >= 0).sum())  # distinct tags
        for i, g in enumerate(routed):
            assert tags[slot[i]] == g and used[slot[i]] == step
        seen |= set(routed)
    # a cache at least as large as the universe never evicts
    tags, used = np.full(64, -1), np.zeros(64, dtype=int)
    seen = set()
    for step in range(1, 60):
        routed = [int(x) for x in rng.permutation(40)[:int(rng.integers(1, 9))]]
        tags, used, _, _, nh = oracle.warm_step(tags, used, routed, step)
        assert nh == len(seen & set(routed))
        seen |= set(routed)
        assert set(int(t) for t in tags if t >= 0) == seen


# ------------------------------------------------ max-pooled routing query
def test_max_pooled_routing_with_one_head_is_the_mean():
    """One query head per KV head: the largest of one score is that score, so
    the max-pooled routing query routes exactly as the mean query."""
    _, k, cs, gs, r = tiny_state(T=2048, seed=21)
    for t in (700, 1500, 2047):
        q = r.standard_normal((1, 2, 64))
        a = oracle.select(cfg(kc=5, kg=9), q, t - 1, cs, gs)
        c_max = cfg(kc=5, kg=9)
        c_max.route_max = 1
        b = oracle.select(c_max, q, t - 1, cs, gs)
        assert list(a[0]) == list(b[0])
        np.testing.assert_array_equal(a[2], b[2])


def test_max_pooled_scores_are_the_largest_head_score():
    """Brute force: with 4 query heads and 3 query tokens, each candidate's
    level-1 score is the largest over the heads of the head's token-mean
    rotated query (transformers' RoPE) dotted with the chunk summary, and the
    level-2 scores the same over the group summaries; every such score is at
    least the mean query's score."""
    d, hg, lq = 64, 4, 3
    c = oracle.make_cfg(d, hg, 1, 64, 4, 1, 1, 3, 6, 1e4, 64.0, False, route_max=True)
    c_mean = oracle.make_cfg(d, hg, 1, 64, 4, 1, 1, 3, 6, 1e4, 64.0, False)
    k = RNG.standard_normal((64 * 24, d))
    cs, gs = oracle.summaries(c, k)
    q = RNG.standard_normal((hg, lq, d))
    pos0 = 64 * 23 + 17
    sel, _, scores = oracle.select(c, q, pos0, cs, gs)
    _, _, mean_scores = oracle.select(c_mean, q, pos0, cs, gs)
    qh = np.stack([lib_rope(q[h], np.arange(pos0, pos0 + lq), c).mean(axis=0) for h in range(hg)])
    cand = np.arange(1, 23 - 1)
    want = (cs[cand] @ qh.T / math.sqrt(d)).max(axis=1)
    np.testing.assert_allclose(scores, want, rtol=1e-12, atol=1e-13)
    assert np.all(scores >= mean_scores - 1e-12)
    g_all = np.arange(gs.shape[0])
    want_g = (gs[g_all] @ qh.T / math.sqrt(d)).max(axis=1)
    got_g = oracle.group_scores(c, q, pos0, gs)  # the groups of the chunks before the query's
    np.testing.assert_allclose(got_g, want_g[:len(got_g)], rtol=1e-12, atol=1e-13)
    # the routed groups: top-6 of the groups of the top-3 chunks by these scores
    top1 = cand[np.lexsort((cand, -want))[:3]]
    groups = np.array([ch * 4 + j for ch in sorted(top1) for j in range(4)])
    top2 = set(groups[np.lexsort((groups, -want_g[groups]))[:6]])
    routed = {g for g in sel if 1 <= g // 4 < 22}
    assert routed == top2
