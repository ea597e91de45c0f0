"""Pins for the oracle's attention and merge (CPU only).

* torch's scaled-dot-product attention and logsumexp in float64 (library
  routines) on random small cases, causal and not;
* closed forms: one token, zero query, identical keys, a dominant key;
* brute force with math.fsum on tiny cases;
* the merge invariant of the SGLang page (section "MLA decode dataflow"):
  merging the c striped partials equals the unpartitioned attention, for
  c = 1..8 including shards that are empty; c = 1 is plain attention;
* the Gaussian closed form at long context (a sanity pin, not parity);
* planted mistakes in copies of the oracle fail at least one pin.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle.codecs import bf16_to_f64

SCALE = 1.0 / math.sqrt(192.0)


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _case(rng, q_len, H, L, scale_q=1.0):
    q = _bf16(scale_q * rng.standard_normal((q_len, H, 576)))
    kv = _bf16(rng.standard_normal((L, 576)))
    return q, (kv, None)


def _torch_ref(q_bits, kv_bits, L, scale, causal):
    q = torch.from_numpy(bf16_to_f64(q_bits))          # [q_len][H][576]
    K = torch.from_numpy(bf16_to_f64(kv_bits))         # [L][576]
    q_len, H, _ = q.shape
    qh = q.permute(1, 0, 2)                            # [H][q_len][576]
    Kh = K.unsqueeze(0).expand(H, L, 576)
    Vh = K[:, :512].unsqueeze(0).expand(H, L, 512)
    if causal:
        pos = torch.arange(L)
        lim = torch.tensor([L - q_len + i for i in range(q_len)])
        mask = pos[None, :] <= lim[:, None]
    else:
        mask = torch.ones(q_len, L, dtype=torch.bool)
    o = torch.nn.functional.scaled_dot_product_attention(qh, Kh, Vh, attn_mask=mask, scale=scale)
    s = scale * torch.matmul(qh, Kh.transpose(1, 2))
    s = s.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return o.permute(1, 0, 2).numpy(), lse.permute(1, 0).numpy()


@pytest.mark.parametrize("seed,q_len,H,L,causal", [
    (0, 1, 4, 1, True), (1, 1, 8, 37, True), (2, 4, 4, 4, True), (3, 4, 2, 129, True),
    (4, 3, 6, 70, False), (5, 2, 16, 300, True), (6, 8, 2, 11, True)])
def test_matches_torch_sdpa_float64(seed, q_len, H, L, causal):
    rng = np.random.default_rng(seed)
    q, kv = _case(rng, q_len, H, L)
    o, lse = A.decode_attention(q, kv, L, SCALE, causal=causal)
    o_ref, lse_ref = _torch_ref(q, kv[0], L, SCALE, causal)
    assert np.abs(o - o_ref).max() < 1e-12
    assert np.abs(lse - lse_ref).max() < 1e-12
    o2, lse2 = A.decode_attention(q, kv, L, SCALE, causal=causal, base="2")
    assert np.abs(o2 - o).max() == 0
    assert np.abs(lse2 - lse_ref / math.log(2)).max() < 1e-12


def test_single_token_closed_form():
    rng = np.random.default_rng(7)
    q, kv = _case(rng, 1, 3, 1)
    o, lse = A.decode_attention(q, kv, 1, SCALE)
    K = bf16_to_f64(kv[0])
    qf = bf16_to_f64(q)
    assert np.array_equal(o[0], np.broadcast_to(K[0, :512], (3, 512)))
    s0 = SCALE * (qf[0] @ K[0])
    assert np.abs(lse[0] - s0).max() < 1e-12


def test_zero_query_is_mean_and_log_n():
    rng = np.random.default_rng(8)
    L = 50
    _, kv = _case(rng, 1, 2, L)
    q = np.zeros((1, 2, 576), dtype=np.uint16)
    o, lse = A.decode_attention(q, kv, L, SCALE)
    K = bf16_to_f64(kv[0])
    assert np.abs(o[0] - K[:, :512].mean(axis=0)).max() < 1e-14
    assert np.abs(lse - math.log(L)).max() < 1e-14
    _, lse2 = A.decode_attention(q, kv, L, SCALE, base="2")
    assert np.abs(lse2 - math.log2(L)).max() < 1e-13


def test_identical_keys_uniform_weights():
    rng = np.random.default_rng(9)
    L = 33
    row = _bf16(rng.standard_normal((1, 576)))
    kv = (np.repeat(row, L, axis=0), None)
    q = _bf16(rng.standard_normal((1, 4, 576)))
    o, lse = A.decode_attention(q, kv, L, SCALE)
    K0 = bf16_to_f64(row)[0]
    s = SCALE * (bf16_to_f64(q)[0] @ K0)
    assert np.abs(o[0] - K0[:512]).max() < 1e-14
    assert np.abs(lse[0] - (s + math.log(L))).max() < 1e-12


def test_dominant_key_and_causal_limit():
    rng = np.random.default_rng(10)
    L = 64
    q = _bf16(rng.standard_normal((2, 1, 576)))
    qf = bf16_to_f64(q)
    K = rng.standard_normal((L, 576)) * 0.01
    K[L - 1] = 4.0 * qf[1, 0]             # only the last query row may see it
    K[5] = 4.0 * qf[0, 0]
    kv = (_bf16(K), None)
    o, _ = A.decode_attention(q, kv, L, SCALE, causal=True)
    Kd = bf16_to_f64(kv[0])
    assert np.abs(o[1, 0] - Kd[L - 1, :512]).max() < 1e-6
    assert np.abs(o[0, 0] - Kd[5, :512]).max() < 1e-6


@pytest.mark.parametrize("seed,q_len,L,causal", [(0, 1, 1, True), (1, 1, 5, True), (2, 3, 6, True), (3, 2, 9, False)])
def test_brute_force_fsum(seed, q_len, L, causal):
    rng = np.random.default_rng(100 + seed)
    H = 2
    q, kv = _case(rng, q_len, H, L)
    o, lse = A.decode_attention(q, kv, L, SCALE, causal=causal)
    qf = bf16_to_f64(q)
    K = bf16_to_f64(kv[0])
    for i in range(q_len):
        last = L - q_len + i if causal else L - 1
        for h in range(H):
            s = [SCALE * math.fsum(float(qf[i, h, d]) * float(K[p, d]) for d in range(576))
                 for p in range(last + 1)]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            z = math.fsum(w)
            assert abs(lse[i, h] - (m + math.log(z))) < 1e-12
            for d in range(0, 512, 37):
                ref = math.fsum(w[p] * float(K[p, d]) for p in range(last + 1)) / z
                assert abs(o[i, h, d] - ref) < 1e-12


@pytest.mark.parametrize("L,q_len,c", [(1, 8, 1), (2, 8, 3), (5, 8, 4), (3, 4, 2), (6, 8, 8)])
def test_rows_that_see_no_position_brute_force(L, q_len, c):
    # causal verification with fewer tokens than query rows: row i sits at
    # position L - q_len + i and sees p <= L - q_len + i, so rows with i <
    # q_len - L see nothing.  Brute force over the visible set (math.fsum), for
    # the full context and for every rank's striped share p mod c = r: an empty
    # set gives lse = -inf and o = 0, the others the plain softmax.
    rng = np.random.default_rng(400 + 10 * L + q_len + c)
    H = 2
    q, kv = _case(rng, q_len, H, L)
    qf = bf16_to_f64(q)
    K = bf16_to_f64(kv[0])
    o_full, lse_full = A.decode_attention(q, kv, L, SCALE, causal=True)
    o_p, lse_p = A.rank_partials(q, kv, L, SCALE, c, causal=True)

    def brute(i, h, positions):
        if not positions:
            return None, -math.inf
        s = [SCALE * math.fsum(float(qf[i, h, d]) * float(K[p, d]) for d in range(576)) for p in positions]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        z = math.fsum(w)
        o = [math.fsum(w[k] * float(K[p, d]) for k, p in enumerate(positions)) / z for d in range(512)]
        return np.array(o), m + math.log(z)

    n_empty = 0
    for i in range(q_len):
        last = L - q_len + i
        for h in range(H):
            for r in [None] + list(range(c)):
                pos = [p for p in range(L) if p <= last and (r is None or p % c == r)]
                o_ref, l_ref = brute(i, h, pos)
                o_got, l_got = (o_full[i, h], lse_full[i, h]) if r is None else (o_p[r, i, h], lse_p[r, i, h])
                if o_ref is None:
                    n_empty += r is None
                    assert l_got == -math.inf and not o_got.any(), (i, h, r)
                else:
                    assert abs(l_got - l_ref) < 1e-12 and np.abs(o_got - o_ref).max() < 1e-12, (i, h, r)
    assert n_empty == H * (q_len - L)


@pytest.mark.parametrize("c", range(1, 9))
@pytest.mark.parametrize("L", [1, 3, 7, 64, 130])
@pytest.mark.parametrize("q_len,base", [(1, "e"), (4, "2")])
def test_striped_merge_equals_full(c, L, q_len, base):
    # with q_len > L the first verification rows see no position at all: their
    # full attention and every partial are (o = 0, lse = -inf), and so is the merge
    rng = np.random.default_rng(c * 1000 + L + q_len)
    q, kv = _case(rng, q_len, 3, L)
    o_full, lse_full = A.decode_attention(q, kv, L, SCALE, causal=True, base=base)
    o_p, lse_p = A.rank_partials(q, kv, L, SCALE, c, causal=True, base=base)
    for r in range(c):
        if r >= L:
            assert np.all(np.isneginf(lse_p[r])) and not o_p[r].any()
    o, lse = A.merge(o_p, lse_p, base)
    empty = np.isneginf(lse_full)
    assert np.array_equal(np.isneginf(lse), empty)
    assert empty.sum() == 3 * max(0, q_len - L)
    assert not o[empty].any() and not o_full[empty].any()
    assert np.abs(o - o_full).max() < 1e-12
    assert np.abs(lse[~empty] - lse_full[~empty]).max(initial=0.0) < 1e-12
    if c == 1:
        assert np.array_equal(o_p[0], o_full) and np.array_equal(lse_p[0], lse_full)


def test_merge_permutation_and_empty_identity():
    rng = np.random.default_rng(11)
    q, kv = _case(rng, 1, 4, 40)
    o_p, lse_p = A.rank_partials(q, kv, 40, SCALE, 5)
    o1, l1 = A.merge(o_p, lse_p)
    perm = [3, 0, 4, 2, 1]
    o2, l2 = A.merge(o_p[perm], lse_p[perm])
    assert np.abs(o1 - o2).max() < 1e-14 and np.abs(l1 - l2).max() < 1e-13
    o3, l3 = A.merge(np.concatenate([o_p, np.zeros_like(o_p[:1])]),
                     np.concatenate([lse_p, np.full_like(lse_p[:1], -np.inf)]))
    assert np.abs(o1 - o3).max() < 1e-14 and np.abs(l1 - l3).max() < 1e-13
    o4, l4 = A.merge(np.zeros((2, 1, 512)), np.full((2, 1), -np.inf))
    assert not o4.any() and np.isneginf(l4).all()


def test_gaussian_closed_form_long_context():
    # K ~ N(0, I) with V = K[:512] and a = scale*q: lse -> ln L + |a|^2/2 and o -> a[:512]
    rng = np.random.default_rng(12)
    L = 32768
    q, kv = _case(rng, 1, 4, L)
    o, lse = A.decode_attention(q, kv, L, SCALE)
    a = SCALE * bf16_to_f64(q)[0]
    a2 = (a * a).sum(axis=1)
    sig = math.sqrt(math.expm1(a2.max()) / L)
    assert np.abs(lse[0] - (math.log(L) + a2 / 2)).max() < 6 * sig
    assert np.abs(o[0] - a[:, :512]).max() < 8 * math.sqrt(math.exp(2 * a2.max()) / L)


# ---- planted mistakes: each copy of the oracle with one plausible bug fails a pin ----

def _mutant_attention(kind):
    def run(q_bits, kv, L, scale, causal=True, base="e"):
        q_len, H, _ = q_bits.shape
        q = bf16_to_f64(q_bits).reshape(q_len * H, 576)
        K = bf16_to_f64(kv[0])
        lim = np.repeat(A._limits(L, q_len, causal), H)
        if kind == "off_by_one_causal":
            lim = lim - 1
        if kind == "no_rope_in_scores":
            K = K.copy()
            K[:, 512:] = 0
        if kind == "v_from_tail":
            V = K[:, 64:]
        else:
            V = K[:, :512]
        sc = scale * (2.0 if kind == "wrong_scale" else 1.0)
        s = sc * (q @ K.T)
        s = np.where(np.arange(L)[None, :] <= lim[:, None], s, -np.inf)
        m = s.max(1)
        e = np.exp(s - m[:, None])
        ell = e.sum(1)
        o = (e @ V) / ell[:, None]
        lse = m + np.log(ell) + (1e-3 if kind == "lse_bias" else 0.0)
        return o.reshape(q_len, H, 512), lse.reshape(q_len, H)
    return run


@pytest.mark.parametrize("kind", ["off_by_one_causal", "no_rope_in_scores", "v_from_tail", "wrong_scale", "lse_bias"])
def test_planted_attention_mistakes_fail_sdpa_pin(kind):
    rng = np.random.default_rng(13)
    q_len, H, L = 2, 4, 40
    q, kv = _case(rng, q_len, H, L)
    o_ref, lse_ref = _torch_ref(q, kv[0], L, SCALE, True)
    o, lse = _mutant_attention(kind)(q, kv, L, SCALE)
    assert np.abs(o - o_ref).max() > 1e-9 or np.abs(lse - lse_ref).max() > 1e-9


@pytest.mark.parametrize("kind", ["no_max_shift_sign", "weights_not_normalised", "base_mixup"])
def test_planted_merge_mistakes_fail_partition_pin(kind):
    rng = np.random.default_rng(14)
    L, c = 50, 4
    q, kv = _case(rng, 1, 3, L)
    base = "2" if kind == "base_mixup" else "e"
    o_full, lse_full = A.decode_attention(q, kv, L, SCALE, base=base)
    o_p, lse_p = A.rank_partials(q, kv, L, SCALE, c, base=base)
    ln = lse_p
    if kind == "no_max_shift_sign":
        w = np.exp(-(ln - ln.max(0)))
    elif kind == "weights_not_normalised":
        w = np.exp(ln - ln.max(0))
    else:
        w = np.exp(ln - ln.max(0))              # treats base-2 values as natural logs
    tot = w.sum(0)
    wn = w / tot if kind != "weights_not_normalised" else w
    o = (wn[..., None] * o_p).sum(0)
    lse = ln.max(0) + np.log(tot)
    assert np.abs(o - o_full).max() > 1e-9 or np.abs(lse - lse_full).max() > 1e-9


@pytest.mark.parametrize("I,causal,q_len", [(2, True, 1), (4, True, 4), (16, True, 4), (3, False, 2)])
def test_interleaved_partials_merge_to_full_attention(I, causal, q_len):
    # the ranks' shares under interleave I partition the context: the exact merge
    # of their partials is the full attention (and the causal limits of the
    # verify rows hold per rank)
    rng = np.random.default_rng(11 + I)
    L, c = 97, 4
    q, kv = _case(rng, q_len, 2, L)
    o_full, l_full = A.decode_attention(q, kv, L, SCALE, causal, "e")
    op, lp = A.rank_partials(q, kv, L, SCALE, c, causal, "e", I=I)
    o, l = A.merge(op, lp, "e")
    assert np.abs(o - o_full).max() < 1e-12 and np.abs(l - l_full).max() < 1e-12


def test_interleaved_rank_share_is_the_dealt_positions():
    # rank r's partial with interleave I equals full attention over exactly the
    # positions dealt to r in chunks of I (built without the closed form)
    rng = np.random.default_rng(5)
    L, c, I = 50, 3, 4
    q, (kv, _) = _case(rng, 1, 2, L)
    dealt = [[] for _ in range(c)]
    for p in range(L):
        dealt[(p // I) % c].append(p)
    for r in range(c):
        pos = np.array(dealt[r])
        o_r, l_r = A.decode_attention(q, (kv, None), L, SCALE, False, "e", c=c, r=r, I=I)
        o_s, l_s = A.decode_attention(q, (kv[pos], None), len(pos), SCALE, False, "e")
        assert np.abs(o_r - o_s).max() < 1e-12 and np.abs(l_r - l_s).max() < 1e-12
